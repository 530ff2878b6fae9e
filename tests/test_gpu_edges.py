"""GPU parity at the edges of the attention path, against the CPU oracle.

The decode kernel spreads a sequence's cached positions over the splits of
each kv head tile by tile (32 positions per tile) and attends the step's new
row from its LDS copy.  These cases reach what the full-length workloads do
not:
- a step at position 0: no cached position, every split but the one holding
  the new row is empty;
- positions whose cache ends inside a tile (ragged tails) or exactly on a
  tile boundary;
- the last position the cache can hold;
- a batch of sequences of different lengths in one step;
- verify blocks of 8 rows starting at position 0 (causal mask only among the
  drafts) and at a different position in every sequence.

Each case runs on a two-layer prefix of the 92-layer stack (the layers are the
same data as in the full stack) and compares the step's output, the expert
sets and the routing weights with the oracle walked over the same bytes.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_layer_stack_amd as mk
    mk.lib()
    return torch


def _check_step(torch, st, w, run, hid, pos):
    from parity_util import assert_close, assert_kv_rows, assert_routing_weights, oracle_walk, tolerances
    kv_before = [st.host_kv(l) for l in range(st.L)]
    out = run.step(hid, pos)
    torch.cuda.synchronize()
    ids, wts, logits = run.trace()
    rps = run.cfg.rows_per_seq
    ref, rep = oracle_walk(st, hid.cpu().numpy(), pos, ids, rows_per_seq=rps, kv_hosts=kv_before)
    assert not rep["mismatch"], f"expert sets differ beyond the tie margin: {rep['mismatch'][:5]}"
    c = assert_close(out.cpu().numpy(), ref, tolerances(w), f"{w.name} positions {pos}")
    assert_routing_weights(ids, wts, logits, rep, run.M, st.L, what=f"{w.name} positions {pos}")
    # the new K/V rows at their positions, every layer, row and kv head: the
    # oracle's bf16 rows within one bf16 step
    c.update(assert_kv_rows(st, rep, pos, rps, what=f"{w.name} positions {pos}"))
    _say(f"{w.name} positions {pos}: {c} forced={rep['forced']}")
    return c


def test_short_and_ragged_contexts_batch1(env):
    """Batch 1 at positions 0, 1, 31, 32, 33, 95, 4095 and the cache's last slot."""
    from parity_util import GpuRun
    from synth.stack import DeviceStack
    from synth.workloads import ATTN92_B1
    torch = env
    w = ATTN92_B1
    st = DeviceStack(w, n_layers=2)
    run = GpuRun(st)
    try:
        for i, p in enumerate((0, 1, 31, 32, 33, 95, 4095, w.capacity - 1)):
            _say(f"{w.name} L=2 position {p}")
            _check_step(torch, st, w, run, st.hidden(i), [p])
    finally:
        run.close()


def test_sequences_of_different_lengths_batch8(env):
    """Eight sequences in one step, each at its own position: empty, tile-edge,
    ragged and full-length caches side by side."""
    from parity_util import GpuRun
    from synth.stack import DeviceStack
    from synth.workloads import ATTN92_B8
    torch = env
    w = ATTN92_B8
    st = DeviceStack(w, n_layers=2)
    run = GpuRun(st)
    try:
        pos = [0, 1, 31, 33, 100, 1000, 4095, 4096]
        _say(f"{w.name} L=2 positions {pos}")
        _check_step(torch, st, w, run, st.hidden(0), pos)
    finally:
        run.close()


def test_verify_blocks_at_start_and_ragged(env):
    """Verify of 8 rows per sequence: one sequence starting at position 0, then
    8 sequences each starting at a different position (one launch per
    sequence)."""
    from parity_util import GpuRun
    from synth.stack import DeviceStack
    from synth.workloads import VERIFY92_M8, VERIFY92_M64
    torch = env
    w = VERIFY92_M8
    st = DeviceStack(w, n_layers=2)
    run = GpuRun(st)
    try:
        pos = list(range(8))
        _say(f"{w.name} L=2 positions {pos}")
        _check_step(torch, st, w, run, st.hidden(0), pos)
    finally:
        run.close()
    del st
    torch.cuda.empty_cache()
    w = VERIFY92_M64
    st = DeviceStack(w, n_layers=2)
    run = GpuRun(st)
    try:
        starts = [0, 5, 24, 57, 100, 2000, 4000, 4096]
        pos = [s0 + r for s0 in starts for r in range(8)]
        _say(f"{w.name} L=2 block starts {starts}")
        _check_step(torch, st, w, run, st.hidden(0), pos)
    finally:
        run.close()
