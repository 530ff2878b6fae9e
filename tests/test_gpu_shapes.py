"""GPU parity on stack shapes the benchmark workloads do not use, against the
CPU oracle: no shared expert and two shared experts (bf16, one row and
several rows), and attention with 4 and 2 kv heads (8 and 16 query heads per
kv head, so a decode step's attention tasks take the 16-query path) at one
and eight rows.  Each runs on a stack of two or three layers built from the
same generator as the workloads.

A single row with more than 4 query heads per kv head must run the
single-row kernel (one DOWN phase), as the host lays out the workspace and
the per-phase launches for one row; the one-launch-per-phase entry point,
which runs the same phase code, must agree with the persistent kernel bit
for bit on these shapes."""
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


def _parity(torch, w):
    from parity_util import GpuRun, assert_close, oracle_walk, tolerances
    from synth.stack import DeviceStack
    _say(f"{w.name} L={w.L} M={w.M} S={w.n_shared} G={w.G}")
    st = DeviceStack(w)
    kv_before = [st.host_kv(l) for l in range(st.L)] if w.has_attn else None
    hid = st.hidden(0)
    run = GpuRun(st)
    try:
        pos = w.positions(0)
        out = run.step(hid, pos)
        torch.cuda.synchronize()
        ids, wts, _ = run.trace()
        ref, rep = oracle_walk(st, hid.cpu().numpy(), pos, ids, rows_per_seq=w.rows_per_seq, kv_hosts=kv_before)
        assert not rep["mismatch"], rep["mismatch"][:5]
        c = assert_close(out.cpu().numpy(), ref, tolerances(w), w.name)
        _say(f"{w.name}: {c} forced={rep['forced']}")
    finally:
        run.close()


@pytest.mark.parametrize("n_shared,M", [(0, 1), (0, 8), (2, 1), (2, 4)])
def test_shared_expert_counts(env, n_shared, M):
    # two shared experts at 8 rows would need 64 KiB of staged activations,
    # beyond the LDS x region (mk_create rejects it), so that case runs 4 rows
    from synth.workloads import MOE16_B1
    w = MOE16_B1.with_(name=f"moe_s{n_shared}_m{M}", L=2, n_shared=n_shared, M=M, input_seed=7)
    _parity(env, w)


@pytest.mark.parametrize("G,M,L", [(4, 1, 3), (4, 8, 2), (2, 1, 3), (1, 1, 2)])
def test_fewer_kv_heads(env, G, M, L):
    # G = 1 (one kv head for all 32 query heads): 32 queries per task at one
    # row, in two groups of 16
    from synth.workloads import ATTN92_B1
    w = ATTN92_B1.with_(name=f"attn_g{G}_m{M}", L=L, G=G, M=M, input_seed=8)
    _parity(env, w)


@pytest.mark.parametrize("G,rps", [(4, 4), (2, 2)])
def test_verify_fewer_kv_heads(env, G, rps):
    # 8 rows as 8 / rps sequences of rps verify rows: rps * 32 / G = 32 queries
    # per (sequence, kv head), in two groups of 16
    from synth.workloads import VERIFY92_M8
    w = VERIFY92_M8.with_(name=f"verify_g{G}_rps{rps}", L=2, G=G, rows_per_seq=rps, input_seed=8)
    _parity(env, w)


@pytest.mark.parametrize("M,rps", [(3, 1), (6, 3), (5, 1)])
def test_odd_row_counts(env, M, rps):
    # row counts between 1 and 8 run the 8-row kernel on M rows; 3 verify rows
    # of 4 heads give 12 queries per (sequence, kv head), a partly filled
    # 16-query operand
    from synth.workloads import ATTN92_B1
    w = ATTN92_B1.with_(name=f"attn_m{M}_rps{rps}", L=2, M=M, rows_per_seq=rps, input_seed=10)
    _parity(env, w)


@pytest.mark.parametrize("G", [4, 2, 1])
def test_fewer_kv_heads_phased_equals_persistent(env, G):
    import moe_layer_stack_amd as mk
    from synth.stack import DeviceStack
    from synth.workloads import ATTN92_B1
    torch = env
    w = ATTN92_B1.with_(name=f"attn_g{G}_m1", L=3, G=G, M=1, input_seed=8)
    _say(f"{w.name} L={w.L}: persistent vs phased")
    st = DeviceStack(w)
    h = mk.mk_create(st.config(), st.layer_weights())
    try:
        hid = st.hidden(0)
        pos = torch.tensor(w.positions(0), dtype=torch.int32, device="cuda")
        outs = []
        for fn in (mk.mk_decode_step, mk.mk_decode_step_phased):
            out = torch.empty_like(hid)
            fn(h, hid.data_ptr(), pos.data_ptr(), st.kv(), out.data_ptr(), 0)
            assert mk.mk_sync(h, 0) == mk.MK_OK, mk.mk_last_error()
            outs.append(out)
        torch.cuda.synchronize()
        assert torch.isfinite(outs[0]).all()
        assert torch.equal(outs[0], outs[1]), f"max |diff| {(outs[0] - outs[1]).abs().max().item()}"
        _say(f"{w.name}: identical")
    finally:
        mk.mk_destroy(h)
