"""GPU parity: libmk.so against the CPU oracle on seeded inputs.

All tests call through the C ABI (moe_layer_stack_amd is a ctypes binding)."""
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


def _run_and_check(env, w, n_layers=None, step=0, check_kv=True):
    from parity_util import GpuRun, assert_close, assert_kv_rows, assert_routing_weights, oracle_walk, tolerances
    from synth.stack import DeviceStack
    torch = env
    _say(f"{w.name} L={n_layers or w.L} M={w.M} rps={w.rows_per_seq}")
    st = DeviceStack(w, n_layers=n_layers)
    kv_before = [st.host_kv(l) for l in range(st.L)] if w.has_attn else None
    hid = st.hidden(step)
    run = GpuRun(st)
    try:
        pos = w.positions(step)
        out = run.step(hid, pos)
        torch.cuda.synchronize()
        ids, wts, logits = run.trace()
        ref, rep = oracle_walk(st, hid.cpu().numpy(), pos, ids, rows_per_seq=w.rows_per_seq, kv_hosts=kv_before)
        assert not rep["mismatch"], f"expert sets differ beyond the tie margin: {rep['mismatch'][:5]}"
        c = assert_close(out.cpu().numpy(), ref, tolerances(w), w.name)
        assert_routing_weights(ids, wts, logits, rep, w.M, st.L, what=w.name)
        if w.has_attn and check_kv:
            # every row this step appended (each layer, row and kv head) is
            # the oracle's bf16 row within one bf16 step
            c.update(assert_kv_rows(st, rep, pos, w.rows_per_seq, what=w.name))
        _say(f"{w.name} ok {c} forced={rep['forced']}")
        return out, ids
    finally:
        run.close()


def test_tiny_fp32_stack(env):
    from synth.workloads import TINY
    _run_and_check(env, TINY)


def test_moe16_batch1(env):
    from synth.workloads import MOE16_B1
    _run_and_check(env, MOE16_B1)


def test_moe16_batch8(env):
    from synth.workloads import MOE16_B8
    _run_and_check(env, MOE16_B8)


def test_attn_stack_prefix_batch1(env):
    from synth.workloads import ATTN92_B1
    _run_and_check(env, ATTN92_B1, n_layers=2)


def test_attn_stack_prefix_batch8(env):
    from synth.workloads import ATTN92_B8
    _run_and_check(env, ATTN92_B8, n_layers=2)


def test_verify_prefix_m8(env):
    from synth.workloads import VERIFY92_M8
    _run_and_check(env, VERIFY92_M8, n_layers=2)


@pytest.mark.parametrize("M", [16, 32])
def test_row_groups_in_one_launch_moe16(env, M):
    """2 and 4 row groups of 8 independent rows in one launch on the MoE-only
    stack (no attention: the routed tasks read each row's layer input, the
    step input at layer 0 and the previous layer's output after it), 3
    layers, against the oracle."""
    import moe_layer_stack_amd as mk
    from synth.stack import DeviceStack
    from synth.workloads import MOE16_B8
    w = MOE16_B8.with_(name=f"moe16_rows{M}", M=M)
    st = DeviceStack(w, n_layers=3)
    h = mk.mk_create(st.config(), st.layer_weights())
    try:
        assert mk.mk_get_info(h).launches_per_step == 1
    finally:
        mk.mk_destroy(h)
    del st
    _run_and_check(env, w, n_layers=3)


@pytest.mark.parametrize("M", [16, 32])
def test_row_groups_in_one_launch_verify(env, M):
    """2 and 4 sequences x 8 verify rows in one launch (row groups with
    routed tasks), 2-layer prefix of the 92-layer stack, against the oracle."""
    from synth.workloads import VERIFY92_M64
    _run_and_check(env, VERIFY92_M64.with_(name=f"verify92_m{M}", M=M), n_layers=2)


def test_device_generator_matches_host(env):
    import synth
    torch = env
    for dt, tdt in ((synth.F32, torch.float32), (synth.BF16, torch.bfloat16)):
        n = 100003
        t = torch.empty(n, dtype=tdt, device="cuda")
        synth.device_normal(t.data_ptr(), n, dt, 77, synth.stream_id(3, synth.K_WQ), 0.0, 0.02)
        torch.cuda.synchronize()
        from synth.stack import DeviceStack
        dev = DeviceStack.to_host(t)
        host = synth.host_normal((n,), dt, 77, synth.stream_id(3, synth.K_WQ), 0.0, 0.02)
        # libm and the device math library may differ in the last bit of a double
        if dt == synth.F32:
            ulp = np.abs(dev.view(np.int32).astype(np.int64) - host.view(np.int32).astype(np.int64))
        else:
            ulp = np.abs(dev.astype(np.int64) - host.astype(np.int64))
        assert ulp.max() <= 1 and (ulp != 0).sum() <= 2, (dt, ulp.max(), (ulp != 0).sum())


def test_verify_prefix_m64(env):
    """8 sequences x 8 draft rows (a step of more than 8 rows: one launch per
    8 rows, whole sequences each)."""
    from synth.workloads import VERIFY92_M64
    _run_and_check(env, VERIFY92_M64, n_layers=2)
