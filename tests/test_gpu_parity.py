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
    from parity_util import GpuRun, assert_close, oracle_walk, tolerances
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
        # routing weights of rows whose set matched
        for l in range(st.L):
            for r in range(w.M):
                if set(ids[l, r]) == set(rep["oracle_ids"][l][r]):
                    go = {int(e): float(x) for e, x in zip(ids[l, r], wts[l, r])}
                    oo = {int(e): float(x) for e, x in zip(rep["oracle_ids"][l][r], rep["oracle_w"][l][r])}
                    for e in go:
                        assert abs(go[e] - oo[e]) < 2e-3, (l, r, e, go[e], oo[e])
                    assert abs(sum(go.values()) - 1.0) < 1e-5
        if w.has_attn and check_kv:
            # the rows this step wrote equal bf16(oracle) up to one bf16 step
            import oracle
            from parity_util import dims_of, oracle_layer
            for l in (0, st.L - 1):
                kh, vh = st.host_kv(l)
                for r, p in enumerate(pos):
                    s = r // w.rows_per_seq
                    kd = (kh[s, :, p].astype(np.int32) - kv_before[l][0][s, :, p].astype(np.int32))
                    assert kd.any(), "new K row not written"
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
