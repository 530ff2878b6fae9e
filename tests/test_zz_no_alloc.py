"""mk_decode_step_noalloc: the step with its workspace in the library's fixed
per-device array instead of the handle's, for callers that cannot allocate.

Two calls in a row on one device (the second with fewer rows) must each equal
mk_decode_step on the same handle bit for bit, and a handle whose workspace
does not fit the array is refused before anything is launched."""
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


def test_noalloc_equals_the_allocating_step_on_two_calls(env):
    import moe_layer_stack_amd as mk
    from parity_util import GpuRun
    from synth.stack import DeviceStack
    from synth.workloads import ATTN92_B8
    torch = env
    w = ATTN92_B8
    st = DeviceStack(w, n_layers=2)
    r8 = GpuRun(st)                         # 8 rows (8 sequences)
    r1 = GpuRun(st, rows=1, rows_per_seq=1)  # 1 row: the smaller second call
    try:
        for run in (r8, r1):
            info = mk.mk_get_info(run.h)
            assert info.workspace_bytes < mk.NOALLOC_SCRATCH_BYTES, info.workspace_bytes
        h8, p8 = st.hidden(0), w.positions(0)
        h1, p1 = st.hidden(1, rows=1), w.positions(0)[:1]
        _say("reference steps (handle workspace)")
        ref8 = r8.step(h8, p8).clone()
        ids8, _, _ = r8.trace()
        ref1 = r1.step(h1, p1).clone()
        ids1, _, _ = r1.trace()
        _say("no-allocation steps, 8 rows then 1 row")
        for run, hid, pos, ref, ids in ((r8, h8, p8, ref8, ids8), (r1, h1, p1, ref1, ids1)):
            out = torch.empty_like(hid)
            pos_d = torch.as_tensor(np.asarray(pos, dtype=np.int32), device="cuda")
            mk.mk_decode_step_noalloc(run.h, hid.data_ptr(), pos_d.data_ptr(), st.kv(), out.data_ptr(), 0)
            rc = mk.mk_sync(run.h, 0)
            assert rc == mk.MK_OK, mk.mk_last_error()
            assert torch.equal(out, ref), f"rows={run.M}: max |d| {float((out - ref).abs().max())}"
            ids_n, _, _ = run.trace()
            assert np.array_equal(ids_n, ids)
        # and the handle's own workspace still gives the same step afterwards
        again = r8.step(h8, p8)
        assert torch.equal(again, ref8)
        _say("no-allocation steps equal the allocating ones")
    finally:
        r8.close()
        r1.close()


def test_noalloc_refuses_a_workspace_beyond_the_array(env):
    """60 attention layers at one row need about 72 MB of workspace: refused
    (UNSUPPORTED), nothing launched.  The layers reuse a two-layer stack's
    weights, since only the workspace size matters here."""
    import moe_layer_stack_amd as mk
    from synth.stack import DeviceStack
    from synth.workloads import ATTN92_B1
    w = ATTN92_B1
    st = DeviceStack(w, n_layers=2)
    lw = st.layer_weights()
    L = 60
    cfg = st.config(rows=1, rows_per_seq=1)
    cfg.n_layers = L
    torch = env
    h = mk.mk_create(cfg, [lw[l % 2] for l in range(L)])
    # valid buffers of the full 60-layer shape, so that even a launch would
    # stay inside its memory
    kc = torch.zeros(L, 1, w.G, w.capacity, w.hd, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    kv = mk.mk_kv_cache(kc.data_ptr(), vc.data_ptr(), 1, w.capacity)
    hid = st.hidden(0, rows=1)
    out = torch.empty_like(hid)
    pos = torch.tensor([w.past], dtype=torch.int32, device="cuda")
    try:
        assert mk.mk_get_info(h).workspace_bytes > mk.NOALLOC_SCRATCH_BYTES
        with pytest.raises(mk.MkError) as ei:
            mk.mk_decode_step_noalloc(h, hid.data_ptr(), pos.data_ptr(), kv, out.data_ptr(), 0)
        assert ei.value.status == mk.MK_ERR_UNSUPPORTED
        assert "workspace" in mk.mk_last_error()
        assert mk.mk_sync(h, 0) == mk.MK_OK
    finally:
        mk.mk_destroy(h)
