"""The many-kernels baseline (mk_decode_step_phased: one launch per phase of
every layer, no prefetch across launches) runs the same phase code as the
persistent kernel, so its step output and routing trace must equal the
persistent kernel's bit for bit on every path: fp32 and bf16 stacks, one and
eight rows, decode and verify attention."""
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


def _trace_bufs(torch, L, M, w):
    return (torch.zeros(L, M, w.k, dtype=torch.int32, device="cuda"),
            torch.zeros(L, M, w.k, dtype=torch.float32, device="cuda"),
            torch.zeros(L, M, w.E, dtype=torch.float32, device="cuda"))


@pytest.mark.parametrize("name,layers", [("tiny_fp32_b1", None), ("moe16_b8", 2), ("attn92_b1", 2),
                                         ("attn92_b8", 2), ("verify92_m8", 2), ("verify92_m64", 2)])
def test_phased_equals_persistent(env, name, layers):
    import moe_layer_stack_amd as mk
    from synth.stack import DeviceStack
    from synth.workloads import ALL
    torch = env
    w = ALL[name]
    _say(f"{name} L={layers or w.L} M={w.M} rps={w.rows_per_seq}: persistent vs phased")
    st = DeviceStack(w, n_layers=layers)
    h = mk.mk_create(st.config(), st.layer_weights())
    try:
        # every row of a step in one launch, row groups included (bf16 stacks)
        assert mk.mk_get_info(h).launches_per_step == 1
        hid = st.hidden(0)
        pos = torch.tensor(w.positions(0), dtype=torch.int32, device="cuda")
        outs, traces = [], []
        for fn in (mk.mk_decode_step, mk.mk_decode_step_phased):
            tr = _trace_bufs(torch, st.L, w.M, w)
            mk.mk_set_trace(h, tr[0].data_ptr(), tr[1].data_ptr(), tr[2].data_ptr())
            out = torch.empty_like(hid)
            fn(h, hid.data_ptr(), pos.data_ptr(), st.kv(), out.data_ptr(), 0)
            assert mk.mk_sync(h, 0) == mk.MK_OK, mk.mk_last_error()
            outs.append(out)
            traces.append(tr)
        torch.cuda.synchronize()
        assert torch.isfinite(outs[0]).all()
        assert torch.equal(outs[0], outs[1]), f"{name}: max |diff| {(outs[0] - outs[1]).abs().max().item()}"
        for a, b in zip(traces[0], traces[1]):
            assert torch.equal(a, b)
        _say(f"{name}: identical")
    finally:
        mk.mk_destroy(h)
