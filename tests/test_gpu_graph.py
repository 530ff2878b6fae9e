"""A step captured into a HIP graph and replayed with new inputs.

The attention split combine accepts only partial words that carry the
launch's tag.  Tags are taken on the device at launch start, so every replay
of a captured step gets a new one; a replay that accepted the previous
replay's partials would differ from the eager step on the same input.  Each
replay is checked against an eager step, with the eager work between the
replays, for the persistent kernel and for the one-launch-per-phase
baseline."""
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


@pytest.mark.parametrize("name", ["attn92_b1", "verify92_m8"])
@pytest.mark.parametrize("phased", [False, True])
def test_graph_replays_equal_eager_steps(env, name, phased):
    import moe_layer_stack_amd as mk
    from synth.stack import DeviceStack
    from synth.workloads import ALL
    torch = env
    w = ALL[name]
    fn = mk.mk_decode_step_phased if phased else mk.mk_decode_step
    _say(f"{name} L=2 {'phased' if phased else 'persistent'}: graph replays")
    st = DeviceStack(w, n_layers=2)
    h = mk.mk_create(st.config(), st.layer_weights())
    try:
        s = torch.cuda.Stream()
        hin = st.hidden(0).clone()
        hout = torch.empty_like(hin)
        ref = torch.empty_like(hin)
        pos = torch.tensor(w.positions(0), dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            fn(h, hin.data_ptr(), pos.data_ptr(), st.kv(), ref.data_ptr(), s.cuda_stream)
        s.synchronize()
        assert mk.mk_sync(h, s.cuda_stream) == mk.MK_OK
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            fn(h, hin.data_ptr(), pos.data_ptr(), st.kv(), hout.data_ptr(), s.cuda_stream)
        torch.cuda.synchronize()
        for r in range(4):
            hin.copy_(st.hidden(r + 1))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert mk.mk_sync(h, 0) == mk.MK_OK, mk.mk_last_error()
            with torch.cuda.stream(s):
                fn(h, hin.data_ptr(), pos.data_ptr(), st.kv(), ref.data_ptr(), s.cuda_stream)
            s.synchronize()
            assert mk.mk_sync(h, s.cuda_stream) == mk.MK_OK, mk.mk_last_error()
            assert torch.isfinite(hout).all()
            assert torch.equal(hout, ref), f"replay {r}: max |diff| {(hout - ref).abs().max().item()}"
        _say(f"{name} {'phased' if phased else 'persistent'}: 4 replays equal")
        del g
    finally:
        mk.mk_destroy(h)
