"""Steps of two handles enqueued on two streams with no host synchronisation
in between.  A step needs every CU at once (one workgroup per CU, grid
barriers), so two steps that ran at the same time would each wait for
workgroups the other holds; the library orders the steps of a device across
streams.  Each output must equal the same step run alone, bit for bit, and
no barrier may time out (the watchdog is cut to 50 ms so that a wait for
workgroups that cannot be placed would report within the test)."""
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_layer_stack_amd as mk
    mk.lib()
    return torch


def test_steps_of_two_handles_on_two_streams(env):
    import moe_layer_stack_amd as mk
    from synth.stack import DeviceStack
    from synth.workloads import MOE16_B8
    torch = env
    w = MOE16_B8
    print(f"[gpu-case] two handles on two streams {w.name} L=4", flush=True)
    st = DeviceStack(w, n_layers=4)
    h1 = mk.mk_create(st.config(rows=1, rows_per_seq=1), st.layer_weights())
    h8 = mk.mk_create(st.config(rows=8, rows_per_seq=1), st.layer_weights())
    try:
        for h in (h1, h8):
            mk.mk_set_watchdog(h, 5_000_000)  # 50 ms of the 100 MHz counter
        x8 = st.hidden(0)
        x1 = x8[:1].clone()
        p8 = torch.as_tensor(w.positions(0), dtype=torch.int32, device="cuda")
        p1 = p8[:1].clone()
        ref1, ref8 = torch.empty_like(x1), torch.empty_like(x8)
        mk.mk_decode_step(h1, x1.data_ptr(), p1.data_ptr(), None, ref1.data_ptr(), 0)
        assert mk.mk_sync(h1, 0) == mk.MK_OK
        mk.mk_decode_step(h8, x8.data_ptr(), p8.data_ptr(), None, ref8.data_ptr(), 0)
        assert mk.mk_sync(h8, 0) == mk.MK_OK

        s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
        rounds = 4
        o1 = [torch.full_like(x1, float("nan")) for _ in range(2 * rounds)]
        o8 = [torch.full_like(x8, float("nan")) for _ in range(rounds)]
        torch.cuda.synchronize()
        for i in range(rounds):
            # batch 1 on s1, batch 8 on s2, then batch 1 again on s2 (per phase)
            # and, next round, on s1: every step after the first changes stream
            mk.mk_decode_step(h1, x1.data_ptr(), p1.data_ptr(), None, o1[2 * i].data_ptr(), s1.cuda_stream)
            mk.mk_decode_step(h8, x8.data_ptr(), p8.data_ptr(), None, o8[i].data_ptr(), s2.cuda_stream)
            mk.mk_decode_step_phased(h1, x1.data_ptr(), p1.data_ptr(), None, o1[2 * i + 1].data_ptr(),
                                     s2.cuda_stream)
        rc1 = mk.mk_sync(h1, s1.cuda_stream)
        rc1b = mk.mk_sync(h1, s2.cuda_stream)
        rc8 = mk.mk_sync(h8, s2.cuda_stream)
        torch.cuda.synchronize()
        assert (rc1, rc1b, rc8) == (mk.MK_OK, mk.MK_OK, mk.MK_OK), (rc1, rc1b, rc8, mk.mk_last_error())
        for i, o in enumerate(o1):
            assert torch.equal(o, ref1), f"batch-1 step {i}: max diff {(o - ref1).abs().max().item()}"
        for i, o in enumerate(o8):
            assert torch.equal(o, ref8), f"batch-8 step {i}: max diff {(o - ref8).abs().max().item()}"
    finally:
        mk.mk_destroy(h1)
        mk.mk_destroy(h8)
