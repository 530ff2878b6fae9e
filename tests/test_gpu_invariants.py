"""GPU checks through the C ABI that do not need the oracle's arithmetic, or
only a little of it: exact identities of the method, determinism, device-side
error reporting, the batch and verify equivalences, multi-step feedback and a
full-depth run of the 92-layer stack."""
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


def _stack(w, n_layers=None):
    from synth.stack import DeviceStack
    return DeviceStack(w, n_layers=n_layers)


def test_zero_router_routes_first_k_with_equal_weights(env):
    """W_r = 0 and b = 0: every logit is exactly 0, so the first k experts are
    chosen (equal values rank the lower id first) with weights exactly 1/k."""
    from parity_util import GpuRun, assert_close, oracle_walk, tolerances
    from synth.workloads import MOE16_B8
    torch = env
    w = MOE16_B8
    _say(f"zero router {w.name} L=2")
    st = _stack(w, 2)
    for t in st.layers:
        t["wr"].zero_()
        t["br"].zero_()
    run = GpuRun(st)
    try:
        hid = st.hidden(0)
        out = run.step(hid, w.positions(0))
        ids, wts, logits = run.trace()
        assert (logits == 0).all()
        assert (ids == np.arange(w.k, dtype=np.int32)).all(), ids[:, 0]
        assert (wts == np.float32(1.0) / np.float32(w.k)).all(), np.unique(wts)
        ref, rep = oracle_walk(st, hid.cpu().numpy(), w.positions(0), ids)
        assert not rep["mismatch"]
        assert_close(out.cpu().numpy(), ref, tolerances(w), "zero router")
    finally:
        run.close()


@pytest.mark.parametrize("M", [1, 8])
def test_zero_gates_leave_the_residual_exactly(env, M):
    """Every gate projection zero: silu(0) = 0, so every expert returns 0 and
    the step maps hidden_in to itself bit for bit."""
    from parity_util import GpuRun
    from synth.workloads import MOE16_B8
    torch = env
    w = MOE16_B8.with_(M=M)
    _say(f"zero gates {w.name} M={M} L=3")
    st = _stack(w, 3)
    for t in st.layers:
        t["wg"].zero_()
        t["sg"].zero_()
    run = GpuRun(st)
    try:
        hid = st.hidden(0)
        out = run.step(hid, w.positions(0))
        assert torch.equal(out, hid), (out - hid).abs().max().item()
    finally:
        run.close()


def test_identical_experts_make_routing_irrelevant(env):
    """All routed experts equal to expert 0: the weights sum to 1, so the
    output equals h + y_0 + shared whatever the router picks.  Two routers
    (the generated one and its negation) must give the same result."""
    from parity_util import GpuRun, assert_close, oracle_walk, tolerances
    from synth.workloads import MOE16_B8
    torch = env
    w = MOE16_B8
    _say(f"identical experts {w.name} L=2")
    st = _stack(w, 2)
    for t in st.layers:
        for k in ("wg", "wu", "wd"):
            t[k][1:].copy_(t[k][0:1].expand_as(t[k][1:]))
    hid = st.hidden(0)
    run = GpuRun(st)
    try:
        out_a = run.step(hid, w.positions(0)).clone()
        ids_a, _, _ = run.trace()
        for t in st.layers:
            t["wr"].neg_()
            t["br"].neg_()
        out_b = run.step(hid, w.positions(0)).clone()
        ids_b, _, _ = run.trace()
        assert (np.sort(ids_a, axis=-1) != np.sort(ids_b, axis=-1)).any(), "negated router chose the same experts"
        assert_close(out_b.cpu().numpy(), out_a.cpu().numpy(), tolerances(w), "identical experts, two routers")
        ref, rep = oracle_walk(st, hid.cpu().numpy(), w.positions(0), ids_b)
        assert_close(out_b.cpu().numpy(), ref, tolerances(w), "identical experts vs oracle")
    finally:
        run.close()


@pytest.mark.parametrize("name", ["moe16_b8", "attn92_b8"])
def test_repeated_steps_are_bitwise_identical(env, name):
    """No floating-point atomics on the path: the same inputs give the same
    bits (the attention step rewrites the same KV rows with the same values)."""
    from parity_util import GpuRun
    from synth import workloads
    torch = env
    w = {"moe16_b8": workloads.MOE16_B8, "attn92_b8": workloads.ATTN92_B8}[name]
    _say(f"determinism {name} L=2")
    st = _stack(w, 2)
    run = GpuRun(st)
    try:
        hid = st.hidden(0)
        a = run.step(hid, w.positions(0)).clone()
        ta = [x.copy() for x in run.trace()]
        b = run.step(hid, w.positions(0)).clone()
        tb = run.trace()
        assert torch.equal(a, b)
        for x, y in zip(ta, tb):
            assert np.array_equal(x, y)
    finally:
        run.close()


def test_row_order_does_not_change_a_row(env):
    """A row's arithmetic does not depend on its place among the 8 rows of a
    step: reversing the rows (every row changes all three bits of its index)
    reverses the outputs and the routing trace bit for bit.  The one-launch
    64-row verify relies on this: its routed work puts a row at any place of
    an 8-row task."""
    from parity_util import GpuRun
    from synth.workloads import MOE16_B8
    torch = env
    w = MOE16_B8
    _say(f"row order {w.name} L=2")
    st = _stack(w, 2)
    run = GpuRun(st)
    try:
        hid = st.hidden(0)
        rev = torch.arange(w.M - 1, -1, -1, device="cuda")
        a = run.step(hid, w.positions(0)).clone()
        ta = [x.copy() for x in run.trace()]
        b = run.step(hid[rev].contiguous(), w.positions(0)[::-1]).clone()
        tb = run.trace()
        assert torch.equal(a, b[rev]), (a - b[rev]).abs().max().item()
        for x, y in zip(ta, tb):
            assert np.array_equal(x, y[:, ::-1]), "trace differs under the row reversal"
    finally:
        run.close()


def test_bad_positions_are_reported_and_the_handle_recovers(env):
    """A position outside [0, capacity) or two rows of one sequence at the same
    position: the step writes nothing it should not and the next mk_sync
    returns MK_ERR_INVALID_ARG; the following valid step is unaffected."""
    import moe_layer_stack_amd as mk
    from parity_util import GpuRun
    from synth.workloads import VERIFY92_M8
    torch = env
    w = VERIFY92_M8
    _say(f"bad positions {w.name} L=2")
    st = _stack(w, 2)
    run = GpuRun(st)
    try:
        hid = st.hidden(0)
        good = run.step(hid, w.positions(0)).clone()
        kv0 = [(st.kc[l].clone(), st.vc[l].clone()) for l in range(st.L)]
        for bad in ([w.capacity] + w.positions(0)[1:], [w.past] * w.M, [-1] + w.positions(0)[1:]):
            _say(f"bad positions {bad}")
            pos = torch.as_tensor(np.asarray(bad, dtype=np.int32), device="cuda")
            out = torch.full_like(hid, 7.0)
            mk.mk_decode_step(run.h, hid.data_ptr(), pos.data_ptr(), st.kv(), out.data_ptr(), 0)
            assert mk.mk_sync(run.h, 0) == mk.MK_ERR_INVALID_ARG
            assert (out == 7.0).all(), "a rejected step wrote its output"
            for l in range(st.L):
                assert torch.equal(st.kc[l], kv0[l][0]) and torch.equal(st.vc[l], kv0[l][1]), "KV written"
        again = run.step(hid, w.positions(0))
        assert torch.equal(again, good)
    finally:
        run.close()


def test_host_side_argument_errors_launch_nothing(env):
    """Arguments the host can check are refused before any launch, for both
    entry points: hidden_out overlapping hidden_in (the same buffer, or one
    row apart), a NULL positions pointer, a KV cache of another capacity.
    The output stays untouched and the handle's next step is unchanged."""
    import moe_layer_stack_amd as mk
    from moe_layer_stack_amd import mk_kv_cache
    from parity_util import GpuRun
    from synth.workloads import ATTN92_B8
    torch = env
    w = ATTN92_B8
    _say(f"host-side argument errors {w.name} L=2")
    st = _stack(w, 2)
    run = GpuRun(st)
    try:
        hid = st.hidden(0)
        good = run.step(hid, w.positions(0)).clone()
        pos = torch.as_tensor(np.asarray(w.positions(0), dtype=np.int32), device="cuda")
        big = torch.zeros(w.M + 1, w.d, dtype=torch.float32, device="cuda")
        big[:w.M].copy_(hid)
        wrong_cap = mk_kv_cache(st.kc.data_ptr(), st.vc.data_ptr(), w.n_seq, w.capacity + 1)
        out = torch.full_like(hid, 7.0)
        cases = [
            ("same buffer", hid.data_ptr(), pos.data_ptr(), st.kv(), hid.data_ptr(), "overlaps"),
            ("one row apart", big.data_ptr(), pos.data_ptr(), st.kv(), big[1:].data_ptr(), "overlaps"),
            ("NULL positions", hid.data_ptr(), 0, st.kv(), out.data_ptr(), "NULL"),
            ("capacity", hid.data_ptr(), pos.data_ptr(), wrong_cap, out.data_ptr(), "capacity"),
        ]
        for fn in (mk.mk_decode_step, mk.mk_decode_step_phased):
            for name, a, p_, kv, b, msg in cases:
                with pytest.raises(mk.MkError) as ei:
                    fn(run.h, a, p_, kv, b, 0)
                assert ei.value.status == mk.MK_ERR_INVALID_ARG and msg in mk.mk_last_error(), (name, str(ei.value))
        torch.cuda.synchronize()
        assert mk.mk_sync(run.h, 0) == mk.MK_OK
        assert (out == 7.0).all()
        assert torch.equal(big[:w.M], hid)
        again = run.step(hid, w.positions(0))
        assert torch.equal(again, good)
    finally:
        run.close()


@pytest.mark.parametrize("name,G,M", [("attn92_b1", 8, 1), ("attn92_b8", 8, 8), ("attn92_b1", 4, 1)])
def test_timing_stamps_fill_their_buffer_exactly(env, name, G, M):
    """mk_set_timing: the kernel writes [n_cu][4 * (barriers + 1)] stamps and
    nothing past them (a guard region stays at its sentinel); each phase's
    start and end stamps are set and in time order per workgroup, the tile
    loop's stamps (where written) inside them; the output equals the untimed
    step bit for bit."""
    import moe_layer_stack_amd as mk
    from parity_util import GpuRun
    from synth.workloads import ALL
    torch = env
    w = ALL[name].with_(G=G, M=M)
    _say(f"timing stamps {w.name} G={G} M={M} L=2")
    st = _stack(w, 2)
    run = GpuRun(st)
    try:
        hid = st.hidden(0)
        plain = run.step(hid, w.positions(0)).clone()
        info = mk.mk_get_info(run.h)
        n_cu, nb = info.n_cu, info.barriers_per_step
        per = 4 * (nb + 1)
        guard = 4096
        sentinel = -7
        buf = torch.full((n_cu * per + guard,), sentinel, dtype=torch.int64, device="cuda")
        buf[:n_cu * per].zero_()
        mk.mk_set_timing(run.h, buf.data_ptr())
        timed = run.step(hid, w.positions(0))
        mk.mk_set_timing(run.h, 0)
        torch.cuda.synchronize()
        assert torch.equal(timed, plain)
        b = buf.cpu().numpy()
        assert (b[n_cu * per:] == sentinel).all(), "stamps written past the buffer"
        t = b[:n_cu * per].reshape(n_cu, nb + 1, 4)
        start, end = t[:, :, 0], t[:, :, 3]
        assert (start > 0).all() and (end > 0).all(), "a phase start or end stamp is missing"
        assert (end >= start).all()
        assert (start[:, 1:] >= end[:, :-1]).all(), "phases out of order within a workgroup"
        for k in (1, 2):
            v = t[:, :, k]
            ok = (v == 0) | ((v >= start) & (v <= end))
            assert ok.all(), f"tile-loop stamp {k} outside its phase"
        _say(f"timing stamps {w.name} G={G} M={M}: {n_cu} x {nb + 1} phases, guard intact")
    finally:
        run.close()


def test_watchdog_timeout_is_reported_and_the_handle_recovers(env):
    """The device watchdog, forced from the host: with a limit of a few ticks
    every grid-barrier poll gives up at once, every workgroup leaves the
    kernel at its next barrier, and mk_sync returns MK_ERR_TIMEOUT and resets
    the handle; back at the default limit, the next step equals a clean step
    bit for bit (its KV rows are rewritten at the same positions)."""
    import moe_layer_stack_amd as mk
    from parity_util import GpuRun
    from synth.workloads import ATTN92_B1
    torch = env
    w = ATTN92_B1
    _say(f"watchdog {w.name} L=2")
    st = _stack(w, 2)
    run = GpuRun(st)
    try:
        hid = st.hidden(0)
        good = run.step(hid, w.positions(0)).clone()
        with pytest.raises(mk.MkError):
            mk.mk_set_watchdog(run.h, 0)
        mk.mk_set_watchdog(run.h, 2)
        pos = torch.as_tensor(np.asarray(w.positions(0), dtype=np.int32), device="cuda")
        out = torch.empty_like(hid)
        mk.mk_decode_step(run.h, hid.data_ptr(), pos.data_ptr(), st.kv(), out.data_ptr(), 0)
        rc = mk.mk_sync(run.h, 0)
        assert rc == mk.MK_ERR_TIMEOUT, (rc, mk.mk_last_error())
        mk.mk_set_watchdog(run.h, 200_000_000)
        again = run.step(hid, w.positions(0))
        assert torch.equal(again, good)
        _say("watchdog: timeout reported, next step equal")
    finally:
        run.close()


def test_batch8_row_equals_batch1(env):
    """Sequences are independent: row 0 of a batch-8 step equals the batch-1
    step of sequence 0 (same row, same position, same cache)."""
    from parity_util import GpuRun, assert_close, tolerances
    from synth.workloads import ATTN92_B8
    torch = env
    w8 = ATTN92_B8
    _say(f"batch 8 row 0 vs batch 1 {w8.name} L=3")
    st = _stack(w8, 3)
    hid = st.hidden(0)
    r8 = GpuRun(st)
    r1 = GpuRun(st, rows=1, rows_per_seq=1)
    try:
        o8 = r8.step(hid, w8.positions(0)).clone()
        o1 = r1.step(hid[:1].contiguous(), w8.positions(0)[:1]).clone()
        assert_close(o1.cpu().numpy(), o8[:1].cpu().numpy(), tolerances(w8), "batch-8 row 0 vs batch 1")
        assert (r1.trace()[0][:, 0] == r8.trace()[0][:, 0]).all()
    finally:
        r8.close()
        r1.close()


def test_verify_rows_equal_sequential_decode(env):
    """Verify row r (positions p..p+7 of one sequence, causal among the
    drafts) equals decode step r run on its own after steps 0..r-1."""
    from parity_util import GpuRun, assert_close, tolerances
    from synth.workloads import VERIFY92_M8
    torch = env
    w = VERIFY92_M8
    _say(f"verify vs sequential decode {w.name} L=2")
    st = _stack(w, 2)
    kv0 = [(st.kc[l].clone(), st.vc[l].clone()) for l in range(st.L)]
    hid = st.hidden(0)
    pos = w.positions(0)
    rv = GpuRun(st)
    try:
        ov = rv.step(hid, pos).clone()
    finally:
        rv.close()
    for l in range(st.L):
        st.kc[l].copy_(kv0[l][0])
        st.vc[l].copy_(kv0[l][1])
    r1 = GpuRun(st, rows=1, rows_per_seq=1)
    try:
        for r in range(w.M):
            o1 = r1.step(hid[r:r + 1].contiguous(), [pos[r]])
            assert_close(o1.cpu().numpy(), ov[r:r + 1].cpu().numpy(), tolerances(w), f"verify row {r}")
    finally:
        r1.close()


def test_moe16_feedback_steps(env):
    """Four steps of the 16-layer stack with the output fed back; every step
    matches the oracle run on the GPU's input of that step."""
    from parity_util import GpuRun, assert_close, oracle_walk, tolerances
    from synth.workloads import MOE16_B1
    torch = env
    w = MOE16_B1
    _say(f"feedback {w.name} 4 steps")
    st = _stack(w)
    run = GpuRun(st)
    try:
        h = st.hidden(0)
        for s in range(4):
            out = run.step(h, w.positions(s))
            ids, _, _ = run.trace()
            ref, rep = oracle_walk(st, h.cpu().numpy(), w.positions(s), ids)
            assert not rep["mismatch"], rep["mismatch"][:3]
            c = assert_close(out.cpu().numpy(), ref, tolerances(w), f"step {s}")
            _say(f"step {s} {c} forced={rep['forced']}")
            h = out.clone()
    finally:
        run.close()


# The benchmark's stack at full depth (92 layers), every step against the
# oracle walked over the same bytes, in four tests over one stack (each
# takes the cache as it stands right before its own step): batch 1 (sequence
# 0); batch 8 (all 8 rows, each its own sequence); a verify pass of 8 rows
# of sequence 0; and a verify pass of 8 rows of each of the 8 sequences in
# one launch, whose sequence 5 is walked (its routed work ran in tasks mixed
# with the other sequences' rows).  Every checked step's output, expert sets,
# routing weights and all the K/V rows it appended (92 layers x rows x 8 kv
# heads) are checked.


@pytest.fixture(scope="module")
def stack92(env):
    from synth.workloads import ATTN92_B8
    torch = env
    _say(f"full depth {ATTN92_B8.name}: building L={ATTN92_B8.L}")
    st = _stack(ATTN92_B8)
    yield st
    del st
    torch.cuda.empty_cache()


def _full_depth_check(st, tag, out, hid, pos, run, rps, kv_hosts, rows=None, seq0=0):
    from parity_util import assert_close, assert_kv_rows, assert_routing_weights, oracle_walk, tolerances
    ids, wts, logits = run.trace()
    if rows is not None:  # a slice of the step's rows (whole sequences)
        ids, wts, logits = ids[:, rows], wts[:, rows], logits[:, rows]
    M = ids.shape[1]

    def progress(l):
        if l % 23 == 0:
            _say(f"full depth {tag}: oracle at layer {l}")
    ref, rep = oracle_walk(st, hid, pos, ids, rows_per_seq=rps, kv_hosts=kv_hosts, progress=progress)
    assert not rep["mismatch"], (tag, rep["mismatch"][:3])
    c = assert_close(out.cpu().numpy(), ref, tolerances(st.w), f"full depth {tag}")
    assert_routing_weights(ids, wts, logits, rep, M, st.L, what=tag)
    c.update(assert_kv_rows(st, rep, pos, rps, what=f"full depth {tag}", seq0=seq0))
    _say(f"full depth {tag} {c} forced={rep['forced']}")


@pytest.mark.timeout(900)
def test_attn92_full_depth_batch1(env, stack92):
    """Batch 1 on sequence 0."""
    from parity_util import GpuRun
    st = stack92
    hid = st.hidden(0)
    pos = st.w.positions(0)
    kv0 = [tuple(x[:1].copy() for x in st.host_kv(l)) for l in range(st.L)]
    r1 = GpuRun(st, rows=1, rows_per_seq=1)
    try:
        o1 = r1.step(hid[:1].contiguous(), pos[:1]).clone()
        _full_depth_check(st, "batch 1", o1, hid[:1].cpu().numpy(), pos[:1], r1, 1, kv0)
    finally:
        r1.close()


@pytest.mark.timeout(900)
def test_attn92_full_depth_batch8(env, stack92):
    """Batch 8 on all 8 sequences (one row each); its row 0 also equals a
    batch-1 step of sequence 0 at the same position, taken just before."""
    from parity_util import GpuRun, assert_close, tolerances
    st = stack92
    hid = st.hidden(0)
    pos = st.w.positions(0)
    r1 = GpuRun(st, rows=1, rows_per_seq=1)
    try:
        o1 = r1.step(hid[:1].contiguous(), pos[:1]).cpu().numpy()
    finally:
        r1.close()
    # the batch-1 step wrote sequence 0's row at pos[0]; batch 8 rewrites it
    kv8 = [st.host_kv(l) for l in range(st.L)]
    r8 = GpuRun(st)
    try:
        o8 = r8.step(hid, pos).clone()
        _full_depth_check(st, "batch 8", o8, hid.cpu().numpy(), pos, r8, 1, kv8)
    finally:
        r8.close()
    assert_close(o8[:1].cpu().numpy(), o1, tolerances(st.w), "full depth batch-8 row 0")


@pytest.mark.timeout(900)
def test_attn92_full_depth_verify8(env, stack92):
    """8 rows of sequence 0 at positions past .. past+7, causal among the
    drafts (the first of them overwrites the batch steps' row)."""
    from parity_util import GpuRun
    st = stack92
    pv = [st.w.past + r for r in range(8)]
    kvv = [tuple(x[:1].copy() for x in st.host_kv(l)) for l in range(st.L)]
    rv = GpuRun(st, rows=8, rows_per_seq=8)
    try:
        hv = st.hidden(1)
        ov = rv.step(hv, pv).clone()
        _full_depth_check(st, "verify 1 x 8", ov, hv.cpu().numpy(), pv, rv, 8, kvv)
    finally:
        rv.close()


@pytest.mark.timeout(900)
def test_attn92_full_depth_verify64(env, stack92):
    """8 rows of each of the 8 sequences in one launch; sequence 5 walked."""
    import moe_layer_stack_amd as mk
    from parity_util import GpuRun
    torch = env
    st = stack92
    s5 = 5
    p64 = [st.w.past + r for _ in range(8) for r in range(8)]
    kv5 = [tuple(x[s5:s5 + 1].copy() for x in st.host_kv(l)) for l in range(st.L)]
    r64 = GpuRun(st, rows=64, rows_per_seq=8)
    try:
        assert mk.mk_get_info(r64.h).launches_per_step == 1
        h64 = st.hidden(2, rows=64)
        o64 = r64.step(h64, p64).clone()
        rows5 = slice(8 * s5, 8 * s5 + 8)
        _full_depth_check(st, "verify 8 x 8, sequence 5", o64[rows5], h64[rows5].cpu().numpy(), p64[rows5], r64, 8,
                          kv5, rows=rows5, seq0=s5)
        assert torch.isfinite(o64).all()
    finally:
        r64.close()
