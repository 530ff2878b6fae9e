"""Speculative decoding around the verify step: rollback of rejected drafts.

A verify step writes the K/V rows of all 8 of its rows (the last accepted
token and 7 drafts) before attending.  When only the first a drafts are
accepted, the next step starts at position p + a + 1 and its rows overwrite
the rejected drafts' cache entries before anything reads them.  So nothing of
a rejected draft may reach a later step: the step after a rejection must give
the same bits whether the rejected positions hold the drafts or anything
else, and it must match the oracle walked over the cache as it stands.
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


def test_rejected_drafts_do_not_reach_the_next_step(env):
    from parity_util import GpuRun, assert_close, assert_kv_rows, oracle_walk, tolerances
    from synth.stack import DeviceStack
    from synth.workloads import VERIFY92_M8
    torch = env
    w = VERIFY92_M8
    st = DeviceStack(w, n_layers=2)
    run = GpuRun(st)
    try:
        p0 = w.past
        accepted = 2  # drafts accepted in step 1: tokens p0 .. p0+2 stay, p0+3 .. p0+7 are rolled back
        p1 = p0 + accepted + 1
        pristine = [(st.kc[l, 0].clone(), st.vc[l, 0].clone()) for l in range(st.L)]
        kv0 = [st.host_kv(l) for l in range(st.L)]
        pos1 = [p0 + r for r in range(8)]
        hid1 = st.hidden(0)
        _say(f"{w.name} L=2 step 1 at {p0}..{p0 + 7}")
        out1 = run.step(hid1, pos1).clone()
        ids1, _, _ = run.trace()
        # step 1 against the oracle, and the 8 rows it appended (all of them,
        # the drafts to be rejected included) before anything reuses the cache
        ref1, rep1 = oracle_walk(st, hid1.cpu().numpy(), pos1, ids1, rows_per_seq=8, kv_hosts=kv0)
        assert not rep1["mismatch"], rep1["mismatch"][:5]
        c1 = assert_close(out1.cpu().numpy(), ref1, tolerances(w), "verify step 1")
        c1.update(assert_kv_rows(st, rep1, pos1, 8, what="verify step 1"))
        _say(f"{w.name} step 1 ok {c1}")
        after1 = [(st.kc[l, 0].clone(), st.vc[l, 0].clone()) for l in range(st.L)]
        kv_hosts = [st.host_kv(l) for l in range(st.L)]
        pos2 = [p1 + r for r in range(8)]
        hid2 = st.hidden(1)
        _say(f"{w.name} step 2 at {p1}..{p1 + 7} over the rejected drafts")
        out_a = run.step(hid2, pos2).clone()
        ids_a, _, _ = run.trace()
        # the same step over a cache whose rejected positions never held the drafts
        for l in range(st.L):
            st.kc[l, 0].copy_(after1[l][0])
            st.vc[l, 0].copy_(after1[l][1])
            st.kc[l, 0, :, p1:p0 + 8].copy_(pristine[l][0][:, p1:p0 + 8])
            st.vc[l, 0, :, p1:p0 + 8].copy_(pristine[l][1][:, p1:p0 + 8])
        torch.cuda.synchronize()
        _say(f"{w.name} step 2 again with positions {p1}..{p0 + 7} restored")
        out_b = run.step(hid2, pos2).clone()
        torch.cuda.synchronize()
        assert torch.equal(out_a, out_b), "a rejected draft reached the next step"
        ref, rep = oracle_walk(st, hid2.cpu().numpy(), pos2, ids_a, rows_per_seq=8, kv_hosts=kv_hosts)
        assert not rep["mismatch"], rep["mismatch"][:5]
        c = assert_close(out_a.cpu().numpy(), ref, tolerances(w), "step after rollback")
        # run b rewrote the same rows from the same inputs
        c.update(assert_kv_rows(st, rep, pos2, 8, what="step after rollback"))
        _say(f"{w.name} rollback ok {c}")
    finally:
        run.close()
