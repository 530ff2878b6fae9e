"""Parity harness: run a step through libmk.so with routing traced, then walk
the CPU oracle layer by layer over the same bytes and compare.

Several expert sets are correct when the k-th and (k+1)-th router logits are
(nearly) equal.  Where the oracle's margin is <= TIE_MARGIN and the GPU chose
a different set, the oracle adopts the GPU's set for that (layer, row),
recomputing the weights from its own probabilities, and continues; with a
larger margin a different set is a failure.
"""
import numpy as np

import moe_layer_stack_amd as mk
import oracle
import synth
from synth.stack import DeviceStack

TIE_MARGIN = 1e-3
TOL_BF16 = dict(max_abs=2e-2, rel_l2=5e-3)
TOL_F32 = dict(max_abs=1e-4, rel_l2=1e-4)


def tolerances(w):
    return TOL_F32 if w.dtype == synth.F32 else TOL_BF16


def dims_of(w):
    return oracle.make_dims(w.d, w.E, w.k, w.F, w.n_shared, oracle.BF16 if w.dtype == synth.BF16 else oracle.F32,
                            rms_eps=w.rms_eps, n_heads=w.H if w.has_attn else 0, n_kv_heads=w.G if w.has_attn else 0,
                            head_dim=w.hd if w.has_attn else 0, rope_theta=w.rope_theta)


def oracle_layer(H):
    return oracle.OracleLayer(H["g2"], H["wr"], H["br"], H["w_gate"], H["w_up"], H["w_down"], H["s_gate"],
                              H["s_up"], H["s_down"], g1=H["g1"], wq=H["wq"], wk=H["wk"], wv=H["wv"], wo=H["wo"])


class GpuRun:
    """One handle over a DeviceStack with routing traced."""

    def __init__(self, stack: DeviceStack, rows=None, rows_per_seq=None):
        import torch
        self.torch = torch
        self.stack = stack
        self.cfg = stack.config(rows, rows_per_seq)
        self.M = self.cfg.rows
        self.h = mk.mk_create(self.cfg, stack.layer_weights())
        w = stack.w
        L = stack.L
        self.t_ids = torch.zeros(L, self.M, w.k, dtype=torch.int32, device="cuda")
        self.t_w = torch.zeros(L, self.M, w.k, dtype=torch.float32, device="cuda")
        self.t_logits = torch.zeros(L, self.M, w.E, dtype=torch.float32, device="cuda")
        mk.mk_set_trace(self.h, self.t_ids.data_ptr(), self.t_w.data_ptr(), self.t_logits.data_ptr())

    def step(self, hidden, positions, out=None):
        torch = self.torch
        pos = torch.as_tensor(np.asarray(positions, dtype=np.int32), device="cuda")
        if out is None:
            out = torch.empty_like(hidden)
        mk.mk_decode_step(self.h, hidden.data_ptr(), pos.data_ptr(), self.stack.kv(), out.data_ptr(), 0)
        rc = mk.mk_sync(self.h, 0)
        if rc != mk.MK_OK:
            raise mk.MkError(rc, mk.mk_last_error())
        return out

    def trace(self):
        return (self.t_ids.cpu().numpy(), self.t_w.cpu().numpy(), self.t_logits.cpu().numpy())

    def close(self):
        if self.h is not None:
            mk.mk_destroy(self.h)
            self.h = None


def oracle_walk(stack: DeviceStack, hidden_in, positions, gpu_ids, rows_per_seq=1, kv_hosts=None, progress=None):
    """Teacher-forced oracle pass.  Returns (out fp32, report dict).

    For attention stacks the report's "kv_rows" holds, per layer, the bf16
    rows the oracle wrote into its cache: (k, v) uint16 [M][G][hd], row r at
    sequence r // rows_per_seq and position positions[r].  progress(l), when
    given, is called before layer l."""
    w = stack.w
    dims = dims_of(w)
    h = np.asarray(hidden_in, dtype=np.float64)
    M = h.shape[0]
    rep = dict(forced=0, mismatch=[], margins=[], oracle_ids=[], oracle_w=[], oracle_logits=[], kv_rows=[])
    seqs = [r // rows_per_seq for r in range(M)]
    for l in range(stack.L):
        if progress is not None:
            progress(l)
        need = set(np.unique(gpu_ids[l]).tolist())
        H = stack.host_layer(l, experts=need) if w.E > 16 else stack.host_layer(l)
        ly = oracle_layer(H)
        if w.has_attn:
            if kv_hosts is not None:
                kh, vh = kv_hosts[l]
            else:
                kh, vh = stack.host_kv(l)
            kv = oracle.OracleKV(kh.copy(), vh.copy())
            h1 = oracle.attn_block(dims, ly, h, positions, kv, rows_per_seq=rows_per_seq)
            rep["kv_rows"].append((np.stack([kv.k[s, :, p] for s, p in zip(seqs, positions)]),
                                   np.stack([kv.v[s, :, p] for s, p in zip(seqs, positions)])))
        else:
            h1 = h
        logits, ids, wts, margin = oracle.route(dims, ly, h1)
        forced = ids.copy()
        any_forced = False
        for r in range(M):
            if set(ids[r].tolist()) != set(gpu_ids[l, r].tolist()):
                if margin[r] > TIE_MARGIN:
                    rep["mismatch"].append((l, r, float(margin[r]), ids[r].tolist(), gpu_ids[l, r].tolist()))
                forced[r] = gpu_ids[l, r]
                any_forced = True
                rep["forced"] += 1
        if any_forced:
            missing = set(forced.ravel().tolist()) - need
            if missing and w.E > 16:
                H = stack.host_layer(l, experts=need | missing)
                ly = oracle_layer(H)
            logits, ids, wts, margin2 = oracle.route(dims, ly, h1, forced=forced)
        rep["margins"].append(margin)
        rep["oracle_logits"].append(logits)
        rep["oracle_ids"].append(ids)
        rep["oracle_w"].append(wts)
        h = oracle.moe_block(dims, ly, h1, ids, wts)
    return h.astype(np.float32), rep


def gpu_kv_rows(stack: DeviceStack, l, positions, rows_per_seq=1, seq0=0):
    """The GPU cache rows of layer l at the step's positions: (k, v) uint16
    [M][G][hd], row r at sequence seq0 + r // rows_per_seq."""
    import torch
    s = torch.as_tensor([seq0 + r // rows_per_seq for r in range(len(positions))], device=stack.kc.device)
    p = torch.as_tensor(np.asarray(positions, dtype=np.int64), device=stack.kc.device)
    k = stack.kc[l][s, :, p]  # [M][G][hd]
    v = stack.vc[l][s, :, p]
    return DeviceStack.to_host(k), DeviceStack.to_host(v)


def bf16_values(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# Appended K/V rows.  At the first layer both sides start from the same
# hidden rows: the GPU rounds its fp32 k, v to bf16 and the oracle its fp64
# values, so the two differ by at most one bf16 step (2^(e-7) for a value in
# [2^e, 2^(e+1))) plus the difference of the unrounded values, which is the
# fp32 projection's error (below 1e-5): one step everywhere above 2^-9 and an
# absolute 2^-16 below.  At later layers the rows are projections of hidden
# states that already differ by up to the stack's output tolerance (a step
# attending one or two positions carries a bf16 rounding of v straight into
# the next layer), so there the bound is one step plus that tolerance's
# max|d|, and the rows' relative L2 error must meet its rel_l2.
KV_ABS_FLOOR = 2.0 ** -16


def kv_row_excess(gpu_bits, oracle_bits, extra=0.0):
    """Worst ratio |gpu - oracle| / (max(one bf16 step of the larger value,
    KV_ABS_FLOOR) + extra) over the rows (<= 1 passes), and the count of
    differing elements."""
    g = bf16_values(gpu_bits)
    o = bf16_values(oracle_bits)
    assert np.isfinite(g).all(), "non-finite value in a GPU cache row"
    mag = np.maximum(np.abs(g), np.abs(o))
    step = np.where(mag > 0, np.exp2(np.floor(np.log2(np.where(mag > 0, mag, 1.0))) - 7), 0.0)
    allowed = np.maximum(step, KV_ABS_FLOOR) + extra
    diff = np.abs(g - o)
    return float(np.max(diff / allowed)), int(np.count_nonzero(diff))


def assert_kv_rows(stack: DeviceStack, rep, positions, rows_per_seq=1, layers=None, what="", tol=TOL_BF16, seq0=0):
    """Every cache row the step wrote (every layer, row and kv head) against
    the oracle's bf16 row: within one bf16 step at the first layer, within one
    step plus tol's max|d| (and tol's rel_l2 over the layer's rows) after it.
    The rows are those of sequences seq0, seq0 + 1, ... of the cache."""
    worst0, worst, ndiff, n = 0.0, 0.0, 0, 0
    for l in (range(stack.L) if layers is None else layers):
        gk, gv = gpu_kv_rows(stack, l, positions, rows_per_seq, seq0)
        ok_, ov_ = rep["kv_rows"][l]
        for name, g, o in (("K", gk, ok_), ("V", gv, ov_)):
            assert g.shape == o.shape, (g.shape, o.shape)
            x, nd = kv_row_excess(g, o, 0.0 if l == 0 else tol["max_abs"])
            assert x <= 1.0, f"{what} layer {l}: {name} rows differ from the oracle by {x:.3g} of the bound"
            if l > 0:
                gd, od = bf16_values(g), bf16_values(o)
                rel = float(np.linalg.norm(gd - od) / np.linalg.norm(od))
                assert rel <= tol["rel_l2"], f"{what} layer {l}: {name} rows rel-L2 {rel:.3g}"
            x1, _ = kv_row_excess(g, o)
            if l == 0:
                worst0 = max(worst0, x1)
            else:
                worst = max(worst, x1)
            ndiff, n = ndiff + nd, n + g.size
    return dict(kv_steps_layer0=worst0, kv_steps_later=worst, kv_differing=ndiff, kv_elements=n)


def assert_routing_weights(ids, wts, logits, rep, M, L, tol=1e-5, what=""):
    """Routing weights of every (layer, row):
    - the GPU's weights sum to 1 and equal the oracle's renormalised softmax
      applied to the GPU's own traced logits at the GPU's experts, within tol
      (this isolates the weight computation from upstream differences);
    - where the expert sets agree, they equal the oracle's weights within
      0.5 * max|logit difference| + tol: the renormalised top-k softmax moves
      each weight by at most 2 w (1 - w) <= 1/2 times the largest logit change
      (to first order)."""
    import oracle
    for l in range(L):
        for r in range(M):
            g = np.asarray(wts[l, r], dtype=np.float64)
            assert abs(float(np.sum(g)) - 1.0) < tol, (what, l, r)
            p = oracle.softmax(np.asarray(logits[l, r], dtype=np.float64))
            sel = p[np.asarray(ids[l, r], dtype=np.int64)]
            own = sel / np.sum(sel)
            err = float(np.max(np.abs(g - own)))
            assert err < tol, (what, l, r, "weights vs renormalised softmax of the traced logits", err)
            if set(ids[l, r].tolist()) == set(rep["oracle_ids"][l][r].tolist()):
                dz = float(np.max(np.abs(np.asarray(logits[l, r], dtype=np.float64) - rep["oracle_logits"][l][r])))
                go = {int(e): float(x) for e, x in zip(ids[l, r], wts[l, r])}
                oo = {int(e): float(x) for e, x in zip(rep["oracle_ids"][l][r], rep["oracle_w"][l][r])}
                for e in go:
                    assert abs(go[e] - oo[e]) <= 0.5 * dz + tol, (what, l, r, e, go[e], oo[e], dz)


def compare(gpu_out, ref_out):
    g = np.asarray(gpu_out, dtype=np.float64)
    r = np.asarray(ref_out, dtype=np.float64)
    diff = g - r
    return dict(max_abs=float(np.max(np.abs(diff))), rel_l2=float(np.linalg.norm(diff) / np.linalg.norm(r)))


def assert_close(gpu_out, ref_out, tol, what=""):
    c = compare(gpu_out, ref_out)
    assert c["max_abs"] <= tol["max_abs"] and c["rel_l2"] <= tol["rel_l2"], f"{what}: {c} vs {tol}"
    return c
