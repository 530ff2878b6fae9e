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


def oracle_walk(stack: DeviceStack, hidden_in, positions, gpu_ids, rows_per_seq=1, kv_hosts=None):
    """Teacher-forced oracle pass.  Returns (out fp32, report dict)."""
    w = stack.w
    dims = dims_of(w)
    h = np.asarray(hidden_in, dtype=np.float64)
    M = h.shape[0]
    rep = dict(forced=0, mismatch=[], margins=[], oracle_ids=[], oracle_w=[])
    for l in range(stack.L):
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
        rep["oracle_ids"].append(ids)
        rep["oracle_w"].append(wts)
        h = oracle.moe_block(dims, ly, h1, ids, wts)
    return h.astype(np.float32), rep


def compare(gpu_out, ref_out):
    g = np.asarray(gpu_out, dtype=np.float64)
    r = np.asarray(ref_out, dtype=np.float64)
    diff = g - r
    return dict(max_abs=float(np.max(np.abs(diff))), rel_l2=float(np.linalg.norm(diff) / np.linalg.norm(r)))


def assert_close(gpu_out, ref_out, tol, what=""):
    c = compare(gpu_out, ref_out)
    assert c["max_abs"] <= tol["max_abs"] and c["rel_l2"] <= tol["rel_l2"], f"{what}: {c} vs {tol}"
    return c
