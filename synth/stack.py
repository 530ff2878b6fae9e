"""A synthetic MoE stack in device memory, filled by the seeded generator.

torch allocates the device memory (plumbing only); the device generator fills
every tensor from its own Philox stream, so the host can regenerate or copy
back any one tensor.  Layout per layer follows include/mk.h: matrices are
[out][in] row-major, experts packed [E][F][d] / [E][d][F]; the KV cache is
[L][n_seq][G][capacity][hd] bf16 for K and for V.

No decode arithmetic lives here.
"""
import numpy as np

from . import (BF16, F32, K_BR, K_G1, K_G2, K_HIDDEN, K_KCACHE, K_SDOWN, K_SGATE, K_SUP, K_VCACHE, K_WDOWN,
               K_WGATE, K_WK, K_WO, K_WQ, K_WR, K_WUP, K_WV, device_normal, device_uniform, host_normal, stream_id)
from .workloads import Workload


def _torch():
    import torch
    return torch


class DeviceStack:
    """Weights (and KV cache) of a workload on the current GPU.

    n_layers overrides the workload's layer count (parity tests on a prefix
    of a deep stack: layer l is the same data whatever n_layers is)."""

    def __init__(self, w: Workload, n_layers=None, device="cuda", fill=True, progress=None):
        torch = _torch()
        self.w = w
        self.L = w.L if n_layers is None else n_layers
        self.device = device
        wdt = torch.bfloat16 if w.dtype == BF16 else torch.float32
        self.wdt = wdt
        self.layers = []
        for l in range(self.L):
            t = {}
            t["g2"] = torch.empty(w.d, dtype=wdt, device=device)
            t["wr"] = torch.empty(w.E, w.d, dtype=wdt, device=device)
            t["br"] = torch.empty(w.E, dtype=torch.float32, device=device) if w.router_bias else None
            t["wg"] = torch.empty(w.E, w.F, w.d, dtype=wdt, device=device)
            t["wu"] = torch.empty(w.E, w.F, w.d, dtype=wdt, device=device)
            t["wd"] = torch.empty(w.E, w.d, w.F, dtype=wdt, device=device)
            if w.n_shared:
                t["sg"] = torch.empty(w.n_shared, w.F, w.d, dtype=wdt, device=device)
                t["su"] = torch.empty(w.n_shared, w.F, w.d, dtype=wdt, device=device)
                t["sd"] = torch.empty(w.n_shared, w.d, w.F, dtype=wdt, device=device)
            if w.has_attn:
                t["g1"] = torch.empty(w.d, dtype=wdt, device=device)
                t["wq"] = torch.empty(w.H * w.hd, w.d, dtype=wdt, device=device)
                t["wk"] = torch.empty(w.G * w.hd, w.d, dtype=wdt, device=device)
                t["wv"] = torch.empty(w.G * w.hd, w.d, dtype=wdt, device=device)
                t["wo"] = torch.empty(w.d, w.H * w.hd, dtype=wdt, device=device)
            self.layers.append(t)
        if w.has_attn:
            shape = (self.L, w.n_seq, w.G, w.capacity, w.hd)
            self.kc = torch.empty(shape, dtype=torch.bfloat16, device=device)
            self.vc = torch.empty(shape, dtype=torch.bfloat16, device=device)
        else:
            self.kc = self.vc = None
        if fill:
            self.fill(progress)

    # ------------------------------------------------------------ generation
    def _dt(self):
        return BF16 if self.w.dtype == BF16 else F32

    def fill(self, progress=None):
        """progress(l) is called after each layer's tensors are enqueued."""
        w, dt, seed = self.w, self._dt(), self.w.weight_seed
        for l, t in enumerate(self.layers):
            if progress is not None:
                progress(l)
            device_uniform(t["g2"].data_ptr(), w.d, dt, seed, stream_id(l, K_G2), 0.9, 1.1)
            device_normal(t["wr"].data_ptr(), t["wr"].numel(), dt, seed, stream_id(l, K_WR), 0.0, w.weight_std)
            if t["br"] is not None:
                device_normal(t["br"].data_ptr(), w.E, F32, seed, stream_id(l, K_BR), 0.0, w.bias_std)
            n = w.F * w.d
            es = t["wg"].element_size()
            for e in range(w.E):
                device_normal(t["wg"].data_ptr() + e * n * es, n, dt, seed, stream_id(l, K_WGATE, e), 0.0, w.weight_std)
                device_normal(t["wu"].data_ptr() + e * n * es, n, dt, seed, stream_id(l, K_WUP, e), 0.0, w.weight_std)
                device_normal(t["wd"].data_ptr() + e * n * es, n, dt, seed, stream_id(l, K_WDOWN, e), 0.0, w.weight_std)
            for s in range(w.n_shared):
                device_normal(t["sg"].data_ptr() + s * n * es, n, dt, seed, stream_id(l, K_SGATE, s), 0.0, w.weight_std)
                device_normal(t["su"].data_ptr() + s * n * es, n, dt, seed, stream_id(l, K_SUP, s), 0.0, w.weight_std)
                device_normal(t["sd"].data_ptr() + s * n * es, n, dt, seed, stream_id(l, K_SDOWN, s), 0.0, w.weight_std)
            if w.has_attn:
                device_uniform(t["g1"].data_ptr(), w.d, dt, seed, stream_id(l, K_G1), 0.9, 1.1)
                for name, kind in (("wq", K_WQ), ("wk", K_WK), ("wv", K_WV), ("wo", K_WO)):
                    device_normal(t[name].data_ptr(), t[name].numel(), dt, seed, stream_id(l, kind), 0.0, w.weight_std)
        if w.has_attn:
            self.fill_kv()

    def fill_kv(self):
        """Past positions of every (layer, sequence): N(0, 1) bf16 over the whole capacity."""
        w = self.w
        per = w.G * w.capacity * w.hd
        for l in range(self.L):
            for s in range(w.n_seq):
                off = ((l * w.n_seq + s) * per) * 2
                device_normal(self.kc.data_ptr() + off, per, BF16, w.input_seed, stream_id(l, K_KCACHE, s), 0.0, 1.0)
                device_normal(self.vc.data_ptr() + off, per, BF16, w.input_seed, stream_id(l, K_VCACHE, s), 0.0, 1.0)

    def hidden(self, step=0, seed=None, rows=None):
        """Step input rows [M][d] fp32 N(0, 1), as a device tensor (rows
        overrides the workload's M; the first rows are the same either way)."""
        torch = _torch()
        h = torch.empty(self.w.M if rows is None else rows, self.w.d, dtype=torch.float32, device=self.device)
        device_normal(h.data_ptr(), h.numel(), F32, self.w.input_seed if seed is None else seed,
                      stream_id(-1, K_HIDDEN, step), 0.0, 1.0)
        return h

    # ------------------------------------------------------------ ABI views
    def layer_weights(self):
        from moe_layer_stack_amd import mk_layer_weights
        out = []
        for t in self.layers:
            def p(name):
                v = t.get(name)
                return v.data_ptr() if v is not None else None
            out.append(mk_layer_weights(p("g1"), p("wq"), p("wk"), p("wv"), p("wo"), p("g2"), p("wr"), p("br"),
                                        p("wg"), p("wu"), p("wd"), p("sg"), p("su"), p("sd")))
        return out

    def config(self, rows=None, rows_per_seq=None):
        from moe_layer_stack_amd import MK_BF16, MK_F32, mk_config
        w = self.w
        return mk_config(self.L, w.d, w.E, w.k, w.n_shared, w.F, MK_BF16 if w.dtype == BF16 else MK_F32,
                         1 if w.router_bias else 0, w.rms_eps, 1 if w.has_attn else 0, w.H, w.G, w.hd,
                         w.rope_theta, w.M if rows is None else rows,
                         w.rows_per_seq if rows_per_seq is None else rows_per_seq, w.capacity)

    def kv(self):
        from moe_layer_stack_amd import mk_kv_cache
        if not self.w.has_attn:
            return None
        return mk_kv_cache(self.kc.data_ptr(), self.vc.data_ptr(), self.w.n_seq, self.w.capacity)

    # ------------------------------------------------------------ host copies
    @staticmethod
    def to_host(t):
        """Device tensor -> numpy (bf16 as uint16 bit patterns)."""
        torch = _torch()
        if t is None:
            return None
        c = t.detach().cpu().contiguous()
        if c.dtype == torch.bfloat16:
            return c.view(torch.int16).numpy().view(np.uint16)
        return c.numpy()

    def host_layer(self, l, experts=None):
        """Numpy arrays of layer l; experts (iterable) limits which routed
        experts are copied (the others are None)."""
        t = self.layers[l]
        w = self.w
        sel = range(w.E) if experts is None else sorted(set(int(e) for e in experts))
        H = {k: self.to_host(t.get(k)) for k in ("g1", "wq", "wk", "wv", "wo", "g2", "wr", "br")}
        wg, wu, wd = [None] * w.E, [None] * w.E, [None] * w.E
        for e in sel:
            wg[e], wu[e], wd[e] = self.to_host(t["wg"][e]), self.to_host(t["wu"][e]), self.to_host(t["wd"][e])
        H["w_gate"], H["w_up"], H["w_down"] = wg, wu, wd
        if w.n_shared:
            H["s_gate"] = [self.to_host(t["sg"][s]) for s in range(w.n_shared)]
            H["s_up"] = [self.to_host(t["su"][s]) for s in range(w.n_shared)]
            H["s_down"] = [self.to_host(t["sd"][s]) for s in range(w.n_shared)]
        else:
            H["s_gate"] = H["s_up"] = H["s_down"] = []
        return H

    def host_kv(self, l):
        """(k, v) numpy uint16 [n_seq][G][capacity][hd] of layer l."""
        return self.to_host(self.kc[l]), self.to_host(self.vc[l])


def host_hidden(w: Workload, step=0, seed=None):
    """The same step input generated on the host."""
    return host_normal((w.M, w.d), F32, w.input_seed if seed is None else seed, stream_id(-1, K_HIDDEN, step))
