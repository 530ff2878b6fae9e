"""Decode-step benchmark of the MI355X MoE megakernel (one GPU).

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Workload (synthetic, seeded): the 92-layer stack, d=4096, 64 routed experts
top-8 + 1 shared expert (F=1024, SwiGLU), GQA attention (32 q heads, 8 kv
heads, head_dim 128, RoPE theta 1e6) over a bf16 KV cache of 4096 past
positions; bf16 weights N(0, 0.02) (158 GB resident in HBM, far above the
256 MB Infinity Cache), fp32 accumulation.  Each step feeds its output back
as the next step's input and advances the positions.

Prints ONE JSON line.  value = decode tokens/s at batch 1 (whole job, one
GPU).  The batch-8 figures over the same weights are reported under
"batch8".  roofline: algorithmic bytes of one step (attention weights, router
weights, union of activated experts + shared expert, KV read) divided by the
kernel's average duration from HIP events on its stream, against 8 TB/s.
cpu_baseline: the CPU oracle timed on a bounded sample of layers of the same
step, scaled to tokens/s.

Other legs, reported beside the headline: batch 8 over the same weights; the
verify pass (1 and 8 sequences x 8 rows); speculative decoding around the
verify pass with a synthetic acceptance process (effective tokens/s at about
6 tokens per step); the same step as one kernel launch per phase of every
layer (the many-kernels baseline, batch 1 and 8, and at batch 1 replayed
from a HIP graph); the 16-layer MoE-only stack at batch 1 and 8; the MLA
attention over a latent cache (include/mk_mla.h) at 1, 8 and 8 x 8 rows.

HBM traffic (roofline.traffic) comes from two rocprofv3 counter passes over
this script with --calib-copy-mib, one with --pmc FETCH_SIZE and one with
--pmc WRITE_SIZE; `python bench.py --parse-pmc FETCH_DIR WRITE_DIR` reads
their CSV output, scales each counter by what it reads for the calibration
copy (a plain device-to-device copy of known size) and writes
profiles/traffic_attn92_b1.json, which later runs report while the kernel
sources are unchanged.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
METRIC = "decode tokens/s at batch 1 and 8; achieved HBM GB/s as % of MI355X peak"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_hash():
    """Hash of the decode kernel's sources (the mk_* files): counter records
    taken on other sources are not reported."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(os.path.join(ROOT, "moe_layer_stack_amd", "csrc"))):
        if not f.startswith("mk_"):
            continue
        with open(os.path.join(ROOT, "moe_layer_stack_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def step_bytes(w, M, n_seq, union_per_layer, kv_read_positions):
    """Algorithmic bytes of one step: weights that must be streamed (attention,
    router, union of routed experts + shared) plus KV rows read."""
    es = 2 if w.dtype == 1 else 4
    be = 3 * w.d * w.F * es
    attn = (2 * w.d * w.H * w.hd + 2 * w.d * w.G * w.hd) * es if w.has_attn else 0
    router = w.d * w.E * es
    total = 0
    for u in union_per_layer:
        total += attn + router + (u + w.n_shared) * be
    if w.has_attn:
        total += len(union_per_layer) * kv_read_positions * 2 * w.G * w.hd * 2
    return total


def run_leg(torch, mk, st, w, M, rows_per_seq, steps, warmup, trace_union, flush=None, phased=False):
    """Time `steps` decode steps of batch M (after `warmup`).  Returns dict.

    flush: (src, dst) device buffers; when given, dst.copy_(src) runs on the
    stream before every launch, outside the events that time the launch, so
    each step starts with nothing of the stack in the Infinity Cache or L2.
    phased: run the step as one launch per phase of every layer
    (mk_decode_step_phased) instead of the persistent kernel."""
    import numpy as np
    cfg = st.config(rows=M, rows_per_seq=rows_per_seq)
    h = mk.mk_create(cfg, st.layer_weights())
    info = mk.mk_get_info(h)
    stream = torch.cuda.current_stream()
    n_seq = M // rows_per_seq
    total = warmup + steps
    p0 = w.past
    pos = np.array([[p0 + t * rows_per_seq + (r % rows_per_seq) for r in range(M)] for t in range(total)],
                   dtype=np.int32)
    pos_d = torch.as_tensor(pos, device="cuda")
    bufs = [st.hidden(0, rows=M), torch.empty(M, w.d, dtype=torch.float32, device="cuda")]
    kv = st.kv()
    ids = torch.zeros(total, st.L, M, w.k, dtype=torch.int32, device="cuda") if trace_union else None
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    sp = stream.cuda_stream
    for t in range(total):
        if trace_union:
            mk.mk_set_trace(h, ids[t].data_ptr(), 0, 0)
        timed = t >= warmup
        if t == warmup:
            torch.cuda.synchronize()
            t_wall0 = time.perf_counter()
        if flush is not None:
            flush[1].copy_(flush[0])
        if timed:
            ev[t - warmup][0].record(stream)
        step_fn = mk.mk_decode_step_phased if phased else mk.mk_decode_step
        step_fn(h, bufs[t % 2].data_ptr(), pos_d[t].data_ptr(), kv, bufs[(t + 1) % 2].data_ptr(), sp)
        if timed:
            ev[t - warmup][1].record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    rc = mk.mk_sync(h, sp)
    if rc != mk.MK_OK:
        raise mk.MkError(rc, mk.mk_last_error())
    durs = np.array([a.elapsed_time(b) for a, b in ev])  # ms, per launch
    tasks = None
    if trace_union:
        idn = ids.cpu().numpy()
        unions = [[len(np.unique(idn[t, l])) for l in range(st.L)] for t in range(total)]
        if M > 8:  # row groups in one launch: routed tasks of at most 8 rows per expert
            tasks = float(np.mean([sum(-(-int(c) // 8) for c in np.bincount(idn[t, l].ravel(), minlength=w.E))
                                   for t in range(warmup, total) for l in range(st.L)]))
    else:
        unions = [[w.k] * st.L for _ in range(total)]
    byts = [step_bytes(w, M, n_seq, unions[t], 0) + st.L * n_seq * (int(pos[t].max()) + 1) * 2 * w.G * w.hd * 2
            for t in range(warmup, total)]
    mk.mk_destroy(h)
    ms = float(durs.mean())
    gbps = float(np.mean(byts)) / (ms * 1e-3) / 1e9
    finite = bool(torch.isfinite(bufs[total % 2]).all().item())
    union_layers = [round(float(np.mean([unions[t][l] for t in range(warmup, total)])), 2) for l in range(st.L)]
    n_groups = max(1, M // 8)
    launches = (n_groups * st.L * ((6 if w.has_attn else 3) + (1 if M > 1 else 0)) if phased
                else info.launches_per_step)
    return dict(M=M, ms_per_step=ms, ms_median=float(np.median(durs)), ms_p10=float(np.percentile(durs, 10)),
                ms_p90=float(np.percentile(durs, 90)),
                wall_ms_per_step=t_wall * 1e3 / steps, tok_s=M / (ms * 1e-3), bytes_per_step=float(np.mean(byts)),
                achieved_gbps=gbps, frac=gbps / PEAK_HBM_GBPS,
                union_mean=float(np.mean([np.mean(u) for u in unions[warmup:]])), barriers=info.barriers_per_step,
                finite=finite, union_per_layer=union_layers if trace_union else None, launches=launches,
                **({"tasks_per_layer": tasks} if tasks is not None else {}))


def spec_leg(torch, mk, st, w, n_seq, steps, warmup, alpha=0.9155, seed=5):
    """Speculative decoding around the verify step, with a synthetic acceptance
    process: each step runs 8 rows per sequence (the last accepted token and
    7 drafts) at positions p .. p+7; each draft is accepted with probability
    alpha until the first rejection, so a step yields 1 + a tokens (a <= 7,
    mean 6.0 at alpha 0.9155) and the sequence continues at p + 1 + a.  The
    rejected drafts' cache entries are overwritten by the next step's rows
    before they could be read, which is the rollback.  effective tok/s =
    tokens yielded / time of the timed steps (HIP events around each launch)."""
    import numpy as np
    rng = np.random.default_rng(seed)
    M = 8 * n_seq
    cfg = st.config(rows=M, rows_per_seq=8)
    h = mk.mk_create(cfg, st.layer_weights())
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    bufs = [st.hidden(100 + i, rows=M) for i in range(2)]
    out = torch.empty(M, w.d, dtype=torch.float32, device="cuda")
    kv = st.kv()
    p = np.full(n_seq, w.past, dtype=np.int64)
    ev, toks = [], []
    for t in range(warmup + steps):
        pos = np.array([p[s] + r for s in range(n_seq) for r in range(8)], dtype=np.int32)
        if pos.max() >= w.capacity:
            raise SystemExit("spec leg: KV capacity too small for the steps asked")
        pos_d = torch.as_tensor(pos, device="cuda")
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        mk.mk_decode_step(h, bufs[t % 2].data_ptr(), pos_d.data_ptr(), kv, out.data_ptr(), sp)
        b.record(stream)
        acc = np.zeros(n_seq, dtype=np.int64)
        for s in range(n_seq):
            while acc[s] < 7 and rng.random() < alpha:
                acc[s] += 1
        p += 1 + acc
        if t >= warmup:
            ev.append((a, b))
            toks.append(int((1 + acc).sum()))
    torch.cuda.synchronize()
    rc = mk.mk_sync(h, sp)
    mk.mk_destroy(h)
    if rc != mk.MK_OK:
        raise mk.MkError(rc, mk.mk_last_error())
    ms = float(np.mean([x.elapsed_time(y) for x, y in ev]))
    return dict(sequences=n_seq, rows=M, ms_per_step=ms, tokens_per_step=float(np.mean(toks)) / n_seq,
                effective_tok_s=float(np.sum(toks)) / (ms * 1e-3 * len(ev)), accept_alpha=alpha,
                finite=bool(torch.isfinite(out).all().item()))


def graph_leg(torch, mk, st, w, M, steps, warmup):
    """The one-launch-per-phase step captured once into a HIP graph and
    replayed: the launches keep their boundaries (no prefetch across them)
    but lose the host's launch gaps.  Each replay is timed by events on the
    replay stream."""
    import numpy as np
    h = mk.mk_create(st.config(rows=M, rows_per_seq=1), st.layer_weights())
    s = torch.cuda.Stream()
    hin = st.hidden(0, rows=M)
    hout = torch.empty_like(hin)
    pos = torch.tensor([w.past] * M, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        mk.mk_decode_step_phased(h, hin.data_ptr(), pos.data_ptr(), st.kv(), hout.data_ptr(), s.cuda_stream)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        mk.mk_decode_step_phased(h, hin.data_ptr(), pos.data_ptr(), st.kv(), hout.data_ptr(), s.cuda_stream)
    torch.cuda.synchronize()
    ev = []
    for t in range(warmup + steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(s):
            a.record(s)
            g.replay()
            b.record(s)
        if t >= warmup:
            ev.append((a, b))
    torch.cuda.synchronize()
    rc = mk.mk_sync(h, 0)
    del g
    mk.mk_destroy(h)
    if rc != mk.MK_OK:
        raise mk.MkError(rc, mk.mk_last_error())
    return float(np.mean([a.elapsed_time(b) for a, b in ev]))


def moe16_legs(torch, mk, steps, warmup):
    """The 16-layer MoE-only stack (d=2048, 64 experts top-6 + 1 shared,
    F=1024, router bias): batch 1 and batch 8, each step fed the previous
    step's output.  Its 13 GB of weights are far larger than the Infinity
    Cache, but a step touches only 1.4 GB (batch 1), of which the shared
    experts and routers (205 MB) are the same every step; so each launch is
    timed after a 1 GiB device copy that evicts the caches, and a
    back-to-back run without the copy is reported as the control."""
    from synth.stack import DeviceStack
    from synth.workloads import MOE16_B8
    st = DeviceStack(MOE16_B8)
    torch.cuda.synchronize()
    n = (1 << 30) // 4
    flush = (torch.ones(n, dtype=torch.float32, device="cuda"), torch.empty(n, dtype=torch.float32, device="cuda"))
    out = {}
    for name, M in (("moe16_b1", 1), ("moe16_b8", 8)):
        w = MOE16_B8.with_(name=name, M=M)
        r = run_leg(torch, mk, st, w, M, 1, steps, warmup, trace_union=True, flush=flush)
        ctl = run_leg(torch, mk, st, w, M, 1, steps, warmup, trace_union=False)
        r["unflushed_ms_per_step"] = ctl["ms_per_step"]
        if M == 1:
            r.pop("union_per_layer")
        log(f"{name}: {r['ms_per_step'] * 1e3:.1f} us/step flushed ({ctl['ms_per_step'] * 1e3:.1f} back-to-back), "
            f"{r['tok_s']:.0f} tok/s, {r['achieved_gbps']:.0f} GB/s ({100 * r['frac']:.1f}% of peak), "
            f"union {r['union_mean']:.1f}")
        out[name] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}
    del st, flush
    torch.cuda.empty_cache()
    return out


def mla_legs(torch, steps, warmup):
    """MLA attention at decode over a latent cache (include/mk_mla.h; H=64
    heads, latent 512 + rotary 64 per cache row, bf16): one call = the split
    and combine launches.  Shapes: 1 sequence at 4096 past positions, 8
    sequences, 8 sequences x 8 verify rows, and 1 sequence at 32768.  Each
    timed call follows a 1 GiB device copy (outside the events) so the cache
    is read from HBM; a back-to-back run is the control.  Bytes: the cache
    rows read plus queries and outputs."""
    import numpy as np
    import synth
    from moe_layer_stack_amd import mla
    H, DK, DC = 64, mla.MLA_LATENT_DIM + mla.MLA_ROPE_DIM, mla.MLA_LATENT_DIM
    n = (1 << 30) // 4
    flush = (torch.ones(n, dtype=torch.float32, device="cuda"), torch.empty(n, dtype=torch.float32, device="cuda"))
    out = {}
    for name, rows, rps, n_seq, cap, p0 in (("mla_b1", 1, 1, 1, 4160, 4096), ("mla_b8", 8, 1, 8, 4160, 4096),
                                             ("mla_verify64", 64, 8, 8, 4160, 4096),
                                             ("mla_b1_32k", 1, 1, 1, 32832, 32768)):
        cfg = mla.mk_mla_config(n_heads=H, latent_dim=DC, rope_dim=DK - DC, rows=rows, rows_per_seq=rps, n_seq=n_seq,
                                capacity=cap, scale=float(1.0 / np.sqrt(128 + DK - DC)))
        h = mla.mk_mla_create(cfg)
        info = mla.mk_mla_get_info(h)
        cache = torch.empty(n_seq, cap, DK, dtype=torch.bfloat16, device="cuda")
        synth.device_normal(cache.data_ptr(), cache.numel(), synth.BF16, 9, synth.stream_id(-1, synth.K_MLA_CACHE))
        q = torch.empty(rows, H, DK, dtype=torch.float32, device="cuda")
        synth.device_normal(q.data_ptr(), q.numel(), synth.F32, 9, synth.stream_id(-1, synth.K_MLA_Q), 0.0, 0.25)
        pos = torch.tensor([p0 + r % rps for r in range(rows)], dtype=torch.int32, device="cuda")
        o = torch.empty(rows, H, DC, dtype=torch.float32, device="cuda")
        stream = torch.cuda.current_stream()
        res = {}
        for tag, fl in (("flushed", True), ("back_to_back", False)):
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
            for t in range(warmup + steps):
                if fl:
                    flush[1].copy_(flush[0])
                if t >= warmup:
                    ev[t - warmup][0].record(stream)
                mla.mk_mla_attention(h, q.data_ptr(), cache.data_ptr(), pos.data_ptr(), o.data_ptr(),
                                     stream.cuda_stream)
                if t >= warmup:
                    ev[t - warmup][1].record(stream)
            rc = mla.mk_mla_sync(h, stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"{name}: mk_mla_sync returned {rc}")
            res[tag] = float(np.mean([a.elapsed_time(b) for a, b in ev]))
        mla.mk_mla_destroy(h)
        n_rows_read = (p0 + rps) * n_seq  # each sequence's rows 0 .. its last position, read once
        byts = n_rows_read * DK * 2 + q.numel() * 4 + o.numel() * 4
        ms = res["flushed"]
        gbps = byts / (ms * 1e-3) / 1e9
        r = dict(rows=rows, rows_per_seq=rps, sequences=n_seq, past_positions=p0, heads=H, splits=info.splits,
                 workgroups=info.workgroups, launches=2, ms_per_call=ms, unflushed_ms_per_call=res["back_to_back"],
                 bytes_per_call=float(byts), achieved_gbps=gbps, frac=gbps / PEAK_HBM_GBPS,
                 finite=bool(torch.isfinite(o).all().item()))
        log(f"{name}: {ms * 1e3:.1f} us per call flushed ({res['back_to_back'] * 1e3:.1f} back-to-back), "
            f"{byts / 1e6:.1f} MB, {gbps:.0f} GB/s ({100 * r['frac']:.1f}% of peak), {info.workgroups} workgroups")
        out[name] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}
        del cache, q, o
    del flush
    torch.cuda.empty_cache()
    return out


def cpu_model():
    """The host CPU's model name (first processor of /proc/cpuinfo) and the
    number of processors the process may run on."""
    name = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    name = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count()
    return name, n


def gpu_step_b1(torch, mk, st, w):
    """One batch-1 step of the decode kernel on the input the CPU leg uses
    (row 0 of hidden(0), position w.past, sequence 0 of the cache), with its
    routing traced: (output [1][d] fp64, expert ids [L][1][k])."""
    import numpy as np
    h = mk.mk_create(st.config(rows=1, rows_per_seq=1), st.layer_weights())
    try:
        ids = torch.zeros(st.L, 1, w.k, dtype=torch.int32, device="cuda")
        mk.mk_set_trace(h, ids.data_ptr(), 0, 0)
        x = st.hidden(0)[:1].contiguous()
        out = torch.empty_like(x)
        pos = torch.tensor([w.past], dtype=torch.int32, device="cuda")
        mk.mk_decode_step(h, x.data_ptr(), pos.data_ptr(), st.kv(), out.data_ptr(), 0)
        rc = mk.mk_sync(h, 0)
        if rc != mk.MK_OK:
            raise mk.MkError(rc, mk.mk_last_error())
        return out.cpu().numpy().astype(np.float64), ids.cpu().numpy()
    finally:
        mk.mk_destroy(h)


def cpu_baseline(torch, st, w, n_layers_sample, threads=None, gpu=None):
    """The CPU oracle (as it stands) on the first layers of a batch-1 step:
    host copies of the touched tensors are made before the timer starts.
    threads: the oracle's thread count for this sample (default: all).
    gpu: (output, expert ids) of the same step on the GPU (gpu_step_b1); with
    the whole step sampled, the result then carries a parity verdict of the
    GPU output against the oracle's (which routes by itself)."""
    import numpy as np
    import oracle
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from parity_util import dims_of, oracle_layer
    dims = dims_of(w)
    all_threads = oracle.num_threads()
    used = oracle.set_threads(threads) if threads else all_threads
    h = st.hidden(0)[:1].cpu().numpy().astype(np.float64)
    pos = [w.past]
    t_compute = 0.0
    ids_differ = []
    for l in range(n_layers_sample):
        H = st.host_layer(l, experts=[])  # attention, router, shared
        kv = oracle.OracleKV(st.to_host(st.kc[l, :1]), st.to_host(st.vc[l, :1]))
        ly = oracle_layer(H)
        t0 = time.perf_counter()
        h1 = oracle.attn_block(dims, ly, h, pos, kv)
        _, ids, wts, _ = oracle.route(dims, ly, h1)
        t_compute += time.perf_counter() - t0
        if gpu is not None and set(np.asarray(ids[0]).tolist()) != set(gpu[1][l, 0].tolist()):
            ids_differ.append(l)
        H = st.host_layer(l, experts=ids[0])
        ly = oracle_layer(H)
        t0 = time.perf_counter()
        h = oracle.moe_block(dims, ly, h1, ids, wts)
        t_compute += time.perf_counter() - t0
    if threads:
        oracle.set_threads(all_threads)
    per_layer = t_compute / n_layers_sample
    step_s = per_layer * w.L
    model, n_avail = cpu_model()
    res = dict(value=1.0 / step_s, unit="tokens/s", cores=used, kind="oracle", cpu_model=model,
               cpus_available=n_avail,
               sample=f"first {n_layers_sample} of {w.L} layers of one batch-1 step (fp64 C oracle, OpenMP over "
                      f"output rows); compute time {t_compute:.1f} s, scaled by {w.L}/{n_layers_sample}")
    if gpu is not None and n_layers_sample == w.L:
        from parity_util import compare, tolerances
        c = compare(gpu[0], h)
        tol = tolerances(w)
        res["parity"] = dict(rows=1, layers=w.L, max_abs=c["max_abs"], rel_l2=c["rel_l2"],
                             tol_max_abs=tol["max_abs"], tol_rel_l2=tol["rel_l2"],
                             expert_sets_differ=len(ids_differ), first_differing_layer=(ids_differ or [None])[0],
                             ok=bool(c["max_abs"] <= tol["max_abs"] and c["rel_l2"] <= tol["rel_l2"]
                                     and not ids_differ))
    return res


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_attn92_b1.json")
KERNEL_B1 = "decode_step_kernel<unsigned short, 1, 1>"


def _pmc_rows(d, counter):
    """(kernel name, value) of every dispatch in the rocprofv3 counter CSVs under d."""
    import csv
    rows = []
    for dirpath, _, files in os.walk(d):
        for f in files:
            if not f.endswith("counter_collection.csv"):
                continue
            with open(os.path.join(dirpath, f), newline="") as fh:
                for r in csv.DictReader(fh):
                    if r.get("Counter_Name") == counter:
                        rows.append((r.get("Kernel_Name", ""), float(r.get("Counter_Value", "nan"))))
    return rows


def parse_pmc(fetch_dir, write_dir, copy_mib, kernel="1, 1>", out_file=TRAFFIC_FILE):
    """Per-launch HBM bytes of a decode kernel (the instantiation whose name
    contains `kernel`; by default the batch-1 kernel) from FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), each scaled by the counter's reading for
    the calibration copy of copy_mib MiB (read once, written once).  Every
    dispatch of that kernel in the runs counts (warm-up included), so each
    pass should run one leg (--only)."""
    import numpy as np
    out = {"source_hash": source_hash(), "copy_mib": copy_mib, "kernel": kernel}
    for name, d in (("fetch", fetch_dir), ("write", write_dir)):
        counter = "FETCH_SIZE" if name == "fetch" else "WRITE_SIZE"
        rows = _pmc_rows(d, counter)
        kern = [v for k, v in rows if "decode_step_kernel" in k and kernel in k]
        copies = [v for k, v in rows if "copy" in k.lower()]
        if not kern or not copies:
            raise SystemExit(f"{counter}: no decode-kernel or copy dispatches under {d}")
        copy_kib = max(copies)  # the calibration copy is the largest copy dispatch
        scale = copy_mib * 1024.0 / copy_kib
        out[f"{name}_kib_per_launch"] = float(np.mean(kern))
        out[f"{name}_copy_kib"] = copy_kib
        out[f"{name}_scale"] = scale
        out[f"{name}_bytes_per_launch"] = float(np.mean(kern)) * 1024.0 * scale
        out[f"{name}_launches"] = len(kern)
    out["bytes_per_launch"] = out["fetch_bytes_per_launch"] + out["write_bytes_per_launch"]
    if out_file:
        os.makedirs(os.path.dirname(os.path.abspath(out_file)), exist_ok=True)
        with open(out_file, "w") as fh:
            json.dump(out, fh, indent=1)
    print(json.dumps(out))


def calib_copy(torch, mib):
    """One device-to-device copy of mib MiB (read once, written once): the
    reference dispatch that scales the HBM byte counters."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"calibration copy: {mib} MiB")
    del src, dst


def only_leg(torch, mk, args):
    """One leg by itself (its warm-up and timed steps), then the calibration
    copy: the program of a counter pass, in which every dispatch of the leg's
    kernel instantiation belongs to that leg."""
    from synth.stack import DeviceStack
    from synth.workloads import ATTN92_B8, MOE16_B8
    leg = args.only
    if leg == "mla":
        r = mla_legs(torch, args.steps, args.warmup)
        if args.calib_copy_mib:
            calib_copy(torch, args.calib_copy_mib)
        print(json.dumps({"leg": leg, **r}), flush=True)
        return
    if leg.startswith("moe16"):
        M = 1 if leg == "moe16_b1" else 8
        st = DeviceStack(MOE16_B8, n_layers=args.layers)
        w = MOE16_B8.with_(name=leg, M=M)
        r = run_leg(torch, mk, st, w, M, 1, args.steps, args.warmup, trace_union=M > 1)
    else:
        M, rps = {"batch1": (1, 1), "batch8": (8, 1), "verify8": (8, 8), "verify64": (64, 8),
                  "phased_b1": (1, 1)}[leg]
        w8 = ATTN92_B8.with_(cap_extra=max(64, 8 * (args.warmup + args.steps + 2)))
        st = DeviceStack(w8, n_layers=args.layers)
        w = w8.with_(M=M, rows_per_seq=rps)
        r = run_leg(torch, mk, st, w, M, rps, args.steps, args.warmup, trace_union=M > 1,
                    phased=leg.startswith("phased"))
    log(f"{leg}: {r['ms_per_step']:.3f} ms/step, {r['achieved_gbps']:.0f} GB/s algorithmic "
        f"({100 * r['frac']:.1f}% of peak), {r['launches']} launch(es) per step")
    if args.calib_copy_mib:
        calib_copy(torch, args.calib_copy_mib)
    r.pop("union_per_layer", None)
    print(json.dumps({"leg": leg, "layers": st.L, "source_hash": source_hash(),
                      **{k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}}), flush=True)
    torch.cuda.synchronize()
    del st
    torch.cuda.empty_cache()
    torch.cuda.synchronize()


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-batch8", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-verify", action="store_true", help="skip the 8- and 64-row verify and speculative legs")
    ap.add_argument("--no-moe16", action="store_true", help="skip the 16-layer MoE-only legs")
    ap.add_argument("--no-phased", action="store_true", help="skip the one-launch-per-phase baseline legs")
    ap.add_argument("--no-mla", action="store_true", help="skip the MLA attention legs")
    ap.add_argument("--moe16-steps", type=int, default=256, help="timed steps of the 16-layer legs")
    ap.add_argument("--cpu-layers", type=int, default=92, help="layers in the CPU-oracle sample (default: a whole step)")
    ap.add_argument("--cpu-layers-1t", type=int, default=12,
                    help="layers in the single-thread CPU-oracle sample (0: skip it)")
    ap.add_argument("--layers", type=int, default=None, help="stack depth (default: the workload's 92)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after the timed legs, one device copy of this size (counter calibration)")
    ap.add_argument("--maps-out", default=None,
                    help="after the teardown, copy /proc/self/maps to this file (to name the owner of an address "
                         "in a crash report at exit)")
    ap.add_argument("--only", choices=["batch1", "batch8", "verify8", "verify64", "moe16_b1", "moe16_b8", "mla",
                                       "phased_b1"],
                    default=None, help="run only this leg (and --calib-copy-mib), print its record as JSON: the "
                                       "program of a counter pass")
    ap.add_argument("--pmc-kernel", default="1, 1>",
                    help="with --parse-pmc: the decode-kernel instantiation to count (a substring of its name)")
    ap.add_argument("--pmc-out", default=TRAFFIC_FILE, help="with --parse-pmc: the record's file ('' for none)")
    ap.add_argument("--parse-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the traffic record from two rocprofv3 --pmc runs and exit")
    args = ap.parse_args()
    if args.parse_pmc:
        parse_pmc(args.parse_pmc[0], args.parse_pmc[1], args.calib_copy_mib or 1024, args.pmc_kernel,
                  args.pmc_out)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the decode kernel runs on a single MI355X and the library has no "
              f"multi-GPU path (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(2)
    import moe_layer_stack_amd as mk
    from moe_layer_stack_amd import build
    if not os.path.exists(build.LIB):
        build.build()
    import synth
    from synth.stack import DeviceStack
    from synth.workloads import ATTN92_B8
    if not os.path.exists(synth.LIB):
        synth.build()
    if args.only:
        only_leg(torch, mk, args)
        return
    need = args.warmup + args.steps
    n_seq = 1 if args.no_batch8 else 8
    w8 = ATTN92_B8.with_(cap_extra=max(64, 8 * (need + 2)), M=n_seq)  # room for 8 positions per spec step
    t0 = time.perf_counter()
    def prog(l):
        if l % 16 == 0:
            torch.cuda.synchronize()
            log(f"filling layer {l} ({time.perf_counter() - t0:.0f} s)")
    st = DeviceStack(w8, n_layers=args.layers, progress=prog)
    torch.cuda.synchronize()
    log(f"stack: {st.L} layers, {sum(t.numel() * t.element_size() for ly in st.layers for t in ly.values() if t is not None) / 1e9:.1f} GB "
        f"weights + {2 * st.kc.numel() * 2 / 1e9:.1f} GB KV, built in {time.perf_counter() - t0:.1f} s")
    w1 = w8.with_(M=1)
    b1 = run_leg(torch, mk, st, w1, 1, 1, args.steps, args.warmup, trace_union=False)
    log(f"batch 1: {b1['ms_per_step']:.3f} ms/step, {b1['tok_s']:.1f} tok/s, {b1['achieved_gbps']:.0f} GB/s "
        f"({100 * b1['frac']:.1f}% of peak)")
    b8 = None
    if not args.no_batch8:
        b8 = run_leg(torch, mk, st, w8, 8, 1, args.steps, args.warmup, trace_union=True)
        log(f"batch 8: {b8['ms_per_step']:.3f} ms/step, {b8['tok_s']:.1f} tok/s, {b8['achieved_gbps']:.0f} GB/s "
            f"({100 * b8['frac']:.1f}% of peak), union {b8['union_mean']:.1f}")
    # The legs after the headline ones are reported beside it; a failure in
    # one is logged and recorded, and does not cost the headline line.
    failed = {}

    def optional(name, fn):
        try:
            fn()
        except Exception as e:  # noqa: BLE001
            log(f"{name} failed: {e!r}")
            failed[name] = repr(e)[:300]

    verify = {}

    def verify_legs():
        vsteps = min(args.steps, 5)
        for M in ((8, 64) if st.w.n_seq >= 8 else (8,)):
            wv = w8.with_(M=M, rows_per_seq=8)
            v = run_leg(torch, mk, st, wv, M, 8, vsteps, 1, trace_union=True)
            log(f"verify {M // 8} x 8 rows: {v['ms_per_step']:.3f} ms/step, {v['tok_s']:.1f} rows/s, "
                f"{v['achieved_gbps']:.0f} GB/s algorithmic ({100 * v['frac']:.1f}% of peak), union {v['union_mean']:.1f}")
            v["rows_s"] = v.pop("tok_s")
            verify[f"verify{M}"] = {k: (round(x, 4) if isinstance(x, float) else x) for k, x in v.items()}

    def spec_legs():
        for n_sp in ((1, 8) if st.w.n_seq >= 8 else (1,)):
            sp_steps = args.steps if n_sp == 1 else min(args.steps, 10)
            r = spec_leg(torch, mk, st, w8, n_sp, sp_steps, 1)
            log(f"speculative, {n_sp} sequence(s) x 8 rows: {r['ms_per_step']:.3f} ms/step, "
                f"{r['tokens_per_step']:.2f} tokens per sequence and step, {r['effective_tok_s']:.1f} effective tok/s")
            verify[f"spec{8 * n_sp}"] = {k: (round(x, 4) if isinstance(x, float) else x) for k, x in r.items()}

    if not args.no_verify:
        optional("verify", verify_legs)
        optional("speculative", spec_legs)
    phased = {}

    def phased_legs():
        # the same step as one kernel launch per phase of every layer: the
        # many-kernels execution the persistent kernel replaces
        for name, M, wl in (("phased_b1", 1, w1), ("phased_b8", 8, w8)):
            if M > st.w.n_seq:
                continue
            r = run_leg(torch, mk, st, wl, M, 1, min(args.steps, 10), 2, trace_union=M > 1, phased=True)
            r.pop("union_per_layer", None)
            ref = b1 if M == 1 else b8
            r["persistent_ms_per_step"] = ref["ms_per_step"] if ref else None
            log(f"{name}: {r['ms_per_step']:.3f} ms/step as {r['launches']} launches, {r['tok_s']:.1f} tok/s "
                f"({100 * r['frac']:.1f}% of peak); the persistent kernel: "
                f"{ref['ms_per_step'] if ref else float('nan'):.3f} ms/step")
            phased[name] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}

    def graph_legs():
        g_ms = graph_leg(torch, mk, st, w1, 1, min(args.steps, 10), 2)
        log(f"phased_b1 replayed from a HIP graph: {g_ms:.3f} ms/step ({g_ms / b1['ms_per_step']:.2f} x the "
            f"persistent kernel)")
        phased["phased_graph_b1"] = {"ms_per_step": round(g_ms, 4), "tok_s": round(1e3 / g_ms, 3),
                                     "launches": phased["phased_b1"]["launches"] if "phased_b1" in phased else None}

    if not args.no_phased:
        optional("phased", phased_legs)
        optional("phased_graph", graph_legs)
    moe16 = {}
    if not args.no_moe16:
        optional("moe16", lambda: moe16.update(moe16_legs(torch, mk, args.moe16_steps, args.warmup)))
    mla_res = {}
    if not args.no_mla:
        optional("mla", lambda: mla_res.update(mla_legs(torch, min(args.steps, 20), args.warmup)))
    cpu = None
    if not args.no_cpu_baseline:
        def cpu_leg():
            nonlocal cpu
            gpu = gpu_step_b1(torch, mk, st, w1)
            t0 = time.perf_counter()
            cpu = cpu_baseline(torch, st, w1, min(args.cpu_layers, st.L), gpu=gpu)
            log(f"cpu oracle: {cpu['value']:.3f} tok/s on {cpu['cores']} threads ({time.perf_counter() - t0:.1f} s)")
            if "parity" in cpu:
                pv = cpu["parity"]
                log(f"parity of the batch-1 step against the oracle ({pv['layers']} layers): max_abs "
                    f"{pv['max_abs']:.2e}, rel_l2 {pv['rel_l2']:.2e}, expert sets differing in "
                    f"{pv['expert_sets_differ']} layers, {'ok' if pv['ok'] else 'NOT ok'}")
            if args.cpu_layers_1t > 0:
                t0 = time.perf_counter()
                one = cpu_baseline(torch, st, w1, min(args.cpu_layers_1t, st.L), threads=1)
                cpu["single_thread"] = {k: one[k] for k in ("value", "unit", "cores", "sample")}
                log(f"cpu oracle, one thread: {one['value']:.4f} tok/s ({time.perf_counter() - t0:.1f} s)")
        optional("cpu_baseline", cpu_leg)
    if args.calib_copy_mib:
        calib_copy(torch, args.calib_copy_mib)
    traffic = None
    tf = TRAFFIC_FILE
    if os.path.exists(tf):
        try:
            rec = json.load(open(tf))
            if rec.get("source_hash") == source_hash():
                traffic = rec.get("bytes_per_launch")
        except (OSError, ValueError):
            traffic = None
    out = {
        "metric": METRIC,
        "value": round(b1["tok_s"], 3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(b1["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "attn92_b1", "layers": st.L, "d_model": w1.d, "experts": w1.E, "top_k": w1.k,
                   "shared_experts": w1.n_shared, "d_ff": w1.F, "q_heads": w1.H, "kv_heads": w1.G,
                   "head_dim": w1.hd, "kv_past_positions": w1.past, "batch": 1, "weights_dtype": "bf16",
                   "accumulate": "f32"},
        "roofline": {"bound": "hbm", "achieved": round(b1["achieved_gbps"], 1), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(b1["frac"], 4), "traffic": traffic,
                     "bytes_per_launch": b1["bytes_per_step"]},
        "parity": cpu.pop("parity", None) if cpu else None,
        "cpu_baseline": cpu,
        "batch1": {k: (round(v, 4) if isinstance(v, float) else v) for k, v in b1.items()},
        "batch8": None if b8 is None else {k: (round(v, 4) if isinstance(v, float) else v) for k, v in b8.items()},
    }
    out.update(verify)
    out.update(phased)
    out.update(moe16)
    out.update(mla_res)
    if failed:
        out["failed_legs"] = failed
    print(json.dumps(out), flush=True)
    # Release the device state before the interpreter exits: every handle is
    # already destroyed by its leg; the stack's tensors and torch's cached
    # blocks go here, after the last kernel has finished.
    torch.cuda.synchronize()
    del st
    torch.cuda.empty_cache()
    torch.cuda.synchronize()
    if args.maps_out:
        with open("/proc/self/maps") as src, open(args.maps_out, "w") as dst:
            dst.write(src.read())
    log("teardown done")


if __name__ == "__main__":
    main()
