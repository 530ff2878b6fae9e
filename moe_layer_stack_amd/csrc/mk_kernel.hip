// mk_kernel.hip -- the persistent decode kernel for gfx950.
//
// One launch runs a whole decode step through all L layers [P3 "TPU
// Megakernel Achieves 709 tokens/s on Kimi K3, Outpacing GB200", section "The
// Key Innovation: 92 MoE Layers in a Single Pallas Kernel"; P4 tanhow.com
// translation of the authors' post, paragraph on the megakernel: weight loads
// are no longer bound to the kernel that uses them].  The grid is one
// workgroup per CU (256 on MI355X); dependent phases are separated by a grid
// barrier on device-scope atomics.  Per layer:
//
//   QKV   (attention stacks) raw q, k, v rows of [Wq; Wk; Wv] . (h*g1) -> scratch
//   ATTN  split-KV GQA over the bf16 cache; the split owning a new position
//         writes its RoPE'd bf16 k and v row; the last split of each
//         (sequence, kv head) to finish combines the partial softmax states
//   WO    h1 = h + Wo . o
//   RS    router logits and shared-expert gate/up (silu(g) * u)
//   RG    top-k, expert union (every CU, redundantly), routed gate/up rows
//   DOWN  h2 = h1 + sum_shared Wd_s a_s + sum_{e in top-k} w_e Wd_e a_e
//
// Weights stream through an LDS ring of 8 KiB tiles filled with
// global_load_lds (nontemporal), each wave loading and consuming its own
// quarter of every tile, so the vector-memory counter alone orders a wave's
// loads and reads.  Cross-CU activations are written with device-scope (sc1)
// stores, which write through the per-XCD L2, and every scratch location is
// written at most once per launch, so consumers read them with ordinary loads
// after the barrier and no cache writeback/invalidate is needed.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "mk_internal.h"

namespace mk {

typedef __attribute__((address_space(3))) void lds_void_t;

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// binary32 -> bf16, round to nearest even
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <typename WT>
__device__ __forceinline__ float wload(const WT* p, int i);
template <>
__device__ __forceinline__ float wload<float>(const float* p, int i) { return p[i]; }
template <>
__device__ __forceinline__ float wload<uint16_t>(const uint16_t* p, int i) { return bf16_to_f32(p[i]); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// device-scope (write-through) stores for data other CUs read in this launch
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned ld_dev(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev_u(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 16 bytes per lane, global -> LDS at (wave-uniform base + lane*16), nontemporal
__device__ __forceinline__ void g2l(const void* g, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t*)lds_wave_base, 16, 0, 2);
}

// s_waitcnt encodings (gfx9): vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4]<<14
#define MK_VMCNT(n) (((n)&15) | ((((n) >> 4) & 3) << 14) | 0x70 | 0xF00)
__device__ __forceinline__ void wait_all() { __builtin_amdgcn_s_waitcnt(0); }
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
#define MK_CASE(k) \
  case k:          \
    __builtin_amdgcn_s_waitcnt(MK_VMCNT(k)); \
    break;
    MK_CASE(0) MK_CASE(1) MK_CASE(2) MK_CASE(3) MK_CASE(4) MK_CASE(5) MK_CASE(6) MK_CASE(7)
    MK_CASE(8) MK_CASE(9) MK_CASE(10) MK_CASE(11) MK_CASE(12) MK_CASE(13) MK_CASE(14) MK_CASE(15)
    MK_CASE(16) MK_CASE(17) MK_CASE(18) MK_CASE(19) MK_CASE(20) MK_CASE(21) MK_CASE(22) MK_CASE(23)
    MK_CASE(24) MK_CASE(25) MK_CASE(26) MK_CASE(27) MK_CASE(28) MK_CASE(29) MK_CASE(30) MK_CASE(31)
    MK_CASE(32) MK_CASE(33) MK_CASE(34) MK_CASE(35) MK_CASE(36) MK_CASE(37) MK_CASE(38) MK_CASE(39)
    MK_CASE(40) MK_CASE(41) MK_CASE(42) MK_CASE(43) MK_CASE(44) MK_CASE(45) MK_CASE(46) MK_CASE(47)
#undef MK_CASE
    default:
      __builtin_amdgcn_s_waitcnt(MK_VMCNT(0));
  }
}

// ------------------------------------------------------------------ LDS carve-up

struct Misc {
  int pos[kMaxRows];
  int ids[kMaxRows * kMaxTopK];
  float wts[kMaxRows * kMaxTopK];
  int uni[kMaxExperts];
  int n_uni;
  int flag;
  int last;
  int pad;
  float rinv[kMaxRows];
  unsigned char used[kMaxExperts];
  // attention state
  float am[kMaxQ];
  float al[kMaxQ];
  float acorr[kMaxQ];
};
static_assert(sizeof(Misc) <= kMiscBytes, "misc region too small");

struct Smem {
  char* ring;
  float* x;
  float* part;
  Misc* misc;
};

extern __shared__ __attribute__((aligned(16))) char smem_raw[];

// ------------------------------------------------------------------ grid barrier
//
// Hierarchical: workgroups of the same XCD (blockIdx % 8 under the round-robin
// dispatch) arrive on a group counter; the group's last arriver arrives on the
// global counter; the global last arriver publishes the barrier's target on
// every group's release flag, which the group's workgroups poll.  Counters
// only grow (targets are epoch + barrier index), so nothing is reset between
// launches.  A poll that exceeds the watchdog sets the error flag and every
// workgroup leaves the kernel at its next barrier.
__device__ bool grid_sync(const KParams& p, Smem& sm, unsigned target) {
  wait_all();
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned* s = p.sync;
    const int ngrp = p.n_cu < 8 ? p.n_cu : 8;
    const int grp = blockIdx.x % ngrp;
    const unsigned gsize = (unsigned)((p.n_cu - grp + ngrp - 1) / ngrp);
    unsigned old = __hip_atomic_fetch_add(s + SyncLayout::kGroup + grp * SyncLayout::kLine, 1u, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
    if (old + 1u == gsize * target) {
      unsigned o2 = __hip_atomic_fetch_add(s + SyncLayout::kGlobal, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (o2 + 1u == (unsigned)ngrp * target) {
        for (int g = 0; g < ngrp; ++g) st_dev_u(s + SyncLayout::kFlag + g * SyncLayout::kLine, target);
      }
    }
    int ok = 1;
    const unsigned* flag = s + SyncLayout::kFlag + grp * SyncLayout::kLine;
    long long t0 = wall_clock64();
    while ((int)(ld_dev(flag) - target) < 0) {
      if (ld_dev(s + SyncLayout::kErr) != 0u) { ok = 0; break; }
      if (wall_clock64() - t0 > p.timeout_ticks) {
        __hip_atomic_fetch_or(s + SyncLayout::kErr, kErrTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    sm.misc->flag = ok;
  }
  __syncthreads();
  return sm.misc->flag != 0;
}

// ------------------------------------------------------------------ tile ring
//
// A phase's weights are a sequence of 8 KiB tiles (contiguous rows of one
// row-major matrix).  Wave w loads bytes [2w KiB, 2w+2 KiB) of each tile into
// the same bytes of a ring slot and later reads only those bytes.  Lanes past
// a partial tile's valid bytes re-load the tile's first 16 bytes (always
// valid), so no load leaves the matrix.
struct TileSrc {
  const char* g;
  int valid;
};

__device__ __forceinline__ void issue_quarter(TileSrc t, char* slot, int wave, int lane) {
  const int off0 = wave * 2048 + lane * 16;
  const int off1 = off0 + 1024;
  g2l(t.g + (off0 < t.valid ? off0 : 0), slot + wave * 2048);
  g2l(t.g + (off1 < t.valid ? off1 : 0), slot + wave * 2048 + 1024);
}

// Row r of a tile that holds rows of rb bytes; the wave's chunks c = 0, 1 sit
// at byte wave*2048 + c*1024 of the tile.
struct GemvTile {
  int rb;        // row bytes (1..8 KiB)
  int kbase;     // element offset of this tile's rows in x (always 0: rows are full)
  int row_base;  // first part-row of this tile within the round
  int nrows;     // valid rows in this tile
  int accum;     // 0: store, 1: accumulate into part
};

// Dot products of the wave's quarter of one weight tile with up to MT token
// vectors.  xoff[t] < 0 skips token t; tw[t] scales its contribution.
// x vectors are fp32 rows; in LDS (XL) or global memory; gam (nullable) is a
// per-element gain multiplied into x on the fly (global x only).
template <typename WT, int MT, bool XL>
__device__ __forceinline__ void gemv_tile(const char* slot, const GemvTile& gt, const float* xb, const int* xoff,
                                          const float* tw, const WT* gam, float* part, int M, int wave, int lane) {
  constexpr int ES = sizeof(WT);
  constexpr int EPL = 16 / ES;  // elements per lane per chunk
  float acc[2][MT];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[c][t] = 0.f;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int off = wave * 2048 + c * 1024 + lane * 16;
    const int row = off / gt.rb;
    if (row >= gt.nrows) continue;
    const int k0 = (off % gt.rb) / ES;
    const uint4 wv = *reinterpret_cast<const uint4*>(slot + off);
    float w[EPL];
    if constexpr (ES == 2) {
      w[0] = bf16_lo(wv.x); w[1] = bf16_hi(wv.x); w[2] = bf16_lo(wv.y); w[3] = bf16_hi(wv.y);
      w[4] = bf16_lo(wv.z); w[5] = bf16_hi(wv.z); w[6] = bf16_lo(wv.w); w[7] = bf16_hi(wv.w);
    } else {
      w[0] = __uint_as_float(wv.x); w[1] = __uint_as_float(wv.y);
      w[2] = __uint_as_float(wv.z); w[3] = __uint_as_float(wv.w);
    }
    float g[EPL];
    if (!XL && gam) {
#pragma unroll
      for (int j = 0; j < EPL; ++j) g[j] = wload<WT>(gam, k0 + j);
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      if (t >= M || xoff[t] < 0) continue;
      const float* xp = xb + xoff[t] + k0;
      float s = 0.f;
      if constexpr (EPL == 8) {
        const float4 x0 = *reinterpret_cast<const float4*>(xp);
        const float4 x1 = *reinterpret_cast<const float4*>(xp + 4);
        float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        if (!XL && gam) {
#pragma unroll
          for (int j = 0; j < 8; ++j) xv[j] *= g[j];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) s = fmaf(w[j], xv[j], s);
      } else {
        const float4 x0 = *reinterpret_cast<const float4*>(xp);
        float xv[4] = {x0.x, x0.y, x0.z, x0.w};
        if (!XL && gam) {
#pragma unroll
          for (int j = 0; j < 4; ++j) xv[j] *= g[j];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) s = fmaf(w[j], xv[j], s);
      }
      acc[c][t] += s;
    }
  }
  // reduce across lanes and record the wave's share of each row
  if (gt.rb >= 2048) {
    const int row = (wave * 2048) / gt.rb;
    if (row < gt.nrows) {
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        if (t >= M || xoff[t] < 0) continue;
        float v = wave_sum(acc[0][t] + acc[1][t]);
        if (lane == 0) {
          float* dst = part + ((gt.row_base + row) * kWaves + wave) * M + t;
          *dst = gt.accum ? *dst + tw[t] * v : tw[t] * v;
        }
      }
    }
  } else {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int row = (wave * 2048 + c * 1024) / gt.rb;
      if (row >= gt.nrows) continue;
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        if (t >= M || xoff[t] < 0) continue;
        float v = wave_sum(acc[c][t]);
        if (lane == 0) {
          float* dst = part + ((gt.row_base + row) * kWaves + wave) * M + t;
          *dst = gt.accum ? *dst + tw[t] * v : tw[t] * v;
        }
      }
    }
  }
}

// sum over the waves that hold a share of tile row q (rows of rb bytes)
__device__ __forceinline__ float part_row(const float* part, int prow, int q_in_tile, int rb, int M, int t) {
  int w0 = (q_in_tile * rb) / 2048;
  int w1 = ((q_in_tile + 1) * rb + 2047) / 2048;
  float s = 0.f;
  for (int w = w0; w < w1; ++w) s += part[(prow * kWaves + w) * M + t];
  return s;
}

// ------------------------------------------------------------------ x staging

// Copy M rows of n fp32 (row stride src_ld) from global to LDS (row stride n),
// multiplying by a per-column gain when gam != nullptr.
template <typename WT>
__device__ void stage_x(float* dst, const float* src, int M, int n, int src_ld, const WT* gam) {
  const int nv = n / 4;
  for (int i = threadIdx.x; i < M * nv; i += kThreads) {
    const int t = i / nv, c = (i % nv) * 4;
    float4 v = *reinterpret_cast<const float4*>(src + (size_t)t * src_ld + c);
    if (gam) {
      v.x *= wload<WT>(gam, c); v.y *= wload<WT>(gam, c + 1);
      v.z *= wload<WT>(gam, c + 2); v.w *= wload<WT>(gam, c + 3);
    }
    *reinterpret_cast<float4*>(dst + t * n + c) = v;
  }
}

// 1 / sqrt(mean(h^2) + eps) per row, into misc->rinv
__device__ void row_rinv(Smem& sm, const float* h, int M, int d, float eps) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int t = wave; t < M; t += kWaves) {
    float s = 0.f;
    for (int i = lane * 4; i < d; i += 256) {
      float4 v = *reinterpret_cast<const float4*>(h + (size_t)t * d + i);
      s += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    s = wave_sum(s);
    if (lane == 0) sm.misc->rinv[t] = 1.0f / sqrtf(s / (float)d + eps);
  }
}

// ------------------------------------------------------------------ phase driver
//
// Streams `ntiles` tiles through the ring.  tile(i) gives the source and the
// GEMV description of tile i; xsel(i, xoff, tw) fills the per-token x offsets
// and weights; round_end(first, last) runs after the tiles first..last (all
// waves synchronised before and after) and must consume and clear the part
// entries it owns.  is_round_end(i) marks where rounds close.
template <typename WT, int MT, bool XL, class TileFn, class XSel, class RoundEnd, class IsEnd>
__device__ void run_tiles(const KParams& p, Smem& sm, int ntiles, TileFn tile, XSel xsel, const float* xb,
                          const WT* gam, IsEnd is_round_end, RoundEnd round_end) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nt = p.ring_tiles;
  const int pre = ntiles < nt - 1 ? ntiles : nt - 1;
  for (int i = 0; i < pre; ++i) {
    GemvTile gt;
    TileSrc src = tile(i, gt);
    issue_quarter(src, sm.ring + (size_t)(i % nt) * kTileBytes, wave, lane);
  }
  int round_first = 0;
  for (int i = 0; i < ntiles; ++i) {
    const int nxt = i + nt - 1;
    if (nxt < ntiles) {
      wait_lgkm0();  // our reads of the slot being refilled are done
      GemvTile gt2;
      TileSrc src = tile(nxt, gt2);
      issue_quarter(src, sm.ring + (size_t)(nxt % nt) * kTileBytes, wave, lane);
    }
    int ahead = ntiles - 1 - i;
    if (ahead > nt - 1) ahead = nt - 1;
    wait_vm(2 * ahead);
    GemvTile gt;
    (void)tile(i, gt);
    int xoff[MT];
    float tw[MT];
    xsel(i, xoff, tw);
    gemv_tile<WT, MT, XL>(sm.ring + (size_t)(i % nt) * kTileBytes, gt, xb, xoff, tw, gam, sm.part, p.M, wave, lane);
    if (is_round_end(i)) {
      __syncthreads();
      round_end(round_first, i);
      __syncthreads();
      round_first = i + 1;
    }
  }
}

__device__ void zero_part(Smem& sm) {
  for (int i = threadIdx.x; i < kPartBytes / 4; i += kThreads) sm.part[i] = 0.f;
  __syncthreads();
}

// rows of part that fit one round: part holds rows * 4 waves * M floats
__device__ __forceinline__ int round_rows(const KParams& p) { return (kPartBytes / 4) / (kWaves * p.M); }

__device__ __forceinline__ const float* act_f(const KParams& p, int l, size_t off) {
  return reinterpret_cast<const float*>(p.act + (size_t)l * p.al.stride + off);
}
__device__ __forceinline__ float* act_w(const KParams& p, int l, size_t off) {
  return reinterpret_cast<float*>(p.act + (size_t)l * p.al.stride + off);
}

// input rows of layer l
__device__ __forceinline__ const float* layer_in(const KParams& p, int l) {
  return l == 0 ? p.hidden_in : act_f(p, l - 1, p.al.h2);
}

// h1 of layer l: the attention block's output, or the layer input when the
// stack has no attention
__device__ __forceinline__ const float* layer_h1(const KParams& p, int l) {
  return p.attn ? act_f(p, l, p.al.h1) : layer_in(p, l);
}

// balanced split of n items over the grid
__device__ __forceinline__ void my_range(int n, int ncu, int& lo, int& hi) {
  lo = (int)(((long long)blockIdx.x * n) / ncu);
  hi = (int)(((long long)(blockIdx.x + 1) * n) / ncu);
}

// ------------------------------------------------------------------ phases

// QKV: raw projections of (h * g1) for every row; the row scale rinv is
// applied in the epilogue.
template <typename WT, int MT, bool XL>
__device__ void phase_qkv(const KParams& p, Smem& sm, int l) {
  const DevLayer& Ly = p.layers[l];
  const float* h = layer_in(p, l);
  const int d = p.d;
  const int rb = d * (int)sizeof(WT);
  const int rpt = kTileBytes / rb;
  const int nq = p.H * p.hd, nk = p.G * p.hd;
  const int nrows = nq + 2 * nk;
  const int ntile_all = nrows / rpt;
  int lo, hi;
  my_range(ntile_all, p.n_cu, lo, hi);
  const WT* g1 = reinterpret_cast<const WT*>(Ly.attn_norm);
  row_rinv(sm, h, p.M, d, p.eps);
  if (XL) stage_x<WT>(sm.x, h, p.M, d, d, g1);
  zero_part(sm);
  const int rows_round = round_rows(p);
  const int tiles_round = rows_round / rpt > 0 ? rows_round / rpt : 1;
  float* qkv = act_w(p, l, p.al.qkv);
  auto tile = [&](int i, GemvTile& gt) -> TileSrc {
    const int row0 = (lo + i) * rpt;
    const char* base;
    if (row0 < nq) base = (const char*)Ly.wq + (size_t)row0 * rb;
    else if (row0 < nq + nk) base = (const char*)Ly.wk + (size_t)(row0 - nq) * rb;
    else base = (const char*)Ly.wv + (size_t)(row0 - nq - nk) * rb;
    gt.rb = rb; gt.kbase = 0; gt.row_base = (i % tiles_round) * rpt; gt.nrows = rpt; gt.accum = 0;
    return TileSrc{base, kTileBytes};
  };
  auto xsel = [&](int, int* xoff, float* tw) {
#pragma unroll
    for (int t = 0; t < MT; ++t) { xoff[t] = t < p.M ? (XL ? t * d : t * d) : -1; tw[t] = 1.f; }
  };
  auto is_end = [&](int i) { return ((i + 1) % tiles_round) == 0 || i == hi - lo - 1; };
  auto round_end = [&](int first, int last) {
    const int nr = (last - first + 1) * rpt;
    for (int it = threadIdx.x; it < nr * p.M; it += kThreads) {
      const int q = it / p.M, t = it % p.M;
      const int row = (lo + first) * rpt + q;
      float v = part_row(sm.part, q, q % rpt, rb, p.M, t) * sm.misc->rinv[t];
      st_dev(qkv + (size_t)t * nrows + row, v);
    }
  };
  run_tiles<WT, MT, XL>(p, sm, hi - lo, tile, xsel, XL ? sm.x : h, XL ? nullptr : g1, is_end, round_end);
}

// Split-KV GQA attention.  Task = (sequence, kv head, split).  Query vector
// q = rr*HG + hh is row seq*rps + rr, head g*HG + hh.
__device__ void phase_attn(const KParams& p, Smem& sm, int l) {
  const int HG = p.H / p.G, hd = p.hd, rps = p.rps;
  const int Q = rps * HG;
  const int S = p.n_splits;
  const int ntask = p.n_seq * p.G * S;
  const int nrows_qkv = (p.H + 2 * p.G) * hd;
  const float* qkv = act_f(p, l, p.al.qkv);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float* Qv = sm.x;                    // [Q][hd]
  float* Sc = sm.x + kMaxQ * 128;      // [Q][32] probabilities of the current tile
  Misc* ms = sm.misc;
  const float scale = 1.0f / sqrtf((float)hd);
  for (int task = blockIdx.x; task < ntask; task += p.n_cu) {
    const int seq = task / (p.G * S), g = (task / S) % p.G, s = task % S;
    int maxpos = 0;
    for (int rr = 0; rr < rps; ++rr) maxpos = max(maxpos, ms->pos[seq * rps + rr]);
    const int npos = maxpos + 1;
    int sl = (npos + S - 1) / S;
    sl = (sl + kAttnTile - 1) / kAttnTile * kAttnTile;
    const int p_lo = s * sl;
    const int p_hi = min(p_lo + sl, npos);
    const size_t kv_base = ((((size_t)l * p.n_seq + seq) * p.G + g) * (size_t)p.cap) * hd;
    uint16_t* kc = p.kcache + kv_base;
    uint16_t* vc = p.vcache + kv_base;
    // queries with RoPE, pre-scaled
    for (int it = threadIdx.x; it < Q * (hd / 2); it += kThreads) {
      const int q = it / (hd / 2), i = it % (hd / 2);
      const int rr = q / HG, hh = q % HG;
      const int row = seq * rps + rr, head = g * HG + hh;
      const float* src = qkv + (size_t)row * nrows_qkv + head * hd;
      const double inv = pow((double)p.theta, -2.0 * i / (double)hd);
      const double a = (double)ms->pos[row] * inv;
      const float c = (float)cos(a), sn = (float)sin(a);
      const float x0 = src[i], x1 = src[i + hd / 2];
      Qv[q * hd + i] = (x0 * c - x1 * sn) * scale;
      Qv[q * hd + i + hd / 2] = (x1 * c + x0 * sn) * scale;
    }
    // new rows of this sequence that fall in the split: RoPE'd bf16 k, bf16 v
    for (int rr = 0; rr < rps; ++rr) {
      const int row = seq * rps + rr;
      const int pos = ms->pos[row];
      if (pos < p_lo || pos >= p_hi) continue;
      const float* ksrc = qkv + (size_t)row * nrows_qkv + p.H * hd + g * hd;
      const float* vsrc = qkv + (size_t)row * nrows_qkv + (p.H + p.G) * hd + g * hd;
      for (int i = threadIdx.x; i < hd / 2; i += kThreads) {
        const double inv = pow((double)p.theta, -2.0 * i / (double)hd);
        const double a = (double)pos * inv;
        const float c = (float)cos(a), sn = (float)sin(a);
        const float x0 = ksrc[i], x1 = ksrc[i + hd / 2];
        kc[(size_t)pos * hd + i] = f32_to_bf16(x0 * c - x1 * sn);
        kc[(size_t)pos * hd + i + hd / 2] = f32_to_bf16(x1 * c + x0 * sn);
        vc[(size_t)pos * hd + i] = f32_to_bf16(vsrc[i]);
        vc[(size_t)pos * hd + i + hd / 2] = f32_to_bf16(vsrc[i + hd / 2]);
      }
    }
    for (int q = threadIdx.x; q < Q; q += kThreads) { ms->am[q] = -INFINITY; ms->al[q] = 0.f; }
    wait_all();
    __syncthreads();
    // PV accumulators: item = (q, dim block of 8, position group of 8)
    const int nitem = Q * (hd / 8) * 4;
    constexpr int kMaxItems = kMaxQ * 16 * 4 / kThreads;  // 8
    float acc[kMaxItems][8];
#pragma unroll
    for (int a = 0; a < kMaxItems; ++a)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[a][j] = 0.f;
    const int ntkv = (p_hi > p_lo) ? (p_hi - p_lo + kAttnTile - 1) / kAttnTile : 0;
    const int ntiles = 2 * ntkv;  // K0 V0 K1 V1 ...
    const int nt = p.ring_tiles;
    auto src_of = [&](int i) -> TileSrc {
      const int t0 = p_lo + (i >> 1) * kAttnTile;
      const int nv = min(kAttnTile, p_hi - t0);
      const uint16_t* base = (i & 1) ? vc : kc;
      return TileSrc{reinterpret_cast<const char*>(base + (size_t)t0 * hd), nv * hd * 2};
    };
    const int pre = ntiles < nt - 1 ? ntiles : nt - 1;
    for (int i = 0; i < pre; ++i) issue_quarter(src_of(i), sm.ring + (size_t)(i % nt) * kTileBytes, wave, lane);
    for (int i = 0; i < ntiles; ++i) {
      const int nxt = i + nt - 1;
      if (nxt < ntiles) issue_quarter(src_of(nxt), sm.ring + (size_t)(nxt % nt) * kTileBytes, wave, lane);
      int ahead = min(ntiles - 1 - i, nt - 1);
      wait_vm(2 * ahead);
      __syncthreads();
      const char* slot = sm.ring + (size_t)(i % nt) * kTileBytes;
      const int t0 = p_lo + (i >> 1) * kAttnTile;
      if ((i & 1) == 0) {
        // scores and online-softmax update: wave handles queries 2w + 8k (+1)
        for (int base = wave * 64; base < Q * 32; base += kThreads) {
          const int item = base + lane;
          const int q = item / 32, jj = item % 32;
          float sc = -INFINITY;
          const int j = t0 + jj;
          if (q < Q) {
            const int row = seq * rps + q / HG;
            if (j < p_hi && j <= ms->pos[row]) {
              const uint16_t* kr = reinterpret_cast<const uint16_t*>(slot + jj * hd * 2);
              const float* qr = Qv + q * hd;
              float dsum = 0.f;
              for (int b = 0; b < hd / 8; ++b) {
                const int bb = (b + jj) % (hd / 8);
                const uint4 kv = *reinterpret_cast<const uint4*>(kr + bb * 8);
                const float4 q0 = *reinterpret_cast<const float4*>(qr + bb * 8);
                const float4 q1 = *reinterpret_cast<const float4*>(qr + bb * 8 + 4);
                dsum = fmaf(bf16_lo(kv.x), q0.x, dsum); dsum = fmaf(bf16_hi(kv.x), q0.y, dsum);
                dsum = fmaf(bf16_lo(kv.y), q0.z, dsum); dsum = fmaf(bf16_hi(kv.y), q0.w, dsum);
                dsum = fmaf(bf16_lo(kv.z), q1.x, dsum); dsum = fmaf(bf16_hi(kv.z), q1.y, dsum);
                dsum = fmaf(bf16_lo(kv.w), q1.z, dsum); dsum = fmaf(bf16_hi(kv.w), q1.w, dsum);
              }
              sc = dsum;
            }
          }
          // 32-lane max / sum (lanes 0-31 and 32-63 are different queries)
          float mt = sc;
#pragma unroll
          for (int o = 16; o > 0; o >>= 1) mt = fmaxf(mt, __shfl_xor(mt, o));
          const float m_old = q < Q ? ms->am[q] : -INFINITY;
          const float m_new = fmaxf(m_old, mt);
          const float pr = (m_new == -INFINITY || sc == -INFINITY) ? 0.f : __expf(sc - m_new);
          float ps = pr;
#pragma unroll
          for (int o = 16; o > 0; o >>= 1) ps += __shfl_xor(ps, o);
          if (q < Q) {
            Sc[q * 32 + jj] = pr;
            if (jj == 0) {
              const float corr = (m_new == -INFINITY) ? 1.f : __expf(m_old - m_new);
              ms->acorr[q] = corr;
              ms->al[q] = ms->al[q] * corr + ps;
              ms->am[q] = m_new;
            }
          }
        }
      } else {
        // PV: acc = acc * corr + sum_j p_j V_j over this tile
#pragma unroll
        for (int a = 0; a < kMaxItems; ++a) {
          const int item = threadIdx.x + a * kThreads;
          if (item >= nitem) break;
          const int q = item / 64, db = (item / 4) % 16, jg = item % 4;
          const float corr = ms->acorr[q];
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[a][j] *= corr;
          for (int u = 0; u < 8; ++u) {
            const int jj = jg * 8 + u;
            const float pr = Sc[q * 32 + jj];
            if (pr == 0.f) continue;
            const uint4 vv = *reinterpret_cast<const uint4*>(slot + jj * hd * 2 + db * 16);
            acc[a][0] = fmaf(pr, bf16_lo(vv.x), acc[a][0]); acc[a][1] = fmaf(pr, bf16_hi(vv.x), acc[a][1]);
            acc[a][2] = fmaf(pr, bf16_lo(vv.y), acc[a][2]); acc[a][3] = fmaf(pr, bf16_hi(vv.y), acc[a][3]);
            acc[a][4] = fmaf(pr, bf16_lo(vv.z), acc[a][4]); acc[a][5] = fmaf(pr, bf16_hi(vv.z), acc[a][5]);
            acc[a][6] = fmaf(pr, bf16_lo(vv.w), acc[a][6]); acc[a][7] = fmaf(pr, bf16_hi(vv.w), acc[a][7]);
          }
        }
      }
      __syncthreads();
    }
    // reduce position groups (lanes 4n..4n+3) and write the partial state
    float* part = act_w(p, l, p.al.part) + ((size_t)((seq * p.G + g) * S + s) * Q) * (hd + 2);
#pragma unroll
    for (int a = 0; a < kMaxItems; ++a) {
      const int item = threadIdx.x + a * kThreads;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float v = acc[a][j];
        v += __shfl_xor(v, 1);
        v += __shfl_xor(v, 2);
        acc[a][j] = v;
      }
      if (item < nitem && (item % 4) == 0) {
        const int q = item / 64, db = (item / 4) % 16;
#pragma unroll
        for (int j = 0; j < 8; ++j) st_dev(part + (size_t)q * (hd + 2) + 2 + db * 8 + j, acc[a][j]);
      }
    }
    for (int q = threadIdx.x; q < Q; q += kThreads) {
      st_dev(part + (size_t)q * (hd + 2) + 0, ms->am[q]);
      st_dev(part + (size_t)q * (hd + 2) + 1, ms->al[q]);
    }
    wait_all();
    __syncthreads();
    if (threadIdx.x == 0) {
      unsigned* cnt = p.attn_cnt + ((size_t)l * p.n_seq + seq) * p.G + g;
      unsigned old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int last = (old + 1u == (unsigned)S);
      if (last) st_dev_u(cnt, 0u);
      ms->last = last;
    }
    __syncthreads();
    if (ms->last) {
      const float* pall = act_f(p, l, p.al.part) + ((size_t)((seq * p.G + g) * S) * Q) * (hd + 2);
      float* o = act_w(p, l, p.al.o);
      for (int it = threadIdx.x; it < Q * hd; it += kThreads) {
        const int q = it / hd, i = it % hd;
        float mx = -INFINITY;
        for (int z = 0; z < S; ++z) mx = fmaxf(mx, pall[((size_t)z * Q + q) * (hd + 2)]);
        float L = 0.f, num = 0.f;
        for (int z = 0; z < S; ++z) {
          const float* pz = pall + ((size_t)z * Q + q) * (hd + 2);
          const float mz = pz[0];
          if (mz == -INFINITY) continue;
          const float e = __expf(mz - mx);
          L += pz[1] * e;
          num += pz[2 + i] * e;
        }
        const int rr = q / HG, hh = q % HG;
        const int row = seq * rps + rr, head = g * HG + hh;
        st_dev(o + (size_t)row * (p.H * hd) + head * hd + i, num / L);
      }
    }
    __syncthreads();
  }
}

// WO: h1 = h + Wo . o
template <typename WT, int MT, bool XL>
__device__ void phase_wo(const KParams& p, Smem& sm, int l) {
  const DevLayer& Ly = p.layers[l];
  const int K = p.H * p.hd;
  const int rb = K * (int)sizeof(WT);
  const int rpt = kTileBytes / rb;
  const int ntile_all = p.d / rpt;
  int lo, hi;
  my_range(ntile_all, p.n_cu, lo, hi);
  const float* o = act_f(p, l, p.al.o);
  const float* h = layer_in(p, l);
  float* h1 = act_w(p, l, p.al.h1);
  if (XL) stage_x<WT>(sm.x, o, p.M, K, K, nullptr);
  zero_part(sm);
  const int rows_round = round_rows(p);
  const int tiles_round = rows_round / rpt > 0 ? rows_round / rpt : 1;
  auto tile = [&](int i, GemvTile& gt) -> TileSrc {
    const int row0 = (lo + i) * rpt;
    gt.rb = rb; gt.kbase = 0; gt.row_base = (i % tiles_round) * rpt; gt.nrows = rpt; gt.accum = 0;
    return TileSrc{(const char*)Ly.wo + (size_t)row0 * rb, kTileBytes};
  };
  auto xsel = [&](int, int* xoff, float* tw) {
#pragma unroll
    for (int t = 0; t < MT; ++t) { xoff[t] = t < p.M ? t * K : -1; tw[t] = 1.f; }
  };
  auto is_end = [&](int i) { return ((i + 1) % tiles_round) == 0 || i == hi - lo - 1; };
  auto round_end = [&](int first, int last) {
    const int nr = (last - first + 1) * rpt;
    for (int it = threadIdx.x; it < nr * p.M; it += kThreads) {
      const int q = it / p.M, t = it % p.M;
      const int row = (lo + first) * rpt + q;
      const float v = part_row(sm.part, q, q % rpt, rb, p.M, t);
      st_dev(h1 + (size_t)t * p.d + row, h[(size_t)t * p.d + row] + v);
    }
  };
  run_tiles<WT, MT, XL>(p, sm, hi - lo, tile, xsel, XL ? sm.x : o, (const WT*)nullptr, is_end, round_end);
}

// RS: router logits and shared-expert gate/up.  Work units: router tiles
// (weight 1) then shared pairs (gate tile, up tile; weight 2), split over the
// grid by cumulative weight so that a pair never straddles two CUs.
template <typename WT, int MT, bool XL>
__device__ void phase_rs(const KParams& p, Smem& sm, int l) {
  const DevLayer& Ly = p.layers[l];
  const int d = p.d, F = p.F, E = p.E;
  const int rb = d * (int)sizeof(WT);
  const int rpt = kTileBytes / rb;
  const int nrt = (E + rpt - 1) / rpt;
  const int fb_per = F / rpt;  // f-blocks per shared expert
  const int npair = p.S * fb_per;
  const int T = nrt + 2 * npair;
  int lo, hi;
  my_range(T, p.n_cu, lo, hi);
  const int r_lo = min(lo, nrt), r_hi = min(hi, nrt);
  // pairs whose first tile index nrt + 2j lies in [lo, hi)
  auto ceil_half = [](int x) { return x <= 0 ? 0 : (x + 1) / 2; };
  const int p_lo = min(npair, ceil_half(lo - nrt)), p_hi = min(npair, ceil_half(hi - nrt));
  const int n_rt = r_hi - r_lo, n_pt = 2 * (p_hi - p_lo);
  const int ntiles = n_rt + n_pt;
  const float* h1 = layer_h1(p, l);
  const WT* g2 = reinterpret_cast<const WT*>(Ly.moe_norm);
  row_rinv(sm, h1, p.M, d, p.eps);
  if (XL) stage_x<WT>(sm.x, h1, p.M, d, d, g2);
  zero_part(sm);
  float* logits = act_w(p, l, p.al.logits);
  float* a_s = act_w(p, l, p.al.a_s);
  const int rows_round = round_rows(p);
  int tiles_round = rows_round / rpt > 0 ? rows_round / rpt : 1;
  if (tiles_round > 1) tiles_round &= ~1;  // keep gate/up of a pair in one round
  auto tile = [&](int i, GemvTile& gt) -> TileSrc {
    gt.rb = rb; gt.kbase = 0; gt.accum = 0;
    if (i < n_rt) {
      const int row0 = (r_lo + i) * rpt;
      gt.nrows = min(rpt, E - row0);
      gt.row_base = (i % tiles_round) * rpt;
      return TileSrc{(const char*)Ly.w_router + (size_t)row0 * rb, gt.nrows * rb};
    }
    const int k = i - n_rt;
    const int pj = p_lo + k / 2;
    const int sx = pj / fb_per, fb = pj % fb_per;
    const char* base = (const char*)((k & 1) ? Ly.s_up : Ly.s_gate) + ((size_t)sx * F + (size_t)fb * rpt) * rb;
    gt.nrows = rpt;
    gt.row_base = (k % tiles_round) * rpt;
    return TileSrc{base, kTileBytes};
  };
  auto xsel = [&](int, int* xoff, float* tw) {
#pragma unroll
    for (int t = 0; t < MT; ++t) { xoff[t] = t < p.M ? t * d : -1; tw[t] = 1.f; }
  };
  auto is_end = [&](int i) {
    if (i == ntiles - 1) return true;
    if (i < n_rt) return i == n_rt - 1 || ((i + 1) % tiles_round) == 0;
    return ((i - n_rt + 1) % tiles_round) == 0;
  };
  auto round_end = [&](int first, int last) {
    if (first < n_rt) {
      const int nr = (last - first + 1) * rpt;
      for (int it = threadIdx.x; it < nr * p.M; it += kThreads) {
        const int q = it / p.M, t = it % p.M;
        const int e = (r_lo + first) * rpt + q;
        if (e >= E) continue;
        float v = part_row(sm.part, q, q % rpt, rb, p.M, t) * sm.misc->rinv[t];
        if (p.has_bias) v += Ly.b_router[e];
        st_dev(logits + (size_t)t * E + e, v);
      }
    } else {
      const int k0 = first - n_rt;
      const int npairs_r = (last - first + 1) / 2;
      for (int it = threadIdx.x; it < npairs_r * rpt * p.M; it += kThreads) {
        const int pr = it / (rpt * p.M), q = (it / p.M) % rpt, t = it % p.M;
        const int pj = p_lo + k0 / 2 + pr;
        const int sx = pj / fb_per, f = (pj % fb_per) * rpt + q;
        const int prow_g = ((k0 + 2 * pr) % tiles_round) * rpt + q;
        const int prow_u = ((k0 + 2 * pr + 1) % tiles_round) * rpt + q;
        const float ri = sm.misc->rinv[t];
        const float gv = part_row(sm.part, prow_g, q, rb, p.M, t) * ri;
        const float uv = part_row(sm.part, prow_u, q, rb, p.M, t) * ri;
        const float av = gv / (1.f + __expf(-gv)) * uv;
        st_dev(a_s + ((size_t)t * p.S + sx) * F + f, av);
      }
    }
  };
  run_tiles<WT, MT, XL>(p, sm, ntiles, tile, xsel, XL ? sm.x : h1, XL ? nullptr : g2, is_end, round_end);
}

// Top-k over the router logits of every row (all CUs, redundantly), then the
// union of chosen experts.  Selection is on the logits, larger first, equal
// logits ranked by lower expert id; weights are softmax probabilities
// renormalised over the chosen set.
__device__ void route_topk(const KParams& p, Smem& sm, int l) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int E = p.E, k = p.k;
  const float* logits = act_f(p, l, p.al.logits);
  Misc* ms = sm.misc;
  for (int e = threadIdx.x; e < kMaxExperts; e += kThreads) ms->used[e] = 0;
  __syncthreads();
  for (int t = wave; t < p.M; t += kWaves) {
    const float z = lane < E ? logits[(size_t)t * E + lane] : -INFINITY;
    bool taken = lane >= E;
    const float zmax = wave_max(z);
    float psum = 0.f;
    float pmine = 0.f;
    int sel[kMaxTopK];
    for (int i = 0; i < k; ++i) {
      // best (z desc, id asc) among untaken lanes
      float bz = taken ? -INFINITY : z;
      int bi = taken ? 1 << 30 : lane;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float oz = __shfl_xor(bz, o);
        const int oi = __shfl_xor(bi, o);
        if (oz > bz || (oz == bz && oi < bi)) { bz = oz; bi = oi; }
      }
      if (lane == bi) {
        taken = true;
        pmine = __expf(z - zmax);
      }
      sel[i] = bi;
      psum += __shfl(lane == bi ? __expf(z - zmax) : 0.f, bi);
    }
    // weights in selection order
    for (int i = 0; i < k; ++i) {
      const int e = sel[i];
      const float pe = __shfl(pmine, e);
      if (lane == 0) {
        ms->ids[t * k + i] = e;
        ms->wts[t * k + i] = pe / psum;
        ms->used[e] = 1;
      }
    }
  }
  __syncthreads();
  if (wave == 0) {
    const bool u = lane < E && ms->used[lane];
    const unsigned long long m = __ballot(u);
    if (u) {
      const int idx = __popcll(m & ((1ull << lane) - 1ull));
      ms->uni[idx] = lane;
    }
    if (lane == 0) ms->n_uni = __popcll(m);
  }
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int i = threadIdx.x; i < p.M * k; i += kThreads) {
      if (p.t_ids) p.t_ids[(size_t)l * p.M * k + i] = ms->ids[i];
      if (p.t_w) p.t_w[(size_t)l * p.M * k + i] = ms->wts[i];
    }
    if (p.t_logits)
      for (int i = threadIdx.x; i < p.M * E; i += kThreads) p.t_logits[(size_t)l * p.M * E + i] = logits[i];
  }
}

// slot of expert e in row t's top-k list, or -1
__device__ __forceinline__ int slot_of(const Misc* ms, int t, int k, int e) {
  for (int i = 0; i < k; ++i)
    if (ms->ids[t * k + i] == e) return i;
  return -1;
}

// RG: routed gate/up rows for the union experts; a[t][slot][f] for rows
// routed to the expert.
template <typename WT, int MT, bool XL>
__device__ void phase_rg(const KParams& p, Smem& sm, int l) {
  const DevLayer& Ly = p.layers[l];
  const int d = p.d, F = p.F, k = p.k;
  const int rb = d * (int)sizeof(WT);
  const int rpt = kTileBytes / rb;
  const int fb_per = F / rpt;
  const float* h1 = layer_h1(p, l);
  const WT* g2 = reinterpret_cast<const WT*>(Ly.moe_norm);
  route_topk(p, sm, l);
  const int U = sm.misc->n_uni;
  const int npair = U * fb_per;
  int lo, hi;
  my_range(npair, p.n_cu, lo, hi);
  const int ntiles = 2 * (hi - lo);
  row_rinv(sm, h1, p.M, d, p.eps);
  if (XL) stage_x<WT>(sm.x, h1, p.M, d, d, g2);
  zero_part(sm);
  float* a = act_w(p, l, p.al.a);
  const int rows_round = round_rows(p);
  int tiles_round = rows_round / rpt > 0 ? rows_round / rpt : 1;
  if (tiles_round > 1) tiles_round &= ~1;
  const Misc* ms = sm.misc;
  auto tile = [&](int i, GemvTile& gt) -> TileSrc {
    const int pj = lo + i / 2;
    const int e = ms->uni[pj / fb_per], fb = pj % fb_per;
    const char* base = (const char*)((i & 1) ? Ly.w_up : Ly.w_gate) + ((size_t)e * F + (size_t)fb * rpt) * rb;
    gt.rb = rb; gt.kbase = 0; gt.accum = 0; gt.nrows = rpt; gt.row_base = (i % tiles_round) * rpt;
    return TileSrc{base, kTileBytes};
  };
  auto xsel = [&](int i, int* xoff, float* tw) {
    const int e = ms->uni[(lo + i / 2) / fb_per];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      xoff[t] = (t < p.M && slot_of(ms, t, k, e) >= 0) ? t * d : -1;
      tw[t] = 1.f;
    }
  };
  auto is_end = [&](int i) { return ((i + 1) % tiles_round) == 0 || i == ntiles - 1; };
  auto round_end = [&](int first, int last) {
    const int npairs_r = (last - first + 1) / 2;
    for (int it = threadIdx.x; it < npairs_r * rpt * p.M; it += kThreads) {
      const int pr = it / (rpt * p.M), q = (it / p.M) % rpt, t = it % p.M;
      const int pj = lo + first / 2 + pr;
      const int e = ms->uni[pj / fb_per], f = (pj % fb_per) * rpt + q;
      const int sl = slot_of(ms, t, k, e);
      if (sl < 0) continue;
      const int prow_g = ((first + 2 * pr) % tiles_round) * rpt + q;
      const int prow_u = ((first + 2 * pr + 1) % tiles_round) * rpt + q;
      const float ri = ms->rinv[t];
      const float gv = part_row(sm.part, prow_g, q, rb, p.M, t) * ri;
      const float uv = part_row(sm.part, prow_u, q, rb, p.M, t) * ri;
      st_dev(a + ((size_t)t * k + sl) * F + f, gv / (1.f + __expf(-gv)) * uv);
    }
  };
  run_tiles<WT, MT, XL>(p, sm, ntiles, tile, xsel, XL ? sm.x : h1, XL ? nullptr : g2, is_end, round_end);
}

// DOWN: for this CU's blocks of output columns j, accumulate over the shared
// experts and the union experts (each row weighted by its routing weight),
// then h2 = h1 + sum.  a_s and a are adjacent in the scratch, so x for the
// phase is one [M][(n_shared + k)][F] block.
template <typename WT, int MT, bool XL>
__device__ void phase_down(const KParams& p, Smem& sm, int l) {
  const DevLayer& Ly = p.layers[l];
  const int d = p.d, F = p.F, k = p.k, S = p.S;
  const int rb = F * (int)sizeof(WT);
  const int rpt = kTileBytes / rb;
  const int JB = d / rpt;
  int lo, hi;
  my_range(JB, p.n_cu, lo, hi);
  const Misc* ms = sm.misc;
  const int U = ms->n_uni;
  const int per_block = S + U;
  const int ntiles = (hi - lo) * per_block;
  const float* h1 = layer_h1(p, l);
  const float* xs = act_f(p, l, p.al.a_s);  // a follows a_s in the scratch
  float* h2 = (l == p.L - 1) ? p.hidden_out : act_w(p, l, p.al.h2);
  const bool last_layer = (l == p.L - 1);
  const int xrow = (S + k) * F;  // floats per row t in the combined block
  if (XL) {
    // a_s [M][S][F] and a [M][k][F] -> LDS [M][S+k][F]
    const float* a = act_f(p, l, p.al.a);
    for (int i = threadIdx.x; i < p.M * (S + k) * (F / 4); i += kThreads) {
      const int t = i / ((S + k) * (F / 4));
      const int r = (i / (F / 4)) % (S + k);
      const int c = (i % (F / 4)) * 4;
      const float* src = r < S ? xs + ((size_t)t * S + r) * F + c : a + ((size_t)t * k + (r - S)) * F + c;
      const float4 v = *reinterpret_cast<const float4*>(src);
      *reinterpret_cast<float4*>(sm.x + (size_t)t * xrow + r * F + c) = v;
    }
  }
  zero_part(sm);
  auto tile = [&](int i, GemvTile& gt) -> TileSrc {
    const int jb = lo + i / per_block, u = i % per_block;
    const char* base;
    if (u < S) base = (const char*)Ly.s_down + ((size_t)u * d + (size_t)jb * rpt) * rb;
    else base = (const char*)Ly.w_down + ((size_t)ms->uni[u - S] * d + (size_t)jb * rpt) * rb;
    gt.rb = rb; gt.kbase = 0; gt.accum = 1; gt.nrows = rpt; gt.row_base = 0;
    return TileSrc{base, kTileBytes};
  };
  // global x: a_s rows at xs + (t*S + s)*F; a rows at a + (t*k + slot)*F
  const float* a_g = act_f(p, l, p.al.a);
  auto xsel = [&](int i, int* xoff, float* tw) {
    const int u = i % per_block;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      xoff[t] = -1;
      tw[t] = 0.f;
      if (t >= p.M) continue;
      if (u < S) {
        xoff[t] = XL ? t * xrow + u * F : (int)(((size_t)t * S + u) * F);
        tw[t] = 1.f;
      } else {
        const int e = ms->uni[u - S];
        const int sl = slot_of(ms, t, k, e);
        if (sl >= 0) {
          xoff[t] = XL ? t * xrow + (S + sl) * F : (int)((a_g - xs) + ((size_t)t * k + sl) * F);
          tw[t] = ms->wts[t * k + sl];
        }
      }
    }
  };
  auto is_end = [&](int i) { return ((i + 1) % per_block) == 0; };
  auto round_end = [&](int first, int) {
    const int jb = lo + first / per_block;
    for (int it = threadIdx.x; it < rpt * p.M; it += kThreads) {
      const int q = it / p.M, t = it % p.M;
      const int j = jb * rpt + q;
      const float v = part_row(sm.part, q, q, rb, p.M, t);
      const float out = h1[(size_t)t * d + j] + v;
      if (last_layer) h2[(size_t)t * d + j] = out;
      else st_dev(h2 + (size_t)t * d + j, out);
      // clear this row's part entries for the next block
      for (int w = 0; w < kWaves; ++w) sm.part[(q * kWaves + w) * p.M + t] = 0.f;
    }
  };
  run_tiles<WT, MT, XL>(p, sm, ntiles, tile, xsel, XL ? sm.x : xs, (const WT*)nullptr, is_end, round_end);
}

// ------------------------------------------------------------------ kernel

template <typename WT, int MT>
__global__ void __launch_bounds__(kThreads, 1) decode_step_kernel(KParams p) {
  Smem sm;
  sm.ring = smem_raw;
  sm.x = reinterpret_cast<float*>(smem_raw + (size_t)p.ring_tiles * kTileBytes);
  sm.part = reinterpret_cast<float*>(smem_raw + (size_t)p.ring_tiles * kTileBytes + p.x_bytes);
  sm.misc = reinterpret_cast<Misc*>(smem_raw + (size_t)p.ring_tiles * kTileBytes + p.x_bytes + kPartBytes);
  Misc* ms = sm.misc;
  // positions: range and distinctness within a sequence (every CU checks the
  // same data, so all leave together on a bad input)
  if (threadIdx.x == 0) {
    int bad = 0;
    for (int r = 0; r < p.M; ++r) {
      const int pos = p.positions[r];
      ms->pos[r] = pos;
      if (p.attn && (pos < 0 || pos >= p.cap)) bad |= kErrPosition;
    }
    if (p.attn)
      for (int r = 0; r < p.M; ++r)
        for (int r2 = r + 1; r2 < p.M && r2 / p.rps == r / p.rps; ++r2)
          if (ms->pos[r] == ms->pos[r2]) bad |= kErrDupPosition;
    ms->flag = bad;
    ms->last = (int)ld_dev(p.sync + SyncLayout::kEpoch);
  }
  __syncthreads();
  if (ms->flag) {
    if (blockIdx.x == 0 && threadIdx.x == 0)
      __hip_atomic_fetch_or(p.sync + SyncLayout::kErr, (unsigned)ms->flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  const unsigned epoch0 = (unsigned)ms->last;
  unsigned b = 0;
  const bool x_fits_d = p.M * p.d * 4 <= p.x_bytes;
  const bool x_fits_o = p.M * p.H * p.hd * 4 <= p.x_bytes;
  const bool x_fits_down = p.M * (p.S + p.k) * p.F * 4 <= p.x_bytes;
  for (int l = 0; l < p.L; ++l) {
    if (p.attn) {
      if (x_fits_d) phase_qkv<WT, MT, true>(p, sm, l);
      else phase_qkv<WT, MT, false>(p, sm, l);
      if (!grid_sync(p, sm, epoch0 + ++b)) return;
      phase_attn(p, sm, l);
      if (!grid_sync(p, sm, epoch0 + ++b)) return;
      if (x_fits_o) phase_wo<WT, MT, true>(p, sm, l);
      else phase_wo<WT, MT, false>(p, sm, l);
      if (!grid_sync(p, sm, epoch0 + ++b)) return;
    }
    if (x_fits_d) phase_rs<WT, MT, true>(p, sm, l);
    else phase_rs<WT, MT, false>(p, sm, l);
    if (!grid_sync(p, sm, epoch0 + ++b)) return;
    if (x_fits_d) phase_rg<WT, MT, true>(p, sm, l);
    else phase_rg<WT, MT, false>(p, sm, l);
    if (!grid_sync(p, sm, epoch0 + ++b)) return;
    if (x_fits_down) phase_down<WT, MT, true>(p, sm, l);
    else phase_down<WT, MT, false>(p, sm, l);
    if (l + 1 < p.L)
      if (!grid_sync(p, sm, epoch0 + ++b)) return;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) st_dev_u(p.sync + SyncLayout::kEpoch, epoch0 + b);
}

}  // namespace mk

extern "C" int mk_launch_kernel(const mk::KParams* pp, void* stream) {
  using namespace mk;
  KParams p = *pp;
  const size_t lds = (size_t)p.ring_tiles * kTileBytes + p.x_bytes + kPartBytes + kMiscBytes;
  if (lds > (size_t)kLdsTotal || p.M > 8) return -2;
  const void* fn;
  if (p.wide) fn = p.M == 1 ? (const void*)decode_step_kernel<float, 1> : (const void*)decode_step_kernel<float, 8>;
  else fn = p.M == 1 ? (const void*)decode_step_kernel<uint16_t, 1> : (const void*)decode_step_kernel<uint16_t, 8>;
  static bool attr_done[4] = {false, false, false, false};
  const int idx = (p.wide ? 2 : 0) + (p.M == 1 ? 0 : 1);
  if (!attr_done[idx]) {
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess) return -1;
    attr_done[idx] = true;
  }
  void* args[] = {&p};
  hipError_t e = hipLaunchCooperativeKernel(fn, dim3(p.n_cu), dim3(kThreads), args, (unsigned)lds, (hipStream_t)stream);
  return e == hipSuccess ? 0 : (int)e;
}
