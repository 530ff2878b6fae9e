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
//   QKV   (attention stacks) raw q, k, v rows of [Wq; Wk; Wv] . (h*g1)
//   ATTN  split-KV GQA over the bf16 cache; the split owning a new position
//         writes its RoPE'd bf16 k and v row; the last split of each
//         (sequence, kv head) to finish combines the partial softmax states
//   WO    h1 = h + Wo . o
//   RS    router logits and shared-expert gate/up (silu(g) * u)
//   RG    shared-expert down projection y_s; top-k and the expert union
//         (every CU, redundantly); routed gate/up rows
//   DOWN  h2 = h1 + y_s + sum_{e in top-k} w_e Wd_e a_e
//
// Weights stream through an LDS ring of 8 KiB tiles filled with
// global_load_lds (nontemporal).  Wave w loads and reads only bytes
// [2w KiB, 2w+2 KiB) of every GEMV tile, so the vector-memory counter alone
// orders a wave's loads and reads, and the tile loop issues nothing else on
// that counter (parameters live in LDS, activations in registers).  The
// tiles of one step form a single stream: while a phase's last tiles are
// being consumed, the ring is already filling with the next phase's tiles,
// and those loads stay in flight through the phase's epilogue and the grid
// barrier, so HBM does not idle at phase boundaries [P3, section
// "Cross-Layer Weight Prefetching": the next layer's weights are moved to
// fast memory while the current layer computes; P2 section
// "把几百个小 kernel，焊成一个大程序": layer N+1's attention weights load during
// layer N's MoE].  The only boundary without lookahead is router -> routed
// experts (which experts to load is not known yet); the shared expert's
// down projection, which depends on nothing routed, fills it.
//
// Cross-CU activations are written with device-scope (sc1) stores, which
// write through the per-XCD L2, and every scratch location is written at
// most once per launch, so consumers read them with ordinary loads after the
// barrier and no cache writeback/invalidate is needed.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "mk_internal.h"
#include "mk_lanes.h"

namespace mk {

typedef __attribute__((address_space(3))) void lds_void_t;

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// binary32 -> bf16, round to nearest even
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// the EPL elements of one 16-byte weight chunk as fp32
template <typename WT>
__device__ __forceinline__ void unpack16(uint4 v, float* w);
template <>
__device__ __forceinline__ void unpack16<uint16_t>(uint4 v, float* w) {
  w[0] = bf16_lo(v.x); w[1] = bf16_hi(v.x); w[2] = bf16_lo(v.y); w[3] = bf16_hi(v.y);
  w[4] = bf16_lo(v.z); w[5] = bf16_hi(v.z); w[6] = bf16_lo(v.w); w[7] = bf16_hi(v.w);
}
template <>
__device__ __forceinline__ void unpack16<float>(uint4 v, float* w) {
  w[0] = __uint_as_float(v.x); w[1] = __uint_as_float(v.y);
  w[2] = __uint_as_float(v.z); w[3] = __uint_as_float(v.w);
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
// wait until at most 2*ahead vector-memory operations of this wave are outstanding
__device__ __forceinline__ void wait_tiles_ahead(int ahead) {
  static_assert(2 * (kRing - 1) <= 63, "vmcnt range");
  if (ahead >= kRing - 1) {
    __builtin_amdgcn_s_waitcnt(MK_VMCNT(2 * (kRing - 1)));
    return;
  }
  switch (ahead) {
#define MK_CASE(k) \
  case k:          \
    __builtin_amdgcn_s_waitcnt(MK_VMCNT(2 * k)); \
    break;
    MK_CASE(1) MK_CASE(2) MK_CASE(3) MK_CASE(4) MK_CASE(5) MK_CASE(6) MK_CASE(7) MK_CASE(8) MK_CASE(9) MK_CASE(10)
#undef MK_CASE
    default:
      __builtin_amdgcn_s_waitcnt(MK_VMCNT(0));
  }
}
static_assert(kRing - 2 <= 10, "extend wait_tiles_ahead");

__device__ __forceinline__ int ilog2(int x) { return 31 - __builtin_clz(x); }

// ------------------------------------------------------------------ LDS carve-up

struct Misc {
  KParams p;  // kernel arguments, read from LDS (keeps them off the vector-memory counter)
  int pos[kMaxRows];
  int ids[kMaxRows * kMaxTopK];
  float wts[kMaxRows * kMaxTopK];
  int uni[kMaxExperts];
  int n_uni;
  int flag;
  int last;
  int epoch;
  float rinv[kMaxRows];
  unsigned char used[kMaxExperts];
  float rope[kMaxRows * 64 * 2];  // (cos, sin) per row and frequency (head_dim 128)
};
static_assert(sizeof(Misc) <= kMiscBytes, "misc region too small");

struct Smem {
  char* ring;
  float* xs;
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
// workgroup leaves the kernel at its next barrier.  Ring loads issued before
// the barrier stay in flight through it.
__device__ __forceinline__ bool grid_sync(const KParams& p, Smem sm, unsigned target) {
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned* s = p.sync;
    const int ncu = p.n_cu;
    const int ngrp = ncu < 8 ? ncu : 8;
    const int grp = blockIdx.x % ngrp;
    const unsigned gsize = (unsigned)((ncu - grp + ngrp - 1) / ngrp);
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
    const long long t0 = wall_clock64();
    const long long lim = p.timeout_ticks;
    while ((int)(ld_dev(flag) - target) < 0) {
      if (ld_dev(s + SyncLayout::kErr) != 0u) { ok = 0; break; }
      if (wall_clock64() - t0 > lim) {
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

// ------------------------------------------------------------------ layer data access

__device__ __forceinline__ const float* act_f(const KParams& p, int l, size_t off) {
  return reinterpret_cast<const float*>(p.act + (size_t)l * p.al.stride + off);
}
__device__ __forceinline__ float* act_w(const KParams& p, int l, size_t off) {
  return reinterpret_cast<float*>(p.act + (size_t)l * p.al.stride + off);
}
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

// ------------------------------------------------------------------ phase plans
//
// A plan lists the 8 KiB tiles one CU streams in one phase, in order.  Plans
// of static phases can be built before the phase starts, which is what lets
// the ring run ahead across phase boundaries.

enum PlanKind { PK_NONE = 0, PK_QKV, PK_ATTN, PK_WO, PK_RS, PK_RG, PK_DOWN };

struct Plan {
  int kind;
  int n;             // tiles
  int lo;            // first unit of the first segment
  int lrb, rpt;      // first segment: log2 row bytes, rows per tile
  int n1;            // tiles of the first segment (RS: router; RG: shared down)
  int lo2;           // first unit of the second segment
  int lrb2, rpt2;    // second segment geometry (RS, RG)
  int fb_per;        // f-blocks per expert in the second segment
  int a0, a1;        // QKV: nq, nk; ATTN: p_lo, p_hi; RS: E; RG, DOWN: unused
  int d, F, S, U;
  const char* b0;
  const char* b1;
  const char* b2;
};

struct TileSrc {
  const char* g;
  int valid;  // bytes of the tile that exist; lanes past it re-load byte 0
};

__device__ __forceinline__ TileSrc plan_tile(const Plan& P, int i, const Misc* ms) {
  switch (P.kind) {
    case PK_QKV: {
      const int row0 = (P.lo + i) * P.rpt;
      const char* b = row0 < P.a0 ? P.b0 + ((size_t)row0 << P.lrb)
                      : row0 < P.a0 + P.a1 ? P.b1 + ((size_t)(row0 - P.a0) << P.lrb)
                                           : P.b2 + ((size_t)(row0 - P.a0 - P.a1) << P.lrb);
      return TileSrc{b, kTileBytes};
    }
    case PK_ATTN: {
      const int t0 = P.a0 + (i >> 1) * kAttnTile;
      const int nv = min(kAttnTile, P.a1 - t0);
      return TileSrc{((i & 1) ? P.b1 : P.b0) + (size_t)t0 * 256, nv * 256};
    }
    case PK_WO:
      return TileSrc{P.b0 + ((size_t)(P.lo + i) * P.rpt << P.lrb), kTileBytes};
    case PK_RS: {
      if (i < P.n1) {
        const int row0 = (P.lo + i) * P.rpt;
        const int nr = min(P.rpt, P.a0 - row0);
        return TileSrc{P.b0 + ((size_t)row0 << P.lrb), nr << P.lrb};
      }
      const int k = i - P.n1;
      const int pj = P.lo2 + (k >> 1);
      const int sx = pj / P.fb_per, fb = pj % P.fb_per;
      return TileSrc{((k & 1) ? P.b2 : P.b1) + (((size_t)sx * P.F + (size_t)fb * P.rpt) << P.lrb), kTileBytes};
    }
    case PK_RG: {
      if (i < P.n1) {  // shared down: unit = j-block, S tiles per unit
        const int unit = P.lo + i / P.S, s = i % P.S;
        return TileSrc{P.b0 + (((size_t)s * P.d + (size_t)unit * P.rpt) << P.lrb), kTileBytes};
      }
      const int k = i - P.n1;
      const int pj = P.lo2 + (k >> 1);
      const int e = ms->uni[pj / P.fb_per], fb = pj % P.fb_per;
      return TileSrc{((k & 1) ? P.b2 : P.b1) + (((size_t)e * P.F + (size_t)fb * P.rpt2) << P.lrb2), kTileBytes};
    }
    case PK_DOWN: {
      const int jb = P.lo + i / P.U, u = i % P.U;
      return TileSrc{P.b0 + (((size_t)ms->uni[u] * P.d + (size_t)jb * P.rpt) << P.lrb), kTileBytes};
    }
    default:
      return TileSrc{nullptr, 0};
  }
}

template <typename WT>
__device__ __forceinline__ Plan plan_qkv(const KParams& p, int l) {
  const DevLayer& Ly = p.layers[l];
  Plan P{};
  P.kind = PK_QKV;
  P.lrb = ilog2(p.d * (int)sizeof(WT));
  P.rpt = kTileBytes >> P.lrb;
  P.a0 = p.H * p.hd;
  P.a1 = p.G * p.hd;
  int lo, hi;
  my_range((P.a0 + 2 * P.a1) / P.rpt, p.n_cu, lo, hi);
  P.lo = lo;
  P.n = hi - lo;
  P.b0 = (const char*)Ly.wq;
  P.b1 = (const char*)Ly.wk;
  P.b2 = (const char*)Ly.wv;
  return P;
}

// attention split owned by this CU (tasks never outnumber CUs)
__device__ __forceinline__ Plan plan_attn(const KParams& p, const Misc* ms, int l) {
  Plan P{};
  P.kind = PK_ATTN;
  const int S = p.n_splits;
  const int task = blockIdx.x;
  if (task >= p.n_seq * p.G * S) return P;
  const int seq = task / (p.G * S), g = (task / S) % p.G, s = task % S;
  int maxpos = 0;
  for (int rr = 0; rr < p.rps; ++rr) maxpos = max(maxpos, ms->pos[seq * p.rps + rr]);
  const int npos = maxpos + 1;
  int sl = (npos + S - 1) / S;
  sl = (sl + kAttnTile - 1) / kAttnTile * kAttnTile;
  P.a0 = s * sl;
  P.a1 = min(P.a0 + sl, npos);
  P.n = P.a1 > P.a0 ? 2 * ((P.a1 - P.a0 + kAttnTile - 1) / kAttnTile) : 0;
  const size_t kv_base = ((((size_t)l * p.n_seq + seq) * p.G + g) * (size_t)p.cap) * p.hd;
  P.b0 = reinterpret_cast<const char*>(p.kcache + kv_base);
  P.b1 = reinterpret_cast<const char*>(p.vcache + kv_base);
  P.lo = task;
  return P;
}

template <typename WT>
__device__ __forceinline__ Plan plan_wo(const KParams& p, int l) {
  Plan P{};
  P.kind = PK_WO;
  P.lrb = ilog2(p.H * p.hd * (int)sizeof(WT));
  P.rpt = kTileBytes >> P.lrb;
  int lo, hi;
  my_range(p.d / P.rpt, p.n_cu, lo, hi);
  P.lo = lo;
  P.n = hi - lo;
  P.b0 = (const char*)p.layers[l].wo;
  return P;
}

// router tiles (weight 1) then shared pairs (gate tile, up tile; weight 2),
// split by cumulative weight so that a pair never straddles two CUs
template <typename WT>
__device__ __forceinline__ Plan plan_rs(const KParams& p, int l) {
  const DevLayer& Ly = p.layers[l];
  Plan P{};
  P.kind = PK_RS;
  P.lrb = ilog2(p.d * (int)sizeof(WT));
  P.rpt = kTileBytes >> P.lrb;
  P.a0 = p.E;
  P.F = p.F;
  const int nrt = (p.E + P.rpt - 1) / P.rpt;
  P.fb_per = p.F / P.rpt;
  const int npair = p.S * P.fb_per;
  int lo, hi;
  my_range(nrt + 2 * npair, p.n_cu, lo, hi);
  const int r_lo = min(lo, nrt), r_hi = min(hi, nrt);
  auto ceil_half = [](int x) { return x <= 0 ? 0 : (x + 1) / 2; };
  const int pl = min(npair, ceil_half(lo - nrt)), ph = min(npair, ceil_half(hi - nrt));
  P.lo = r_lo;
  P.n1 = r_hi - r_lo;
  P.lo2 = pl;
  P.n = P.n1 + 2 * (ph - pl);
  P.b0 = (const char*)Ly.w_router;
  P.b1 = (const char*)Ly.s_gate;
  P.b2 = (const char*)Ly.s_up;
  return P;
}

// shared-expert down projection (j-blocks, S tiles each) then, when the
// routing is known (routed = true), the routed gate/up pairs
template <typename WT>
__device__ __forceinline__ Plan plan_rg(const KParams& p, const Misc* ms, int l, bool routed) {
  const DevLayer& Ly = p.layers[l];
  Plan P{};
  P.kind = PK_RG;
  P.lrb = ilog2(p.F * (int)sizeof(WT));
  P.rpt = kTileBytes >> P.lrb;
  P.lrb2 = ilog2(p.d * (int)sizeof(WT));
  P.rpt2 = kTileBytes >> P.lrb2;
  P.d = p.d;
  P.F = p.F;
  P.S = p.S;
  int lo, hi;
  my_range(p.S > 0 ? p.d / P.rpt : 0, p.n_cu, lo, hi);
  P.lo = lo;
  P.n1 = (hi - lo) * p.S;
  P.fb_per = p.F / P.rpt2;
  P.n = P.n1;
  if (routed) {
    int l2, h2;
    my_range(ms->n_uni * P.fb_per, p.n_cu, l2, h2);
    P.lo2 = l2;
    P.n += 2 * (h2 - l2);
  }
  P.b0 = (const char*)Ly.s_down;
  P.b1 = (const char*)Ly.w_gate;
  P.b2 = (const char*)Ly.w_up;
  return P;
}

template <typename WT>
__device__ __forceinline__ Plan plan_down(const KParams& p, const Misc* ms, int l) {
  Plan P{};
  P.kind = PK_DOWN;
  P.lrb = ilog2(p.F * (int)sizeof(WT));
  P.rpt = kTileBytes >> P.lrb;
  P.d = p.d;
  P.U = ms->n_uni;
  int lo, hi;
  my_range(p.d / P.rpt, p.n_cu, lo, hi);
  P.lo = lo;
  P.n = (hi - lo) * P.U;
  P.b0 = (const char*)p.layers[l].w_down;
  return P;
}

// ------------------------------------------------------------------ tile stream

__device__ __forceinline__ void issue_quarter(TileSrc t, char* slot, int wave, int lane) {
  const int off0 = wave * 2048 + lane * 16;
  const int off1 = off0 + 1024;
  g2l(t.g + (off0 < t.valid ? off0 : 0), slot + wave * 2048);
  g2l(t.g + (off1 < t.valid ? off1 : 0), slot + wave * 2048 + 1024);
}

// The stream of one phase followed by the next: tile j < cur.n is the
// current phase's tile j, later tiles belong to `nxt` (when its plan is
// known).  Tile j lives in ring slot (slot0 + j) % kRing and may be issued
// once tile j - kRing has been consumed.
struct Stream {
  int slot0;
  int issued;
  __device__ __forceinline__ char* slot(Smem sm, int j) const {
    return sm.ring + (size_t)((slot0 + j) % kRing) * kTileBytes;
  }
  // issue while ring slots are free; `consumed` tiles of cur are done
  __device__ __forceinline__ void fill(Smem sm, const Plan& cur, const Plan& nxt, int consumed, int wave,
                                       int lane) {
    const int limit = min(consumed + kRing, cur.n + nxt.n);
    if (issued >= limit) return;
    wait_lgkm0();  // this wave's reads of the slots being refilled are done
    const Misc* ms = sm.misc;
    for (; issued < limit; ++issued) {
      const TileSrc t = issued < cur.n ? plan_tile(cur, issued, ms) : plan_tile(nxt, issued - cur.n, ms);
      issue_quarter(t, slot(sm, issued), wave, lane);
    }
  }
  // wait until tile i of cur has landed (this wave's quarter)
  __device__ __forceinline__ void wait(int i) const { wait_tiles_ahead(issued - 1 - i); }
  // hand over to the next phase: its first tiles are already issued
  __device__ __forceinline__ void advance(const Plan& cur) {
    slot0 = (slot0 + cur.n) % kRing;
    issued -= cur.n;
  }
};

// ------------------------------------------------------------------ GEMV pieces

// Lane `lane` of wave `wave` reads bytes wave*2048 + c*1024 + lane*16 of each
// tile (c = 0, 1); with rows of 2^lrb bytes that is element k0(c) of the row.
template <typename WT>
__device__ __forceinline__ int lane_k0(int wave, int lane, int c, int lrb) {
  const int off = wave * 2048 + c * 1024 + lane * 16;
  return (off & ((1 << lrb) - 1)) / (int)sizeof(WT);
}

// x registers: the EPL activation elements each chunk of this lane meets, per token
template <typename WT, int MT>
struct XRegs {
  static constexpr int EPL = 16 / sizeof(WT);
  float v[MT][2][EPL];
};

// Fill x registers from fp32 rows: token t reads src + t*ld (+ k0); gam
// (nullable) multiplies element-wise.  Tokens >= M are zero.
template <typename WT, int MT>
__device__ __forceinline__ void load_x(XRegs<WT, MT>& xr, const float* src, int ld, const WT* gam, int M, int wave,
                                       int lane, int lrb) {
  constexpr int EPL = XRegs<WT, MT>::EPL;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int k0 = lane_k0<WT>(wave, lane, c, lrb);
    float g[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) g[j] = 1.f;
    if (gam) unpack16<WT>(*reinterpret_cast<const uint4*>(gam + k0), g);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      if (t < M) {
        const float* s = src + (size_t)t * ld + k0;
#pragma unroll
        for (int j = 0; j < EPL; j += 4) {
          const float4 a = *reinterpret_cast<const float4*>(s + j);
          xr.v[t][c][j] = a.x * g[j]; xr.v[t][c][j + 1] = a.y * g[j + 1];
          xr.v[t][c][j + 2] = a.z * g[j + 2]; xr.v[t][c][j + 3] = a.w * g[j + 3];
        }
      } else {
#pragma unroll
        for (int j = 0; j < EPL; ++j) xr.v[t][c][j] = 0.f;
      }
    }
  }
}

// One wave's quarter of a weight tile against the x registers.  For chunk c
// and token t the dot product of this wave's part of the row is summed over
// the wave and written (scaled by tw[t]; added when accum) to
// part_wave[c*MT + t].  tmask selects the tokens that take part.
template <typename WT, int MT>
__device__ __forceinline__ void gemv_quarter(const char* slot, const XRegs<WT, MT>& xr, unsigned tmask,
                                             const float (&tw)[MT], float* part_wave, bool accum, int wave,
                                             int lane) {
  constexpr int EPL = XRegs<WT, MT>::EPL;
  float acc[2 * MT];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const uint4 wv = *reinterpret_cast<const uint4*>(slot + wave * 2048 + c * 1024 + lane * 16);
    float w[EPL];
    unpack16<WT>(wv, w);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      float s = 0.f;
      if (tmask & (1u << t)) {
#pragma unroll
        for (int j = 0; j < EPL; ++j) s = fmaf(w[j], xr.v[t][c][j], s);
        s *= tw[t];
      }
      acc[c * MT + t] = s;
    }
  }
  const float r = xreduce<2 * MT>(acc, lane);
  if (xreduce_writer<2 * MT>(lane)) {
    const int idx = xreduce_index<2 * MT>(lane);
    if (accum) part_wave[idx] += r;
    else part_wave[idx] = r;
  }
}

// part block layout: [wave][c][MT]; the row of (wave, c) in a tile of
// 2^lrb-byte rows is (wave*2048 + c*1024) >> lrb.
template <int MT>
__device__ __forceinline__ float part_row(const float* part, int block, int q, int lrb, int t) {
  const float* b = part + (size_t)block * (kWaves * 2 * MT);
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w)
#pragma unroll
    for (int c = 0; c < 2; ++c)
      if (((w * 2048 + c * 1024) >> lrb) == q) s += b[(w * 2 + c) * MT + t];
  return s;
}

// Consume the tiles of GEMV phase `cur`.  pre(i, tmask, tw, accum) may
// refresh the x registers and gives tile i's token mask, token weights and
// whether it accumulates into its part block; block(i) gives the block;
// is_end(i) closes a round, after which round_end(first, last) runs with all
// waves synchronised.  The stream keeps issuing `nxt`'s tiles meanwhile.
template <typename WT, int MT, class PreFn, class BlockFn, class IsEnd, class RoundEnd>
__device__ __forceinline__ void run_gemv(Smem sm, Stream& st, const Plan& cur, const Plan& nxt, XRegs<WT, MT>& xr,
                                         PreFn pre, BlockFn block, IsEnd is_end, RoundEnd round_end) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  st.fill(sm, cur, nxt, 0, wave, lane);
  int round_first = 0;
  for (int i = 0; i < cur.n; ++i) {
    unsigned tmask;
    float tw[MT];
    bool accum;
    pre(i, tmask, tw, accum);
    st.wait(i);
    gemv_quarter<WT, MT>(st.slot(sm, i), xr, tmask, tw,
                         sm.part + (size_t)block(i) * (kWaves * 2 * MT) + wave * 2 * MT, accum, wave, lane);
    st.fill(sm, cur, nxt, i + 1, wave, lane);
    if (is_end(i)) {
      __syncthreads();
      round_end(round_first, i);
      __syncthreads();
      round_first = i + 1;
    }
  }
}

__device__ __forceinline__ void zero_part(Smem sm) {
  for (int i = threadIdx.x; i < kPartBytes / 4; i += kThreads) sm.part[i] = 0.f;
}

// 1 / sqrt(mean(h^2) + eps) per row, into misc->rinv
__device__ __forceinline__ void row_rinv(Smem sm, const float* h, int M, int d, float eps) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int t = wave; t < M; t += kWaves) {
    float s = 0.f;
    for (int i = lane * 4; i < d; i += 256) {
      const float4 v = *reinterpret_cast<const float4*>(h + (size_t)t * d + i);
      s += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    s = sum_rows(sum_row16(s));
    if (lane == 0) sm.misc->rinv[t] = 1.0f / sqrtf(s / (float)d + eps);
  }
}

template <int MT>
__device__ __forceinline__ void all_tokens(int M, unsigned& tmask, float (&tw)[MT], bool& accum) {
  tmask = (1u << M) - 1u;
#pragma unroll
  for (int t = 0; t < MT; ++t) tw[t] = 1.f;
  accum = false;
}

// ------------------------------------------------------------------ phases

// QKV: raw projections of (h * g1); the row scale rinv is applied in the epilogue.
template <typename WT, int MT>
__device__ __forceinline__ void phase_qkv(const KParams& p, Smem sm, int l, Stream& st, const Plan& P, const Plan& N) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int d = p.d, M = p.M;
  const int nrows = P.a0 + 2 * P.a1;
  const float* h = layer_in(p, l);
  float* qkv = act_w(p, l, p.al.qkv);
  XRegs<WT, MT> xr;
  load_x<WT, MT>(xr, h, d, reinterpret_cast<const WT*>(p.layers[l].attn_norm), M, wave, lane, P.lrb);
  row_rinv(sm, h, M, d, p.eps);
  zero_part(sm);
  __syncthreads();
  constexpr int kRound = (kPartBytes / 4) / (kWaves * 2 * MT);
  const Misc* ms = sm.misc;
  const int rpt = P.rpt, lo = P.lo, lrb = P.lrb, n = P.n;
  run_gemv<WT, MT>(
      sm, st, P, N, xr, [&](int, unsigned& tm, float (&tw)[MT], bool& ac) { all_tokens<MT>(M, tm, tw, ac); },
      [](int i) { return i % kRound; }, [=](int i) { return ((i + 1) % kRound) == 0 || i == n - 1; },
      [&](int first, int last) {
        const int nr = (last - first + 1) * rpt;
        for (int it = threadIdx.x; it < nr * M; it += kThreads) {
          const int q = it / M, t = it - q * M;
          const int row = (lo + first) * rpt + q;
          st_dev(qkv + (size_t)t * nrows + row, part_row<MT>(sm.part, q / rpt, q % rpt, lrb, t) * ms->rinv[t]);
        }
      });
}

// Split-KV GQA attention.  Task = (sequence, kv head, split) = this CU.
// Query vector q = rr*HG + hh is row seq*rps + rr, head g*HG + hh.  Every wave
// reads every position of a tile; wave w owns the queries q = w, w+4, ...  A
// lane covers 8 dims (lane & 15) of one position (lane >> 4) per 1 KiB chunk.
// The split's tiles may have been loaded before this step's rows reached the
// cache, so the positions written by this step are taken from LDS.
template <int QW>
__device__ __forceinline__ void phase_attn(const KParams& p, Smem sm, int l, Stream& st, const Plan& P, const Plan& N) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int HG = p.H / p.G, hd = p.hd, rps = p.rps;
  const int Q = rps * HG;
  const int S = p.n_splits;
  const int ntask = p.n_seq * p.G * S;
  const int nrows_qkv = (p.H + 2 * p.G) * hd;
  const float* qkv = act_f(p, l, p.al.qkv);
  Misc* ms = sm.misc;
  float* Qv = sm.xs;                          // [Q][hd] queries, RoPE'd and scaled
  float* newk = sm.xs + kMaxQ * 128;          // [rps][hd] this step's k rows (bf16-rounded)
  float* newv = newk + kMaxRows * 128;        // [rps][hd]
  float* coef = newv + kMaxRows * 128;        // [Q][S] combine weights
  const int task = blockIdx.x;
  const bool active = task < ntask;
  const int seq = active ? task / (p.G * S) : 0, g = active ? (task / S) % p.G : 0, s = active ? task % S : 0;
  const int p_lo = P.a0, p_hi = P.a1;
  const float scale = 1.0f / sqrtf((float)hd);
  const int d0 = (lane & 15) * 8;
  const int pg = lane >> 4;
  if (active) {
    for (int it = threadIdx.x; it < Q * (hd / 2); it += kThreads) {
      const int q = it / (hd / 2), i = it % (hd / 2);
      const int row = seq * rps + q / HG, head = g * HG + q % HG;
      const float* src = qkv + (size_t)row * nrows_qkv + head * hd;
      const float c = ms->rope[(row * 64 + i) * 2], sn = ms->rope[(row * 64 + i) * 2 + 1];
      const float x0 = src[i], x1 = src[i + hd / 2];
      Qv[q * hd + i] = (x0 * c - x1 * sn) * scale;
      Qv[q * hd + i + hd / 2] = (x1 * c + x0 * sn) * scale;
    }
    // this step's rows of the sequence inside the split: RoPE'd bf16 k, bf16 v
    uint16_t* kc = reinterpret_cast<uint16_t*>(const_cast<char*>(P.b0));
    uint16_t* vc = reinterpret_cast<uint16_t*>(const_cast<char*>(P.b1));
    for (int it = threadIdx.x; it < rps * (hd / 2); it += kThreads) {
      const int rr = it / (hd / 2), i = it % (hd / 2);
      const int row = seq * rps + rr;
      const int pos = ms->pos[row];
      if (pos < p_lo || pos >= p_hi) continue;
      const float* ksrc = qkv + (size_t)row * nrows_qkv + p.H * hd + g * hd;
      const float* vsrc = qkv + (size_t)row * nrows_qkv + (p.H + p.G) * hd + g * hd;
      const float c = ms->rope[(row * 64 + i) * 2], sn = ms->rope[(row * 64 + i) * 2 + 1];
      const float x0 = ksrc[i], x1 = ksrc[i + hd / 2];
      const uint16_t k0 = f32_to_bf16(x0 * c - x1 * sn), k1 = f32_to_bf16(x1 * c + x0 * sn);
      const uint16_t v0 = f32_to_bf16(vsrc[i]), v1 = f32_to_bf16(vsrc[i + hd / 2]);
      kc[(size_t)pos * hd + i] = k0;
      kc[(size_t)pos * hd + i + hd / 2] = k1;
      vc[(size_t)pos * hd + i] = v0;
      vc[(size_t)pos * hd + i + hd / 2] = v1;
      newk[rr * 128 + i] = __uint_as_float((uint32_t)k0 << 16);
      newk[rr * 128 + i + hd / 2] = __uint_as_float((uint32_t)k1 << 16);
      newv[rr * 128 + i] = __uint_as_float((uint32_t)v0 << 16);
      newv[rr * 128 + i + hd / 2] = __uint_as_float((uint32_t)v1 << 16);
    }
  }
  __syncthreads();
  // new positions inside this split, per sequence row (-1: none)
  int newpos[kMaxRows];
#pragma unroll
  for (int rr = 0; rr < kMaxRows; ++rr) {
    newpos[rr] = -1;
    if (active && rr < rps) {
      const int pos = ms->pos[seq * rps + rr];
      if (pos >= p_lo && pos < p_hi) newpos[rr] = pos;
    }
  }
  float qr[QW][8], acc[QW][8], m[QW], lsum[QW], pr[QW][8];
  int qlim[QW];
#pragma unroll
  for (int i = 0; i < QW; ++i) {
    const int q = wave + 4 * i;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      acc[i][j] = 0.f;
      pr[i][j] = 0.f;
      qr[i][j] = (active && q < Q) ? Qv[q * hd + d0 + j] : 0.f;
    }
    m[i] = -INFINITY;
    lsum[i] = 0.f;
    qlim[i] = (active && q < Q) ? min(p_hi - 1, ms->pos[seq * rps + q / HG]) : -1;  // last visible position
  }
  st.fill(sm, P, N, 0, wave, lane);
  for (int i = 0; i < P.n; ++i) {
    st.wait(i);
    __syncthreads();  // tile i landed for every wave; every wave is done with tile i-1
    st.fill(sm, P, N, i, wave, lane);
    const char* slot = st.slot(sm, i);
    const int t0 = p_lo + (i >> 1) * kAttnTile;
    const bool is_v = (i & 1) != 0;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int j = t0 + 4 * c + pg;
      float kf[8];
      unpack16<uint16_t>(*reinterpret_cast<const uint4*>(slot + c * 1024 + lane * 16), kf);
#pragma unroll
      for (int rr = 0; rr < kMaxRows; ++rr) {
        if (newpos[rr] == j) {
          const float* src = (is_v ? newv : newk) + rr * 128 + d0;
#pragma unroll
          for (int e = 0; e < 8; ++e) kf[e] = src[e];
        }
      }
      if (!is_v) {
#pragma unroll
        for (int i2 = 0; i2 < QW; ++i2) {
          float dsum = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) dsum = fmaf(kf[e], qr[i2][e], dsum);
          dsum = sum_row16(dsum);
          pr[i2][c] = (j <= qlim[i2]) ? dsum : -INFINITY;  // scores for now
        }
      } else {
#pragma unroll
        for (int i2 = 0; i2 < QW; ++i2)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[i2][e] = fmaf(pr[i2][c], kf[e], acc[i2][e]);
      }
    }
    if (!is_v) {
      // online softmax over this tile's 32 positions
#pragma unroll
      for (int i2 = 0; i2 < QW; ++i2) {
        float mt = pr[i2][0];
#pragma unroll
        for (int c = 1; c < 8; ++c) mt = fmaxf(mt, pr[i2][c]);
        mt = fmaxf(mt, __shfl_xor(mt, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float mn = fmaxf(m[i2], mt);
        const float corr = (mn == -INFINITY) ? 1.f : __expf(m[i2] - mn);
        float ps = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          pr[i2][c] = (pr[i2][c] == -INFINITY) ? 0.f : __expf(pr[i2][c] - mn);
          ps += pr[i2][c];
        }
        ps = sum_rows(ps);
        lsum[i2] = lsum[i2] * corr + ps;
        m[i2] = mn;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i2][j] *= corr;
      }
    }
  }
  st.fill(sm, P, N, P.n, wave, lane);
  if (!active) return;
  // sum the 4 position groups; lanes 0-15 hold acc for dims d0..d0+7
  float* part = act_w(p, l, p.al.part) + ((size_t)((seq * p.G + g) * S + s) * Q) * kPartStride;
#pragma unroll
  for (int i = 0; i < QW; ++i) {
    const int q = wave + 4 * i;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = sum_rows(acc[i][j]);
    if (q < Q && lane < 16) {
      float* dst = part + (size_t)q * kPartStride;
#pragma unroll
      for (int j = 0; j < 8; ++j) st_dev(dst + 4 + d0 + j, acc[i][j]);
      if (lane == 0) {
        st_dev(dst + 0, m[i]);
        st_dev(dst + 1, lsum[i]);
      }
    }
  }
  wait_all();
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned* cnt = p.attn_cnt + ((size_t)l * p.n_seq + seq) * p.G + g;
    const unsigned old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = (old + 1u == (unsigned)S);
    if (last) st_dev_u(cnt, 0u);
    ms->last = last;
  }
  __syncthreads();
  if (ms->last) {
    // combine the S partial softmax states of each query
    const float* pall = act_f(p, l, p.al.part) + ((size_t)((seq * p.G + g) * S) * Q) * kPartStride;
    for (int it = threadIdx.x; it < Q; it += kThreads) {
      float mx = -INFINITY;
      for (int z = 0; z < S; ++z) mx = fmaxf(mx, pall[((size_t)z * Q + it) * kPartStride]);
      float L = 0.f;
      for (int z = 0; z < S; ++z) {
        const float* pz = pall + ((size_t)z * Q + it) * kPartStride;
        const float e = pz[0] == -INFINITY ? 0.f : __expf(pz[0] - mx);
        coef[it * S + z] = e;
        L += pz[1] * e;
      }
      const float invL = 1.f / L;
      for (int z = 0; z < S; ++z) coef[it * S + z] *= invL;
    }
    __syncthreads();
    float* o = act_w(p, l, p.al.o);
    for (int it = threadIdx.x; it < Q * (hd / 4); it += kThreads) {
      const int q = it / (hd / 4), i4 = (it % (hd / 4)) * 4;
      float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
      for (int z = 0; z < S; ++z) {
        const float cz = coef[q * S + z];
        const float4 a = *reinterpret_cast<const float4*>(pall + ((size_t)z * Q + q) * kPartStride + 4 + i4);
        num.x = fmaf(cz, a.x, num.x); num.y = fmaf(cz, a.y, num.y);
        num.z = fmaf(cz, a.z, num.z); num.w = fmaf(cz, a.w, num.w);
      }
      const int row = seq * rps + q / HG, head = g * HG + q % HG;
      float* dst = o + (size_t)row * (p.H * hd) + head * hd + i4;
      st_dev(dst, num.x); st_dev(dst + 1, num.y); st_dev(dst + 2, num.z); st_dev(dst + 3, num.w);
    }
  }
}

// WO: h1 = h + Wo . o
template <typename WT, int MT>
__device__ __forceinline__ void phase_wo(const KParams& p, Smem sm, int l, Stream& st, const Plan& P, const Plan& N) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int M = p.M, d = p.d;
  const int K = p.H * p.hd;
  const float* o = act_f(p, l, p.al.o);
  const float* h = layer_in(p, l);
  float* h1 = act_w(p, l, p.al.h1);
  XRegs<WT, MT> xr;
  load_x<WT, MT>(xr, o, K, (const WT*)nullptr, M, wave, lane, P.lrb);
  zero_part(sm);
  __syncthreads();
  constexpr int kRound = (kPartBytes / 4) / (kWaves * 2 * MT);
  const int rpt = P.rpt, lo = P.lo, lrb = P.lrb, n = P.n;
  run_gemv<WT, MT>(
      sm, st, P, N, xr, [&](int, unsigned& tm, float (&tw)[MT], bool& ac) { all_tokens<MT>(M, tm, tw, ac); },
      [](int i) { return i % kRound; }, [=](int i) { return ((i + 1) % kRound) == 0 || i == n - 1; },
      [&](int first, int last) {
        const int nr = (last - first + 1) * rpt;
        for (int it = threadIdx.x; it < nr * M; it += kThreads) {
          const int q = it / M, t = it - q * M;
          const int row = (lo + first) * rpt + q;
          st_dev(h1 + (size_t)t * d + row, h[(size_t)t * d + row] + part_row<MT>(sm.part, q / rpt, q % rpt, lrb, t));
        }
      });
}

// RS: router logits and shared-expert gate/up.  The x registers (h1 * g2)
// stay loaded for the routed gate/up rows of the next phase.
template <typename WT, int MT>
__device__ __forceinline__ void phase_rs(const KParams& p, Smem sm, int l, Stream& st, const Plan& P, const Plan& N,
                         XRegs<WT, MT>& xr) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const DevLayer& Ly = p.layers[l];
  const int d = p.d, F = p.F, E = p.E, M = p.M, S = p.S;
  const float* h1 = layer_h1(p, l);
  const float* br = Ly.b_router;
  const int has_bias = p.has_bias;
  float* logits = act_w(p, l, p.al.logits);
  float* a_s = act_w(p, l, p.al.a_s);
  load_x<WT, MT>(xr, h1, d, reinterpret_cast<const WT*>(Ly.moe_norm), M, wave, lane, P.lrb);
  row_rinv(sm, h1, M, d, p.eps);
  zero_part(sm);
  __syncthreads();
  constexpr int kRound = ((kPartBytes / 4) / (kWaves * 2 * MT)) & ~1;  // even: a pair stays in one round
  const Misc* ms = sm.misc;
  const int rpt = P.rpt, lrb = P.lrb, n1 = P.n1, n = P.n, r_lo = P.lo, p_lo = P.lo2, fb_per = P.fb_per;
  run_gemv<WT, MT>(
      sm, st, P, N, xr, [&](int, unsigned& tm, float (&tw)[MT], bool& ac) { all_tokens<MT>(M, tm, tw, ac); },
      [=](int i) { return i < n1 ? i % kRound : (i - n1) % kRound; },
      [=](int i) {
        if (i == n - 1) return true;
        if (i < n1) return i == n1 - 1 || ((i + 1) % kRound) == 0;
        return ((i - n1 + 1) % kRound) == 0;
      },
      [&](int first, int last) {
        if (first < n1) {
          const int nr = (last - first + 1) * rpt;
          for (int it = threadIdx.x; it < nr * M; it += kThreads) {
            const int q = it / M, t = it - q * M;
            const int e = (r_lo + first) * rpt + q;
            if (e >= E) continue;
            float v = part_row<MT>(sm.part, q / rpt, q % rpt, lrb, t) * ms->rinv[t];
            if (has_bias) v += br[e];
            st_dev(logits + (size_t)t * E + e, v);
          }
        } else {
          const int k0 = first - n1;
          const int npairs_r = (last - first + 1) / 2;
          for (int it = threadIdx.x; it < npairs_r * rpt * M; it += kThreads) {
            const int pr = it / (rpt * M), q = (it / M) % rpt, t = it % M;
            const int pj = p_lo + k0 / 2 + pr;
            const int sx = pj / fb_per, f = (pj % fb_per) * rpt + q;
            const float ri = ms->rinv[t];
            const float gv = part_row<MT>(sm.part, 2 * pr, q, lrb, t) * ri;
            const float uv = part_row<MT>(sm.part, 2 * pr + 1, q, lrb, t) * ri;
            st_dev(a_s + ((size_t)t * S + sx) * F + f, gv / (1.f + __expf(-gv)) * uv);
          }
        }
      });
}

// Top-k over the router logits of every row (all CUs, redundantly), then the
// union of chosen experts.  Selection is on the logits, larger first, equal
// logits ranked by lower expert id; weights are softmax probabilities
// renormalised over the chosen set.
__device__ __forceinline__ void route_topk(const KParams& p, Smem sm, int l) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int E = p.E, k = p.k, M = p.M;
  const float* logits = act_f(p, l, p.al.logits);
  Misc* ms = sm.misc;
  for (int e = threadIdx.x; e < kMaxExperts; e += kThreads) ms->used[e] = 0;
  __syncthreads();
  for (int t = wave; t < M; t += kWaves) {
    const float z = lane < E ? logits[(size_t)t * E + lane] : -INFINITY;
    bool taken = lane >= E;
    const float zmax = wave_max(z);
    const float pz = lane < E ? __expf(z - zmax) : 0.f;
    float psum = 0.f;
    int sel[kMaxTopK];
#pragma unroll
    for (int i = 0; i < kMaxTopK; ++i) {
      sel[i] = 0;
      if (i < k) {
        float bz = taken ? -INFINITY : z;
        int bi = taken ? 1 << 30 : lane;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
          const float oz = __shfl_xor(bz, o);
          const int oi = __shfl_xor(bi, o);
          if (oz > bz || (oz == bz && oi < bi)) { bz = oz; bi = oi; }
        }
        if (lane == bi) taken = true;
        sel[i] = bi;
        psum += __shfl(pz, bi);
      }
    }
#pragma unroll
    for (int i = 0; i < kMaxTopK; ++i) {
      if (i < k) {
        const int e = sel[i];
        const float pe = __shfl(pz, e);
        if (lane == 0) {
          ms->ids[t * k + i] = e;
          ms->wts[t * k + i] = pe / psum;
          ms->used[e] = 1;
        }
      }
    }
  }
  __syncthreads();
  if (wave == 0) {
    const bool u = lane < E && ms->used[lane];
    const unsigned long long mm = __ballot(u);
    if (u) ms->uni[__popcll(mm & ((1ull << lane) - 1ull))] = lane;
    if (lane == 0) ms->n_uni = __popcll(mm);
  }
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int i = threadIdx.x; i < M * k; i += kThreads) {
      if (p.t_ids) p.t_ids[(size_t)l * M * k + i] = ms->ids[i];
      if (p.t_w) p.t_w[(size_t)l * M * k + i] = ms->wts[i];
    }
    if (p.t_logits)
      for (int i = threadIdx.x; i < M * E; i += kThreads) p.t_logits[(size_t)l * M * E + i] = logits[i];
  }
}

// slot of expert e in row t's top-k list, or -1
__device__ __forceinline__ int slot_of(const Misc* ms, int t, int k, int e) {
  for (int i = 0; i < k; ++i)
    if (ms->ids[t * k + i] == e) return i;
  return -1;
}
__device__ __forceinline__ unsigned routed_mask(const Misc* ms, int M, int k, int e) {
  unsigned m = 0;
  for (int t = 0; t < M; ++t)
    if (slot_of(ms, t, k, e) >= 0) m |= 1u << t;
  return m;
}

// x registers for one tile from LDS rows: token t uses row rows[t] of [M][..][F]
template <typename WT, int MT>
__device__ __forceinline__ void load_x_lds(XRegs<WT, MT>& xr, const float* base, const int (&rowoff)[MT],
                                           unsigned tm, int wave, int lane, int lrb) {
  constexpr int EPL = XRegs<WT, MT>::EPL;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int k0 = lane_k0<WT>(wave, lane, c, lrb);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      if (tm & (1u << t)) {
        const float* s = base + rowoff[t] + k0;
#pragma unroll
        for (int j = 0; j < EPL; j += 4) {
          const float4 a4 = *reinterpret_cast<const float4*>(s + j);
          xr.v[t][c][j] = a4.x; xr.v[t][c][j + 1] = a4.y; xr.v[t][c][j + 2] = a4.z; xr.v[t][c][j + 3] = a4.w;
        }
      }
    }
  }
}

// RG: shared-expert down projection y_s = sum_s Wd_s a_s (x from LDS), then
// the routed gate/up rows for the union experts (x registers from RS):
// a[t][slot][f] for rows routed to the expert.
template <typename WT, int MT>
__device__ __forceinline__ void phase_rg(const KParams& p, Smem sm, int l, Stream& st, const Plan& P, const Plan& N,
                         XRegs<WT, MT>& xr) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int d = p.d, F = p.F, k = p.k, M = p.M, S = p.S;
  const float* h1 = layer_h1(p, l);
  const float* as_g = act_f(p, l, p.al.a_s);
  float* a = act_w(p, l, p.al.a);
  float* ys = act_w(p, l, p.al.y_s);
  row_rinv(sm, h1, M, d, p.eps);
  // shared activations a_s [M][S][F] -> LDS
  for (int i = threadIdx.x; i < M * S * F / 4; i += kThreads)
    reinterpret_cast<float4*>(sm.xs)[i] = reinterpret_cast<const float4*>(as_g)[i];
  zero_part(sm);
  __syncthreads();
  const Misc* ms = sm.misc;
  XRegs<WT, MT> xsd;
  constexpr int kRound = ((kPartBytes / 4) / (kWaves * 2 * MT)) & ~1;
  const int n1 = P.n1, n = P.n, lrb = P.lrb, lrb2 = P.lrb2, rpt = P.rpt, rpt2 = P.rpt2, fb_per = P.fb_per;
  const int sd_lo = P.lo, p_lo = P.lo2;
  // shared-down units (S tiles, accumulated) use blocks 0.. of the first round
  auto pre = [&](int i, unsigned& tm, float (&tw)[MT], bool& ac) {
#pragma unroll
    for (int t = 0; t < MT; ++t) tw[t] = 1.f;
    if (i < n1) {
      const int sx = i % S;
      tm = (1u << M) - 1u;
      int ro[MT];
#pragma unroll
      for (int t = 0; t < MT; ++t) ro[t] = (t * S + sx) * F;
      load_x_lds<WT, MT>(xsd, sm.xs, ro, tm, wave, lane, lrb);
      ac = true;
    } else {
      const int pj = p_lo + ((i - n1) >> 1);
      tm = routed_mask(ms, M, k, ms->uni[pj / fb_per]);
      ac = false;
    }
  };
  {
    st.fill(sm, P, N, 0, wave, lane);
    int round_first = 0;
    for (int i = 0; i < n; ++i) {
      unsigned tmask;
      float tw[MT];
      bool accum;
      pre(i, tmask, tw, accum);
      const int blk = i < n1 ? (i / S) : (i - n1) % kRound;
      st.wait(i);
      gemv_quarter<WT, MT>(st.slot(sm, i), i < n1 ? xsd : xr, tmask, tw,
                           sm.part + (size_t)blk * (kWaves * 2 * MT) + wave * 2 * MT, accum, wave, lane);
      st.fill(sm, P, N, i + 1, wave, lane);
      const bool end = (i == n - 1) || (i == n1 - 1) || (i >= n1 && ((i - n1 + 1) % kRound) == 0);
      if (end) {
        __syncthreads();
        if (round_first < n1) {
          // shared-down j-blocks of this CU: y_s[t][j]
          const int nunits = n1 / S;
          for (int it = threadIdx.x; it < nunits * rpt * M; it += kThreads) {
            const int u = it / (rpt * M), q = (it / M) % rpt, t = it % M;
            const int j = (sd_lo + u) * rpt + q;
            st_dev(ys + (size_t)t * d + j, part_row<MT>(sm.part, u, q, lrb, t));
          }
          __syncthreads();
          for (int z = threadIdx.x; z < kPartBytes / 4; z += kThreads) sm.part[z] = 0.f;
        } else {
          const int k0 = round_first - n1;
          const int npairs_r = (i - round_first + 1) / 2;
          for (int it = threadIdx.x; it < npairs_r * rpt2 * M; it += kThreads) {
            const int pr = it / (rpt2 * M), q = (it / M) % rpt2, t = it % M;
            const int pj = p_lo + k0 / 2 + pr;
            const int e = ms->uni[pj / fb_per], f = (pj % fb_per) * rpt2 + q;
            const int sl = slot_of(ms, t, k, e);
            if (sl < 0) continue;
            const float ri = ms->rinv[t];
            const float gv = part_row<MT>(sm.part, 2 * pr, q, lrb2, t) * ri;
            const float uv = part_row<MT>(sm.part, 2 * pr + 1, q, lrb2, t) * ri;
            st_dev(a + ((size_t)t * k + sl) * F + f, gv / (1.f + __expf(-gv)) * uv);
          }
        }
        __syncthreads();
        round_first = i + 1;
      }
    }
  }
}

// DOWN: for this CU's blocks of output columns j, accumulate the union
// experts (each row weighted by its routing weight), then
// h2 = h1 + y_s + sum.  x rows a[t][slot] come from LDS when they fit.
template <typename WT, int MT>
__device__ __forceinline__ void phase_down(const KParams& p, Smem sm, int l, Stream& st, const Plan& P, const Plan& N) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int d = p.d, F = p.F, k = p.k, M = p.M;
  const int U = P.U, rpt = P.rpt, lrb = P.lrb, lo = P.lo;
  const float* h1 = layer_h1(p, l);
  const float* a_g = act_f(p, l, p.al.a);    // [M][k][F]
  const float* ys = act_f(p, l, p.al.y_s);   // [M][d]
  float* h2 = (l == p.L - 1) ? p.hidden_out : act_w(p, l, p.al.h2);
  const bool last_layer = (l == p.L - 1);
  const bool xl = (size_t)M * k * F * 4 <= (size_t)kXsBytes;
  if (xl)
    for (int i = threadIdx.x; i < M * k * F / 4; i += kThreads)
      reinterpret_cast<float4*>(sm.xs)[i] = reinterpret_cast<const float4*>(a_g)[i];
  zero_part(sm);
  __syncthreads();
  const Misc* ms = sm.misc;
  const bool has_shared = p.S > 0;
  XRegs<WT, MT> xr;
  run_gemv<WT, MT>(
      sm, st, P, N, xr,
      [&](int i, unsigned& tm, float (&tw)[MT], bool& ac) {
        const int e = ms->uni[i % U];
        tm = 0;
        int ro[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          tw[t] = 0.f;
          ro[t] = 0;
          if (t < M) {
            const int sl = slot_of(ms, t, k, e);
            if (sl >= 0) {
              ro[t] = (t * k + sl) * F;
              tw[t] = ms->wts[t * k + sl];
              tm |= 1u << t;
            }
          }
        }
        if (xl) load_x_lds<WT, MT>(xr, sm.xs, ro, tm, wave, lane, lrb);
        else load_x_lds<WT, MT>(xr, a_g, ro, tm, wave, lane, lrb);
        ac = true;
      },
      [](int) { return 0; }, [=](int i) { return ((i + 1) % U) == 0; },
      [&](int first, int) {
        const int jb = lo + first / U;
        for (int it = threadIdx.x; it < rpt * M; it += kThreads) {
          const int q = it / M, t = it - q * M;
          const int j = jb * rpt + q;
          float out = h1[(size_t)t * d + j] + part_row<MT>(sm.part, 0, q, lrb, t);
          if (has_shared) out += ys[(size_t)t * d + j];
          if (last_layer) h2[(size_t)t * d + j] = out;
          else st_dev(h2 + (size_t)t * d + j, out);
        }
        __syncthreads();
        for (int i = threadIdx.x; i < kWaves * 2 * MT; i += kThreads) sm.part[i] = 0.f;
      });
}

// ------------------------------------------------------------------ kernel

template <typename WT, int MT, int QW>
__global__ void __launch_bounds__(kThreads, 1) decode_step_kernel(KParams kp) {
  Smem sm;
  sm.ring = smem_raw;
  sm.xs = reinterpret_cast<float*>(smem_raw + (size_t)kRing * kTileBytes);
  sm.part = reinterpret_cast<float*>(smem_raw + (size_t)kRing * kTileBytes + kXsBytes);
  sm.misc = reinterpret_cast<Misc*>(smem_raw + (size_t)kRing * kTileBytes + kXsBytes + kPartBytes);
  Misc* ms = sm.misc;
  const KParams& p = kp;
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
    ms->epoch = (int)ld_dev(p.sync + SyncLayout::kEpoch);
  }
  __syncthreads();
  if (ms->flag) {
    if (blockIdx.x == 0 && threadIdx.x == 0)
      __hip_atomic_fetch_or(p.sync + SyncLayout::kErr, (unsigned)ms->flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  if (p.attn) {
    // RoPE table: angle = pos * theta^(-2i/hd), evaluated in double, rounded to fp32
    for (int it = threadIdx.x; it < p.M * (p.hd / 2); it += kThreads) {
      const int r = it / (p.hd / 2), i = it % (p.hd / 2);
      const double inv = pow((double)p.theta, -2.0 * i / (double)p.hd);
      const double a = (double)ms->pos[r] * inv;
      ms->rope[(r * 64 + i) * 2] = (float)cos(a);
      ms->rope[(r * 64 + i) * 2 + 1] = (float)sin(a);
    }
  }
  const unsigned epoch0 = (unsigned)ms->epoch;
  __syncthreads();
  unsigned b = 0;
  long long* stamp = p.stamps ? p.stamps + (size_t)blockIdx.x * 2 * (p.barriers + 1) : nullptr;
  auto mark = [&](int slot) {
    if (stamp && threadIdx.x == 0) stamp[slot] = wall_clock64();
  };
  // phase i starts at slot 2i (after barrier i) and ends at slot 2i+1
#define MK_SYNC()                                   \
  do {                                              \
    mark(2 * (int)b + 1);                           \
    if (!grid_sync(p, sm, epoch0 + ++b)) return;    \
    mark(2 * (int)b);                               \
  } while (0)
  mark(0);
  XRegs<WT, MT> xr_moe;
  Stream st{0, 0};
  const Plan none{};
  Plan cur = p.attn ? plan_qkv<WT>(p, 0) : plan_rs<WT>(p, 0);
  for (int l = 0; l < p.L; ++l) {
    if (p.attn) {
      {
        const Plan nxt = plan_attn(p, ms, l);
        phase_qkv<WT, MT>(p, sm, l, st, cur, nxt);
        MK_SYNC();
        st.advance(cur);
        cur = nxt;
      }
      {
        const Plan nxt = plan_wo<WT>(p, l);
        phase_attn<QW>(p, sm, l, st, cur, nxt);
        MK_SYNC();
        st.advance(cur);
        cur = nxt;
      }
      {
        const Plan nxt = plan_rs<WT>(p, l);
        phase_wo<WT, MT>(p, sm, l, st, cur, nxt);
        MK_SYNC();
        st.advance(cur);
        cur = nxt;
      }
    }
    {
      const Plan nxt = plan_rg<WT>(p, ms, l, false);  // shared down only: routing not known yet
      phase_rs<WT, MT>(p, sm, l, st, cur, nxt, xr_moe);
      MK_SYNC();
      st.advance(cur);
    }
    {
      route_topk(p, sm, l);
      cur = plan_rg<WT>(p, ms, l, true);  // same first tiles as the prefetched plan
      const Plan nxt = plan_down<WT>(p, ms, l);
      phase_rg<WT, MT>(p, sm, l, st, cur, nxt, xr_moe);
      MK_SYNC();
      st.advance(cur);
      cur = nxt;
    }
    {
      const Plan nxt = (l + 1 < p.L) ? (p.attn ? plan_qkv<WT>(p, l + 1) : plan_rs<WT>(p, l + 1)) : none;
      phase_down<WT, MT>(p, sm, l, st, cur, nxt);
      if (l + 1 < p.L) MK_SYNC();
      st.advance(cur);
      cur = nxt;
    }
  }
#undef MK_SYNC
  wait_all();
  mark(2 * (int)b + 1);
  if (blockIdx.x == 0 && threadIdx.x == 0) st_dev_u(p.sync + SyncLayout::kEpoch, epoch0 + b);
}

}  // namespace mk

extern "C" int mk_launch_kernel(const mk::KParams* pp, void* stream) {
  using namespace mk;
  KParams p = *pp;
  const size_t lds = (size_t)kLdsTotal;
  if (p.M > kMaxRows) return -2;
  if (p.attn && p.n_seq * p.G * p.n_splits > p.n_cu) return -2;
  const int Q = p.attn ? p.q_per_task : 0;
  const void* fn;
  int idx;
  // instantiations: weight dtype x token group (1 or 8) x queries per wave (1 or 8)
  if (p.wide) {
    fn = p.M == 1 ? (const void*)decode_step_kernel<float, 1, 1> : (const void*)decode_step_kernel<float, 8, 1>;
    idx = p.M == 1 ? 0 : 1;
  } else if (Q <= 4) {
    fn = p.M == 1 ? (const void*)decode_step_kernel<uint16_t, 1, 1> : (const void*)decode_step_kernel<uint16_t, 8, 1>;
    idx = p.M == 1 ? 2 : 3;
  } else {
    if (Q > 4 * 8) return -2;
    fn = (const void*)decode_step_kernel<uint16_t, 8, 8>;
    idx = 4;
  }
  static bool attr_done[5] = {false, false, false, false, false};
  if (!attr_done[idx]) {
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess) return -1;
    attr_done[idx] = true;
  }
  void* args[] = {&p};
  hipError_t e = hipLaunchCooperativeKernel(fn, dim3(p.n_cu), dim3(kThreads), args, (unsigned)lds, (hipStream_t)stream);
  return e == hipSuccess ? 0 : (int)e;
}
