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

// wave index as a wave-uniform (scalar) value
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

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
// 64-bit word = float value (low half) and launch tag (high half), written
// and read as one single-copy-atomic access, so a reader that sees this
// launch's tag also sees the value stored with it
typedef unsigned long long tagword_t;
__device__ __forceinline__ void st_tag(tagword_t* p, float v, unsigned tag) {
  __hip_atomic_store(p, ((tagword_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// one tag word by buffer load with cache policy CPOL (a single 8-byte access)
constexpr int kCpolSc1 = 16;
constexpr int kBufferDword3 = 0x00020000;  // raw 32-bit buffer descriptor word 3 (gfx9)
template <int CPOL>
__device__ __forceinline__ tagword_t ld_word(__amdgpu_buffer_rsrc_t r, int off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, CPOL);
  return ((tagword_t)v[1] << 32) | v[0];
}

// 16 bytes per lane, global -> LDS at (wave-uniform base + lane*16),
// nontemporal.  Issued from inline assembly on purpose: the compiler's
// wait-count pass cannot tell LDS DMA destinations apart from other LDS data,
// so for a DMA it can see it puts a full vector-memory drain in front of
// every later LDS access, which would serialise the ring.  Here the ring's
// waits are all explicit (wait_tiles_ahead / wait_all), and every wait is a
// compiler memory barrier so no LDS read of a slot moves above it.  M0 is
// set here and nowhere else in the kernel (no LDS DMA builtins, no
// dynamically indexed register arrays), so the clobber cannot disturb it.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}
__device__ __forceinline__ void g2l(const void* g, unsigned lds_wave_base) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(lds_wave_base);
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %0, off nt"
      :
      : "v"(g), "s"(m0)
      : "memory", "m0");
}

// Two 1 KiB chunks: g -> LDS base and g + 1024 -> base + 1024 (the
// instruction offset applies to the global and the LDS address alike), one
// M0 write for both.  keep: without the nontemporal hint, so that the lines
// stay in the caches for other workgroups that load the same tile (row
// groups of one launch); nontemporal otherwise (every tile is read once).
__device__ __forceinline__ void g2l2(const void* g, unsigned lds_wave_base, bool keep) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(lds_wave_base);
  if (keep) {
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "global_load_lds_dwordx4 %0, off\n\t"
        "global_load_lds_dwordx4 %0, off offset:1024"
        :
        : "v"(g), "s"(m0)
        : "memory", "m0");
  } else {
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "global_load_lds_dwordx4 %0, off nt\n\t"
        "global_load_lds_dwordx4 %0, off offset:1024 nt"
        :
        : "v"(g), "s"(m0)
        : "memory", "m0");
  }
}

// s_waitcnt with compiler memory-barrier semantics
#define MK_WAIT_ASM(text) asm volatile(text ::: "memory")
__device__ __forceinline__ void wait_all() { MK_WAIT_ASM("s_waitcnt vmcnt(0) expcnt(0) lgkmcnt(0)"); }
// Wait for everything, through the builtin the compiler's wait-count pass
// understands: called before each tile loop, it leaves no compiler-visible
// load pending, so the pass puts no waits inside the loop (which, not seeing
// the ring's loads, would otherwise drain the ring every tile).
__device__ __forceinline__ void settle() { __builtin_amdgcn_s_waitcnt(0); }
__device__ __forceinline__ void wait_lgkm0() { MK_WAIT_ASM("s_waitcnt lgkmcnt(0)"); }
// wait until at most 2*ahead vector-memory operations of this wave are outstanding
__device__ __forceinline__ void wait_tiles_ahead(int ahead) {
  static_assert(2 * (kRing - 1) <= 63, "vmcnt range");
  if (ahead >= kRing - 1) {
    MK_WAIT_ASM("s_waitcnt vmcnt(22)");
    return;
  }
  if (ahead >= 8) {  // steady state of the grouped GEMV loop; conservative above 8
    MK_WAIT_ASM("s_waitcnt vmcnt(16)");
    return;
  }
  switch (ahead) {
#define MK_CASE(k, n)          \
  case k:                      \
    MK_WAIT_ASM("s_waitcnt vmcnt(" #n ")"); \
    break;
    MK_CASE(1, 2) MK_CASE(2, 4) MK_CASE(3, 6) MK_CASE(4, 8) MK_CASE(5, 10) MK_CASE(6, 12) MK_CASE(7, 14)
    MK_CASE(8, 16) MK_CASE(9, 18) MK_CASE(10, 20)
#undef MK_CASE
    default:
      MK_WAIT_ASM("s_waitcnt vmcnt(0)");
  }
}
static_assert(kRing == 12, "wait_tiles_ahead is written for a ring of 12 tiles");

__device__ __forceinline__ int ilog2(int x) { return 31 - __builtin_clz(x); }

// Tasks of a row-group launch: an expert's list of pairs is cut into pieces
// of at most kMaxRows, so there are at most E + (rows * k) / kMaxRows.
constexpr int kMaxTasks = kMaxExperts + kMaxGroups * kMaxTopK;

// ------------------------------------------------------------------ LDS carve-up

struct Misc {
  int pos[kMaxRows];
  int ids[kMaxRows * kMaxTopK];
  float wts[kMaxRows * kMaxTopK];
  int uni[kMaxExperts];
  int n_uni;
  int flag;
  int last;
  int epoch;
  unsigned tag;         // this launch's tag: the tag epoch at launch start, plus one
  int gbad[2][kWaves];  // split combine: per wave, words not yet of this launch (by round parity)
  float rinv[kMaxRows];
  float ssq[kWaves * kMaxRows];
  unsigned umask[kMaxExperts];                 // union expert u: rows routed to it
  signed char uslot[kMaxExperts * kMaxRows];   // [u][t]: top-k slot of expert u in row t, or -1
  float rope[kMaxRows * 64 * 2];  // (cos, sin) per row and frequency (head_dim 128)
  // Row-group launches: the routed work as tasks, each an expert and at most
  // kMaxRows of the (row, top-k slot) pairs of all groups routed to it.
  // tent: entries expert << 9 | row << 3 | slot (row = group * M + row in
  // group), by expert, rows ascending; task t owns tent[tbeg[t] .. tbeg[t+1]).
  unsigned short tent[kMaxGroups * kMaxRows * kMaxTopK];
  unsigned short tbeg[kMaxTasks + 2];
  int n_task;
  float rinv_row[kMaxGroups * kMaxRows];  // 1/rms of h1 per row, set when a task's rows are loaded
  float task_w[kMaxRows];                 // routing weights of the current task's pairs (DOWN)
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
// workgroup leaves the kernel at its next barrier.  Cross-CU data is written
// with device-scope stores to write-once locations, and every wave waits for
// its stores before the arrival; readers use plain loads after the barrier.
__device__ __forceinline__ bool grid_sync(const KParams& p, Smem sm, unsigned target) {
  // Release: every wave's device-scope stores of the phase have completed
  // before the arrival can be seen.  Vector memory has one counter on this
  // chip, so this also waits for the ring loads the wave has in flight.
  wait_all();
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

// The weight-pointer table is written by the host before the launch and never
// by the kernel, so it is read through the constant address space: uniform
// reads become scalar loads, which count on lgkmcnt and do not wait behind
// the ring's outstanding vector-memory loads.
typedef const __attribute__((address_space(4))) DevLayer* ConstLayers;
__device__ __forceinline__ ConstLayers layer_tab(const KParams& p) { return (ConstLayers)p.layers; }


// Row groups (several sequences of a verify pass in one launch).  Workgroup b
// runs on XCD b % 8; group g's position c (0 <= c < vncu) is workgroup
// 8 * (g * cpx + c % cpx) + c / cpx, cpx = vncu / 8, so position c of every
// group sits on the same XCD and the groups' loads of one weight tile (the
// same tile for position c of every group) meet in that XCD's L2.
__device__ __forceinline__ int grp_of(const KParams& p) {
  return p.n_groups == 1 ? 0 : (int)(blockIdx.x >> 3) >> p.cpx_log2;
}
__device__ __forceinline__ int vcu_of(const KParams& p) {
  if (p.n_groups == 1) return (int)blockIdx.x;
  return (int)((blockIdx.x & 7) << p.cpx_log2) + (int)((blockIdx.x >> 3) & ((1u << p.cpx_log2) - 1));
}

__device__ __forceinline__ const float* act_f(const KParams& p, int l, size_t off) {
  return reinterpret_cast<const float*>(p.act + (size_t)grp_of(p) * p.act_gstride + (size_t)l * p.al.stride + off);
}
__device__ __forceinline__ float* act_w(const KParams& p, int l, size_t off) {
  return reinterpret_cast<float*>(p.act + (size_t)grp_of(p) * p.act_gstride + (size_t)l * p.al.stride + off);
}
// this group's rows of the step's input and output
__device__ __forceinline__ const float* hidden_in_g(const KParams& p) {
  return p.hidden_in + (size_t)grp_of(p) * p.M * p.d;
}
__device__ __forceinline__ float* hidden_out_g(const KParams& p) {
  return p.hidden_out + (size_t)grp_of(p) * p.M * p.d;
}
__device__ __forceinline__ const float* layer_in(const KParams& p, int l) {
  return l == 0 ? hidden_in_g(p) : act_f(p, l - 1, p.al.h2);
}
// h1 of layer l: the attention block's output, or the layer input when the
// stack has no attention
__device__ __forceinline__ const float* layer_h1(const KParams& p, int l) {
  return p.attn ? act_f(p, l, p.al.h1) : layer_in(p, l);
}
// The same for any row group g of the launch (tasks of a row-group launch
// read and write the rows of every group).
__device__ __forceinline__ char* grp_act(const KParams& p, int g, int l) {
  return p.act + (size_t)g * p.act_gstride + (size_t)l * p.al.stride;
}
__device__ __forceinline__ const float* grp_h1(const KParams& p, int g, int l) {
  if (p.attn) return reinterpret_cast<const float*>(grp_act(p, g, l) + p.al.h1);
  if (l == 0) return p.hidden_in + (size_t)g * p.M * p.d;
  return reinterpret_cast<const float*>(grp_act(p, g, l - 1) + p.al.h2);
}
// every group's routing of layer l (in group 0's workspace)
__device__ __forceinline__ int* rtab_ids(const KParams& p, int l) {
  return reinterpret_cast<int*>(grp_act(p, 0, l) + p.al.rtab);
}
__device__ __forceinline__ float* rtab_wts(const KParams& p, int l) {
  return reinterpret_cast<float*>(rtab_ids(p, l) + (size_t)p.n_groups * p.M * p.k);
}
// a task entry's parts: expert, row of the launch, top-k slot
__device__ __forceinline__ int ent_expert(unsigned en) { return (int)(en >> 9); }
__device__ __forceinline__ int ent_row(unsigned en) { return (int)((en >> 3) & 63u); }
__device__ __forceinline__ int ent_slot(unsigned en) { return (int)(en & 7u); }
// q = a / b, r = a % b for 0 <= a < 2^24, 1 <= b and a / b < 2^22: the float
// estimate of the quotient is within one of the truth, and one correction
// each way makes it exact.  A few instructions instead of the generic
// integer division's dozens (code size matters: the kernel streams through
// more instructions per layer than the instruction cache holds).
struct QR {
  int q, r;
};
__device__ __forceinline__ QR divmod_small(int a, int b) {
  int q = (int)((float)a * __builtin_amdgcn_rcpf((float)b));
  int r = a - q * b;
  if (r < 0) {
    q -= 1;
    r += b;
  }
  if (r >= b) {
    q += 1;
    r -= b;
  }
  return QR{q, r};
}
// balanced split of n items over the group's workgroups (c * n stays below 2^32)
__device__ __forceinline__ void my_range(int n, const KParams& p, int& lo, int& hi) {
  const unsigned c = (unsigned)vcu_of(p), ncu = (unsigned)p.vncu;
  lo = (int)((c * (unsigned)n) / ncu);
  hi = (int)(((c + 1) * (unsigned)n) / ncu);
}

// ------------------------------------------------------------------ phase plans
//
// A plan lists the 8 KiB tiles one CU streams in one phase, in order.  Plans
// of static phases can be built before the phase starts, which is what lets
// the ring run ahead across phase boundaries.

enum PlanKind { PK_NONE = 0, PK_QKV, PK_ATTN, PK_WO, PK_RS, PK_RG, PK_DOWN, PK_DOWNA, PK_RGT, PK_DOWNT };

struct Plan {
  int kind;
  int n;             // tiles
  int lo;            // first unit of the first segment
  int lrb, rpt;      // first segment: log2 row bytes, rows per tile
  int n1;            // tiles of the first segment (RS: router; RG: shared down)
  int lo2;           // first unit of the second segment
  int lrb2, rpt2;    // second segment geometry (RS, RG)
  int fb_per;        // f-blocks per expert in the second segment
  int nj;            // RG: shared-down units; DOWN: this CU's j-blocks; DOWNA: j-blocks per expert
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
      const QR sf = divmod_small(pj, P.fb_per);
      const int sx = sf.q, fb = sf.r;
      return TileSrc{((k & 1) ? P.b2 : P.b1) + (((size_t)sx * P.F + (size_t)fb * P.rpt) << P.lrb), kTileBytes};
    }
    case PK_RG: {
      if (i < P.n1) {  // shared down, expert-major: tile = s * nj + unit
        const QR su = divmod_small(i, P.nj);
        const int s = su.q, unit = P.lo + su.r;
        return TileSrc{P.b0 + (((size_t)s * P.d + (size_t)unit * P.rpt) << P.lrb), kTileBytes};
      }
      const int k = i - P.n1;
      const int pj = P.lo2 + (k >> 1);
      const QR ef = divmod_small(pj, P.fb_per);
      const int e = ms->uni[ef.q], fb = ef.r;
      return TileSrc{((k & 1) ? P.b2 : P.b1) + (((size_t)e * P.F + (size_t)fb * P.rpt2) << P.lrb2), kTileBytes};
    }
    case PK_DOWN: {  // expert-major: tile = u * nj + (jb - lo)
      const QR uj = divmod_small(i, P.nj);
      const int u = uj.q, jb = P.lo + uj.r;
      return TileSrc{P.b0 + (((size_t)ms->uni[u] * P.d + (size_t)jb * P.rpt) << P.lrb), kTileBytes};
    }
    case PK_DOWNA: {  // flat (union expert, j-block) index, expert-major
      const QR uj = divmod_small(P.lo + i, P.nj);
      const int u = uj.q, jb = uj.r;
      return TileSrc{P.b0 + (((size_t)ms->uni[u] * P.d + (size_t)jb * P.rpt) << P.lrb), kTileBytes};
    }
    case PK_RGT: {  // shared down as PK_RG, then (task, f-block) pairs
      if (i < P.n1) {
        const QR su = divmod_small(i, P.nj);
        const int s = su.q, unit = P.lo + su.r;
        return TileSrc{P.b0 + (((size_t)s * P.d + (size_t)unit * P.rpt) << P.lrb), kTileBytes};
      }
      const int k = i - P.n1;
      const QR tf = divmod_small(P.lo2 + (k >> 1), P.fb_per);
      const int e = ent_expert(ms->tent[ms->tbeg[tf.q]]), fb = tf.r;
      return TileSrc{((k & 1) ? P.b2 : P.b1) + (((size_t)e * P.F + (size_t)fb * P.rpt2) << P.lrb2), kTileBytes};
    }
    case PK_DOWNT: {  // flat (task, j-block) index, task-major
      const QR tj = divmod_small(P.lo + i, P.nj);
      const int e = ent_expert(ms->tent[ms->tbeg[tj.q]]), jb = tj.r;
      return TileSrc{P.b0 + (((size_t)e * P.d + (size_t)jb * P.rpt) << P.lrb), kTileBytes};
    }
    default:
      return TileSrc{nullptr, 0};
  }
}
// plan_tile for a plan of kind K known at compile time (the switch folds to
// one case), or of any kind for K = kAnyKind
constexpr int kAnyKind = -1;
template <int K>
__device__ __forceinline__ TileSrc plan_tile_k(const Plan& P, int i, const Misc* ms) {
  if constexpr (K == kAnyKind) {
    return plan_tile(P, i, ms);
  } else {
    Plan Q = P;
    Q.kind = K;
    return plan_tile(Q, i, ms);
  }
}

template <typename WT>
__device__ __forceinline__ Plan plan_qkv(const KParams& p, int l) {
  const auto& Ly = layer_tab(p)[l];
  Plan P{};
  P.kind = PK_QKV;
  P.lrb = ilog2(p.d * (int)sizeof(WT));
  P.rpt = kTileBytes >> P.lrb;
  P.a0 = p.H * p.hd;
  P.a1 = p.G * p.hd;
  int lo, hi;
  my_range((P.a0 + 2 * P.a1) / P.rpt, p, lo, hi);
  P.lo = lo;
  P.n = hi - lo;
  P.b0 = (const char*)Ly.wq;
  P.b1 = (const char*)Ly.wk;
  P.b2 = (const char*)Ly.wv;
  return P;
}

// attention split owned by this CU (tasks never outnumber CUs)
// CU -> attention task (sequence, kv head, split).  Workgroups are dealt to
// the 8 XCDs round-robin; tasks are numbered XCD by XCD, so the splits of one
// (sequence, kv head), consecutive tasks, share an XCD when the split count
// divides the CUs per XCD, and their partial records meet in that XCD's L2.
__device__ __forceinline__ int attn_task(const KParams& p) {
  const int b = vcu_of(p), ncu = p.vncu;
  return (ncu & 7) ? b : (b & 7) * (ncu >> 3) + (b >> 3);
}

// trail: one row per sequence (decode); its new position, the sequence's
// last, is attended from the copy in LDS instead of a cache tile, and the
// split S-1 owns it (P.U = 1, P.F = its position).  The cached positions are
// spread over the splits tile by tile.
__device__ __forceinline__ Plan plan_attn(const KParams& p, const Misc* ms, int l, bool trail) {
  Plan P{};
  P.kind = PK_ATTN;
  const int S = p.n_splits, QG = p.q_groups;
  const int task = attn_task(p);
  if (task >= p.n_seq * p.G * QG * S) return P;
  const int seq = task / (p.G * QG * S), g = (task / (QG * S)) % p.G, s = task % S;
  int maxpos = 0;
  for (int rr = 0; rr < p.rps; ++rr) maxpos = max(maxpos, ms->pos[seq * p.rps + rr]);
  const bool tr = trail && p.rps == 1;
  const int npos = tr ? maxpos : maxpos + 1;  // positions read from the cache
  const int ntile = (npos + kAttnTile - 1) / kAttnTile;
  const int t_lo = (int)(((unsigned)s * ntile) / (unsigned)S), t_hi = (int)(((unsigned)(s + 1) * ntile) / (unsigned)S);
  P.a0 = min(t_lo * kAttnTile, npos);
  P.a1 = min(t_hi * kAttnTile, npos);
  P.n = 2 * (t_hi - t_lo);
  P.U = (tr && s == S - 1) ? 1 : 0;
  P.F = maxpos;
  const size_t kv_base =
      ((((size_t)l * p.kv_seqs + p.seq0 + (size_t)grp_of(p) * p.n_seq + seq) * p.G + g) * (size_t)p.cap) * p.hd;
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
  my_range(p.d / P.rpt, p, lo, hi);
  P.lo = lo;
  P.n = hi - lo;
  P.b0 = (const char*)layer_tab(p)[l].wo;
  return P;
}

// router tiles (weight 1) then shared pairs (gate tile, up tile; weight 2),
// split by cumulative weight so that a pair never straddles two CUs
template <typename WT>
__device__ __forceinline__ Plan plan_rs(const KParams& p, int l) {
  const auto& Ly = layer_tab(p)[l];
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
  my_range(nrt + 2 * npair, p, lo, hi);
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
  const auto& Ly = layer_tab(p)[l];
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
  my_range(p.S > 0 ? p.d / P.rpt : 0, p, lo, hi);
  P.lo = lo;
  P.nj = hi - lo;
  P.n1 = (hi - lo) * p.S;
  P.fb_per = p.F / P.rpt2;
  P.n = P.n1;
  if (routed) {
    int l2, h2;
    my_range(ms->n_uni * P.fb_per, p, l2, h2);
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
  my_range(p.d / P.rpt, p, lo, hi);
  P.lo = lo;
  P.nj = hi - lo;
  P.n = (hi - lo) * P.U;
  P.b0 = (const char*)layer_tab(p)[l].w_down;
  return P;
}

// DOWN with several rows, first half: the (union expert, j-block) tiles of
// all experts in one expert-major order, cut into contiguous ranges, so a CU
// meets one or two experts; lo2 / n1 are this CU's output column blocks for
// the second half.
template <typename WT>
__device__ __forceinline__ Plan plan_down_a(const KParams& p, const Misc* ms, int l) {
  Plan P{};
  P.kind = PK_DOWNA;
  P.lrb = ilog2(p.F * (int)sizeof(WT));
  P.rpt = kTileBytes >> P.lrb;
  P.d = p.d;
  P.U = ms->n_uni;
  P.nj = p.d / P.rpt;
  int lo, hi;
  my_range(P.U * P.nj, p, lo, hi);
  P.lo = lo;
  P.n = hi - lo;
  my_range(P.nj, p, lo, hi);
  P.lo2 = lo;
  P.n1 = hi - lo;
  P.b0 = (const char*)layer_tab(p)[l].w_down;
  return P;
}

// Row-group launches: the routed tiles of the launch's tasks, split over all
// of its workgroups (c * n stays below 2^32).
__device__ __forceinline__ void grid_range(int n, const KParams& p, int& lo, int& hi) {
  const unsigned c = blockIdx.x, ncu = (unsigned)p.n_cu;
  lo = (int)((c * (unsigned)n) / ncu);
  hi = (int)(((c + 1) * (unsigned)n) / ncu);
}
// RG: this group's shared-down tiles (as plan_rg), then this workgroup's
// range of the (task, f-block) gate/up pairs
template <typename WT>
__device__ __forceinline__ Plan plan_rg_t(const KParams& p, const Misc* ms, int l) {
  Plan P = plan_rg<WT>(p, ms, l, false);
  P.kind = PK_RGT;
  int l2, h2;
  grid_range(ms->n_task * P.fb_per, p, l2, h2);
  P.lo2 = l2;
  P.n = P.n1 + 2 * (h2 - l2);
  return P;
}
// DOWN, first half: this workgroup's range of the (task, j-block) tiles;
// lo2 / n1 are this group's output column blocks for the second half
template <typename WT>
__device__ __forceinline__ Plan plan_down_t(const KParams& p, const Misc* ms, int l) {
  Plan P = plan_down_a<WT>(p, ms, l);
  P.kind = PK_DOWNT;
  P.U = ms->n_task;
  int lo, hi;
  grid_range(P.U * P.nj, p, lo, hi);
  P.lo = lo;
  P.n = hi - lo;
  return P;
}

// ------------------------------------------------------------------ tile stream

// Tile addresses of one plan for 64 consecutive tiles, one per lane (lane j
// holds tile w0 + j), evaluated in parallel by plan_tile; issuing a tile then
// costs two v_readlane.  hi keeps the upper address bits in 0..26 and
// (kTileBytes - valid) / 256 in bits 27..31.
struct Win {
  unsigned lo, hi;
  int w0;
};
constexpr int kNoWin = -(1 << 24);
template <int K>
__device__ __forceinline__ Win build_win(const Plan& P, int w0, const Misc* ms, int lane) {
  const int j = w0 + lane;
  TileSrc t{nullptr, kTileBytes};
  if (j < P.n) t = plan_tile_k<K>(P, j, ms);
  const unsigned long long a = (unsigned long long)(uintptr_t)t.g;
  Win w;
  w.lo = (unsigned)a;
  w.hi = (unsigned)(a >> 32) | ((unsigned)((kTileBytes - t.valid) >> 8) << 27);
  w.w0 = w0;
  return w;
}

// issue this wave's quarter of tile j (of the window's plan) into `slot`
__device__ __forceinline__ void issue_tile(const Win& w, int j, unsigned slot_lds, int wave, int lane, bool keep) {
  const int idx = j - w.w0;
  const unsigned lo = __builtin_amdgcn_readlane(w.lo, idx);
  const unsigned hi = __builtin_amdgcn_readlane(w.hi, idx);
  const char* g = reinterpret_cast<const char*>(((unsigned long long)(hi & 0x07ffffffu) << 32) | lo);
  const int off0 = wave * 2048 + lane * 16;
  if ((hi >> 27) == 0) {  // a whole tile (the common case; wave-uniform)
    g2l2(g + off0, slot_lds + wave * 2048, keep);
    return;
  }
  const int valid = kTileBytes - (int)((hi >> 27) << 8);
  const int off1 = off0 + 1024;
  g2l(g + (off0 < valid ? off0 : 0), slot_lds + wave * 2048);
  g2l(g + (off1 < valid ? off1 : 0), slot_lds + wave * 2048 + 1024);
}

// Copy `bytes` (a multiple of 1 KiB) from global memory to LDS by DMA, 1 KiB
// per wave instruction.  Completion needs wait_all() and a workgroup sync.
__device__ __forceinline__ void dma_to_lds(char* lds, const char* g, int bytes, int wave, int lane) {
  const unsigned base = lds_addr(lds);
  for (int c = wave * 1024; c < bytes; c += kWaves * 1024) g2l(g + c + lane * 16, base + c);
}

// The stream of one phase followed by the next: tile j < cur.n is the
// current phase's tile j, later tiles belong to `nxt` (when its plan is
// known).  Tile j lives in ring slot (slot0 + j) % kRing and may be issued
// once tile j - kRing has been consumed.
struct Stream {
  int slot0;
  int issued;
  long long* ts;  // this phase's 4 timestamp slots, or null
  Win wc, wn;     // address windows of the current and the next plan
  int islot;      // ring slot of tile `issued`
  unsigned ring_lds;
  bool keep;      // tile loads keep their lines in the caches (row groups of one launch)
  __device__ __forceinline__ void mark(int k) const {
    if (ts && threadIdx.x == 0) ts[k] = wall_clock64();
  }
  __device__ __forceinline__ char* slot(Smem sm, int j) const {
    return sm.ring + (size_t)((slot0 + j) % kRing) * kSlotBytes;
  }
  // issue while ring slots are free; `consumed` tiles of cur are done.  KC,
  // KN: the kinds of cur and nxt when known at compile time
  template <int KC, int KN>
  __device__ __forceinline__ void fill(Smem sm, const Plan& cur, const Plan& nxt, int consumed, int wave,
                                       int lane) {
    // The slots being refilled held tiles whose reads this wave has already
    // consumed (their values fed the arithmetic), so no LDS wait is needed.
    const int limit = min(consumed + kRing, cur.n + nxt.n);
    for (; issued < limit; ++issued) {
      const unsigned s = ring_lds + (unsigned)islot * kSlotBytes;
      islot = islot == kRing - 1 ? 0 : islot + 1;
      if (issued < cur.n) {
        if ((unsigned)(issued - wc.w0) >= 64u) wc = build_win<KC>(cur, issued, sm.misc, lane);
        issue_tile(wc, issued, s, wave, lane, keep);
      } else {
        const int j = issued - cur.n;
        if ((unsigned)(j - wn.w0) >= 64u) wn = build_win<KN>(nxt, j, sm.misc, lane);
        issue_tile(wn, j, s, wave, lane, keep);
      }
    }
  }
  // wait until tile i of cur has landed (this wave's quarter)
  __device__ __forceinline__ void wait(int i) const { wait_tiles_ahead(issued - 1 - i); }
  // hand over to the next phase: its first tiles are already issued.  The
  // next phase may re-plan (same leading tiles), so both windows are rebuilt.
  __device__ __forceinline__ void advance(const Plan& cur) {
    slot0 = (slot0 + cur.n) % kRing;
    issued -= cur.n;
    wc.w0 = kNoWin;
    wn.w0 = kNoWin;
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

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// x registers: the EPL activation elements each chunk of this lane meets, per token
template <typename WT, int MT>
struct XRegs {
  static constexpr int EPL = 16 / sizeof(WT);
  float v[MT][2][EPL];
};
// 8 rows, bf16 weights: x for the matrix-core GEMV (gemv_group below).  Lane
// 4b + t holds tokens t and t + 4 (index h) at the k-elements kq + kc*64 + 4b
// + j (kc < 16, j < 4; kq = the wave's first k-element of its 2 KiB quarter of
// a tile), as bf16 high and low parts of the fp32 value.
template <>
struct XRegs<uint16_t, 8> {
  static constexpr int EPL = 8;
  s16x4_t hi[2][16];
  s16x4_t lo[2][16];
};
__device__ __forceinline__ void split_bf16x4(float4 a, s16x4_t& hi, s16x4_t& lo) {
  const float x[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const __bf16 h = (__bf16)x[j];
    hi[j] = __builtin_bit_cast(short, h);
    lo[j] = __builtin_bit_cast(short, (__bf16)(x[j] - (float)h));
  }
}
__device__ __forceinline__ int m8_kq(int wave, int lrb) { return ((wave * 2048) & ((1 << lrb) - 1)) >> 1; }

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

// load_x for an RMSNorm'd input: x = h * gain, and misc->rinv[t] =
// 1/sqrt(mean(h_t^2) + eps) from the same loads.  Each element of a row is
// loaded by rpt = kTileBytes >> lrb lanes of the workgroup (one per row of a
// tile), so the workgroup's sum of squares is rpt times the row's.  rinv is
// ready after the workgroup's next synchronisation.
template <typename WT, int MT>
__device__ __forceinline__ void load_x_norm(XRegs<WT, MT>& xr, Smem sm, const float* src, int ld, const WT* gam,
                                            int M, int d, float eps, int wave, int lane, int lrb) {
  constexpr int EPL = XRegs<WT, MT>::EPL;
  float ss[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) ss[t] = 0.f;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int k0 = lane_k0<WT>(wave, lane, c, lrb);
    float g[EPL];
    unpack16<WT>(*reinterpret_cast<const uint4*>(gam + k0), g);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      if (t < M) {
        const float* s = src + (size_t)t * ld + k0;
#pragma unroll
        for (int j = 0; j < EPL; j += 4) {
          const float4 a = *reinterpret_cast<const float4*>(s + j);
          ss[t] = fmaf(a.x, a.x, fmaf(a.y, a.y, fmaf(a.z, a.z, fmaf(a.w, a.w, ss[t]))));
          xr.v[t][c][j] = a.x * g[j]; xr.v[t][c][j + 1] = a.y * g[j + 1];
          xr.v[t][c][j + 2] = a.z * g[j + 2]; xr.v[t][c][j + 3] = a.w * g[j + 3];
        }
      } else {
#pragma unroll
        for (int j = 0; j < EPL; ++j) xr.v[t][c][j] = 0.f;
      }
    }
  }
  const float r = xreduce<MT>(ss, lane);
  if (xreduce_writer<MT>(lane)) {
    const int t = xreduce_index<MT>(lane);
    if (t < M) sm.misc->ssq[wave * kMaxRows + t] = r;
  }
  __syncthreads();
  if ((int)threadIdx.x < M) {
    const int t = threadIdx.x;
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) tot += sm.misc->ssq[w * kMaxRows + t];
    const float rpt = (float)(kTileBytes >> lrb);
    sm.misc->rinv[t] = 1.0f / sqrtf(tot / (rpt * (float)d) + eps);
  }
}

// x loaders for 8 rows with bf16 weights (the matrix-core layout of
// XRegs<uint16_t, 8>): token t4 + 4h, elements kq + kc*64 + 4b + j.
template <>
__device__ __forceinline__ void load_x<uint16_t, 8>(XRegs<uint16_t, 8>& xr, const float* src, int ld,
                                                    const uint16_t* gam, int M, int wave, int lane, int lrb) {
  const int t4 = lane & 3, b = lane >> 2;
  const int k0 = m8_kq(wave, lrb) + b * 4;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int t = t4 + 4 * h;
    const bool ok = t < M;
    const float* s = src + (size_t)(ok ? t : 0) * ld + k0;
#pragma unroll
    for (int kc = 0; kc < 16; ++kc) {
      float4 a = *reinterpret_cast<const float4*>(s + kc * 64);
      if (gam) {
        const uint2 gg = *reinterpret_cast<const uint2*>(gam + k0 + kc * 64);
        a.x *= __uint_as_float(gg.x << 16); a.y *= __uint_as_float(gg.x & 0xffff0000u);
        a.z *= __uint_as_float(gg.y << 16); a.w *= __uint_as_float(gg.y & 0xffff0000u);
      }
      if (!ok) a = make_float4(0.f, 0.f, 0.f, 0.f);
      split_bf16x4(a, xr.hi[h][kc], xr.lo[h][kc]);
    }
  }
}
// The 8-row loader for rows given by row(t) (a pointer to the row's first
// element, called with t < n only; rows t >= n are zero).  set_rinv(t, v)
// receives 1/rms of row t < n after a workgroup synchronisation inside.
// lead: synchronise first, for a caller that may still be reading the
// sum-of-squares slots of an earlier call.
template <class RowFn, class RinvFn>
__device__ __forceinline__ void load_x_norm8(XRegs<uint16_t, 8>& xr, Smem sm, RowFn row, int n, const uint16_t* gam,
                                             int d, float eps, int wave, int lane, int lrb, RinvFn set_rinv,
                                             bool lead) {
  const int t4 = lane & 3, b = lane >> 2;
  const int k0 = m8_kq(wave, lrb) + b * 4;
  float ss[2] = {0.f, 0.f};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int t = t4 + 4 * h;
    const bool ok = t < n;
    const float* s = row(ok ? t : 0) + k0;
#pragma unroll
    for (int kc = 0; kc < 16; ++kc) {
      float4 a = *reinterpret_cast<const float4*>(s + kc * 64);
      if (!ok) a = make_float4(0.f, 0.f, 0.f, 0.f);
      ss[h] = fmaf(a.x, a.x, fmaf(a.y, a.y, fmaf(a.z, a.z, fmaf(a.w, a.w, ss[h]))));
      const uint2 gg = *reinterpret_cast<const uint2*>(gam + k0 + kc * 64);
      a.x *= __uint_as_float(gg.x << 16); a.y *= __uint_as_float(gg.x & 0xffff0000u);
      a.z *= __uint_as_float(gg.y << 16); a.w *= __uint_as_float(gg.y & 0xffff0000u);
      split_bf16x4(a, xr.hi[h][kc], xr.lo[h][kc]);
    }
  }
  // sum of squares of token t over the workgroup: the lanes of one t (bits
  // 2-5) here, the waves through LDS; each element is met by rpt waves
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float x = ss[h];
    x += dpp<kDppRor4>(x);
    x += dpp<kDppRor8>(x);
    ss[h] = sum_rows(x);
  }
  if (lead) __syncthreads();
  if (b == 0) {
    sm.misc->ssq[wave * kMaxRows + t4] = ss[0];
    sm.misc->ssq[wave * kMaxRows + t4 + 4] = ss[1];
  }
  __syncthreads();
  if ((int)threadIdx.x < n) {
    const int t = threadIdx.x;
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) tot += sm.misc->ssq[w * kMaxRows + t];
    const float rpt = (float)(kTileBytes >> lrb);
    set_rinv(t, 1.0f / sqrtf(tot / (rpt * (float)d) + eps));
  }
}
template <>
__device__ __forceinline__ void load_x_norm<uint16_t, 8>(XRegs<uint16_t, 8>& xr, Smem sm, const float* src, int ld,
                                                         const uint16_t* gam, int M, int d, float eps, int wave,
                                                         int lane, int lrb) {
  load_x_norm8(
      xr, sm, [&](int t) { return src + (size_t)t * ld; }, M, gam, d, eps, wave, lane, lrb,
      [&](int t, float v) { sm.misc->rinv[t] = v; }, false);
}
// 8 rows of plain x from rows given by row(t) (called with t < n only; rows
// t >= n repeat row 0, which the token mask then drops)
template <class RowFn>
__device__ __forceinline__ void load_x8_rows(XRegs<uint16_t, 8>& xr, RowFn row, int n, int wave, int lane, int lrb) {
  const int t4 = lane & 3, b = lane >> 2;
  const int k0 = m8_kq(wave, lrb) + b * 4;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int t = t4 + 4 * h;
    const float* s = row(t < n ? t : 0) + k0;
#pragma unroll
    for (int kc = 0; kc < 16; ++kc)
      split_bf16x4(*reinterpret_cast<const float4*>(s + kc * 64), xr.hi[h][kc], xr.lo[h][kc]);
  }
}

// Part-block slots per wave: a wave reads 2 KiB of every tile as two 1 KiB
// chunks; with bf16 weights every row is at least 2 KiB (the host checks), so
// both chunks of a wave lie in one row and their sums are added before the
// cross-lane reduction (one slot); fp32 rows may be 1 KiB (two slots).
template <typename WT>
struct Slots {
  static constexpr int C = sizeof(WT) == 2 ? 1 : 2;
  static constexpr int kUnitLog2 = C == 1 ? 11 : 10;  // bytes of tile behind one slot
};

// Tiles consumed per step of the GEMV loop: one cross-lane reduction serves
// the whole group.  8 rows with bf16 weights: groups of 4 tiles (the matrix
// cores take 4 weight rows at a time).
template <typename WT, int MT>
struct GroupOf {
  static constexpr int G = (MT == 1 || sizeof(WT) == 2) ? 4 : 1;
};

// This wave's quarter of g <= G consecutive tiles (ring slots of tiles i ..
// i+g-1) against the x registers.  For tile i+u, chunk c and token t the dot
// product over the wave is scaled by tw[t] and stored (added when accum) at
// part[(blk0 + u) * kWaves*2*MT + (wave*2 + c)*MT + t].  Tokens outside tmask
// contribute zero.
template <typename WT, int MT>
__device__ __forceinline__ void gemv_group(Smem sm, const Stream& st, int i, int g, const XRegs<WT, MT>& xr,
                                           unsigned tmask, const float (&tw)[MT], int blk0, bool accum, int wave,
                                           int lane) {
  constexpr int G = GroupOf<WT, MT>::G;
  constexpr int EPL = XRegs<WT, MT>::EPL;
  constexpr int C = Slots<WT>::C;
  constexpr int NV = G * C * MT;
  uint4 wv[G][2];
  const int rs0 = (st.slot0 + i) % kRing;
#pragma unroll
  for (int u = 0; u < G; ++u) {
    if (u < g) {
      const int rs = rs0 + u < kRing ? rs0 + u : rs0 + u - kRing;
      const char* sl = sm.ring + (size_t)rs * kSlotBytes + wave * 2048 + lane * 16;
      wv[u][0] = *reinterpret_cast<const uint4*>(sl);
      wv[u][1] = *reinterpret_cast<const uint4*>(sl + 1024);
    }
  }
  float acc[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) acc[v] = 0.f;
#pragma unroll
  for (int u = 0; u < G; ++u) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float w[EPL];
      unpack16<WT>(wv[u][c], w);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        float s0 = 0.f, s1 = 0.f;
        if (u < g && (tmask & (1u << t))) {
#pragma unroll
          for (int j = 0; j < EPL; j += 2) {
            s0 = fmaf(w[j], xr.v[t][c][j], s0);
            s1 = fmaf(w[j + 1], xr.v[t][c][j + 1], s1);
          }
        }
        acc[(u * C + (C == 1 ? 0 : c)) * MT + t] += (s0 + s1) * tw[t];
      }
    }
  }
  const float r = xreduce<NV>(acc, lane);
  if (xreduce_writer<NV>(lane)) {
    const int idx = xreduce_index<NV>(lane);
    const int u = idx / (C * MT), c = (idx / MT) % C, t = idx % MT;
    if (u < g) {
      float* dst = sm.part + (size_t)(blk0 + u) * (kWaves * C * MT) + (wave * C + c) * MT + t;
      if (accum) *dst += r;
      else *dst = r;
    }
  }
}

// 8 rows, bf16 weights, on the matrix cores.  A group is 4 tiles; for a wave
// each holds the 1024 k-elements of its 2 KiB quarter of one weight row r.
// v_mfma_f32_4x4x4_16b_bf16 computes 16 independent 4x4x4 blocks: block b
// takes the k-elements kc*64 + 4b .. +3 of 4 tokens (A: lane 4b + t) and of
// 4 rows (B: lane 4b + r), so one instruction covers 64 k-elements of
// 4 tokens x 4 rows and 16 of them the quarter.  x enters as bf16 high and
// low parts (two products, fp32 accumulation); the weights are bf16 exactly.
// D_b[t][r] (lane 4b + r, register t) is summed over the 16 blocks by row
// rotations and the permlane swaps, then over the waves through the part
// block, as on the vector path.  Slot pitch kSlotBytes keeps the 4 rows of
// one read in different LDS bank halves.
template <>
__device__ __forceinline__ void gemv_group<uint16_t, 8>(Smem sm, const Stream& st, int i, int g,
                                                        const XRegs<uint16_t, 8>& xr, unsigned tmask,
                                                        const float (&tw)[8], int blk0, bool accum, int wave,
                                                        int lane) {
  const int r = lane & 3, b = lane >> 2;
  const int rs0 = (st.slot0 + i) % kRing;
  const int u = r < g ? r : 0;  // rows past the group read row 0; their sums are dropped
  const int rs = rs0 + u < kRing ? rs0 + u : rs0 + u - kRing;
  const char* wp = sm.ring + (size_t)rs * kSlotBytes + wave * 2048 + b * 8;
  // All 16 reads are issued before the first product (a fence keeps the
  // scheduler from sinking them): one LDS round trip per group, not eight.
  s16x4_t w[16];
#pragma unroll
  for (int kc = 0; kc < 16; ++kc) w[kc] = *reinterpret_cast<const s16x4_t*>(wp + kc * 128);
  __builtin_amdgcn_sched_barrier(0);
  f32x4_t d0 = {0.f, 0.f, 0.f, 0.f}, d1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kc = 0; kc < 16; ++kc) {
    d0 = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(xr.hi[0][kc], w[kc], d0, 0, 0, 0);
    d0 = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(xr.lo[0][kc], w[kc], d0, 0, 0, 0);
    d1 = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(xr.hi[1][kc], w[kc], d1, 0, 0, 0);
    d1 = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(xr.lo[1][kc], w[kc], d1, 0, 0, 0);
  }
  // Sum over the 16 blocks (lane bits 2-5) in halving steps, each leaving
  // half of the token values in a lane, summed with its partner's copy:
  // bit 5 (tokens t < 4 stay where the bit is clear), bit 4, then bit 2 by a
  // row rotation by 4 (the lanes it pairs always differ in bit 2) and a plain
  // sum over bit 3 by a rotation by 8.  Lane l with bit 3 clear then holds
  // token t = 4*bit5 + 2*bit4 + bit2 of row r.  Lanes with bit 2 clear take
  // the rotation one way, lanes with it set the other way, so that the
  // tokens of both kinds add the same pairs of lanes in the same tree (only
  // the operand order of an addition differs, which is exact): a token's
  // sum does not depend on its place among the 8 rows.
  float w4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w4[i] = swap32_sum(d0[i], d1[i]);
  float w2[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) w2[i] = swap16_sum(w4[i], w4[2 + i]);
  const bool b2 = (lane >> 2) & 1;
  const float from_dn = dpp<kDppRor4>(w2[0]), from_up = dpp<kDppRor12>(w2[1]);
  float x = b2 ? w2[1] + from_up : w2[0] + from_dn;
  x += dpp<kDppRor8>(x);
  if (((lane >> 3) & 1) == 0 && r < g) {
    const bool b4 = (lane >> 4) & 1, b5 = (lane >> 5) & 1;
    const int t = 4 * b5 + 2 * b4 + b2;
    // the token's weight by a select tree on the lane bits; the values pass
    // through an empty asm so that the selects are not folded back into an
    // indexed access, which would go through scratch memory
    float q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      q[i] = tw[i];
      asm volatile("" : "+v"(q[i]));
    }
    const float a0 = b2 ? q[1] : q[0], a1 = b2 ? q[3] : q[2];
    const float a2 = b2 ? q[5] : q[4], a3 = b2 ? q[7] : q[6];
    const float twt = b5 ? (b4 ? a3 : a2) : (b4 ? a1 : a0);
    const float val = ((tmask >> t) & 1u) ? x * twt : 0.f;
    float* dst = sm.part + (size_t)(blk0 + r) * (kWaves * 8) + wave * 8 + t;
    if (accum) *dst += val;
    else *dst = val;
  }
}

// One row per step: this wave's quarter of the g <= G tiles i .. i+g-1
// against x, each slot's dot product scaled by tw and added to the lane's
// running sums pacc[u*C + c] (no cross-lane reduction here).
template <typename WT>
__device__ __forceinline__ void gemv_acc1(Smem sm, const Stream& st, int i, int g, const XRegs<WT, 1>& xr, float tw,
                                          float (&pacc)[GroupOf<WT, 1>::G * Slots<WT>::C], int wave, int lane) {
  constexpr int C = Slots<WT>::C;
  constexpr int G = GroupOf<WT, 1>::G;
  constexpr int EPL = XRegs<WT, 1>::EPL;
  uint4 wv[G][2];
  const int rs0 = (st.slot0 + i) % kRing;
#pragma unroll
  for (int u = 0; u < G; ++u) {
    if (u < g) {
      const int rs = rs0 + u < kRing ? rs0 + u : rs0 + u - kRing;
      const char* sl = sm.ring + (size_t)rs * kSlotBytes + wave * 2048 + lane * 16;
      wv[u][0] = *reinterpret_cast<const uint4*>(sl);
      wv[u][1] = *reinterpret_cast<const uint4*>(sl + 1024);
    }
  }
#pragma unroll
  for (int u = 0; u < G; ++u) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float w[EPL];
      unpack16<WT>(wv[u][c], w);
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int j = 0; j < EPL; j += 2) {
        s0 = fmaf(w[j], xr.v[0][c][j], s0);
        s1 = fmaf(w[j + 1], xr.v[0][c][j + 1], s1);
      }
      if (u < g) pacc[u * C + (C == 1 ? 0 : c)] = fmaf(s0 + s1, tw, pacc[u * C + (C == 1 ? 0 : c)]);
    }
  }
}

// A run of tiles that share x registers, token mask and weights, with
// consecutive part blocks starting at blk0; the loop calls the phase's
// epilogue after the run when round_end is set.
template <int MT>
struct Seg {
  int end;
  int blk0;
  bool accum;
  bool round_end;
  unsigned tmask;
  float tw[MT];
};
template <int MT>
__device__ __forceinline__ void seg_all(Seg<MT>& sg, int M) {
  sg.tmask = (1u << M) - 1u;
#pragma unroll
  for (int t = 0; t < MT; ++t) sg.tw[t] = 1.f;
}

// part block layout: [wave][c][MT] with C slots c per wave; slot (wave, c)
// holds the tile bytes from wave*2048 + c*2^U (U = kUnitLog2), so row q of
// 2^lrb-byte rows covers slots q*upr .. q*upr+upr-1, upr = 2^(lrb-U).
template <typename WT, int MT>
__device__ __forceinline__ float part_row(const float* part, int block, int q, int lrb, int t) {
  constexpr int C = Slots<WT>::C;
  constexpr int NS = kWaves * C;
  const float* b = part + (size_t)block * (NS * MT);
  const int upr = 1 << (lrb - Slots<WT>::kUnitLog2), c0 = q * upr;
  float v[NS];
#pragma unroll
  for (int ch = 0; ch < NS; ++ch) v[ch] = b[ch * MT + t];
  // One use of every value before the selects: otherwise the compiler moves
  // each read under its select's branch and the reads run one after another,
  // a full LDS round trip each.
  if constexpr (NS == 8)
    asm volatile("" ::"v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]));
  else
    asm volatile("" ::"v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]));
  float s = 0.f;
#pragma unroll
  for (int ch = 0; ch < NS; ++ch) s += (ch >= c0 && ch < c0 + upr) ? v[ch] : 0.f;
  return s;
}

// Consume the tiles of GEMV phase `cur` in groups.  seg(i, sg) describes the
// run starting at tile i (and may reload the x registers); after a run with
// round_end set, all waves synchronise and epi(first, last) runs over the
// round's tiles.  The stream keeps issuing `nxt`'s tiles meanwhile.
template <typename WT, int MT, int KC, int KN, bool kSettle = true, class SegFn, class EpiFn>
__device__ __forceinline__ void run_gemv(Smem sm, Stream& st, const Plan& cur, const Plan& nxt, XRegs<WT, MT>& xr,
                                         SegFn seg, EpiFn epi) {
  constexpr int G = GroupOf<WT, MT>::G;
  const int wave = wave_id(), lane = threadIdx.x & 63;
  st.mark(1);
  if constexpr (kSettle) settle();
  st.fill<KC, KN>(sm, cur, nxt, 0, wave, lane);
  int round_first = 0;
  for (int i = 0; i < cur.n;) {
    Seg<MT> sg;
    seg(i, sg);
    for (int j = i; j < sg.end; j += G) {
      const int g = min(G, sg.end - j);
      st.wait(j + g - 1);
      gemv_group<WT, MT>(sm, st, j, g, xr, sg.tmask, sg.tw, sg.blk0 + (j - i), sg.accum, wave, lane);
      st.fill<KC, KN>(sm, cur, nxt, j + g, wave, lane);
    }
    if (sg.round_end) {
      __syncthreads();
      epi(round_first, sg.end - 1);
      __syncthreads();
      round_first = sg.end;
    }
    i = sg.end;
  }
  st.mark(2);
}

// The part region holds the GEMV accumulators (kPartAcc floats) followed by
// the residual slice (kResFloats) an epilogue adds: epilogues read it from
// LDS because a global load there would wait behind the ring's loads.
__device__ __forceinline__ float* res_slice(Smem sm) { return sm.part + kPartAcc; }
__device__ __forceinline__ void zero_part(Smem sm) {
  for (int i = threadIdx.x; i < kPartAcc; i += kThreads) sm.part[i] = 0.f;
}
// res[t*ncol + c] = a[t*ld + c0 + c] (+ b[t*ld + c0 + c])
__device__ __forceinline__ void load_res(Smem sm, const float* a, const float* b, int ld, int c0, int ncol, int M) {
  float* res = res_slice(sm);
  for (int it = threadIdx.x; it < ncol * M; it += kThreads) {
    const int t = it / ncol, c = it - t * ncol;
    float v = a[(size_t)t * ld + c0 + c];
    if (b) v += b[(size_t)t * ld + c0 + c];
    res[it] = v;
  }
}

// Runs of the tiles [base, end) in rounds of kRound tiles (one part block
// per tile, all tokens); i is the first tile of a round.
template <int MT>
__device__ __forceinline__ void seg_rounds(Seg<MT>& sg, int i, int base, int end, int kRound, int M) {
  const int k = i - base;
  sg.end = base + min(end - base, (k / kRound + 1) * kRound);
  sg.blk0 = k % kRound;
  sg.accum = false;
  sg.round_end = true;
  seg_all<MT>(sg, M);
}

// ------------------------------------------------------------------ phases

// QKV: raw projections of (h * g1); the row scale rinv is applied in the epilogue.
template <typename WT, int MT>
__device__ __forceinline__ void phase_qkv(const KParams& p, Smem sm, int l, Stream& st, const Plan& P, const Plan& N) {
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int d = p.d, M = p.M;
  const int nrows = P.a0 + 2 * P.a1;
  const float* h = layer_in(p, l);
  float* qkv = act_w(p, l, p.al.qkv);
  XRegs<WT, MT> xr;
  load_x_norm<WT, MT>(xr, sm, h, d, reinterpret_cast<const WT*>(layer_tab(p)[l].attn_norm), M, d, p.eps, wave, lane,
                      P.lrb);
  zero_part(sm);
  __syncthreads();
  constexpr int kRound = kPartAcc / (kWaves * Slots<WT>::C * MT);
  const Misc* ms = sm.misc;
  const int rpt = P.rpt, lo = P.lo, lrb = P.lrb, n = P.n;
  run_gemv<WT, MT, PK_QKV, PK_ATTN>(
      sm, st, P, N, xr, [&](int i, Seg<MT>& sg) { seg_rounds<MT>(sg, i, 0, n, kRound, M); },
      [&](int first, int last) {
        const int nr = (last - first + 1) * rpt;
        for (int it = threadIdx.x; it < nr * M; it += kThreads) {
          const int q = it / M, t = it - q * M;
          const int row = (lo + first) * rpt + q;
          st_dev(qkv + (size_t)t * nrows + row, part_row<WT, MT>(sm.part, q / rpt, q % rpt, lrb, t) * ms->rinv[t]);
        }
      });
}

// Split combine (flash-decoding reduction): o[q][d] = sum_z w_z acc_z[q][d] /
// sum_z w_z l_z[q], w_z = exp(m_z[q] - max_z m_z[q]), over the S split
// partials of (sequence, kv head g).  Partial record: kPartStride tag words,
// m, l, -, -, acc[hd] (acc = sum_t exp(s_t - m) v_t).  Every split CU takes a
// slice of the Q*hd outputs, [s*nper, s*nper + nper): it reads, for all
// splits, the m and l of the slice's queries and the slice's acc values, and
// reads again until every word carries this launch's tag (no counter, no
// last arriver).  Thread = (output, group of splits); the groups of an output
// are neighbouring lanes, merged by butterfly shuffles.
__device__ __forceinline__ void attn_gather(const KParams& p, Smem sm, int l, int seq, int g, int qg, int s, int Q) {
  const int S = p.n_splits, HG = p.H / p.G, rps = p.rps, hd = p.hd;
  const int nout = Q * hd;
  const int nper = (nout + S - 1) / S;
  const int o0 = s * nper, o1 = min(o0 + nper, nout);
  if (o0 >= o1) return;
  const int q0 = o0 / hd, nq = (o1 - 1) / hd - q0 + 1;
  const int nw = 2 * nq + (o1 - o0);  // words per split: (m, l) per query, then the acc slice
  const int nload = S * nw;
  const tagword_t* rec0 = reinterpret_cast<const tagword_t*>(act_f(p, l, p.al.part)) +
                          (size_t)(((seq * p.G + g) * p.q_groups + qg) * S) * Q * kPartStride;
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<tagword_t*>(rec0), (short)0, S * Q * kPartStride * 8, kBufferDword3);
  float* scr = sm.xs;  // [S][nw]
  Misc* ms = sm.misc;
  auto word = [&](int it) -> int {  // byte offset of word it
    const QR zw = divmod_small(it, nw);
    const int z = zw.q, w = zw.r;
    const QR od = divmod_small(o0 + w - 2 * nq, hd);
    const int q = w < 2 * nq ? q0 + (w >> 1) : od.q;
    const int c = w < 2 * nq ? (w & 1) : 4 + od.r;
    return ((z * Q + q) * kPartStride + c) * 8;
  };
  if (threadIdx.x == 0) ms->last = 0;  // set on a time-out (read after the first synchronisation)
  const long long t0 = wall_clock64();
  const int wave = wave_id();
  for (int round = 0;; ++round) {
    int bad = 0;
    for (int b0 = threadIdx.x; b0 < nload; b0 += 4 * kThreads) {
      // device-coherent reads (sc1): the writers sit on other XCDs
      tagword_t v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = ld_word<kCpolSc1>(rsrc, word(min(b0 + u * kThreads, nload - 1)));
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int it = b0 + u * kThreads;
        if (it < nload) {
          if ((unsigned)(v[u] >> 32) != ms->tag) bad = 1;
          else scr[it] = __uint_as_float((unsigned)v[u]);
        }
      }
    }
    if (threadIdx.x == 0 && wall_clock64() - t0 > p.timeout_ticks) {
      __hip_atomic_fetch_or(p.sync + SyncLayout::kErr, kErrTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ms->last = 1;
    }
    // workgroup OR of bad through per-wave slots (two sets: a wave that runs
    // ahead writes the other set, which every wave has read a round ago)
    const int wbad = __builtin_amdgcn_ballot_w64(bad != 0) != 0;
    if ((threadIdx.x & 63) == 0) ms->gbad[round & 1][wave] = wbad;
    __syncthreads();
    int any = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) any |= ms->gbad[round & 1][w];
    if (!any) break;
    if (ms->last) break;  // timed out: the error flag is set, the values are not used
    __builtin_amdgcn_s_sleep(1);
  }
  __syncthreads();
  // merge: ZG split groups per output (a power of two, <= 64: one wave)
  const int nouts = o1 - o0;
  int ZG = 1;
  while (ZG * 2 <= 64 && ZG * 2 * nouts <= kThreads) ZG *= 2;
  float* o = act_w(p, l, p.al.o);
  for (int t0i = 0; t0i < nouts * ZG; t0i += kThreads) {
    const int t = t0i + (int)threadIdx.x;
    const int oi = min(t / ZG, nouts - 1), zg = t % ZG;
    const int q = (o0 + oi) / hd, d = (o0 + oi) % hd, qi = q - q0;
    float M = -INFINITY;
    for (int z = zg; z < S; z += ZG) M = fmaxf(M, scr[z * nw + 2 * qi]);
    for (int sh = 1; sh < ZG; sh <<= 1) M = fmaxf(M, __shfl_xor(M, sh));
    float L = 0.f, A = 0.f;
    for (int z = zg; z < S; z += ZG) {
      const float mz = scr[z * nw + 2 * qi];
      const float w = mz == -INFINITY ? 0.f : __expf(mz - M);
      L = fmaf(w, scr[z * nw + 2 * qi + 1], L);
      A = fmaf(w, scr[z * nw + 2 * nq + oi], A);
    }
    for (int sh = 1; sh < ZG; sh <<= 1) {
      L += __shfl_xor(L, sh);
      A += __shfl_xor(A, sh);
    }
    if (t < nouts * ZG && zg == 0) {
      const int qa = qg * Q + q;  // query index within the (sequence, kv head)
      const int row = seq * rps + qa / HG, head = g * HG + qa % HG;
      st_dev(o + (size_t)row * (p.H * hd) + head * hd + d, A / L);
    }
  }
}

// Queries of a task (query group qbase / Q of its sequence and kv head),
// their rotary embedding and this step's new k, v rows: Qv[q][hd] (RoPE'd,
// scaled by 1/sqrt(hd)) and, for the rows whose position falls in the split,
// the bf16-rounded copies nkb, nvb [rps][hd] in LDS (the split's tiles may
// have been loaded before the rows reached the cache) and, when write_cache,
// the cache writes.
__device__ __forceinline__ void attn_prologue(const KParams& p, const Misc* ms, int l, int seq, int g, int qbase,
                                              int Q, int p_lo, int p_hi, const Plan& P, float* Qv, uint16_t* nkb,
                                              uint16_t* nvb, bool write_cache) {
  if (P.U) p_hi = P.F + 1;  // this split also writes the trailing row
  const int HG = p.H / p.G, hd = p.hd, rps = p.rps;
  const int nrows_qkv = (p.H + 2 * p.G) * hd;
  const float* qkv = act_f(p, l, p.al.qkv);
  const float scale = 1.0f / sqrtf((float)hd);
  uint16_t* kc = reinterpret_cast<uint16_t*>(const_cast<char*>(P.b0));
  uint16_t* vc = reinterpret_cast<uint16_t*>(const_cast<char*>(P.b1));
  // One pass over the query items and the new-row items (item it covers
  // element pair i, i + hd/2 of both kinds): every global read of an item is
  // issued before its arithmetic, so the split that owns this step's row
  // reads its k, v in the same round trip as the queries.
  const int nq_it = Q * (hd / 2), nk_it = rps * (hd / 2);
  const int n_it = nq_it > nk_it ? nq_it : nk_it;
  for (int it = threadIdx.x; it < n_it; it += kThreads) {
    const int i = it % (hd / 2);
    const bool dq = it < nq_it;
    const int q = it / (hd / 2);
    const int qa = qbase + q;  // query index within the (sequence, kv head)
    const int qrow = seq * rps + qa / HG, head = g * HG + qa % HG;
    float x0 = 0.f, x1 = 0.f;
    if (dq) {
      const float* src = qkv + (size_t)qrow * nrows_qkv + head * hd;
      x0 = src[i];
      x1 = src[i + hd / 2];
    }
    const int rr = it / (hd / 2);
    const int krow = seq * rps + rr;
    const int pos = it < nk_it ? ms->pos[krow] : -1;
    const bool dk = it < nk_it && pos >= p_lo && pos < p_hi;
    float y0 = 0.f, y1 = 0.f, u0 = 0.f, u1 = 0.f;
    if (dk) {
      const float* ksrc = qkv + (size_t)krow * nrows_qkv + p.H * hd + g * hd;
      const float* vsrc = qkv + (size_t)krow * nrows_qkv + (p.H + p.G) * hd + g * hd;
      y0 = ksrc[i];
      y1 = ksrc[i + hd / 2];
      u0 = vsrc[i];
      u1 = vsrc[i + hd / 2];
    }
    if (dq) {
      const float c = ms->rope[(qrow * 64 + i) * 2], sn = ms->rope[(qrow * 64 + i) * 2 + 1];
      Qv[q * hd + i] = (x0 * c - x1 * sn) * scale;
      Qv[q * hd + i + hd / 2] = (x1 * c + x0 * sn) * scale;
    }
    if (dk) {
      const float c = ms->rope[(krow * 64 + i) * 2], sn = ms->rope[(krow * 64 + i) * 2 + 1];
      const uint16_t k0 = f32_to_bf16(y0 * c - y1 * sn), k1 = f32_to_bf16(y1 * c + y0 * sn);
      const uint16_t v0 = f32_to_bf16(u0), v1 = f32_to_bf16(u1);
      if (write_cache) {  // one query group of the (sequence, kv head) writes the cache
        kc[(size_t)pos * hd + i] = k0;
        kc[(size_t)pos * hd + i + hd / 2] = k1;
        vc[(size_t)pos * hd + i] = v0;
        vc[(size_t)pos * hd + i + hd / 2] = v1;
      }
      nkb[rr * 128 + i] = k0;
      nkb[rr * 128 + i + hd / 2] = k1;
      nvb[rr * 128 + i] = v0;
      nvb[rr * 128 + i + hd / 2] = v1;
    }
  }
}

// Lane groups used by the decode attention: lane l covers position l >> 3
// of the wave's 8 and dims 16 * (l & 7) .. +16.
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror: i <-> 7 - i within 8 lanes
constexpr int kDppMirror = 0x140;      // row_mirror: i <-> 15 - i within 16 lanes
// sum over the 8 lanes of a position group (lane bits 0-2), in every lane
__device__ __forceinline__ float sum_oct(float v) {
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppHalfMirror>(v);  // values are uniform within quads here
  return v;
}
// max over the 8 position groups of a value uniform within each group
__device__ __forceinline__ float max_groups(float v) {
  v = fmaxf(v, dpp<kDppMirror>(v));  // uniform within 8-lane groups: the mirror is the other group
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
// sum over the 8 position groups (lane bits 3-5) of a per-lane value, in every lane
__device__ __forceinline__ float sum_groups(float v) {
  v += dpp<kDppRor8>(v);  // lane bit 3
  return sum_rows(v);     // lane bits 4, 5
}

// Split-KV GQA decode attention on the matrix cores, for tasks of at most NQ
// query vectors.  The rows * heads-per-kv-head queries of a (sequence, kv
// head) form q_groups groups of q_per_task (one group for a decode step, two
// of 16 for 8 verify rows); task = (sequence, kv head, query group, split) =
// this CU.  The groups of a split read the same tiles; the cached positions
// are spread over the splits
// tile by tile and stream as K, V tile pairs of 32 positions.  Wave w owns
// positions 8w .. 8w+7 of every tile (its 2 KiB quarter, as in a GEMV tile)
// and takes two pairs (a, b) per step: 16 positions r, r < 8 from a.
//  - Scores S^T[r][q] = K[r][:] . q[:] as 16x16x32 bf16 products with q split
//    into bf16 high and low parts (two products, fp32 accumulation), so the
//    scores carry about 16 bits of q and all of K.
//  - Online softmax on S^T in the product's layout (lane l: query l & 15,
//    positions 4(l >> 4) .. +3), in log2 units (q is prescaled by log2(e) /
//    sqrt(hd)); the running maximum is raised only when a score exceeds it
//    by more than 8, so probabilities stay below 2^8.
//  - out^T[dim][q] += V^T[dim][r] P^T[r][q] as 16x16x16 bf16 products: V^T
//    comes from LDS transpose loads, P is split into high and low parts, and
//    the score layout is already the operand layout P^T needs.
// The four wave states are merged through LDS into the split's partial
// (maximum stored in natural units).
__device__ __forceinline__ s16x4_t lds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t*)(const_cast<char*>(p)));
}
__device__ __forceinline__ short bf16_bits(__bf16 h) { return __builtin_bit_cast(short, h); }

template <int NQ>
__device__ __forceinline__ void phase_attn_dec(const KParams& p, Smem sm, int l, Stream& st, const Plan& P,
                                               const Plan& N) {
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int HG = p.H / p.G, hd = p.hd, rps = p.rps;
  const int Q = p.q_per_task;  // query vectors of this task: query group qg of its (sequence, kv head)
  const int S = p.n_splits, QG = p.q_groups;
  const int ntask = p.n_seq * p.G * QG * S;
  Misc* ms = sm.misc;
  // x region: the queries, read into registers before the tile loop, share
  // their space with the wave states written after it (a workgroup sync
  // separates the two); the bf16 copies of this step's k, v rows follow.
  constexpr int kQvF = NQ * 128, kWstF = kWaves * NQ * kPartStride;
  constexpr int kHeadF = kQvF > kWstF ? kQvF : kWstF;
  float* Qv = sm.xs;   // [NQ][128]
  float* wst = sm.xs;  // [kWaves][NQ][kPartStride] wave states; later the combine scratch
  uint16_t* nkb = reinterpret_cast<uint16_t*>(sm.xs + kHeadF);  // [rps][128] bf16 copies
  uint16_t* nvb = nkb + kMaxRows * 128;
  static_assert(kHeadF * 4 + 2 * kMaxRows * 128 * 2 <= kXsBytes, "attention scratch exceeds the x region");
  const int task = attn_task(p);
  const bool active = task < ntask;
  const int seq = active ? task / (p.G * QG * S) : 0, g = active ? (task / (QG * S)) % p.G : 0;
  const int qg = active ? (task / S) % QG : 0, s = active ? task % S : 0;
  const int qbase = qg * Q;
  const int p_lo = P.a0, p_hi = P.a1;
  if (active) attn_prologue(p, ms, l, seq, g, qbase, Q, p_lo, p_hi, P, Qv, nkb, nvb, qg == 0);
  __syncthreads();
  constexpr float kLog2e = 1.4426950408889634f;
  const int qq = lane & 15, lg = lane >> 4;
  // Set-up reads are unconditional (every index stays inside its array) and
  // masked by selects: conditional LDS reads would each wait a round trip.
  // This step's rows inside the split's tiles: their positions, and the span.
  int newpos[kMaxRows];
  int new_lo = 1 << 30, new_hi = -1;
#pragma unroll
  for (int rr = 0; rr < kMaxRows; ++rr) {
    const int pos = ms->pos[min(seq * rps + rr, kMaxRows - 1)];
    const bool in = active & (rr < rps) & (pos >= p_lo) & (pos < p_hi);
    newpos[rr] = in ? pos : -1;
    new_lo = in ? min(new_lo, pos) : new_lo;
    new_hi = in ? max(new_hi, pos) : new_hi;
  }
  // q^T operand, lane l: query l & 15, dims 32kb + 8(l >> 4) .. +7, high and low bf16 parts
  bf16x8_t qh[4], ql[4];
  const bool qok = active & (qq < Q);
  {
    const float* src = Qv + min(qq, NQ - 1) * 128 + lg * 8;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const float4 a0 = *reinterpret_cast<const float4*>(src + kb * 32);
      const float4 a1 = *reinterpret_cast<const float4*>(src + kb * 32 + 4);
      const float x[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float v = qok ? x[j] * kLog2e : 0.f;
        const __bf16 h = (__bf16)v;
        qh[kb][j] = h;
        ql[kb][j] = (__bf16)(v - (float)h);
      }
    }
  }
  const int rowpos = ms->pos[min(seq * rps + (qbase + qq) / HG, kMaxRows - 1)];
  const int qvis = qok ? rowpos : -1;          // last position the lane's query sees
  const int qlim = min(p_hi - 1, qvis);        // ... among the split's tiles
  f32x4_t acc[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_l = -INFINITY, lsum = 0.f;
  // One step over 16 positions: rows r < 8 at kA/vA + r*rs, rows r >= 8 at
  // kB/vB + (r-8)*rs; position of row r is j0a + r (r < 8) or j0b + r - 8.
  auto step = [&](const char* kA, const char* kB, const char* vA, const char* vB, int rs, int j0a, int j0b,
                  int lim) __attribute__((always_inline)) {
    const int mr = lane & 15;
    const char* kr = (mr < 8 ? kA : kB) + (mr & 7) * rs + lg * 16;
    f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const bf16x8_t kf = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(kr + kb * 64));
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qh[kb], sc, 0, 0, 0);
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, ql[kb], sc, 0, 0, 0);
    }
    float sv[4];
    bool up = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * lg + i;
      const int jpos = r < 8 ? j0a + r : j0b + (r - 8);
      sv[i] = jpos <= lim ? sc[i] : -INFINITY;
      up |= sv[i] > m_l + 8.f;
    }
    if (__builtin_amdgcn_ballot_w64(up) != 0) {  // wave-uniform and rare: raise the reference maxima
      float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const bool raise = mx > m_l + 8.f;
      const float corr = !raise ? 1.f : (m_l == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_l - mx);
      lsum *= corr;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) acc[nb] *= corr;
      m_l = raise ? mx : m_l;
    }
    s16x4_t ph, pl;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pv = sv[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[i] - m_l);
      lsum += pv;
      const __bf16 h = (__bf16)pv;
      ph[i] = bf16_bits(h);
      pl[i] = bf16_bits((__bf16)(pv - (float)h));
    }
    // V^T operand by transpose loads: lane 16g + 4j + c reads row 4g + j, dims 16nb + 4c .. +3
    const int rv = 4 * lg + ((lane >> 2) & 3);
    const char* vr = (rv < 8 ? vA : vB) + (rv & 7) * rs + (lane & 3) * 8;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const s16x4_t vt = lds_read_tr16(vr + nb * 32);
      acc[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, ph, acc[nb], 0, 0, 0);
      acc[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, pl, acc[nb], 0, 0, 0);
    }
  };
  // This step's rows that fall in a tile of the split replace the tile's
  // rows in LDS (the tiles may have been loaded before the rows reached the
  // cache); each wave patches its own quarter after its own wait.
  auto patch = [&](char* kq, char* vq, int t0q) {
#pragma unroll
    for (int rr = 0; rr < kMaxRows; ++rr) {
      const int r = newpos[rr] - t0q;
      if (newpos[rr] >= 0 && r >= 0 && r < 8) {
        reinterpret_cast<uint32_t*>(kq + r * 256)[lane] = reinterpret_cast<const uint32_t*>(nkb + rr * 128)[lane];
        reinterpret_cast<uint32_t*>(vq + r * 256)[lane] = reinterpret_cast<const uint32_t*>(nvb + rr * 128)[lane];
      }
    }
  };
  st.mark(1);
  settle();
  st.fill<PK_ATTN, PK_WO>(sm, P, N, 0, wave, lane);
  const int nt = P.n / 2;  // position tiles
  for (int t = 0; t < nt; t += 2) {
    const bool hb = t + 1 < nt;
    const int last = hb ? 2 * t + 3 : 2 * t + 1;
    st.wait(last);
    char* ka = st.slot(sm, 2 * t) + wave * 2048;
    char* va = st.slot(sm, 2 * t + 1) + wave * 2048;
    char* kb = hb ? st.slot(sm, 2 * t + 2) + wave * 2048 : ka;
    char* vb = hb ? st.slot(sm, 2 * t + 3) + wave * 2048 : va;
    const int j0a = p_lo + t * kAttnTile + wave * 8;
    const int j0b = hb ? j0a + kAttnTile : (1 << 30);
    if (new_lo < p_lo + (t + 2) * kAttnTile && new_hi >= p_lo + t * kAttnTile) {  // rare
      patch(ka, va, j0a);
      if (hb) patch(kb, vb, j0b);
    }
    step(ka, kb, va, vb, 256, j0a, j0b, qlim);
    st.fill<PK_ATTN, PK_WO>(sm, P, N, last + 1, wave, lane);
  }
  if (P.U && wave == 0) {  // the trailing row, from its bf16 copy in LDS (rows r > 0 masked)
    const char* kr = reinterpret_cast<const char*>(nkb);
    const char* vr = reinterpret_cast<const char*>(nvb);
    step(kr, kr, vr, vr, 0, P.F, 1 << 30, qvis);
  }
  st.mark(2);
  if (!active) return;
  __syncthreads();  // every wave has its queries in registers before the wave states overwrite them
  // Wave state: lane l holds query l & 15's sums over dims 16nb + 4(l >> 4)
  // + i; lsum is the lane's share of the query's sum (over 4 lane groups).
  constexpr float kLn2 = 0.6931471805599453f;
  float lw = lsum;
  lw += __shfl_xor(lw, 16);
  lw += __shfl_xor(lw, 32);
  if (qok) {
    float* dst = wst + (size_t)(wave * NQ + min(qq, NQ - 1)) * kPartStride;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
      *reinterpret_cast<float4*>(dst + 4 + nb * 16 + 4 * lg) = make_float4(acc[nb][0], acc[nb][1], acc[nb][2], acc[nb][3]);
    if (lg == 0) {
      dst[0] = m_l == -INFINITY ? -INFINITY : m_l * kLn2;  // natural units
      dst[1] = lw;
    }
  }
  __syncthreads();
  // merge the 4 wave states into the split partial
  tagword_t* part = reinterpret_cast<tagword_t*>(act_w(p, l, p.al.part)) +
                    ((size_t)(((seq * p.G + g) * QG + qg) * S + s) * Q) * kPartStride;
  for (int it = threadIdx.x; it < Q * (hd / 4 + 1); it += kThreads) {
    const int q = it / (hd / 4 + 1), k4 = it % (hd / 4 + 1);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, wst[(size_t)(w * NQ + q) * kPartStride]);
    float cw[kWaves];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = wst[(size_t)(w * NQ + q) * kPartStride];
      cw[w] = (mw == -INFINITY) ? 0.f : __expf(mw - M);
    }
    tagword_t* dst = part + (size_t)q * kPartStride;
    if (k4 == hd / 4) {
      float L = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) L += cw[w] * wst[(size_t)(w * NQ + q) * kPartStride + 1];
      st_tag(dst + 0, M, ms->tag);
      st_tag(dst + 1, L, ms->tag);
    } else {
      float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float* src = wst + (size_t)(w * NQ + q) * kPartStride + 4 + 4 * k4;
        a.x += cw[w] * src[0]; a.y += cw[w] * src[1]; a.z += cw[w] * src[2]; a.w += cw[w] * src[3];
      }
      st_tag(dst + 4 + 4 * k4, a.x, ms->tag); st_tag(dst + 5 + 4 * k4, a.y, ms->tag);
      st_tag(dst + 6 + 4 * k4, a.z, ms->tag); st_tag(dst + 7 + 4 * k4, a.w, ms->tag);
    }
  }
  __syncthreads();  // the wave states are read before the gather reuses the x region
  attn_gather(p, sm, l, seq, g, qg, s, Q);
}

// WO: h1 = h + Wo . o
template <typename WT, int MT>
__device__ __forceinline__ void phase_wo(const KParams& p, Smem sm, int l, Stream& st, const Plan& P, const Plan& N) {
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int M = p.M, d = p.d;
  const int K = p.H * p.hd;
  const float* o = act_f(p, l, p.al.o);
  const float* h = layer_in(p, l);
  float* h1 = act_w(p, l, p.al.h1);
  XRegs<WT, MT> xr;
  load_x<WT, MT>(xr, o, K, (const WT*)nullptr, M, wave, lane, P.lrb);
  zero_part(sm);
  const int rpt = P.rpt, lo = P.lo, lrb = P.lrb, n = P.n;
  const int ncol = n * rpt;
  load_res(sm, h, nullptr, d, lo * rpt, ncol, M);
  __syncthreads();
  constexpr int kRound = kPartAcc / (kWaves * Slots<WT>::C * MT);
  const float* res = res_slice(sm);
  run_gemv<WT, MT, PK_WO, PK_RS>(
      sm, st, P, N, xr, [&](int i, Seg<MT>& sg) { seg_rounds<MT>(sg, i, 0, n, kRound, M); },
      [&](int first, int last) {
        const int nr = (last - first + 1) * rpt;
        for (int it = threadIdx.x; it < nr * M; it += kThreads) {
          const int q = it / M, t = it - q * M;
          const int row = (lo + first) * rpt + q;
          st_dev(h1 + (size_t)t * d + row, res[t * ncol + row - lo * rpt] + part_row<WT, MT>(sm.part, q / rpt, q % rpt, lrb, t));
        }
      });
}

// RS: router logits and shared-expert gate/up.  The x registers (h1 * g2)
// stay loaded for the routed gate/up rows of the next phase.
template <typename WT, int MT>
__device__ __forceinline__ void phase_rs(const KParams& p, Smem sm, int l, Stream& st, const Plan& P, const Plan& N,
                         XRegs<WT, MT>& xr) {
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const auto& Ly = layer_tab(p)[l];
  const int d = p.d, F = p.F, E = p.E, M = p.M, S = p.S;
  const float* h1 = layer_h1(p, l);
  const float* br = Ly.b_router;
  const int has_bias = p.has_bias;
  float* logits = act_w(p, l, p.al.logits);
  float* a_s = act_w(p, l, p.al.a_s);
  load_x_norm<WT, MT>(xr, sm, h1, d, reinterpret_cast<const WT*>(Ly.moe_norm), M, d, p.eps, wave, lane, P.lrb);
  zero_part(sm);
  if (has_bias) load_res(sm, br, nullptr, 0, 0, E, 1);
  __syncthreads();
  const float* res = res_slice(sm);
  constexpr int kRound = (kPartAcc / (kWaves * Slots<WT>::C * MT)) & ~1;  // even: a pair stays in one round
  const Misc* ms = sm.misc;
  const int rpt = P.rpt, lrb = P.lrb, n1 = P.n1, n = P.n, r_lo = P.lo, p_lo = P.lo2, fb_per = P.fb_per;
  run_gemv<WT, MT, PK_RS, PK_RG>(
      sm, st, P, N, xr,
      [&](int i, Seg<MT>& sg) {
        if (i < n1) seg_rounds<MT>(sg, i, 0, n1, kRound, M);
        else seg_rounds<MT>(sg, i, n1, n, kRound, M);
      },
      [&](int first, int last) {
        if (first < n1) {
          const int nr = (last - first + 1) * rpt;
          for (int it = threadIdx.x; it < nr * M; it += kThreads) {
            const int q = it / M, t = it - q * M;
            const int e = (r_lo + first) * rpt + q;
            if (e >= E) continue;
            float v = part_row<WT, MT>(sm.part, q / rpt, q % rpt, lrb, t) * ms->rinv[t];
            if (has_bias) v += res[e];
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
            const float gv = part_row<WT, MT>(sm.part, 2 * pr, q, lrb, t) * ri;
            const float uv = part_row<WT, MT>(sm.part, 2 * pr + 1, q, lrb, t) * ri;
            st_dev(a_s + ((size_t)t * S + sx) * F + f, gv / (1.f + __expf(-gv)) * uv);
          }
        }
      });
}

// Top-k over the router logits of every row (all CUs, redundantly), then the
// union of chosen experts.  Selection is on the logits, larger first, equal
// logits ranked by lower expert id; weights are softmax probabilities
// renormalised over the chosen set.
__device__ __forceinline__ void route_rank(const KParams& p, Smem sm, int l) {
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int E = p.E, k = p.k, M = p.M;
  const float* logits = act_f(p, l, p.al.logits);
  Misc* ms = sm.misc;
  // rank[t][e]: top-k slot of expert e in row t, or -1.  Kept in the
  // epilogue residual slice of the part region, which is free until DOWN.
  int* rank_tab = reinterpret_cast<int*>(res_slice(sm));
  static_assert(kMaxRows * kMaxExperts <= kResFloats, "rank table does not fit");
  // Item (t, e) = it = 64 t + e: one wave holds whole rows, a lane one expert.
  // Sort key: the logit's bits made order-preserving as an unsigned integer,
  // above 63 - e, so that equal logits rank the lower id first and all keys
  // of a row differ; rank = number of larger keys in the row.  The keys sit
  // in the GEMV partial-sum region, unused until the phase's GEMV starts.
  unsigned long long* keys = reinterpret_cast<unsigned long long*>(sm.part);
  static_assert(kMaxRows * kMaxExperts * 8 <= kPartAcc * 4, "key table does not fit");
  constexpr int kItems = kMaxRows * kMaxExperts / kThreads;
  float zi[kItems], zmi[kItems];
  unsigned long long ki[kItems];
#pragma unroll
  for (int q = 0; q < kItems; ++q) {
    const int it = threadIdx.x + q * kThreads;
    const int t = it >> 6, e = it & 63;
    const float z = (t < M && e < E) ? logits[(size_t)t * E + e] : -INFINITY;
    unsigned u = __float_as_uint(z + 0.0f);  // -0 counts as +0
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    ki[q] = ((unsigned long long)u << 32) | (unsigned)(63 - e);
    keys[it] = ki[q];
    // row maximum over the wave
    float m = z;
    m = fmaxf(m, dpp<kDppXor1>(m));
    m = fmaxf(m, dpp<kDppXor2>(m));
    m = fmaxf(m, dpp<kDppRor4>(m));
    m = fmaxf(m, dpp<kDppRor8>(m));
    auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    m = fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
    auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    zmi[q] = fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
    zi[q] = z;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kItems; ++q) {
    const int it = threadIdx.x + q * kThreads;
    const int t = it >> 6, e = it & 63;
    if (t < M) {
      const unsigned long long* kr = keys + (it & ~63);
      int r = 0;
#pragma unroll 8
      for (int j = 0; j < kMaxExperts; j += 2) {
        const ulonglong2 kk = *reinterpret_cast<const ulonglong2*>(kr + j);
        r += (kk.x > ki[q] ? 1 : 0) + (kk.y > ki[q] ? 1 : 0);
      }
      const bool sel = e < E && r < k;
      rank_tab[it] = sel ? r : -1;
      if (sel) {
        ms->ids[t * k + r] = e;
        ms->wts[t * k + r] = __expf(zi[q] - zmi[q]);  // normalised below
      }
    }
  }
  __syncthreads();
  // renormalise over the chosen set: w = p_e / sum_{top-k} p
  {
    const int t = threadIdx.x / kMaxTopK, i = threadIdx.x % kMaxTopK;
    float w = 0.f, psum = 0.f;
    if (t < M && i < k) {
      w = ms->wts[t * k + i];
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j) psum += (j < k) ? ms->wts[t * k + min(j, k - 1)] : 0.f;
    }
    __syncthreads();
    if (t < M && i < k) ms->wts[t * k + i] = w / psum;
  }
  __syncthreads();
  // union of the rows' experts (ascending ids), read without branches
  if (wave == 0) {
    bool u = false;
#pragma unroll
    for (int t = 0; t < kMaxRows; ++t) u |= (t < M) & (rank_tab[t * kMaxExperts + lane] >= 0);
    const unsigned long long mm = __ballot(u);
    if (u) ms->uni[__popcll(mm & ((1ull << lane) - 1ull))] = lane;
    if (lane == 0) ms->n_uni = __popcll(mm);
  }
  __syncthreads();
}

// The routing step's tables, after route_rank: uslot[u][t] (top-k slot of
// union expert u in row t, or -1), umask[u] (its rows), and the trace.
__device__ __forceinline__ void route_tables(const KParams& p, Smem sm, int l) {
  const int E = p.E, k = p.k, M = p.M;
  const float* logits = act_f(p, l, p.al.logits);
  Misc* ms = sm.misc;
  const int* rank_tab = reinterpret_cast<const int*>(res_slice(sm));
  const int n_uni = ms->n_uni;
  for (int it = threadIdx.x; it < kMaxExperts * kMaxRows; it += kThreads) {
    const int u = it / kMaxRows, t = it % kMaxRows;
    const int e = ms->uni[u] & (kMaxExperts - 1);
    const int r = rank_tab[t * kMaxExperts + e];
    ms->uslot[it] = (signed char)((u < n_uni && t < M) ? r : -1);
  }
  __syncthreads();
  for (int u = threadIdx.x; u < kMaxExperts; u += kThreads) {
    const signed char* us = ms->uslot + u * kMaxRows;
    unsigned m = 0;
#pragma unroll
    for (int t = 0; t < kMaxRows; ++t) m |= (us[t] >= 0 ? 1u : 0u) << t;
    ms->umask[u] = m;
  }
  __syncthreads();
  if (vcu_of(p) == 0) {  // one workgroup of each row group
    const int row0 = p.row0 + grp_of(p) * M;
    for (int i = threadIdx.x; i < M * k; i += kThreads) {
      if (p.t_ids) p.t_ids[((size_t)l * p.Mt + row0) * k + i] = ms->ids[i];
      if (p.t_w) p.t_w[((size_t)l * p.Mt + row0) * k + i] = ms->wts[i];
    }
    if (p.t_logits)
      for (int i = threadIdx.x; i < M * E; i += kThreads) p.t_logits[((size_t)l * p.Mt + row0) * E + i] = logits[i];
  }
}

__device__ __forceinline__ void route_topk(const KParams& p, Smem sm, int l) {
  route_rank(p, sm, l);
  route_tables(p, sm, l);
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
    for (int t = 0; t < MT; ++t) {  // every row offset is valid; tm masks the arithmetic
      const float* s = base + rowoff[t] + k0;
#pragma unroll
      for (int j = 0; j < EPL; j += 4) {
        const float4 a4 = *reinterpret_cast<const float4*>(s + j);
        xr.v[t][c][j] = a4.x; xr.v[t][c][j + 1] = a4.y; xr.v[t][c][j + 2] = a4.z; xr.v[t][c][j + 3] = a4.w;
      }
    }
  }
}

// x registers from LDS rows given by rowof(t) (the row offset of token t,
// every offset valid; the token mask is applied to the results).  8 rows with
// bf16 weights: each lane forms the offsets of its own two tokens.
template <typename WT, int MT, class RowFn>
__device__ __forceinline__ void load_x_rows(XRegs<WT, MT>& xr, const float* base, RowFn rowof, int wave, int lane,
                                            int lrb) {
  if constexpr (std::is_same<WT, uint16_t>::value && MT == 8) {
    const int t4 = lane & 3, b = lane >> 2;
    const int k0 = m8_kq(wave, lrb) + b * 4;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float* s = base + rowof(t4 + 4 * h) + k0;
#pragma unroll
      for (int kc = 0; kc < 16; ++kc)
        split_bf16x4(*reinterpret_cast<const float4*>(s + kc * 64), xr.hi[h][kc], xr.lo[h][kc]);
    }
  } else {
    int ro[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) ro[t] = rowof(t);
    load_x_lds<WT, MT>(xr, base, ro, 0u, wave, lane, lrb);
  }
}

// Shared activations a_s [M][S][F] -> LDS by DMA (whole KiB; F*4 bytes is a
// multiple of 1 KiB), issued right after the RS -> RG barrier so that its
// latency overlaps the routing step's load of the logits.
__device__ __forceinline__ void rg_stage(const KParams& p, Smem sm, int l) {
  dma_to_lds((char*)sm.xs, (const char*)act_f(p, l, p.al.a_s), p.M * p.S * p.F * 4, wave_id(), threadIdx.x & 63);
}

// RG: shared-expert down projection y_s = sum_s Wd_s a_s (x from LDS), then
// the routed gate/up rows for the union experts (x = y from RS):
// a[t][slot][f] for the rows routed to the expert.
// early: tiles of P issued after the shared activations' DMA (rg_stage),
// before this call; 0 when none.  The wait below then leaves them in flight.
template <typename WT, int MT>
__device__ __forceinline__ void phase_rg(const KParams& p, Smem sm, int l, Stream& st, const Plan& P, const Plan& N,
                                         const XRegs<WT, MT>& xr, int early) {
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int d = p.d, F = p.F, k = p.k, M = p.M, S = p.S;
  float* a = act_w(p, l, p.al.a);
  float* ys = act_w(p, l, p.al.y_s);
  // misc->rinv still holds RS's 1/rms of h1; the shared activations are on
  // their way to LDS (rg_stage, issued before the routing step).  This
  // wave's part of them has landed once at most 2 * early of its vector
  // memory operations are outstanding (they complete in order); no
  // compiler-visible load is pending here, so the GEMV needs no full drain.
  zero_part(sm);
  if (early > 0) wait_tiles_ahead(early);
  else wait_all();
  __syncthreads();
  const Misc* ms = sm.misc;
  constexpr int kRound = (kPartAcc / (kWaves * Slots<WT>::C * MT)) & ~1;  // even: a gate/up pair stays in one round
  const int n1 = P.n1, n = P.n, nj = P.nj, lrb = P.lrb, lrb2 = P.lrb2, rpt = P.rpt, rpt2 = P.rpt2;
  const int fb_per = P.fb_per, sd_lo = P.lo, p_lo = P.lo2;
  XRegs<WT, MT> xw;  // a_s rows for the shared-down tiles, then y
  run_gemv<WT, MT, PK_RG, MT == 1 ? PK_DOWN : PK_DOWNA, false>(
      sm, st, P, N, xw,
      [&](int i, Seg<MT>& sg) {
        seg_all<MT>(sg, M);
        if (i < n1) {  // expert s of the shared down projection, all of this CU's j-blocks
          const int sx = i / nj;
          load_x_rows<WT, MT>(xw, sm.xs, [&](int t) { return (t * S + sx) * F; }, wave, lane, lrb);
          sg.end = i + nj;
          sg.blk0 = 0;
          sg.accum = true;
          sg.round_end = sg.end == n1;
        } else {
          if (i == n1) xw = xr;
          const int k0 = i - n1;
          int end = n1 + min(n - n1, (k0 / kRound + 1) * kRound);
          if (M > 1) {  // one run per expert: its rows only
            const int u = (p_lo + k0 / 2) / fb_per;
            end = min(end, n1 + 2 * ((u + 1) * fb_per - p_lo));
            sg.tmask = ms->umask[u];
          }
          sg.end = end;
          sg.blk0 = k0 % kRound;
          sg.accum = false;
          sg.round_end = end == n || ((end - n1) % kRound) == 0;
        }
      },
      [&](int first, int last) {
        if (first < n1) {
          // shared-down j-blocks of this CU: y_s[t][j]
          for (int it = threadIdx.x; it < nj * rpt * M; it += kThreads) {
            const int u = it / (rpt * M), q = (it / M) % rpt, t = it % M;
            const int j = (sd_lo + u) * rpt + q;
            st_dev(ys + (size_t)t * d + j, part_row<WT, MT>(sm.part, u, q, lrb, t));
          }
        } else {
          const int k0 = first - n1;
          const int npairs_r = (last - first + 1) / 2;
          for (int it = threadIdx.x; it < npairs_r * rpt2 * M; it += kThreads) {
            const int pr = it / (rpt2 * M), q = (it / M) % rpt2, t = it % M;
            const int pj = p_lo + k0 / 2 + pr;
            const int u = pj / fb_per, f = (pj % fb_per) * rpt2 + q;
            const int sl = ms->uslot[u * kMaxRows + t];
            if (sl < 0) continue;
            const float ri = ms->rinv[t];
            const float gv = part_row<WT, MT>(sm.part, 2 * pr, q, lrb2, t) * ri;
            const float uv = part_row<WT, MT>(sm.part, 2 * pr + 1, q, lrb2, t) * ri;
            st_dev(a + ((size_t)t * k + sl) * F + f, gv / (1.f + __expf(-gv)) * uv);
          }
        }
      });
}

// RG of a row-group launch (8-row token groups, bf16 weights): this group's
// shared-down tiles as in phase_rg, then this workgroup's range of the
// tasks' gate/up pairs.  A task's x rows are its rows' h1, normed with the
// same arithmetic as the groups' own RS (the register layout does not
// depend on a row's place in the group), loaded when the task starts; each
// row's 1/rms goes to rinv_row.  Outputs go to the rows' own groups.
template <typename WT>
__device__ __forceinline__ void phase_rg_t(const KParams& p, Smem sm, int l, Stream& st, const Plan& P,
                                           const Plan& N, int early) {
  constexpr int MT = 8;
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int d = p.d, F = p.F, k = p.k, M = p.M, S = p.S;
  float* ys = act_w(p, l, p.al.y_s);
  zero_part(sm);
  if (early > 0) wait_tiles_ahead(early);
  else wait_all();
  __syncthreads();
  Misc* ms = sm.misc;
  constexpr int kRound = (kPartAcc / (kWaves * Slots<WT>::C * MT)) & ~1;  // even: a gate/up pair stays in one round
  const int n1 = P.n1, n = P.n, nj = P.nj, lrb = P.lrb, lrb2 = P.lrb2, rpt = P.rpt, rpt2 = P.rpt2;
  const int fb_per = P.fb_per, sd_lo = P.lo, p_lo = P.lo2;
  const WT* gam = reinterpret_cast<const WT*>(layer_tab(p)[l].moe_norm);
  XRegs<WT, MT> xw;  // a_s rows for the shared-down tiles, then a task's rows
  int xt = -1;       // task whose rows the registers hold
  run_gemv<WT, MT, PK_RGT, PK_DOWNT, false>(
      sm, st, P, N, xw,
      [&](int i, Seg<MT>& sg) {
        seg_all<MT>(sg, M);
        if (i < n1) {  // expert s of the shared down projection, all of this CU's j-blocks
          const int sx = i / nj;
          load_x_rows<WT, MT>(xw, sm.xs, [&](int t) { return (t * S + sx) * F; }, wave, lane, lrb);
          sg.end = i + nj;
          sg.blk0 = 0;
          sg.accum = true;
          sg.round_end = sg.end == n1;
        } else {
          const int k0 = i - n1;
          const int tk = (p_lo + k0 / 2) / fb_per;
          const int e0 = ms->tbeg[tk], cnt = ms->tbeg[tk + 1] - e0;
          int end = n1 + min(n - n1, (k0 / kRound + 1) * kRound);
          end = min(end, n1 + 2 * ((tk + 1) * fb_per - p_lo));  // one run per task
          sg.tmask = (1u << cnt) - 1u;
          if (tk != xt) {
            xt = tk;
            load_x_norm8(
                xw, sm,
                [&](int t) {
                  const int r = ent_row(ms->tent[e0 + t]);
                  return grp_h1(p, r / M, l) + (size_t)(r % M) * d;
                },
                cnt, gam, d, p.eps, wave, lane, lrb2,
                [&](int t, float v) { ms->rinv_row[ent_row(ms->tent[e0 + t])] = v; }, true);
          }
          sg.end = end;
          sg.blk0 = k0 % kRound;
          sg.accum = false;
          sg.round_end = end == n || ((end - n1) % kRound) == 0;
        }
      },
      [&](int first, int last) {
        if (first < n1) {
          // shared-down j-blocks of this CU: y_s[t][j]
          for (int it = threadIdx.x; it < nj * rpt * M; it += kThreads) {
            const int u = it / (rpt * M), q = (it / M) % rpt, t = it % M;
            const int j = (sd_lo + u) * rpt + q;
            st_dev(ys + (size_t)t * d + j, part_row<WT, MT>(sm.part, u, q, lrb, t));
          }
        } else {
          const int k0 = first - n1;
          const int npairs_r = (last - first + 1) / 2;
          for (int it = threadIdx.x; it < npairs_r * rpt2 * MT; it += kThreads) {
            const int pr = it / (rpt2 * MT), q = (it / MT) % rpt2, t = it % MT;
            const int pj = p_lo + k0 / 2 + pr;
            const QR tf = divmod_small(pj, fb_per);
            const int e0 = ms->tbeg[tf.q];
            if (t >= ms->tbeg[tf.q + 1] - e0) continue;
            const unsigned en = ms->tent[e0 + t];
            const int r = ent_row(en), f = tf.r * rpt2 + q;
            const float ri = ms->rinv_row[r];
            const float gv = part_row<WT, MT>(sm.part, 2 * pr, q, lrb2, t) * ri;
            const float uv = part_row<WT, MT>(sm.part, 2 * pr + 1, q, lrb2, t) * ri;
            float* a = reinterpret_cast<float*>(grp_act(p, r / M, l) + p.al.a);
            st_dev(a + ((size_t)(r % M) * k + ent_slot(en)) * F + f, gv / (1.f + __expf(-gv)) * uv);
          }
        }
      });
}

// DOWN: for this CU's j-blocks (output columns), accumulate the union
// experts one after another (expert-major, so an expert's x rows are loaded
// once), each row weighted by its routing weight; then h2 = h1 + y_s + sum.
// The x rows a[t][slot] come from LDS when they fit.
template <typename WT, int MT>
__device__ __forceinline__ void phase_down(const KParams& p, Smem sm, int l, Stream& st, const Plan& P, const Plan& N) {
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int d = p.d, F = p.F, k = p.k, M = p.M;
  const int nj = P.nj, rpt = P.rpt, lrb = P.lrb, lo = P.lo, n = P.n;
  const float* h1 = layer_h1(p, l);
  const float* a_g = act_f(p, l, p.al.a);    // [M][k][F]
  const float* ys = act_f(p, l, p.al.y_s);   // [M][d]
  float* h2 = (l == p.L - 1) ? hidden_out_g(p) : act_w(p, l, p.al.h2);
  const bool last_layer = (l == p.L - 1);
  const bool xl = (size_t)M * k * F * 4 <= (size_t)kXsBytes;
  if (xl) dma_to_lds((char*)sm.xs, (const char*)a_g, M * k * F * 4, wave, lane);
  zero_part(sm);
  const bool has_shared = p.S > 0;
  const int ncol = nj * rpt;
  load_res(sm, h1, has_shared ? ys : nullptr, d, lo * rpt, ncol, M);
  wait_all();
  __syncthreads();
  const Misc* ms = sm.misc;
  const float* res = res_slice(sm);
  auto epilogue = [&](int, int) {
    for (int it = threadIdx.x; it < ncol * M; it += kThreads) {
      const int q = MT == 1 ? it : it / M, t = MT == 1 ? 0 : it - q * M;
      const int j = lo * rpt + q;
      const float out = res[t * ncol + q] + part_row<WT, MT>(sm.part, q >> (13 - lrb), q & (rpt - 1), lrb, t);
      if (last_layer) h2[(size_t)t * d + j] = out;
      else st_dev(h2 + (size_t)t * d + j, out);
    }
  };
  if constexpr (MT == 1) {
    constexpr int G = GroupOf<WT, 1>::G;
    if (nj <= G && xl) {
      // One row: the union experts are its k experts, each expert's j-blocks
      // form one group, and the weighted partial sums of all experts stay in
      // registers until one cross-lane reduction at the end.  The next
      // expert's x registers are read from LDS while the current expert's
      // tiles are consumed.  Lane u < U holds expert u's x offset and weight.
      const int U = P.U;
      const int su = ms->uslot[(lane & (kMaxTopK - 1)) * kMaxRows];
      const int sc = su < 0 ? 0 : su;
      const int xoff_l = sc * F;
      const float wt_l = ms->wts[sc];
      XRegs<WT, 1> xa, xb;
      auto ldx = [&](XRegs<WT, 1>& x, int u) {
        const int ro[1] = {__builtin_amdgcn_readlane(xoff_l, u)};
        load_x_lds<WT, 1>(x, sm.xs, ro, 1u, wave, lane, lrb);
      };
      constexpr int C = Slots<WT>::C;
      float pacc[G * C];
#pragma unroll
      for (int v = 0; v < G * C; ++v) pacc[v] = 0.f;
      st.mark(1);
      settle();
      st.fill<PK_DOWN, kAnyKind>(sm, P, N, 0, wave, lane);
      ldx(xa, 0);
      for (int u = 0; u < (nj > 0 ? U : 0); ++u) {
        if (u + 1 < U) ldx(xb, u + 1);
        const float tw = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wt_l), u));
        const int j = u * nj;
        st.wait(j + nj - 1);
        gemv_acc1<WT>(sm, st, j, nj, xa, tw, pacc, wave, lane);
        st.fill<PK_DOWN, kAnyKind>(sm, P, N, j + nj, wave, lane);
        xa = xb;
      }
      const float r = xreduce<G * C>(pacc, lane);
      if (xreduce_writer<G * C>(lane)) {
        const int idx = xreduce_index<G * C>(lane);
        if (idx / C < nj) sm.part[(idx / C) * (kWaves * C) + wave * C + idx % C] = r;
      }
      __syncthreads();
      epilogue(0, n - 1);
      __syncthreads();
      st.mark(2);
      return;
    }
  }
  XRegs<WT, MT> xr;
  run_gemv<WT, MT, PK_DOWN, kAnyKind>(
      sm, st, P, N, xr,
      [&](int i, Seg<MT>& sg) {
        const int u = i / nj;
        unsigned tm = 0;
#pragma unroll
        for (int t = 0; t < MT; ++t) {  // uslot is -1 for rows beyond M
          const int sl = ms->uslot[u * kMaxRows + t];
          const int slc = sl < 0 ? 0 : sl;
          const float wt = ms->wts[min(t * k + slc, kMaxRows * kMaxTopK - 1)];
          sg.tw[t] = sl < 0 ? 0.f : wt;
          tm |= (sl < 0 ? 0u : 1u) << t;
        }
        load_x_rows<WT, MT>(
            xr, xl ? sm.xs : a_g,
            [&](int t) {  // t may differ across lanes: the slot is read per lane
              const int sl = ms->uslot[u * kMaxRows + t];
              return sl < 0 ? 0 : (t * k + sl) * F;
            },
            wave, lane, lrb);
        sg.tmask = tm;
        sg.end = i + nj;
        sg.blk0 = 0;
        sg.accum = true;
        sg.round_end = sg.end == n;
      },
      epilogue);
}

// DOWN with several rows, first half: this CU's contiguous range of the
// (union expert, j-block) tiles, expert-major, so the x rows of an expert
// (the activations of the rows routed to it) are loaded once per CU instead
// of once per expert.  Each tile's weighted products for the routed rows go
// to yp[t][slot][j]; the second half sums a row's slots per column.  The
// residual h1 + y_s of the second half's columns goes to LDS here.
template <typename WT, int MT>
__device__ __forceinline__ void phase_down_a(const KParams& p, Smem sm, int l, Stream& st, const Plan& P,
                                             const Plan& N) {
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int d = p.d, F = p.F, k = p.k, M = p.M;
  const int nj = P.nj, rpt = P.rpt, lrb = P.lrb, lo = P.lo, n = P.n;
  const float* h1 = layer_h1(p, l);
  const float* a_g = act_f(p, l, p.al.a);    // [M][k][F]
  const float* ys = act_f(p, l, p.al.y_s);   // [M][d]
  float* yp = act_w(p, l, p.al.yp);          // [M][k][d]
  const bool xl = (size_t)M * k * F * 4 <= (size_t)kXsBytes;
  if (xl) dma_to_lds((char*)sm.xs, (const char*)a_g, M * k * F * 4, wave, lane);
  zero_part(sm);
  load_res(sm, h1, p.S > 0 ? ys : nullptr, d, P.lo2 * rpt, P.n1 * rpt, M);
  wait_all();
  __syncthreads();
  const Misc* ms = sm.misc;
  constexpr int kRound = kPartAcc / (kWaves * Slots<WT>::C * MT);
  const int lrpt = 13 - lrb;  // log2 rows per tile
  XRegs<WT, MT> xr;
  int xu = -1;  // expert whose x rows the registers hold
  run_gemv<WT, MT, PK_DOWNA, kAnyKind>(
      sm, st, P, N, xr,
      [&](int i, Seg<MT>& sg) {
        const int u = (lo + i) / nj;
        sg.end = min(min(n, (u + 1) * nj - lo), (i / kRound + 1) * kRound);
        sg.blk0 = i % kRound;
        sg.accum = false;
        sg.round_end = sg.end == n || sg.end % kRound == 0;
        sg.tmask = ms->umask[u];
#pragma unroll
        for (int t = 0; t < MT; ++t) {  // uslot is -1 for rows beyond M
          const int sl = ms->uslot[u * kMaxRows + t];
          sg.tw[t] = sl < 0 ? 0.f : ms->wts[t * k + sl];
        }
        if (u != xu) {
          xu = u;
          load_x_rows<WT, MT>(
              xr, xl ? sm.xs : a_g,
              [&](int t) {  // t may differ across lanes: the slot is read per lane
                const int sl = ms->uslot[u * kMaxRows + t];
                return sl < 0 ? 0 : (t * k + sl) * F;
              },
              wave, lane, lrb);
        }
      },
      [&](int first, int last) {
        for (int it = threadIdx.x; it < (last - first + 1) << lrpt; it += kThreads) {
          const int b = it >> lrpt, r = it & (rpt - 1);
          const int g = lo + first + b, u = g / nj, jb = g - u * nj;
          float* dst = yp + (size_t)jb * rpt + r;
          for (unsigned m = ms->umask[u]; m; m &= m - 1) {
            const int t = __builtin_ctz(m);
            const int sl = ms->uslot[u * kMaxRows + t];
            st_dev(dst + ((size_t)t * k + sl) * d, part_row<WT, MT>(sm.part, b, r, lrb, t));
          }
        }
      });
}

// DOWN of a row-group launch, first half: this workgroup's range of the
// (task, j-block) tiles; a task's x rows are a[row][slot] of its pairs, in
// the rows' own groups, weighted by their routing weights; the products go
// to yp[row][slot][j] of the rows' groups.  The residual h1 + y_s of this
// group's second-half columns goes to LDS here.
template <typename WT>
__device__ __forceinline__ void phase_down_a_t(const KParams& p, Smem sm, int l, Stream& st, const Plan& P,
                                               const Plan& N) {
  constexpr int MT = 8;
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int d = p.d, F = p.F, k = p.k, M = p.M;
  const int nj = P.nj, rpt = P.rpt, lrb = P.lrb, lo = P.lo, n = P.n;
  const float* h1 = layer_h1(p, l);
  const float* ys = act_f(p, l, p.al.y_s);
  const float* wts = rtab_wts(p, l);
  zero_part(sm);
  load_res(sm, h1, p.S > 0 ? ys : nullptr, d, P.lo2 * rpt, P.n1 * rpt, M);
  wait_all();
  __syncthreads();
  Misc* ms = sm.misc;
  constexpr int kRound = kPartAcc / (kWaves * Slots<WT>::C * MT);
  const int lrpt = 13 - lrb;  // log2 rows per tile
  XRegs<WT, MT> xr;
  int xt = -1;  // task whose x rows the registers hold
  run_gemv<WT, MT, PK_DOWNT, kAnyKind>(
      sm, st, P, N, xr,
      [&](int i, Seg<MT>& sg) {
        const int tk = (lo + i) / nj;
        const int e0 = ms->tbeg[tk], cnt = ms->tbeg[tk + 1] - e0;
        sg.end = min(min(n, (tk + 1) * nj - lo), (i / kRound + 1) * kRound);
        sg.blk0 = i % kRound;
        sg.accum = false;
        sg.round_end = sg.end == n || sg.end % kRound == 0;
        sg.tmask = (1u << cnt) - 1u;
        if (tk != xt) {
          xt = tk;
          // every wave has taken the last task's weights before they change
          __syncthreads();
          if ((int)threadIdx.x < MT) {
            const int t = threadIdx.x;
            const unsigned en = ms->tent[e0 + min(t, cnt - 1)];
            ms->task_w[t] = t < cnt ? wts[ent_row(en) * k + ent_slot(en)] : 0.f;
          }
          load_x8_rows(
              xr,
              [&](int t) {
                const unsigned en = ms->tent[e0 + t];
                const int r = ent_row(en);
                return reinterpret_cast<const float*>(grp_act(p, r / M, l) + p.al.a) +
                       ((size_t)(r % M) * k + ent_slot(en)) * F;
              },
              cnt, wave, lane, lrb);
          __syncthreads();
        }
#pragma unroll
        for (int t = 0; t < MT; ++t) sg.tw[t] = ms->task_w[t];
      },
      [&](int first, int last) {
        for (int it = threadIdx.x; it < (last - first + 1) << lrpt; it += kThreads) {
          const int b = it >> lrpt, r = it & (rpt - 1);
          const int g = lo + first + b;
          const QR tj = divmod_small(g, nj);
          const int e0 = ms->tbeg[tj.q], cnt = ms->tbeg[tj.q + 1] - e0;
          for (int t = 0; t < cnt; ++t) {
            const unsigned en = ms->tent[e0 + t];
            const int row = ent_row(en);
            float* yp = reinterpret_cast<float*>(grp_act(p, row / M, l) + p.al.yp);
            st_dev(yp + ((size_t)(row % M) * k + ent_slot(en)) * d + (size_t)tj.r * rpt + r,
                   part_row<WT, MT>(sm.part, b, r, lrb, t));
          }
        }
      });
}

// DOWN with several rows, second half: h2[t][j] = h1 + y_s + the sum of
// yp[t][slot][j] over the row's top-k slots, for this CU's output columns
// [c0, c0 + ncol) (the residual is in LDS from the first half).
__device__ __forceinline__ void phase_down_b(const KParams& p, Smem sm, int l, int c0, int ncol) {
  const int d = p.d, k = p.k, M = p.M;
  const float* yp = act_f(p, l, p.al.yp);
  const bool last_layer = (l == p.L - 1);
  float* h2 = last_layer ? hidden_out_g(p) : act_w(p, l, p.al.h2);
  const float* res = res_slice(sm);
  for (int it = threadIdx.x; it < ncol * M; it += kThreads) {
    const int t = it / ncol, c = it - t * ncol;
    const float* src = yp + (size_t)t * k * d + c0 + c;
    float v[kMaxTopK];
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s) v[s] = s < k ? src[(size_t)s * d] : 0.f;
    float out = res[it];
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s) out += v[s];
    if (last_layer) h2[(size_t)t * d + c0 + c] = out;
    else st_dev(h2 + (size_t)t * d + c0 + c, out);
  }
}

// ------------------------------------------------------------------ kernel

// LDS carve-up of the kernels
__device__ __forceinline__ Smem smem_carve() {
  Smem sm;
  sm.ring = smem_raw;
  sm.xs = reinterpret_cast<float*>(smem_raw + (size_t)kRing * kSlotBytes);
  sm.part = reinterpret_cast<float*>(smem_raw + (size_t)kRing * kSlotBytes + kXsBytes);
  sm.misc = reinterpret_cast<Misc*>(smem_raw + (size_t)kRing * kSlotBytes + kXsBytes + kPartBytes);
  return sm;
}

// Launch set-up: positions (range and distinctness within a sequence; every
// CU checks the same data, so all leave together on a bad input, which
// block 0 reports on the error flag), the launch's barrier epoch and the
// RoPE table.  Returns false when the launch must end.
__device__ __forceinline__ bool launch_setup(const KParams& p, Smem sm) {
  Misc* ms = sm.misc;
  if (threadIdx.x == 0) {
    int bad = 0;
    const int* positions = p.positions + (size_t)grp_of(p) * p.M;
    for (int r = 0; r < p.M; ++r) {
      const int pos = positions[r];
      ms->pos[r] = pos;
      if (p.attn && (pos < 0 || pos >= p.cap)) bad |= kErrPosition;
    }
    if (p.attn)
      for (int r = 0; r < p.M; ++r)
        for (int r2 = r + 1; r2 < p.M && r2 / p.rps == r / p.rps; ++r2)
          if (ms->pos[r] == ms->pos[r2]) bad |= kErrDupPosition;
    ms->flag = bad;
    ms->epoch = (int)ld_dev(p.sync + SyncLayout::kEpoch);
    // The tag epoch changes only where no block of a launch that uses tags
    // can still read it (after the persistent kernel's last grid barrier; in
    // phase launches other than attention), so all blocks of a launch read
    // the same value.  Taken on the device, it also differs between replays
    // of a captured graph.
    ms->tag = ld_dev(p.sync + SyncLayout::kTag) + 1u;
  }
  __syncthreads();
  if (ms->flag) {
    if (blockIdx.x == 0 && threadIdx.x == 0)
      __hip_atomic_fetch_or(p.sync + SyncLayout::kErr, (unsigned)ms->flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return false;
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
  return true;
}

// Row groups: the routed work of all groups of the launch as tasks.  Each
// group's routing (route_rank, the same in all its workgroups) is published
// by one workgroup per group (write-once per launch); after the next grid
// barrier every workgroup builds the same task table from all of it
// (build_tasks), and the routed tiles of the tasks are spread over every
// workgroup of the launch.  An expert chosen by n rows of the launch is then
// streamed ceil(n / kMaxRows) times, instead of once per group.
__device__ __forceinline__ void publish_routing(const KParams& p, Smem sm, int l) {
  if (vcu_of(p) != 0) return;
  const int mk_ = p.M * p.k, g = grp_of(p);
  int* ids = rtab_ids(p, l) + g * mk_;
  float* wts = rtab_wts(p, l) + g * mk_;
  const Misc* ms = sm.misc;
  for (int i = threadIdx.x; i < mk_; i += kThreads) {
    st_dev_u(reinterpret_cast<unsigned*>(ids + i), (unsigned)ms->ids[i]);
    st_dev(wts + i, ms->wts[i]);
  }
}

// The task table of layer l from the published routing: per expert in
// ascending id order, its (row, slot) pairs with rows ascending, cut into
// tasks of at most kMaxRows pairs.  Wave w counts and places the pairs of a
// quarter of the rows, lane e those of expert e; the counts' prefix sums
// over the experts give each expert's first entry and first task.  Scratch
// in the part region, which is free until the RG GEMV starts.
__device__ __forceinline__ void build_tasks(const KParams& p, Smem sm, int l) {
  Misc* ms = sm.misc;
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int nr = p.n_groups * p.M, k = p.k;
  const int* ids = rtab_ids(p, l);
  unsigned char* idb = reinterpret_cast<unsigned char*>(sm.part);  // [nr][8] expert ids, 0xff past k
  int* cnt = reinterpret_cast<int*>(sm.part) + kMaxGroups * kMaxRows * 8 / 4;  // [kWaves][64]
  static_assert(kMaxGroups * kMaxRows * 8 + kWaves * 64 * 4 <= kPartAcc * 4, "task scratch does not fit");
  for (int it = threadIdx.x; it < nr * 8; it += kThreads) {
    const int r = it >> 3, s = it & 7;
    idb[it] = (unsigned char)(s < k ? ids[r * k + s] : 0xff);
  }
  __syncthreads();
  const int r0 = wave * nr / kWaves, r1 = (wave + 1) * nr / kWaves;
  const int e = lane;
  int c = 0;
  for (int r = r0; r < r1; ++r) {
    const unsigned long long v = *reinterpret_cast<const unsigned long long*>(idb + r * 8);
#pragma unroll
    for (int s = 0; s < 8; ++s) c += (int)((v >> (8 * s)) & 0xffu) == e ? 1 : 0;
  }
  cnt[wave * 64 + e] = c;
  __syncthreads();
  if (wave == 0) {
    int n_e = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) n_e += cnt[w * 64 + e];
    const int nt_e = (n_e + kMaxRows - 1) / kMaxRows;
    // inclusive prefix sums over the lanes
    int ie = n_e, it = nt_e;
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) {
      const int ue = __shfl_up(ie, sh), ut = __shfl_up(it, sh);
      if (lane >= sh) {
        ie += ue;
        it += ut;
      }
    }
    const int eb = ie - n_e, tb = it - nt_e;
    for (int q = 0; q < nt_e; ++q) ms->tbeg[tb + q] = (unsigned short)(eb + q * kMaxRows);
    if (lane == 63) {
      ms->tbeg[it] = (unsigned short)ie;
      ms->n_task = it;
    }
    // first entry of each wave's pairs of expert e
    int off = eb;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int cw = cnt[w * 64 + e];
      cnt[w * 64 + e] = off;
      off += cw;
    }
  }
  __syncthreads();
  int pos = cnt[wave * 64 + e];
  for (int r = r0; r < r1; ++r) {
    const unsigned long long v = *reinterpret_cast<const unsigned long long*>(idb + r * 8);
#pragma unroll
    for (int s = 0; s < 8; ++s)
      if ((int)((v >> (8 * s)) & 0xffu) == e) ms->tent[pos++] = (unsigned short)((e << 9) | (r << 3) | s);
  }
  __syncthreads();
}

// WT: weight element type; MT: rows of the token group (1 or 8); QK: kind of
// attention task, 1: at most 4 query vectors, 2: at most 16
template <typename WT, int MT, int QK>
__global__ void __launch_bounds__(kThreads, 1) decode_step_kernel(KParams kp) {
  const Smem sm = smem_carve();
  Misc* ms = sm.misc;
  const KParams& p = kp;
  if (!launch_setup(p, sm)) return;
  const unsigned epoch0 = (unsigned)ms->epoch;
  __syncthreads();
  unsigned b = 0;
  long long* stamp = p.stamps ? p.stamps + (size_t)blockIdx.x * 4 * (p.barriers + 1) : nullptr;
  XRegs<WT, MT> xr_moe;
  Stream st{0, 0, stamp, Win{0u, 0u, kNoWin}, Win{0u, 0u, kNoWin}, 0, lds_addr(sm.ring), p.n_groups > 1};
  // row groups in one launch: 8-row token groups with bf16 weights only (the
  // host runs other row groups one launch each)
  constexpr bool kTasks = MT == 8 && std::is_same<WT, uint16_t>::value;
  const int wave = wave_id(), lane = threadIdx.x & 63;
  // phase i owns slots 4i..4i+3: start (after barrier i), tile loop start,
  // tile loop end, end (before barrier i+1)
#define MK_SYNC()                                   \
  do {                                              \
    st.mark(3);                                     \
    if (!grid_sync(p, sm, epoch0 + ++b)) return;    \
    if (st.ts) st.ts += 4;                          \
    st.mark(0);                                     \
  } while (0)
  st.mark(0);
  const Plan none{};
  Plan cur = p.attn ? plan_qkv<WT>(p, 0) : plan_rs<WT>(p, 0);
  for (int l = 0; l < p.L; ++l) {
    if (p.attn) {
      {
        const Plan nxt = plan_attn(p, ms, l, true);
        phase_qkv<WT, MT>(p, sm, l, st, cur, nxt);
        MK_SYNC();
        st.advance(cur);
        cur = nxt;
      }
      {
        const Plan nxt = plan_wo<WT>(p, l);
        phase_attn_dec<QK == 1 ? 4 : 16>(p, sm, l, st, cur, nxt);
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
      rg_stage(p, sm, l);
      route_rank(p, sm, l);
      if (kTasks && p.n_groups > 1) {  // the routed work of all row groups as tasks
        if constexpr (kTasks) {
          publish_routing(p, sm, l);
          MK_SYNC();
          build_tasks(p, sm, l);
          cur = plan_rg_t<WT>(p, ms, l);  // same first tiles as the prefetched plan
          const Plan nxt = plan_down_t<WT>(p, ms, l);
          const int pre = st.issued;
          st.fill<PK_RGT, PK_DOWNT>(sm, cur, nxt, 0, wave, lane);
          route_tables(p, sm, l);  // the trace
          phase_rg_t<WT>(p, sm, l, st, cur, nxt, st.issued - pre);
          MK_SYNC();
          st.advance(cur);
          cur = nxt;
        }
      } else {
        cur = plan_rg<WT>(p, ms, l, true);  // same first tiles as the prefetched plan
        const Plan nxt = MT == 1 ? plan_down<WT>(p, ms, l) : plan_down_a<WT>(p, ms, l);
        // the routed tiles start streaming as soon as the union is known
        const int pre = st.issued;
        st.fill<PK_RG, MT == 1 ? PK_DOWN : PK_DOWNA>(sm, cur, nxt, 0, wave, lane);
        route_tables(p, sm, l);
        phase_rg<WT, MT>(p, sm, l, st, cur, nxt, xr_moe, st.issued - pre);
        MK_SYNC();
        st.advance(cur);
        cur = nxt;
      }
    }
    {
      const Plan nxt = (l + 1 < p.L) ? (p.attn ? plan_qkv<WT>(p, l + 1) : plan_rs<WT>(p, l + 1)) : none;
      if constexpr (MT == 1) {
        phase_down<WT, MT>(p, sm, l, st, cur, nxt);
        if (l + 1 < p.L) MK_SYNC();
        st.advance(cur);
        cur = nxt;
      } else {
        const int c0 = cur.lo2 * cur.rpt, ncol = cur.n1 * cur.rpt;
        if (kTasks && p.n_groups > 1) {
          if constexpr (kTasks) phase_down_a_t<WT>(p, sm, l, st, cur, nxt);
        } else {
          phase_down_a<WT, MT>(p, sm, l, st, cur, nxt);
        }
        MK_SYNC();
        st.advance(cur);
        cur = nxt;
        phase_down_b(p, sm, l, c0, ncol);  // no tiles: the next layer's first tiles stay in flight
        if (l + 1 < p.L) MK_SYNC();
      }
    }
  }
#undef MK_SYNC
  wait_all();
  st.mark(3);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    st_dev_u(p.sync + SyncLayout::kEpoch, epoch0 + b);
    st_dev_u(p.sync + SyncLayout::kTag, ms->tag);  // every block read the tag epoch before the first barrier
  }
}

// One phase of one layer per launch: the same phase code as the persistent
// kernel, with an empty ring at the start and no next phase to prefetch.
// The state a phase inherits inside the persistent kernel is rebuilt from
// the workspace: the normed x registers of the MoE block (RG), the routing
// tables (recomputed from the stored logits; deterministic) and the
// residual slice of the second DOWN half.  The kernel boundary replaces the
// grid barrier.  This is the many-kernels baseline the persistent kernel is
// measured against.
template <typename WT, int MT, int QK>
__global__ void __launch_bounds__(kThreads, 1) phase_step_kernel(KParams kp) {
  const Smem sm = smem_carve();
  Misc* ms = sm.misc;
  const KParams& p = kp;
  if (!launch_setup(p, sm)) return;
  __syncthreads();
  const int l = p.only_l;
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const Plan none{};
  Stream st{0, 0, nullptr, Win{0u, 0u, kNoWin}, Win{0u, 0u, kNoWin}, 0, lds_addr(sm.ring), false};
  XRegs<WT, MT> xr;
  switch (p.only_ph) {
    case PH_QKV:
      phase_qkv<WT, MT>(p, sm, l, st, plan_qkv<WT>(p, l), none);
      break;
    case PH_ATTN:
      phase_attn_dec<QK == 1 ? 4 : 16>(p, sm, l, st, plan_attn(p, ms, l, true), none);
      break;
    case PH_WO:
      phase_wo<WT, MT>(p, sm, l, st, plan_wo<WT>(p, l), none);
      break;
    case PH_RS:
      phase_rs<WT, MT>(p, sm, l, st, plan_rs<WT>(p, l), none, xr);
      break;
    case PH_RG: {
      load_x_norm<WT, MT>(xr, sm, layer_h1(p, l), p.d, reinterpret_cast<const WT*>(layer_tab(p)[l].moe_norm), p.M,
                          p.d, p.eps, wave, lane, plan_rs<WT>(p, l).lrb);
      rg_stage(p, sm, l);
      route_topk(p, sm, l);
      phase_rg<WT, MT>(p, sm, l, st, plan_rg<WT>(p, ms, l, true), none, xr, 0);
      break;
    }
    case PH_DOWN:
      route_topk(p, sm, l);
      if constexpr (MT == 1) phase_down<WT, MT>(p, sm, l, st, plan_down<WT>(p, ms, l), none);
      else phase_down_a<WT, MT>(p, sm, l, st, plan_down_a<WT>(p, ms, l), none);
      break;
    case PH_DOWNB: {
      route_topk(p, sm, l);
      const Plan P = plan_down_a<WT>(p, ms, l);
      const int c0 = P.lo2 * P.rpt, ncol = P.n1 * P.rpt;
      load_res(sm, layer_h1(p, l), p.S > 0 ? act_f(p, l, p.al.y_s) : nullptr, p.d, c0, ncol, p.M);
      __syncthreads();
      phase_down_b(p, sm, l, c0, ncol);
      break;
    }
    default:
      break;
  }
  wait_all();
  // a launch without tagged words moves the tag epoch on: a late block of
  // this launch may read either value, which no phase here depends on
  if (p.only_ph != PH_ATTN && blockIdx.x == 0 && threadIdx.x == 0) st_dev_u(p.sync + SyncLayout::kTag, ms->tag);
}

}  // namespace mk

// kernel of (weight dtype, token group, attention task kind) for a launch.
// The token group follows the row count: one row takes the single-row
// kernel, whose DOWN is one phase; more rows take the 8-row kernel, whose
// DOWN runs as two phases over the per-expert partials.  The host sizes the
// barriers, the partial buffer and the per-phase launches by that same rule,
// so an 8-row kernel never runs a single row.
constexpr int kKernelKinds = 6;
static int mk_pick(const mk::KParams& p, bool phased, const void** fn, int* idx) {
  using namespace mk;
  if (p.M < 1 || p.M > kMaxRows) return -2;
  if (p.attn && p.n_seq * p.G * p.q_groups * p.n_splits > p.vncu) return -2;
  if (p.n_groups < 1 || p.n_groups * p.vncu != p.n_cu || (p.n_groups > 1 && p.vncu != 8 << p.cpx_log2)) return -2;
  if (p.n_groups > 1 && (p.wide || p.M != kMaxRows || p.n_groups > kMaxGroups)) return -2;  // tasks: 8-row bf16 groups
  const int Q = p.attn ? p.q_per_task : 0;
  const bool one = p.M == 1;
  // instantiations: weight dtype x token group (1 or 8) x attention task
  // kind (1: at most 4 query vectors; 2: at most 16, several rows of a
  // sequence or many query heads per kv head)
  static const void* const persistent[kKernelKinds] = {
      (const void*)decode_step_kernel<float, 1, 1>,    (const void*)decode_step_kernel<float, 8, 1>,
      (const void*)decode_step_kernel<uint16_t, 1, 1>, (const void*)decode_step_kernel<uint16_t, 8, 1>,
      (const void*)decode_step_kernel<uint16_t, 1, 2>, (const void*)decode_step_kernel<uint16_t, 8, 2>};
  static const void* const per_phase[kKernelKinds] = {
      (const void*)phase_step_kernel<float, 1, 1>,    (const void*)phase_step_kernel<float, 8, 1>,
      (const void*)phase_step_kernel<uint16_t, 1, 1>, (const void*)phase_step_kernel<uint16_t, 8, 1>,
      (const void*)phase_step_kernel<uint16_t, 1, 2>, (const void*)phase_step_kernel<uint16_t, 8, 2>};
  int k;
  if (p.wide) {
    if (Q > 4) return -2;
    k = 0;
  } else if (Q <= 4) {
    k = 2;
  } else {
    if (Q > kMaxQTask) return -2;
    k = 4;
  }
  k += one ? 0 : 1;
  *fn = phased ? per_phase[k] : persistent[k];
  *idx = k + (phased ? kKernelKinds : 0);
  return 0;
}

extern "C" int mk_launch_kernel(const mk::KParams* pp, void* stream) {
  using namespace mk;
  KParams p = *pp;
  const size_t lds = (size_t)kLdsTotal;
  const void* fn = nullptr;
  int idx = 0;
  const int pk = mk_pick(p, p.only_ph >= 0, &fn, &idx);
  if (pk != 0) return pk;
  // The dynamic-LDS limit is a per-device attribute of each kernel: set it
  // once per (device, kernel); devices beyond the table set it every launch.
  // Concurrent first launches may both set it, which is harmless.
  constexpr int kAttrDevices = 16;
  static bool attr_done[kAttrDevices][2 * kKernelKinds] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  bool* done = (dev >= 0 && dev < kAttrDevices) ? &attr_done[dev][idx] : nullptr;
  if (!done || !*done) {
    // the kernel takes all of the CU's LDS dynamically: any static LDS (a
    // library routine that declares its own) would make the launch fail
    hipFuncAttributes fa;
    if (hipFuncGetAttributes(&fa, fn) != hipSuccess || fa.sharedSizeBytes != 0) return -3;
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess) return -1;
    if (done) *done = true;
  }
  // A plain launch.  Every workgroup takes the whole LDS of a CU, so the grid
  // (one per CU) places exactly one on each CU; the grid barriers need all of
  // them resident, which work on other streams can delay (the watchdog ends
  // a step that waits too long) but not prevent.  The cooperative launch API
  // makes the same placement and measured slower: batch 1 of 92 attention +
  // MoE layers 7.95 vs 7.85 ms, 16 MoE layers 0.553 vs 0.533 ms, batch 8
  // equal.
  void* args[] = {&p};
  hipError_t e = hipLaunchKernel(fn, dim3(p.n_cu), dim3(kThreads), args, (unsigned)lds, (hipStream_t)stream);
  return e == hipSuccess ? 0 : (int)e;
}
