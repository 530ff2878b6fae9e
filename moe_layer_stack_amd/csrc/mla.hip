// mla.hip -- multi-head latent attention (MLA) at decode over a latent KV
// cache (include/mk_mla.h): the split launch on the matrix cores and the
// combine launch, and their C ABI.
//
// Definition (absorbed form of the published MLA, DeepSeek-V2 report,
// section 2.1; the pages only name MLA, P4 paragraph on VMEM budgeting): row
// r, head h attends the cache rows 0 .. positions[r] of its sequence with
// scores scale * q . row and returns the softmax-weighted sum of the rows'
// first 512 (latent) columns.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>

#include "mk_mla.h"

namespace mla {

constexpr int kDc = 512;                         // latent columns (the values)
constexpr int kDr = 64;                          // rotary key columns
constexpr int kDk = kDc + kDr;                   // a cache row: the key
constexpr int kRowBytes = kDk * 2;               // 1152 bytes of bf16
constexpr int kTile = 32;                        // positions per tile: two halves of 16
constexpr int kRowU4 = kRowBytes / 16;           // 72 per row
// LDS row pitch: 1152 bytes is 288 dwords, which would put all 16 rows of a
// matrix-core read on the same banks; 16 bytes of padding spread them.
constexpr int kPitch = kRowBytes + 16;
constexpr int kChunks = kDk / 32;                // 18 key chunks of 32 columns
constexpr int kPartStride = 4 + kDc;             // floats per query of a split partial: m, l, -, -, acc[512]
constexpr int kTileU4 = kTile * kRowBytes / 16;  // 16-byte pieces of a tile (2304)

struct Params {
  const float* q;            // [M][H][kDk]
  const uint16_t* cache;     // [n_seq][cap][kDk]
  const int32_t* positions;  // [M]
  float* out;                // [M][H][kDc]
  float* part;               // [n_seq_step][QG][S][QW][kPartStride]
  unsigned* err;             // set when a position is outside the cache
  int M, H, rps, cap, QG, S;
  int QW;                    // query vectors per workgroup (16 or 64)
  float qscale;              // scale * log2(e): scores in base-2 exponent units
};

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ s16x4_t lds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t*)(const_cast<char*>(p)));
}
__device__ __forceinline__ short bf16_bits(__bf16 h) { return __builtin_bit_cast(short, h); }

// Workgroup b's (sequence, query group, split).  The QG workgroups of one
// (sequence, split) pair read the same cache tiles, and workgroups are dealt
// to the 8 XCDs round-robin by index, so in each block of 8 pairs the QG
// workgroups of a pair take indices 8 apart: one XCD, whose L2 then serves
// each tile to all of them.  The last (pairs % 8) pairs take consecutive
// indices.  Any such numbering computes the same results.
__device__ __forceinline__ void wg_coords(const Params& p, int b, int& seq, int& qg, int& s) {
  const int QG = p.QG, U = (int)gridDim.x / QG;  // (sequence, split) pairs
  const int head = (U & ~7) * QG;                  // workgroups of the full blocks
  int u;
  if (b < head) {
    const int blk = b / (8 * QG), r = b % (8 * QG);
    qg = r >> 3;
    u = blk * 8 + (r & 7);
  } else {
    const int t = b - head, rest = U & 7;
    qg = t / rest;
    u = (U & ~7) + t % rest;
  }
  seq = u / p.S;
  s = u % p.S;
}

// Few query vectors per sequence (decode: H of one row): workgroups of 16
// vectors, two per CU, the 576 key columns split over the 4 waves.
namespace q16 {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kQ = 16;                // query vectors per workgroup: one matrix-core operand
constexpr int kMaxChunks = 5;         // waves take 5, 5, 4 and 4 chunks
constexpr int kVals = kDc / kWaves;   // latent columns per wave (128)
constexpr int kLoads = (kTileU4 + kThreads - 1) / kThreads;  // 16-byte loads per thread per tile (9)
static_assert(kChunks == 2 * kMaxChunks + 2 * (kMaxChunks - 1), "chunk split");

// A tile of 32 cache rows in flight through registers: piece u = thread +
// 256k of the tile (row u / 72, 16 bytes at u % 72); 2304 pieces, 9 per
// thread exactly.  A thread's pieces sit at the same place in every tile, so
// their rows and offsets are worked out once (TileMap) and a tile costs one
// row clamp and one 32-bit offset per piece.  Rows past the capacity re-read
// the last row (their scores are masked).  (A native vector type: an array
// of HIP's uint4 structs would be kept in scratch memory.)
static_assert(kTileU4 == kLoads * kThreads, "every thread moves the same number of pieces");
struct Prefetch {
  u32x4_t v[kLoads];
};
struct TileMap {
  int row[kLoads];  // row of the piece within the tile
  int off[kLoads];  // byte offset of the piece within its row
};
__device__ __forceinline__ TileMap tile_map() {
  TileMap m;
#pragma unroll
  for (int k = 0; k < kLoads; ++k) {
    const int u = (int)threadIdx.x + k * kThreads;
    m.row[k] = u / kRowU4;
    m.off[k] = (u % kRowU4) * 16;
  }
  return m;
}
// rows: the sequence's cache (its first row); offsets stay below 2^32 for
// capacities below 3.7 million positions (the host checks)
__device__ __forceinline__ void load_tile(Prefetch& pf, const char* rows, const TileMap& m, int t, int cap) {
#pragma unroll
  for (int k = 0; k < kLoads; ++k) {
    const unsigned r = (unsigned)min(t * kTile + m.row[k], cap - 1);
    pf.v[k] = *reinterpret_cast<const u32x4_t*>(rows + (r * (unsigned)kRowBytes + (unsigned)m.off[k]));
  }
}
__device__ __forceinline__ void store_tile(const Prefetch& pf, char* tile, const TileMap& m) {
#pragma unroll
  for (int k = 0; k < kLoads; ++k)
    *reinterpret_cast<u32x4_t*>(tile + m.row[k] * kPitch + m.off[k]) = pf.v[k];
}

// Workgroup (seq, qg, s): the 16 query vectors qg*16 .. qg*16+15 of sequence
// seq (query i of a sequence is row i / H, head i % H; H is a multiple of
// 16, so the 16 share one row and one position) against split s of the
// row's positions, tiles of 32 positions.  With one split the workgroup
// writes the outputs itself (no combine launch).
__global__ void __launch_bounds__(kThreads, 2) split_kernel(Params p) {
  __shared__ __attribute__((aligned(16))) char tile[kTile * kPitch];
  __shared__ __attribute__((aligned(16))) f32x4_t exch[2][kWaves][64];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  int seq, qg, s;
  wg_coords(p, (int)blockIdx.x, seq, qg, s);
  const int row = seq * p.rps + (qg * kQ) / p.H;
  const int pos = p.positions[row];
  const bool ok = pos >= 0 && pos < p.cap;
  if (!ok && threadIdx.x == 0 && s == 0) __hip_atomic_fetch_or(p.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int npos = ok ? pos + 1 : 0;
  const int ntile = (npos + kTile - 1) / kTile;
  const int t_lo = (int)(((long long)s * ntile) / p.S), t_hi = (int)(((long long)(s + 1) * ntile) / p.S);
  const char* rows = reinterpret_cast<const char*>(p.cache + (size_t)seq * p.cap * kDk);
  const int qq = lane & 15, lg = lane >> 4;
  // This wave's key chunks and its query operand for them, lane l: query
  // l & 15, columns 32c + 8(l >> 4) .. +7, bf16 high and low parts.
  const int c0 = wave < 2 ? kMaxChunks * wave : 2 * kMaxChunks + (kMaxChunks - 1) * (wave - 2);
  const int nc = wave < 2 ? kMaxChunks : kMaxChunks - 1;
  bf16x8_t qh[kMaxChunks], ql[kMaxChunks];
  {
    const float* src = p.q + ((size_t)row * p.H + (qg * kQ) % p.H + qq) * kDk + lg * 8;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
      const int cc = c0 + (c < nc ? c : 0);
      const float4 a0 = *reinterpret_cast<const float4*>(src + cc * 32);
      const float4 a1 = *reinterpret_cast<const float4*>(src + cc * 32 + 4);
      const float x[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float v = x[j] * p.qscale;
        const __bf16 hi = (__bf16)v;
        qh[c][j] = hi;
        ql[c][j] = (__bf16)(v - (float)hi);
      }
    }
  }
  f32x4_t acc[kVals / 16];
#pragma unroll
  for (int nb = 0; nb < kVals / 16; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_l = -INFINITY, lsum = 0.f;
  Prefetch pf;
  const TileMap tm = tile_map();
  if (t_lo < t_hi) {
    load_tile(pf, rows, tm, t_lo, p.cap);
    store_tile(pf, tile, tm);
  }
  __syncthreads();
  for (int t = t_lo; t < t_hi; ++t) {
    // the next tile (at the last one, this one again) lands while this one is used
    load_tile(pf, rows, tm, min(t + 1, t_hi - 1), p.cap);
    // partial scores over this wave's chunks for both halves of the tile:
    // D lane l = positions 4(l>>4)+i of the half, query l&15
    f32x4_t sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
    {
      const char* kr = tile + qq * kPitch + lg * 16;
#pragma unroll
      for (int c = 0; c < kMaxChunks; ++c) {
        if (c < nc) {
          const bf16x8_t ka = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(kr + (c0 + c) * 64));
          const bf16x8_t kb =
              __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(kr + 16 * kPitch + (c0 + c) * 64));
          sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qh[c], sa, 0, 0, 0);
          sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qh[c], sb, 0, 0, 0);
          sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, ql[c], sa, 0, 0, 0);
          sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, ql[c], sb, 0, 0, 0);
        }
      }
    }
    exch[0][wave][lane] = sa;
    exch[1][wave][lane] = sb;
    __syncthreads();
    // full scores: the four waves' partials in a fixed order (every wave
    // then holds the same values); sv[0..3] first half, sv[4..7] second
    float sv[8];
    {
      f32x4_t ta = exch[0][0][lane], tb = exch[1][0][lane];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) {
        ta += exch[0][w][lane];
        tb += exch[1][w][lane];
      }
      bool up = false;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ja = t * kTile + 4 * lg + i;
        sv[i] = ja < npos ? ta[i] : -INFINITY;
        sv[4 + i] = ja + 16 < npos ? tb[i] : -INFINITY;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) up |= sv[i] > m_l + 8.f;
      // online softmax in base 2 with a reference maximum that is raised
      // only when a score exceeds it by more than 8 (2^8 stays exact enough
      // in fp32); wave-uniform
      if (__builtin_amdgcn_ballot_w64(up) != 0) {
        float mx = sv[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sv[i]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const bool raise = mx > m_l + 8.f;
        const float corr = !raise ? 1.f : (m_l == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_l - mx);
        lsum *= corr;
#pragma unroll
        for (int nb = 0; nb < kVals / 16; ++nb) acc[nb] *= corr;
        m_l = raise ? mx : m_l;
      }
    }
    // The weights as the B operand of a 32-deep product, lane l: query l&15,
    // k-slots 8(l>>4) .. +7 = positions 4(l>>4) .. +3 of the first half and
    // of the second half (the score layouts as they are); the V^T operand
    // below uses the same k-slot order.
    s16x8_t ph, pl;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float pv = sv[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[i] - m_l);
      lsum += pv;
      const __bf16 h = (__bf16)pv;
      ph[i] = bf16_bits(h);
      pl[i] = bf16_bits((__bf16)(pv - (float)h));
    }
    // this wave's 128 latent columns: V^T by transpose loads, lane 16g + 4j
    // + c reads position 4g + j of each half, columns 128w + 16nb + 4c .. +3
    {
      const char* vr = tile + (4 * lg + ((lane >> 2) & 3)) * kPitch + wave * kVals * 2 + (lane & 3) * 8;
      const bf16x8_t bh = __builtin_bit_cast(bf16x8_t, ph), bl = __builtin_bit_cast(bf16x8_t, pl);
#pragma unroll
      for (int nb = 0; nb < kVals / 16; ++nb) {
        const s16x4_t va = lds_read_tr16(vr + nb * 32);
        const s16x4_t vb = lds_read_tr16(vr + 16 * kPitch + nb * 32);
        const bf16x8_t v8 = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v8, bh, acc[nb], 0, 0, 0);
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v8, bl, acc[nb], 0, 0, 0);
      }
    }
    __syncthreads();  // every wave is done with the tile and the exchange slots
    store_tile(pf, tile, tm);
    __syncthreads();
  }
  float lw = lsum;
  lw += __shfl_xor(lw, 16);
  lw += __shfl_xor(lw, 32);
  if (p.S == 1) {  // the whole range: the outputs themselves (zero for a rejected row)
    const float inv = lw > 0.f ? 1.f / lw : 0.f;
    float* o = p.out + ((size_t)row * p.H + (qg * kQ) % p.H + qq) * kDc + wave * kVals + 4 * lg;
#pragma unroll
    for (int nb = 0; nb < kVals / 16; ++nb)
      *reinterpret_cast<float4*>(o + nb * 16) =
          make_float4(acc[nb][0] * inv, acc[nb][1] * inv, acc[nb][2] * inv, acc[nb][3] * inv);
    return;
  }
  // the split's partial: m (natural units), l, and the sums, query-major
  constexpr float kLn2 = 0.6931471805599453f;
  float* dst = p.part + ((size_t)((seq * p.QG + qg) * p.S + s) * kQ + qq) * kPartStride;
#pragma unroll
  for (int nb = 0; nb < kVals / 16; ++nb)
    *reinterpret_cast<float4*>(dst + 4 + wave * kVals + nb * 16 + 4 * lg) =
        make_float4(acc[nb][0], acc[nb][1], acc[nb][2], acc[nb][3]);
  if (wave == 0 && lg == 0) {
    dst[0] = m_l == -INFINITY ? -INFINITY : m_l * kLn2;
    dst[1] = lw;
  }
}

}  // namespace q16

// Many query vectors per sequence (verify blocks: rows_per_seq x H): every
// tile read once for 64 vectors.
namespace q64 {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;  // 8: two per SIMD
constexpr int kQ = 16;                 // query vectors per wave pair: one matrix-core operand
constexpr int kQW = kWaves / 2 * kQ;   // query vectors per workgroup (64)
constexpr int kHalfChunks = kChunks / 2;
constexpr int kNB = kDc / 16;          // 32 blocks of 16 latent columns
constexpr int kHalfNB = kNB / 2;
constexpr int kLoads = (kTileU4 + kThreads - 1) / kThreads;  // 16-byte loads per thread per tile (5, the last by half the threads)
constexpr int kTileLds = kTile * kPitch;                     // one tile in LDS (37376 bytes)
constexpr int kExchLds = kWaves * 64 * 8 * 4;                // partial scores: 8 floats per lane and wave
constexpr int kLdsBytes = 2 * kTileLds + kExchLds;

// A tile of 32 cache rows in flight through registers: piece u = thread +
// 512k of the tile (row u / 72, 16 bytes at u % 72); 2304 pieces: 4 per
// thread and a fifth for the first 256 threads, which the others repeat
// (the last piece: same address, same bytes), so that every thread issues
// the same loads and the compiler's wait counts stay exact.  A thread's
// pieces sit at the same place in every tile, so their rows and offsets are
// worked out once (TileMap) and a tile costs one row clamp and one 32-bit
// offset per piece.  Rows past the capacity re-read the last row (their
// scores are masked).  (A native vector type: an array of HIP's uint4
// structs would be kept in scratch memory.)
static_assert(kTileU4 == (kLoads - 1) * kThreads + kThreads / 2, "pieces per thread");
struct Prefetch {
  u32x4_t v[kLoads];
};
struct TileMap {
  int row[kLoads];  // row of the piece within the tile
  int off[kLoads];  // byte offset of the piece within its row
};
__device__ __forceinline__ TileMap tile_map() {
  TileMap m;
#pragma unroll
  for (int k = 0; k < kLoads; ++k) {
    const int u = min((int)threadIdx.x + k * kThreads, kTileU4 - 1);
    m.row[k] = u / kRowU4;
    m.off[k] = (u % kRowU4) * 16;
  }
  return m;
}
// rows: the sequence's cache (its first row); offsets stay below 2^32 for
// capacities below 3.7 million positions (the host checks)
__device__ __forceinline__ void load_tile(Prefetch& pf, const char* rows, const TileMap& m, int t, int cap) {
#pragma unroll
  for (int k = 0; k < kLoads; ++k) {
    const unsigned r = (unsigned)min(t * kTile + m.row[k], cap - 1);
    pf.v[k] = *reinterpret_cast<const u32x4_t*>(rows + (r * (unsigned)kRowBytes + (unsigned)m.off[k]));
  }
}
__device__ __forceinline__ void store_tile(const Prefetch& pf, char* tile, const TileMap& m) {
#pragma unroll
  for (int k = 0; k < kLoads; ++k)
    *reinterpret_cast<u32x4_t*>(tile + m.row[k] * kPitch + m.off[k]) = pf.v[k];
}

// Workgroup (seq, qg, s): the 64 query vectors qg*64 .. qg*64+63 of sequence
// seq (query i of a sequence is row i / H, head i % H) against split s of the
// positions its rows attend, tiles of 32 positions: every tile is read from
// memory once for the 64 vectors.  Waves 2j and 2j+1 take the 16 vectors
// qg*64 + 16j .. +15 (H is a multiple of 16, so they share one row and one
// position): each forms the scores over half of the 576 key columns, the two
// halves are summed through LDS in a fixed order (both waves then hold the
// same scores and the same softmax state), and each wave accumulates half of
// the 512 latent columns.  The next two tiles are in flight through
// registers while one is used from one of two LDS buffers.  With one split
// the workgroup writes the outputs itself (no combine launch).
__global__ void __launch_bounds__(kThreads, 1) split_kernel(Params p) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  f32x4_t* exch = reinterpret_cast<f32x4_t*>(lds + 2 * kTileLds);  // [wave][2][64]
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int pr = wave >> 1, hf = wave & 1;
  int seq, qg, s;
  wg_coords(p, (int)blockIdx.x, seq, qg, s);
  const int nqs = p.H * p.rps;  // query vectors of a sequence
  // positions attended by each pair's row; the workgroup's tiles cover the longest
  int npos_w = 0, npos_max = 0;
#pragma unroll
  for (int j = 0; j < kWaves / 2; ++j) {
    const int qb = qg * kQW + j * kQ;
    int np = 0;
    if (qb < nqs) {
      const int pos = p.positions[seq * p.rps + qb / p.H];
      const bool ok = pos >= 0 && pos < p.cap;
      if (!ok && threadIdx.x == 0 && s == 0)
        __hip_atomic_fetch_or(p.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      np = ok ? pos + 1 : 0;
    }
    npos_w = j == pr ? np : npos_w;
    npos_max = max(npos_max, np);
  }
  const int ntile = (npos_max + kTile - 1) / kTile;
  const int t_lo = (int)(((long long)s * ntile) / p.S), t_hi = (int)(((long long)(s + 1) * ntile) / p.S);
  const char* rows = reinterpret_cast<const char*>(p.cache + (size_t)seq * p.cap * kDk);
  const int qq = lane & 15, lg = lane >> 4;
  const int qb = qg * kQW + pr * kQ;
  const bool wact = qb < nqs;
  const int row = seq * p.rps + (wact ? qb : 0) / p.H, head0 = (wact ? qb : 0) % p.H;
  // query operand for this wave's key half, lane l: query l & 15, columns
  // 32c + 8(l >> 4) .. +7 of chunk c, bf16 high and low parts
  const int c0 = hf * kHalfChunks;
  bf16x8_t qh[kHalfChunks], ql[kHalfChunks];
  {
    const float* src = p.q + ((size_t)row * p.H + head0 + qq) * kDk + lg * 8;
#pragma unroll
    for (int c = 0; c < kHalfChunks; ++c) {
      const float4 a0 = *reinterpret_cast<const float4*>(src + (c0 + c) * 32);
      const float4 a1 = *reinterpret_cast<const float4*>(src + (c0 + c) * 32 + 4);
      const float x[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float v = x[j] * p.qscale;
        const __bf16 hi = (__bf16)v;
        qh[c][j] = hi;
        ql[c][j] = (__bf16)(v - (float)hi);
      }
    }
  }
  f32x4_t acc[kHalfNB];
#pragma unroll
  for (int nb = 0; nb < kHalfNB; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_l = -INFINITY, lsum = 0.f;
  const TileMap tm = tile_map();
  // two tiles in flight through registers (pa, pb) while one is used from
  // LDS.  Every step issues the same loads (tiles past the split's last one
  // re-read it), so the compiler's wait counts see the two in flight.
  if (t_lo < t_hi) {  // workgroup-uniform; a split without positions leaves an empty partial
    const int t_last = t_hi - 1;
    Prefetch pa, pb;
    load_tile(pa, rows, tm, t_lo, p.cap);
    store_tile(pa, lds, tm);
    load_tile(pa, rows, tm, min(t_lo + 1, t_last), p.cap);
    load_tile(pb, rows, tm, min(t_lo + 2, t_last), p.cap);
    __syncthreads();
    // tile t from LDS; then tile t + 1 from pf into the other LDS buffer, and
    // tile t + 3 into pf
    auto run_tile = [&](int t, Prefetch& pf) __attribute__((always_inline)) {
      const char* tile = lds + ((t - t_lo) & 1) * kTileLds;
      // wave-uniform: a tile of the split holding positions this pair's row attends
      const bool work = t < t_hi && npos_w > t * kTile;
      // partial scores over this wave's key half for both halves of the tile:
      // D lane l = positions 4(l>>4)+i of the half, query l&15
      if (work) {
        f32x4_t sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
        const char* kr = tile + qq * kPitch + lg * 16 + c0 * 64;
#pragma unroll
        for (int c = 0; c < kHalfChunks; ++c) {
          const bf16x8_t ka = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(kr + c * 64));
          const bf16x8_t kb = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(kr + 16 * kPitch + c * 64));
          sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qh[c], sa, 0, 0, 0);
          sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qh[c], sb, 0, 0, 0);
          sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, ql[c], sa, 0, 0, 0);
          sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, ql[c], sb, 0, 0, 0);
        }
        exch[(wave * 2 + 0) * 64 + lane] = sa;
        exch[(wave * 2 + 1) * 64 + lane] = sb;
      }
      __syncthreads();
      if (work) {
        // full scores: the pair's two halves, lower key columns first (both
        // waves of the pair then hold the same values); sv[0..3] first half of
        // the tile, sv[4..7] second
        const int w0 = pr * 2;
        const f32x4_t ta = exch[(w0 * 2 + 0) * 64 + lane] + exch[((w0 + 1) * 2 + 0) * 64 + lane];
        const f32x4_t tb = exch[(w0 * 2 + 1) * 64 + lane] + exch[((w0 + 1) * 2 + 1) * 64 + lane];
        float sv[8];
        bool up = false;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ja = t * kTile + 4 * lg + i;
          sv[i] = ja < npos_w ? ta[i] : -INFINITY;
          sv[4 + i] = ja + 16 < npos_w ? tb[i] : -INFINITY;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) up |= sv[i] > m_l + 8.f;
        // online softmax in base 2 with a reference maximum that is raised
        // only when a score exceeds it by more than 8 (2^8 stays exact enough
        // in fp32); wave-uniform
        if (__builtin_amdgcn_ballot_w64(up) != 0) {
          float mx = sv[0];
#pragma unroll
          for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sv[i]);
          mx = fmaxf(mx, __shfl_xor(mx, 16));
          mx = fmaxf(mx, __shfl_xor(mx, 32));
          const bool raise = mx > m_l + 8.f;
          const float corr = !raise ? 1.f : (m_l == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_l - mx);
          lsum *= corr;
#pragma unroll
          for (int nb = 0; nb < kHalfNB; ++nb) acc[nb] *= corr;
          m_l = raise ? mx : m_l;
        }
        // The weights as the B operand of a 32-deep product, lane l: query
        // l&15, k-slots 8(l>>4) .. +7 = positions 4(l>>4) .. +3 of the first
        // half and of the second half (the score layouts as they are); the V^T
        // operand below uses the same k-slot order.
        s16x8_t ph, pl;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float pv = sv[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[i] - m_l);
          lsum += pv;
          const __bf16 h = (__bf16)pv;
          ph[i] = bf16_bits(h);
          pl[i] = bf16_bits((__bf16)(pv - (float)h));
        }
        // this wave's 256 latent columns: V^T by transpose loads, lane 16g +
        // 4j + c reads position 4g + j of each half, columns 256hf + 16nb + 4c .. +3
        const char* vr = tile + (4 * lg + ((lane >> 2) & 3)) * kPitch + hf * (kDc / 2) * 2 + (lane & 3) * 8;
        const bf16x8_t bh = __builtin_bit_cast(bf16x8_t, ph), bl = __builtin_bit_cast(bf16x8_t, pl);
#pragma unroll
        for (int nb = 0; nb < kHalfNB; ++nb) {
          const s16x4_t va = lds_read_tr16(vr + nb * 32);
          const s16x4_t vb = lds_read_tr16(vr + 16 * kPitch + nb * 32);
          const bf16x8_t v8 = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7));
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v8, bh, acc[nb], 0, 0, 0);
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v8, bl, acc[nb], 0, 0, 0);
        }
      }
      // the other buffer was last read in the previous step, before its barrier
      store_tile(pf, lds + ((t + 1 - t_lo) & 1) * kTileLds, tm);
      load_tile(pf, rows, tm, min(t + 3, t_last), p.cap);
      __syncthreads();
    };
    for (int t = t_lo; t < t_hi; t += 2) {
      run_tile(t, pa);
      run_tile(t + 1, pb);
    }
  }
  if (!wact) return;
  float lw = lsum;
  lw += __shfl_xor(lw, 16);
  lw += __shfl_xor(lw, 32);
  const int col0 = hf * (kDc / 2) + 4 * lg;  // this lane's first latent column
  if (p.S == 1) {  // the whole range: the outputs themselves (zero for a rejected row)
    const float inv = lw > 0.f ? 1.f / lw : 0.f;
    float* o = p.out + ((size_t)row * p.H + head0 + qq) * kDc + col0;
#pragma unroll
    for (int nb = 0; nb < kHalfNB; ++nb)
      *reinterpret_cast<float4*>(o + nb * 16) =
          make_float4(acc[nb][0] * inv, acc[nb][1] * inv, acc[nb][2] * inv, acc[nb][3] * inv);
    return;
  }
  // the split's partial: m (natural units), l, and the sums, query-major
  constexpr float kLn2 = 0.6931471805599453f;
  float* dst = p.part + ((size_t)((seq * p.QG + qg) * p.S + s) * kQW + pr * kQ + qq) * kPartStride;
#pragma unroll
  for (int nb = 0; nb < kHalfNB; ++nb)
    *reinterpret_cast<float4*>(dst + 4 + col0 + nb * 16) = make_float4(acc[nb][0], acc[nb][1], acc[nb][2], acc[nb][3]);
  if (lg == 0 && hf == 0) {
    dst[0] = m_l == -INFINITY ? -INFINITY : m_l * kLn2;
    dst[1] = lw;
  }
}

}  // namespace q64

// out[r][h][:] from the S split partials of its query: weights e^(m_s - max)
// over the splits.  Thread t takes 4 output columns (t % 128) and every
// fourth split (from t / 128); the four split groups are summed in order
// through LDS.  A row whose position was rejected gets 0.
constexpr int kCombineThreads = 512;
__global__ void __launch_bounds__(kCombineThreads) combine_kernel(Params p) {
  __shared__ float red[4][kDc + 4];
  __shared__ float wmax[kCombineThreads / 64];
  const int r = blockIdx.x / p.H, h = blockIdx.x % p.H;
  const int seq = r / p.rps, qi = (r % p.rps) * p.H + h;
  const int qg = qi / p.QW, q = qi % p.QW;
  const float* base = p.part + ((size_t)((seq * p.QG + qg) * p.S) * p.QW + q) * kPartStride;
  const size_t sstride = (size_t)p.QW * kPartStride;
  const int t = threadIdx.x, o4 = t & 127, g = t >> 7;
  float M = -INFINITY;
  for (int s = t; s < p.S; s += kCombineThreads) M = fmaxf(M, base[s * sstride]);
  for (int sh = 1; sh < 64; sh <<= 1) M = fmaxf(M, __shfl_xor(M, sh));
  if ((t & 63) == 0) wmax[t >> 6] = M;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kCombineThreads / 64; ++w) M = fmaxf(M, wmax[w]);
  float L = 0.f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
  for (int s = g; s < p.S; s += 4) {
    const float* b = base + s * sstride;
    const float w = b[0] == -INFINITY ? 0.f : __expf(b[0] - M);
    L = fmaf(w, b[1], L);
    const float4 a = *reinterpret_cast<const float4*>(b + 4 + 4 * o4);
    o.x = fmaf(w, a.x, o.x); o.y = fmaf(w, a.y, o.y); o.z = fmaf(w, a.z, o.z); o.w = fmaf(w, a.w, o.w);
  }
  *reinterpret_cast<float4*>(&red[g][4 * o4]) = o;
  if (o4 == 0) red[g][kDc] = L;
  __syncthreads();
  if (g == 0) {
    float4 sum = *reinterpret_cast<const float4*>(&red[0][4 * o4]);
    float ls = red[0][kDc];
#pragma unroll
    for (int k = 1; k < 4; ++k) {
      const float4 a = *reinterpret_cast<const float4*>(&red[k][4 * o4]);
      sum.x += a.x; sum.y += a.y; sum.z += a.z; sum.w += a.w;
      ls += red[k][kDc];
    }
    const float inv = ls > 0.f ? 1.f / ls : 0.f;
    *reinterpret_cast<float4*>(p.out + ((size_t)r * p.H + h) * kDc + 4 * o4) =
        make_float4(sum.x * inv, sum.y * inv, sum.z * inv, sum.w * inv);
  }
}

}  // namespace mla

struct mk_mla_handle {
  mk_mla_config cfg;
  int device;
  int QG, S, n_seq_step;
  int QW;  // query vectors per split workgroup: 16 (q16 kernel) or 64 (q64 kernel)
  float* part;
  unsigned* err;
  size_t part_bytes;
};

namespace {

thread_local std::string g_mla_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_mla_error = buf;
  return status;
}

}  // namespace

extern "C" {

const char* mk_mla_last_error(void) { return g_mla_error.c_str(); }

int mk_mla_create(const mk_mla_config* cfg, mk_mla_handle** out) {
  using namespace mla;
  if (!cfg || !out) return fail(MK_ERR_INVALID_ARG, "NULL argument");
  const mk_mla_config c = *cfg;
  if (c.rows < 1 || c.rows_per_seq < 1 || c.rows % c.rows_per_seq != 0 || c.n_seq < c.rows / c.rows_per_seq ||
      c.capacity < 1 || !(c.scale > 0.f) || !std::isfinite(c.scale) || c.n_heads < 1)
    return fail(MK_ERR_INVALID_ARG, "inconsistent config (rows %d, rows_per_seq %d, n_seq %d, capacity %d, scale %g)",
                c.rows, c.rows_per_seq, c.n_seq, c.capacity, (double)c.scale);
  if (c.latent_dim != kDc || c.rope_dim != kDr)
    return fail(MK_ERR_UNSUPPORTED, "latent_dim %d / rope_dim %d: the kernel is built for %d / %d", c.latent_dim,
                c.rope_dim, kDc, kDr);
  if (c.n_heads % 16 != 0 || c.n_heads > 128 || c.rows > 64 || c.capacity > (1 << 21))
    return fail(MK_ERR_UNSUPPORTED, "n_heads %d (16, 32, 64 or 128), rows %d (<= 64) or capacity %d (<= 2^21) out of range",
                c.n_heads, c.rows, c.capacity);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(MK_ERR_DEVICE, "no HIP device");
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return fail(MK_ERR_DEVICE, "hipGetDeviceProperties failed");
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(MK_ERR_DEVICE, "device %d is %s, not gfx950", dev, prop.gcnArchName);
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(q64::split_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                          q64::kLdsBytes) != hipSuccess)
    return fail(MK_ERR_HIP, "setting the split kernel's LDS size failed");
  mk_mla_handle* h = new (std::nothrow) mk_mla_handle();
  if (!h) return fail(MK_ERR_HIP, "out of host memory");
  h->cfg = c;
  h->device = dev;
  h->n_seq_step = c.rows / c.rows_per_seq;
  // Query vectors per workgroup: 64 (every tile read once for them) when a
  // sequence has at least 128 (verify blocks), else 16 with two workgroups
  // per CU, which spreads a decode row's few vectors over more CUs.
  const int nqs = c.n_heads * c.rows_per_seq;
  h->QW = nqs >= 128 ? q64::kQW : q16::kQ;
  h->QG = (nqs + h->QW - 1) / h->QW;
  const int base = h->n_seq_step * h->QG;
  const int ncu = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1;
  if (h->QW == q16::kQ) {
    // about two workgroups per CU (two tiles in flight per CU), each with at
    // least 4 tiles of the full capacity (a split's partial, 33 KB, should
    // stay well below the 147 KB of cache rows it reads)
    const int want = (2 * ncu + base / 2) / base;
    const int most = (c.capacity + 4 * kTile - 1) / (4 * kTile);
    h->S = want < 1 ? 1 : (want > most ? most : want);
  } else {
    // the S that minimises a cost model of the call at full capacity, in
    // microseconds: the split's tiles (about 3 us each for 64 vectors) and
    // its start-up (the 147 KB of queries and the first tiles, about 4 us),
    // times the rounds of workgroups over the CUs, plus writing and
    // combining the partials (64 x 2 KB per split, about 5 TB/s each way);
    // at least two tiles per split
    const int ntile = (c.capacity + kTile - 1) / kTile;
    const int most = ntile / 2 > 1 ? ntile / 2 : 1;
    double best = 1e30;
    h->S = 1;
    for (int S = 1; S <= most && S <= 4096; ++S) {
      const double rounds = (double)((base * S + ncu - 1) / ncu);
      const double t = (3.0 * ((ntile + S - 1) / S) + 4.0) * rounds + (S > 1 ? 0.053 * base * S : 0.0);
      if (t < best) {
        best = t;
        h->S = S;
      }
    }
  }
  h->part_bytes = (size_t)base * h->S * h->QW * kPartStride * sizeof(float);
  if (hipMalloc(&h->part, h->part_bytes) != hipSuccess) {
    delete h;
    return fail(MK_ERR_HIP, "hipMalloc of %zu bytes failed", h->part_bytes);
  }
  if (hipMalloc(&h->err, 256) != hipSuccess || hipMemset(h->err, 0, 256) != hipSuccess) {
    (void)hipFree(h->part);
    delete h;
    return fail(MK_ERR_HIP, "hipMalloc of the error word failed");
  }
  *out = h;
  return MK_OK;
}

int mk_mla_attention(mk_mla_handle* h, const float* q, const uint16_t* cache, const int32_t* positions, float* out,
                     void* stream) {
  using namespace mla;
  if (!h || !q || !cache || !positions || !out) return fail(MK_ERR_INVALID_ARG, "NULL argument");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != h->device)
    return fail(MK_ERR_INVALID_ARG, "current device differs from the handle's device");
  const mk_mla_config& c = h->cfg;
  Params p{};
  p.q = q;
  p.cache = cache;
  p.positions = positions;
  p.out = out;
  p.part = h->part;
  p.err = h->err;
  p.M = c.rows;
  p.H = c.n_heads;
  p.rps = c.rows_per_seq;
  p.cap = c.capacity;
  p.QG = h->QG;
  p.S = h->S;
  p.QW = h->QW;
  p.qscale = c.scale * 1.4426950408889634f;
  const hipStream_t st = (hipStream_t)stream;
  const dim3 grid(h->n_seq_step * h->QG * h->S);
  if (h->QW == q64::kQW)
    hipLaunchKernelGGL(q64::split_kernel, grid, dim3(q64::kThreads), q64::kLdsBytes, st, p);
  else
    hipLaunchKernelGGL(q16::split_kernel, grid, dim3(q16::kThreads), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MK_ERR_HIP, "split launch failed: %s", hipGetErrorString(e));
  if (h->S == 1) return MK_OK;  // the split launch wrote the outputs
  hipLaunchKernelGGL(combine_kernel, dim3(c.rows * c.n_heads), dim3(kCombineThreads), 0, st, p);
  e = hipGetLastError();
  if (e != hipSuccess) return fail(MK_ERR_HIP, "combine launch failed: %s", hipGetErrorString(e));
  return MK_OK;
}

int mk_mla_sync(mk_mla_handle* h, void* stream) {
  if (!h) return fail(MK_ERR_INVALID_ARG, "NULL handle");
  const hipStream_t st = (hipStream_t)stream;
  unsigned flag = 0;
  if (hipStreamSynchronize(st) != hipSuccess ||
      hipMemcpy(&flag, h->err, sizeof flag, hipMemcpyDeviceToHost) != hipSuccess)
    return fail(MK_ERR_HIP, "synchronising the stream failed");
  if (flag) {
    if (hipMemset(h->err, 0, sizeof flag) != hipSuccess) return fail(MK_ERR_HIP, "clearing the error word failed");
    return fail(MK_ERR_INVALID_ARG, "a row's position was outside [0, capacity %d)", h->cfg.capacity);
  }
  return MK_OK;
}

int mk_mla_get_info(const mk_mla_handle* h, mk_mla_info* info) {
  if (!h || !info) return fail(MK_ERR_INVALID_ARG, "NULL argument");
  info->splits = h->S;
  info->workgroups = h->n_seq_step * h->QG * h->S;
  info->workspace_bytes = (int64_t)(h->part_bytes + 256);
  return MK_OK;
}

int mk_mla_destroy(mk_mla_handle* h) {
  if (!h) return MK_OK;
  (void)hipFree(h->part);
  (void)hipFree(h->err);
  delete h;
  return MK_OK;
}

}  // extern "C"
