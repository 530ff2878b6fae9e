// mk_lanes.h -- cross-lane sums within one wave64 on gfx950 (VALU only:
// DPP and the permlane swaps, no LDS round trip).
#pragma once
#include <hip/hip_runtime.h>

namespace mk {

// ---- cross-lane reductions on VALU (no LDS round trip)
// Lane pairings that flip exactly one lane bit and keep all others:
//   bit 0, 1: DPP quad_perm [1,0,3,2] and [2,3,0,1]
//   bit 4:    v_permlane16_swap (rows r <-> r^1 at the same position)
//   bit 5:    v_permlane32_swap (lanes l <-> l^32)
// Bits 2 and 3 are summed with row rotations by 4 and 8 (the orbit of a lane
// under them is the four lanes that differ only in bits 2 and 3).
constexpr int kDppXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppRor4 = 0x124;  // row_ror:4
constexpr int kDppRor8 = 0x128;  // row_ror:8
constexpr int kDppRor12 = 0x12C; // row_ror:12 (a rotation by 4 the other way)
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// a holds the lower-half value, b the upper-half value of each lane; the
// result is the sum over the lane pair of the half this lane keeps (the
// lower half in the lane with the bit clear, the upper half in the other).
__device__ __forceinline__ float swap16_sum(float a, float b) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap32_sum(float a, float b) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// sum of v over the four 16-lane rows (lanes with equal bits 0-3), in every lane
__device__ __forceinline__ float sum_rows(float v) {
  const float t = swap16_sum(v, v);
  return swap32_sum(t, t);
}
template <int N>
struct Log2 {
  static constexpr int v = (N >= 16) ? 4 : (N >= 8) ? 3 : (N >= 4) ? 2 : (N >= 2) ? 1 : 0;
  static_assert((1 << v) == N, "power of two <= 16");
};

// Sum N = 2^n (n <= 4) values over all 64 lanes.  Halving steps over lane
// bits 5, 4, 0, 1 (in that order) each leave half of the values in a lane,
// summed with its partner's copy of that half; so after the n halving steps
// lane l holds one value whose index is bit 5, bit 4, bit 0, bit 1 of l (the
// first n of them, most significant first).  Plain sums over the remaining
// bits finish the total.  Lanes whose non-index bits are all clear hold the
// N distinct totals.
template <int N>
__device__ __forceinline__ float xreduce(const float (&v)[N], int lane) {
  constexpr int n = Log2<N>::v;
  float w[N];
#pragma unroll
  for (int i = 0; i < N; ++i) w[i] = v[i];
  // bit 5
  if constexpr (n >= 1) {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) w[i] = swap32_sum(w[i], w[N / 2 + i]);
  } else {
    w[0] = swap32_sum(w[0], w[0]);
  }
  // bit 4
  if constexpr (n >= 2) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) w[i] = swap16_sum(w[i], w[N / 4 + i]);
  } else {
    w[0] = swap16_sum(w[0], w[0]);
  }
  // bit 0
  if constexpr (n >= 3) {
    const bool up = lane & 1;
#pragma unroll
    for (int i = 0; i < N / 8; ++i) {
      const float mine = up ? w[N / 8 + i] : w[i];
      const float other = up ? w[i] : w[N / 8 + i];
      w[i] = mine + dpp<kDppXor1>(other);
    }
  } else {
    w[0] += dpp<kDppXor1>(w[0]);
  }
  // bit 1
  if constexpr (n >= 4) {
    const bool up = (lane >> 1) & 1;
    const float mine = up ? w[1] : w[0];
    const float other = up ? w[0] : w[1];
    w[0] = mine + dpp<kDppXor2>(other);
  } else {
    w[0] += dpp<kDppXor2>(w[0]);
  }
  // bits 2, 3
  w[0] += dpp<kDppRor4>(w[0]);
  w[0] += dpp<kDppRor8>(w[0]);
  return w[0];
}
template <int N>
__device__ __forceinline__ int xreduce_index(int lane) {
  constexpr int n = Log2<N>::v;
  const int bits[4] = {(lane >> 5) & 1, (lane >> 4) & 1, lane & 1, (lane >> 1) & 1};
  int idx = 0;
#pragma unroll
  for (int s = 0; s < n; ++s) idx = (idx << 1) | bits[s];
  return idx;
}
template <int N>
__device__ __forceinline__ bool xreduce_writer(int lane) {
  constexpr int n = Log2<N>::v;
  // index bits in use: 5 (n>=1), 4 (n>=2), 0 (n>=3), 1 (n>=4); all other bits clear
  int used = 0;
  if (n >= 1) used |= 32;
  if (n >= 2) used |= 16;
  if (n >= 3) used |= 1;
  if (n >= 4) used |= 2;
  return (lane & ~used) == 0;
}

}  // namespace mk
