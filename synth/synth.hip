// Seeded synthetic inputs: Philox4x32-10 (Salmon et al., SC'11) with a
// Box-Muller transform in double precision.  Host and device code compute the
// same expressions; see include/synth.h for the element mapping.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "synth.h"

namespace {

constexpr uint32_t kMul0 = 0xD2511F53u;
constexpr uint32_t kMul1 = 0xCD9E8D57u;
constexpr uint32_t kWeyl0 = 0x9E3779B9u;  // golden ratio
constexpr uint32_t kWeyl1 = 0xBB67AE85u;  // sqrt(3) - 1

__host__ __device__ inline void philox(uint32_t c[4], uint32_t k0, uint32_t k1) {
  for (int r = 0; r < 10; ++r) {
    uint64_t p0 = (uint64_t)kMul0 * c[0];
    uint64_t p1 = (uint64_t)kMul1 * c[2];
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c[1] ^ k0;
    uint32_t n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
    k0 += kWeyl0;
    k1 += kWeyl1;
  }
}

// binary32 -> bf16, round to nearest even (NaN kept quiet)
__host__ __device__ inline uint16_t f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

__host__ __device__ inline void block_values(uint64_t blk, uint64_t seed, uint64_t stream, int normal, double a,
                                             double b, float out[4]) {
  uint32_t c[4] = {(uint32_t)blk, (uint32_t)(blk >> 32), (uint32_t)stream, (uint32_t)(stream >> 32)};
  philox(c, (uint32_t)seed, (uint32_t)(seed >> 32));
  const double two32 = 4294967296.0;
  if (normal) {
    for (int p = 0; p < 2; ++p) {
      double u1 = ((double)c[2 * p] + 1.0) / two32;
      double u2 = (double)c[2 * p + 1] / two32;
      double rad = sqrt(-2.0 * log(u1));
      double ang = 6.283185307179586476925286766559 * u2;
      out[2 * p] = (float)(a + b * (rad * cos(ang)));
      out[2 * p + 1] = (float)(a + b * (rad * sin(ang)));
    }
  } else {
    for (int p = 0; p < 4; ++p) {
      double u = ((double)c[p] + 0.5) / two32;
      out[p] = (float)(a + (b - a) * u);
    }
  }
}

__global__ void fill_kernel(void* dst, int dtype, uint64_t n, uint64_t seed, uint64_t stream, int normal, double a,
                            double b) {
  uint64_t nblk = (n + 3) / 4;
  for (uint64_t blk = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; blk < nblk;
       blk += (uint64_t)gridDim.x * blockDim.x) {
    float v[4];
    block_values(blk, seed, stream, normal, a, b, v);
    uint64_t i0 = blk * 4;
    if (i0 + 4 <= n) {
      if (dtype == SYNTH_BF16) {
        uint32_t lo = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
        uint32_t hi = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
        if ((i0 & 3) == 0 && (((uintptr_t)dst & 7) == 0)) {
          reinterpret_cast<uint2*>(dst)[blk] = make_uint2(lo, hi);
        } else {
          uint16_t* d = (uint16_t*)dst + i0;
          d[0] = (uint16_t)lo; d[1] = (uint16_t)(lo >> 16); d[2] = (uint16_t)hi; d[3] = (uint16_t)(hi >> 16);
        }
      } else {
        float* d = (float*)dst + i0;
        if (((uintptr_t)dst & 15) == 0) *reinterpret_cast<float4*>(d) = make_float4(v[0], v[1], v[2], v[3]);
        else { d[0] = v[0]; d[1] = v[1]; d[2] = v[2]; d[3] = v[3]; }
      }
    } else {
      for (uint64_t j = 0; i0 + j < n; ++j) {
        if (dtype == SYNTH_BF16) ((uint16_t*)dst)[i0 + j] = f32_to_bf16(v[j]);
        else ((float*)dst)[i0 + j] = v[j];
      }
    }
  }
}

int fill_host(void* dst, int dtype, uint64_t n, uint64_t seed, uint64_t stream, int normal, double a, double b) {
  if ((!dst && n) || (dtype != SYNTH_F32 && dtype != SYNTH_BF16)) return -1;
  for (uint64_t blk = 0; blk * 4 < n; ++blk) {
    float v[4];
    block_values(blk, seed, stream, normal, a, b, v);
    for (int j = 0; j < 4 && blk * 4 + j < n; ++j) {
      uint64_t i = blk * 4 + j;
      if (dtype == SYNTH_BF16) ((uint16_t*)dst)[i] = f32_to_bf16(v[j]);
      else ((float*)dst)[i] = v[j];
    }
  }
  return 0;
}

int fill_device(void* dst, int dtype, uint64_t n, uint64_t seed, uint64_t stream, int normal, double a, double b,
                void* hs) {
  if ((!dst && n) || (dtype != SYNTH_F32 && dtype != SYNTH_BF16)) return -1;
  if (n == 0) return 0;
  uint64_t nblk = (n + 3) / 4;
  uint64_t grid = (nblk + 255) / 256;
  if (grid > 65536) grid = 65536;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)hs, dst, dtype, n, seed, stream,
                     normal, a, b);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // namespace

extern "C" {

void synth_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
  philox(c, key[0], key[1]);
  for (int i = 0; i < 4; ++i) out[i] = c[i];
}

int synth_fill_normal_host(void* dst, int dtype, uint64_t n, uint64_t seed, uint64_t stream, double mean,
                           double std) {
  return fill_host(dst, dtype, n, seed, stream, 1, mean, std);
}

int synth_fill_uniform_host(void* dst, int dtype, uint64_t n, uint64_t seed, uint64_t stream, double lo,
                            double hi) {
  return fill_host(dst, dtype, n, seed, stream, 0, lo, hi);
}

int synth_fill_normal_device(void* dst, int dtype, uint64_t n, uint64_t seed, uint64_t stream, double mean,
                             double std, void* hip_stream) {
  return fill_device(dst, dtype, n, seed, stream, 1, mean, std, hip_stream);
}

int synth_fill_uniform_device(void* dst, int dtype, uint64_t n, uint64_t seed, uint64_t stream, double lo,
                              double hi, void* hip_stream) {
  return fill_device(dst, dtype, n, seed, stream, 0, lo, hi, hip_stream);
}

}  // extern "C"
