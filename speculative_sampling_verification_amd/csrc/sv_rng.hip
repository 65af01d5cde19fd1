// Counter-based uniforms on the device: Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel
// random numbers: as easy as 1, 2, 3", SC 2011).  A block of four 64-bit words is a function
// of a 256-bit counter and a 128-bit key only, so every thread computes its own block with no
// state: ten rounds of two 64x64->128-bit products (counter words 0 and 2 by the published
// multipliers), the high halves xored with the other words and the round key, the key
// advanced by the published Weyl constants.  Word i of a stream (key, counter c) is word
// i mod 4 of the block at counter c + floor(i / 4); it becomes the float32 uniform
// (w >> 40) * 2^-24, exact, in [0, 1 - 2^-24].  These uniforms feed the accept tests and the
// draws of spec_verify and spec_sample, so the draft -> verify hand-off needs no host data.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "sv_internal.hpp"

namespace sv {
namespace {

constexpr uint64_t kPhiloxM0 = 0xD2E7470EE14C6C93ull;
constexpr uint64_t kPhiloxM1 = 0xCA5A826395121157ull;
constexpr uint64_t kPhiloxW0 = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kPhiloxW1 = 0xBB67AE8584CAA73Bull;
constexpr int kRngThreads = 256;

__device__ __forceinline__ void philox4x64_10(uint64_t (&x)[4], uint64_t k0, uint64_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t lo0 = kPhiloxM0 * x[0], hi0 = __umul64hi(kPhiloxM0, x[0]);
    const uint64_t lo1 = kPhiloxM1 * x[2], hi1 = __umul64hi(kPhiloxM1, x[2]);
    const uint64_t y0 = hi1 ^ x[1] ^ k0, y2 = hi0 ^ x[3] ^ k1;
    x[0] = y0;
    x[1] = lo1;
    x[2] = y2;
    x[3] = lo0;
    k0 += kPhiloxW0;
    k1 += kPhiloxW1;
  }
}

__device__ __forceinline__ float word_to_uniform(uint64_t w) {
  return (float)(uint32_t)(w >> 40) * 0x1.0p-24f;
}

// One block of four uniforms per thread; `vec` = out is 16-byte aligned (then full blocks
// are stored as one float4).
__global__ __launch_bounds__(kRngThreads) void k_philox_uniform(uint64_t k0, uint64_t k1,
                                                                uint64_t counter, int64_t n,
                                                                float* __restrict__ out,
                                                                int vec) {
  const int64_t blk = (int64_t)blockIdx.x * kRngThreads + threadIdx.x;
  const int64_t i0 = blk * 4;
  if (i0 >= n) return;
  // 256-bit counter = counter + blk (blk >= 0 and counter < 2^64: the carry reaches word 1)
  uint64_t x[4];
  x[0] = counter + (uint64_t)blk;
  x[1] = x[0] < counter ? 1ull : 0ull;
  x[2] = 0ull;
  x[3] = 0ull;
  philox4x64_10(x, k0, k1);
  if (vec && i0 + 3 < n) {
    float4 v;
    v.x = word_to_uniform(x[0]);
    v.y = word_to_uniform(x[1]);
    v.z = word_to_uniform(x[2]);
    v.w = word_to_uniform(x[3]);
    *reinterpret_cast<float4*>(out + i0) = v;
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (i0 + j < n) out[i0 + j] = word_to_uniform(x[j]);
  }
}

}  // namespace

hipError_t launch_philox_uniform(uint64_t key0, uint64_t key1, uint64_t counter, int64_t n,
                                 float* out, hipStream_t stream) {
  const int64_t blocks = (n + 4 * kRngThreads - 1) / (4 * kRngThreads);
  const int vec = (reinterpret_cast<uintptr_t>(out) & 15u) == 0;
  hipLaunchKernelGGL(k_philox_uniform, dim3((unsigned)blocks), dim3(kRngThreads), 0, stream,
                     key0, key1, counter, n, out, vec);
  return hipGetLastError();
}

}  // namespace sv
