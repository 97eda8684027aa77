// probe.hpp -- two micro-kernels that measure what this chip delivers, so
// that roofline fractions can be stated against measured peaks beside the
// published ones.  Included once, by lwattn.hip.
//
//   mfma_probe_kernel  every wave issues eight independent accumulation
//                      chains of v_mfma_f32_32x32x16_bf16 (32 x 32 x 16 x 2 =
//                      32768 flops each) for `iters` rounds; two waves per
//                      SIMD keep the matrix pipe fed.
//   read_probe_kernel  a grid-stride stream of 16-byte loads over a buffer
//                      far larger than the last-level cache (HBM read rate).
// Both write one value per wave or workgroup so that nothing is optimised
// away.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lwk {
namespace probe {

constexpr int MFMA_BLOCKS = 512;     // two per compute unit: 2 waves per SIMD
constexpr int MFMA_THREADS = 256;
constexpr int MFMA_CHAINS = 8;
constexpr int READ_BLOCKS = 4096;
constexpr int READ_THREADS = 256;

typedef float f32x16p __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8p __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(MFMA_THREADS) void mfma_probe_kernel(int iters, float seed, float* out) {
  const int lane = threadIdx.x & 63;
  bf16x8p a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(seed * (float)(lane + e));
    b[e] = (__bf16)(seed * (float)(lane - e));
  }
  f32x16p acc[MFMA_CHAINS];
#pragma unroll
  for (int k = 0; k < MFMA_CHAINS; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[k][r] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < MFMA_CHAINS; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < MFMA_CHAINS; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[k][r];
  if (lane == 0) out[blockIdx.x * (MFMA_THREADS / 64) + (threadIdx.x >> 6)] = s;
}

__global__ __launch_bounds__(READ_THREADS) void read_probe_kernel(const uint4* src, int64_t n16, float* out) {
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * READ_THREADS;
  int64_t i = (int64_t)blockIdx.x * READ_THREADS + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 x0 = src[i], x1 = src[i + stride], x2 = src[i + 2 * stride], x3 = src[i + 3 * stride];
    acc ^= x0.x ^ x0.y ^ x0.z ^ x0.w ^ x1.x ^ x1.y ^ x1.z ^ x1.w;
    acc ^= x2.x ^ x2.y ^ x2.z ^ x2.w ^ x3.x ^ x3.y ^ x3.z ^ x3.w;
  }
  for (; i < n16; i += stride) {
    const uint4 x = src[i];
    acc ^= x.x ^ x.y ^ x.z ^ x.w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
  __shared__ uint32_t part[READ_THREADS / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int w = 0; w < READ_THREADS / 64; ++w) t ^= part[w];
    out[blockIdx.x] = (float)(t & 0xFFFFu);
  }
}

}  // namespace probe
}  // namespace lwk
