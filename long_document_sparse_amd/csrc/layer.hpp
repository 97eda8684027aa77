// The rest of a Longformer encoder layer around the attention, after the
// FasterTransformer Longformer encoder guide (hnwysp.cn), compute flow: five
// projection GEMMs (Q, K, V and the global path's Qg, Kg, Vg), bias add and
// transpose to [B, H, n, d], the attention, the output projection,
// AddBiasResidualLayerNorm, the FFN (intermediate GEMM, bias, GELU, output
// GEMM) and AddBiasResidualLayerNorm again.  The GEMMs are plain library
// GEMMs (rocBLAS, bf16 inputs, fp32 results); the element-wise and row
// reductions here each read the fp32 GEMM result once and write bf16 once.
#pragma once

namespace lwk {
namespace layer {

constexpr int LNT = 256;   // threads per block of the element-wise kernels

__device__ __forceinline__ void load8f(const float* p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void load8b(const __bf16* p, float (&v)[8]) {
  const bf16x8 a = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (float)a[e];
}
__device__ __forceinline__ void store8b(__bf16* p, const float (&v)[8]) {
  bf16x8 a;
#pragma unroll
  for (int e = 0; e < 8; ++e) a[e] = (__bf16)v[e];
  *reinterpret_cast<bf16x8*>(p) = a;
}

// P [M, 3 hid] (fp32, M = B n) + bias [3 hid] -> three [B, H, n, 64] bf16
// tensors (columns 0 .. hid: the first, hid .. 2 hid: the second, 2 hid ..:
// the third; column h 64 + j of a third is head h, element j).  One thread per
// 8 consecutive columns of a row.
__global__ __launch_bounds__(LNT) void split_heads(const float* P, const __bf16* bias, __bf16* o0, __bf16* o1,
                                                   __bf16* o2, int B, int n, int H) {
  const int hid = H * 64, per_row = 3 * hid / 8;
  const int64_t g = (int64_t)blockIdx.x * LNT + threadIdx.x;
  if (g >= (int64_t)B * n * per_row) return;
  const int64_t m = g / per_row;
  const int c = (int)(g % per_row) * 8;
  const int which = c / hid, ch = c % hid, h = ch / 64, j = ch % 64;
  const int b = (int)(m / n), i = (int)(m % n);
  float v[8], bb[8];
  load8f(P + m * 3 * hid + c, v);
  load8b(bias + c, bb);
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] += bb[e];
  __bf16* o = which == 0 ? o0 : (which == 1 ? o1 : o2);
  store8b(o + (((int64_t)b * H + h) * n + i) * 64 + j, v);
}

// [B, H, n, 64] -> [M, hid] (bf16 both), 8 elements a thread.
__global__ __launch_bounds__(LNT) void merge_heads(const __bf16* A, __bf16* out, int B, int n, int H) {
  const int hid = H * 64, per_row = hid / 8;
  const int64_t g = (int64_t)blockIdx.x * LNT + threadIdx.x;
  if (g >= (int64_t)B * n * per_row) return;
  const int64_t m = g / per_row;
  const int c = (int)(g % per_row) * 8;
  const int h = c / 64, j = c % 64;
  const int b = (int)(m / n), i = (int)(m % n);
  *reinterpret_cast<bf16x8*>(out + m * hid + c) =
      *reinterpret_cast<const bf16x8*>(A + (((int64_t)b * H + h) * n + i) * 64 + j);
}

// Y = LayerNorm(G + bias + R) * gamma + beta over each row of hid columns
// (G fp32 from the GEMM, the rest bf16); mean and variance in fp32 (two
// passes over the row held in registers), biased variance, eps inside the
// square root.  One wave per row, hid / 64 columns a lane (hid a multiple of
// 512, at most 4096).
template <int PER>
__global__ __launch_bounds__(LNT) void bias_residual_layernorm(const float* G, const __bf16* bias,
                                                               const __bf16* R, const __bf16* gamma,
                                                               const __bf16* beta, float eps, __bf16* Y,
                                                               int64_t M) {
  constexpr int hid = PER * 64;
  const int lane = threadIdx.x & 63;
  const int64_t m = (int64_t)blockIdx.x * (LNT / 64) + (threadIdx.x >> 6);
  if (m >= M) return;
  float x[PER];
#pragma unroll
  for (int q = 0; q < PER / 8; ++q) {
    const int c = (q * 64 + lane) * 8;
    float g[8], b[8], r[8];
    load8f(G + m * hid + c, g);
    load8b(bias + c, b);
    load8b(R + m * hid + c, r);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[q * 8 + e] = g[e] + b[e] + r[e];
  }
  float s = 0.0f;
#pragma unroll
  for (int e = 0; e < PER; ++e) s += x[e];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
  const float mean = s / hid;
  float v = 0.0f;
#pragma unroll
  for (int e = 0; e < PER; ++e) v = fmaf(x[e] - mean, x[e] - mean, v);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  const float rstd = 1.0f / sqrtf(v / hid + eps);
#pragma unroll
  for (int q = 0; q < PER / 8; ++q) {
    const int c = (q * 64 + lane) * 8;
    float ga[8], be[8], y[8];
    load8b(gamma + c, ga);
    load8b(beta + c, be);
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = (x[q * 8 + e] - mean) * rstd * ga[e] + be[e];
    store8b(Y + m * hid + c, y);
  }
}

// Y = gelu(G + bias), gelu(x) = x Phi(x) = x (1 + erf(x / sqrt 2)) / 2, G fp32
// [M, cols], Y bf16; 8 columns a thread.
__global__ __launch_bounds__(LNT) void bias_gelu(const float* G, const __bf16* bias, __bf16* Y, int64_t M,
                                                 int cols) {
  const int per_row = cols / 8;
  const int64_t g = (int64_t)blockIdx.x * LNT + threadIdx.x;
  if (g >= M * per_row) return;
  const int64_t m = g / per_row;
  const int c = (int)(g % per_row) * 8;
  float v[8], b[8];
  load8f(G + m * cols + c, v);
  load8b(bias + c, b);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = v[e] + b[e];
    v[e] = 0.5f * x * (1.0f + erff(x * 0.70710678118654752f));
  }
  store8b(Y + m * cols + c, v);
}

}  // namespace layer
}  // namespace lwk
