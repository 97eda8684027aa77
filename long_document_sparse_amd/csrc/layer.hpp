// The rest of a Longformer encoder layer around the attention, after the
// FasterTransformer Longformer encoder guide (hnwysp.cn), compute flow: the
// projection GEMMs (Q, K, V for every token; the global path's Kg, Vg for every
// token and Qg for the global tokens only), bias add and transpose to
// [B, H, n, d], the attention, the output projection,
// AddBiasResidualLayerNorm, the FFN (intermediate GEMM, bias, GELU, output
// GEMM) and AddBiasResidualLayerNorm again.  The GEMMs are plain library
// GEMMs (16-bit inputs, fp32 results); the element-wise and row reductions
// here each read the fp32 GEMM result once and write the 16-bit storage type
// (bf16 or fp16, the template argument T) once.
#pragma once

namespace lwk {
namespace layer {

constexpr int LNT = 256;   // threads per block of the element-wise kernels

template <typename T, int N>
using vec_t = T __attribute__((ext_vector_type(N)));

template <int N>
__device__ __forceinline__ void loadf(const float* p, float (&v)[N]) {
#pragma unroll
  for (int q = 0; q < N / 4; ++q) {
    const float4 a = *reinterpret_cast<const float4*>(p + 4 * q);
    v[4 * q] = a.x; v[4 * q + 1] = a.y; v[4 * q + 2] = a.z; v[4 * q + 3] = a.w;
  }
}
template <int N, typename T>
__device__ __forceinline__ void loadh(const T* p, float (&v)[N]) {
  const vec_t<T, N> a = *reinterpret_cast<const vec_t<T, N>*>(p);
#pragma unroll
  for (int e = 0; e < N; ++e) v[e] = (float)a[e];
}
template <int N, typename T>
__device__ __forceinline__ void storeh(T* p, const float (&v)[N]) {
  vec_t<T, N> a;
#pragma unroll
  for (int e = 0; e < N; ++e) a[e] = (T)v[e];
  *reinterpret_cast<vec_t<T, N>*>(p) = a;
}

// P [M, parts hid] (fp32, M = B n) + bias [parts hid] -> `parts` tensors
// [B, H, n, 64] (columns 0 .. hid: the first, hid .. 2 hid: the second, ...;
// column h 64 + j of a part is head h, element j).  One thread per 8
// consecutive columns of a row.
template <typename T>
__global__ __launch_bounds__(LNT) void split_heads(const float* P, const T* bias, T* o0, T* o1, T* o2, int parts,
                                                   int B, int n, int H) {
  const int hid = H * 64, per_row = parts * hid / 8;
  const int64_t g = (int64_t)blockIdx.x * LNT + threadIdx.x;
  if (g >= (int64_t)B * n * per_row) return;
  const int64_t m = g / per_row;
  const int c = (int)(g % per_row) * 8;
  const int which = c / hid, ch = c % hid, h = ch / 64, j = ch % 64;
  const int b = (int)(m / n), i = (int)(m % n);
  float v[8], bb[8];
  loadf<8>(P + m * parts * hid + c, v);
  loadh<8>(bias + c, bb);
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] += bb[e];
  T* o = which == 0 ? o0 : (which == 1 ? o1 : o2);
  storeh<8>(o + (((int64_t)b * H + h) * n + i) * 64 + j, v);
}

// The same split for a GEMM result that already carries the bias and the
// storage type (the GEMM's bias epilogue): a 16-bit [M, parts hid] -> `parts`
// tensors [B, H, n, 64], 8 elements a thread.
template <typename T>
__global__ __launch_bounds__(LNT) void split_heads16(const T* P, T* o0, T* o1, T* o2, int parts, int B, int n,
                                                     int H) {
  const int hid = H * 64, per_row = parts * hid / 8;
  const int64_t g = (int64_t)blockIdx.x * LNT + threadIdx.x;
  if (g >= (int64_t)B * n * per_row) return;
  const int64_t m = g / per_row;
  const int c = (int)(g % per_row) * 8;
  const int which = c / hid, ch = c % hid, h = ch / 64, j = ch % 64;
  const int b = (int)(m / n), i = (int)(m % n);
  T* o = which == 0 ? o0 : (which == 1 ? o1 : o2);
  *reinterpret_cast<vec_t<T, 8>*>(o + (((int64_t)b * H + h) * n + i) * 64 + j) =
      *reinterpret_cast<const vec_t<T, 8>*>(P + m * parts * hid + c);
}

// The global tokens of each batch row (valid and global in the masks), in
// position order, at most mg of them: gpos [B][mg] receives their positions
// and -1 past the row's count.  One workgroup per batch row, 16 positions a
// thread per pass (4096 a pass), stopping once mg are found.
constexpr int GPT = 16;
__global__ __launch_bounds__(LNT) void find_global_rows(const float* lmask, const float* gmask, int n, int mg,
                                                        int32_t* gpos) {
  __shared__ int wsum[LNT / 64];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* lm = lmask + (int64_t)b * n;
  const float* gm = gmask + (int64_t)b * n;
  int32_t* gp = gpos + (int64_t)b * mg;
  int carry = 0;
  for (int base = 0; base < n && carry < mg; base += LNT * GPT) {
    const int j0 = base + tid * GPT;
    uint32_t bits = 0;
#pragma unroll
    for (int e = 0; e < GPT; ++e) {
      const int j = j0 + e;
      const bool is_g = j < n && lm[j] != 0.0f && gm[j] != 0.0f;
      bits |= (is_g ? 1u : 0u) << e;
    }
    // exclusive prefix of the per-thread counts over the workgroup
    const int mine = __popc(bits);
    int incl = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int pre = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < LNT / 64; ++w) {
      pre += w < wave ? wsum[w] : 0;
      tot += wsum[w];
    }
    int k = carry + pre + incl - mine;
    while (bits) {
      const int e = __builtin_ctz(bits);
      bits &= bits - 1;
      if (k < mg) gp[k] = j0 + e;
      ++k;
    }
    carry += tot;
    __syncthreads();
  }
  for (int k = (carry < mg ? carry : mg) + tid; k < mg; k += LNT) gp[k] = -1;
}

// Xg [B mg, hid] = the rows of X at gpos (zero rows where gpos is -1): one
// wave per gathered row, 8 elements a lane at a time.
template <typename T>
__global__ __launch_bounds__(LNT) void gather_global_rows(const T* X, const int32_t* gpos, int n, int hid, int mg,
                                                          int64_t rows, T* Xg) {
  const int64_t r = (int64_t)blockIdx.x * (LNT / 64) + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int lane = threadIdx.x & 63;
  const int pos = gpos[r];
  const int64_t b = r / mg;
  const T* src = X + (b * n + (pos < 0 ? 0 : pos)) * hid;
  T* dst = Xg + r * hid;
  for (int c = lane * 8; c < hid; c += 64 * 8) {
    vec_t<T, 8> v = {};
    if (pos >= 0) v = *reinterpret_cast<const vec_t<T, 8>*>(src + c);
    *reinterpret_cast<vec_t<T, 8>*>(dst + c) = v;
  }
}

// Qg at the global tokens: Pg [B mg, hid] (fp32, the projection of the
// gathered rows) + bias [hid] -> Qg [B, H, n, 64] at row gpos[b][k]; rows of
// Qg at other positions are not written (the attention reads Qg at the global
// tokens only).  One thread per 8 columns of a gathered row.
template <typename T>
__global__ __launch_bounds__(LNT) void scatter_global_rows(const float* Pg, const T* bias, const int32_t* gpos, T* Qg,
                                                           int B, int n, int H, int mg) {
  const int hid = H * 64, per_row = hid / 8;
  const int64_t g = (int64_t)blockIdx.x * LNT + threadIdx.x;
  if (g >= (int64_t)B * mg * per_row) return;
  const int64_t r = g / per_row;
  const int pos = gpos[r];
  if (pos < 0) return;
  const int c = (int)(g % per_row) * 8, h = c / 64, j = c % 64;
  const int b = (int)(r / mg);
  float v[8], bb[8];
  loadf<8>(Pg + r * hid + c, v);
  loadh<8>(bias + c, bb);
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] += bb[e];
  storeh<8>(Qg + (((int64_t)b * H + h) * n + pos) * 64 + j, v);
}

// [B, H, n, 64] -> [M, hid], 8 elements a thread.
template <typename T>
__global__ __launch_bounds__(LNT) void merge_heads(const T* A, T* out, int B, int n, int H) {
  const int hid = H * 64, per_row = hid / 8;
  const int64_t g = (int64_t)blockIdx.x * LNT + threadIdx.x;
  if (g >= (int64_t)B * n * per_row) return;
  const int64_t m = g / per_row;
  const int c = (int)(g % per_row) * 8;
  const int h = c / 64, j = c % 64;
  const int b = (int)(m / n), i = (int)(m % n);
  *reinterpret_cast<vec_t<T, 8>*>(out + m * hid + c) =
      *reinterpret_cast<const vec_t<T, 8>*>(A + (((int64_t)b * H + h) * n + i) * 64 + j);
}

// Y = LayerNorm(G + bias + R) * gamma + beta over each row of hid = 64 PER
// columns (G fp32 from the GEMM, the rest 16-bit); mean and variance in fp32
// (two passes over the row held in registers), biased variance, eps inside the
// square root.  One wave per row: PER columns a lane, as PER / VW groups of VW
// consecutive columns (VW = 8, or 4 when PER is not a multiple of 8).
template <typename T, int PER, bool G16 = false>
__global__ __launch_bounds__(LNT) void bias_residual_layernorm(const void* Gv, const T* bias, const T* R,
                                                               const T* gamma, const T* beta, float eps, T* Y,
                                                               int64_t M) {
  constexpr int hid = PER * 64;
  constexpr int VW = PER % 8 == 0 ? 8 : 4;
  static_assert(PER % VW == 0, "columns per lane");
  const int lane = threadIdx.x & 63;
  const int64_t m = (int64_t)blockIdx.x * (LNT / 64) + (threadIdx.x >> 6);
  if (m >= M) return;
  float x[PER];
#pragma unroll
  for (int q = 0; q < PER / VW; ++q) {
    const int c = (q * 64 + lane) * VW;
    float g[VW], b[VW], r[VW];
    if constexpr (G16) {
      // the GEMM's 16-bit result, the bias already added by its epilogue
      loadh<VW>(static_cast<const T*>(Gv) + m * hid + c, g);
#pragma unroll
      for (int e = 0; e < VW; ++e) b[e] = 0.0f;
    } else {
      loadf<VW>(static_cast<const float*>(Gv) + m * hid + c, g);
      loadh<VW>(bias + c, b);
    }
    loadh<VW>(R + m * hid + c, r);
#pragma unroll
    for (int e = 0; e < VW; ++e) x[q * VW + e] = g[e] + b[e] + r[e];
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
  for (int q = 0; q < PER / VW; ++q) {
    const int c = (q * 64 + lane) * VW;
    float ga[VW], be[VW], y[VW];
    loadh<VW>(gamma + c, ga);
    loadh<VW>(beta + c, be);
#pragma unroll
    for (int e = 0; e < VW; ++e) y[e] = (x[q * VW + e] - mean) * rstd * ga[e] + be[e];
    storeh<VW>(Y + m * hid + c, y);
  }
}

// Y = gelu(G + bias), gelu(x) = x Phi(x) = x (1 + erf(x / sqrt 2)) / 2, G fp32
// [M, cols], Y 16-bit; 8 columns a thread.
template <typename T>
__global__ __launch_bounds__(LNT) void bias_gelu(const float* G, const T* bias, T* Y, int64_t M, int cols) {
  const int per_row = cols / 8;
  const int64_t g = (int64_t)blockIdx.x * LNT + threadIdx.x;
  if (g >= M * per_row) return;
  const int64_t m = g / per_row;
  const int c = (int)(g % per_row) * 8;
  float v[8], b[8];
  loadf<8>(G + m * cols + c, v);
  loadh<8>(bias + c, b);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = v[e] + b[e];
    v[e] = 0.5f * x * (1.0f + erff(x * 0.70710678118654752f));
  }
  storeh<8>(Y + m * cols + c, v);
}

// gelu(x) = x Phi(x) with the normal tail Q(|x|) = (1 - erf(|x| / sqrt 2)) / 2
// from the rational approximation of erf in Abramowitz and Stegun 7.1.26
// (Hastings): erf(a) = 1 - t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) e^(-a^2),
// t = 1 / (1 + p a), absolute error at most 1.5e-7.  Phi(x) = 1 - Q for x >= 0,
// Q for x < 0.  Against the exact erf form, the result's absolute error stays
// below 2.2e-7 everywhere; its relative error is below 1.3e-5 where
// |gelu(x)| > 0.01 and below 1.7e-4 where |gelu(x)| > 0.001 -- under the
// 16-bit rounding of the result (2^-9 for bf16, 2^-11 for fp16).
__device__ __forceinline__ float gelu_as(float x) {
  const float a = fabsf(x) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, a, 1.0f));
  float poly = fmaf(1.061405429f, t, -1.453152027f);
  poly = fmaf(poly, t, 1.421413741f);
  poly = fmaf(poly, t, -0.284496736f);
  poly = fmaf(poly, t, 0.254829592f);
  const float q = 0.5f * poly * t * __builtin_amdgcn_exp2f(-a * a * 1.4426950408889634f);
  return x * (x >= 0.0f ? 1.0f - q : q);
}

// Y = gelu(Y) in place, Y 16-bit [count8 * 8] (the FFN-in GEMM already added
// the bias in its epilogue and wrote the storage type); 8 elements a thread.
template <typename T>
__global__ __launch_bounds__(LNT) void gelu16(T* Y, int64_t count8) {
  const int64_t g = (int64_t)blockIdx.x * LNT + threadIdx.x;
  if (g >= count8) return;
  float v[8];
  loadh<8>(Y + g * 8, v);
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = gelu_as(v[e]);
  storeh<8>(Y + g * 8, v);
}

}  // namespace layer
}  // namespace lwk
