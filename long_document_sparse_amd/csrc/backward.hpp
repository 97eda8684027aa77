// Backward of the window + global attention: gradients for Q, K, V, Qg, Kg, Vg
// given dO, the gradient of a loss with respect to the forward's output O.
//
// What is differentiated is the forward of kernels.hpp: a local row softmaxes
// over its window keys (same residue class, |i - j| <= w/2 in subsequence
// index, real, not global) plus every global key, with (Q, K, V); a global row
// softmaxes over every real key with (Qg, Kg, Vg); padded rows are zero.  By
// the chain rule through O_i = sum_j P_ij v_j and the softmax, with
// dP_ij = <dO_i, v_j> and D_i = <dO_i, O_i> = sum_j P_ij dP_ij:
//   dS_ij = P_ij (dP_ij - D_i)
//   dq_i  = scale sum_j dS_ij k_j      dk_j = scale sum_i dS_ij q_i      dv_j = sum_i P_ij dO_i
// (LongFormer notes, sections "Sliding Window", "Dilated Sliding Window" and
// "Global Attention", for the forward; the gradient is its derivative).
//
// Three launches on the caller's stream:
//   1. the global-index compaction (the forward's compaction workgroup);
//   2. dQ / dQg, one workgroup per 64 query rows (a residue class block of a
//      head, or a tile of global rows): a first pass over the row's keys for
//      the log-sum-exp, a second for dQ; it leaves (log-sum-exp, D) per row;
//   3. dK / dV / dKg / dVg, one workgroup per 64 keys of a residue class (its
//      window rows, then the global rows), and one per tile of global keys
//      (every local row attends to them through K and V).
// Every tile is 64 x 64 in fp32 in LDS (bf16 inputs are widened when staged);
// each thread owns a 4 x 4 block of every 64 x 64 product, rows rg + 16 i and
// columns cg + 16 j with rg = tid / 16, cg = tid % 16, so that the LDS rows
// its wave reads in one instruction fall in different banks.
#pragma once

namespace lwk {
namespace bw {

constexpr int T = 64;            // rows or keys per tile
constexpr int LS = 68;           // LDS row stride in floats
constexpr int TILE = T * LS;     // floats per LDS tile
constexpr int NTH = 256;         // threads per workgroup

struct BwParams {
  const uint8_t *Q, *K, *V, *Qg, *Kg, *Vg, *O, *dO;
  uint8_t *dQ, *dK, *dV, *dQg, *dKg, *dVg;
  const float* lmask;
  const float* gmask;
  const int32_t* gidx;          // [B,n] global positions, ascending
  const int32_t* gcnt;          // [B]
  const int32_t* head_stride;   // [H] dilation stride
  const int32_t* head_blk;      // [H+1] prefix over heads of 64-row blocks (all residue classes)
  float2* stats;                // [B,H,n] (log-sum-exp, D) of every non-padded row; the bf16
                                // kernels keep the log-sum-exp in log2 units
  float* gq;                    // [B,H,max_global,gsplit,68] per-chunk dQg sums, max, sum of exp
  float* gk;                    // [B,H,max_global,gsplit,128] per-chunk dK, dV sums of global keys
  float* gml;                   // [B,H,max_global,gspad,2] per-chunk max and sum of exp of the global rows
  int gsplit, gchunk;           // position chunks of the global rows' / keys' sums, chunk length
  int gspad;                    // gsplit rounded up to even (16-byte rows of gml)
  int comp_fold;                // bf16: the dQ launch compacts the rows (its grid fits one round of slots)
  int merge_fold;               // bf16: the dK/dV launch merges the chunk sums (in its last round's spare slots)
  int B, H, n, r, max_global, ntg, blocks_per_b;
  float scale;
};

// Per-position kind: 0 padded or out of range, 1 global, 2 local.
__device__ __forceinline__ uint8_t kind_of(const BwParams& p, int b, int pos) {
  if (pos < 0) return 0;
  const float lv = p.lmask[(int64_t)b * p.n + pos];
  if (lv == 0.0f) return 0;
  return p.gmask[(int64_t)b * p.n + pos] != 0.0f ? 1 : 2;
}

template <bool BF>
__device__ __forceinline__ void load16(const uint8_t* src, float (&v)[16]) {
  if constexpr (BF) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint4 u = *reinterpret_cast<const uint4*>(src + 16 * h);
      const bf16x8 x = __builtin_bit_cast(bf16x8, u);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[8 * h + e] = (float)x[e];
    }
  } else {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float4 u = *reinterpret_cast<const float4*>(src + 16 * h);
      v[4 * h] = u.x; v[4 * h + 1] = u.y; v[4 * h + 2] = u.z; v[4 * h + 3] = u.w;
    }
  }
}

template <bool BF>
__device__ __forceinline__ void store16(uint8_t* dst, const float (&v)[16]) {
  if constexpr (BF) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bf16x8 x;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = (__bf16)v[8 * h + e];
      *reinterpret_cast<uint4*>(dst + 16 * h) = __builtin_bit_cast(uint4, x);
    }
  } else {
#pragma unroll
    for (int h = 0; h < 4; ++h)
      *reinterpret_cast<float4*>(dst + 16 * h) = make_float4(v[4 * h], v[4 * h + 1], v[4 * h + 2], v[4 * h + 3]);
  }
}

// 64 rows (positions pos[0..63], -1 = zero row) of a [*, 64] head into an LDS
// tile, row-major ([row][d]) or transposed ([d][row]).
template <bool BF>
__device__ __forceinline__ void load_tile(float* dst, const uint8_t* head, const int* pos, bool tr) {
  constexpr int RB = D * (BF ? 2 : 4);
  const int t = threadIdx.x, row = t >> 2, q = t & 3;
  const int ps = pos[row];
  float v[16];
  if (ps >= 0) {
    load16<BF>(head + (int64_t)ps * RB + q * 16 * (BF ? 2 : 4), v);
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = 0.0f;
  }
  if (!tr) {
#pragma unroll
    for (int e = 0; e < 16; e += 4)
      *reinterpret_cast<float4*>(dst + row * LS + 16 * q + e) = make_float4(v[e], v[e + 1], v[e + 2], v[e + 3]);
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e) dst[(16 * q + e) * LS + row] = v[e];
  }
}

// c[i][j] += sum_k A[rg + 16 i][k] * B[cg + 16 j][k] over k < kmax (A and B
// row-major), for i < ni and j < nj: a tile with few live rows (a tile of
// global rows or keys) takes ni or nj = ceil(live / 16) and kmax = the live
// rows rounded up to 4.  The bounds are workgroup-uniform.
__device__ __forceinline__ void gemm_abt(const float* A, const float* B, float (&c)[4][4],
                                         int ni = 4, int nj = 4, int kmax = T) {
  const int t = threadIdx.x, rg = t >> 4, cg = t & 15;
  for (int k = 0; k < kmax; k += 4) {
    float4 a[4], bv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i < ni) a[i] = *reinterpret_cast<const float4*>(A + (rg + 16 * i) * LS + k);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j < nj) bv[j] = *reinterpret_cast<const float4*>(B + (cg + 16 * j) * LS + k);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (i < ni && j < nj) {
          c[i][j] = fmaf(a[i].x, bv[j].x, c[i][j]);
          c[i][j] = fmaf(a[i].y, bv[j].y, c[i][j]);
          c[i][j] = fmaf(a[i].z, bv[j].z, c[i][j]);
          c[i][j] = fmaf(a[i].w, bv[j].w, c[i][j]);
        }
  }
}

__device__ __forceinline__ int groups16(int live) { return live >= T ? 4 : (live + 15) / 16; }

__device__ __forceinline__ void zero(float (&c)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) c[i][j] = 0.0f;
}

// Writes a thread's 4 x 4 block into an LDS tile [rg + 16 i][cg + 16 j].
__device__ __forceinline__ void put(float* dst, const float (&c)[4][4]) {
  const int t = threadIdx.x, rg = t >> 4, cg = t & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) dst[(rg + 16 * i) * LS + cg + 16 * j] = c[i][j];
}

// Rows of a staged [row][d] tile to global memory (rows with pos < 0 or
// keep[row] == 0 are skipped), converted to the storage type.
template <bool BF>
__device__ __forceinline__ void store_tile(uint8_t* head, const float* src, const int* pos,
                                           const uint8_t* keep) {
  constexpr int RB = D * (BF ? 2 : 4);
  const int t = threadIdx.x, row = t >> 2, q = t & 3;
  const int ps = pos[row];
  if (ps < 0 || !keep[row]) return;
  float v[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) v[e] = src[row * LS + 16 * q + e];
  store16<BF>(head + (int64_t)ps * RB + q * 16 * (BF ? 2 : 4), v);
}

// Shared per-tile bookkeeping in LDS.
struct alignas(16) Meta {
  int rpos[T], kpos[T];
  uint8_t rkind[T], kkind[T], rkeep[T], kkeep[T];
  float lse[T], dd[T];
  uint32_t okm[2];   // matrix-core kernels: bit k of word q: tile row / key 32 q + k counts
};

// Every key tile a block of 64 query rows visits: window tiles (kt < nwin),
// then global-key tiles; fills kpos/kkind and says how keys are allowed.
struct KeyTiles {
  int nwin, ntot;
};

// ---------------------------------------------------------------------------
// dQ of 64 local-row candidates (rows I0 .. I0+63 of residue class rho of
// (b, h)); also writes zero dQ / dQg rows where this block's rows have no such
// gradient, and the rows' (log-sum-exp, D).
template <bool BF>
__device__ void dq_local(const BwParams& p, int b, int h, int rho, int blk, float* sm, Meta& mt) {
  constexpr int RB = D * (BF ? 2 : 4);
  float* tQ = sm;
  float* tdO = sm + TILE;
  float* tK = sm + 2 * TILE;
  float* tV = sm + 3 * TILE;
  float* tKt = sm + 4 * TILE;
  float* tS = sm + 5 * TILE;
  const int t = threadIdx.x, rg = t >> 4, cg = t & 15;
  const int n = p.n, s = p.head_stride[h], r = p.r;
  const int nr = (n - rho + s - 1) / s;
  const int I0 = blk * T;
  const int64_t hoff = ((int64_t)b * p.H + h) * n * RB;
  int g = p.gcnt[b];
  if (g > p.max_global) g = p.max_global;
  if (t < T) {
    const int ip = I0 + t;
    const int ps = ip < nr ? rho + ip * s : -1;
    mt.rpos[t] = ps;
    mt.rkind[t] = kind_of(p, b, ps);
  }
  __syncthreads();
  load_tile<BF>(tQ, p.Q + hoff, mt.rpos, false);
  load_tile<BF>(tdO, p.dO + hoff, mt.rpos, false);
  load_tile<BF>(tS, p.O + hoff, mt.rpos, false);
  __syncthreads();
  {
    // D = <dO, O> per row: four threads per row
    const int row = t >> 2, q = t & 3;
    float a = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) a = fmaf(tdO[row * LS + 16 * q + e], tS[row * LS + 16 * q + e], a);
    a += __shfl_xor(a, 1);
    a += __shfl_xor(a, 2);
    if (q == 0) mt.dd[row] = a;
  }
  const int nwin = (T + 2 * r + T - 1) / T;
  const int ntot = nwin + p.ntg;
  auto set_keys = [&](int kt) {
    if (t < T) {
      int ps = -1;
      if (kt < nwin) {
        const int jp = I0 - r + T * kt + t;
        if (jp >= 0 && jp < nr) ps = rho + jp * s;
        mt.kpos[t] = ps;
        mt.kkind[t] = kind_of(p, b, ps);
      } else {
        const int idx = T * (kt - nwin) + t;
        if (idx < g) ps = p.gidx[(int64_t)b * n + idx];
        mt.kpos[t] = ps;
        mt.kkind[t] = ps >= 0 ? 1 : 0;
      }
    }
  };
  auto allowed = [&](int kt, int row, int col) {
    if (mt.rkind[row] != 2) return false;
    if (kt < nwin) {
      const int dlt = (T * kt + col - r) - row;   // key index minus row index (subsequence)
      return mt.kkind[col] == 2 && dlt >= -r && dlt <= r;
    }
    return mt.kkind[col] == 1;
  };
  // pass 1: log-sum-exp of every row over its allowed keys
  float m[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { m[i] = -INFINITY; l[i] = 0.0f; }
  for (int kt = 0; kt < ntot; ++kt) {
    __syncthreads();
    set_keys(kt);
    __syncthreads();
    load_tile<BF>(tK, p.K + hoff, mt.kpos, false);
    __syncthreads();
    float c[4][4];
    zero(c);
    gemm_abt(tQ, tK, c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float mx = m[i];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (allowed(kt, rg + 16 * i, cg + 16 * j)) mx = fmaxf(mx, p.scale * c[i][j]);
      float sum = mx == -INFINITY ? 0.0f : l[i] * __expf(m[i] - mx);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (allowed(kt, rg + 16 * i, cg + 16 * j)) sum += __expf(p.scale * c[i][j] - mx);
      m[i] = mx;
      l[i] = sum;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // combine the 16 threads of the row
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const float mo = __shfl_xor(m[i], o), lo = __shfl_xor(l[i], o);
      const float mx = fmaxf(m[i], mo);
      const float a = m[i] == -INFINITY ? 0.0f : l[i] * __expf(m[i] - mx);
      const float bb = mo == -INFINITY ? 0.0f : lo * __expf(mo - mx);
      m[i] = mx;
      l[i] = a + bb;
    }
    if (cg == 0) mt.lse[rg + 16 * i] = l[i] > 0.0f ? m[i] + __logf(l[i]) : INFINITY;
  }
  // pass 2: dQ = scale dS K with dS = P (dP - D)
  float acc[4][4];
  zero(acc);
  for (int kt = 0; kt < ntot; ++kt) {
    __syncthreads();
    set_keys(kt);
    __syncthreads();
    load_tile<BF>(tK, p.K + hoff, mt.kpos, false);
    load_tile<BF>(tV, p.V + hoff, mt.kpos, false);
    load_tile<BF>(tKt, p.K + hoff, mt.kpos, true);
    __syncthreads();
    float c[4][4], e[4][4];
    zero(c);
    zero(e);
    gemm_abt(tQ, tK, c);
    gemm_abt(tdO, tV, e);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = rg + 16 * i;
      const float ls = mt.lse[row], dv = mt.dd[row];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float pr = allowed(kt, row, cg + 16 * j) ? __expf(p.scale * c[i][j] - ls) : 0.0f;
        c[i][j] = pr * (e[i][j] - dv);
      }
    }
    put(tS, c);
    __syncthreads();
    gemm_abt(tS, tKt, acc);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = mt.rkind[rg + 16 * i] == 2 ? p.scale * acc[i][j] : 0.0f;
  put(tS, acc);
  if (t < T) {
    mt.rkeep[t] = 1;                       // every row of the block gets its dQ row
    mt.kkeep[t] = mt.rkind[t] != 1;        // and its zero dQg row unless it is global
    if (mt.rkind[t] == 2) p.stats[((int64_t)b * p.H + h) * n + mt.rpos[t]] = make_float2(mt.lse[t], mt.dd[t]);
  }
  __syncthreads();
  store_tile<BF>(p.dQ + hoff, tS, mt.rpos, mt.rkeep);
  // zero dQg rows: tS is not needed past this point, reuse tK as a zero tile
  for (int e2 = t; e2 < TILE; e2 += NTH) tK[e2] = 0.0f;
  __syncthreads();
  store_tile<BF>(p.dQg + hoff, tK, mt.rpos, mt.kkeep);
}

// dQg of global rows T*gt .. T*gt+63 of (b, h): every real key, with Qg, Kg, Vg.
template <bool BF>
__device__ void dq_global(const BwParams& p, int b, int h, int gt, float* sm, Meta& mt) {
  constexpr int RB = D * (BF ? 2 : 4);
  float* tQ = sm;
  float* tdO = sm + TILE;
  float* tK = sm + 2 * TILE;
  float* tV = sm + 3 * TILE;
  float* tKt = sm + 4 * TILE;
  float* tS = sm + 5 * TILE;
  const int t = threadIdx.x, rg = t >> 4, cg = t & 15;
  const int n = p.n;
  const int64_t hoff = ((int64_t)b * p.H + h) * n * RB;
  int g = p.gcnt[b];
  if (g > p.max_global) g = p.max_global;
  if (T * gt >= g) return;
  const int ni = groups16(g - T * gt);   // row groups with a live global row
  if (t < T) {
    const int idx = T * gt + t;
    const int ps = idx < g ? p.gidx[(int64_t)b * n + idx] : -1;
    mt.rpos[t] = ps;
    mt.rkind[t] = ps >= 0 ? 1 : 0;
  }
  __syncthreads();
  load_tile<BF>(tQ, p.Qg + hoff, mt.rpos, false);
  load_tile<BF>(tdO, p.dO + hoff, mt.rpos, false);
  load_tile<BF>(tS, p.O + hoff, mt.rpos, false);
  __syncthreads();
  {
    const int row = t >> 2, q = t & 3;
    float a = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) a = fmaf(tdO[row * LS + 16 * q + e], tS[row * LS + 16 * q + e], a);
    a += __shfl_xor(a, 1);
    a += __shfl_xor(a, 2);
    if (q == 0) mt.dd[row] = a;
  }
  const int ntot = (n + T - 1) / T;
  auto set_keys = [&](int kt) {
    if (t < T) {
      const int ps = T * kt + t;
      mt.kpos[t] = ps < n ? ps : -1;
      mt.kkind[t] = kind_of(p, b, ps < n ? ps : -1);
    }
  };
  auto allowed = [&](int row, int col) { return mt.rkind[row] == 1 && mt.kkind[col] != 0; };
  float m[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { m[i] = -INFINITY; l[i] = 0.0f; }
  for (int kt = 0; kt < ntot; ++kt) {
    __syncthreads();
    set_keys(kt);
    __syncthreads();
    load_tile<BF>(tK, p.Kg + hoff, mt.kpos, false);
    __syncthreads();
    float c[4][4];
    zero(c);
    gemm_abt(tQ, tK, c, ni);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float mx = m[i];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (allowed(rg + 16 * i, cg + 16 * j)) mx = fmaxf(mx, p.scale * c[i][j]);
      float sum = mx == -INFINITY ? 0.0f : l[i] * __expf(m[i] - mx);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (allowed(rg + 16 * i, cg + 16 * j)) sum += __expf(p.scale * c[i][j] - mx);
      m[i] = mx;
      l[i] = sum;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const float mo = __shfl_xor(m[i], o), lo = __shfl_xor(l[i], o);
      const float mx = fmaxf(m[i], mo);
      const float a = m[i] == -INFINITY ? 0.0f : l[i] * __expf(m[i] - mx);
      const float bb = mo == -INFINITY ? 0.0f : lo * __expf(mo - mx);
      m[i] = mx;
      l[i] = a + bb;
    }
    if (cg == 0) mt.lse[rg + 16 * i] = l[i] > 0.0f ? m[i] + __logf(l[i]) : INFINITY;
  }
  float acc[4][4];
  zero(acc);
  for (int kt = 0; kt < ntot; ++kt) {
    __syncthreads();
    set_keys(kt);
    __syncthreads();
    load_tile<BF>(tK, p.Kg + hoff, mt.kpos, false);
    load_tile<BF>(tV, p.Vg + hoff, mt.kpos, false);
    load_tile<BF>(tKt, p.Kg + hoff, mt.kpos, true);
    __syncthreads();
    float c[4][4], e[4][4];
    zero(c);
    zero(e);
    gemm_abt(tQ, tK, c, ni);
    gemm_abt(tdO, tV, e, ni);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = rg + 16 * i;
      const float ls = mt.lse[row], dv = mt.dd[row];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float pr = allowed(row, cg + 16 * j) ? __expf(p.scale * c[i][j] - ls) : 0.0f;
        c[i][j] = pr * (e[i][j] - dv);
      }
    }
    put(tS, c);
    __syncthreads();
    gemm_abt(tS, tKt, acc, ni);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] *= p.scale;
  put(tS, acc);
  if (t < T) {
    mt.rkeep[t] = mt.rkind[t] == 1;
    if (mt.rkind[t] == 1) p.stats[((int64_t)b * p.H + h) * n + mt.rpos[t]] = make_float2(mt.lse[t], mt.dd[t]);
  }
  __syncthreads();
  store_tile<BF>(p.dQg + hoff, tS, mt.rpos, mt.rkeep);
}

// One sweep of a key tile (kpos/kkind set, K-side tiles tK, tV staged) over
// query-row tiles: accK += dS^T Q, accV += P^T dO.  set_rows(qt) fills
// rpos/rkind/lse/dd of row tile qt; allowed(qt, key, row) is the mask.
// ni: key groups with a live key; live_rows(qt): live rows of row tile qt
// (rows past them are dead in every row tile but the last).
template <bool BF, class SetRows, class Allowed, class LiveRows>
__device__ __forceinline__ void kv_sweep(const BwParams& p, const uint8_t* Qsrc, int64_t hoff, int nq,
                                         const SetRows& set_rows, const Allowed& allowed,
                                         const LiveRows& live_rows, int ni, float* sm,
                                         Meta& mt, float (&accK)[4][4], float (&accV)[4][4]) {
  float* tK = sm;
  float* tV = sm + TILE;
  float* tQ = sm + 2 * TILE;
  float* tdO = sm + 3 * TILE;
  float* tQt = sm + 4 * TILE;
  float* tdOt = sm + 5 * TILE;
  float* tP = sm + 6 * TILE;
  float* tdS = sm + 7 * TILE;
  const int t = threadIdx.x, rg = t >> 4, cg = t & 15;
  for (int qt = 0; qt < nq; ++qt) {
    __syncthreads();
    set_rows(qt);
    __syncthreads();
    load_tile<BF>(tQ, Qsrc + hoff, mt.rpos, false);
    load_tile<BF>(tdO, p.dO + hoff, mt.rpos, false);
    load_tile<BF>(tQt, Qsrc + hoff, mt.rpos, true);
    load_tile<BF>(tdOt, p.dO + hoff, mt.rpos, true);
    __syncthreads();
    const int lr = live_rows(qt);
    const int nj = groups16(lr), kr = lr >= T ? T : (lr + 3) & ~3;
    float c[4][4], e[4][4];
    zero(c);
    zero(e);
    gemm_abt(tK, tQ, c, ni, nj);     // S^T [key][row]
    gemm_abt(tV, tdO, e, ni, nj);    // dP^T [key][row]
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = cg + 16 * j;
      const float ls = mt.lse[row], dv = mt.dd[row];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pr = allowed(qt, rg + 16 * i, row) ? __expf(p.scale * c[i][j] - ls) : 0.0f;
        c[i][j] = pr;
        e[i][j] = pr * (e[i][j] - dv);
      }
    }
    put(tP, c);
    put(tdS, e);
    __syncthreads();
    gemm_abt(tP, tdOt, accV, ni, 4, kr);    // [key][d] += sum_row P^T dO
    gemm_abt(tdS, tQt, accK, ni, 4, kr);    // [key][d] += sum_row dS^T Q
  }
}

// dK, dV (window part) and dKg, dVg of 64 keys: subsequence keys J0 .. J0+63
// of residue class rho of (b, h).
template <bool BF>
__device__ void dkv_window(const BwParams& p, int b, int h, int rho, int blk, float* sm, Meta& mt) {
  constexpr int RB = D * (BF ? 2 : 4);
  float* tK = sm;
  float* tV = sm + TILE;
  float* tQ = sm + 2 * TILE;
  const int t = threadIdx.x, rg = t >> 4, cg = t & 15;
  const int n = p.n, s = p.head_stride[h], r = p.r;
  const int nr = (n - rho + s - 1) / s;
  const int J0 = blk * T;
  const int64_t hoff = ((int64_t)b * p.H + h) * n * RB;
  const int64_t soff = ((int64_t)b * p.H + h) * n;
  int g = p.gcnt[b];
  if (g > p.max_global) g = p.max_global;
  if (t < T) {
    const int jp = J0 + t;
    const int ps = jp < nr ? rho + jp * s : -1;
    mt.kpos[t] = ps;
    mt.kkind[t] = kind_of(p, b, ps);
  }
  __syncthreads();
  load_tile<BF>(tK, p.K + hoff, mt.kpos, false);
  load_tile<BF>(tV, p.V + hoff, mt.kpos, false);
  const int nwin = (T + 2 * r + T - 1) / T;
  auto win_rows = [&](int qt) {
    if (t < T) {
      const int ip = J0 - r + T * qt + t;
      const int ps = ip >= 0 && ip < nr ? rho + ip * s : -1;
      const uint8_t kd = kind_of(p, b, ps);
      mt.rpos[t] = ps;
      mt.rkind[t] = kd;
      if (kd == 2) {
        const float2 st = p.stats[soff + ps];
        mt.lse[t] = st.x;
        mt.dd[t] = st.y;
      } else {
        mt.lse[t] = 0.0f;
        mt.dd[t] = 0.0f;
      }
    }
  };
  auto win_ok = [&](int qt, int key, int row) {
    const int dlt = (r + key) - (T * qt + row);   // key index minus row index (subsequence)
    return mt.kkind[key] == 2 && mt.rkind[row] == 2 && dlt >= -r && dlt <= r;
  };
  float accK[4][4], accV[4][4];
  zero(accK);
  zero(accV);
  kv_sweep<BF>(p, p.Q, hoff, nwin, win_rows, win_ok, [](int) { return T; }, 4, sm, mt, accK, accV);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) accK[i][j] *= p.scale;
  put(tQ, accK);
  put(tQ + TILE, accV);
  if (t < T) mt.kkeep[t] = mt.kkind[t] != 1;   // global keys' rows come from the global-key pass
  __syncthreads();
  store_tile<BF>(p.dK + hoff, tQ, mt.kpos, mt.kkeep);
  store_tile<BF>(p.dV + hoff, tQ + TILE, mt.kpos, mt.kkeep);
  // the global rows' part: dKg, dVg of the same keys
  __syncthreads();
  load_tile<BF>(tK, p.Kg + hoff, mt.kpos, false);
  load_tile<BF>(tV, p.Vg + hoff, mt.kpos, false);
  auto glob_rows = [&](int qt) {
    if (t < T) {
      const int idx = T * qt + t;
      const int ps = idx < g ? p.gidx[(int64_t)b * n + idx] : -1;
      mt.rpos[t] = ps;
      mt.rkind[t] = ps >= 0 ? 1 : 0;
      if (ps >= 0) {
        const float2 st = p.stats[soff + ps];
        mt.lse[t] = st.x;
        mt.dd[t] = st.y;
      } else {
        mt.lse[t] = 0.0f;
        mt.dd[t] = 0.0f;
      }
    }
  };
  auto glob_ok = [&](int, int key, int row) { return mt.kkind[key] != 0 && mt.rkind[row] == 1; };
  zero(accK);
  zero(accV);
  const int nq = (g + T - 1) / T;
  kv_sweep<BF>(p, p.Qg, hoff, nq, glob_rows, glob_ok, [&](int qt) { return g - T * qt; }, 4, sm, mt,
               accK, accV);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) accK[i][j] *= p.scale;
  put(tQ, accK);
  put(tQ + TILE, accV);
  if (t < T) mt.kkeep[t] = 1;
  __syncthreads();
  store_tile<BF>(p.dKg + hoff, tQ, mt.kpos, mt.kkeep);
  store_tile<BF>(p.dVg + hoff, tQ + TILE, mt.kpos, mt.kkeep);
  (void)rg;
  (void)cg;
}

// dK, dV of global keys T*gt .. T*gt+63 of (b, h): every local row attends to
// them through K and V.
template <bool BF>
__device__ void dkv_global_keys(const BwParams& p, int b, int h, int gt, float* sm, Meta& mt) {
  constexpr int RB = D * (BF ? 2 : 4);
  float* tK = sm;
  float* tV = sm + TILE;
  float* tQ = sm + 2 * TILE;
  const int t = threadIdx.x, rg = t >> 4, cg = t & 15;
  const int n = p.n;
  const int64_t hoff = ((int64_t)b * p.H + h) * n * RB;
  const int64_t soff = ((int64_t)b * p.H + h) * n;
  int g = p.gcnt[b];
  if (g > p.max_global) g = p.max_global;
  if (T * gt >= g) return;
  if (t < T) {
    const int idx = T * gt + t;
    const int ps = idx < g ? p.gidx[(int64_t)b * n + idx] : -1;
    mt.kpos[t] = ps;
    mt.kkind[t] = ps >= 0 ? 1 : 0;
  }
  __syncthreads();
  load_tile<BF>(tK, p.K + hoff, mt.kpos, false);
  load_tile<BF>(tV, p.V + hoff, mt.kpos, false);
  auto all_rows = [&](int qt) {
    if (t < T) {
      const int ps0 = T * qt + t;
      const int ps = ps0 < n ? ps0 : -1;
      const uint8_t kd = kind_of(p, b, ps);
      mt.rpos[t] = ps;
      mt.rkind[t] = kd;
      if (kd == 2) {
        const float2 st = p.stats[soff + ps];
        mt.lse[t] = st.x;
        mt.dd[t] = st.y;
      } else {
        mt.lse[t] = 0.0f;
        mt.dd[t] = 0.0f;
      }
    }
  };
  auto ok = [&](int, int key, int row) { return mt.kkind[key] == 1 && mt.rkind[row] == 2; };
  float accK[4][4], accV[4][4];
  zero(accK);
  zero(accV);
  kv_sweep<BF>(p, p.Q, hoff, (n + T - 1) / T, all_rows, ok, [](int) { return T; }, groups16(g - T * gt),
               sm, mt, accK, accV);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) accK[i][j] *= p.scale;
  put(tQ, accK);
  put(tQ + TILE, accV);
  if (t < T) mt.kkeep[t] = mt.kkind[t] == 1;
  __syncthreads();
  store_tile<BF>(p.dK + hoff, tQ, mt.kpos, mt.kkeep);
  store_tile<BF>(p.dV + hoff, tQ + TILE, mt.kpos, mt.kkeep);
  (void)rg;
  (void)cg;
}

// Block id of a 64-row block (all residue classes of all heads of a batch row)
// into (b, h, rho, block within the class).
template <typename P>
__device__ __forceinline__ void decode_block(const P& p, int lb, int& b, int& h, int& rho, int& blk) {
  b = lb / p.blocks_per_b;
  int rem = lb - b * p.blocks_per_b;
  h = 0;
  while (p.head_blk[h + 1] <= rem) ++h;
  rem -= p.head_blk[h];
  const int s = p.head_stride[h];
  rho = 0;
  for (; rho < s; ++rho) {
    const int nr = (p.n - rho + s - 1) / s;
    const int nb = (nr + T - 1) / T;
    if (rem < nb) break;
    rem -= nb;
  }
  blk = rem;
}

constexpr int DQ_SMEM = 6 * TILE * 4;
constexpr int DKV_SMEM = 8 * TILE * 4;

// Grid order: the global-row (or global-key) tiles first, each of which
// walks the whole sequence, then the residue-class blocks.
template <bool BF>
__global__ __launch_bounds__(NTH) void dq_kernel(BwParams p) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  __shared__ Meta mt;
  const int nglob = p.B * p.H * p.ntg;
  const int bid = blockIdx.x;
  if (bid >= nglob) {
    int b, h, rho, blk;
    decode_block(p, bid - nglob, b, h, rho, blk);
    dq_local<BF>(p, b, h, rho, blk, sm, mt);
  } else {
    const int gt = bid % p.ntg, bh = bid / p.ntg;
    dq_global<BF>(p, bh / p.H, bh % p.H, gt, sm, mt);
  }
}

template <bool BF>
__global__ __launch_bounds__(NTH) void dkv_kernel(BwParams p) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  __shared__ Meta mt;
  const int nglob = p.B * p.H * p.ntg;
  const int bid = blockIdx.x;
  if (bid >= nglob) {
    int b, h, rho, blk;
    decode_block(p, bid - nglob, b, h, rho, blk);
    dkv_window<BF>(p, b, h, rho, blk, sm, mt);
  } else {
    const int gt = bid % p.ntg, bh = bid / p.ntg;
    dkv_global_keys<BF>(p, bh / p.H, bh % p.H, gt, sm, mt);
  }
}

// ---------------------------------------------------------------------------
// bf16 storage: the residue-class blocks on the matrix cores.  Four waves per
// workgroup; wave w owns a 32 x 32 quadrant of every 64-row x 64-key tile pair.
// The products use v_mfma_f32_32x32x16_bf16 with the operand layouts of the
// forward: A and B fragments hold X[row][32 h + 8 c .. +8] for lane row l % 32,
// h = l / 32, over four k-chunks c; an accumulator register r of lane l is
// element (8 (r / 4) + 4 h + r % 4, l % 32).  A product whose contraction runs
// over the accumulator's rows (dQ^T = K^T dS^T, dK^T = Q^T dS, dV^T = dO^T P)
// takes the scores straight from the registers as its B operand (rounded to
// bf16, in the accumulator's row order) and the other side through the
// transposing LDS read, whose addressing yields the same row order.
//
// Tiles are bf16 in LDS, 128-byte rows of eight 16-byte chunks; logical chunk
// c of row R sits at physical chunk c ^ swz(R), swz(R) = 2 (R % 4) ^ bit 2 of R
// ^ 2 bit 3 of R.  Row reads (16 bytes a lane, rows R0 .. R0+15 at one
// logical chunk): swz differs across any 8 aligned consecutive rows and across
// the 8 rows of one parity among 16, so a 128- or a 256-byte bank cycle holds
// distinct chunks.  Transposing reads (8 bytes a lane, rows 4h .. 4h+3 at four
// chunks): swz / 2 takes four distinct values on those rows, and bit 2 of swz
// differs between rows of equal parity, so both bank widths stay free too.
namespace mk {

constexpr int TB = T * 128;   // bytes of one bf16 tile

__device__ __forceinline__ int swz(int row) { return (2 * (row & 3)) ^ ((row >> 2) & 1) ^ (((row >> 3) & 1) << 1); }

__device__ __forceinline__ uint32_t lds_addr(const void* ptr) {
  return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const uint8_t*)ptr);
}

// s_waitcnt vmcnt(N) through the builtin (loads only).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
}

// One dword per lane straight into LDS at m0 = lds_base (lane l writes
// lds_base + 4 l); an offset past the descriptor's range writes zero.  G tags
// the copy of the code: the issue sequences of window tiles (positions from
// arithmetic) and of global tiles (positions read from the index) must stay
// apart, or the compiler's wait for the index reads would land on both.
template <int G>
__device__ __forceinline__ void dma4(const i32x4& desc, int voff, uint32_t lds_base) {
  if constexpr (G == 0)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(desc), "s"(lds_base)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds ; global tile"
                 :
                 : "v"(voff), "s"(desc), "s"(lds_base)
                 : "memory", "m0");
}

// 16 bytes per lane into LDS at m0 = lds_base + IMM (lane l writes 16 l on);
// G as for dma4.
template <int IMM, int G>
__device__ __forceinline__ void dma16g(const i32x4& desc, int voff, uint32_t lds_base) {
  if constexpr (G == 0)
    asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(desc), "s"(lds_base), "n"(IMM)
                 : "memory", "m0", "scc");
  else
    asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds ; global tile"
                 :
                 : "v"(voff), "s"(desc), "s"(lds_base), "n"(IMM)
                 : "memory", "m0", "scc");
}

// This wave's 16 rows of a 64-row tile, straight from global memory into LDS
// at `tile` (an LDS address): lane l fills chunk l % 8 of rows R0 = 16 w + l / 8
// and R0 + 8, whose positions are p0 and p1 (negative: a zero row).  d covers
// the head's n rows.
__device__ __forceinline__ int dma_row0(int w, int lane) { return 16 * w + (lane >> 3); }

template <int G = 0>
__device__ __forceinline__ void dma_tile(const i32x4& d, uint32_t tile, int w, int lane, int p0, int p1) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(tile + w * 2048);
  const int R0 = dma_row0(w, lane);
  const int c16 = ((lane & 7) ^ swz(R0)) * 16;   // swz(R0 + 8) = swz(R0) ^ 2
  dma16g<0, G>(d, p0 >= 0 ? p0 * 128 + c16 : OOB_OFF, base);
  dma16g<1024, G>(d, p1 >= 0 ? p1 * 128 + (c16 ^ 32) : OOB_OFF, base);
}

// s_waitcnt vmcnt(0) through the builtin, which the compiler's own wait
// placement sees: after it, no load of this wave is taken as outstanding (an
// inline-asm wait would leave the compiler waiting again before the first use
// of an older load, and so also for the tile loads issued after it).
__device__ __forceinline__ void wait_all_loads() {
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt 0, expcnt 7, lgkmcnt 15: loads only
}

// Per-tile metadata of the three-slot kernels: log-sum-exp (log2 units) and
// D of the tile's rows where they count (zero elsewhere), and the bits of the
// rows or keys that count.
struct alignas(16) TMeta {
  float lse[T], dd[T];
  uint32_t okm[2], pad[2];
};

// What wave 0 stages per tile and slot, straight from global memory: the
// masks at the tile's 64 positions, and (kernels that need them) the rows'
// statistics.  Positions outside the tile read as zero: a zero local mask,
// so kind 0.
struct Stage {
  float lm[T], gm[T];
};
struct StageS {
  float lm[T], gm[T], lse[T], dd[T];
};

template <typename S>
__device__ __forceinline__ uint8_t stage_kind(const S& sg, int t) {
  if (sg.lm[t] == 0.0f) return 0;
  return sg.gm[t] != 0.0f ? 1 : 2;
}

// A or B fragment c of row `row` of a [row][d] tile
__device__ __forceinline__ bf16x8 frag_row(const uint8_t* tile, int row, int h, int c) {
  return *reinterpret_cast<const bf16x8*>(tile + row * 128 + (((4 * h + c) ^ swz(row)) * 16));
}

// The four fragments of one row in global memory (zeros for pos < 0).
__device__ __forceinline__ void row_frags(bf16x8 (&f)[4], const uint8_t* head, int pos, int h) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (pos >= 0) v = *reinterpret_cast<const uint4*>(head + (int64_t)pos * 128 + (32 * h + 8 * c) * 2);
    f[c] = __builtin_bit_cast(bf16x8, v);
  }
}

// A fragment of X^T for d block db and k-chunk c2 (rows of the tile at
// `tile`): lane l gets X[row(j)][32 db + l % 32] for rows 16 c2 + 4 h + j
// (j < 4) and 16 c2 + 8 + 4 h + j - 4 (j >= 4).  Every row read by a lane has
// row % 4 = e and (row / 4) % 2 = h; bit 3 of the row tells the two reads
// apart (their swizzles differ by 2).
__device__ __forceinline__ bf16x8 frag_tr(const uint8_t* tile, int c2, int db, int lane) {
  const int h = lane >> 5, g1 = (lane >> 4) & 1, e = (lane >> 2) & 3, q = lane & 3;
  const int chunk = (4 * db + 2 * g1 + (q >> 1)) ^ (2 * e) ^ h;
  const uint8_t* a = tile + c2 * 2048 + (4 * h + e) * 128 + (q & 1) * 8;
  const s16x4 lo = tr_read(a + chunk * 16);
  const s16x4 hi = tr_read(a + 1024 + (chunk ^ 2) * 16);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// B fragment for k-chunk c2 taken from an accumulator (its rows 16 c2 ..).
__device__ __forceinline__ bf16x8 acc_frag(const f32x16& x, int c2) {
  bf16x8 f;
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = (__bf16)x[8 * c2 + j];
  return f;
}

__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// The same fragments for either 16-bit storage type S (bf16 or fp16): the
// reads move raw 16-bit values, so a bf16-typed fragment is reinterpreted; the
// accumulator's values are rounded to S.
template <typename S>
__device__ __forceinline__ svec<S, 8> as_frag(const bf16x8& f) {
  return __builtin_bit_cast(svec<S, 8>, f);
}
template <typename S>
__device__ __forceinline__ void row_frags_s(svec<S, 8> (&f)[4], const uint8_t* head, int pos, int h) {
  bf16x8 r[4];
  row_frags(r, head, pos, h);
#pragma unroll
  for (int c = 0; c < 4; ++c) f[c] = as_frag<S>(r[c]);
}
template <typename S>
__device__ __forceinline__ svec<S, 8> acc_frag_s(const f32x16& x, int c2) {
  svec<S, 8> f;
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = (S)x[8 * c2 + j];
  return f;
}

// Row pieces of a [.][64] gradient held as two d-block accumulators (element
// (d, l % 32)) to global memory: lane writes d = 32 db + 8 a + 4 h .. +3.
__device__ __forceinline__ void store_dT(uint8_t* rowptr, const f32x16 (&x)[2], float mul, int h) {
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      bf16x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (__bf16)(x[db][4 * a + e] * mul);
      *reinterpret_cast<bf16x4*>(rowptr + (32 * db + 8 * a + 4 * h) * 2) = v;
    }
}

// store_dT rounding to either 16-bit storage type S.
template <typename S>
__device__ __forceinline__ void store_dT_s(uint8_t* rowptr, const f32x16 (&x)[2], float mul, int h) {
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      svec<S, 4> v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (S)(x[db][4 * a + e] * mul);
      *reinterpret_cast<svec<S, 4>*>(rowptr + (32 * db + 8 * a + 4 * h) * 2) = v;
    }
}

// <dO, O> of a row whose dO fragments are at hand (both half-lanes get it),
// for either 16-bit storage type S.
template <typename S>
__device__ __forceinline__ float row_dot_s(const svec<S, 8> (&df)[4], const uint8_t* O, int pos, int h) {
  svec<S, 8> of[4];
  row_frags_s<S>(of, O, pos, h);
  float a = 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) a = fmaf((float)df[c][e], (float)of[c][e], a);
  return half_sum(a);
}

// <dO, O> of a row whose dO fragments are at hand (both half-lanes get it).
__device__ __forceinline__ float row_dot(const bf16x8 (&df)[4], const uint8_t* O, int pos, int h) {
  bf16x8 of[4];
  row_frags(of, O, pos, h);
  float a = 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) a = fmaf((float)df[c][e], (float)of[c][e], a);
  return half_sum(a);
}

// Tile metadata fetched one tile ahead: raw values in registers (threads
// 0..63, one tile row or key each), turned into a Meta entry once they land.
struct MetaRegs {
  int pos;
  float lv, gv;   // masks at pos (zero when pos < 0)
  float2 st;      // (log-sum-exp, D) at pos, where wanted
};

// lm, gm: the batch row's masks; st: the head's statistics (or null).
__device__ __forceinline__ void fetch_meta(MetaRegs& mr, const float* lm, const float* gm, const float2* st,
                                           int pos, bool masks) {
  mr.pos = pos;
  mr.lv = 0.0f;
  mr.gv = 0.0f;
  mr.st = make_float2(0.0f, 0.0f);
  if (pos >= 0) {
    if (masks) {
      mr.lv = lm[pos];
      mr.gv = gm[pos];
    }
    if (st) mr.st = st[pos];
  }
}

// Kind of the fetched position: from the masks, or 1 (global) without them.
__device__ __forceinline__ uint8_t meta_kind(const MetaRegs& mr, bool masks) {
  if (mr.pos < 0) return 0;
  if (!masks) return 1;
  if (mr.lv == 0.0f) return 0;
  return mr.gv != 0.0f ? 1 : 2;
}

constexpr int DQ_SMEM = 6 * TB + 3 * (int)sizeof(Stage);   // three K, V tile pairs, three Stage records
constexpr int DKV_SMEM = 4 * TB + 2 * 64 * 64 * 4;  // two Q, dO tile pairs; the row quadrants' sums

constexpr float LOG2E = 1.4426950408889634f;

// Wave 0 (threads 0..63, one tile row or key each) publishes which entries of
// the tile count: bit t of the 64-bit word.
template <typename M>
__device__ __forceinline__ void publish_bits(M& mt, bool counts) {
  const uint64_t bits = __ballot(counts);
  if (threadIdx.x == 0) {
    mt.okm[0] = (uint32_t)bits;
    mt.okm[1] = (uint32_t)(bits >> 32);
  }
}

// True when every (row, key) pair of window tile kt (64 rows against keys
// 64 kt - r .. of the same subsequence) lies within r: the pairs' key index
// minus row index, plus r, spans 64 kt - 63 .. 64 kt + 63, inside [0, 2r].
__device__ __forceinline__ bool interior_tile(int kt, int r) { return kt >= 1 && T * kt + 63 <= 2 * r; }

// One key tile of a running-softmax dQ^T sum.  Lane = row, with the row's
// fragments qf, df (B operands) and D = <dO, O>; the wave takes keys 32 kq ..
// of the tile: S^T = K Q^T, dP^T = V dO^T.  Bit k of M: key 32 kq + k counts
// for the lane's row (ignored when `full`, wave-uniform: every key counts).
// Exponents are in log2 units, c = scale log2(e); the running offset m (the
// same in both halves of the row) moves only when a score passes it by more
// than TAU, so the terms stay below 2^TAU; l is this lane's share of the sum.
template <typename S>
__device__ __forceinline__ void dq_tile(f32x16 (&acc)[2], float& m, float& l, const uint8_t* tK,
                                        const uint8_t* tV, const svec<S, 8> (&qf)[4], const svec<S, 8> (&df)[4],
                                        float dsum, uint32_t M, bool full, float c, int kq, int lane) {
  const int h32 = lane >> 5, qi = lane & 31;
  f32x16 x = {}, e = {};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x = mfma16(as_frag<S>(frag_row(tK, 32 * kq + qi, h32, k)), qf[k], x);
    e = mfma16(as_frag<S>(frag_row(tV, 32 * kq + qi, h32, k)), df[k], e);
  }
  if (!full) mask_half(x, M, h32);
  float mr = x[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) mr = fmaxf(mr, x[i]);
  const float mx = half_max(mr) * c;
  if (__any(mx > m + TAU)) {
    const float mn = mx > m + TAU ? mx : m;
    const float alpha = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - mn);
    l *= alpha;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
    m = mn;
  }
  const float mu = m == -INFINITY ? 0.0f : m;   // no counted key yet: every term is exp2(-inf) = 0
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float pr = __builtin_amdgcn_exp2f(fmaf(x[i], c, -mu));
    l += pr;
    x[i] = pr * (e[i] - dsum);
  }
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2) {
    const svec<S, 8> bs = acc_frag_s<S>(x, c2);
#pragma unroll
    for (int db = 0; db < 2; ++db) acc[db] = mfma16(as_frag<S>(frag_tr(tK + 32 * kq * 128, c2, db, lane)), bs, acc[db]);
  }
}

// Merges the two key quadrants' running sums of each row (offsets m in log2
// units): the kq = 1 waves hand theirs over through LDS.  Returns true in the
// kq = 0 waves, whose acc, m and l then hold the row's (l summed over both
// halves of the row).
__device__ __forceinline__ bool merge_key_quadrants(f32x16 (&acc)[2], float& m, float& l, float* xch, int rq,
                                                    int kq, int lane) {
  l = half_sum(l);
  __syncthreads();
  // [rq][8 float4 of acc][lane], then [rq][lane] (m, l): consecutive lanes at
  // consecutive addresses
  float4* xa = reinterpret_cast<float4*>(xch) + rq * 8 * 64 + lane;
  float2* xm = reinterpret_cast<float2*>(xch + 2 * 8 * 64 * 4) + rq * 64 + lane;
  if (kq == 1) {
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        xa[(4 * db + a) * 64] = make_float4(acc[db][4 * a], acc[db][4 * a + 1], acc[db][4 * a + 2], acc[db][4 * a + 3]);
    *xm = make_float2(m, l);
  }
  __syncthreads();
  if (kq != 0) return false;
  const float2 ml = *xm;
  const float m2 = ml.x, l2 = ml.y;
  const float mm = fmaxf(m, m2);
  const float a1 = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - mm);
  const float a2 = m2 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m2 - mm);
  l = l * a1 + l2 * a2;
  m = mm;
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const float4 v = xa[(4 * db + a) * 64];
      acc[db][4 * a] = acc[db][4 * a] * a1 + v.x * a2;
      acc[db][4 * a + 1] = acc[db][4 * a + 1] * a1 + v.y * a2;
      acc[db][4 * a + 2] = acc[db][4 * a + 2] * a1 + v.z * a2;
      acc[db][4 * a + 3] = acc[db][4 * a + 3] * a1 + v.w * a2;
    }
  return true;
}

// dQ of the 64 rows I0 .. of residue class rho of (b, h), in one pass over the
// key tiles (the window's, then the global keys') with a running softmax per
// row: dQ = scale (sum_k e^(s_k - m) (dP_k - D) K_k) / (sum_k e^(s_k - m)),
// m the running maximum.  Also writes zero dQ rows for the block's non-local
// rows, zero dQg rows for its non-global rows, and (log-sum-exp, D) of its
// local rows.
// The row's global-index list comes from the compaction, which publishes the
// epoch and the row's global count in one word.  With CF the
// compaction runs in this launch (the first workgroups, cp): thread 0 polls
// the word in the prologue (in the round trip of the first tiles) and, when
// that came too early, again before the first global tile is issued; the
// count reaches the other threads through LDS across the loop's barrier, and
// the list is read with coherent loads after it.  Without it the compaction
// was an earlier launch and the first poll sees the word.
template <bool CF, typename S>
__device__ void dq_local(const BwParams& p, const Params& cp, int b, int h, int rho, int blk, uint8_t* sm,
                         TMeta (&tm)[3]) {
  // LDS: three slots of (K tile, V tile), then three Stage records; the
  // merge of the key quadrants reuses the slots once the tiles are done
  Stage* stg = reinterpret_cast<Stage*>(sm + 6 * TB);
  float* xch = reinterpret_cast<float*>(sm);
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, rq = w & 1, kq = w >> 1;
  const int h32 = lane >> 5, qi = lane & 31;
  const int n = p.n, s = p.head_stride[h], r = p.r;
  const int nr = (n - rho + s - 1) / s;
  const int I0 = blk * T;
  const int64_t bh = (int64_t)b * p.H + h;
  const int64_t hoff = bh * n * 128;
  const int32_t* gidx = p.gidx + (int64_t)b * n;
  const int nwin = (T + 2 * r + T - 1) / T;
  // the global count and with it the tile count, once the compaction is seen
  __shared__ int s_g;
  uint64_t seen = 0;
  if (CF && t == 0) seen = coherent_load64(cp.ready_cnt + b);
  int g = 0, ntot = nwin;
  if constexpr (!CF) {
    g = p.gcnt[b];
    if (g > p.max_global) g = p.max_global;
    ntot = nwin + (g + T - 1) / T;
  }
  // thread 0, ahead of a barrier: the row's count into s_g (-1: the wait gave
  // up, bounded as in wait_ready, and the fault word is set)
  auto resolve = [&]() {
    if (t != 0) return;
    int spins = 0;
    while ((int32_t)(seen >> 32) != cp.epoch) {
      if (++spins > cp.spin_limit) {
        atomicOr(cp.fault, 1);
        s_g = -1;
        return;
      }
      __builtin_amdgcn_s_sleep(2);
      seen = coherent_load64(cp.ready_cnt + b);
    }
    s_g = (int)(uint32_t)seen;
  };
  // every thread, behind that barrier
  auto adopt = [&]() {
    g = s_g;
    if (g < 0) return false;
    if (g > p.max_global) g = p.max_global;
    ntot = nwin + (g + T - 1) / T;
    return true;
  };
  auto key_pos = [&](int kt, int R) {
    if (kt < nwin) {
      const int jp = I0 - r + T * kt + R;
      return jp >= 0 && jp < nr ? rho + jp * s : -1;
    }
    const int idx = T * (kt - nwin) + R;
    if (idx >= g) return -1;
    if constexpr (CF)
      return coherent_load(gidx + idx);
    else
      return gidx[idx];
  };
  const i32x4 dK = make_desc(p.K + hoff, n * 128);
  const i32x4 dV = make_desc(p.V + hoff, n * 128);
  const i32x4 dLm = make_desc(p.lmask + (int64_t)b * n, n * 4);
  const i32x4 dGm = make_desc(p.gmask + (int64_t)b * n, n * 4);
  const uint32_t lds0 = lds_addr(sm);
  const uint32_t ldsg = lds_addr(stg);
  // tile kt into slot kt % 3: every wave its 16 rows of K and V (4 loads),
  // wave 0 also the masks at the 64 key positions (2 loads)
  auto issue = [&](auto gtag, int kt, int slot) {
    constexpr int G = decltype(gtag)::value;
    const int R0 = dma_row0(w, lane);
    const int p0 = key_pos(kt, R0), p1 = key_pos(kt, R0 + 8);
    const uint32_t buf = lds0 + slot * 2 * TB;
    dma_tile<G>(dK, buf, w, lane, p0, p1);
    dma_tile<G>(dV, buf + TB, w, lane, p0, p1);
    if (w == 0) {
      const int pm = key_pos(kt, lane);
      const int off = pm >= 0 ? pm * 4 : OOB_OFF;
      const uint32_t sb = __builtin_amdgcn_readfirstlane(ldsg + slot * (uint32_t)sizeof(Stage));
      dma4<G>(dLm, off, sb + offsetof(Stage, lm));
      dma4<G>(dGm, off, sb + offsetof(Stage, gm));
    }
  };
  auto prefetch = [&](int kt, int slot) {
    if (kt < nwin)
      issue(std::integral_constant<int, 0>{}, kt, slot);
    else
      issue(std::integral_constant<int, 1>{}, kt, slot);
  };
  prefetch(0, 0);

  const int row = 32 * rq + qi;
  const int rps = I0 + row < nr ? rho + (I0 + row) * s : -1;
  const uint8_t rkd = kind_of(p, b, rps);
  const bool rlocal = rkd == 2;
  svec<S, 8> qf[4], df[4];
  row_frags_s<S>(qf, p.Q + hoff, rps, h32);
  row_frags_s<S>(df, p.dO + hoff, rps, h32);
  const float dsum = row_dot_s<S>(df, p.O + hoff, rps, h32);
  // every load so far has landed, tile 0 too; from here on the only loads in
  // flight are the tiles' (and, at global tiles, the index reads)
  wait_all_loads();
  // the count is needed before the first global tile is issued: at the
  // iteration that issues tile nwin (kt = nwin - 2), or here when that is tile 1
  if (CF && nwin < 2) {
    resolve();
    __syncthreads();
    if (!adopt()) return;
  }
  if (ntot > 1) prefetch(1, 1);

  const float c = p.scale * LOG2E;
  const bool all_local = __all(rlocal);
  float m = -INFINITY, l = 0.0f;
  f32x16 acc[2] = {};
  int cur = 0;
  for (int kt = 0; kt < ntot; ++kt) {
    const bool win = kt < nwin;
    // tile kt landed; tile kt + 1 may still be in flight
    if (kt + 1 < ntot) {
      if (w == 0)
        wait_vm<6>();
      else
        wait_vm<4>();
    } else {
      wait_vm<0>();
    }
    if (t < T) {
      // window tiles count local keys; the global tiles count global keys
      publish_bits(tm[cur], stage_kind(stg[cur], t) == (win ? 2 : 1));
    }
    if (CF && kt + 2 == nwin) resolve();
    __syncthreads();
    if (CF && kt + 2 == nwin && !adopt()) {
      wait_vm<0>();   // no load into this workgroup's LDS outlives it
      return;
    }
    if (kt + 2 < ntot) prefetch(kt + 2, cur == 0 ? 2 : cur - 1);
    const uint8_t* tK = sm + cur * 2 * TB;
    // in the window, key 32 kq + k is within r of the row when key index
    // minus row index, plus r, lies in [0, 2r]: k in [a, a + 2r]
    const uint32_t kb = tm[cur].okm[kq];
    const int a = row - T * kt - 32 * kq;
    const uint32_t M = rlocal ? kb & (win ? bit_range_v(a, a + 2 * r + 1) : 0xFFFFFFFFu) : 0u;
    const bool full = all_local && kb == 0xFFFFFFFFu && (!win || interior_tile(kt, r));
    dq_tile<S>(acc, m, l, tK, tK + TB, qf, df, dsum, M, full, c, kq, lane);
    cur = cur == 2 ? 0 : cur + 1;
  }
  if (merge_key_quadrants(acc, m, l, xch, rq, kq, lane) && rps >= 0) {
    const float L = l, mm = m;
    const float mul = rlocal && L > 0.0f ? p.scale / L : 0.0f;
    store_dT_s<S>(p.dQ + hoff + (int64_t)rps * 128, acc, mul, h32);
    if (rkd != 1) {
      const f32x16 z[2] = {};
      store_dT_s<S>(p.dQg + hoff + (int64_t)rps * 128, z, 0.0f, h32);
    }
    if (rlocal && h32 == 0) p.stats[bh * n + rps] = make_float2(L > 0.0f ? mm + log2f(L) : INFINITY, dsum);
  }
}

// dK^T, dV^T accumulators of one key quadrant (lane = key) over the rows of
// a 64-row tile: S = Q K^T and dP = dO V^T with rows in the accumulator's
// order; P = exp2(c S - lse2(row)) (c = scale log2(e), lse2 the row's
// log-sum-exp in log2 units, from mt.lse), dS = P (dP - D).  Bit k of M: row
// 32 rq + k counts for the lane's key (ignored when `full`: every row counts).
template <typename S, typename MT>
__device__ __forceinline__ void kv_tile(f32x16 (&dk)[2], f32x16 (&dv)[2], const uint8_t* tQ,
                                        const uint8_t* tdO, const svec<S, 8> (&kf)[4], const svec<S, 8> (&vf)[4],
                                        const MT& mt, float c, int rq, int lane, uint32_t M, bool full) {
  const int h32 = lane >> 5, qi = lane & 31;
  f32x16 x = {}, e = {};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x = mfma16(as_frag<S>(frag_row(tQ, 32 * rq + qi, h32, k)), kf[k], x);
    e = mfma16(as_frag<S>(frag_row(tdO, 32 * rq + qi, h32, k)), vf[k], e);
  }
  if (!full) mask_half(x, M, h32);
  f32x16 pp;
  const int r0 = 32 * rq + 4 * h32;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float4 ls = *reinterpret_cast<const float4*>(mt.lse + r0 + 8 * j);
    const float4 dd = *reinterpret_cast<const float4*>(mt.dd + r0 + 8 * j);
    const float lsv[4] = {ls.x, ls.y, ls.z, ls.w}, ddv[4] = {dd.x, dd.y, dd.z, dd.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = 4 * j + u;
      const float pr = __builtin_amdgcn_exp2f(fmaf(x[i], c, -lsv[u]));
      pp[i] = pr;
      x[i] = pr * (e[i] - ddv[u]);
    }
  }
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2) {
    const svec<S, 8> bs = acc_frag_s<S>(x, c2), bp = acc_frag_s<S>(pp, c2);
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      dk[db] = mfma16(as_frag<S>(frag_tr(tQ + 32 * rq * 128, c2, db, lane)), bs, dk[db]);
      dv[db] = mfma16(as_frag<S>(frag_tr(tdO + 32 * rq * 128, c2, db, lane)), bp, dv[db]);
    }
  }
}

// Adds the row-quadrant-1 waves' dK^T, dV^T to the row-quadrant-0 waves'
// (through LDS); returns true in the waves that then hold the sums.
__device__ __forceinline__ bool sum_row_quadrants(f32x16 (&dk)[2], f32x16 (&dv)[2], float* xch, int rq,
                                                  int kq, int lane) {
  __syncthreads();
  // [kq][16 float4 of dk, dv][lane]: consecutive lanes at consecutive addresses
  float4* x = reinterpret_cast<float4*>(xch) + kq * 16 * 64 + lane;
  if (rq == 1) {
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        x[(4 * db + a) * 64] = make_float4(dk[db][4 * a], dk[db][4 * a + 1], dk[db][4 * a + 2], dk[db][4 * a + 3]);
        x[(8 + 4 * db + a) * 64] = make_float4(dv[db][4 * a], dv[db][4 * a + 1], dv[db][4 * a + 2], dv[db][4 * a + 3]);
      }
  }
  __syncthreads();
  if (rq != 0) return false;
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const float4 u = x[(4 * db + a) * 64], v = x[(8 + 4 * db + a) * 64];
      dk[db][4 * a] += u.x;
      dk[db][4 * a + 1] += u.y;
      dk[db][4 * a + 2] += u.z;
      dk[db][4 * a + 3] += u.w;
      dv[db][4 * a] += v.x;
      dv[db][4 * a + 1] += v.y;
      dv[db][4 * a + 2] += v.z;
      dv[db][4 * a + 3] += v.w;
    }
  return true;
}

// dK, dV (window part) and dKg, dVg of the 64 keys J0 .. of residue class rho
// of (b, h), in one pass over the row tiles: the window's (with Q and the
// local rows' statistics), then the global rows' (with Qg and theirs).  The
// statistics must be in place.
template <bool MF, typename S>
__device__ void dkv_local(const BwParams& p, int b, int h, int rho, int blk, uint8_t* sm, Meta (&mt)[2]) {
  float* xch = reinterpret_cast<float*>(sm + 4 * TB);
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, kq = w & 1, rq = w >> 1;
  const int h32 = lane >> 5, qi = lane & 31;
  const int n = p.n, s = p.head_stride[h], r = p.r;
  const int nr = (n - rho + s - 1) / s;
  const int J0 = blk * T;
  const int64_t bh = (int64_t)b * p.H + h;
  const int64_t hoff = bh * n * 128;
  int g = p.gcnt[b];
  if (g > p.max_global) g = p.max_global;
  const int32_t* gidx = p.gidx + (int64_t)b * n;
  const int nwin = (T + 2 * r + T - 1) / T;
  const int ntot = nwin + (g + T - 1) / T;
  auto row_pos = [&](int qt, int R) {
    if (qt < nwin) {
      const int ip = J0 - r + T * qt + R;
      return ip >= 0 && ip < nr ? rho + ip * s : -1;
    }
    const int idx = T * (qt - nwin) + R;
    return idx < g ? gidx[idx] : -1;
  };
  const i32x4 dQd = make_desc(p.Q + hoff, n * 128);
  const i32x4 dQgd = make_desc(p.Qg + hoff, n * 128);
  const i32x4 dOd = make_desc(p.dO + hoff, n * 128);
  const uint32_t lds0 = lds_addr(sm);
  const float* lm = p.lmask + (int64_t)b * n;
  const float* gm = p.gmask + (int64_t)b * n;
  const float2* st = p.stats + bh * n;
  MetaRegs mr;
  auto prefetch = [&](int qt) {
    const int R0 = dma_row0(w, lane);
    const int p0 = row_pos(qt, R0), p1 = row_pos(qt, R0 + 8);
    const int pm = t < T ? row_pos(qt, t) : -1;
    const uint32_t buf = lds0 + (qt & 1) * 2 * TB;
    dma_tile(qt < nwin ? dQd : dQgd, buf, w, lane, p0, p1);
    dma_tile(dOd, buf + TB, w, lane, p0, p1);
    if (t < T) fetch_meta(mr, lm, gm, qt < nwin || !MF ? st : nullptr, pm, qt < nwin);
  };
  if (ntot > 0) prefetch(0);
  // With MF the merge of the chunk sums runs beside this workgroup
  // in the same launch, so the global rows' statistics are not in p.stats:
  // (log-sum-exp, D) of global row `idx` of (b, h) is combined here from the
  // chunks' (max, sum of exp) pairs (log2 units), 32 chunks a round trip
  // (16-byte loads, all in flight together); D was stored beside the first
  // chunk's dQg sum.  Those of the first two global tiles' rows are fetched
  // in the round trip of the first window tile.
  auto global_stat = [&](int idx) {
    if (idx >= g) return make_float2(0.0f, 0.0f);
    const int64_t row = bh * p.max_global + idx;
    const float4* src = reinterpret_cast<const float4*>(p.gml + row * p.gspad * 2);
    const float dd = p.gq[row * p.gsplit * 68 + 66];
    float mm = -INFINITY, L = 0.0f;
    for (int c0 = 0; 2 * c0 < p.gsplit; c0 += 16) {
      float4 v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = 2 * (c0 + j) < p.gsplit ? src[c0 + j] : make_float4(0.f, 0.f, 0.f, 0.f);
      float e[32], f[32];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const bool a0 = 2 * (c0 + j) < p.gsplit, a1 = 2 * (c0 + j) + 1 < p.gsplit;
        e[2 * j] = a0 ? v[j].x : -INFINITY;
        f[2 * j] = a0 ? v[j].y : 0.0f;
        e[2 * j + 1] = a1 ? v[j].z : -INFINITY;
        f[2 * j + 1] = a1 ? v[j].w : 0.0f;
      }
      float gmx = mm;
#pragma unroll
      for (int j = 0; j < 32; ++j) gmx = fmaxf(gmx, e[j]);
      if (gmx == -INFINITY) continue;   // no real key in these chunks yet
      L = mm == -INFINITY ? 0.0f : L * __builtin_amdgcn_exp2f(mm - gmx);
#pragma unroll
      for (int j = 0; j < 32; ++j) L = fmaf(f[j], e[j] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(e[j] - gmx), L);
      mm = gmx;
    }
    return make_float2(L > 0.0f ? mm + log2f(L) : INFINITY, dd);
  };

  const int key = 32 * kq + qi;
  const int kps = J0 + key < nr ? rho + (J0 + key) * s : -1;
  const uint8_t kkd = kind_of(p, b, kps);
  svec<S, 8> kf[4], vf[4];
  row_frags_s<S>(kf, p.K + hoff, kps, h32);
  row_frags_s<S>(vf, p.V + hoff, kps, h32);
  const bool gfold = MF && t < T;
  const float2 gst0 = gfold && ntot > nwin ? global_stat(t) : make_float2(0.0f, 0.0f);
  const float2 gst1 = gfold && ntot > nwin + 1 ? global_stat(T + t) : make_float2(0.0f, 0.0f);
  f32x16 dk[2] = {}, dv[2] = {};
  const float c = p.scale * LOG2E;
  const bool all_win = __all(kkd == 2), all_real = __all(kkd != 0);
  auto finish_window = [&]() {
    // global keys' dK, dV come from the chunk sums
    if (sum_row_quadrants(dk, dv, xch, rq, kq, lane) && kps >= 0 && kkd != 1) {
      store_dT_s<S>(p.dK + hoff + (int64_t)kps * 128, dk, p.scale, h32);
      store_dT_s<S>(p.dV + hoff + (int64_t)kps * 128, dv, 1.0f, h32);
    }
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      dk[db] = f32x16{};
      dv[db] = f32x16{};
    }
    row_frags_s<S>(kf, p.Kg + hoff, kps, h32);
    row_frags_s<S>(vf, p.Vg + hoff, kps, h32);
  };
  auto step = [&](int qt) {
    const int cur = qt & 1;
    wait_all_loads();
    const bool win = qt < nwin;
    if (t < T) {
      // window tiles count local rows; the global tiles count global rows
      const uint8_t kd = meta_kind(mr, win);
      const bool keep = kd == (win ? 2 : 1);
      const float2 sv = win || !MF
                            ? mr.st
                            : (qt == nwin ? gst0 : qt == nwin + 1 ? gst1 : global_stat(T * (qt - nwin) + t));
      mt[cur].rkind[t] = kd;
      mt[cur].lse[t] = keep ? sv.x : 0.0f;
      mt[cur].dd[t] = keep ? sv.y : 0.0f;
      publish_bits(mt[cur], keep);
    }
    __syncthreads();
    if (qt + 1 < ntot) prefetch(qt + 1);
    const uint8_t* tQ = sm + cur * 2 * TB;
    // in the window, row 32 rq + k is within r of the key when key index
    // minus row index, plus r, lies in [0, 2r]: k in [bk - 2r, bk]
    const uint32_t rb = mt[cur].okm[rq];
    const int bk = 2 * r + key - T * qt - 32 * rq;
    const uint32_t M = win ? (kkd == 2 ? rb & bit_range_v(bk - 2 * r, bk + 1) : 0u) : (kkd != 0 ? rb : 0u);
    const bool full = rb == 0xFFFFFFFFu && (win ? all_win && interior_tile(qt, r) : all_real);
    kv_tile<S>(dk, dv, tQ, tQ + TB, kf, vf, mt[cur], c, rq, lane, M, full);
  };
  // the window's row tiles; then the global rows' tiles (Kg, Vg fragments)
  for (int qt = 0; qt < nwin; ++qt) step(qt);
  finish_window();
  for (int qt = nwin; qt < ntot; ++qt) step(qt);
  if (sum_row_quadrants(dk, dv, xch, rq, kq, lane) && kps >= 0) {
    store_dT_s<S>(p.dKg + hoff + (int64_t)kps * 128, dk, p.scale, h32);
    store_dT_s<S>(p.dVg + hoff + (int64_t)kps * 128, dv, 1.0f, h32);
  }
}

// Sums over one chunk of positions P0 .. P1-1 for global tile gt of (b, h):
// (1) the global rows' dQg^T = Kg^T dS^T with a chunk-local running max (an
// online softmax over the chunk's real keys), with the max and the sum of
// exponentials, and (2) the global keys' dK^T = Q^T dS, dV^T = dO^T P over the
// chunk's local rows (their statistics must be in place).  One pass over the
// chunk's tiles for each, the tiles double-buffered as in the dQ kernel.
constexpr int GS_SMEM = 4 * TB + 2 * 64 * 64 * 4;

template <typename S>
__device__ void global_chunk(const BwParams& p, int b, int h, int gt, int sp, uint8_t* sm, Meta (&mt)[2]) {
  float* xch = reinterpret_cast<float*>(sm + 4 * TB);
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int h32 = lane >> 5, qi = lane & 31;
  const int n = p.n;
  const int64_t bh = (int64_t)b * p.H + h;
  const int64_t hoff = bh * n * 128;
  int g = p.gcnt[b];
  if (g > p.max_global) g = p.max_global;
  if (T * gt >= g) return;
  const int32_t* gidx = p.gidx + (int64_t)b * n + T * gt;   // this tile's global positions
  const int P0 = sp * p.gchunk;
  const int P1 = P0 + p.gchunk < n ? P0 + p.gchunk : n;
  const int nt = (P1 - P0 + T - 1) / T;   // tiles per part
  auto pos_of = [&](int st, int R) {
    const int ps = P0 + T * (st < nt ? st : st - nt) + R;
    return ps < P1 ? ps : -1;
  };
  const i32x4 dKg = make_desc(p.Kg + hoff, n * 128);
  const i32x4 dVg = make_desc(p.Vg + hoff, n * 128);
  const i32x4 dQd = make_desc(p.Q + hoff, n * 128);
  const i32x4 dOd = make_desc(p.dO + hoff, n * 128);
  const uint32_t lds0 = lds_addr(sm);
  const float* lm = p.lmask + (int64_t)b * n;
  const float* gm = p.gmask + (int64_t)b * n;
  const float2* stp = p.stats + bh * n;
  MetaRegs mr;
  auto prefetch = [&](int st) {
    const bool two = st >= nt;
    const int R0 = dma_row0(w, lane);
    const int p0 = pos_of(st, R0), p1 = pos_of(st, R0 + 8);
    const int pm = t < T ? pos_of(st, t) : -1;
    const uint32_t buf = lds0 + (st & 1) * 2 * TB;
    dma_tile(two ? dQd : dKg, buf, w, lane, p0, p1);
    dma_tile(two ? dOd : dVg, buf + TB, w, lane, p0, p1);
    if (t < T) fetch_meta(mr, lm, gm, two ? stp : nullptr, pm, true);
  };
  prefetch(0);
  // (1) wave w: global rows 32 (w & 1) + lane % 32 (lane = row), keys 32 (w >> 1) ..
  {
    const int rq = w & 1, kq = w >> 1;
    const int row = 32 * rq + qi;
    const int gps = T * gt + row < g ? gidx[row] : -1;
    svec<S, 8> qf[4], df[4];
    row_frags_s<S>(qf, p.Qg + hoff, gps, h32);
    row_frags_s<S>(df, p.dO + hoff, gps, h32);
    const float dsum = row_dot_s<S>(df, p.O + hoff, gps, h32);
    const float c = p.scale * LOG2E;
    const bool all_live = __all(gps >= 0);
    float m = -INFINITY, l = 0.0f;
    f32x16 acc[2] = {};
    for (int st = 0; st < nt; ++st) {
      const int cur = st & 1;
      wait_all_loads();
      if (t < T) {
        const uint8_t kd = meta_kind(mr, true);
        mt[cur].kkind[t] = kd;
        publish_bits(mt[cur], kd != 0);   // every real key
      }
      __syncthreads();
      prefetch(st + 1);   // the first tile of part (2) follows the last of part (1)
      const uint8_t* tK = sm + cur * 2 * TB;
      const uint32_t kb = mt[cur].okm[kq];
      dq_tile<S>(acc, m, l, tK, tK + TB, qf, df, dsum, gps >= 0 ? kb : 0u, all_live && kb == 0xFFFFFFFFu, c, kq,
              lane);
    }
    if (merge_key_quadrants(acc, m, l, xch, rq, kq, lane) && gps >= 0) {
      float* dst = p.gq + ((bh * p.max_global + T * gt + row) * p.gsplit + sp) * 68;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int a = 0; a < 4; ++a)
          *reinterpret_cast<float4*>(dst + 32 * db + 8 * a + 4 * h32) =
              make_float4(acc[db][4 * a], acc[db][4 * a + 1], acc[db][4 * a + 2], acc[db][4 * a + 3]);
      if (h32 == 0) {
        *reinterpret_cast<float4*>(dst + 64) = make_float4(m, l, dsum, 0.0f);
        *reinterpret_cast<float2*>(p.gml + ((bh * p.max_global + T * gt + row) * p.gspad + sp) * 2) =
            make_float2(m, l);
      }
    }
  }
  // (2) wave w: global keys 32 (w & 1) + lane % 32 (lane = key), rows 32 (w >> 1) ..
  {
    const int kq = w & 1, rq = w >> 1;
    const int key = 32 * kq + qi;
    const int kps = T * gt + key < g ? gidx[key] : -1;
    svec<S, 8> kf[4], vf[4];
    row_frags_s<S>(kf, p.K + hoff, kps, h32);
    row_frags_s<S>(vf, p.V + hoff, kps, h32);
    f32x16 dk[2] = {}, dv[2] = {};
    const float c = p.scale * LOG2E;
    const bool all_live = __all(kps >= 0);
    for (int st = nt; st < 2 * nt; ++st) {
      const int cur = st & 1;
      wait_all_loads();
      if (t < T) {
        const uint8_t kd = meta_kind(mr, true);
        mt[cur].rkind[t] = kd;
        mt[cur].lse[t] = kd == 2 ? mr.st.x : 0.0f;
        mt[cur].dd[t] = kd == 2 ? mr.st.y : 0.0f;
        publish_bits(mt[cur], kd == 2);   // every local row
      }
      __syncthreads();
      if (st + 1 < 2 * nt) prefetch(st + 1);
      const uint8_t* tQ = sm + cur * 2 * TB;
      const uint32_t rb = mt[cur].okm[rq];
      kv_tile<S>(dk, dv, tQ, tQ + TB, kf, vf, mt[cur], c, rq, lane, kps >= 0 ? rb : 0u,
              all_live && rb == 0xFFFFFFFFu);
    }
    if (sum_row_quadrants(dk, dv, xch, rq, kq, lane) && kps >= 0) {
      float* dst = p.gk + ((bh * p.max_global + T * gt + key) * p.gsplit + sp) * 128;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int d = 32 * db + 8 * a + 4 * h32;
          *reinterpret_cast<float4*>(dst + d) =
              make_float4(dk[db][4 * a], dk[db][4 * a + 1], dk[db][4 * a + 2], dk[db][4 * a + 3]);
          *reinterpret_cast<float4*>(dst + 64 + d) =
              make_float4(dv[db][4 * a], dv[db][4 * a + 1], dv[db][4 * a + 2], dv[db][4 * a + 3]);
        }
    }
  }
}

// Neighbouring blocks of a head share most of their window tiles: the
// logical block order keeps them on one XCD, whose L2 then serves the overlap.
// With CF, workgroups 0 .. B-1, first in dispatch order, compact
// batch row blockIdx.x (cp: the forward's compaction and its publication)
// before their own rows.
template <bool CF, typename S>
__global__ __launch_bounds__(NTH) void dq_kernel(BwParams p, Params cp) {
  extern __shared__ __attribute__((aligned(16))) uint8_t sm[];
  __shared__ TMeta mt[3];
  if (CF && (int)blockIdx.x < p.B) {
    compact_row(cp, blockIdx.x, sm);
    __syncthreads();
  }
  int b, h, rho, blk;
  decode_block(p, xcd_remap(blockIdx.x, gridDim.x), b, h, rho, blk);
  dq_local<CF, S>(p, cp, b, h, rho, blk, sm, mt);
}

template <typename S>
__device__ void global_merge(const BwParams& p, int64_t item, int lane);

// With MF, the workgroups past the B * blocks_per_b key blocks (in the last
// round's spare slots) merge the global rows' and keys' chunk sums
// (global_merge, one item a wave): work of its own, which no key block waits
// for (those combine the global rows' statistics themselves).
template <bool MF, typename S>
__global__ __launch_bounds__(NTH) void dkv_kernel(BwParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t sm[];
  __shared__ Meta mt[2];
  const int nblk = p.B * p.blocks_per_b;
  if (MF && (int)blockIdx.x >= nblk) {
    global_merge<S>(p, (int64_t)((int)blockIdx.x - nblk) * (NTH / 64) + (threadIdx.x >> 6), threadIdx.x & 63);
    return;
  }
  int b, h, rho, blk;
  decode_block(p, xcd_remap(blockIdx.x, nblk), b, h, rho, blk);
  dkv_local<MF, S>(p, b, h, rho, blk, sm, mt);
}

template <typename S>
__global__ __launch_bounds__(NTH) void global_chunk_kernel(BwParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t sm[];
  __shared__ Meta mt[2];
  const int sp = blockIdx.x % p.gsplit, rest = blockIdx.x / p.gsplit;
  const int gt = rest % p.ntg, bh = rest / p.ntg;
  global_chunk<S>(p, bh / p.H, bh % p.H, gt, sp, sm, mt);
}

// One wave per (b, h, global index): combines the chunk sums (offsets in log2
// units) into dQg and the global key's dK, dV, and (unless the merge runs
// beside the dK/dV work, which combines them itself) the row's log-sum-exp
// (log2 units) and D.  Lane = d.
template <typename S>
__device__ void global_merge(const BwParams& p, int64_t item, int lane) {
  if (item >= (int64_t)p.B * p.H * p.max_global) return;
  const int gi = (int)(item % p.max_global);
  const int64_t bh = item / p.max_global;
  const int b = (int)(bh / p.H);
  int g = p.gcnt[b];
  if (g > p.max_global) g = p.max_global;
  if (gi >= g) return;
  const int n = p.n;
  const int pos = p.gidx[(int64_t)b * n + gi];
  const float* q = p.gq + item * p.gsplit * 68;
  // lane-parallel maximum over the chunks, then independent loads per chunk
  float mm = -INFINITY;
  for (int sp = lane; sp < p.gsplit; sp += 64) mm = fmaxf(mm, q[sp * 68 + 64]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mm = fmaxf(mm, __shfl_xor(mm, o));
  float L = 0.0f, a = 0.0f;
#pragma unroll 8
  for (int sp = 0; sp < p.gsplit; ++sp) {
    const float m = q[sp * 68 + 64];
    const float f = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - mm);
    L = fmaf(q[sp * 68 + 65], f, L);
    a = fmaf(q[sp * 68 + lane], f, a);
  }
  const float* k = p.gk + item * p.gsplit * 128;
  float sk = 0.0f, sv = 0.0f;
#pragma unroll 8
  for (int sp = 0; sp < p.gsplit; ++sp) {
    sk += k[sp * 128 + lane];
    sv += k[sp * 128 + 64 + lane];
  }
  const int64_t ro = (bh * n + pos) * 128 + lane * 2;
  *reinterpret_cast<S*>(p.dQg + ro) = (S)(L > 0.0f ? p.scale * a / L : 0.0f);
  *reinterpret_cast<S*>(p.dK + ro) = (S)(p.scale * sk);
  *reinterpret_cast<S*>(p.dV + ro) = (S)sv;
  if (!p.merge_fold) {
    const float dov = (float)*reinterpret_cast<const S*>(p.dO + ro);
    float dd = dov * (float)*reinterpret_cast<const S*>(p.O + ro);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) dd += __shfl_xor(dd, o);
    if (lane == 0) p.stats[bh * n + pos] = make_float2(L > 0.0f ? mm + log2f(L) : INFINITY, dd);
  }
}

template <typename S>
__global__ __launch_bounds__(NTH) void global_merge_kernel(BwParams p) {
  global_merge<S>(p, (int64_t)blockIdx.x * (NTH / 64) + (threadIdx.x >> 6), threadIdx.x & 63);
}

}  // namespace mk

// The forward's compaction workgroup, on its own.
__global__ __launch_bounds__(NT) void compact_kernel(Params p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t csm[];
  if ((int)blockIdx.x < p.B) compact_row(p, blockIdx.x, csm);
}

}  // namespace bw
}  // namespace lwk
