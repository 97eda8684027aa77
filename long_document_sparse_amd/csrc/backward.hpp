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
  float2* stats;                // [B,H,n] (log-sum-exp, D) of every non-padded row
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
  constexpr int RB = D * Lay<BF>::ELT;
  const int t = threadIdx.x, row = t >> 2, q = t & 3;
  const int ps = pos[row];
  float v[16];
  if (ps >= 0) {
    load16<BF>(head + (int64_t)ps * RB + q * 16 * Lay<BF>::ELT, v);
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
  constexpr int RB = D * Lay<BF>::ELT;
  const int t = threadIdx.x, row = t >> 2, q = t & 3;
  const int ps = pos[row];
  if (ps < 0 || !keep[row]) return;
  float v[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) v[e] = src[row * LS + 16 * q + e];
  store16<BF>(head + (int64_t)ps * RB + q * 16 * Lay<BF>::ELT, v);
}

// Shared per-tile bookkeeping in LDS.
struct Meta {
  int rpos[T], kpos[T];
  uint8_t rkind[T], kkind[T], rkeep[T], kkeep[T];
  float lse[T], dd[T];
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
  constexpr int RB = D * Lay<BF>::ELT;
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
  constexpr int RB = D * Lay<BF>::ELT;
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
  constexpr int RB = D * Lay<BF>::ELT;
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
  constexpr int RB = D * Lay<BF>::ELT;
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
__device__ __forceinline__ void decode_block(const BwParams& p, int lb, int& b, int& h, int& rho, int& blk) {
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

// The forward's compaction workgroup, on its own.
__global__ __launch_bounds__(NT) void compact_kernel(Params p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t csm[];
  if ((int)blockIdx.x < p.B) compact_row(p, blockIdx.x, csm);
}

}  // namespace bw
}  // namespace lwk
