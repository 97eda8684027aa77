// Causal variant of the window attention, forward and backward, 16-bit
// storage (bf16 or fp16), on the matrix cores.
//
// "LongFormer: The Long-Document Transformer" (reading notes), section
// Implementation: an autoregressive language model uses the dilated sliding
// window, with window sizes that may change from layer to layer, and no global
// attention; "Longformer模型深度解析与应用指南", mask composition: a local mask and a
// causal mask combine by intersection.  Row i of a head with stride s and reach
// r = w/2 attends to the valid taps i - k*s, 0 <= k <= r; a padded row's output
// is zero.  Every (b, h) and residue class is independent, as in the
// bidirectional window.
//
// One workgroup per 64-row block of one residue class (the backward's block
// order), four waves each owning a 32 x 32 quadrant (rows x keys) of every
// 64 x 64 tile pair.  The key tiles of a block cover the subsequence indices
// I0 - r .. I0 + 63; tiles arrive two ahead through direct-to-LDS loads into
// three slots, with their local masks (the same pipeline as the backward's dQ
// kernel).  Per tile: S^T = K Q^T, a running softmax per row (exponents in
// log2 units, offset moved lazily), O^T += V^T P^T; interior tiles of
// all-valid blocks skip the mask.  At the end the two key quadrants merge and
// O = (sum) / l.
#pragma once

namespace lwk {
namespace cz {

using namespace bw::mk;
using bw::T;
using bw::NTH;

struct CzParams {
  const uint8_t *Q, *K, *V;
  uint8_t* O;
  const float* lmask;           // [B,n]
  const int32_t* head_stride;   // [H]
  const int32_t* head_blk;      // [H+1] prefix over heads of 64-row blocks (all residue classes)
  int B, H, n, r, blocks_per_b;
  float scale;
};

// One key tile of the running-softmax sum O^T += V^T P^T (lane = row, with the
// row's Q fragments qf; keys 32 kq .. of the tile).  Bit k of M: key
// 32 kq + k counts for the lane's row (ignored when `full`).
// S: the 16-bit storage type (bf16 or fp16), the matrix cores' operand type.
template <typename S>
__device__ __forceinline__ void pv_tile(f32x16 (&acc)[2], float& m, float& l, const uint8_t* tK,
                                        const uint8_t* tV, const svec<S, 8> (&qf)[4], uint32_t M, bool full,
                                        float c, int kq, int lane) {
  const int h32 = lane >> 5, qi = lane & 31;
  f32x16 x = {};
#pragma unroll
  for (int k = 0; k < 4; ++k) x = mfma16(as_frag<S>(frag_row(tK, 32 * kq + qi, h32, k)), qf[k], x);
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
  const float mu = m == -INFINITY ? 0.0f : m;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    x[i] = __builtin_amdgcn_exp2f(fmaf(x[i], c, -mu));
    l += x[i];
  }
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2) {
    const svec<S, 8> pb = acc_frag_s<S>(x, c2);
#pragma unroll
    for (int db = 0; db < 2; ++db)
      acc[db] = mfma16(as_frag<S>(frag_tr(tV + 32 * kq * 128, c2, db, lane)), pb, acc[db]);
  }
}

// True when every (row, key) pair of tile kt lies within the causal reach:
// row index minus key index, R + r - 64 kt - k, spans r - 64 kt - 63 ..
// r - 64 kt + 63, inside [0, r].
__device__ __forceinline__ bool interior(int kt, int r) { return kt >= 1 && T * kt + 63 <= r; }

constexpr int SMEM = 6 * TB + 3 * (int)sizeof(bw::mk::Stage);   // three K, V tile pairs, three Stage records

template <typename S>
__device__ void causal_block(const CzParams& p, int b, int h, int rho, int blk, uint8_t* sm, TMeta (&tm)[3]) {
  bw::mk::Stage* stg = reinterpret_cast<bw::mk::Stage*>(sm + 6 * TB);
  float* xch = reinterpret_cast<float*>(sm);
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, rq = w & 1, kq = w >> 1;
  const int h32 = lane >> 5, qi = lane & 31;
  const int n = p.n, s = p.head_stride[h], r = p.r;
  const int nr = (n - rho + s - 1) / s;
  const int I0 = blk * T;
  const int64_t bh = (int64_t)b * p.H + h;
  const int64_t hoff = bh * n * 128;
  const int nt = (r + T + T - 1) / T;   // key tiles: subsequence indices I0 - r .. I0 + 63
  auto key_pos = [&](int kt, int R) {
    const int jp = I0 - r + T * kt + R;
    return jp >= 0 && jp < nr ? rho + jp * s : -1;
  };
  const i32x4 dK = make_desc(p.K + hoff, n * 128);
  const i32x4 dV = make_desc(p.V + hoff, n * 128);
  const i32x4 dLm = make_desc(p.lmask + (int64_t)b * n, n * 4);
  const uint32_t lds0 = lds_addr(sm);
  const uint32_t ldsg = lds_addr(stg);
  // tile kt into a slot: every wave its 16 rows of K and V (4 loads), wave 0
  // also the local mask at the 64 key positions (1 load)
  auto prefetch = [&](int kt, int slot) {
    const int R0 = dma_row0(w, lane);
    const int p0 = key_pos(kt, R0), p1 = key_pos(kt, R0 + 8);
    const uint32_t buf = lds0 + slot * 2 * TB;
    dma_tile(dK, buf, w, lane, p0, p1);
    dma_tile(dV, buf + TB, w, lane, p0, p1);
    if (w == 0) {
      const int pm = key_pos(kt, lane);
      const uint32_t sb = __builtin_amdgcn_readfirstlane(ldsg + slot * (uint32_t)sizeof(bw::mk::Stage));
      dma4<0>(dLm, pm >= 0 ? pm * 4 : OOB_OFF, sb + offsetof(bw::mk::Stage, lm));
    }
  };
  prefetch(0, 0);

  const int row = 32 * rq + qi;
  const int rps = I0 + row < nr ? rho + (I0 + row) * s : -1;
  const bool rvalid = rps >= 0 && p.lmask[(int64_t)b * n + rps] != 0.0f;
  svec<S, 8> qf[4];
  row_frags_s<S>(qf, p.Q + hoff, rps, h32);
  wait_all_loads();   // the row's fragments and tile 0
  if (nt > 1) prefetch(1, 1);

  const float c = p.scale * LOG2E;
  const bool all_valid = __all(rvalid);
  float m = -INFINITY, l = 0.0f;
  f32x16 acc[2] = {};
  int cur = 0;
  for (int kt = 0; kt < nt; ++kt) {
    // tile kt landed; tile kt + 1 may still be in flight
    if (kt + 1 < nt) {
      if (w == 0)
        wait_vm<5>();
      else
        wait_vm<4>();
    } else {
      wait_vm<0>();
    }
    if (t < T) publish_bits(tm[cur], stg[cur].lm[t] != 0.0f);
    __syncthreads();
    if (kt + 2 < nt) prefetch(kt + 2, cur == 0 ? 2 : cur - 1);
    const uint8_t* tK = sm + cur * 2 * TB;
    // key 32 kq + k counts when its index is within [row - 64 kt, row - 64 kt + r]
    // of the tile's first key (row index minus key index in [0, r])
    const uint32_t kb = tm[cur].okm[kq];
    const int a = row - T * kt - 32 * kq;
    const uint32_t M = rvalid ? kb & bit_range_v(a, a + r + 1) : 0u;
    const bool full = all_valid && kb == 0xFFFFFFFFu && interior(kt, r);
    pv_tile<S>(acc, m, l, tK, tK + TB, qf, M, full, c, kq, lane);
    cur = cur == 2 ? 0 : cur + 1;
  }
  if (merge_key_quadrants(acc, m, l, xch, rq, kq, lane) && rps >= 0)
    store_dT_s<S>(p.O + hoff + (int64_t)rps * 128, acc, rvalid && l > 0.0f ? 1.0f / l : 0.0f, h32);
}

template <typename S>
__global__ __launch_bounds__(NTH) void causal_kernel(CzParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t sm[];
  __shared__ TMeta tm[3];
  int b, h, rho, blk;
  bw::decode_block(p, xcd_remap(blockIdx.x, gridDim.x), b, h, rho, blk);
  causal_block<S>(p, b, h, rho, blk, sm, tm);
}

// ---------------------------------------------------------------------------
// Backward of the causal variant: the chain rule through the definition above
// (dS = P (dP - D), D = <dO, O>; dQ = scale dS K, dK = scale dS^T Q,
// dV = P^T dO), with the backward's tile steps.  Two launches: dQ with the
// rows' statistics (log-sum-exp in log2 units, D), then dK, dV.

struct CzBwParams {
  const uint8_t *Q, *K, *V, *O, *dO;
  uint8_t *dQ, *dK, *dV;
  const float* lmask;
  float2* stats;                // [B,H,n]
  const int32_t* head_stride;
  const int32_t* head_blk;
  int B, H, n, r, blocks_per_b;
  float scale;
};

// dQ of the 64 rows I0 .. of residue class rho: key tiles I0 - r .. I0 + 63,
// running softmax (the dQ kernel's tile step); stats of the valid rows.
template <typename S>
__device__ void causal_dq_block(const CzBwParams& p, int b, int h, int rho, int blk, uint8_t* sm,
                                TMeta (&tm)[3]) {
  bw::mk::Stage* stg = reinterpret_cast<bw::mk::Stage*>(sm + 6 * TB);
  float* xch = reinterpret_cast<float*>(sm);
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, rq = w & 1, kq = w >> 1;
  const int h32 = lane >> 5, qi = lane & 31;
  const int n = p.n, s = p.head_stride[h], r = p.r;
  const int nr = (n - rho + s - 1) / s;
  const int I0 = blk * T;
  const int64_t bh = (int64_t)b * p.H + h;
  const int64_t hoff = bh * n * 128;
  const int nt = (r + T + T - 1) / T;
  auto key_pos = [&](int kt, int R) {
    const int jp = I0 - r + T * kt + R;
    return jp >= 0 && jp < nr ? rho + jp * s : -1;
  };
  const i32x4 dK = make_desc(p.K + hoff, n * 128);
  const i32x4 dV = make_desc(p.V + hoff, n * 128);
  const i32x4 dLm = make_desc(p.lmask + (int64_t)b * n, n * 4);
  const uint32_t lds0 = lds_addr(sm);
  const uint32_t ldsg = lds_addr(stg);
  auto prefetch = [&](int kt, int slot) {
    const int R0 = dma_row0(w, lane);
    const int p0 = key_pos(kt, R0), p1 = key_pos(kt, R0 + 8);
    const uint32_t buf = lds0 + slot * 2 * TB;
    dma_tile(dK, buf, w, lane, p0, p1);
    dma_tile(dV, buf + TB, w, lane, p0, p1);
    if (w == 0) {
      const int pm = key_pos(kt, lane);
      const uint32_t sb = __builtin_amdgcn_readfirstlane(ldsg + slot * (uint32_t)sizeof(bw::mk::Stage));
      dma4<0>(dLm, pm >= 0 ? pm * 4 : OOB_OFF, sb + offsetof(bw::mk::Stage, lm));
    }
  };
  prefetch(0, 0);
  const int row = 32 * rq + qi;
  const int rps = I0 + row < nr ? rho + (I0 + row) * s : -1;
  const bool rvalid = rps >= 0 && p.lmask[(int64_t)b * n + rps] != 0.0f;
  svec<S, 8> qf[4], df[4];
  row_frags_s<S>(qf, p.Q + hoff, rps, h32);
  row_frags_s<S>(df, p.dO + hoff, rps, h32);
  const float dsum = row_dot_s<S>(df, p.O + hoff, rps, h32);
  wait_all_loads();
  if (nt > 1) prefetch(1, 1);
  const float c = p.scale * LOG2E;
  const bool all_valid = __all(rvalid);
  float m = -INFINITY, l = 0.0f;
  f32x16 acc[2] = {};
  int cur = 0;
  for (int kt = 0; kt < nt; ++kt) {
    if (kt + 1 < nt) {
      if (w == 0)
        wait_vm<5>();
      else
        wait_vm<4>();
    } else {
      wait_vm<0>();
    }
    if (t < T) publish_bits(tm[cur], stg[cur].lm[t] != 0.0f);
    __syncthreads();
    if (kt + 2 < nt) prefetch(kt + 2, cur == 0 ? 2 : cur - 1);
    const uint8_t* tK = sm + cur * 2 * TB;
    const uint32_t kb = tm[cur].okm[kq];
    const int a = row - T * kt - 32 * kq;
    const uint32_t M = rvalid ? kb & bit_range_v(a, a + r + 1) : 0u;
    const bool full = all_valid && kb == 0xFFFFFFFFu && interior(kt, r);
    dq_tile<S>(acc, m, l, tK, tK + TB, qf, df, dsum, M, full, c, kq, lane);
    cur = cur == 2 ? 0 : cur + 1;
  }
  if (merge_key_quadrants(acc, m, l, xch, rq, kq, lane) && rps >= 0) {
    store_dT_s<S>(p.dQ + hoff + (int64_t)rps * 128, acc, rvalid && l > 0.0f ? p.scale / l : 0.0f, h32);
    if (rvalid && h32 == 0) p.stats[bh * n + rps] = make_float2(l > 0.0f ? m + log2f(l) : INFINITY, dsum);
  }
}

// dK, dV of the 64 keys J0 .. of residue class rho: row tiles J0 .. J0 + 63 + r
// (the rows at or after a key, within r), the dK/dV kernel's tile step with
// the rows' statistics.
template <typename S>
__device__ void causal_dkv_block(const CzBwParams& p, int b, int h, int rho, int blk, uint8_t* sm,
                                 TMeta (&tm)[3]) {
  bw::mk::StageS* stg = reinterpret_cast<bw::mk::StageS*>(sm + 6 * TB);
  float* xch = reinterpret_cast<float*>(sm);
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, kq = w & 1, rq = w >> 1;
  const int h32 = lane >> 5, qi = lane & 31;
  const int n = p.n, s = p.head_stride[h], r = p.r;
  const int nr = (n - rho + s - 1) / s;
  const int J0 = blk * T;
  const int64_t bh = (int64_t)b * p.H + h;
  const int64_t hoff = bh * n * 128;
  const int nt = (r + T + T - 1) / T;
  auto row_pos = [&](int qt, int R) {
    const int ip = J0 + T * qt + R;
    return ip < nr ? rho + ip * s : -1;
  };
  const i32x4 dQd = make_desc(p.Q + hoff, n * 128);
  const i32x4 dOd = make_desc(p.dO + hoff, n * 128);
  const i32x4 dLm = make_desc(p.lmask + (int64_t)b * n, n * 4);
  const i32x4 dSt = make_desc(p.stats + bh * n, n * 8);
  const uint32_t lds0 = lds_addr(sm);
  const uint32_t ldsg = lds_addr(stg);
  auto prefetch = [&](int qt, int slot) {
    const int R0 = dma_row0(w, lane);
    const int p0 = row_pos(qt, R0), p1 = row_pos(qt, R0 + 8);
    const uint32_t buf = lds0 + slot * 2 * TB;
    dma_tile(dQd, buf, w, lane, p0, p1);
    dma_tile(dOd, buf + TB, w, lane, p0, p1);
    if (w == 0) {
      const int pm = row_pos(qt, lane);
      const uint32_t sb = __builtin_amdgcn_readfirstlane(ldsg + slot * (uint32_t)sizeof(bw::mk::StageS));
      dma4<0>(dLm, pm >= 0 ? pm * 4 : OOB_OFF, sb + offsetof(bw::mk::StageS, lm));
      dma4<0>(dSt, pm >= 0 ? pm * 8 : OOB_OFF, sb + offsetof(bw::mk::StageS, lse));
      dma4<0>(dSt, pm >= 0 ? pm * 8 + 4 : OOB_OFF, sb + offsetof(bw::mk::StageS, dd));
    }
  };
  prefetch(0, 0);
  const int key = 32 * kq + qi;
  const int kps = J0 + key < nr ? rho + (J0 + key) * s : -1;
  const bool kvalid = kps >= 0 && p.lmask[(int64_t)b * n + kps] != 0.0f;
  svec<S, 8> kf[4], vf[4];
  row_frags_s<S>(kf, p.K + hoff, kps, h32);
  row_frags_s<S>(vf, p.V + hoff, kps, h32);
  wait_all_loads();
  if (nt > 1) prefetch(1, 1);
  const float c = p.scale * LOG2E;
  const bool all_valid = __all(kvalid);
  f32x16 dk[2] = {}, dv[2] = {};
  int cur = 0;
  for (int qt = 0; qt < nt; ++qt) {
    if (qt + 1 < nt) {
      if (w == 0)
        wait_vm<7>();
      else
        wait_vm<4>();
    } else {
      wait_vm<0>();
    }
    if (t < T) {
      const bool keep = stg[cur].lm[t] != 0.0f;
      tm[cur].lse[t] = keep ? stg[cur].lse[t] : 0.0f;
      tm[cur].dd[t] = keep ? stg[cur].dd[t] : 0.0f;
      publish_bits(tm[cur], keep);
    }
    __syncthreads();
    if (qt + 2 < nt) prefetch(qt + 2, cur == 0 ? 2 : cur - 1);
    const uint8_t* tQ = sm + cur * 2 * TB;
    // row 32 rq + k counts when row index minus key index, 64 qt + 32 rq + k - key,
    // lies in [0, r]: k in [b0, b0 + r]
    const uint32_t rb = tm[cur].okm[rq];
    const int b0 = key - T * qt - 32 * rq;
    const uint32_t M = kvalid ? rb & bit_range_v(b0, b0 + r + 1) : 0u;
    const bool full = all_valid && rb == 0xFFFFFFFFu && interior(qt, r);
    kv_tile<S>(dk, dv, tQ, tQ + TB, kf, vf, tm[cur], c, rq, lane, M, full);
    cur = cur == 2 ? 0 : cur + 1;
  }
  if (sum_row_quadrants(dk, dv, xch, rq, kq, lane) && kps >= 0) {
    store_dT_s<S>(p.dK + hoff + (int64_t)kps * 128, dk, kvalid ? p.scale : 0.0f, h32);
    store_dT_s<S>(p.dV + hoff + (int64_t)kps * 128, dv, kvalid ? 1.0f : 0.0f, h32);
  }
}

constexpr int BW_DQ_SMEM = 6 * TB + 3 * (int)sizeof(bw::mk::Stage);
constexpr int BW_DKV_SMEM = 6 * TB + 3 * (int)sizeof(bw::mk::StageS);

template <typename S>
__global__ __launch_bounds__(NTH) void causal_dq_kernel(CzBwParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t sm[];
  __shared__ TMeta tm[3];
  int b, h, rho, blk;
  bw::decode_block(p, xcd_remap(blockIdx.x, gridDim.x), b, h, rho, blk);
  causal_dq_block<S>(p, b, h, rho, blk, sm, tm);
}

template <typename S>
__global__ __launch_bounds__(NTH) void causal_dkv_kernel(CzBwParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t sm[];
  __shared__ TMeta tm[3];
  int b, h, rho, blk;
  bw::decode_block(p, xcd_remap(blockIdx.x, gridDim.x), b, h, rho, blk);
  causal_dkv_block<S>(p, b, h, rho, blk, sm, tm);
}

}  // namespace cz
}  // namespace lwk
