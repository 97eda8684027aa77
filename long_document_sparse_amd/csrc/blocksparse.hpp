// Block-sparse attention over 64 x 64 blocks, 16-bit storage (bf16 or fp16), on the matrix
// cores.
//
// xFormers' attention-mask notes (gitcode xformers page): a per-head layout
// over 64 x 64 blocks of the score matrix says which query block sees which
// key block, and masks compose by intersection (a layout and a causal mask).
// Row i of head h sees key j when block (i / 64, j / 64) is in the layout, j's
// local mask is nonzero and, with `causal`, j <= i; a padded row, or a row that
// sees no key, outputs zero.
//
// The layout arrives as CSR per (head, query block): the key blocks of query
// block qb of head h are cols[rowptr[h nb + qb] .. rowptr[h nb + qb + 1]).
// One workgroup per (b, h, query block), four waves of 32 x 32 quadrants;
// the block's column list goes to LDS first, then the listed K/V tiles stream
// two ahead through direct-to-LDS loads (the causal kernel's pipeline and
// tile step).  Tiles whose keys are all valid and, with `causal`, lie wholly
// before the query block skip the mask.
#pragma once

namespace lwk {
namespace bsp {

using namespace bw::mk;
using bw::T;
using bw::NTH;

struct BsParams {
  const uint8_t *Q, *K, *V;
  uint8_t* O;
  const float* lmask;       // [B,n]
  const int32_t* rowptr;    // [H*nb + 1]
  const int32_t* cols;      // [nnz]
  int B, H, n, nb, causal;
  int nnz;                  // entries of cols: every list is clamped into [0, nnz)
  float scale;
};

// dynamic LDS: three K, V tile pairs, three Stage records, then nb column indices
constexpr int SMEM_BASE = 6 * TB + 3 * (int)sizeof(bw::mk::Stage);

template <typename S>
__device__ void bs_block(const BsParams& p, int b, int h, int qb, uint8_t* sm, TMeta (&tm)[3]) {
  bw::mk::Stage* stg = reinterpret_cast<bw::mk::Stage*>(sm + 6 * TB);
  int32_t* colsl = reinterpret_cast<int32_t*>(sm + SMEM_BASE);
  float* xch = reinterpret_cast<float*>(sm);
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, rq = w & 1, kq = w >> 1;
  const int h32 = lane >> 5, qi = lane & 31;
  const int n = p.n, nb = p.nb;
  const int64_t bh = (int64_t)b * p.H + h;
  const int64_t hoff = bh * n * 128;
  // a malformed CSR (negative, decreasing or out-of-range offsets) reads no
  // column entry outside cols[0, nnz)
  const int rbeg = min(max(p.rowptr[h * nb + qb], 0), p.nnz);
  const int rend = min(max(p.rowptr[h * nb + qb + 1], 0), p.nnz);
  int nt = rend - rbeg;
  nt = nt < 0 ? 0 : (nt > nb ? nb : nt);
  for (int j = t; j < nt; j += NTH) colsl[j] = p.cols[rbeg + j];
  const int P0 = T * qb;
  const int row = 32 * rq + qi;
  const int rps = P0 + row < n ? P0 + row : -1;
  const bool rvalid = rps >= 0 && p.lmask[(int64_t)b * n + rps] != 0.0f;
  svec<S, 8> qf[4];
  row_frags_s<S>(qf, p.Q + hoff, rps, h32);
  wait_all_loads();   // the column list, the row's fragments
  __syncthreads();    // the column list is visible

  auto key_pos = [&](int kt, int R) {
    const int j = T * colsl[kt] + R;
    return j >= 0 && j < n ? j : -1;
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
  if (nt > 0) prefetch(0, 0);
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
    const int kb = colsl[kt];
    const uint32_t vb = tm[cur].okm[kq];
    // causal: key blocks before the query block count whole, its own block up
    // to the row (key 32 kq + k with k <= row - 32 kq), later ones not at all
    uint32_t cm = 0xFFFFFFFFu;
    if (p.causal) cm = kb < qb ? 0xFFFFFFFFu : (kb == qb ? bit_range_v(0, row - 32 * kq + 1) : 0u);
    const uint32_t M = rvalid ? vb & cm : 0u;
    const bool full = all_valid && vb == 0xFFFFFFFFu && (!p.causal || kb < qb);
    cz::pv_tile<S>(acc, m, l, tK, tK + TB, qf, M, full, c, kq, lane);
    cur = cur == 2 ? 0 : cur + 1;
  }
  if (merge_key_quadrants(acc, m, l, xch, rq, kq, lane) && rps >= 0)
    store_dT_s<S>(p.O + hoff + (int64_t)rps * 128, acc, rvalid && l > 0.0f ? 1.0f / l : 0.0f, h32);
}

// Neighbouring query blocks of a head list mostly the same key blocks: the
// logical order keeps them on one XCD.
// S: the 16-bit storage type (bf16 or fp16).
template <typename S>
__global__ __launch_bounds__(NTH) void blocksparse_kernel(BsParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t sm[];
  __shared__ TMeta tm[3];
  const int lb = xcd_remap(blockIdx.x, gridDim.x);
  const int qb = lb % p.nb, bh = lb / p.nb;
  bs_block<S>(p, bh / p.H, bh % p.H, qb, sm, tm);
}

}  // namespace bsp
}  // namespace lwk
