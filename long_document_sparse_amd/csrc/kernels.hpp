// kernels.hpp -- gfx950 kernels of the Longformer window + global attention
// forward.  Included once, by lwattn.hip.
//
// Three kernels run per forward, in order on one stream:
//   compact_kernel  one workgroup per batch row: padding / global flags per
//                   position and the ascending global-index list (wave ballot
//                   + prefix count), the FasterTransformer guide's
//                   global_idx / global_token_nums partition.
//   attn_kernel     one grid with two kinds of workgroups:
//                   * global-row workgroups: the global queries of one
//                     (batch, head) against one slice of all keys under
//                     Qg/Kg/Vg, written as an unnormalised softmax partial
//                     (running max, running sum, weighted value sum);
//                   * band workgroups: 128 query rows of one (batch, head,
//                     residue class of the dilation) against their window
//                     keys and the global keys under Q/K/V, one online
//                     softmax per row, the output row written directly.
//   merge_kernel    log-sum-exp merge of the global-row partials.
//
// Method sources: "LongFormer: The Long-Document Transformer" notes, sections
// "Sliding Window", "Dilated Sliding Window" and "Global Attention" (banded
// Q.K^T: only a fixed set of diagonals is computed); FasterTransformer
// Longformer encoder guide, "compute flow" (masked softmax per row kind,
// padded query rows zeroed).
//
// MFMA tiling.  A wave owns 32 query rows.  For a tile of 32 keys it forms
// S^T = K * Q^T with v_mfma_f32_32x32x16_bf16 (or v_mfma_f32_32x32x2_f32 for
// float32 storage), so each lane holds 16 scores of ONE query: lane l has
// query l%32 and keys 8*(r/4) + 4*(l/32) + r%4 in register r.  Row statistics
// are per-lane reductions plus one exchange with lane l^32.  The probabilities
// stay in registers and are the B operand of O^T += V^T * P^T; V is stored
// transposed in LDS so that each lane reads runs of 4 keys at one d.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace lwk {

constexpr int D = 64;          // head dim (fixed)
constexpr int KT = 32;         // keys per tile
constexpr int NW = 4;          // waves per workgroup
constexpr int NT = 64 * NW;    // threads per workgroup
constexpr int ROWS_WG = 32 * NW;
constexpr float TAU = 8.0f;    // lazy-rescale threshold, log2 units
constexpr float M_INIT = -1e30f;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

struct Params {
  const uint8_t *Q, *K, *V, *Qg, *Kg, *Vg;
  uint8_t* O;
  const float* lmask;
  const float* gmask;
  uint8_t* flags;          // [B][n]: bit0 real token, bit1 global token
  int32_t* gidx;           // [B][n]
  int32_t* gcnt;           // [B]
  int32_t* status;         // [B]: 1 if the row has more than max_global globals
  float* part_o;           // [B][H][nqt][nsplit][32][64]
  float* part_ml;          // [B][H][nqt][nsplit][32][2]
  const int32_t* head_stride;  // [H]: dilation gap + 1
  const int32_t* head_blk;     // [H+1]: prefix of band workgroups per batch row
  int32_t B, H, n, r;      // r = min(window/2, n)
  int32_t max_global, nqt, nqg, nsplit, ksplit;
  int32_t n_glob_wg;       // padded to a multiple of 8
  int32_t n_band_wg;
  int32_t blocks_per_b;    // head_blk[H]
  float c;                 // scale * log2(e)
};

// ---------------------------------------------------------------------------
// Layout of one LDS tile slot.
template <bool BF>
struct Lay;
template <>
struct Lay<true> {             // bf16 storage
  static constexpr int ELT = 2;
  static constexpr int CH = 8;           // 16-byte chunks per 64-element row
  static constexpr int KROW = 144;       // K row stride (128 + 16 pad: conflict-free b128 reads)
  static constexpr int VROW = 72;        // V^T row stride: 32 keys * 2 B + 8 pad
  static constexpr int KBYTES = KT * KROW;
  static constexpr int VBYTES = D * VROW;
};
template <>
struct Lay<false> {            // float32 storage
  static constexpr int ELT = 4;
  static constexpr int CH = 16;
  static constexpr int KROW = 272;
  static constexpr int VROW = 272;       // V kept [key][d]
  static constexpr int KBYTES = KT * KROW;
  static constexpr int VBYTES = KT * VROW;
};
template <bool BF>
struct SlotLay {
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = Lay<BF>::KBYTES;
  static constexpr int POS_OFF = V_OFF + Lay<BF>::VBYTES;
  static constexpr int OK_OFF = POS_OFF + KT * 4;
  static constexpr int CLEAN_OFF = OK_OFF + KT;
  static constexpr int BYTES = (CLEAN_OFF + 4 + 15) / 16 * 16;
  static constexpr int NCH = KT * Lay<BF>::CH / NT;   // chunks per thread per array
};

// Which keys a tile holds.
enum TileMode { TM_BAND = 0, TM_GCOL = 1, TM_SLICE = 2 };
struct TileDesc {
  int mode;
  int j0;      // first key: subsequence index (band), list index (gcol), position (slice)
  int jend;    // one past the last usable j (band: nr, gcol: g, slice: slice end)
};

struct Ctx {
  const uint8_t* fl;       // flags of the batch row
  const int32_t* gi;       // gidx of the batch row
  int rho, s;              // residue class and stride (band)
};

__device__ __forceinline__ void key_pos(const TileDesc& td, const Ctx& cx, int k, int& pos, bool& ok) {
  const int jj = td.j0 + k;
  if (td.mode == TM_GCOL) {
    ok = jj < td.jend;
    pos = ok ? cx.gi[jj] : 0;
  } else if (td.mode == TM_BAND) {
    ok = jj >= 0 && jj < td.jend;
    pos = ok ? cx.rho + jj * cx.s : 0;
    ok = ok && (cx.fl[pos] & 1);
  } else {
    ok = jj < td.jend;
    pos = ok ? jj : 0;
    ok = ok && (cx.fl[pos] & 1);
  }
}

template <bool BF>
struct Stage {
  static constexpr int NCH = SlotLay<BF>::NCH;
  uint4 kr[NCH], vr[NCH];
  int pos;
  bool ok;
};

// Issue the global loads of one tile into registers.
template <bool BF>
__device__ __forceinline__ void stage_load(Stage<BF>& st, const TileDesc& td, const Ctx& cx,
                                           const uint8_t* kbase, const uint8_t* vbase) {
  constexpr int CH = Lay<BF>::CH;
  constexpr int RB = D * Lay<BF>::ELT;
  const int tid = threadIdx.x;
#pragma unroll
  for (int e = 0; e < Stage<BF>::NCH; ++e) {
    const int q = tid + NT * e;
    const int kt = q / CH, ch = q % CH;
    int pos;
    bool ok;
    key_pos(td, cx, kt, pos, ok);
    if (ok) {
      st.kr[e] = *reinterpret_cast<const uint4*>(kbase + (int64_t)pos * RB + ch * 16);
      st.vr[e] = *reinterpret_cast<const uint4*>(vbase + (int64_t)pos * RB + ch * 16);
    } else {
      st.kr[e] = make_uint4(0, 0, 0, 0);
      st.vr[e] = make_uint4(0, 0, 0, 0);
    }
  }
  if (tid < KT) key_pos(td, cx, tid, st.pos, st.ok);
}

// Write the staged registers into an LDS slot (V transposed for bf16).
template <bool BF>
__device__ __forceinline__ void stage_store(const Stage<BF>& st, uint8_t* slot) {
  using SL = SlotLay<BF>;
  constexpr int CH = Lay<BF>::CH;
  const int tid = threadIdx.x;
#pragma unroll
  for (int e = 0; e < Stage<BF>::NCH; ++e) {
    const int q = tid + NT * e;
    const int kt = q / CH, ch = q % CH;
    *reinterpret_cast<uint4*>(slot + SL::K_OFF + kt * Lay<BF>::KROW + ch * 16) = st.kr[e];
    if constexpr (BF) {
      const uint32_t w[4] = {st.vr[e].x, st.vr[e].y, st.vr[e].z, st.vr[e].w};
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint16_t hv = (uint16_t)(w[t >> 1] >> (16 * (t & 1)));
        *reinterpret_cast<uint16_t*>(slot + SL::V_OFF + (ch * 8 + t) * Lay<BF>::VROW + kt * 2) = hv;
      }
    } else {
      *reinterpret_cast<uint4*>(slot + SL::V_OFF + kt * Lay<BF>::VROW + ch * 16) = st.vr[e];
    }
  }
  if (tid < 64) {
    const bool ok = tid < KT ? st.ok : true;
    const uint64_t all = __ballot(ok);
    if (tid < KT) {
      reinterpret_cast<int32_t*>(slot + SL::POS_OFF)[tid] = st.pos;
      slot[SL::OK_OFF + tid] = ok ? 1 : 0;
    }
    if (tid == 0) *reinterpret_cast<int32_t*>(slot + SL::CLEAN_OFF) = (all == ~0ull) ? 1 : 0;
  }
}

// Query operand held in registers for the whole key loop.
template <bool BF>
struct QOp;
template <>
struct QOp<true> {
  bf16x8 q[4];   // Q[row][32*h + 8*c .. +8], c = 0..3
  __device__ void load(const uint8_t* row, bool ok, int h) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (ok) {
        uint4 v = *reinterpret_cast<const uint4*>(row + (32 * h + 8 * c) * 2);
        q[c] = __builtin_bit_cast(bf16x8, v);
      } else {
        q[c] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
      }
    }
  }
};
template <>
struct QOp<false> {
  float q[32];   // Q[row][32*h + c], c = 0..31
  __device__ void load(const uint8_t* row, bool ok, int h) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float4 v = ok ? *reinterpret_cast<const float4*>(row + (32 * h + 4 * c) * 4)
                    : make_float4(0.f, 0.f, 0.f, 0.f);
      q[4 * c + 0] = v.x;
      q[4 * c + 1] = v.y;
      q[4 * c + 2] = v.z;
      q[4 * c + 3] = v.w;
    }
  }
};

// S^T tile: 16 scores of this lane's query.
__device__ __forceinline__ f32x16 qk_tile(const QOp<true>& qo, const uint8_t* slot, int lane) {
  const int key = lane & 31, h = lane >> 5;
  f32x16 s = {};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(slot + SlotLay<true>::K_OFF +
                                                      key * Lay<true>::KROW + (4 * h + c) * 16);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qo.q[c], s, 0, 0, 0);
  }
  return s;
}
__device__ __forceinline__ f32x16 qk_tile(const QOp<false>& qo, const uint8_t* slot, int lane) {
  const int key = lane & 31, h = lane >> 5;
  f32x16 s = {};
#pragma unroll
  for (int c4 = 0; c4 < 8; ++c4) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(slot + SlotLay<false>::K_OFF +
                                                    key * Lay<false>::KROW + (8 * h + c4) * 16);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], qo.q[4 * c4 + e], s, 0, 0, 0);
  }
  return s;
}

// O^T += V^T * P^T for one tile.
__device__ __forceinline__ void pv_tile(f32x16 (&o)[2], const float (&p)[16], const uint8_t* slot,
                                        int lane, std::true_type) {
  const int h = lane >> 5, dl = lane & 31;
  const uint8_t* vt = slot + SlotLay<true>::V_OFF;
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2) {
    bf16x8 bp;
#pragma unroll
    for (int e = 0; e < 8; ++e) bp[e] = (__bf16)p[8 * c2 + e];
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const uint8_t* row = vt + (32 * db + dl) * Lay<true>::VROW;
      const bf16x4 lo = *reinterpret_cast<const bf16x4*>(row + (16 * c2 + 4 * h) * 2);
      const bf16x4 hi = *reinterpret_cast<const bf16x4*>(row + (16 * c2 + 8 + 4 * h) * 2);
      bf16x8 a;
      a[0] = lo[0]; a[1] = lo[1]; a[2] = lo[2]; a[3] = lo[3];
      a[4] = hi[0]; a[5] = hi[1]; a[6] = hi[2]; a[7] = hi[3];
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bp, o[db], 0, 0, 0);
    }
  }
}
__device__ __forceinline__ void pv_tile(f32x16 (&o)[2], const float (&p)[16], const uint8_t* slot,
                                        int lane, std::false_type) {
  const int h = lane >> 5, dl = lane & 31;
  const uint8_t* vb = slot + SlotLay<false>::V_OFF;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int key = 8 * (r >> 2) + 4 * h + (r & 3);
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const float a = *reinterpret_cast<const float*>(vb + key * Lay<false>::VROW + (32 * db + dl) * 4);
      o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, p[r], o[db], 0, 0, 0);
    }
  }
}

// Key index (0..31 within the tile) held in register r by this lane.
__device__ __forceinline__ int key_of(int r, int lane) {
  return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

struct Softmax {
  float m, l;          // running max (log2 units, lazy) and this lane's partial sum
  f32x16 o[2];         // O^T accumulators: d = 32*db + 8*(r/4) + 4*(lane/32) + r%4
  __device__ void init() {
    m = M_INIT;
    l = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) { o[0][r] = 0.f; o[1][r] = 0.f; }
  }
  // s: masked scores (excluded = -inf); returns probabilities in p.
  __device__ __forceinline__ void update(const f32x16& s, float c, float (&p)[16]) {
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(m, mx * c);
    if (__any(mnew > m + TAU)) {
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
      l *= alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) { o[0][r] *= alpha; o[1][r] *= alpha; }
      m = mnew;
    }
    float acc = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = __builtin_amdgcn_exp2f(fmaf(s[r], c, -m));
      acc += p[r];
    }
    l += acc;
  }
};

// ---------------------------------------------------------------------------
// Kernel 1: flags + global-index compaction, one workgroup per batch row.
constexpr int CT = 1024;
__global__ __launch_bounds__(CT) void compact_kernel(Params p) {
  __shared__ int wsum[CT / 64];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = p.n;
  const float* lm = p.lmask + (int64_t)b * n;
  const float* gm = p.gmask + (int64_t)b * n;
  uint8_t* fl = p.flags + (int64_t)b * n;
  int32_t* gi = p.gidx + (int64_t)b * n;
  int carry = 0;
  for (int base = 0; base < n; base += CT) {
    const int j = base + tid;
    bool v = false, g = false;
    if (j < n) {
      v = lm[j] != 0.0f;
      g = v && (gm[j] != 0.0f);
      fl[j] = (uint8_t)((v ? 1 : 0) | (g ? 2 : 0));
    }
    const uint64_t bal = __ballot(g);
    const int before = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[wave] = __popcll(bal);
    __syncthreads();
    int wpre = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < CT / 64; ++w) {
      const int c = wsum[w];
      wpre += (w < wave) ? c : 0;
      tot += c;
    }
    if (g) gi[carry + wpre + before] = j;
    carry += tot;
    __syncthreads();
  }
  for (int k = carry + tid; k < n; k += CT) gi[k] = -1;
  if (tid == 0) {
    p.gcnt[b] = carry;
    p.status[b] = carry > p.max_global ? 1 : 0;
  }
}

// ---------------------------------------------------------------------------
// Kernel 2: attention.
template <bool BF>
__device__ __forceinline__ void process_tile(const QOp<BF>& qo, Softmax& sm, const uint8_t* slot,
                                             int lane, float c, int mask_kind, int my_i, int band_j0,
                                             int r, int rho, int s) {
  using SL = SlotLay<BF>;
  f32x16 sc = qk_tile(qo, slot, lane);
  if (mask_kind != 0) {
    const uint8_t* okv = slot + SL::OK_OFF;
    const int32_t* posv = reinterpret_cast<const int32_t*>(slot + SL::POS_OFF);
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int k = key_of(rr, lane);
      bool allowed = okv[k] != 0;
      if (mask_kind == 1) {            // window tile: |i - j| <= r
        const int dj = my_i - (band_j0 + k);
        allowed = allowed && dj <= r && dj >= -r;
      } else if (mask_kind == 2) {     // global columns: skip the ones already in the window
        const int dp = posv[k] - rho;
        if (dp >= 0 && dp % s == 0) {
          const int dj = my_i - dp / s;
          allowed = allowed && !(dj <= r && dj >= -r);
        }
      }
      if (!allowed) sc[rr] = -INFINITY;
    }
  }
  float pr[16];
  sm.update(sc, c, pr);
  pv_tile(sm.o, pr, slot, lane, std::integral_constant<bool, BF>());
}

template <bool BF>
__device__ __forceinline__ void store_row4(uint8_t* dst, const float* v) {
  if constexpr (BF) {
    bf16x4 t;
    t[0] = (__bf16)v[0]; t[1] = (__bf16)v[1]; t[2] = (__bf16)v[2]; t[3] = (__bf16)v[3];
    *reinterpret_cast<bf16x4*>(dst) = t;
  } else {
    *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

template <bool BF>
__device__ void band_wg(const Params& p, int lb, uint8_t* smem) {
  using SL = SlotLay<BF>;
  constexpr int RB = D * Lay<BF>::ELT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h32 = lane >> 5, qi = lane & 31;
  const int b = lb / p.blocks_per_b;
  int rem = lb - b * p.blocks_per_b;
  int h = 0;
  while (p.head_blk[h + 1] <= rem) ++h;
  int local = rem - p.head_blk[h];
  const int s = p.head_stride[h];
  const int n = p.n;
  int rho = 0, nr = 0;
  for (rho = 0; rho < s; ++rho) {
    nr = (n - rho + s - 1) / s;
    const int nb = (nr + ROWS_WG - 1) / ROWS_WG;
    if (local < nb) break;
    local -= nb;
  }
  const int R0 = local * ROWS_WG;
  const int64_t head = ((int64_t)b * p.H + h) * (int64_t)n;
  Ctx cx;
  cx.fl = p.flags + (int64_t)b * n;
  cx.gi = p.gidx + (int64_t)b * n;
  cx.rho = rho;
  cx.s = s;

  const int my_i = R0 + 32 * wave + qi;
  const bool row_in = my_i < nr;
  const int my_pos = rho + (row_in ? my_i : 0) * s;
  const uint8_t my_fl = row_in ? cx.fl[my_pos] : 0;
  const bool wave_work = __any((my_fl & 3) == 1);

  QOp<BF> qo;
  qo.load(p.Q + (head + my_pos) * RB, row_in && ((my_fl & 3) == 1), h32);
  Softmax sm;
  sm.init();

  int g = p.gcnt[b];
  if (g > p.max_global) g = p.max_global;
  const int ngt = (g + KT - 1) / KT;
  const int r = p.r;
  const int kb = R0 - r;
  const int T = (31 + 2 * r) / 32 + 1;
  const int t_lo = (-kb - 31 > 0) ? (-kb - 31 + 31) / 32 : 0;
  int t_hi = (nr - 1 - kb) / 32;
  if (t_hi > NW - 1 + T - 1) t_hi = NW - 1 + T - 1;
  const int U = ngt + (t_hi - t_lo + 1);

  const uint8_t* kbase = p.K + head * RB;
  const uint8_t* vbase = p.V + head * RB;
  auto desc = [&](int u) {
    TileDesc td;
    if (u < ngt) {
      td.mode = TM_GCOL;
      td.j0 = u * KT;
      td.jend = g;
    } else {
      td.mode = TM_BAND;
      td.j0 = kb + (t_lo + u - ngt) * KT;
      td.jend = nr;
    }
    return td;
  };

  Stage<BF> st;
  stage_load<BF>(st, desc(0), cx, kbase, vbase);
  stage_store<BF>(st, smem);
  __syncthreads();
  for (int u = 0; u < U; ++u) {
    const bool more = u + 1 < U;
    if (more) stage_load<BF>(st, desc(u + 1), cx, kbase, vbase);
    const uint8_t* slot = smem + (u & 1) * SL::BYTES;
    if (wave_work) {
      if (u < ngt) {
        process_tile<BF>(qo, sm, slot, lane, p.c, 2, my_i, 0, r, rho, s);
      } else {
        const int t = t_lo + (u - ngt);
        const int up = t - wave;
        if (up >= 0 && up < T) {
          const int clean = *reinterpret_cast<const int32_t*>(slot + SL::CLEAN_OFF);
          const bool diag = (up == 0) || (32 * up + 31 > 2 * r);
          process_tile<BF>(qo, sm, slot, lane, p.c, (diag || !clean) ? 1 : 0, my_i, kb + t * KT, r,
                           rho, s);
        }
      }
    }
    if (more) stage_store<BF>(st, smem + ((u + 1) & 1) * SL::BYTES);
    __syncthreads();
  }

  // normalise and store this lane's half of its query row (global rows are
  // written by the merge kernel)
  const float lt = sm.l + __shfl_xor(sm.l, 32);
  if (row_in && (my_fl & 2) == 0) {
    const bool valid = (my_fl & 1) != 0;
    const float inv = valid ? 1.0f / lt : 0.0f;
    uint8_t* orow = p.O + (head + my_pos) * RB;
#pragma unroll
    for (int db = 0; db < 2; ++db) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = valid ? sm.o[db][4 * a + e] * inv : 0.0f;
        store_row4<BF>(orow + (32 * db + 8 * a + 4 * h32) * Lay<BF>::ELT, v);
      }
    }
  }
}

template <bool BF>
__device__ void global_wg(const Params& p, int lg, uint8_t* smem) {
  using SL = SlotLay<BF>;
  constexpr int RB = D * Lay<BF>::ELT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h32 = lane >> 5, qi = lane & 31;
  const int sp = lg % p.nsplit;
  int t = lg / p.nsplit;
  const int qg = t % p.nqg;
  t /= p.nqg;
  const int h = t % p.H;
  const int b = t / p.H;
  int g = p.gcnt[b];
  if (g > p.max_global) g = p.max_global;
  const int nqt_b = (g + 31) / 32;
  if (qg * NW >= nqt_b) return;                     // uniform over the workgroup
  const int qt = qg * NW + wave;
  const bool wave_work = qt < nqt_b;
  const int n = p.n;
  const int64_t head = ((int64_t)b * p.H + h) * (int64_t)n;
  Ctx cx;
  cx.fl = p.flags + (int64_t)b * n;
  cx.gi = p.gidx + (int64_t)b * n;
  cx.rho = 0;
  cx.s = 1;

  const int qidx = qt * 32 + qi;
  const bool qok = wave_work && qidx < g;
  const int qpos = qok ? cx.gi[qidx] : 0;
  QOp<BF> qo;
  qo.load(p.Qg + (head + qpos) * RB, qok, h32);
  Softmax sm;
  sm.init();

  const int j_start = sp * p.ksplit;
  int j_end = j_start + p.ksplit;
  if (j_end > n) j_end = n;
  const int U = (j_end - j_start + KT - 1) / KT;
  const uint8_t* kbase = p.Kg + head * RB;
  const uint8_t* vbase = p.Vg + head * RB;
  auto desc = [&](int u) {
    TileDesc td;
    td.mode = TM_SLICE;
    td.j0 = j_start + u * KT;
    td.jend = j_end;
    return td;
  };
  if (U > 0) {
    Stage<BF> st;
    stage_load<BF>(st, desc(0), cx, kbase, vbase);
    stage_store<BF>(st, smem);
    __syncthreads();
    for (int u = 0; u < U; ++u) {
      const bool more = u + 1 < U;
      if (more) stage_load<BF>(st, desc(u + 1), cx, kbase, vbase);
      const uint8_t* slot = smem + (u & 1) * SL::BYTES;
      if (wave_work) {
        const int clean = *reinterpret_cast<const int32_t*>(slot + SL::CLEAN_OFF);
        process_tile<BF>(qo, sm, slot, lane, p.c, clean ? 0 : 3, 0, 0, 0, 0, 1);
      }
      if (more) stage_store<BF>(st, smem + ((u + 1) & 1) * SL::BYTES);
      __syncthreads();
    }
  }
  const float lt = sm.l + __shfl_xor(sm.l, 32);
  if (qok) {
    const int64_t pidx = ((((int64_t)b * p.H + h) * p.nqt + qt) * p.nsplit + sp) * 32 + qi;
    float* po = p.part_o + pidx * D;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        *reinterpret_cast<float4*>(po + 32 * db + 8 * a + 4 * h32) =
            make_float4(sm.o[db][4 * a], sm.o[db][4 * a + 1], sm.o[db][4 * a + 2], sm.o[db][4 * a + 3]);
    if (h32 == 0) {
      p.part_ml[pidx * 2 + 0] = sm.m;
      p.part_ml[pidx * 2 + 1] = lt;
    }
  }
}

// The logical workgroup order keeps neighbouring query blocks of one head on
// one XCD (workgroups are dealt to the 8 XCDs round-robin by hardware id), so
// that their overlapping key halos are served by that XCD's L2.
__device__ __forceinline__ int xcd_remap(int pid, int count) {
  const int q = count / 8, rem = count % 8;
  const int x = pid % 8, idx = pid / 8;
  return x * q + (x < rem ? x : rem) + idx;
}

template <bool BF>
__global__ __launch_bounds__(NT, 2) void attn_kernel(Params p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int bid = blockIdx.x;
  if (bid < p.n_glob_wg) {
    const int lg = bid;
    if (lg < p.B * p.H * p.nqg * p.nsplit) global_wg<BF>(p, lg, smem);
  } else {
    band_wg<BF>(p, xcd_remap(bid - p.n_glob_wg, p.n_band_wg), smem);
  }
}

// ---------------------------------------------------------------------------
// Kernel 3: merge of the global-row partials, one workgroup per (b, h, 32 globals).
template <bool BF>
__global__ __launch_bounds__(256) void merge_kernel(Params p) {
  const int wg = blockIdx.x;
  const int qt = wg % p.nqt;
  const int bh = wg / p.nqt;
  const int b = bh / p.H;
  int g = p.gcnt[b];
  if (g > p.max_global) g = p.max_global;
  const int q = threadIdx.x >> 3, seg = threadIdx.x & 7;
  const int idx = qt * 32 + q;
  if (idx >= g) return;
  const int64_t base = ((int64_t)bh * p.nqt + qt) * p.nsplit;
  float mstar = -INFINITY;
  for (int sp = 0; sp < p.nsplit; ++sp) mstar = fmaxf(mstar, p.part_ml[((base + sp) * 32 + q) * 2]);
  float L = 0.f;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int sp = 0; sp < p.nsplit; ++sp) {
    const int64_t pi = (base + sp) * 32 + q;
    const float w = __builtin_amdgcn_exp2f(p.part_ml[pi * 2] - mstar);
    L += w * p.part_ml[pi * 2 + 1];
    const float4 a = *reinterpret_cast<const float4*>(p.part_o + pi * D + seg * 8);
    const float4 c = *reinterpret_cast<const float4*>(p.part_o + pi * D + seg * 8 + 4);
    acc[0] += w * a.x; acc[1] += w * a.y; acc[2] += w * a.z; acc[3] += w * a.w;
    acc[4] += w * c.x; acc[5] += w * c.y; acc[6] += w * c.z; acc[7] += w * c.w;
  }
  const float inv = 1.0f / L;
  for (int e = 0; e < 8; ++e) acc[e] *= inv;
  const int pos = p.gidx[(int64_t)b * p.n + idx];
  constexpr int RB = D * Lay<BF>::ELT;
  uint8_t* orow = p.O + ((int64_t)bh * p.n + pos) * RB + seg * 8 * Lay<BF>::ELT;
  store_row4<BF>(orow, acc);
  store_row4<BF>(orow + 4 * Lay<BF>::ELT, acc + 4);
}

}  // namespace lwk
