// kernels.hpp -- gfx950 kernels of the Longformer window + global attention
// forward.  Included once, by lwattn.hip.
//
// One kernel, attn_kernel, runs per forward.  Its grid holds three kinds of
// workgroups, in dispatch order:
//   * compaction workgroups, one per batch row: padding / global flags per
//     position and the ascending global-index list with its count (wave
//     ballot + prefix count; the FasterTransformer guide's global_idx /
//     global_token_nums partition), published to the rest of the grid through
//     a per-row epoch word;
//   * band workgroups: 128 query rows of one (batch, head, residue class of
//     the dilation) against their window keys and the global keys under
//     Q/K/V, one online softmax per row, the output row written directly;
//   * global-row workgroups: the global queries of one (batch, head) against
//     one slice of all keys under Qg/Kg/Vg, written as an unnormalised softmax
//     partial (running max, running sum, weighted value sum); the last slice
//     of a query tile to finish merges all of them (log-sum-exp) and writes
//     the output rows.
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
//
// Staging (general path: rows with scattered padding, float32 storage).
// Every thread of a workgroup loads one 16-byte chunk of K and of V per tile (two for float32) into registers two tiles ahead of its use and
// writes them to one of two LDS slots one step ahead, so a global load has two
// compute steps to arrive.  Key positions are computed, not loaded; the
// padding flag of a key is loaded beside its K/V chunk and padded keys are
// zeroed on the way into LDS.
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
constexpr int MAXH_ARG = 32;   // per-head tables passed by value up to this many heads
constexpr float TAU = 8.0f;    // lazy-rescale threshold, log2 units
constexpr float M_INIT = -1e30f;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// Storage element types: float, or one of the two 16-bit formats (__bf16,
// _Float16), which share every layout and differ only in the matrix-core and
// dot-product instructions and the rounding of conversions.
template <typename S, int N>
using svec = S __attribute__((ext_vector_type(N)));
template <typename S>
__device__ __host__ constexpr bool is16() { return sizeof(S) == 2; }

// 32x32x16 matrix-core product, fp32 accumulation, for either 16-bit format.
__device__ __forceinline__ f32x16 mfma16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma16(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
// acc + a0 b0 + a1 b1 in fp32, for either 16-bit format.
__device__ __forceinline__ float dot2(svec<__bf16, 2> a, svec<__bf16, 2> b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, b, acc, false);
}
__device__ __forceinline__ float dot2(svec<_Float16, 2> a, svec<_Float16, 2> b, float acc) {
  return __builtin_amdgcn_fdot2(a, b, acc, false);
}

// Raw buffer resources over device memory, and their 16-byte loads and stores.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ uint4 bload(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// A 16-byte store that writes through to the device-coherent level (cache
// policy sc1), so that no dirty line is left in L2 for a later release or the
// kernel's end to write back.  It goes through the compiler's buffer-store
// builtin, never inline asm: a store of more than 8 bytes reads its data
// registers after issue, and only a store the compiler can see gets the wait
// states that keep the next instruction from overwriting them.
constexpr int CPOL_SC1 = 16;
typedef unsigned u32x4s __attribute__((__vector_size__(16)));
typedef unsigned u32x2 __attribute__((__vector_size__(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
template <typename V16>
__device__ __forceinline__ void store_wt(__amdgpu_buffer_rsrc_t r, int off, V16 v) {
  static_assert(sizeof(V16) == 16, "16-byte store");
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4s, v), r, off, 0, CPOL_SC1);
}

// s_waitcnt vmcnt(N): at most N of this wave's loads and stores outstanding.
template <int N>
__device__ __forceinline__ void wait_loads() {
  static_assert(N >= 0 && N <= 63, "vmcnt immediate");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}


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
  int32_t* tile_cnt;       // [B][H][nqt]: finished key slices of a query tile (0 between forwards)
  int32_t* ready;          // [B]: epoch of the last forward whose compaction of the row is done
  int32_t* fault;          // sticky: set when a workgroup gave up waiting for its row
  uint64_t* ready_cnt;     // [B] or null: (epoch << 32) | global count, published beside ready
  int32_t epoch;           // this forward's number (> 0): what every workgroup waits for
  int32_t publish;         // what the compaction publishes (= epoch, except in a fault test)
  int32_t spin_limit;      // polls before a wait for a row gives up
  int32_t n_comp_wg;       // compaction workgroups at the head of the attention launch (B padded to 8, or 0)
  int32_t comp_fold;       // 1: no compaction workgroups; band workgroup bid < B compacts row bid first
  const int32_t* head_stride;  // [H]: dilation gap + 1 (device copy, any H)
  const int32_t* head_blk;     // [H+1]: prefix of band workgroups per batch row
  int32_t B, H, n, r;      // r = min(window/2, n)
  int32_t max_global, nqt, nqg, nsplit, ksplit;
  int32_t n_glob_wg;       // padded to a multiple of 8
  int32_t n_band_wg;
  int32_t band_pre;        // band workgroups dispatched before the global-row ones (a multiple of 8)
  // key parts per band block on the register-staged path (1: none).  With
  // more, each wave leaves its rows' partial (offset, sum, O) in the block's
  // slots and the last part to finish merges them.
  int32_t bparts;
  float* bpart_o;          // [blocks][NW][bparts][64 lanes][32]
  float* bpart_ml;         // [blocks][NW][bparts][32 rows][2]: offset, row sum
  int32_t* bcnt;           // [blocks][NW] parts finished (re-armed by the merge)
  int32_t blocks_per_b;    // head_blk[H]
  int32_t mask_vec;        // masks 16-byte aligned and n % 4 == 0
  int32_t uni_stride;      // > 0: every head has this stride
  int32_t blocks_per_head; // band workgroups of one head when uni_stride > 0
  int32_t band_fast;       // band workgroups may take the bf16 fast path
  int32_t o_tok;           // 1: O is token-major [B][n][H][64] (the encoder layer's merged heads), 0: [B][H][n][64]
  // Input rows: row (b, h, pos) of Q, K, V (k = 0), Qg (k = 1) or Kg, Vg
  // (k = 2) starts in_bs[k] b + in_hs[k] h + in_rs[k] pos bytes into its
  // tensor.  [B][H][n][64]: in_bs = H n rb, in_hs = n rb, in_rs = rb; the
  // encoder layer's projections, [B n][c hid] with the heads side by side:
  // in_bs = n in_rs, in_hs = rb, in_rs = c hid elt.
  int64_t in_bs[3], in_hs[3];
  int32_t in_rs[3];
  float c;                 // scale * log2(e)
  int32_t hs[MAXH_ARG];    // head_stride by value when H <= MAXH_ARG
  int32_t hb[MAXH_ARG + 1];
};

// Output row (b, h, pos) of rb bytes, in either output layout, and the byte
// distance between consecutive positions of one head.
__device__ __forceinline__ uint8_t* o_row(const Params& p, int b, int h, int pos, int rb) {
  const int64_t r = p.o_tok ? ((int64_t)b * p.n + pos) * p.H + h : ((int64_t)b * p.H + h) * p.n + pos;
  return p.O + r * rb;
}
__device__ __forceinline__ int o_stride(const Params& p, int rb) { return p.o_tok ? p.H * rb : rb; }
// First row of head (b, h) of an input tensor of class k (see Params).
__device__ __forceinline__ const uint8_t* in_head(const Params& p, const uint8_t* x, int k, int b, int h) {
  return x + (int64_t)b * p.in_bs[k] + (int64_t)h * p.in_hs[k];
}

// ---------------------------------------------------------------------------
// Layout of one LDS tile slot.
struct Lay16 {                 // 16-bit storage
  static constexpr int ELT = 2;
  static constexpr int CH = 8;           // 16-byte chunks per 64-element row
  static constexpr int KROW = 144;       // K row stride (128 + 16 pad: conflict-free b128 reads)
  static constexpr int VROW = 72;        // V^T row stride: 32 keys * 2 B + 8 pad
  static constexpr int KBYTES = KT * KROW;
  static constexpr int VBYTES = D * VROW;
};
struct Lay32 {                 // float32 storage
  static constexpr int ELT = 4;
  static constexpr int CH = 16;
  static constexpr int KROW = 272;
  static constexpr int VROW = 272;       // V kept [key][d]
  static constexpr int KBYTES = KT * KROW;
  static constexpr int VBYTES = KT * VROW;
};
template <typename S>
struct Lay : std::conditional_t<sizeof(S) == 2, Lay16, Lay32> {};
template <typename S>
struct SlotLay {
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = Lay<S>::KBYTES;
  static constexpr int POS_OFF = V_OFF + Lay<S>::VBYTES;
  static constexpr int OK_OFF = POS_OFF + KT * 4;      // uint32: bit k = key k usable
  static constexpr int BYTES = (OK_OFF + 4 + 15) / 16 * 16;
  static constexpr int NCH = KT * Lay<S>::CH / NT;    // chunks per thread per array
};

// Reads of what other workgroups of the launch wrote (the compaction's
// outputs, global-row partials) on the fast paths are agent-scope relaxed
// atomic loads: they compile to loads that are coherent across the XCDs
// (sc1) and so need no acquire fence, whose cache invalidation costs
// microseconds when hundreds of workgroups issue it at once.  They are issued
// only after the epoch (or the slice counter) has been seen, behind a barrier,
// so they observe what the release published.
__device__ __forceinline__ int coherent_load(const int32_t* ptr) {
  return __hip_atomic_load(ptr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t coherent_load64(const uint64_t* ptr) {
  return __hip_atomic_load(ptr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float coherent_loadf(const float* ptr) {
  return __builtin_bit_cast(float, coherent_load(reinterpret_cast<const int32_t*>(ptr)));
}

// Which keys a tile holds.  Positions are computed for every key, clamped to
// an existing row, so that every global load of the staging path is issued
// unconditionally (no divergent branch around a load); keys that do not exist
// or are padding are zeroed on the way into LDS.
struct TileDesc {
  int list;    // 0: position = base + jj*stride;  1: position = gl[jj] (global-index list)
  int j0;      // index of the tile's first key (subsequence index, or list index)
  int jend;    // one past the last existing key index (>= 1 whenever the tile is used)
  int base, stride;
};

struct Ctx {
  const float* lm;         // the batch row's local mask (an input: plain loads)
  const int32_t* gl;       // global positions of the batch row (LDS copy or global memory)
  bool gl_global;          // gl is the compaction's list in global memory (read coherently)
  int rho, s;              // residue class and stride of the band
  int64_t rs;              // bytes between consecutive key rows
};

__device__ __forceinline__ void key_pos(const TileDesc& td, const Ctx& cx, int k, int& pos, bool& in) {
  const int jj = td.j0 + k;
  in = (jj >= 0) & (jj < td.jend);
  const int jc = min(max(jj, 0), td.jend - 1);
  if (td.list)
    pos = cx.gl_global ? coherent_load(cx.gl + jc) : cx.gl[jc];
  else
    pos = td.base + jc * td.stride;
}

template <typename S>
struct Stage {
  static constexpr int NCH = SlotLay<S>::NCH;
  uint4 kr[NCH], vr[NCH];
  bool in[NCH];     // the chunk's key exists
  uint8_t fl[NCH];  // raw flag byte of that key (bit0: real token), inspected at store time
  int pos;          // position of key tid % KT
  bool okin;        // key tid % KT exists
  uint8_t okfl;     // its raw flag byte
  bool list;        // keys come from the global-index list (always real tokens)
};

// Issue the global loads of one tile into registers.  Nothing here consumes a
// loaded value, and no load sits under a divergent branch, so the compiler
// need not wait for them before the next tile's compute.
template <typename S>
__device__ __forceinline__ void stage_load(Stage<S>& st, const TileDesc& td, const Ctx& cx,
                                           const uint8_t* kbase, const uint8_t* vbase) {
  constexpr int CH = Lay<S>::CH;
  const int tid = threadIdx.x;
  st.list = td.list != 0;
#pragma unroll
  for (int e = 0; e < Stage<S>::NCH; ++e) {
    const int q = tid + NT * e;
    const int kt = q / CH, ch = q % CH;
    int pos;
    bool in;
    key_pos(td, cx, kt, pos, in);
    st.in[e] = in;
    st.kr[e] = *reinterpret_cast<const uint4*>(kbase + (int64_t)pos * cx.rs + ch * 16);
    st.vr[e] = *reinterpret_cast<const uint4*>(vbase + (int64_t)pos * cx.rs + ch * 16);
    st.fl[e] = cx.lm[pos] != 0.0f ? 1 : 0;
  }
  int pos;
  bool in;
  key_pos(td, cx, tid & (KT - 1), pos, in);
  st.pos = pos;
  st.okin = in;
  st.okfl = cx.lm[pos] != 0.0f ? 1 : 0;
}

// Sentinel window index of a global key outside the row's residue class.
constexpr int JREL_NONE = -(1 << 30);

// Write the staged registers into an LDS slot (V transposed for bf16).  For a
// global-column tile the slot also gets, per key, its index in the band's
// residue subsequence (or JREL_NONE), used to drop keys already in the window.
template <typename S>
__device__ __forceinline__ void stage_store(const Stage<S>& st, uint8_t* slot, const TileDesc& td,
                                            const Ctx& cx) {
  using SL = SlotLay<S>;
  constexpr int CH = Lay<S>::CH;
  const int tid = threadIdx.x;
#pragma unroll
  for (int e = 0; e < Stage<S>::NCH; ++e) {
    const int q = tid + NT * e;
    const int kt = q / CH, ch = q % CH;
    const uint4 z = make_uint4(0, 0, 0, 0);
    const bool use = st.in[e] && (st.list || (st.fl[e] & 1));
    const uint4 kv = use ? st.kr[e] : z;
    const uint4 vv = use ? st.vr[e] : z;
    *reinterpret_cast<uint4*>(slot + SL::K_OFF + kt * Lay<S>::KROW + ch * 16) = kv;
    if constexpr (is16<S>()) {
      const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint16_t hv = (uint16_t)(w[t >> 1] >> (16 * (t & 1)));
        *reinterpret_cast<uint16_t*>(slot + SL::V_OFF + (ch * 8 + t) * Lay<S>::VROW + kt * 2) = hv;
      }
    } else {
      *reinterpret_cast<uint4*>(slot + SL::V_OFF + kt * Lay<S>::VROW + ch * 16) = vv;
    }
  }
  if (tid < 64) {
    const uint64_t bits = __ballot(tid < KT && st.okin && (st.list || (st.okfl & 1)));
    if (tid < KT && td.list) {
      const int dp = st.pos - cx.rho;
      const int jrel = (dp >= 0 && dp % cx.s == 0) ? dp / cx.s : JREL_NONE;
      reinterpret_cast<int32_t*>(slot + SL::POS_OFF)[tid] = jrel;
    }
    if (tid == 0) *reinterpret_cast<uint32_t*>(slot + SL::OK_OFF) = (uint32_t)bits;
  }
}

// Runs `comp(u, slot)` for tiles u = 0..U-1 with a two-deep register
// prefetch: a tile's loads are issued two steps before its LDS store (fp32
// measured on par with or slightly faster than a one-step prefetch).  `pre()` runs once
// after the first loads are issued and before the first barrier.  Every
// thread of the workgroup must call it with the same U >= 1.
template <typename S, class DescFn, class CompFn, class PreFn>
__device__ __forceinline__ void tile_pipeline(int U, DescFn desc, CompFn comp, PreFn pre,
                                              const Ctx& cx, const uint8_t* kbase,
                                              const uint8_t* vbase, uint8_t* smem) {
  using SL = SlotLay<S>;
  uint8_t* slot0 = smem;
  uint8_t* slot1 = smem + SL::BYTES;
  Stage<S> s0, s1;
  stage_load<S>(s0, desc(0), cx, kbase, vbase);
  if (U > 1) stage_load<S>(s1, desc(1), cx, kbase, vbase);
  pre();
  stage_store<S>(s0, slot0, desc(0), cx);
  __syncthreads();
  for (int u = 0; u < U; u += 2) {
    if (u + 2 < U) stage_load<S>(s0, desc(u + 2), cx, kbase, vbase);
    comp(u, slot0);
    if (u + 1 < U) stage_store<S>(s1, slot1, desc(u + 1), cx);
    __syncthreads();
    if (u + 1 >= U) break;
    if (u + 3 < U) stage_load<S>(s1, desc(u + 3), cx, kbase, vbase);
    comp(u + 1, slot1);
    if (u + 2 < U) stage_store<S>(s0, slot0, desc(u + 2), cx);
    __syncthreads();
  }
}

// Query operand held in registers for the whole key loop.
template <typename S>
struct QOp {                   // 16-bit storage
  svec<S, 8> q[4];   // Q[row][32*h + 8*c .. +8], c = 0..3
  __device__ void load(const uint8_t* row, bool ok, int h) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (ok) v = *reinterpret_cast<const uint4*>(row + (32 * h + 8 * c) * 2);
      q[c] = __builtin_bit_cast(svec<S, 8>, v);
    }
  }
};
template <>
struct QOp<float> {
  float q[32];   // Q[row][32*h + c], c = 0..31
  __device__ void load(const uint8_t* row, bool ok, int h) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (ok) v = *reinterpret_cast<const float4*>(row + (32 * h + 4 * c) * 4);
      q[4 * c + 0] = v.x;
      q[4 * c + 1] = v.y;
      q[4 * c + 2] = v.z;
      q[4 * c + 3] = v.w;
    }
  }
};

// S^T tile: 16 scores of this lane's query.
template <typename S>
__device__ __forceinline__ f32x16 qk_tile(const QOp<S>& qo, const uint8_t* slot, int lane) {
  const int key = lane & 31, h = lane >> 5;
  f32x16 s = {};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const svec<S, 8> a = *reinterpret_cast<const svec<S, 8>*>(slot + SlotLay<S>::K_OFF +
                                                              key * Lay<S>::KROW + (4 * h + c) * 16);
    s = mfma16(a, qo.q[c], s);
  }
  return s;
}
__device__ __forceinline__ f32x16 qk_tile(const QOp<float>& qo, const uint8_t* slot, int lane) {
  const int key = lane & 31, h = lane >> 5;
  // two independent accumulation chains (even and odd channel groups), so
  // each MFMA waits on the one two back instead of the one just before it
  f32x16 s0 = {}, s1 = {};
#pragma unroll
  for (int c4 = 0; c4 < 8; ++c4) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(slot + SlotLay<float>::K_OFF +
                                                    key * Lay<float>::KROW + (8 * h + c4) * 16);
#pragma unroll
    for (int e = 0; e < 4; e += 2) {
      s0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], qo.q[4 * c4 + e], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e + 1], qo.q[4 * c4 + e + 1], s1, 0, 0, 0);
    }
  }
  return s0 + s1;
}

// O^T += V^T * P^T for one tile.
template <typename S>
__device__ __forceinline__ void pv_tile(f32x16 (&o)[2], const float (&p)[16], const uint8_t* slot,
                                        int lane) {
  const int h = lane >> 5, dl = lane & 31;
  const uint8_t* vt = slot + SlotLay<S>::V_OFF;
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2) {
    svec<S, 8> bp;
#pragma unroll
    for (int e = 0; e < 8; ++e) bp[e] = (S)p[8 * c2 + e];
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const uint8_t* row = vt + (32 * db + dl) * Lay<S>::VROW;
      const svec<S, 4> lo = *reinterpret_cast<const svec<S, 4>*>(row + (16 * c2 + 4 * h) * 2);
      const svec<S, 4> hi = *reinterpret_cast<const svec<S, 4>*>(row + (16 * c2 + 8 + 4 * h) * 2);
      svec<S, 8> a;
      a[0] = lo[0]; a[1] = lo[1]; a[2] = lo[2]; a[3] = lo[3];
      a[4] = hi[0]; a[5] = hi[1]; a[6] = hi[2]; a[7] = hi[3];
      o[db] = mfma16(a, bp, o[db]);
    }
  }
}
template <>
__device__ __forceinline__ void pv_tile<float>(f32x16 (&o)[2], const float (&p)[16], const uint8_t* slot,
                                               int lane) {
  const int h = lane >> 5, dl = lane & 31;
  const uint8_t* vb = slot + SlotLay<float>::V_OFF;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int key = 8 * (r >> 2) + 4 * h + (r & 3);
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const float a = *reinterpret_cast<const float*>(vb + key * Lay<float>::VROW + (32 * db + dl) * 4);
      o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, p[r], o[db], 0, 0, 0);
    }
  }
}

// Key index (0..31 within the tile) held in register r by this lane.
__device__ __forceinline__ int key_of(int r, int lane) {
  return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// Maximum of x over lanes l and l^32 (the two lanes holding one query row).
// v_permlane32_swap exchanges the upper half of its first operand with the
// lower half of its second; with both operands x, the two results hold x of
// both halves, and x itself is kept in the max.
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(x, fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
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
  // s: masked scores (excluded = -inf); returns probabilities in p.  The max
  // is only raised when some row's scores exceed it by more than 2^TAU, so the
  // O rescale is rare; every probability stays below 2^TAU.
  __device__ __forceinline__ void update(const f32x16& s, float c, float (&p)[16]) {
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = half_max(mx);
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
// Compaction, inside the attention launch: workgroup b (of the first B) does
// batch row b with NT threads, 16 consecutive positions per thread and pass
// (four float4 of each mask), counting a wave's globals with 5 ballots (per-
// thread counts are 0..16), then publishes the row by storing this forward's
// epoch into ready[b].  Every other workgroup of the launch waits for the
// epoch of its row before reading what the compaction wrote.
constexpr int C_PT = 16;
__device__ __forceinline__ void wave_count5(int mine, int lane, int& before, int& total) {
  before = 0;
  total = 0;
#pragma unroll
  for (int bit = 0; bit < 5; ++bit) {
    const uint64_t bal = __ballot((mine >> bit) & 1);
    before += __popcll(bal & ((1ull << lane) - 1ull)) << bit;
    total += __popcll(bal) << bit;
  }
}

__device__ void compact_row(const Params& p, int b, uint8_t* smem) {
  int* wsum = reinterpret_cast<int*>(smem);            // [NW] globals per wave
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = p.n;
  const float* lm = p.lmask + (int64_t)b * n;
  const float* gm = p.gmask + (int64_t)b * n;
  uint8_t* fl = p.flags + (int64_t)b * n;
  int32_t* gi = p.gidx + (int64_t)b * n;
  int carry = 0;
  const bool vec = p.mask_vec != 0;   // masks 16-byte aligned and n % 4 == 0
  for (int base = 0; base < n; base += NT * C_PT) {
    const int j0 = base + tid * C_PT;
    float lv[C_PT], gv[C_PT];
    if (vec && j0 + C_PT <= n) {
#pragma unroll
      for (int k = 0; k < C_PT / 4; ++k) {
        const float4 a = *reinterpret_cast<const float4*>(lm + j0 + 4 * k);
        const float4 c = *reinterpret_cast<const float4*>(gm + j0 + 4 * k);
        lv[4 * k] = a.x; lv[4 * k + 1] = a.y; lv[4 * k + 2] = a.z; lv[4 * k + 3] = a.w;
        gv[4 * k] = c.x; gv[4 * k + 1] = c.y; gv[4 * k + 2] = c.z; gv[4 * k + 3] = c.w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < C_PT; ++e) {
        lv[e] = (j0 + e < n) ? lm[j0 + e] : 0.0f;
        gv[e] = (j0 + e < n) ? gm[j0 + e] : 0.0f;
      }
    }
    uint32_t gbits = 0, packed[C_PT / 4];
    int mine = 0;
#pragma unroll
    for (int k = 0; k < C_PT / 4; ++k) packed[k] = 0;
#pragma unroll
    for (int e = C_PT - 1; e >= 0; --e) {
      const bool v = lv[e] != 0.0f;
      const bool g = v && (gv[e] != 0.0f);
      packed[e / 4] |= (uint32_t)((v ? 1 : 0) | (g ? 2 : 0)) << (8 * (e % 4));
      gbits |= (uint32_t)(g ? 1 : 0) << e;
      mine += g ? 1 : 0;
    }
    if ((n % 4) == 0 && j0 + C_PT <= n) {
#pragma unroll
      for (int k = 0; k < C_PT / 4; ++k)
        *reinterpret_cast<uint32_t*>(fl + j0 + 4 * k) = packed[k];   // 4-byte aligned
    } else {
#pragma unroll
      for (int e = 0; e < C_PT; ++e)
        if (j0 + e < n) fl[j0 + e] = (uint8_t)(packed[e / 4] >> (8 * (e % 4)));
    }
    int before, wtot;
    wave_count5(mine, lane, before, wtot);
    if (lane == 0) wsum[wave] = wtot;
    __syncthreads();
    int wpre = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int cw = wsum[w];
      wpre += (w < wave) ? cw : 0;
      tot += cw;
    }
    int k = carry + wpre + before;
    while (gbits) {
      const int e = __builtin_ctz(gbits);
      gbits &= gbits - 1;
      gi[k++] = j0 + e;
    }
    carry += tot;
    __syncthreads();
  }
  for (int k = carry + tid; k < n; k += NT) gi[k] = -1;
  if (tid == 0) {
    p.gcnt[b] = carry;
    p.status[b] = carry > p.max_global ? 1 : 0;
  }
  // the row's flags, list and count are written back before
  // the epoch is published (a release; no acquire, which would invalidate
  // this XCD's caches)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (tid == 0) {
    __hip_atomic_store(p.ready + b, p.publish, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    // the epoch and the count in one word, for readers that want both from a
    // single load (ordered after the release above)
    if (p.ready_cnt)
      __hip_atomic_store(p.ready_cnt + b, ((uint64_t)(uint32_t)p.publish << 32) | (uint32_t)carry,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Wait until batch row b is compacted for this forward.  The compaction
// workgroups come first in dispatch order, so they run; the wait is bounded
// all the same, and a row that never becomes ready is reported in the sticky
// fault word (the workgroup then skips its work) instead of hanging the
// launch.  One thread polls with relaxed loads and sleeps between polls; the
// barrier passes what it saw on to the rest of the workgroup.  Every caller
// reads the compaction's outputs with coherent loads (no acquire fence: each
// one invalidates the XCD's caches, the key tiles other workgroups are
// reusing included).
// The limit (p.spin_limit, set by the host) allows at least ~2^18 polls (each
// sleeps >= 128 clocks) plus n / 4 for the compaction of long rows, far beyond
// the time it takes.
__device__ __forceinline__ bool wait_ready(const Params& p, int b) {
  __shared__ int s_ok;
  if (threadIdx.x == 0) {
    int spins = 0, good = 1;
    while (coherent_load(p.ready + b) != p.epoch) {
      if (++spins > p.spin_limit) {
        good = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    if (!good) atomicOr(p.fault, 1);
    s_ok = good;
  }
  __syncthreads();
  return s_ok != 0;
}

// ---------------------------------------------------------------------------
// Attention.
// mask_kind: 0 none, 1 window tile (key usable and |i - j| <= r),
//            2 global columns (usable and not already in the row's window),
//            3 key usable only.  Every mask is a select, never a branch.
template <typename S>
__device__ __forceinline__ void process_tile(const QOp<S>& qo, Softmax& sm, const uint8_t* slot,
                                             int lane, float c, int mask_kind, int my_i, int band_j0,
                                             int r) {
  using SL = SlotLay<S>;
  f32x16 sc = qk_tile(qo, slot, lane);
  if (mask_kind != 0) {
    const uint32_t okb = *reinterpret_cast<const uint32_t*>(slot + SL::OK_OFF);
    const int h = lane >> 5;
    if (mask_kind == 2) {
      const int4* jr = reinterpret_cast<const int4*>(slot + SL::POS_OFF);
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int4 v = jr[2 * a + h];          // keys 8a + 4h .. 8a + 4h + 3
        const int jv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int k = 8 * a + 4 * h + e;
          const int dj = my_i - jv[e];
          const bool allowed = ((okb >> k) & 1u) && !(dj <= r && dj >= -r);
          sc[4 * a + e] = allowed ? sc[4 * a + e] : -INFINITY;
        }
      }
    } else {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int k = key_of(rr, lane);
        bool allowed = (okb >> k) & 1u;
        if (mask_kind == 1) {
          const int dj = my_i - (band_j0 + k);
          allowed = allowed && dj <= r && dj >= -r;
        }
        sc[rr] = allowed ? sc[rr] : -INFINITY;
      }
    }
  }
  float pr[16];
  sm.update(sc, c, pr);
  pv_tile<S>(sm.o, pr, slot, lane);
}

template <typename S>
__device__ __forceinline__ void store_row4(uint8_t* dst, const float* v) {
  if constexpr (is16<S>()) {
    svec<S, 4> t;
    t[0] = (S)v[0]; t[1] = (S)v[1]; t[2] = (S)v[2]; t[3] = (S)v[3];
    *reinterpret_cast<svec<S, 4>*>(dst) = t;
  } else {
    *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

// Number of global positions a band workgroup keeps in LDS; global columns
// beyond it are read from the global-index list directly (second pass).
constexpr int GL_MAX = 512;

template <typename S>
constexpr int smem_bytes_general() { return 2 * SlotLay<S>::BYTES + GL_MAX * 4; }

// Key parts of a band block (register-staged path): each wave leaves its 32
// rows' partial result -- offset m, row sum l, unnormalised O^T accumulators
// in register order -- in the block's slot of this part and counts itself
// on the (block, wave) counter; the wave that counts the last part merges the
// parts by log-sum-exp into sm and lt (offsets are in the exponent's log2
// units, so the weights are 2^(m_k - max m)) and returns true, the others
// false.  The merging wave re-arms the counter for the next forward.  Parts
// with no key of a row carry (M_INIT, 0, 0) and weigh nothing.
__device__ bool merge_band_parts(const Params& p, int blk, int part, int wave, int lane, Softmax& sm, float& lt) {
  const int P = p.bparts, qi = lane & 31;
  const int64_t wslot = ((int64_t)blk * NW + wave) * P;
  float* po = p.bpart_o + ((wslot + part) * 64 + lane) * 32;
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int k = 0; k < 4; ++k)
      *reinterpret_cast<float4*>(po + 16 * db + 4 * k) =
          make_float4(sm.o[db][4 * k], sm.o[db][4 * k + 1], sm.o[db][4 * k + 2], sm.o[db][4 * k + 3]);
  if (lane < 32) *reinterpret_cast<float2*>(p.bpart_ml + ((wslot + part) * 32 + qi) * 2) = make_float2(sm.m, lt);
  // this part is written back before it is counted; the wave that counts the
  // last part reads all of them with agent-coherent loads (here a fence
  // measured faster than write-through stores and a wait for them)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  int32_t* cnt = p.bcnt + (int64_t)blk * NW + wave;
  int old = 0;
  if (lane == 0) old = atomicAdd(cnt, 1);
  old = __builtin_amdgcn_readfirstlane(old);
  if (old != P - 1) return false;
  const __amdgpu_buffer_rsrc_t ro =
      __builtin_amdgcn_make_buffer_rsrc(p.bpart_o + wslot * 64 * 32, (short)0, P * 64 * 32 * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t rml =
      __builtin_amdgcn_make_buffer_rsrc(p.bpart_ml + wslot * 32 * 2, (short)0, P * 32 * 2 * 4, 0x00020000);
  float mrun = M_INIT, L = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) { sm.o[0][r] = 0.f; sm.o[1][r] = 0.f; }
  // the parts' loads leave four at a time (coherent loads take a round trip
  // to memory each: two round trips for up to eight parts, not eight); parts
  // past P read as zeros through the ranges and weigh nothing
  constexpr int G = 4;
  for (int k0 = 0; k0 < P; k0 += G) {
    float2 ml[G];
    float4 o[G][8];
#pragma unroll
    for (int e = 0; e < G; ++e) {
      const int k = k0 + e;
      ml[e] = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(rml, (k * 32 + qi) * 8, 0, 16));
#pragma unroll
      for (int j = 0; j < 8; ++j)
        o[e][j] = __builtin_bit_cast(float4,
                                     __builtin_amdgcn_raw_buffer_load_b128(ro, ((k * 64 + lane) * 32 + 4 * j) * 4, 0, 16));
    }
#pragma unroll
    for (int e = 0; e < G; ++e) {
      const bool live = k0 + e < P;
      const float mn = live ? fmaxf(mrun, ml[e].x) : mrun;
      const float wa = __builtin_amdgcn_exp2f(mrun - mn), wb = live ? __builtin_amdgcn_exp2f(ml[e].x - mn) : 0.f;
      L = wa * L + wb * ml[e].y;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int db = j >> 2, r = 4 * (j & 3);
        sm.o[db][r] = wa * sm.o[db][r] + wb * o[e][j].x;
        sm.o[db][r + 1] = wa * sm.o[db][r + 1] + wb * o[e][j].y;
        sm.o[db][r + 2] = wa * sm.o[db][r + 2] + wb * o[e][j].z;
        sm.o[db][r + 3] = wa * sm.o[db][r + 3] + wb * o[e][j].w;
      }
      mrun = mn;
    }
  }
  sm.m = mrun;
  lt = L;
  if (lane == 0) *cnt = 0;
  return true;
}

template <typename S>
__device__ void band_wg(const Params& p, int b, int h, int local, int s, int blk, int part, uint8_t* smem) {
  using SL = SlotLay<S>;
  constexpr int RB = D * Lay<S>::ELT;
  const int tid = threadIdx.x, lane = tid & 63, h32 = lane >> 5, qi = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int n = p.n;
  int rho = 0, nr = 0;
  for (rho = 0; rho < s; ++rho) {
    nr = (n - rho + s - 1) / s;
    const int nb = (nr + ROWS_WG - 1) / ROWS_WG;
    if (local < nb) break;
    local -= nb;
  }
  const int R0 = local * ROWS_WG;
  const int32_t* gidx_b = p.gidx + (int64_t)b * n;
  int32_t* gl_lds = reinterpret_cast<int32_t*>(smem + 2 * SL::BYTES);
  Ctx cx;
  cx.lm = p.lmask + (int64_t)b * n;
  cx.gl = gl_lds;
  cx.gl_global = false;
  cx.rho = rho;
  cx.s = s;
  cx.rs = p.in_rs[0];

  const int r = p.r;
  const int kb = R0 - r;
  const int T = (31 + 2 * r) / 32 + 1;
  const int t_lo = (-kb - 31 > 0) ? (-kb - 31 + 31) / 32 : 0;
  int t_hi = (nr - 1 - kb) / 32;
  if (t_hi > NW - 1 + T - 1) t_hi = NW - 1 + T - 1;
  const int nband = t_hi - t_lo + 1;
  int g = coherent_load(p.gcnt + b);
  if (g > p.max_global) g = p.max_global;
  const int gmain = g < GL_MAX ? g : GL_MAX;
  const int ngt = (gmain + KT - 1) / KT;
  const int U = nband + ngt;

  const int my_i = R0 + 32 * wave + qi;
  const bool row_in = my_i < nr;
  const int my_pos = rho + (row_in ? my_i : 0) * s;
  // the row's flags (bit 0 real token, bit 1 global) from the masks
  const bool my_real = cx.lm[my_pos] != 0.0f;
  const uint8_t my_fl = (my_real ? 1 : 0) | (my_real && p.gmask[(int64_t)b * n + my_pos] != 0.0f ? 2 : 0);
  QOp<S> qo;
  qo.load(in_head(p, p.Q, 0, b, h) + (int64_t)my_pos * cx.rs, row_in, h32);
  Softmax sm;
  sm.init();
  const bool wave_work = __any(row_in && (my_fl & 3) == 1);

  auto desc = [&](int u) {
    TileDesc td;
    if (u < nband) {
      td.list = 0;
      td.j0 = kb + (t_lo + u) * KT;
      td.jend = nr;
      td.base = rho;
      td.stride = s;
    } else {
      td.list = 1;
      td.j0 = (u - nband) * KT;
      td.jend = gmain;
      td.base = 0;
      td.stride = 0;
    }
    return td;
  };
  auto comp = [&](int u, const uint8_t* slot) {
    if (!wave_work) return;
    if (u < nband) {
      const int t = t_lo + u;
      const int up = t - wave;
      if (up >= 0 && up < T) {
        const uint32_t okb = *reinterpret_cast<const uint32_t*>(slot + SL::OK_OFF);
        const bool diag = (up == 0) || (32 * up + 31 > 2 * r);
        process_tile<S>(qo, sm, slot, lane, p.c, (diag || okb != 0xFFFFFFFFu) ? 1 : 0, my_i,
                         kb + t * KT, r);
      }
    } else {
      process_tile<S>(qo, sm, slot, lane, p.c, 2, my_i, 0, r);
    }
  };
  auto fill_gl = [&]() {
    for (int j = tid; j < gmain; j += NT) gl_lds[j] = coherent_load(gidx_b + j);
  };
  auto nothing = []() {};
  const uint8_t* kbase = in_head(p, p.K, 0, b, h);
  const uint8_t* vbase = in_head(p, p.V, 0, b, h);
  // this workgroup's tiles [u0, u1) of the U (all of them unless the block's
  // keys are cut into parts; the last part also takes the columns past the
  // LDS list)
  const int P = p.bparts;
  const int u0 = (int)((int64_t)U * part / P), u1 = (int)((int64_t)U * (part + 1) / P);
  auto desc_p = [&](int u) { return desc(u0 + u); };
  auto comp_p = [&](int u, const uint8_t* slot) { comp(u0 + u, slot); };
  if (u1 > u0) {
    if (u1 <= nband) {
      tile_pipeline<S>(u1 - u0, desc_p, comp_p, nothing, cx, kbase, vbase, smem);
    } else if (nband - u0 >= 2) {
      // the list is filled while the first (band) tiles load
      tile_pipeline<S>(u1 - u0, desc_p, comp_p, fill_gl, cx, kbase, vbase, smem);
    } else {
      fill_gl();
      __syncthreads();
      tile_pipeline<S>(u1 - u0, desc_p, comp_p, nothing, cx, kbase, vbase, smem);
    }
  }
  if (g > GL_MAX && part == P - 1) {
    // global columns past the LDS copy: positions straight from the list
    Ctx cx2 = cx;
    cx2.gl = gidx_b + GL_MAX;
    cx2.gl_global = true;
    const int U2 = (g - GL_MAX + KT - 1) / KT;
    auto desc2 = [&](int u) {
      TileDesc td;
      td.list = 1;
      td.j0 = u * KT;
      td.jend = g - GL_MAX;
      td.base = 0;
      td.stride = 0;
      return td;
    };
    auto comp2 = [&](int u, const uint8_t* slot) {
      if (wave_work) process_tile<S>(qo, sm, slot, lane, p.c, 2, my_i, 0, r);
    };
    tile_pipeline<S>(U2, desc2, comp2, nothing, cx2, kbase, vbase, smem);
  }

  // normalise and store this lane's half of its query row (global rows are
  // written by the merge kernel, padded rows get exact zeros)
  float lt = sm.l + __shfl_xor(sm.l, 32);
  if (P > 1 && !merge_band_parts(p, blk, part, wave, lane, sm, lt)) return;
  if (row_in && (my_fl & 2) == 0) {
    const bool valid = (my_fl & 1) != 0;
    const float inv = valid ? 1.0f / lt : 0.0f;
    uint8_t* orow = o_row(p, b, h, my_pos, RB);
#pragma unroll
    for (int db = 0; db < 2; ++db) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = valid ? sm.o[db][4 * a + e] * inv : 0.0f;
        store_row4<S>(orow + (32 * db + 8 * a + 4 * h32) * Lay<S>::ELT, v);
      }
    }
  }
}

// Global-row merge, fused into the attention kernel.  Every (b, h, query
// tile) has a counter of finished key slices; the wave that finishes the last
// slice of a tile combines the nsplit partial results of its 32 rows (the
// log-sum-exp merge of split softmax, taken online: a running maximum, the
// running sum and output rescaled as each partial arrives) and writes them,
// then re-arms the counter for the next forward.  Lane l merges row l % 32,
// channels 32 (l / 32) .. +31; pos is that row's sequence position.  The
// partials are streamed two chunks deep, so the merge waits for about one
// memory round trip instead of one per chunk.
// One wave's partial result of a global-row query tile over one key slice
// (32 rows: unnormalised O^T accumulators in register order, offset m, row
// sum l), written through (sc1) to its slot, so that waiting for the stores'
// completion publishes it (no release fence, whose write-back of the whole L2
// serialises over the workgroups of an XCD).
__device__ __forceinline__ void store_global_partial(const Params& p, int64_t slot, int qi, int h32,
                                                     const f32x16 (&o)[2], float m, float l) {
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(p.part_o + slot * 32 * D, 32 * D * 4);
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const f32x4 v = {o[db][4 * a], o[db][4 * a + 1], o[db][4 * a + 2], o[db][4 * a + 3]};
      store_wt(ro, (qi * D + 32 * db + 8 * a + 4 * h32) * 4, v);
    }
  if (h32 == 0) {
    const f32x2 ml = {m, l};
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, ml), make_rsrc(p.part_ml + slot * 32 * 2, 32 * 2 * 4),
                                          qi * 8, 0, CPOL_SC1);
  }
}

template <typename S, bool WT = false>
__device__ void finish_global_tile(const Params& p, int b, int h, int qt, int g, int lane, int pos) {
  // this slice's partial rows are visible device-wide before it is counted:
  // written through (WT: sc1 stores, whose completion is waited for here) or
  // written back by a release fence; the wave that counts the last slice
  // reads all of them with coherent loads
  if constexpr (WT)
    wait_loads<0>();
  else
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  int32_t* cnt = p.tile_cnt + ((int64_t)b * p.H + h) * p.nqt + qt;
  int old = 0;
  if (lane == 0) old = atomicAdd(cnt, 1);
  old = __builtin_amdgcn_readfirstlane(old);
  if (old != p.nsplit - 1) return;
  const int q = lane & 31, ch = lane >> 5;
  const int idx = qt * 32 + q;
  if (idx < g) {
    const int64_t base = (((int64_t)b * p.H + h) * p.nqt + qt) * p.nsplit;
    const int ns = p.nsplit;
    // this tile's partials, read through buffer ranges with the sc1
    // (agent-coherent) cache policy
    const __amdgpu_buffer_rsrc_t ro =
        __builtin_amdgcn_make_buffer_rsrc(p.part_o + base * 32 * D, (short)0, ns * 32 * D * 4, 0x00020000);
    const __amdgpu_buffer_rsrc_t rml =
        __builtin_amdgcn_make_buffer_rsrc(p.part_ml + base * 32 * 2, (short)0, ns * 32 * 2 * 4, 0x00020000);
    constexpr int U = 2;   // partials per chunk
    struct Chunk {
      float2 ml[U];
      float4 o[U][8];
    };
    // partials past ns read as zeros through the ranges and are skipped
    auto load = [&](int s0, Chunk& c) {
#pragma unroll
      for (int e = 0; e < U; ++e) {
        const int sl = s0 + e;
        c.ml[e] = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(rml, (sl * 32 + q) * 8, 0, 16));
        const int ob = ((sl * 32 + q) * D + 32 * ch) * 4;
#pragma unroll
        for (int k = 0; k < 8; ++k)
          c.o[e][k] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(ro, ob + 16 * k, 0, 16));
      }
    };
    float mrun = -INFINITY, L = 0.f, acc[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] = 0.f;
    auto merge = [&](int s0, const Chunk& c) {
#pragma unroll
      for (int e = 0; e < U; ++e) {
        // an empty slice (no real key) carries offset -inf
        const bool live = s0 + e < ns && c.ml[e].x != -INFINITY;
        const float mn = live ? fmaxf(mrun, c.ml[e].x) : mrun;
        const float wa = live ? __builtin_amdgcn_exp2f(mrun - mn) : 1.0f;
        const float wb = live ? __builtin_amdgcn_exp2f(c.ml[e].x - mn) : 0.0f;
        L = wa * L + wb * c.ml[e].y;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          acc[4 * k + 0] = wa * acc[4 * k + 0] + wb * c.o[e][k].x;
          acc[4 * k + 1] = wa * acc[4 * k + 1] + wb * c.o[e][k].y;
          acc[4 * k + 2] = wa * acc[4 * k + 2] + wb * c.o[e][k].z;
          acc[4 * k + 3] = wa * acc[4 * k + 3] + wb * c.o[e][k].w;
        }
        mrun = mn;
      }
    };
    Chunk ca, cb;
    load(0, ca);
    for (int s0 = 0; s0 < ns; s0 += 2 * U) {
      if (s0 + U < ns) load(s0 + U, cb);
      merge(s0, ca);
      if (s0 + U >= ns) break;
      if (s0 + 2 * U < ns) load(s0 + 2 * U, ca);
      merge(s0 + U, cb);
    }
    const float inv = 1.0f / L;
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] *= inv;
    constexpr int RB = D * Lay<S>::ELT;
    uint8_t* orow = o_row(p, b, h, pos, RB) + 32 * ch * Lay<S>::ELT;
#pragma unroll
    for (int k = 0; k < 8; ++k) store_row4<S>(orow + 4 * k * Lay<S>::ELT, acc + 4 * k);
  }
  if (lane == 0) *cnt = 0;
}

template <typename S>
__device__ void global_wg(const Params& p, int b, int h, int qg, int sp, uint8_t* smem) {
  const int tid = threadIdx.x, lane = tid & 63, h32 = lane >> 5, qi = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  int g = coherent_load(p.gcnt + b);
  if (g > p.max_global) g = p.max_global;
  const int nqt_b = (g + 31) / 32;
  if (qg * NW >= nqt_b) return;                     // uniform over the workgroup
  const int qt = qg * NW + wave;
  const bool wave_work = qt < nqt_b;
  const int n = p.n;
  const int32_t* gidx_b = p.gidx + (int64_t)b * n;
  Ctx cx;
  cx.lm = p.lmask + (int64_t)b * n;
  cx.gl = gidx_b;
  cx.gl_global = true;
  cx.rho = 0;
  cx.s = 1;
  cx.rs = p.in_rs[2];

  const int qidx = qt * 32 + qi;
  const bool qok = wave_work && qidx < g;
  const int qpos = coherent_load(gidx_b + (qok ? qidx : 0));
  QOp<S> qo;
  qo.load(in_head(p, p.Qg, 1, b, h) + (int64_t)(qok ? qpos : 0) * p.in_rs[1], qok, h32);
  Softmax sm;
  sm.init();

  const int j_start = sp * p.ksplit;
  int j_end = j_start + p.ksplit;
  if (j_end > n) j_end = n;
  const int U = (j_end - j_start + KT - 1) / KT;
  auto desc = [&](int u) {
    TileDesc td;
    td.list = 0;
    td.j0 = j_start + u * KT;
    td.jend = j_end;
    td.base = 0;
    td.stride = 1;
    return td;
  };
  auto comp = [&](int u, const uint8_t* slot) {
    if (!wave_work) return;
    const uint32_t okb = *reinterpret_cast<const uint32_t*>(slot + SlotLay<S>::OK_OFF);
    process_tile<S>(qo, sm, slot, lane, p.c, okb == 0xFFFFFFFFu ? 0 : 3, 0, 0, 0);
  };
  auto nothing = []() {};
  tile_pipeline<S>(U, desc, comp, nothing, cx, in_head(p, p.Kg, 2, b, h), in_head(p, p.Vg, 2, b, h), smem);

  const float lt = sm.l + __shfl_xor(sm.l, 32);
  if (qok) store_global_partial(p, (((int64_t)b * p.H + h) * p.nqt + qt) * p.nsplit + sp, qi, h32, sm.o, sm.m, lt);
  if (wave_work) finish_global_tile<S, true>(p, b, h, qt, g, lane, qpos);
}

// ---------------------------------------------------------------------------
// Fast path for bf16 storage where the real tokens among the keys a workgroup
// reads are a prefix of them (no padding, or a padded tail): the common case.
// Each workgroup checks this itself, from the mask, over the keys it reads
// (a band workgroup over its band, a global-row workgroup over its slice).
//
// Keys are fetched with buffer loads whose range ends at the first padded
// row, so the hardware returns zeros for every key before the start, past the
// end or in the padded tail -- no clamping, no flag loads, no zeroing
// selects.  Validity of the keys of a tile is then pure scalar arithmetic.
// K and V tiles are stored row-major (128 B rows) with 16-byte chunks XOR-
// swizzled per row, so that the b128 reads of the QK^T A operand and the
// transposing reads of the PV A operand are free of bank conflicts; a
// buffer-to-LDS load writes 64 consecutive physical chunks, each lane fetching
// the logical chunk that belongs there.  The PV A operand
// (V^T, four consecutive keys at one d per lane) comes from ds_read_b64_tr_b16:
// within a 16-lane group, source lane 4e+q reads V[k0+e][d0+4q .. +3] and
// output lane i receives V[k0+e][d0+i] for e = 0..3.
typedef short s16x4 __attribute__((ext_vector_type(4)));
constexpr int OOB_OFF = 0x7FFFFF00;             // a buffer offset past any range

__device__ __forceinline__ int swz_k(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int swz_v(int row) { return 2 * (row & 3); }


// Per-lane LDS byte offsets used by the compute of every tile.
struct FLane {
  int k[4];   // offsets in a K tile: row lane%32, logical chunk 4*(lane/32) + c
  int v[2];   // offsets in a V tile: transpose-read source for d block db (c2 / key-block offsets are immediates)
  __device__ void init(int lane) {
    const int row = lane & 31, h = lane >> 5;
#pragma unroll
    for (int c = 0; c < 4; ++c) k[c] = row * 128 + (((4 * h + c) ^ swz_k(row)) * 16);
    const int g1 = (lane >> 4) & 1, e = (lane >> 2) & 3, q = lane & 3;
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int chunk = (4 * db + 2 * g1 + (q >> 1)) ^ (2 * e);   // row & 3 == e for every row read
      v[db] = (4 * h + e) * 128 + chunk * 16 + (q & 1) * 8;
    }
  }
};

template <typename S>
__device__ __forceinline__ f32x16 fqk(const QOp<S>& qo, const uint8_t* kt, const FLane& fl) {
  f32x16 s = {};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const svec<S, 8> a = *reinterpret_cast<const svec<S, 8>*>(kt + fl.k[c]);
    s = mfma16(a, qo.q[c], s);
  }
  return s;
}

__device__ __forceinline__ s16x4 tr_read(const uint8_t* addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(addr));
}

template <typename S>
__device__ __forceinline__ void fpv(f32x16 (&o)[2], const svec<S, 8> (&pb)[2], const uint8_t* vt,
                                    const FLane& fl) {
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2) {
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const s16x4 lo = tr_read(vt + fl.v[db] + c2 * 2048);            // keys 16c2 + 4h + e
      const s16x4 hi = tr_read(vt + fl.v[db] + c2 * 2048 + 1024);     // keys 16c2 + 8 + 4h + e
      typedef short s16x8 __attribute__((ext_vector_type(8)));
      const s16x8 a8 = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      o[db] = mfma16(__builtin_bit_cast(svec<S, 8>, a8), pb[c2], o[db]);
    }
  }
}

__device__ __forceinline__ f32x16 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Bits [lo, hi) of a 32-bit word (empty when hi <= lo).
__device__ __forceinline__ uint32_t bit_range(int lo, int hi) {
  lo = lo < 0 ? 0 : lo;
  hi = hi > 32 ? 32 : hi;
  if (hi <= lo) return 0u;
  const uint32_t upto_hi = hi >= 32 ? 0xFFFFFFFFu : ((1u << hi) - 1u);
  return upto_hi & ~((1u << lo) - 1u);
}

// What one wave does with tile u (wave-uniform).
struct FTile {
  bool act;        // this wave computes on the tile
  int kind;        // 0 no mask, 1 window tile, 2 global columns, 3 usable keys only
  uint32_t okb;    // usable keys
  int j0;          // band: subsequence index of key 0; global columns: list index of key 0
};

// Bits [lo, hi) of a 32-bit word, per lane.
__device__ __forceinline__ uint32_t bit_range_v(int lo, int hi) {
  lo = min(max(lo, 0), 32);
  hi = min(max(hi, 0), 32);
  const uint64_t m = ((1ull << hi) - 1ull) & ~((1ull << lo) - 1ull);
  return (uint32_t)m;
}

// This lane's allowed keys of a masked tile (bit k = key k).
__device__ __forceinline__ uint32_t lane_mask(const FTile& ti, int my_i, int r, const int32_t* jr,
                                              int lane) {
  if (ti.kind == 1) return ti.okb & bit_range_v(my_i - r - ti.j0, my_i + r - ti.j0 + 1);
  if (ti.kind == 2) {
    // drop the global keys that already sit in this row's window (only this
    // lane's 16 keys matter: 8a + 4h + e)
    const int h = lane >> 5;
    uint32_t m = ti.okb;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int4 v = *reinterpret_cast<const int4*>(jr + 8 * a + 4 * h);
      const int jv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int dj = my_i - jv[e];
        const uint32_t inwin = (uint32_t)(dj <= r && dj >= -r);
        m &= ~(inwin << (8 * a + 4 * h + e));
      }
    }
    return m;
  }
  return ti.okb;
}

// Excluded scores become -inf: one bit extract and one bit-select per score.
__device__ __forceinline__ void apply_mask(f32x16& sc, uint32_t m, int lane) {
  const uint32_t m4 = m >> (4 * (lane >> 5));
#pragma unroll
  for (int a = 0; a < 4; ++a) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int bit = 8 * a + e;
      const uint32_t keep = (uint32_t)((int32_t)(m4 << (31 - bit)) >> 31);
      const uint32_t x = __float_as_uint(sc[4 * a + e]);
      sc[4 * a + e] = __uint_as_float((x & keep) | (0xFF800000u & ~keep));
    }
  }
}

// v_max3_f32 without the NaN-quieting copies the compiler adds around fmaxf.
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float d;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}

// Online-softmax update of one tile; the probabilities come out in the 16-bit
// storage format and the row sum is taken over those rounded values (the ones
// PV multiplies).
template <typename S>
__device__ __forceinline__ void softmax16(Softmax& sm, const f32x16& s, float c, svec<S, 8> (&pb)[2]) {
  float mx = max3f(s[0], s[1], s[2]);
#pragma unroll
  for (int r = 3; r < 15; r += 2) mx = max3f(mx, s[r], s[r + 1]);
  mx = max3f(mx, s[15], s[15]);
  mx = half_max(mx);
  const float mnew = fmaxf(sm.m, mx * c);
  if (__any(mnew > sm.m + TAU)) {
    const float alpha = __builtin_amdgcn_exp2f(sm.m - mnew);
    sm.l *= alpha;
#pragma unroll
    for (int r = 0; r < 16; ++r) { sm.o[0][r] *= alpha; sm.o[1][r] *= alpha; }
    sm.m = mnew;
  }
  const svec<S, 2> ones = {(S)1.0f, (S)1.0f};
  float acc = sm.l;
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2) {
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      svec<S, 2> pp;
      pp[0] = (S)__builtin_amdgcn_exp2f(fmaf(s[8 * c2 + e], c, -sm.m));
      pp[1] = (S)__builtin_amdgcn_exp2f(fmaf(s[8 * c2 + e + 1], c, -sm.m));
      pb[c2][e] = pp[0];
      pb[c2][e + 1] = pp[1];
      acc = dot2(pp, ones, acc);
    }
  }
  sm.l = acc;
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource: base, stride 0, num_records = bytes; out-of-range loads
// return zeros.
__device__ __forceinline__ i32x4 make_desc(const void* base, int bytes) {
  const uint64_t a = (uint64_t)base;
  i32x4 d;
  d[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  d[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xFFFF);
  d[2] = __builtin_amdgcn_readfirstlane(bytes);
  d[3] = 0x00020000;
  return d;
}



// ---------------------------------------------------------------------------
// Band workgroups on the bf16 fast path (the real tokens among their keys
// form a prefix).  Each of the NW waves owns 32 query rows of a residue class;
// the workgroup walks the union of their windows in steps of 64 subsequence
// keys (two 32-key halves), then the global columns: up to 32 as one extra
// half, more 64 at a time.
//
// Per wave, a step u runs in two phases, each pairing the softmax of one half
// on the VALU with eight MFMAs on the matrix cores, interleaved:
//   phase A: softmax of half 0 of u  |  QK^T of half 1 of u, PV of half 1 of u-1
//   phase B: softmax of half 1 of u  |  QK^T of half 0 of u+1, PV of half 0 of u
// so every MFMA consumes results that were computed a phase earlier.  K and V
// of a step go to LDS by buffer-to-LDS loads in two rings of four slots: the
// batch issued at step u carries K of step u+3 and V of step u+2, and step u
// waits for the batch of step u-2, so every load has two steps to land.
//
// Softmax bookkeeping: p = 2^(c*s - m) with a per-row offset m (log2 units)
// that starts at the row's score against its own key.  Every local row attends
// to itself, so its running sum is at least about 1 and cannot underflow; m
// only moves when a half's probabilities of a row sum above SUM_HI, and then
// jumps to the half's maximum while the accumulators are rescaled.  So the
// common half computes no maximum at all, and every probability stays below
// SUM_HI.
constexpr int B_STEP = 8192;            // K (or V) of one step: keys 0-31 | keys 32-63
constexpr int B_NSLOT = 4;
constexpr int B_V_OFF = B_NSLOT * B_STEP;
constexpr int B_GL_OFF = 2 * B_NSLOT * B_STEP;
constexpr int B_JR_OFF = B_GL_OFF + GL_MAX * 4;
constexpr int B_GH_OFF = B_JR_OFF + GL_MAX * 4;   // up to 32 global keys: K half | V half
constexpr int B_GH_MAX = 32;
constexpr int B_SMEM = B_GH_OFF + 2 * (B_STEP / 2);
constexpr int B_CH = 512 / NT;          // 16-byte chunks per thread per 8 KB array of a step
constexpr float SUM_HI = 16384.0f;      // 2^14
static_assert(B_CH == 2, "each thread stages two chunks of every 8 KB array");

// One 16-byte buffer load per lane into LDS at m0 = lds_base + IMM (lane l
// writes m0 + 16 l).
template <int IMM>
__device__ __forceinline__ void dma16i(i32x4 desc, int voff, uint32_t lds_base) {
  asm volatile(
      "s_add_u32 m0, %2, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen lds"
      :
      : "v"(voff), "s"(desc), "s"(lds_base), "n"(IMM)
      : "memory", "m0", "scc");
}

__device__ __forceinline__ int floordiv(int a, int b) {   // b > 0
  return a >= 0 ? a / b : -((-a + b - 1) / b);
}

// Excluded scores become -inf: bit k of m (key k of a 32-key half) keeps
// score k; this lane's registers hold keys 8(r/4) + 4h + r%4.
__device__ __forceinline__ void mask_half(f32x16& sc, uint32_t m, int h32) {
  const uint32_t m4 = m >> (4 * h32);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int bit = 8 * (r >> 2) + (r & 3);
    const uint32_t keep = (uint32_t)__builtin_amdgcn_sbfe((int)m4, bit, 1);   // 0 or ~0
    sc[r] = __uint_as_float((__float_as_uint(sc[r]) & keep) | (0xFF800000u & ~keep));
  }
}

struct BandRow {
  f32x16 o[2];   // O^T accumulators: d = 32 db + 8 (r/4) + 4 h + r%4 of query lane%32
  float m;       // offset of the exponent, log2 units (same in both half-lanes)
  float l;       // this lane's share of the row sum
  bool first;    // the offset is still to be set from the first half with a live key
};

// Probabilities of one 32-key half (16-bit, as PV multiplies them) and this
// lane's share of their sum.  The scores arrive already scaled and offset
// (c s - m0: the QK^T accumulator starts at -m0 / c and is multiplied by c in
// fp32, so Q enters the matrix cores exactly as stored), so
// p = 2^(s - x) with x the part of the row's offset beyond m0 -- zero until a
// rebase, and then the subtraction is only paid off the fast loop.
template <bool OFF, typename S>
__device__ __forceinline__ float band_exp_half(const f32x16& s, float x, svec<S, 8> (&pb)[2]) {
  const svec<S, 2> ones = {(S)1.0f, (S)1.0f};
  float acc = 0.f;
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2) {
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      svec<S, 2> q;
      q[0] = (S)__builtin_amdgcn_exp2f(OFF ? s[8 * c2 + e] - x : s[8 * c2 + e]);
      q[1] = (S)__builtin_amdgcn_exp2f(OFF ? s[8 * c2 + e + 1] - x : s[8 * c2 + e + 1]);
      pb[c2][e] = q[0];
      pb[c2][e + 1] = q[1];
      acc = dot2(q, ones, acc);
    }
  }
  return acc;
}

// The rare half: some row's probabilities summed above SUM_HI, or a row's
// offset is still unset.  Such rows move their offset to the half's maximum,
// rescale what they have accumulated and recompute the half.  s is relative
// to the row's m0.
template <typename S>
__device__ __forceinline__ void band_rebase(BandRow& st, const f32x16& s, float m0,
                                            svec<S, 8> (&pb)[2], float& ts) {
  float mx = s[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
  mx = half_max(mx);
  const float tsrow = half_sum(ts);     // both half-lanes of the row
  float delta = 0.f;
  const bool live = mx != -INFINITY;
  if (live && (tsrow > SUM_HI || st.first)) delta = (m0 + mx) - st.m;
  // nothing has been accumulated while the offset is unset
  const float alpha = st.first ? 1.0f : __builtin_amdgcn_exp2f(-delta);
  st.first = st.first && !live;
  st.l *= alpha;
#pragma unroll
  for (int r = 0; r < 16; ++r) { st.o[0][r] *= alpha; st.o[1][r] *= alpha; }
  st.m += delta;
  ts = band_exp_half<true, S>(s, st.m - m0, pb);
}

template <typename S>
__device__ __forceinline__ svec<S, 8> vfrag(const uint8_t* vt, int off) {
  const s16x4 lo = tr_read(vt + off);
  const s16x4 hi = tr_read(vt + off + 1024);
  return __builtin_bit_cast(svec<S, 8>, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Scheduling template for one phase: each of the 8 MFMAs followed by the LDS
// read(s) of the operand that replaces its own (two transposing reads for a
// V^T fragment, one for a K fragment) and a share of the softmax VALU work,
// then the rest of the softmax.
__device__ __forceinline__ void interleave_hint() {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // PV MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // its V^T fragment for the next phase
    __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);   // 6 VALU
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // QK^T MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // its K fragment for the next phase
    __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);   // 6 VALU
  }
  __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);             // the rest of the softmax
}

// MFMA operands of one phase: K of one half (A of QK^T) and V^T of one half
// (A of PV), read from LDS one phase ahead.
template <typename S>
struct PhaseOps {
  svec<S, 8> kf[4];
  svec<S, 8> vf[2][2];
};

// Where thread (wave w, lane l) stages its two 16-byte chunks q = (2 w + e) 64
// + l of each 8 KB array of a step: key row q / 8, physical chunk q % 8, the
// logical chunk that sits there (K and V swizzles).
__device__ __forceinline__ void stage_chunk(int wave, int lane, int e, int& srow, int& ck16, int& cv16) {
  const int q = (B_CH * wave + e) * 64 + lane;
  srow = q >> 3;
  ck16 = ((q & 7) ^ swz_k(srow & 31)) * 16;
  cv16 = ((q & 7) ^ swz_v(srow & 31)) * 16;
}

// The half-step pipeline over U steps of 64 keys, shared by band and global
// workgroups.  Policy callbacks:
//   issue(t, is_v)  stage K (is_v false) or V of step t into its ring slot
//   active(u)       this wave computes on step u
//   masked(u)       step u needs a per-row key mask; mask_of(u, hf) is this
//                   lane's allowed keys of half hf (bit k = key k)
//   pre()           runs while the prologue loads are in flight (it loads the
//                   rows' queries and sets their offsets)
//   idle()          (after pre) this wave has no row of its own: it only stages
//                   its share and keeps the barriers  Every step runs the same interleaved schedule; a step that is masked (or
// where this wave has no key at all: masked(u) covers those, and their mask
// is empty) applies its mask to the scores first, so its probabilities are
// exactly zero where excluded.
//
// Steps plain_lo..plain_hi are "plain" for this wave: active, without a masked
// key, and with both loads of their batch band steps (issue_band).  Their head
// is lean: a fixed load wait and no mask or issue-kind tests.
//
// With extra_half, after the last step the wave takes one more 32-key half
// whose K and V sit at smem + B_GH_OFF (K half, then V half) under the lane
// mask extra_mask() -- the few global columns of band rows.
template <typename S, class Idle, class Issue, class IssueBand, class Active, class Masked, class MaskOf,
          class Pre, class ExtraMask>
__device__ __forceinline__ void half_pipe(const int& U, int plain_lo, int plain_hi, const Idle& idle,
                                          const Issue& issue, const IssueBand& issue_band,
                                          const Active& active, const Masked& masked,
                                          const MaskOf& mask_of, const Pre& pre,
                                          const bool& extra_half, const ExtraMask& extra_mask,
                                          const QOp<S>& qo, float c, const FLane& fl, BandRow& st,
                                          int h32, uint8_t* smem) {
  // the batch of step t: K of step t+3 and V of step t+2 (those that exist);
  // two loads per thread for each
  auto batch = [&](int t) {
    if (t + 3 < U) issue(t + 3, false);
    if (t + 2 >= 0 && t + 2 < U) issue(t + 2, true);
  };
  auto kslot = [&](int t) { return smem + (t % B_NSLOT) * B_STEP; };
  auto vslot = [&](int t) { return smem + B_V_OFF + (t % B_NSLOT) * B_STEP; };
  // QK^T of one half of a step; PV of one half of a step
  // the row's fixed exponent offset, folded into every QK^T accumulator as
  // -m0 / c, the accumulator then multiplied by c = scale log2(e) in fp32: the
  // scores come out as c s - m0 (and Q is never rounded again after scaling);
  // set again after the first-half maximum of rows without an anchor
  const float inv_c = 1.0f / c;
  float m0 = st.m;
  f32x16 mvec;
#pragma unroll
  for (int i = 0; i < 16; ++i) mvec[i] = -m0 * inv_c;
  auto qk_half = [&](f32x16& sx, const uint8_t* ks) {
    f32x16 a = mvec;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
      a = mfma16(*reinterpret_cast<const svec<S, 8>*>(ks + fl.k[cc]), qo.q[cc], a);
    sx = a * c;
  };
  auto pv_half = [&](const svec<S, 8> (&pb)[2], const uint8_t* vs) {
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int db = 0; db < 2; ++db)
        st.o[db] = mfma16(vfrag<S>(vs, fl.v[db] + c2 * 2048), pb[c2], st.o[db]);
  };
  auto load_ops = [&](PhaseOps<S>& ops, const uint8_t* ks, const uint8_t* vs) {
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) ops.kf[cc] = *reinterpret_cast<const svec<S, 8>*>(ks + fl.k[cc]);
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int db = 0; db < 2; ++db) ops.vf[c2][db] = vfrag<S>(vs, fl.v[db] + c2 * 2048);
  };
  // the MFMAs of a phase: QK^T of one half into sq and PV of one half, the
  // two chains alternating so that no MFMA waits on the one just before it,
  // each followed by the LDS read of the operand that replaces its own in the
  // next phase (K rows at ks, V^T at vs): the reads
  // leave in a stream across the phase instead of in one burst, and the
  // registers of an operand are reused as soon as its MFMA has taken it
  auto phase_mfma_next = [&](f32x16& sq, PhaseOps<S>& ops, const svec<S, 8> (&pp)[2], const uint8_t* ks,
                             const uint8_t* vs) {
    f32x16 a = mvec;
    st.o[0] = mfma16(ops.vf[0][0], pp[0], st.o[0]);
    ops.vf[0][0] = vfrag<S>(vs, fl.v[0]);
    a = mfma16(ops.kf[0], qo.q[0], a);
    ops.kf[0] = *reinterpret_cast<const svec<S, 8>*>(ks + fl.k[0]);
    st.o[1] = mfma16(ops.vf[0][1], pp[0], st.o[1]);
    ops.vf[0][1] = vfrag<S>(vs, fl.v[1]);
    a = mfma16(ops.kf[1], qo.q[1], a);
    ops.kf[1] = *reinterpret_cast<const svec<S, 8>*>(ks + fl.k[1]);
    st.o[0] = mfma16(ops.vf[1][0], pp[1], st.o[0]);
    ops.vf[1][0] = vfrag<S>(vs, fl.v[0] + 2048);
    a = mfma16(ops.kf[2], qo.q[2], a);
    ops.kf[2] = *reinterpret_cast<const svec<S, 8>*>(ks + fl.k[2]);
    st.o[1] = mfma16(ops.vf[1][1], pp[1], st.o[1]);
    ops.vf[1][1] = vfrag<S>(vs, fl.v[1] + 2048);
    a = mfma16(ops.kf[3], qo.q[3], a);
    ops.kf[3] = *reinterpret_cast<const svec<S, 8>*>(ks + fl.k[3]);
    sq = a * c;
  };
  auto soft_half = [&](f32x16& sx, svec<S, 8> (&pb)[2]) {
    float ts = band_exp_half<true, S>(sx, st.m - m0, pb);
    if (__builtin_expect(__any(ts > SUM_HI || st.first), 0)) band_rebase<S>(st, sx, m0, pb, ts);
    st.l += ts;
  };

  // prologue: the batches of steps -3, -2, -1 (K of 0, 1, 2; V of 0, 1) in
  // flight, K of step 0 resident
  batch(-3);
  batch(-2);
  batch(-1);
  for (int i = threadIdx.x; i < B_STEP / 16; i += NT)   // V slot of "step -1"
    reinterpret_cast<uint4*>(smem + B_V_OFF + (B_NSLOT - 1) * B_STEP)[i] = make_uint4(0, 0, 0, 0);
  pre();
  {
    const int later = 2 * ((1 < U) + (0 < U) + (2 < U) + (1 < U));   // loads of batches -2, -1
    if (later >= 8)
      wait_loads<8>();
    else if (later >= 6)
      wait_loads<6>();
    else if (later >= 4)
      wait_loads<4>();
    else if (later >= 2)
      wait_loads<2>();
    else
      wait_loads<0>();
  }
  __syncthreads();

  f32x16 sx, sy;           // the two halves of the step being softmaxed
  svec<S, 8> pa[2], pb[2];     // probabilities of half 0 / half 1
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2) {
#pragma unroll
    for (int e = 0; e < 8; ++e) { pa[c2][e] = (S)0.0f; pb[c2][e] = (S)0.0f; }
  }
  if (U > 0) qk_half(sx, kslot(0));
  if (st.first && U > 0) {
    // rows without an anchor take the maximum of the allowed keys of their
    // first half as offset
    if (masked(0)) mask_half(sx, mask_of(0, 0), h32);
    float mx = sx[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sx[r]);
    mx = half_max(mx);
    if (mx != -INFINITY) {
      st.m = m0 + mx;
      st.first = false;
    }
    // from here on the offset in the accumulator is the row's offset
#pragma unroll
    for (int r = 0; r < 16; ++r) sx[r] -= st.m - m0;
    m0 = st.m;
#pragma unroll
    for (int i = 0; i < 16; ++i) mvec[i] = -m0 * inv_c;
  }

  auto head_of_step = [&](int u) {
    // the batch of step u-2 (K of u+1, V of u) has landed everywhere; the
    // slots the batch of step u overwrites were last read in step u-1
    const int later = 2 * ((u + 2 < U) + (u + 1 < U));   // loads of batch u-1
    if (later == 4)
      wait_loads<4>();
    else if (later == 2)
      wait_loads<2>();
    else
      wait_loads<0>();
    __syncthreads();
    batch(u);
  };
  auto slow_step = [&](int u) {
    head_of_step(u);
    const uint8_t* kc = kslot(u);
    const uint8_t* kn = kslot(u + 1);
    const uint8_t* vp = vslot(u + B_NSLOT - 1);
    const uint8_t* vc = vslot(u);
    const bool a_prev = active(u - 1), a_cur = active(u), a_next = active(u + 1);
    const bool msk = masked(u);
    // phase A
    if (a_cur && msk) mask_half(sx, mask_of(u, 0), h32);
    if (a_cur) qk_half(sy, kc + 4096);
    if (a_prev) pv_half(pb, vp + 4096);
    if (a_cur) soft_half(sx, pa);
    __builtin_amdgcn_sched_barrier(0);
    // phase B
    if (a_cur && msk) mask_half(sy, mask_of(u, 1), h32);
    if (a_next) qk_half(sx, kn);
    if (a_cur) pv_half(pa, vc);
    if (a_cur) soft_half(sy, pb);
    __builtin_amdgcn_sched_barrier(0);
  };

  // Phase A of step u multiplies K of half 1 of u and V of half 1 of u-1;
  // phase B, K of half 0 of u+1 and V of half 0 of u.  Each phase reads the
  // operands of the next one once its own MFMAs are issued: those slots were
  // filled by batches already waited for, and the batch of the next step
  // writes other slots.  Step 0's phase A reads the V slot of "step -1",
  // zeroed above, against probabilities that are zero.  A half whose
  // probabilities overflow SUM_HI leaves the loop: the rescale of O happens
  // outside it (keeping O in place through the loop), and the remaining steps
  // run on the slow path.
  if (idle()) {
    for (int u = 0; u < U; ++u) head_of_step(u);
    return;
  }
  PhaseOps<S> ops;
  if (U > 0) load_ops(ops, kslot(0) + 4096, vslot(B_NSLOT - 1) + 4096);
  int rare_at = 0;
  float ts_rare = 0.f;
  int u = 0;
  for (; u < U; ++u) {
    const bool plain = u >= plain_lo && u <= plain_hi;
    if (plain) {
      // batch u-2 has landed (the 4 loads of batch u-1 may still fly)
      wait_loads<4>();
      __syncthreads();
      issue_band(u + 3, false);
      issue_band(u + 2, true);
    } else {
      head_of_step(u);
    }
    const bool msk = !plain && masked(u);
    if (msk) mask_half(sx, mask_of(u, 0), h32);
    // phase A
    phase_mfma_next(sy, ops, pb, kslot(u + 1), vslot(u));
    float ts = band_exp_half<false, S>(sx, 0.f, pa);   // st.m == m0 in this loop
    interleave_hint();
    if (__builtin_expect(__any(ts > SUM_HI), 0)) {
      rare_at = 1;
      ts_rare = ts;
      break;
    }
    st.l += ts;
    if (msk) mask_half(sy, mask_of(u, 1), h32);
    // phase B (the operands read for step u+1 = U are never used; the reads
    // stay inside the ring)
    phase_mfma_next(sx, ops, pa, kslot(u + 1) + 4096, vslot(u) + 4096);
    ts = band_exp_half<false, S>(sy, 0.f, pb);
    interleave_hint();
    if (__builtin_expect(__any(ts > SUM_HI), 0)) {
      rare_at = 2;
      ts_rare = ts;
      break;
    }
    st.l += ts;
  }
  if (rare_at == 1) {
    // half 0 of step u overflowed: rescale, then phase B of step u
    band_rebase<S>(st, sx, m0, pa, ts_rare);
    st.l += ts_rare;
    if (masked(u)) mask_half(sy, mask_of(u, 1), h32);
    if (u + 1 < U) qk_half(sx, kslot(u + 1));
    pv_half(pa, vslot(u));
    soft_half(sy, pb);
    ++u;
  } else if (rare_at == 2) {
    // half 1 of step u overflowed
    band_rebase<S>(st, sy, m0, pb, ts_rare);
    st.l += ts_rare;
    ++u;
  }
  for (; u < U; ++u) slow_step(u);
  // PV of half 1 of the last step (its V landed with the batch of step U-3)
  if (U > 0) pv_half(pb, vslot(U - 1) + 4096);
  if (extra_half) {
    // staged before the loop; every step's wait and barrier has passed since
    const uint8_t* gk = smem + B_GH_OFF;
    f32x16 sg;
    qk_half(sg, gk);
    mask_half(sg, extra_mask(), h32);
    svec<S, 8> pg[2];
    soft_half(sg, pg);
    pv_half(pg, gk + B_STEP / 2);
  }
}

// Padding of the positions rho + i s, i in [lo, hi), read from the local
// attention mask by the whole workgroup: the first padded index (none_val if
// there is none) and the number of padded ones.  Ends with a barrier.
__device__ __forceinline__ void pad_scan(const float* lmb, int rho, int s, int lo, int hi,
                                         int none_val, int& first, int& ninv) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  first = none_val;
  ninv = 0;
  for (int i0 = lo + tid; i0 < hi; i0 += 4 * NT) {
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = i0 + e * NT;
      v[e] = i < hi ? lmb[rho + i * s] : 1.0f;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool pad = v[e] == 0.0f;
      const int i = i0 + e * NT;
      first = pad && i < first ? i : first;
      ninv += pad ? 1 : 0;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const int f2 = __shfl_xor(first, o);
    first = f2 < first ? f2 : first;
    ninv += __shfl_xor(ninv, o);
  }
  __shared__ int s_pad[2 * NW];
  if (lane == 0) {
    s_pad[2 * wave] = first;
    s_pad[2 * wave + 1] = ninv;
  }
  __syncthreads();
  first = none_val;
  ninv = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    first = s_pad[2 * w] < first ? s_pad[2 * w] : first;
    ninv += s_pad[2 * w + 1];
  }
}

// Band workgroup on the fast path.  It does not wait for the compaction of its
// batch row before it starts: the padding of the keys its band steps can read
// and of its own rows comes straight from the local attention mask, and the
// row's global-position list is needed only for the global columns, which
// follow the band steps; the wait for it sits after the first key batches are
// issued.  Returns false, having written nothing, when the real tokens among
// those keys are not a prefix of them; the general path then takes the
// workgroup.
template <typename S>
__device__ bool band_wg_fast(const Params& p, int b, int h, int local, int s, uint8_t* smem) {
  constexpr int RB = 128;
  const int tid = threadIdx.x, lane = tid & 63, h32 = lane >> 5, qi = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int n = p.n;
  int rho = 0, nr = 0;
  for (rho = 0; rho < s; ++rho) {
    nr = (n - rho + s - 1) / s;
    const int nb = (nr + ROWS_WG - 1) / ROWS_WG;
    if (local < nb) break;
    local -= nb;
  }
  const int R0 = local * ROWS_WG;
  const int r = p.r;
  // this head's K and V rows: rs bytes apart (offsets of every key a step can
  // name fit in 32 bits: the plan takes this path only then)
  const uint8_t* kh = in_head(p, p.K, 0, b, h);
  const uint8_t* vh = in_head(p, p.V, 0, b, h);
  const int rs = p.in_rs[0];
  auto span = [&](int rows) { return rows > 0 ? (rows - 1) * rs + RB : 0; };

  // band steps: step u holds subsequence keys kb0 + 64 u .. + 63
  const int kb = R0 - r;
  const int T = (ROWS_WG - 1 + 2 * r) / 64 + 1;
  const int t_lo = (-kb - 63 > 0) ? (-kb - 63 + 63) / 64 : 0;
  const int kb0 = kb + 64 * t_lo;

  const int R0w = R0 + 32 * wave;
  const int my_i = R0w + qi;
  const bool row_in = my_i < nr;
  const int my_pos = rho + (row_in ? my_i : 0) * s;

  // Padding of the subsequence keys [sc_lo, sc_hi) that any band step can
  // read, and the flags of this lane's row, from the masks.
  const float* lmb = p.lmask + (int64_t)b * n;
  const float* gmb = p.gmask + (int64_t)b * n;
  const float l_row = row_in ? lmb[my_pos] : 0.0f;
  const float g_row = row_in ? gmb[my_pos] : 0.0f;
  // this lane's query row and its own key row (the initial offset), in the
  // same round trip as the masks
  QOp<S> qo;
  qo.load(in_head(p, p.Q, 0, b, h) + (int64_t)my_pos * rs, row_in, h32);
  uint4 kdiag[4];
  {
    const uint8_t* krow = kh + (int64_t)my_pos * rs + 64 * h32;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) kdiag[cc] = *reinterpret_cast<const uint4*>(krow + 16 * cc);
  }
  // the output row, kept in registers: reloading the pointer at the end
  // would be a scalar load that misses by then
  const int sc_lo = kb0 > 0 ? kb0 : 0;
  const int sc_hi = kb + 64 * T < nr ? kb + 64 * T : nr;
  int first, ninv;
  pad_scan(lmb, rho, s, sc_lo, sc_hi, nr, first, ninv);
  // real tokens among the readable keys must be exactly [.., first)
  if (ninv != 0 && ninv != sc_hi - first) return false;
  const int nrv = first;                                 // subsequence keys below are real
  const int nv_pos = ninv ? rho + first * s : n;         // positions below are readable

  int t_hi = nrv - 1 - kb >= 0 ? (nrv - 1 - kb) / 64 : -1;
  if (t_hi > T - 1) t_hi = T - 1;
  const int nband = R0 < nrv && t_hi >= t_lo ? t_hi - t_lo + 1 : 0;
  // the global columns, known once the row's compaction is visible
  int g = 0, gmain = 0, U = nband;

  const uint8_t my_fl = (uint8_t)((l_row != 0.0f ? 1 : 0) | (l_row != 0.0f && g_row != 0.0f ? 2 : 0));
  const bool wave_work = __any(row_in && (my_fl & 3) == 1);   // the wave has a local row

  // this wave's band steps with any key of its windows [ua, ub], and those
  // with every key inside all of its rows' windows [fa, fb]
  const int lo_w = R0w - r > 0 ? R0w - r : 0;
  const int hi_w = (R0w + 31 + r < nrv - 1) ? R0w + 31 + r : nrv - 1;
  const int ua = floordiv(lo_w - kb0, 64);
  const int ub = floordiv(hi_w - kb0, 64);
  const int fl_lo = (R0w + 31 - r > 0) ? R0w + 31 - r : 0;
  const int fl_hi = (R0w + r < nrv - 1) ? R0w + r : nrv - 1;
  const int fa = floordiv(fl_lo - kb0 + 63, 64);
  const int fb = floordiv(fl_hi - 63 - kb0, 64);
  auto active = [&](int u) {
    return u >= 0 && u < U && (u < nband ? (u >= ua && u <= ub) : wave_work);
  };
  auto masked = [&](int u) { return u < fa || u > fb || u >= nband; };

  // Q is complete here (the scan waited for every load): take it out of the
  // compiler's view of outstanding loads, since the loop below issues
  // buffer-to-LDS loads the compiler does not count, and a wait it placed for
  // Q inside the loop would also wait for those.
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) asm volatile("" : "+v"(qo.q[cc]));
  BandRow st;
  {
    // the row's own score sets the initial offset (this lane's 32 channels,
    // then both half-lanes)

    float sd = 0.f;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const svec<S, 8> k8 = __builtin_bit_cast(svec<S, 8>, kdiag[cc]);
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const svec<S, 2> a = {qo.q[cc][e], qo.q[cc][e + 1]};
        const svec<S, 2> bb = {k8[e], k8[e + 1]};
        sd = dot2(a, bb, sd);
      }
    }
    st.m = p.c * half_sum(sd);   // c s_ii, the offset in the exponent's units
    asm volatile("" : "+v"(st.m));
  }
  st.l = 0.f;
  st.first = false;
#pragma unroll
  for (int i = 0; i < 16; ++i) { st.o[0][i] = 0.f; st.o[1][i] = 0.f; }
  FLane fl;
  fl.init(lane);

  int32_t* gl = reinterpret_cast<int32_t*>(smem + B_GL_OFF);
  int32_t* jr = reinterpret_cast<int32_t*>(smem + B_JR_OFF);
  const i32x4 dk = make_desc(kh, span(nv_pos));
  const i32x4 dv = make_desc(vh, span(nv_pos));
  int kbase[B_CH], vbase[B_CH];
  const int step_b = 64 * s * rs;
#pragma unroll
  for (int e = 0; e < B_CH; ++e) {
    int srow, ck16, cv16;
    stage_chunk(wave, lane, e, srow, ck16, cv16);
    const int rowoff = (rho + (kb0 + srow) * s) * rs;
    kbase[e] = rowoff + ck16;
    vbase[e] = rowoff + cv16;
  }
  const int32_t* gidx_b = p.gidx + (int64_t)b * n;
  const uint32_t lds_w = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)smem) +
                         wave * (B_CH * 1024);
  // K (is_v false) or V of step t into its ring slot: band steps are strided
  // subsequence rows, global steps the listed global positions (real tokens
  // anywhere in the row, so read through a range over all n rows)
  auto issue = [&](int t, bool is_v) {
    const uint32_t base = lds_w + (is_v ? B_V_OFF : 0) + (t % B_NSLOT) * B_STEP;
    int off[B_CH];
    i32x4 d = is_v ? dv : dk;
    if (t < nband) {
      const int adv = t * step_b;
#pragma unroll
      for (int e = 0; e < B_CH; ++e) off[e] = (is_v ? vbase[e] : kbase[e]) + adv;
    } else {
      d[2] = span(n);
#pragma unroll
      for (int e = 0; e < B_CH; ++e) {
        int srow, ck16, cv16;
        stage_chunk(wave, lane, e, srow, ck16, cv16);
        const int idx = (t - nband) * 64 + srow;
        const bool in = idx < gmain;
        const int rowoff = gl[in ? idx : 0] * rs;
        off[e] = in ? rowoff + (is_v ? cv16 : ck16) : OOB_OFF;
      }
    }
    dma16i<0>(d, off[0], base);
    dma16i<1024>(d, off[1], base);
  };
  auto issue_band = [&](int t, bool is_v) {   // t < nband
    const uint32_t base = lds_w + (is_v ? B_V_OFF : 0) + (t % B_NSLOT) * B_STEP;
    const int adv = t * step_b;
    const i32x4 d = is_v ? dv : dk;
    dma16i<0>(d, (is_v ? vbase[0] : kbase[0]) + adv, base);
    dma16i<1024>(d, (is_v ? vbase[1] : kbase[1]) + adv, base);
  };
  auto fill = [&]() {
    for (int j = tid; j < gmain; j += NT) {
      const int pos = coherent_load(gidx_b + j);
      const int dp = pos - rho;
      gl[j] = pos;
      jr[j] = (dp >= 0 && dp % s == 0) ? dp / s : JREL_NONE;
    }
  };
  auto mask_of = [&](int u, int hf) {
    uint32_t m;
    if (u < nband) {
      const int j0 = kb0 + 64 * u + 32 * hf;
      m = bit_range(-j0, nrv - j0) & bit_range_v(my_i - r - j0, my_i + r - j0 + 1);
    } else {
      FTile ti;
      ti.act = true;
      ti.kind = 2;
      ti.j0 = (u - nband) * 64 + 32 * hf;
      ti.okb = bit_range(0, gmain - ti.j0);
      m = lane_mask(ti, my_i, r, jr + ti.j0, lane);
    }
    return m;
  };

  // the global columns: wait for the row's compaction, then count them; up to
  // 32 of them take one extra half after the band steps (their K and V
  // staged once, below), more take whole pipeline steps
  bool gh = false;
  auto learn_globals = [&]() {
    if (wait_ready(p, b)) {
      g = coherent_load(p.gcnt + b);
      if (g > p.max_global) g = p.max_global;
    }
    gmain = g < GL_MAX ? g : GL_MAX;
    gh = R0 < nrv && gmain > 0 && gmain <= B_GH_MAX;
    U = nband + (R0 < nrv && !gh ? (gmain + 63) / 64 : 0);
  };
  // K and V rows of the <= 32 global keys into the extra half (waves 0 and 1
  // stage its 32 rows, two chunks per lane per array), after gl[] is visible
  auto stage_gh = [&]() {
    if (wave < 2) {
      i32x4 d = dk;
      d[2] = span(n);
      i32x4 e = dv;
      e[2] = span(n);
      const uint32_t base = lds_w + (uint32_t)B_GH_OFF;   // this wave's 2 KB of the K half
      int offk[B_CH], offv[B_CH];
#pragma unroll
      for (int c2 = 0; c2 < B_CH; ++c2) {
        int srow, ck16, cv16;
        stage_chunk(wave, lane, c2, srow, ck16, cv16);
        const bool in = srow < gmain;
        const int rowoff = gl[in ? srow : 0] * rs;
        offk[c2] = in ? rowoff + ck16 : OOB_OFF;
        offv[c2] = in ? rowoff + cv16 : OOB_OFF;
      }
      dma16i<0>(d, offk[0], base);
      dma16i<1024>(d, offk[1], base);
      dma16i<0>(e, offv[0], base + B_STEP / 2);
      dma16i<1024>(e, offv[1], base + B_STEP / 2);
    }
  };
  // the global-position list must be in LDS before a global step is staged;
  // with fewer band steps than the prologue stages, that is before it
  const bool early_fill = nband < B_NSLOT - 1;
  if (early_fill) {
    learn_globals();
    fill();
    __syncthreads();
    if (gh) stage_gh();
  }
  auto pre = [&]() {
    if (!early_fill) {
      learn_globals();
      fill();
      if (gh) {
        __syncthreads();
        stage_gh();
      }
    }
  };
  auto gh_mask = [&]() {
    FTile ti;
    ti.act = true;
    ti.kind = 2;
    ti.j0 = 0;
    ti.okb = bit_range(0, gmain);
    return lane_mask(ti, my_i, r, jr, lane);
  };
  auto idle = [&]() { return !wave_work; };
  // plain steps of this wave: every key inside all of its rows' windows, and
  // the batch (K of u+3, V of u+2) made of band steps
  const int plain_lo = fa > 0 ? fa : 0;
  const int plain_hi = fb < nband - 4 ? fb : nband - 4;
  half_pipe(U, plain_lo, plain_hi, idle, issue, issue_band, active, masked, mask_of, pre, gh, gh_mask,
            qo, p.c, fl, st, h32, smem);

  if (g > GL_MAX && R0 < nrv) {
    // global columns past the LDS copy, 32 at a time through the first K and
    // V slots (the older Softmax helpers keep the same offset convention)
    Softmax sm;
    sm.m = st.m;
    sm.l = st.l;
    sm.o[0] = st.o[0];
    sm.o[1] = st.o[1];
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kh, span(n));
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vh, span(n));
    const int U2 = (g - GL_MAX + KT - 1) / KT;
    for (int u2 = 0; u2 < U2; ++u2) {
      __syncthreads();
      const int jb = GL_MAX + u2 * KT;
      for (int j = tid; j < KT; j += NT) {
        const int idx = jb + j;
        const int pos = idx < g ? coherent_load(gidx_b + idx) : 0;
        const int dp = pos - rho;
        gl[j] = pos;
        jr[j] = (idx < g && dp >= 0 && dp % s == 0) ? dp / s : JREL_NONE;
      }
      __syncthreads();
      for (int q = tid; q < 256; q += NT) {     // chunk of the 32-key tile
        const int row = q >> 3;
        const bool in = jb + row < g;
        const int rowoff = gl[row] * rs;
        const int k16 = ((q & 7) ^ swz_k(row)) * 16, v16 = ((q & 7) ^ swz_v(row)) * 16;
        *reinterpret_cast<uint4*>(smem + q * 16) = bload(rk, in ? rowoff + k16 : OOB_OFF);
        *reinterpret_cast<uint4*>(smem + B_V_OFF + q * 16) = bload(rv, in ? rowoff + v16 : OOB_OFF);
      }
      __syncthreads();
      if (wave_work) {
        FTile ti;
        ti.act = true;
        ti.kind = 2;
        ti.okb = bit_range(0, g - jb);
        ti.j0 = 0;
        f32x16 sc = fqk(qo, smem, fl);
        apply_mask(sc, lane_mask(ti, my_i, r, jr, lane), lane);
        svec<S, 8> pq[2];
        softmax16<S>(sm, sc, p.c, pq);
        fpv<S>(sm.o, pq, smem + B_V_OFF, fl);
      }
    }
    st.m = sm.m;
    st.l = sm.l;
    st.o[0] = sm.o[0];
    st.o[1] = sm.o[1];
  }

  // normalise and store (global rows are written by the merge of their key
  // slices, padded rows get exact zeros).  The wave's 32 rows are staged in
  // LDS (free once every wave is past the ring) and leave as whole 128-byte
  // rows, eight lanes per row, with the agent-scope write-through policy: the
  // lines are not left dirty in L2 for the end of the kernel (or a global
  // merge's release) to write back, and no line is written in pieces.
  const float lt = half_sum(st.l);
  const bool keep = row_in && (my_fl & 2) == 0;
  const bool valid = (my_fl & 1) != 0;
  const float inv = valid ? 1.0f / lt : 0.0f;
  __syncthreads();
  uint8_t* stg = smem + wave * 4096;   // 32 rows x 128 bytes, 16-byte chunks swizzled by row
#pragma unroll
  for (int db = 0; db < 2; ++db) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      svec<S, 4> t;
#pragma unroll
      for (int e = 0; e < 4; ++e) t[e] = (S)(valid ? st.o[db][4 * a + e] * inv : 0.0f);
      const int chunk = (4 * db + a) ^ (qi & 7);
      *reinterpret_cast<svec<S, 4>*>(stg + qi * 128 + chunk * 16 + h32 * 8) = t;
    }
  }
  // the head's rows span (n - 1) ostr + RB bytes (below 2^31: the plan
  // takes the token-major layout only then)
  const int ostr = o_stride(p, RB);
  const __amdgpu_buffer_rsrc_t rout = make_rsrc(o_row(p, b, h, 0, RB), (n - 1) * ostr + RB);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 8 * i + (lane >> 3), c = lane & 7;
    const i32x4 v = *reinterpret_cast<const i32x4*>(stg + row * 128 + ((c ^ (row & 7)) * 16));
    const int off = __shfl(my_pos, row) * ostr + c * 16;
    if (__shfl(keep ? 1 : 0, row)) store_wt(rout, off, v);
  }
  return true;
}

// Global-row workgroups on the bf16 fast path: up to NW query tiles of 32
// global rows (one per wave) against one key slice [j_start, j_end), through
// the same pipeline; each wave leaves an unnormalised partial result (offset,
// sum, O) that the merge of the tile's key slices combines.  The rows' offsets
// are set from the maximum of their first half (there is no own key in a
// slice to anchor them).  Like the band path, the workgroup reads the padding
// of its slice from the mask and issues its first key batches before it waits
// for the row's compaction (which names its query rows).  Returns false,
// having written nothing, when the slice's real tokens are not a prefix of it.
template <typename S>
__device__ bool global_wg_fast(const Params& p, int b, int h, int qg, int sp, uint8_t* smem) {
  constexpr int RB = 128;
  const int tid = threadIdx.x, lane = tid & 63, h32 = lane >> 5, qi = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int n = p.n;
  const int32_t* gidx_b = p.gidx + (int64_t)b * n;
  const int j_start = sp * p.ksplit;
  int j_end = j_start + p.ksplit;
  if (j_end > n) j_end = n;
  int first, ninv;
  pad_scan(p.lmask + (int64_t)b * n, 0, 1, j_start, j_end, j_end, first, ninv);
  if (ninv != 0 && ninv != j_end - first) return false;
  const int j_use = first;                          // keys of the slice that are real tokens
  int U = j_use > j_start ? (j_use - j_start + 63) / 64 : 0;

  // the query tiles, known once the row's compaction is visible
  int g = 0, qt = 0, qpos_row = 0;
  bool wave_work = false, qok = false;
  QOp<S> qo;
  auto load_rows = [&]() {   // while the first keys are in flight
    if (wait_ready(p, b)) {
      g = coherent_load(p.gcnt + b);
      if (g > p.max_global) g = p.max_global;
    }
    const int nqt_b = (g + 31) / 32;
    if (qg * NW >= nqt_b) {                         // no query tile here: drain and leave
      U = 0;
      return;
    }
    qt = qg * NW + wave;
    wave_work = qt < nqt_b;
    const int qidx = qt * 32 + qi;
    qok = wave_work && qidx < g;
    const int qpos = qok ? coherent_load(gidx_b + qidx) : 0;
    qpos_row = qpos;
    qo.load(in_head(p, p.Qg, 1, b, h) + (int64_t)qpos * p.in_rs[1], qok, h32);
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) asm volatile("" : "+v"(qo.q[cc]));
  };
  BandRow st;
  st.m = 0.f;
  st.l = 0.f;
  st.first = true;
#pragma unroll
  for (int i = 0; i < 16; ++i) { st.o[0][i] = 0.f; st.o[1][i] = 0.f; }
  FLane fl;
  fl.init(lane);

  // this head's Kg and Vg rows, rsg bytes apart (offsets in 32 bits: the
  // plan takes this path only then)
  const int rsg = p.in_rs[2];
  const int span_g = j_use > 0 ? (j_use - 1) * rsg + RB : 0;
  const i32x4 dk = make_desc(in_head(p, p.Kg, 2, b, h), span_g);
  const i32x4 dv = make_desc(in_head(p, p.Vg, 2, b, h), span_g);
  int kbase[B_CH], vbase[B_CH];
#pragma unroll
  for (int e = 0; e < B_CH; ++e) {
    int srow, ck16, cv16;
    stage_chunk(wave, lane, e, srow, ck16, cv16);
    const int rowoff = (j_start + srow) * rsg;
    kbase[e] = rowoff + ck16;
    vbase[e] = rowoff + cv16;
  }
  const uint32_t lds_w = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)smem) +
                         wave * (B_CH * 1024);
  auto issue = [&](int t, bool is_v) {
    const uint32_t base = lds_w + (is_v ? B_V_OFF : 0) + (t % B_NSLOT) * B_STEP;
    const int adv = t * 64 * rsg;
    const i32x4 d = is_v ? dv : dk;
    dma16i<0>(d, (is_v ? vbase[0] : kbase[0]) + adv, base);
    dma16i<1024>(d, (is_v ? vbase[1] : kbase[1]) + adv, base);
  };
  auto active = [&](int u) { return u >= 0 && u < U && wave_work; };
  // only the last step can hold keys past the slice's real tokens
  auto masked = [&](int u) { return j_start + 64 * u + 64 > j_use; };
  auto mask_of = [&](int u, int hf) { return bit_range(0, j_use - (j_start + 64 * u + 32 * hf)); };
  auto idle = [&]() { return !wave_work; };
  const bool no_extra = false;
  half_pipe(U, 1, 0, idle, issue, issue, active, masked, mask_of, load_rows, no_extra,
            [] { return 0u; }, qo, p.c, fl, st, h32, smem);

  const float lt = half_sum(st.l);
  // a slice with no real key leaves an empty partial
  if (qok)
    store_global_partial(p, (((int64_t)b * p.H + h) * p.nqt + qt) * p.nsplit + sp, qi, h32, st.o,
                         st.first ? -INFINITY : st.m, lt);
  if (wave_work) finish_global_tile<S, true>(p, b, h, qt, g, lane, qpos_row);
  return true;
}

template <typename S>
constexpr int smem_bytes() {
  return (is16<S>() && B_SMEM > smem_bytes_general<S>()) ? B_SMEM : smem_bytes_general<S>();
}

// The logical workgroup order keeps neighbouring query blocks of one head on
// one XCD (workgroups are dealt to the 8 XCDs round-robin by hardware id), so
// that their overlapping key halos are served by that XCD's L2.
__device__ __forceinline__ int xcd_remap(int pid, int count) {
  const int q = count / 8, rem = count % 8;
  const int x = pid % 8, idx = pid / 8;
  return x * q + (x < rem ? x : rem) + idx;
}

// Dispatch order: the compaction workgroups (one per batch row, padded to a
// multiple of 8 so that the band workgroups behind them keep their XCD
// placement), then the first band_pre band workgroups, then the global-row
// workgroups, then the rest of the band workgroups.  When the grid fits one
// round of workgroup slots, band_pre is every band workgroup and the
// global-row ones fill the gaps behind them.  On longer grids they follow the
// first round: they start as slots free up (the compaction is done by then)
// and finish under the later rounds, where at the end of the grid they would
// run on as a tail (each takes several band workgroups' time).  band_pre and
// the global-row count are multiples of 8, so every band workgroup keeps the
// XCD its band index names.
template <typename S>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2))) void attn_kernel(Params p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int bid = blockIdx.x;
  if (bid < p.n_comp_wg) {
    if (bid < p.B) compact_row(p, bid, smem);
    return;
  }
  bid -= p.n_comp_wg;
  if (bid >= p.band_pre && bid < p.band_pre + p.n_glob_wg) {
    const int lg = bid - p.band_pre;
    if (lg >= p.B * p.H * p.nqg * p.nsplit) return;
    const int sp = lg % p.nsplit;
    int t = lg / p.nsplit;
    const int qg = t % p.nqg;
    t /= p.nqg;
    const int h = t % p.H;
    const int b = t / p.H;
    if constexpr (is16<S>()) {
      if (global_wg_fast<S>(p, b, h, qg, sp, smem)) return;
    }
    if (!wait_ready(p, b)) return;
    global_wg<S>(p, b, h, qg, sp, smem);
  } else {
    if (bid >= p.band_pre) bid -= p.n_glob_wg;
    if (p.comp_fold && bid < p.B) {
      // the band grid fits one round of slots here, so the compacting
      // workgroups are resident beside every workgroup that waits for them
      compact_row(p, bid, smem);
      __syncthreads();
    }
    int lb = xcd_remap(bid, p.n_band_wg), part = 0;
    if (p.bparts > 1) {
      part = lb % p.bparts;
      lb /= p.bparts;
    }
    const int b = lb / p.blocks_per_b;
    const int rem = lb - b * p.blocks_per_b;
    int h, local, s;
    if (p.uni_stride > 0) {
      h = rem / p.blocks_per_head;
      local = rem - h * p.blocks_per_head;
      s = p.uni_stride;
    } else if (p.H <= MAXH_ARG) {
      h = 0;
      while (p.hb[h + 1] <= rem) ++h;
      local = rem - p.hb[h];
      s = p.hs[h];
    } else {
      h = 0;
      while (p.head_blk[h + 1] <= rem) ++h;
      local = rem - p.head_blk[h];
      s = p.head_stride[h];
    }
    if constexpr (is16<S>()) {
      if (p.band_fast && band_wg_fast<S>(p, b, h, local, s, smem)) return;
    }
    if (!wait_ready(p, b)) return;
    band_wg<S>(p, b, h, local, s, lb, part, smem);
  }
}

}  // namespace lwk
