// lwattn.hip -- host runtime and C ABI of the Longformer window + global
// attention forward (declared in include/lwattn.h).
//
// A plan validates the configuration once, derives the launch geometry and
// owns the device workspace; a forward only enqueues three kernels on the
// caller's stream (see kernels.hpp) and never allocates or synchronizes.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "kernels.hpp"
#include "backward.hpp"
#include "causal.hpp"
#include "blocksparse.hpp"
#include "layer.hpp"
#include "probe.hpp"

#include <rocblas/rocblas.h>
#include "lwattn.h"

namespace {

constexpr int kNumKernels = 1;
// backward kernel slots: compaction, dQ, chunk sums, merge, dK/dV (the fp32
// storage path runs the compaction, dQ and dK/dV only)
constexpr int kNumBwKernels = 5;

// LWATTN_DEBUG=1 in the environment prints every failing HIP call to stderr.
bool hip_ok(hipError_t e, const char* what) {
  if (e == hipSuccess) return true;
  static const bool debug = [] {
    const char* v = std::getenv("LWATTN_DEBUG");
    return v && *v && *v != '0';
  }();
  if (debug) std::fprintf(stderr, "lwattn: %s failed: %s\n", what, hipGetErrorString(e));
  return false;
}

}  // namespace

// Launch geometry of the forward (attn_kernel), shared by the plan and the
// allocation-free entry point.
struct FwdGeom {
  int nqt = 0, nqg = 0, nsplit = 0, ksplit = 0;
  int n_comp_wg = 0, n_glob_wg = 0, n_band_wg = 0, blocks_per_b = 0;
  int band_pre = 0;   // band workgroups dispatched before the global-row ones
  int uni_stride = 0, blocks_per_head = 0, band_fast = 0;
  int n_band_blk = 0;  // band blocks (B * blocks_per_b)
  int bparts = 1;      // key parts per band block on the register-staged path
  int comp_fold = 0;   // band workgroups 0 .. B-1 compact row bid first (no compaction workgroups)
  size_t smem = 0;
};

struct lwattn_plan_s {
  lwattn_config cfg;
  std::vector<int32_t> gap;
  int device = 0;
  // geometry
  int nqt = 0, nqg = 0, nsplit = 0, ksplit = 0;
  int n_comp_wg = 0, n_glob_wg = 0, n_band_wg = 0, blocks_per_b = 0;
  int uni_stride = 0, blocks_per_head = 0;
  int band_fast = 0;
  std::vector<int32_t> stride_host, blk_host;
  size_t smem = 0;
  FwdGeom geom;
  // workspace
  uint8_t* flags = nullptr;
  int32_t* gidx = nullptr;
  int32_t* gcnt = nullptr;
  int32_t* status = nullptr;
  float* part_o = nullptr;
  float* part_ml = nullptr;
  int32_t* tile_cnt = nullptr;
  float* bpart_o = nullptr;   // band blocks' key parts (bparts > 1)
  float* bpart_ml = nullptr;
  int32_t* bcnt = nullptr;
  int32_t* ready = nullptr;   // [B] epoch of the last compaction of each batch row
  uint64_t* ready_cnt = nullptr;   // [B] (epoch << 32) | global count, written by the backward's compaction
  int32_t* fault = nullptr;   // sticky: a workgroup gave up waiting for its row
  int32_t epoch = 0;          // forwards launched (kept in 1 .. INT32_MAX - 1)
  bool inject_timeout = false; // fault test: the next forward's (or 16-bit backward's) waits give up
  int32_t* head_stride = nullptr;
  int32_t* head_blk = nullptr;
  // backward: 64-row blocks per head (all residue classes), per-row statistics
  int32_t* head_blk64 = nullptr;
  int blocks64_per_b = 0;
  int ncu = 256;   // compute units of the plan's device
  float2* stats = nullptr;
  // bf16 backward: the global rows' and global keys' sums over position chunks
  int gsplit = 0, gchunk = 0;
  float* gq = nullptr;
  float* gk = nullptr;
  float* gml = nullptr;
  // timing
  int timing_cap = 0;
  int timing_calls = 0;
  int timing_every = 1;    // record the events of every k-th forward
  int64_t timing_seen = 0; // forwards since timing was enabled
  std::vector<hipEvent_t> events;   // (kNumKernels + 1) per recorded forward
  int bw_calls = 0;                 // backwards recorded
  int64_t bw_seen = 0;              // backwards since timing was enabled
  std::vector<hipEvent_t> bw_events;   // 2 kNumBwKernels per recorded backward
  std::vector<uint8_t> bw_launched;    // per recorded backward: bit k = slot k's kernel ran
};

static void free_plan(lwattn_plan_s* p) {
  if (!p) return;
  (void)hipFree(p->flags);
  (void)hipFree(p->gidx);
  (void)hipFree(p->gcnt);
  (void)hipFree(p->status);
  (void)hipFree(p->part_o);
  (void)hipFree(p->part_ml);
  (void)hipFree(p->tile_cnt);
  (void)hipFree(p->bpart_o);
  (void)hipFree(p->bpart_ml);
  (void)hipFree(p->bcnt);
  (void)hipFree(p->ready);
  (void)hipFree(p->ready_cnt);
  (void)hipFree(p->fault);
  (void)hipFree(p->head_stride);
  (void)hipFree(p->head_blk);
  (void)hipFree(p->head_blk64);
  (void)hipFree(p->stats);
  (void)hipFree(p->gq);
  (void)hipFree(p->gk);
  (void)hipFree(p->gml);
  for (hipEvent_t e : p->events) (void)hipEventDestroy(e);
  for (hipEvent_t e : p->bw_events) (void)hipEventDestroy(e);
  delete p;
}

static int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }


// ---------------------------------------------------------------------------
// Encoder layer around the attention (16-bit storage, the plan's): the plan
// gives B, H, n, the window, dilation and globals; the layer object owns the
// intermediate buffers and a rocBLAS handle.
// One GEMM shape of the layer in hipBLASLt: row-major Y[M, N] (fp32) =
// X[M, K] W[K, N] (16-bit), set up as the column-major product
// Y^T = W^T X^T; or, with the bias epilogue, Y = X W + bias rounded once to
// the 16-bit type (bias [N] of that type, added in fp32).  At set-up the (up
// to 8) algorithms its heuristic ranks first are timed on scratch operands
// and the fastest is kept; when hipBLASLt has none for a shape, the layer
// runs it in rocBLAS (fp32 result, the bias added by the split kernel).
struct LtGemm {
  bool ok = false;
  bool bias16 = false;   // bias epilogue, 16-bit result
  int64_t M = 0, N = 0, K = 0, ldw = 0;
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t lw = nullptr, lx = nullptr, ly = nullptr;
  hipblasLtMatmulAlgo_t algo;
  size_t ws = 0;
};

static void lt_free(LtGemm& g) {
  if (g.desc) (void)hipblasLtMatmulDescDestroy(g.desc);
  if (g.lw) (void)hipblasLtMatrixLayoutDestroy(g.lw);
  if (g.lx) (void)hipblasLtMatrixLayoutDestroy(g.lx);
  if (g.ly) (void)hipblasLtMatrixLayoutDestroy(g.ly);
  g = LtGemm();
}

// Scratch operands for timing the candidates: W, X (16-bit), Y (fp32) and
// the workspace, zero-filled, on a stream of their own.
struct LtTune {
  void *w = nullptr, *x = nullptr, *ws = nullptr;
  float* y = nullptr;
  size_t ws_cap = 0;
  hipStream_t stream = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
};

static void lt_setup(hipblasLtHandle_t h, LtGemm& g, hipDataType dt, int64_t M, int64_t N, int64_t K, int64_t ldw,
                     const LtTune& tu, bool bias16 = false) {
  g.M = M; g.N = N; g.K = K; g.ldw = ldw;
  if (!h || !tu.stream || M == 0 || N == 0 || K == 0) return;
  const hipblasOperation_t op = HIPBLAS_OP_N;
  bool ok = hipblasLtMatmulDescCreate(&g.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) == HIPBLAS_STATUS_SUCCESS &&
            hipblasLtMatmulDescSetAttribute(g.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &op, sizeof(op)) ==
                HIPBLAS_STATUS_SUCCESS &&
            hipblasLtMatmulDescSetAttribute(g.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &op, sizeof(op)) ==
                HIPBLAS_STATUS_SUCCESS &&
            hipblasLtMatrixLayoutCreate(&g.lw, dt, (uint64_t)N, (uint64_t)K, ldw) == HIPBLAS_STATUS_SUCCESS &&
            hipblasLtMatrixLayoutCreate(&g.lx, dt, (uint64_t)K, (uint64_t)M, K) == HIPBLAS_STATUS_SUCCESS &&
            hipblasLtMatrixLayoutCreate(&g.ly, bias16 ? dt : HIP_R_32F, (uint64_t)N, (uint64_t)M, N) ==
                HIPBLAS_STATUS_SUCCESS;
  if (ok && bias16) {
    // the bias vector runs along D^T's rows (the output's columns); a dummy
    // (zero) one while the candidates are timed, the weights' at each call
    const uint32_t epi = HIPBLASLT_EPILOGUE_BIAS;
    const int32_t bt = dt;
    const void* bp = tu.w;
    ok = hipblasLtMatmulDescSetAttribute(g.desc, HIPBLASLT_MATMUL_DESC_EPILOGUE, &epi, sizeof(epi)) ==
             HIPBLAS_STATUS_SUCCESS &&
         hipblasLtMatmulDescSetAttribute(g.desc, HIPBLASLT_MATMUL_DESC_BIAS_DATA_TYPE, &bt, sizeof(bt)) ==
             HIPBLAS_STATUS_SUCCESS &&
         hipblasLtMatmulDescSetAttribute(g.desc, HIPBLASLT_MATMUL_DESC_BIAS_POINTER, &bp, sizeof(bp)) ==
             HIPBLAS_STATUS_SUCCESS;
  }
  hipblasLtMatmulPreference_t pref = nullptr;
  ok = ok && hipblasLtMatmulPreferenceCreate(&pref) == HIPBLAS_STATUS_SUCCESS;
  const uint64_t cap = tu.ws_cap;
  ok = ok && hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &cap,
                                                   sizeof(cap)) == HIPBLAS_STATUS_SUCCESS;
  constexpr int kCand = 8;   // candidates timed per shape (24 measured no better)
  hipblasLtMatmulHeuristicResult_t res[kCand];
  int nret = 0;
  ok = ok && hipblasLtMatmulAlgoGetHeuristic(h, g.desc, g.lw, g.lx, g.ly, g.ly, pref, kCand, res, &nret) ==
                 HIPBLAS_STATUS_SUCCESS;
  if (pref) (void)hipblasLtMatmulPreferenceDestroy(pref);
  float best = 0.f;
  int pick = -1;
  const float one = 1.0f, zero = 0.0f;
  for (int a = 0; ok && a < nret; ++a) {
    if (res[a].state != HIPBLAS_STATUS_SUCCESS || res[a].workspaceSize > tu.ws_cap) continue;
    auto run = [&]() {
      return hipblasLtMatmul(h, g.desc, &one, tu.w, g.lw, tu.x, g.lx, &zero, tu.y, g.ly, tu.y, g.ly, &res[a].algo,
                             tu.ws, res[a].workspaceSize, tu.stream) == HIPBLAS_STATUS_SUCCESS;
    };
    if (!run()) continue;   // warm-up (and a check that it runs)
    bool good = hipEventRecord(tu.e0, tu.stream) == hipSuccess;
    for (int r = 0; good && r < 3; ++r) good = run();
    good = good && hipEventRecord(tu.e1, tu.stream) == hipSuccess && hipEventSynchronize(tu.e1) == hipSuccess;
    float ms = 0.f;
    if (!good || hipEventElapsedTime(&ms, tu.e0, tu.e1) != hipSuccess) continue;
    if (pick < 0 || ms < best) {
      best = ms;
      pick = a;
    }
  }
  (void)hipGetLastError();
  if (!ok || pick < 0) {
    lt_free(g);
    g.M = M; g.N = N; g.K = K; g.ldw = ldw;
    return;
  }
  g.algo = res[pick].algo;
  g.ws = res[pick].workspaceSize;
  g.ok = true;
  g.bias16 = bias16;
}

struct lwattn_layer_s {
  lwattn_plan_t attn = nullptr;   // not owned
  int32_t inter = 0;
  float eps = 0.f;
  int mg = 0;                          // gathered global rows per batch row: min(max_global, n)
  rocblas_handle blas = nullptr;
  float* P = nullptr;                  // [M, max(3 hid, inter)] fp32 GEMM results (or 16-bit ones)
  void* P2 = nullptr;                  // [M, 2 hid] 16-bit: the Kg|Vg GEMM's result, read by the attention
  float* Pg = nullptr;                 // [B mg, hid] fp32: Qg of the gathered rows
  void* qkv[6] = {};                   // Q, K, V, Qg, Kg, Vg [B, H, n, 64]
  void* A = nullptr;                   // attention output [B, H, n, 64]
  void* Am = nullptr;                  // [M, hid]
  void* H1 = nullptr;                  // [M, hid]
  void* F = nullptr;                   // [M, inter]
  void* Xg = nullptr;                  // [B mg, hid] rows of X at the global tokens
  int32_t* gpos = nullptr;             // [B, mg] their positions (-1 past the count)
  hipblasLtHandle_t lt = nullptr;
  void* lt_ws = nullptr;               // hipBLASLt workspace
  size_t lt_ws_bytes = 0;
  void* lt_ws_side = nullptr;          // the Qg GEMM's own workspace (it runs beside the others)
  LtGemm g_qkv, g_kv, g_qg, g_o, g_f1, g_f2;
  // the global rows' Qg chain (find, gather, GEMM, scatter) runs on a stream
  // of its own beside the Q|K|V and Kg|Vg projections: forked from the
  // caller's stream at the start of a layer, joined before the attention
  hipStream_t side = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};

static void free_layer(lwattn_layer_t L) {
  if (!L) return;
  if (L->attn) (void)hipSetDevice(L->attn->device);
  (void)hipFree(L->P);
  (void)hipFree(L->P2);
  (void)hipFree(L->Pg);
  for (auto* q : L->qkv) (void)hipFree(q);
  (void)hipFree(L->A);
  (void)hipFree(L->Am);
  (void)hipFree(L->H1);
  (void)hipFree(L->F);
  (void)hipFree(L->Xg);
  (void)hipFree(L->gpos);
  for (LtGemm* g : {&L->g_qkv, &L->g_kv, &L->g_qg, &L->g_o, &L->g_f1, &L->g_f2}) lt_free(*g);
  (void)hipFree(L->lt_ws);
  (void)hipFree(L->lt_ws_side);
  if (L->fork) (void)hipEventDestroy(L->fork);
  if (L->join) (void)hipEventDestroy(L->join);
  if (L->side) (void)hipStreamDestroy(L->side);
  if (L->lt) (void)hipblasLtDestroy(L->lt);
  if (L->blas) (void)rocblas_destroy_handle(L->blas);
  delete L;
}

// Row-major Y[M, N] (fp32, row stride N) = X[M, K] W[K, N] (16-bit of type
// dt, X rows of stride K, W rows of stride ldw >= N), as the column-major
// product Y^T = W^T X^T.
static bool gemm_rm(rocblas_handle h, rocblas_datatype dt, int64_t M, int64_t N, int64_t K, const void* X,
                    const void* W, int64_t ldw, float* Y) {
  const float one = 1.0f, zero = 0.0f;
  const rocblas_status st = rocblas_gemm_ex(h, rocblas_operation_none, rocblas_operation_none, (rocblas_int)N,
                                            (rocblas_int)M, (rocblas_int)K, &one, W, dt, (rocblas_int)ldw, X, dt,
                                            (rocblas_int)K, &zero, Y, rocblas_datatype_f32_r, (rocblas_int)N, Y,
                                            rocblas_datatype_f32_r, (rocblas_int)N, rocblas_datatype_f32_r,
                                            rocblas_gemm_algo_standard, 0, 0);
  if (st != rocblas_status_success) {
    std::fprintf(stderr, "lwattn: rocblas_gemm_ex failed (%d)\n", (int)st);
    return false;
  }
  return true;
}

// One of the layer's GEMMs: hipBLASLt with the algorithm chosen at set-up,
// else rocBLAS.
static bool layer_gemm(lwattn_layer_t L, const LtGemm& g, rocblas_datatype dt, const void* X, const void* W, float* Y,
                       hipStream_t stream, void* ws = nullptr) {
  if (g.ok) {
    const float one = 1.0f, zero = 0.0f;
    const hipblasStatus_t st = hipblasLtMatmul(L->lt, g.desc, &one, W, g.lw, X, g.lx, &zero, Y, g.ly, Y, g.ly, &g.algo,
                                               ws ? ws : L->lt_ws, g.ws, stream);
    if (st != HIPBLAS_STATUS_SUCCESS) {
      std::fprintf(stderr, "lwattn: hipblasLtMatmul failed (%d)\n", (int)st);
      return false;
    }
    return true;
  }
  return gemm_rm(L->blas, dt, g.M, g.N, g.K, X, W, g.ldw, Y);
}

// A GEMM set up with the bias epilogue: Y16 [M, N] = X W + bias, in the
// storage type (only when g.bias16).
static bool layer_gemm_bias(lwattn_layer_t L, const LtGemm& g, const void* X, const void* W, const void* bias,
                            void* Y16, hipStream_t stream) {
  if (hipblasLtMatmulDescSetAttribute(g.desc, HIPBLASLT_MATMUL_DESC_BIAS_POINTER, &bias, sizeof(bias)) !=
      HIPBLAS_STATUS_SUCCESS)
    return false;
  const float one = 1.0f, zero = 0.0f;
  const hipblasStatus_t st = hipblasLtMatmul(L->lt, g.desc, &one, W, g.lw, X, g.lx, &zero, Y16, g.ly, Y16, g.ly,
                                             &g.algo, L->lt_ws, g.ws, stream);
  if (st != HIPBLAS_STATUS_SUCCESS) {
    std::fprintf(stderr, "lwattn: hipblasLtMatmul failed (%d)\n", (int)st);
    return false;
  }
  return true;
}

template <typename T, int PER>
static void launch_ln(const void* G, bool g16, const void* b, const void* R, const void* g, const void* be,
                      float eps, void* Y, int64_t M, hipStream_t stream) {
  if (g16)
    hipLaunchKernelGGL((lwk::layer::bias_residual_layernorm<T, PER, true>), dim3((uint32_t)((M + 3) / 4)),
                       dim3(lwk::layer::LNT), 0, stream, G, (const T*)b, (const T*)R, (const T*)g, (const T*)be, eps,
                       (T*)Y, M);
  else
    hipLaunchKernelGGL((lwk::layer::bias_residual_layernorm<T, PER, false>), dim3((uint32_t)((M + 3) / 4)),
                       dim3(lwk::layer::LNT), 0, stream, G, (const T*)b, (const T*)R, (const T*)g, (const T*)be, eps,
                       (T*)Y, M);
}

// Heads the layer takes: H a multiple of 4 up to 64 (hid = 64 H columns, held
// H to a lane by the LayerNorm).
static bool layer_heads_ok(int H) { return H >= 4 && H <= 64 && H % 4 == 0; }

template <typename T>
static bool layernorm(int H, const void* G, bool g16, const void* b, const void* R, const void* g, const void* be,
                      float eps, void* Y, int64_t M, hipStream_t stream) {
  switch (H) {
#define LWATTN_LN_CASE(h) \
  case h: launch_ln<T, h>(G, g16, b, R, g, be, eps, Y, M, stream); return true;
    LWATTN_LN_CASE(4) LWATTN_LN_CASE(8) LWATTN_LN_CASE(12) LWATTN_LN_CASE(16)
    LWATTN_LN_CASE(20) LWATTN_LN_CASE(24) LWATTN_LN_CASE(28) LWATTN_LN_CASE(32)
    LWATTN_LN_CASE(36) LWATTN_LN_CASE(40) LWATTN_LN_CASE(44) LWATTN_LN_CASE(48)
    LWATTN_LN_CASE(52) LWATTN_LN_CASE(56) LWATTN_LN_CASE(60) LWATTN_LN_CASE(64)
#undef LWATTN_LN_CASE
    default: return false;
  }
}


// Launch geometry of the forward (attn_kernel), computed by forward_geometry
// below.  stride [H] and blk [H + 1] receive each head's stride and the prefix
// of band workgroups per batch row.

static bool forward_geometry(const lwattn_config& c, const int32_t* gap, int ncu, FwdGeom& g, int32_t* stride,
                             int32_t* blk) {
  const int B = c.B, H = c.H, n = c.n;
  blk[0] = 0;
  for (int h = 0; h < H; ++h) {
    const int s = gap[h] + 1;
    stride[h] = s;
    int64_t nb = 0;
    for (int rho = 0; rho < s && rho < n; ++rho) {
      const int64_t nr = ((int64_t)n - rho + s - 1) / s;
      nb += (nr + lwk::ROWS_WG - 1) / lwk::ROWS_WG;
    }
    if ((int64_t)blk[h] + nb > INT32_MAX) return false;
    blk[h + 1] = blk[h] + (int32_t)nb;
  }
  g.blocks_per_b = blk[H];
  bool uni = H > 0;
  for (int h = 1; h < H; ++h) uni = uni && stride[h] == stride[0];
  g.uni_stride = uni ? stride[0] : 0;
  g.blocks_per_head = uni ? blk[1] : 0;
  const int64_t nblk = (int64_t)B * blk[H];
  // band workgroups may take the bf16 fast path when every subsequence key
  // they stage has a byte offset that fits in 32 bits
  int smax = 1;
  for (int h = 0; h < H; ++h) smax = std::max(smax, stride[h]);
  g.band_fast = (c.dtype != LWATTN_F32 && (int64_t)n + 128 * (int64_t)smax < ((int64_t)1 << 24)) ? 1 : 0;
  // On the register-staged path (fp32 storage; 16-bit past 32-bit offsets),
  // whose tiles are long (fp32 MFMA), a grid of band blocks that fills at
  // most half a round of workgroup slots leaves most SIMDs idle: cut each
  // block's key tiles into parts (up to 8, and no more than its band tiles),
  // one workgroup each, merged by log-sum-exp.
  {
    const int64_t slots = 2 * (int64_t)ncu;
    const int r = (int)std::min<int64_t>(c.window / 2, n);
    const int64_t tiles = (31 + 2 * (int64_t)r) / 32 + 1;
    g.bparts = 1;
    if (!g.band_fast && nblk > 0 && 2 * nblk <= slots)
      g.bparts = (int)std::max<int64_t>(1, std::min<int64_t>({slots / nblk, 8, tiles}));
  }
  g.n_band_blk = (int)std::min<int64_t>(nblk, INT32_MAX);
  const int64_t nband = nblk * g.bparts;
  // compaction workgroups lead the grid, padded to a multiple of 8 so that the
  // band workgroups behind them keep their XCD placement.  When the band
  // workgroups alone fit one round of slots but not with those ahead of them
  // (B=1, H=16, n=4096: 512 band workgroups), the last band workgroups would
  // run as a second round: then band workgroups 0 .. B-1 each compact a row
  // before their band work instead.
  int64_t ncomp = ((int64_t)B + 7) / 8 * 8;
  g.comp_fold = 0;
  if (ncomp + nband > 2 * (int64_t)ncu && nband <= 2 * (int64_t)ncu && B <= nband) {
    g.comp_fold = 1;
    ncomp = 0;
  }
  // global-row geometry: the key slices are sized so that the global-row
  // workgroups fill what the compaction and band workgroups leave of the last
  // round of workgroup slots (two per compute unit), with at least 64 of them.
  // When that round is nearly empty (under a quarter used), a full round of
  // global-row workgroups would run behind the band ones with long merges of
  // many slices: a quarter of the slots serves them better (measured at
  // B=1, H=16, n=4096, 64 globals: 47 instead of 105 us; B=4: 114 instead of
  // 134 us)
  const int64_t slots = 2 * (int64_t)ncu;
  g.nqt = ceil_div(c.max_global, 32);
  g.nqg = ceil_div(g.nqt, lwk::NW);
  int64_t nglob = 0;
  g.ksplit = g.nsplit = 0;
  if (g.nqt > 0 && n > 0 && B > 0 && H > 0) {
    const int64_t units = (int64_t)B * H * g.nqg;
    const int64_t used = (ncomp + nband) % slots;
    int64_t target = used < slots / 4 ? slots / 4 : slots - used;
    if (target < 64) target = 64;
    int64_t want = (target + units - 1) / units;
    const int64_t maxs = (n + 63) / 64;   // slices of at least one 64-key step
    if (want > maxs) want = maxs;
    // at most 8 slices (unless the 4096-key bound below asks for more): the
    // merge reads every slice's partial (8 KB per query tile) back through
    // agent-coherent loads, which run at a few hundred GB/s (B=1, H=8,
    // n=4096, 64 globals: 22 slices 36.4 us, 8 slices 28.8 us)
    if (want > 8) want = 8;
    if (want < 1) want = 1;
    // but no slice longer than 4096 keys, so that no global-row workgroup
    // outlasts the band ones on long sequences
    if (want < (n + 4095) / 4096) want = (n + 4095) / 4096;
    g.ksplit = ceil_div(ceil_div(n, want), 64) * 64;   // whole 64-key steps
    g.nsplit = ceil_div(n, g.ksplit);
    nglob = units * g.nsplit;
  }
  const int64_t nglob_pad = (nglob + 7) / 8 * 8;
  if (ncomp + nband + nglob_pad > INT32_MAX) return false;
  g.n_comp_wg = (int)ncomp;
  g.n_band_wg = (int)nband;
  g.n_glob_wg = (int)nglob_pad;
  // one round: the global-row workgroups go last, into the gaps; more: they
  // follow the first round of band workgroups (measured, B=4, H=16, n=4096,
  // 64 globals: about 90 instead of 114 us; at B=8, n=16384, 128 globals the
  // two orders are within the run-to-run spread)
  g.band_pre = (int)(ncomp + nband <= slots
                         ? nband
                         : std::min<int64_t>(nband, std::max<int64_t>(0, (slots - ncomp) / 8 * 8)));
  g.smem = c.dtype == LWATTN_F32 ? lwk::smem_bytes<float>() : lwk::smem_bytes<__bf16>();   // fp16 as bf16
  return true;
}

// Device workspace of one forward: where attn_kernel keeps the flags, the
// global index, the per-row status and readiness words, the fault word, the
// global rows' partials and the merge counters.
struct FwdWork {
  uint8_t* flags;
  int32_t *gidx, *gcnt, *status, *tile_cnt, *ready, *fault;
  float *part_o, *part_ml;
  const int32_t *head_stride, *head_blk;   // device copies (read only when H > MAXH_ARG)
  float *bpart_o, *bpart_ml;               // bparts > 1: the band blocks' key parts
  int32_t* bcnt;                           // bparts > 1: [blocks][NW] parts finished
};

// Floats of the band blocks' key parts: O [blocks][NW][bparts][64][32] and
// (offset, sum) [blocks][NW][bparts][32][2]; words of their counters.
static size_t bpart_o_floats(const FwdGeom& g) {
  return g.bparts > 1 ? (size_t)g.n_band_blk * lwk::NW * g.bparts * 64 * 32 : 0;
}
static size_t bpart_ml_floats(const FwdGeom& g) {
  return g.bparts > 1 ? (size_t)g.n_band_blk * lwk::NW * g.bparts * 32 * 2 : 0;
}
static size_t bcnt_words(const FwdGeom& g) { return g.bparts > 1 ? (size_t)g.n_band_blk * lwk::NW : 0; }

static size_t fwd_parts(const lwattn_config& c, const FwdGeom& g) {
  return (size_t)c.B * c.H * g.nqt * (g.nsplit > 0 ? g.nsplit : 0) * 32;
}

static void forward_params(lwk::Params& prm, const lwattn_config& c, const FwdGeom& g, const FwdWork& w,
                           const int32_t* stride, const int32_t* blk, const void* Q, const void* K, const void* V,
                           const void* Qg, const void* Kg, const void* Vg, const float* lmask, const float* gmask,
                           void* O, int32_t epoch) {
  std::memset(&prm, 0, sizeof(prm));
  prm.Q = (const uint8_t*)Q;
  prm.K = (const uint8_t*)K;
  prm.V = (const uint8_t*)V;
  prm.Qg = (const uint8_t*)Qg;
  prm.Kg = (const uint8_t*)Kg;
  prm.Vg = (const uint8_t*)Vg;
  prm.O = (uint8_t*)O;
  prm.lmask = lmask;
  prm.gmask = gmask;
  prm.flags = w.flags;
  prm.gidx = w.gidx;
  prm.gcnt = w.gcnt;
  prm.status = w.status;
  prm.part_o = w.part_o;
  prm.part_ml = w.part_ml;
  prm.tile_cnt = w.tile_cnt;
  prm.bparts = g.bparts;
  prm.bpart_o = w.bpart_o;
  prm.bpart_ml = w.bpart_ml;
  prm.bcnt = w.bcnt;
  prm.ready = w.ready;
  prm.fault = w.fault;
  prm.epoch = epoch;
  prm.publish = epoch;
  prm.spin_limit = (1 << 18) + (int32_t)(c.n >> 2);
  prm.n_comp_wg = g.n_comp_wg;
  prm.comp_fold = g.comp_fold;
  prm.head_stride = w.head_stride;
  prm.head_blk = w.head_blk;
  prm.B = c.B;
  prm.H = c.H;
  prm.n = c.n;
  prm.r = (int)std::min<int64_t>(c.window / 2, c.n);
  prm.max_global = c.max_global;
  prm.nqt = g.nqt;
  prm.nqg = g.nqg;
  prm.nsplit = g.nsplit;
  prm.ksplit = g.ksplit;
  prm.n_glob_wg = g.n_glob_wg;
  prm.n_band_wg = g.n_band_wg;
  prm.band_pre = g.band_pre;
  prm.blocks_per_b = g.blocks_per_b;
  prm.c = c.scale * 1.4426950408889634f;
  prm.o_tok = 0;
  // inputs [B][H][n][64]
  const int64_t rb = (int64_t)64 * (c.dtype == LWATTN_F32 ? 4 : 2);
  for (int k = 0; k < 3; ++k) {
    prm.in_bs[k] = (int64_t)c.H * c.n * rb;
    prm.in_hs[k] = (int64_t)c.n * rb;
    prm.in_rs[k] = (int32_t)rb;
  }
  prm.mask_vec = ((((uintptr_t)lmask | (uintptr_t)gmask) & 15u) == 0 && (c.n % 4) == 0) ? 1 : 0;
  prm.uni_stride = g.uni_stride;
  prm.blocks_per_head = g.blocks_per_head;
  prm.band_fast = g.band_fast;
  for (int h = 0; h < lwk::MAXH_ARG; ++h) prm.hs[h] = h < c.H ? stride[h] : 0;
  for (int h = 0; h <= lwk::MAXH_ARG; ++h) prm.hb[h] = h <= c.H ? blk[h] : 0;
}

static bool launch_forward(const lwattn_config& c, const FwdGeom& g, const lwk::Params& prm, hipStream_t stream,
                           hipEvent_t ev0, hipEvent_t ev1) {
  const int grid = g.n_comp_wg + g.n_band_wg + g.n_glob_wg;
  if (c.dtype == LWATTN_BF16)
    hipExtLaunchKernelGGL(lwk::attn_kernel<__bf16>, dim3(grid), dim3(lwk::NT), (uint32_t)g.smem, stream, ev0, ev1,
                          0u, prm);
  else if (c.dtype == LWATTN_F16)
    hipExtLaunchKernelGGL(lwk::attn_kernel<_Float16>, dim3(grid), dim3(lwk::NT), (uint32_t)g.smem, stream, ev0,
                          ev1, 0u, prm);
  else
    hipExtLaunchKernelGGL(lwk::attn_kernel<float>, dim3(grid), dim3(lwk::NT), (uint32_t)g.smem, stream, ev0, ev1,
                          0u, prm);
  return hip_ok(hipGetLastError(), "hipGetLastError");
}

static bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

// Checks shared by the forward entry points: LWATTN_OK when the call may
// launch (or is empty, *empty set).
static lwattn_status forward_args(const lwattn_config& c, const void* Q, const void* K, const void* V, const void* Qg,
                                  const void* Kg, const void* Vg, const float* lmask, const float* gmask, void* O,
                                  bool* empty) {
  *empty = (int64_t)c.B * c.H * c.n == 0;
  if (*empty) return LWATTN_OK;
  const void* ptrs[] = {Q, K, V, Qg, Kg, Vg, O};
  for (const void* q : ptrs)
    if (!q || !aligned16(q)) return LWATTN_E_INVALID;
  if (!lmask || !gmask || ((uintptr_t)lmask & 3u) || ((uintptr_t)gmask & 3u)) return LWATTN_E_INVALID;
  return LWATTN_OK;
}


// ---------------------------------------------------------------------------
// Allocation-free forward.  Its workspace is one file-scope device array per
// GPU, `scratch`, of kScratchBytes; the host never passes the array's name to
// a kernel (in host code that name is a stand-in, not a device address) but
// the address hipGetSymbolAddress returned for that device, looked up once per
// device with the device current.
constexpr size_t kScratchBytes = (size_t)32 << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
int g_scratch_ncu[kMaxDevices];

// The per-device address of `scratch` and the device's compute-unit count;
// nullptr if the lookup failed.  The device must be current.
void* scratch_of(int dev) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (!hip_ok(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress") || !ptr) return nullptr;
    int ncu = 0;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0) ncu = 256;
    g_scratch_ncu[dev] = ncu;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
}  // namespace

// Zeroes `count` 32-bit words (a kernel rather than a memset, so that the
// call can sit in a captured graph).
__global__ void zero_words_kernel(int32_t* p, int count) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < count; i += gridDim.x * blockDim.x) p[i] = 0;
}

extern "C" {

const char* lwattn_strerror(lwattn_status s) {
  switch (s) {
    case LWATTN_OK: return "ok";
    case LWATTN_E_INVALID: return "invalid argument";
    case LWATTN_E_UNSUPPORTED: return "unsupported configuration (head dim must be 64)";
    case LWATTN_E_NOMEM: return "device workspace allocation failed";
    case LWATTN_E_DEVICE: return "HIP runtime error";
    case LWATTN_E_TOO_MANY_GLOBALS: return "a batch row has more global tokens than max_global";
    case LWATTN_E_SCRATCH: return "the problem needs more workspace than the static no-allocation buffer holds";
  }
  return "unknown status";
}

lwattn_status lwattn_check_config(const lwattn_config* c) {
  if (!c) return LWATTN_E_INVALID;
  if (c->B < 0 || c->H < 0 || c->n < 0 || c->d <= 0) return LWATTN_E_INVALID;
  if (c->window < 0 || (c->window & 1)) return LWATTN_E_INVALID;
  if (c->max_global < 0) return LWATTN_E_INVALID;
  if (!(c->scale > 0.0f) || !std::isfinite(c->scale)) return LWATTN_E_INVALID;
  if (c->dtype != LWATTN_F32 && c->dtype != LWATTN_BF16 && c->dtype != LWATTN_F16) return LWATTN_E_INVALID;
  if (c->dilation) {
    for (int h = 0; h < c->H; ++h) {
      if (c->dilation[h] < 0) return LWATTN_E_INVALID;
      if ((int64_t)c->dilation[h] + 1 > (int64_t)INT32_MAX / 2) return LWATTN_E_INVALID;
    }
  }
  const int64_t elems = (int64_t)c->B * c->H * c->n * c->d;
  if (elems > ((int64_t)1 << 40)) return LWATTN_E_INVALID;
  if ((int64_t)c->B * c->n > ((int64_t)1 << 31) - 1) return LWATTN_E_INVALID;
  if (c->n > (1 << 23)) return LWATTN_E_INVALID;   // keeps row byte offsets of one head in int32
  if (c->d != lwk::D) return LWATTN_E_UNSUPPORTED;
  return LWATTN_OK;
}

lwattn_status lwattn_plan(const lwattn_config* cfg, int hip_device, lwattn_plan_t* out) {
  if (!out) return LWATTN_E_INVALID;
  *out = nullptr;
  lwattn_status st = lwattn_check_config(cfg);
  if (st != LWATTN_OK) return st;
  int ndev = 0;
  if (!hip_ok(hipGetDeviceCount(&ndev), "hipGetDeviceCount") || hip_device < 0 || hip_device >= ndev)
    return hip_device < 0 ? LWATTN_E_INVALID : LWATTN_E_DEVICE;
  if (!hip_ok(hipSetDevice(hip_device), "hipSetDevice")) return LWATTN_E_DEVICE;

  lwattn_plan_s* p = new (std::nothrow) lwattn_plan_s();
  if (!p) return LWATTN_E_NOMEM;
  p->cfg = *cfg;
  p->device = hip_device;
  const int B = cfg->B, H = cfg->H, n = cfg->n;
  p->gap.assign(H, 0);
  if (cfg->dilation)
    for (int h = 0; h < H; ++h) p->gap[h] = cfg->dilation[h];
  p->cfg.dilation = nullptr;   // the plan keeps its own copy

  // band geometry of the forward (per head, sum over residue classes of
  // ceil(n_rho / 128)) and of the backward (of ceil(n_rho / 64))
  int ncu = 256;
  {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, hip_device) == hipSuccess && v > 0)
      ncu = v;
  }
  p->ncu = ncu;
  std::vector<int32_t> stride(H), blk(H + 1, 0), blk64(H + 1, 0);
  FwdGeom g;
  if (!forward_geometry(p->cfg, p->gap.data(), ncu, g, stride.data(), blk.data())) {
    free_plan(p);
    return LWATTN_E_INVALID;
  }
  for (int h = 0; h < H; ++h) {
    const int s = stride[h];
    int64_t nb64 = 0;
    for (int rho = 0; rho < s && rho < n; ++rho) {
      const int64_t nr = ((int64_t)n - rho + s - 1) / s;
      nb64 += (nr + lwk::bw::T - 1) / lwk::bw::T;
    }
    blk64[h + 1] = blk64[h] + (int32_t)nb64;
  }
  p->geom = g;
  p->blocks64_per_b = blk64[H];
  p->blocks_per_b = g.blocks_per_b;
  p->stride_host = stride;
  p->blk_host = blk;
  p->uni_stride = g.uni_stride;
  p->blocks_per_head = g.blocks_per_head;
  p->band_fast = g.band_fast;
  p->nqt = g.nqt;
  p->nqg = g.nqg;
  p->ksplit = g.ksplit;
  p->nsplit = g.nsplit;
  p->n_comp_wg = g.n_comp_wg;
  p->n_band_wg = g.n_band_wg;
  p->n_glob_wg = g.n_glob_wg;
  p->smem = g.smem;

  // workspace
  const size_t bn = (size_t)B * n;
  bool ok = true;
  auto alloc = [&](void** ptr, size_t bytes) {
    if (!ok) return;
    if (bytes == 0) bytes = 16;
    if (!hip_ok(hipMalloc(ptr, bytes), "hipMalloc")) { ok = false; *ptr = nullptr; }
  };
  alloc((void**)&p->flags, bn);
  alloc((void**)&p->gidx, bn * 4);
  alloc((void**)&p->gcnt, (size_t)B * 4);
  alloc((void**)&p->status, (size_t)B * 4);
  const size_t nparts = fwd_parts(p->cfg, g);
  alloc((void**)&p->part_o, nparts * lwk::D * 4);
  alloc((void**)&p->part_ml, nparts * 2 * 4);
  alloc((void**)&p->tile_cnt, (size_t)B * H * (p->nqt > 0 ? p->nqt : 1) * 4);
  alloc((void**)&p->bpart_o, bpart_o_floats(g) * 4);
  alloc((void**)&p->bpart_ml, bpart_ml_floats(g) * 4);
  alloc((void**)&p->bcnt, std::max<size_t>(bcnt_words(g), 1) * 4);
  alloc((void**)&p->ready, (size_t)B * 4);
  alloc((void**)&p->ready_cnt, (size_t)B * 8);
  alloc((void**)&p->fault, 4);
  alloc((void**)&p->head_stride, (size_t)H * 4);
  alloc((void**)&p->head_blk, (size_t)(H + 1) * 4);
  alloc((void**)&p->head_blk64, (size_t)(H + 1) * 4);
  alloc((void**)&p->stats, (size_t)B * H * n * sizeof(float2));
  if (cfg->dtype != LWATTN_F32 && cfg->max_global > 0 && n > 0 && B > 0 && H > 0) {
    // the positions of a head are cut into chunks of whole 64-row tiles, as
    // many as bring the workgroups of the chunk sums (one per batch row, head,
    // 64 global rows and chunk) to about one round of slots, two per compute
    // unit (measured against twice that: base 21.5 -> 15.7 us for the chunk
    // sums and their merge, qa 56 -> 47 us; long unchanged)
    const int64_t ntile = ((int64_t)n + lwk::bw::T - 1) / lwk::bw::T;
    const int64_t units = (int64_t)B * H * ceil_div(cfg->max_global, lwk::bw::T);
    const int64_t round = 2 * (int64_t)ncu;
    const int64_t want = std::max<int64_t>(1, std::min<int64_t>(ntile, (round + units - 1) / units));
    const int64_t tiles = (ntile + want - 1) / want;
    p->gchunk = (int)(tiles * lwk::bw::T);
    p->gsplit = (int)((ntile + tiles - 1) / tiles);
    const size_t rows = (size_t)B * H * cfg->max_global * p->gsplit;
    alloc((void**)&p->gq, rows * 68 * 4);
    alloc((void**)&p->gk, rows * 128 * 4);
    alloc((void**)&p->gml, (size_t)B * H * cfg->max_global * ((p->gsplit + 1) / 2 * 2) * 2 * 4);
  }
  if (!ok) {
    free_plan(p);
    return LWATTN_E_NOMEM;
  }
  if ((H > 0 && !hip_ok(hipMemcpy(p->head_stride, stride.data(), (size_t)H * 4, hipMemcpyHostToDevice), "hipMemcpy")) ||
      !hip_ok(hipMemcpy(p->head_blk, blk.data(), (size_t)(H + 1) * 4, hipMemcpyHostToDevice), "hipMemcpy") ||
      !hip_ok(hipMemcpy(p->head_blk64, blk64.data(), (size_t)(H + 1) * 4, hipMemcpyHostToDevice), "hipMemcpy") ||
      (B > 0 && !hip_ok(hipMemset(p->status, 0, (size_t)B * 4), "hipMemset")) ||
      (B > 0 && !hip_ok(hipMemset(p->gcnt, 0, (size_t)B * 4), "hipMemset")) ||
      !hip_ok(hipMemset(p->tile_cnt, 0, (size_t)B * H * (p->nqt > 0 ? p->nqt : 1) * 4), "hipMemset") ||
      (B > 0 && !hip_ok(hipMemset(p->ready, 0, (size_t)B * 4), "hipMemset")) ||
      (B > 0 && !hip_ok(hipMemset(p->ready_cnt, 0, (size_t)B * 8), "hipMemset")) ||
      !hip_ok(hipMemset(p->fault, 0, 4), "hipMemset") ||
      !hip_ok(hipMemset(p->bcnt, 0, std::max<size_t>(bcnt_words(g), 1) * 4), "hipMemset") ||
      !hip_ok(hipDeviceSynchronize(), "hipDeviceSynchronize")) {
    free_plan(p);
    return LWATTN_E_DEVICE;
  }
  *out = p;
  return LWATTN_OK;
}

lwattn_status lwattn_destroy(lwattn_plan_t p) {
  if (!p) return LWATTN_OK;
  (void)hipSetDevice(p->device);
  free_plan(p);
  return LWATTN_OK;
}

// Inputs in the encoder layer's projection layout: Q, K, V rows of
// `rs_qkv` bytes ([B n][3 hid]: Q, K, V are the column blocks) and Kg, Vg
// rows of `rs_kv` bytes ([B n][2 hid]); head h at column h 64.  Qg keeps
// [B][H][n][64].
struct InRows {
  int64_t rs_qkv = 0, rs_kv = 0;
};

// The forward; o_tok: O token-major [B][n][H][64] instead of [B][H][n][64]
// (the encoder layer's merged heads; taken only where a head's rows span less
// than 2^31 bytes); rows: inputs in the projection layout (nullptr:
// [B][H][n][64]).
static lwattn_status forward_impl(lwattn_plan_t p, const void* Q, const void* K, const void* V, const void* Qg,
                                  const void* Kg, const void* Vg, const float* lmask, const float* gmask, void* O,
                                  bool o_tok, const InRows* rows, hipStream_t stream) {
  if (!p) return LWATTN_E_INVALID;
  const lwattn_config& c = p->cfg;
  bool empty = false;
  const lwattn_status ast = forward_args(c, Q, K, V, Qg, Kg, Vg, lmask, gmask, O, &empty);
  if (ast != LWATTN_OK || empty) return ast;
  if (!hip_ok(hipSetDevice(p->device), "hipSetDevice")) return LWATTN_E_DEVICE;

  FwdWork w;
  w.flags = p->flags;
  w.gidx = p->gidx;
  w.gcnt = p->gcnt;
  w.status = p->status;
  w.tile_cnt = p->tile_cnt;
  w.ready = p->ready;
  w.fault = p->fault;
  w.part_o = p->part_o;
  w.part_ml = p->part_ml;
  w.head_stride = p->head_stride;
  w.head_blk = p->head_blk;
  w.bpart_o = p->bpart_o;
  w.bpart_ml = p->bpart_ml;
  w.bcnt = p->bcnt;
  p->epoch = p->epoch >= INT32_MAX - 1 ? 1 : p->epoch + 1;
  lwk::Params prm;
  forward_params(prm, c, p->geom, w, p->stride_host.data(), p->blk_host.data(), Q, K, V, Qg, Kg, Vg, lmask, gmask, O,
                 p->epoch);
  prm.o_tok = o_tok ? 1 : 0;
  if (rows) {
    const int64_t rs[3] = {rows->rs_qkv, (int64_t)64 * 2, rows->rs_kv};
    for (int k : {0, 2}) {
      prm.in_bs[k] = (int64_t)c.n * rs[k];
      prm.in_hs[k] = 64 * 2;
      prm.in_rs[k] = (int32_t)rs[k];
    }
  }
  if (p->inject_timeout) {
    // the rows are published under another number and nobody waits long:
    // every waiting workgroup gives up, sets the fault word and skips its work
    p->inject_timeout = false;
    prm.publish = -1;
    prm.spin_limit = 64;
  }

  bool timed = false;
  if (p->timing_cap > 0 && p->timing_calls < p->timing_cap) {
    timed = (p->timing_seen % p->timing_every) == 0;
    ++p->timing_seen;
  }
  // timed forwards take their events from the dispatch itself (start and end
  // of the kernel's execution), untimed ones launch plainly
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  if (timed) {
    ev0 = p->events[(size_t)p->timing_calls * (kNumKernels + 1)];
    ev1 = p->events[(size_t)p->timing_calls * (kNumKernels + 1) + 1];
  }
  if (!launch_forward(c, p->geom, prm, stream, ev0, ev1)) return LWATTN_E_DEVICE;
  if (timed) ++p->timing_calls;
  return LWATTN_OK;
}

lwattn_status lwattn_forward(lwattn_plan_t p, const void* Q, const void* K, const void* V,
                             const void* Qg, const void* Kg, const void* Vg,
                             const float* lmask, const float* gmask, void* O, hipStream_t stream) {
  return forward_impl(p, Q, K, V, Qg, Kg, Vg, lmask, gmask, O, false, nullptr, stream);
}

lwattn_status lwattn_forward_causal(lwattn_plan_t p, const void* Q, const void* K, const void* V,
                                    const float* lmask, void* O, hipStream_t stream) {
  if (!p) return LWATTN_E_INVALID;
  const lwattn_config& c = p->cfg;
  if ((int64_t)c.B * c.H * c.n == 0) return LWATTN_OK;   // empty problem
  if (c.dtype == LWATTN_F32) return LWATTN_E_UNSUPPORTED;
  // tiles are read through 32-bit buffer offsets over a head's n rows
  if ((int64_t)c.n * 128 >= lwk::OOB_OFF) return LWATTN_E_UNSUPPORTED;
  const void* ptrs[] = {Q, K, V, O};
  for (const void* q : ptrs)
    if (!q || !aligned16(q)) return LWATTN_E_INVALID;
  if (!lmask || ((uintptr_t)lmask & 3u)) return LWATTN_E_INVALID;
  if (!hip_ok(hipSetDevice(p->device), "hipSetDevice")) return LWATTN_E_DEVICE;
  lwk::cz::CzParams cp;
  cp.Q = (const uint8_t*)Q;
  cp.K = (const uint8_t*)K;
  cp.V = (const uint8_t*)V;
  cp.O = (uint8_t*)O;
  cp.lmask = lmask;
  cp.head_stride = p->head_stride;
  cp.head_blk = p->head_blk64;
  cp.B = c.B;
  cp.H = c.H;
  cp.n = c.n;
  cp.r = (int)std::min<int64_t>(c.window / 2, c.n);
  cp.blocks_per_b = p->blocks64_per_b;
  cp.scale = c.scale;
  const int64_t grid = (int64_t)c.B * p->blocks64_per_b;
  if (grid > INT32_MAX) return LWATTN_E_UNSUPPORTED;
  const auto kern = c.dtype == LWATTN_F16 ? lwk::cz::causal_kernel<_Float16> : lwk::cz::causal_kernel<__bf16>;
  (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lwk::cz::SMEM);
  hipLaunchKernelGGL(kern, dim3((uint32_t)grid), dim3(lwk::bw::NTH), lwk::cz::SMEM, stream, cp);
  if (!hip_ok(hipGetLastError(), "hipGetLastError")) return LWATTN_E_DEVICE;
  return LWATTN_OK;
}

lwattn_status lwattn_backward_causal(lwattn_plan_t p, const void* Q, const void* K, const void* V,
                                     const float* lmask, const void* O, const void* dO, void* dQ, void* dK,
                                     void* dV, hipStream_t stream) {
  if (!p) return LWATTN_E_INVALID;
  const lwattn_config& c = p->cfg;
  if ((int64_t)c.B * c.H * c.n == 0) return LWATTN_OK;   // empty problem
  if (c.dtype == LWATTN_F32) return LWATTN_E_UNSUPPORTED;
  if ((int64_t)c.n * 128 >= lwk::OOB_OFF) return LWATTN_E_UNSUPPORTED;
  const void* ptrs[] = {Q, K, V, O, dO, dQ, dK, dV};
  for (const void* q : ptrs)
    if (!q || !aligned16(q)) return LWATTN_E_INVALID;
  if (!lmask || ((uintptr_t)lmask & 3u)) return LWATTN_E_INVALID;
  if (!hip_ok(hipSetDevice(p->device), "hipSetDevice")) return LWATTN_E_DEVICE;
  lwk::cz::CzBwParams bp;
  bp.Q = (const uint8_t*)Q;
  bp.K = (const uint8_t*)K;
  bp.V = (const uint8_t*)V;
  bp.O = (const uint8_t*)O;
  bp.dO = (const uint8_t*)dO;
  bp.dQ = (uint8_t*)dQ;
  bp.dK = (uint8_t*)dK;
  bp.dV = (uint8_t*)dV;
  bp.lmask = lmask;
  bp.stats = p->stats;
  bp.head_stride = p->head_stride;
  bp.head_blk = p->head_blk64;
  bp.B = c.B;
  bp.H = c.H;
  bp.n = c.n;
  bp.r = (int)std::min<int64_t>(c.window / 2, c.n);
  bp.blocks_per_b = p->blocks64_per_b;
  bp.scale = c.scale;
  const int64_t grid = (int64_t)c.B * p->blocks64_per_b;
  if (grid > INT32_MAX) return LWATTN_E_UNSUPPORTED;
  const bool f16 = c.dtype == LWATTN_F16;
  const auto dqk = f16 ? lwk::cz::causal_dq_kernel<_Float16> : lwk::cz::causal_dq_kernel<__bf16>;
  const auto dkvk = f16 ? lwk::cz::causal_dkv_kernel<_Float16> : lwk::cz::causal_dkv_kernel<__bf16>;
  (void)hipFuncSetAttribute((const void*)dqk, hipFuncAttributeMaxDynamicSharedMemorySize, lwk::cz::BW_DQ_SMEM);
  (void)hipFuncSetAttribute((const void*)dkvk, hipFuncAttributeMaxDynamicSharedMemorySize, lwk::cz::BW_DKV_SMEM);
  // dQ and the rows' statistics first; dK, dV read those statistics
  hipLaunchKernelGGL(dqk, dim3((uint32_t)grid), dim3(lwk::bw::NTH), lwk::cz::BW_DQ_SMEM, stream, bp);
  hipLaunchKernelGGL(dkvk, dim3((uint32_t)grid), dim3(lwk::bw::NTH), lwk::cz::BW_DKV_SMEM, stream, bp);
  if (!hip_ok(hipGetLastError(), "hipGetLastError")) return LWATTN_E_DEVICE;
  return LWATTN_OK;
}

lwattn_status lwattn_forward_blocksparse(lwattn_plan_t p, const void* Q, const void* K, const void* V,
                                         const float* lmask, const int32_t* rowptr, const int32_t* cols,
                                         int32_t nnz, int32_t causal, void* O, hipStream_t stream) {
  if (!p) return LWATTN_E_INVALID;
  const lwattn_config& c = p->cfg;
  if ((int64_t)c.B * c.H * c.n == 0) return LWATTN_OK;   // empty problem
  if (c.dtype == LWATTN_F32) return LWATTN_E_UNSUPPORTED;
  // tiles are read through 32-bit buffer offsets over a head's n rows; the
  // column list of a query block lives in LDS
  const int64_t nb = ((int64_t)c.n + 63) / 64;
  if ((int64_t)c.n * 128 >= lwk::OOB_OFF || nb > 4096) return LWATTN_E_UNSUPPORTED;
  const void* ptrs[] = {Q, K, V, O};
  for (const void* q : ptrs)
    if (!q || !aligned16(q)) return LWATTN_E_INVALID;
  if (!lmask || ((uintptr_t)lmask & 3u) || !rowptr || ((uintptr_t)rowptr & 3u) || !cols ||
      ((uintptr_t)cols & 3u) || nnz < 0)
    return LWATTN_E_INVALID;
  if (!hip_ok(hipSetDevice(p->device), "hipSetDevice")) return LWATTN_E_DEVICE;
  lwk::bsp::BsParams bp;
  bp.Q = (const uint8_t*)Q;
  bp.K = (const uint8_t*)K;
  bp.V = (const uint8_t*)V;
  bp.O = (uint8_t*)O;
  bp.lmask = lmask;
  bp.rowptr = rowptr;
  bp.cols = cols;
  bp.B = c.B;
  bp.H = c.H;
  bp.n = c.n;
  bp.nb = (int)nb;
  bp.causal = causal ? 1 : 0;
  bp.nnz = nnz;
  bp.scale = c.scale;
  const int64_t grid = (int64_t)c.B * c.H * nb;
  if (grid > INT32_MAX) return LWATTN_E_UNSUPPORTED;
  const uint32_t smem = (uint32_t)(lwk::bsp::SMEM_BASE + 4 * nb);
  const auto kern =
      c.dtype == LWATTN_F16 ? lwk::bsp::blocksparse_kernel<_Float16> : lwk::bsp::blocksparse_kernel<__bf16>;
  (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  hipLaunchKernelGGL(kern, dim3((uint32_t)grid), dim3(lwk::bw::NTH), smem, stream, bp);
  if (!hip_ok(hipGetLastError(), "hipGetLastError")) return LWATTN_E_DEVICE;
  return LWATTN_OK;
}

lwattn_status lwattn_backward(lwattn_plan_t p, const void* Q, const void* K, const void* V,
                              const void* Qg, const void* Kg, const void* Vg,
                              const float* lmask, const float* gmask, const void* O, const void* dO,
                              void* dQ, void* dK, void* dV, void* dQg, void* dKg, void* dVg,
                              hipStream_t stream) {
  if (!p) return LWATTN_E_INVALID;
  const lwattn_config& c = p->cfg;
  if ((int64_t)c.B * c.H * c.n == 0) return LWATTN_OK;   // empty problem
  const void* ptrs[] = {Q, K, V, Qg, Kg, Vg, O, dO, dQ, dK, dV, dQg, dKg, dVg};
  for (const void* q : ptrs)
    if (!q || !aligned16(q)) return LWATTN_E_INVALID;
  if (!lmask || !gmask || ((uintptr_t)lmask & 3u) || ((uintptr_t)gmask & 3u)) return LWATTN_E_INVALID;
  if (!hip_ok(hipSetDevice(p->device), "hipSetDevice")) return LWATTN_E_DEVICE;

  // 1. the global-index compaction (published under a fresh epoch, so that the
  //    next forward's waits still see a new number): inside the dQ launch for
  //    bf16, a launch of its own for fp32
  lwk::Params cp;
  std::memset(&cp, 0, sizeof(cp));
  cp.lmask = lmask;
  cp.gmask = gmask;
  cp.flags = p->flags;
  cp.gidx = p->gidx;
  cp.gcnt = p->gcnt;
  cp.status = p->status;
  cp.ready = p->ready;
  cp.ready_cnt = p->ready_cnt;
  cp.fault = p->fault;
  p->epoch = p->epoch >= INT32_MAX - 1 ? 1 : p->epoch + 1;
  cp.epoch = p->epoch;
  cp.publish = p->epoch;
  cp.B = c.B;
  cp.H = c.H;
  cp.n = c.n;
  cp.max_global = c.max_global;
  cp.mask_vec = ((((uintptr_t)lmask | (uintptr_t)gmask) & 15u) == 0 && (c.n % 4) == 0) ? 1 : 0;
  bool timed = false;
  if (p->timing_cap > 0 && p->bw_calls < p->timing_cap) {
    timed = (p->bw_seen % p->timing_every) == 0;
    ++p->bw_seen;
  }
  // a timed backward launches each kernel with the pair of events its
  // dispatch records (slot k: events 2k, 2k + 1 of the call's record)
  uint8_t launched = 0;   // slots whose kernel this call launches
  auto ev = [&](int k, int e) -> hipEvent_t {
    if (!timed) return nullptr;
    launched |= (uint8_t)(1u << k);
    return p->bw_events[(size_t)p->bw_calls * 2 * kNumBwKernels + 2 * k + e];
  };
  cp.spin_limit = (1 << 18) + (int32_t)(c.n >> 2);   // as the forward's waits
  if (p->inject_timeout && c.dtype != LWATTN_F32) {
    // fault test: the rows are published under another number and the dQ
    // workgroups that wait for them (compaction inside dQ) give up at once
    p->inject_timeout = false;
    cp.publish = -1;
    cp.spin_limit = 64;
  }

  lwk::bw::BwParams bp;
  bp.Q = (const uint8_t*)Q;
  bp.K = (const uint8_t*)K;
  bp.V = (const uint8_t*)V;
  bp.Qg = (const uint8_t*)Qg;
  bp.Kg = (const uint8_t*)Kg;
  bp.Vg = (const uint8_t*)Vg;
  bp.O = (const uint8_t*)O;
  bp.dO = (const uint8_t*)dO;
  bp.dQ = (uint8_t*)dQ;
  bp.dK = (uint8_t*)dK;
  bp.dV = (uint8_t*)dV;
  bp.dQg = (uint8_t*)dQg;
  bp.dKg = (uint8_t*)dKg;
  bp.dVg = (uint8_t*)dVg;
  bp.lmask = lmask;
  bp.gmask = gmask;
  bp.gidx = p->gidx;
  bp.gcnt = p->gcnt;
  bp.head_stride = p->head_stride;
  bp.head_blk = p->head_blk64;
  bp.stats = p->stats;
  bp.gq = p->gq;
  bp.gk = p->gk;
  bp.gml = p->gml;
  bp.gspad = (p->gsplit + 1) / 2 * 2;
  bp.comp_fold = 0;
  bp.merge_fold = 0;
  bp.gsplit = p->gsplit;
  bp.gchunk = p->gchunk;
  bp.B = c.B;
  bp.H = c.H;
  bp.n = c.n;
  bp.r = (int)std::min<int64_t>(c.window / 2, c.n);
  bp.max_global = c.max_global;
  bp.ntg = (c.max_global + lwk::bw::T - 1) / lwk::bw::T;
  bp.blocks_per_b = p->blocks64_per_b;
  bp.scale = c.scale;
  const int64_t grid = (int64_t)c.B * p->blocks64_per_b + (int64_t)c.B * c.H * bp.ntg;
  if (grid > INT32_MAX) return LWATTN_E_UNSUPPORTED;
  if (c.dtype != LWATTN_F32) {
    // 2. dQ, dQg (zero) and the local rows' statistics; 3. the chunk sums of
    // the global rows and keys; 4. their merge: dQg, the global keys' dK, dV
    // (and the global rows' statistics, unless it runs inside 5); 5. dK, dV
    // (window), dKg, dVg
    namespace mk = lwk::bw::mk;
    const int64_t nblk = (int64_t)c.B * p->blocks64_per_b;
    const int64_t nchunk = (int64_t)c.B * c.H * bp.ntg * p->gsplit;
    const int64_t nmerge = ((int64_t)c.B * c.H * c.max_global + 3) / 4;
    // tiles are read through 32-bit buffer offsets over a head's n rows
    if (nchunk > INT32_MAX || nmerge > INT32_MAX || (int64_t)c.n * 128 >= lwk::OOB_OFF)
      return LWATTN_E_UNSUPPORTED;
    // the kernels of the plan's 16-bit storage type (bf16 or fp16)
    const bool f16 = c.dtype == LWATTN_F16;
    const auto dq_fold = f16 ? mk::dq_kernel<true, _Float16> : mk::dq_kernel<true, __bf16>;
    const auto dq_plain = f16 ? mk::dq_kernel<false, _Float16> : mk::dq_kernel<false, __bf16>;
    const auto dkv_fold = f16 ? mk::dkv_kernel<true, _Float16> : mk::dkv_kernel<true, __bf16>;
    const auto dkv_plain = f16 ? mk::dkv_kernel<false, _Float16> : mk::dkv_kernel<false, __bf16>;
    const auto chunk_k = f16 ? mk::global_chunk_kernel<_Float16> : mk::global_chunk_kernel<__bf16>;
    const auto merge_k = f16 ? mk::global_merge_kernel<_Float16> : mk::global_merge_kernel<__bf16>;
    for (const void* f : {(const void*)dq_fold, (const void*)dq_plain})
      (void)hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, mk::DQ_SMEM);
    for (const void* f : {(const void*)dkv_fold, (const void*)dkv_plain})
      (void)hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, mk::DKV_SMEM);
    (void)hipFuncSetAttribute((const void*)chunk_k, hipFuncAttributeMaxDynamicSharedMemorySize, mk::GS_SMEM);
    // When the dQ grid fits one round of workgroup slots (three per compute
    // unit), its first B workgroups compact the batch rows and the others
    // wait for their row before their global tiles: no launch of its own.  On
    // longer grids the first round would stall on that wait, so the
    // compaction is a launch of its own there (measured, base: 101 -> 94 us
    // with both folds; qa and long slower folded).
    bp.comp_fold = nblk <= 3 * (int64_t)p->ncu && c.B <= nblk ? 1 : 0;
    if (!bp.comp_fold)
      hipExtLaunchKernelGGL(lwk::bw::compact_kernel, dim3(c.B), dim3(lwk::NT), (uint32_t)(lwk::NW * 4), stream,
                            ev(0, 0), ev(0, 1), 0u, cp);
    hipExtLaunchKernelGGL(bp.comp_fold ? dq_fold : dq_plain, dim3((uint32_t)nblk),
                          dim3(lwk::bw::NTH), mk::DQ_SMEM, stream, ev(1, 0), ev(1, 1), 0u, bp, cp);
    if (nchunk > 0)
      hipExtLaunchKernelGGL(chunk_k, dim3((uint32_t)nchunk), dim3(lwk::bw::NTH), mk::GS_SMEM,
                            stream, ev(2, 0), ev(2, 1), 0u, bp);
    // The merge of the chunk sums runs in workgroups behind the key blocks of
    // the dK/dV launch when the last round of that grid (two workgroups per
    // compute unit) has the spare slots for them; otherwise (each merge
    // workgroup would hold a key block's slot while it waits on memory) it is
    // a launch of its own, which also leaves the global rows' statistics.
    const int64_t dslots = 2 * (int64_t)p->ncu;
    const int64_t mwg = nchunk > 0 ? nmerge : 0;
    const int64_t spare = (nblk + dslots - 1) / dslots * dslots - nblk;
    bp.merge_fold = mwg > 0 && mwg <= spare ? 1 : 0;
    if (mwg > 0 && !bp.merge_fold)
      hipExtLaunchKernelGGL(merge_k, dim3((uint32_t)nmerge), dim3(lwk::bw::NTH), 0, stream,
                            ev(3, 0), ev(3, 1), 0u, bp);
    const int64_t ndkv = nblk + (bp.merge_fold ? mwg : 0);
    hipExtLaunchKernelGGL(bp.merge_fold ? dkv_fold : dkv_plain, dim3((uint32_t)ndkv),
                          dim3(lwk::bw::NTH), mk::DKV_SMEM, stream, ev(4, 0), ev(4, 1), 0u, bp);
  } else {
    hipExtLaunchKernelGGL(lwk::bw::compact_kernel, dim3(c.B), dim3(lwk::NT), (uint32_t)(lwk::NW * 4), stream,
                          ev(0, 0), ev(0, 1), 0u, cp);
    // 2. dQ, dQg and the rows' statistics; 3. dK, dV, dKg, dVg
    (void)hipFuncSetAttribute((const void*)lwk::bw::dq_kernel<false>, hipFuncAttributeMaxDynamicSharedMemorySize, lwk::bw::DQ_SMEM);
    (void)hipFuncSetAttribute((const void*)lwk::bw::dkv_kernel<false>, hipFuncAttributeMaxDynamicSharedMemorySize, lwk::bw::DKV_SMEM);
    hipExtLaunchKernelGGL(lwk::bw::dq_kernel<false>, dim3((uint32_t)grid), dim3(lwk::bw::NTH), lwk::bw::DQ_SMEM,
                          stream, ev(1, 0), ev(1, 1), 0u, bp);
    hipExtLaunchKernelGGL(lwk::bw::dkv_kernel<false>, dim3((uint32_t)grid), dim3(lwk::bw::NTH), lwk::bw::DKV_SMEM,
                          stream, ev(4, 0), ev(4, 1), 0u, bp);
  }
  if (!hip_ok(hipGetLastError(), "hipGetLastError")) return LWATTN_E_DEVICE;
  if (timed) {
    p->bw_launched[(size_t)p->bw_calls] = launched;
    ++p->bw_calls;
  }
  return LWATTN_OK;
}

lwattn_status lwattn_global_index(lwattn_plan_t p, int32_t* gidx, int32_t* gcnt, hipStream_t stream) {
  if (!p || !gidx || !gcnt) return LWATTN_E_INVALID;
  const size_t B = (size_t)p->cfg.B, n = (size_t)p->cfg.n;
  if (B == 0) return LWATTN_OK;
  if (!hip_ok(hipSetDevice(p->device), "hipSetDevice")) return LWATTN_E_DEVICE;
  if (n > 0 && !hip_ok(hipMemcpyAsync(gidx, p->gidx, B * n * 4, hipMemcpyDeviceToDevice, stream), "hipMemcpyAsync"))
    return LWATTN_E_DEVICE;
  if (!hip_ok(hipMemcpyAsync(gcnt, p->gcnt, B * 4, hipMemcpyDeviceToDevice, stream), "hipMemcpyAsync"))
    return LWATTN_E_DEVICE;
  return LWATTN_OK;
}

lwattn_status lwattn_sync_status(lwattn_plan_t p, hipStream_t stream) {
  if (!p) return LWATTN_E_INVALID;
  if (!hip_ok(hipSetDevice(p->device), "hipSetDevice")) return LWATTN_E_DEVICE;
  if (!hip_ok(hipStreamSynchronize(stream), "hipStreamSynchronize")) return LWATTN_E_DEVICE;
  const int B = p->cfg.B;
  if (B == 0) return LWATTN_OK;
  int32_t fault = 0;
  if (!hip_ok(hipMemcpy(&fault, p->fault, 4, hipMemcpyDeviceToHost), "hipMemcpy")) return LWATTN_E_DEVICE;
  if (fault) return LWATTN_E_DEVICE;
  std::vector<int32_t> st(B);
  if (!hip_ok(hipMemcpy(st.data(), p->status, (size_t)B * 4, hipMemcpyDeviceToHost), "hipMemcpy"))
    return LWATTN_E_DEVICE;
  for (int b = 0; b < B; ++b)
    if (st[b]) return LWATTN_E_TOO_MANY_GLOBALS;
  return LWATTN_OK;
}

lwattn_status lwattn_timing_enable(lwattn_plan_t p, int32_t max_calls) {
  if (!p || max_calls <= 0) return LWATTN_E_INVALID;
  if (!hip_ok(hipSetDevice(p->device), "hipSetDevice")) return LWATTN_E_DEVICE;
  for (hipEvent_t e : p->events) (void)hipEventDestroy(e);
  for (hipEvent_t e : p->bw_events) (void)hipEventDestroy(e);
  p->events.clear();
  p->bw_events.clear();
  p->timing_cap = 0;
  p->timing_calls = 0;
  p->timing_seen = 0;
  p->bw_calls = 0;
  p->bw_seen = 0;
  auto make = [&](std::vector<hipEvent_t>& v, size_t ne) {
    v.reserve(ne);
    for (size_t i = 0; i < ne; ++i) {
      hipEvent_t e;
      if (!hip_ok(hipEventCreate(&e), "hipEventCreate")) return false;
      v.push_back(e);
    }
    return true;
  };
  if (!make(p->events, (size_t)max_calls * (kNumKernels + 1)) ||
      !make(p->bw_events, (size_t)max_calls * 2 * kNumBwKernels))
    return LWATTN_E_DEVICE;
  p->bw_launched.assign((size_t)max_calls, 0);
  p->timing_cap = max_calls;
  return LWATTN_OK;
}

lwattn_status lwattn_timing_every(lwattn_plan_t p, int32_t every) {
  if (!p || every < 1) return LWATTN_E_INVALID;
  p->timing_every = every;
  p->timing_seen = 0;
  p->bw_seen = 0;
  return LWATTN_OK;
}

lwattn_status lwattn_timing_read(lwattn_plan_t p, float* ms, int32_t cap, int32_t* nkernels,
                                 int32_t* ncalls) {
  if (!p || !nkernels || !ncalls || (cap > 0 && !ms)) return LWATTN_E_INVALID;
  if (!hip_ok(hipSetDevice(p->device), "hipSetDevice")) return LWATTN_E_DEVICE;
  float tot[kNumKernels] = {};
  for (int call = 0; call < p->timing_calls; ++call) {
    hipEvent_t* ev = &p->events[(size_t)call * (kNumKernels + 1)];
    if (!hip_ok(hipEventSynchronize(ev[kNumKernels]), "hipEventSynchronize")) return LWATTN_E_DEVICE;
    for (int k = 0; k < kNumKernels; ++k) {
      float t = 0.f;
      if (!hip_ok(hipEventElapsedTime(&t, ev[k], ev[k + 1]), "hipEventElapsedTime")) return LWATTN_E_DEVICE;
      tot[k] += t;
    }
  }
  for (int k = 0; k < kNumKernels && k < cap; ++k) ms[k] = tot[k];
  *nkernels = kNumKernels;
  *ncalls = p->timing_calls;
  return LWATTN_OK;
}

lwattn_status lwattn_test_inject_wait_timeout(lwattn_plan_t p) {
  if (!p) return LWATTN_E_INVALID;
  p->inject_timeout = true;
  return LWATTN_OK;
}

lwattn_status lwattn_timing_disable(lwattn_plan_t p) {
  if (!p) return LWATTN_E_INVALID;
  (void)hipSetDevice(p->device);
  for (hipEvent_t e : p->events) (void)hipEventDestroy(e);
  for (hipEvent_t e : p->bw_events) (void)hipEventDestroy(e);
  p->events.clear();
  p->bw_events.clear();
  p->timing_cap = 0;
  p->timing_calls = 0;
  p->bw_calls = 0;
  return LWATTN_OK;
}

lwattn_status lwattn_layer_create(lwattn_plan_t p, int32_t inter, float eps, lwattn_layer_t* out) {
  if (!out) return LWATTN_E_INVALID;
  *out = nullptr;
  if (!p || inter <= 0 || (inter % 8) != 0 || !(eps > 0.0f)) return LWATTN_E_INVALID;
  const lwattn_config& c = p->cfg;
  const int H = c.H;
  if (c.dtype == LWATTN_F32 || !layer_heads_ok(H)) return LWATTN_E_UNSUPPORTED;
  const int64_t M = (int64_t)c.B * c.n, hid = (int64_t)H * 64;
  const int mg = std::min(c.max_global, c.n);
  if (M * std::max<int64_t>(3 * hid, inter) >= ((int64_t)1 << 31) || (int64_t)c.B * mg * hid >= ((int64_t)1 << 31))
    return LWATTN_E_UNSUPPORTED;
  if (!hip_ok(hipSetDevice(p->device), "hipSetDevice")) return LWATTN_E_DEVICE;
  lwattn_layer_t L = new (std::nothrow) lwattn_layer_s;
  if (!L) return LWATTN_E_NOMEM;
  L->attn = p;
  L->inter = inter;
  L->eps = eps;
  L->mg = mg;
  bool ok = true;
  auto alloc = [&](void** ptr, size_t bytes) {
    if (!ok) return;
    if (bytes == 0) bytes = 16;
    if (!hip_ok(hipMalloc(ptr, bytes), "hipMalloc")) { ok = false; *ptr = nullptr; }
  };
  alloc((void**)&L->P, (size_t)M * std::max<int64_t>(3 * hid, inter) * 4);
  alloc(&L->P2, (size_t)M * 2 * hid * 2);
  alloc((void**)&L->Pg, (size_t)c.B * mg * hid * 4);
  for (auto*& q : L->qkv) alloc(&q, (size_t)M * hid * 2);
  alloc(&L->A, (size_t)M * hid * 2);
  alloc(&L->Am, (size_t)M * hid * 2);
  alloc(&L->H1, (size_t)M * hid * 2);
  alloc(&L->F, (size_t)M * inter * 2);
  alloc(&L->Xg, (size_t)c.B * mg * hid * 2);
  alloc((void**)&L->gpos, (size_t)c.B * mg * 4);
  if (ok && rocblas_create_handle(&L->blas) != rocblas_status_success) ok = false;
  // hipBLASLt for the GEMMs (rocBLAS takes a shape it has no algorithm for),
  // each shape's algorithm timed here on scratch operands
  if (ok && hipblasLtCreate(&L->lt) != HIPBLAS_STATUS_SUCCESS) L->lt = nullptr;
  if (ok && L->lt) {
    const hipDataType dt = c.dtype == LWATTN_F16 ? HIP_R_16F : HIP_R_16BF;
    const int64_t Mg = (int64_t)c.B * mg, big = std::max<int64_t>(3 * hid, inter);
    LtTune tu;
    tu.ws_cap = (size_t)32 << 20;
    const size_t wb = (size_t)std::max(hid, (int64_t)inter) * big * 2, xb = (size_t)M * big * 2,
                 yb = (size_t)M * big * 4;
    bool tok = hipMalloc(&tu.w, wb) == hipSuccess && hipMalloc(&tu.x, xb) == hipSuccess &&
               hipMalloc((void**)&tu.y, yb) == hipSuccess && hipMalloc(&tu.ws, tu.ws_cap) == hipSuccess &&
               hipStreamCreate(&tu.stream) == hipSuccess && hipEventCreate(&tu.e0) == hipSuccess &&
               hipEventCreate(&tu.e1) == hipSuccess && hipMemset(tu.w, 0, wb) == hipSuccess &&
               hipMemset(tu.x, 0, xb) == hipSuccess && hipDeviceSynchronize() == hipSuccess;
    if (!tok) tu.stream = nullptr;   // no tuning: every shape goes to rocBLAS
    // Q|K|V and Kg|Vg: bias epilogue, 16-bit result (the split kernel then
    // only moves it)
    lt_setup(L->lt, L->g_qkv, dt, M, 3 * hid, hid, 3 * hid, tu, true);
    lt_setup(L->lt, L->g_kv, dt, M, 2 * hid, hid, 3 * hid, tu, true);
    lt_setup(L->lt, L->g_qg, dt, Mg, hid, hid, 3 * hid, tu);
    lt_setup(L->lt, L->g_o, dt, M, hid, hid, hid, tu, true);
    lt_setup(L->lt, L->g_f1, dt, M, inter, hid, inter, tu, true);
    lt_setup(L->lt, L->g_f2, dt, M, hid, inter, hid, tu, true);
    if (tu.e0) (void)hipEventDestroy(tu.e0);
    if (tu.e1) (void)hipEventDestroy(tu.e1);
    if (tu.stream) (void)hipStreamDestroy(tu.stream);
    (void)hipFree(tu.w);
    (void)hipFree(tu.x);
    (void)hipFree(tu.y);
    (void)hipFree(tu.ws);
    (void)hipGetLastError();
    for (const LtGemm* g : {&L->g_qkv, &L->g_kv, &L->g_qg, &L->g_o, &L->g_f1, &L->g_f2})
      if (g->ok) L->lt_ws_bytes = std::max(L->lt_ws_bytes, g->ws);
    if (L->lt_ws_bytes) alloc(&L->lt_ws, L->lt_ws_bytes);
    if (L->g_qg.ok && L->g_qg.ws) alloc(&L->lt_ws_side, L->g_qg.ws);
  }
  // the side stream (default priority) only when the Qg GEMM runs on
  // hipBLASLt (rocBLAS's handle follows the caller's stream)
  if (ok && mg > 0 && L->g_qg.ok) {
    ok = hip_ok(hipStreamCreateWithFlags(&L->side, hipStreamNonBlocking), "hipStreamCreateWithFlags") &&
         hip_ok(hipEventCreateWithFlags(&L->fork, hipEventDisableTiming), "hipEventCreateWithFlags") &&
         hip_ok(hipEventCreateWithFlags(&L->join, hipEventDisableTiming), "hipEventCreateWithFlags");
  }
  if (!ok) {
    free_layer(L);
    return LWATTN_E_NOMEM;
  }
  *out = L;
  return LWATTN_OK;
}

// (a template inside the extern "C" block: C++ linkage of its own)
extern "C++" {
template <typename T>
static lwattn_status layer_forward(lwattn_layer_t L, rocblas_datatype dt, const void* X, const lwattn_layer_weights* w,
                                   const float* lmask, const float* gmask, void* Y, hipStream_t stream) {
  lwattn_plan_t p = L->attn;
  const lwattn_config& c = p->cfg;
  const int H = c.H, mg = L->mg;
  const int64_t M = (int64_t)c.B * c.n, hid = (int64_t)H * 64, inter = L->inter;
  namespace ly = lwk::layer;
  auto blocks = [](int64_t threads) { return dim3((uint32_t)((threads + ly::LNT - 1) / ly::LNT)); };
  T* const* t = reinterpret_cast<T* const*>(L->qkv);
  // 1. projections.  Q, K, V: every row, the bias added by the GEMM's
  // epilogue (or while splitting heads, on the fallback).
  const T* wg = (const T*)w->w_g;
  auto project = [&](const LtGemm& g, const void* W, const T* bias, T* o0, T* o1, T* o2, int parts) {
    if (g.bias16) {
      if (!layer_gemm_bias(L, g, X, W, bias, L->P, stream)) return false;
      hipLaunchKernelGGL(ly::split_heads16<T>, blocks(M * parts * hid / 8), dim3(ly::LNT), 0, stream,
                         (const T*)L->P, o0, o1, o2, parts, c.B, c.n, H);
    } else {
      if (!layer_gemm(L, g, dt, X, W, L->P, stream)) return false;
      hipLaunchKernelGGL(ly::split_heads<T>, blocks(M * parts * hid / 8), dim3(ly::LNT), 0, stream, L->P, bias,
                         o0, o1, o2, parts, c.B, c.n, H);
    }
    return true;
  };
  // Qg: only the global tokens' rows (the attention reads Qg nowhere else),
  // gathered, projected by the first column block of w_g and scattered back;
  // a chain of small launches that runs on the side stream beside the big
  // projections
  const bool side = mg > 0 && L->side;
  if (mg > 0) {
    hipStream_t qs = stream;
    if (side) {
      if (!hip_ok(hipEventRecord(L->fork, stream), "hipEventRecord") ||
          !hip_ok(hipStreamWaitEvent(L->side, L->fork, 0), "hipStreamWaitEvent"))
        return LWATTN_E_DEVICE;
      qs = L->side;
    }
    const int64_t rows = (int64_t)c.B * mg;
    hipLaunchKernelGGL(ly::find_global_rows, dim3((uint32_t)c.B), dim3(ly::LNT), 0, qs, lmask, gmask, c.n, mg,
                       L->gpos);
    hipLaunchKernelGGL(ly::gather_global_rows<T>, dim3((uint32_t)((rows + 3) / 4)), dim3(ly::LNT), 0, qs,
                       (const T*)X, L->gpos, c.n, (int)hid, mg, rows, (T*)L->Xg);
    if (!layer_gemm(L, L->g_qg, dt, L->Xg, wg, L->Pg, qs, side ? L->lt_ws_side : nullptr)) return LWATTN_E_DEVICE;
    hipLaunchKernelGGL(ly::scatter_global_rows<T>, blocks((int64_t)c.B * mg * hid / 8), dim3(ly::LNT), 0, qs,
                       L->Pg, (const T*)w->b_g, L->gpos, t[3], c.B, c.n, H, mg);
    if (side && !hip_ok(hipEventRecord(L->join, L->side), "hipEventRecord")) return LWATTN_E_DEVICE;
  }
  // Q, K, V and Kg, Vg (every row: the global rows attend to all keys, from
  // the last two column blocks of w_g).  With both GEMMs' 16-bit bias
  // epilogues, the attention reads the heads straight from the GEMM results
  // ([M, 3 hid] and [M, 2 hid] row-major) when every key offset its fast path
  // forms fits in 32 bits; else the heads are split into [B, H, n, 64].
  int smax = 1;
  for (int32_t v : p->stride_host) smax = std::max(smax, (int)v);
  const int64_t rs_qkv = 3 * hid * 2, rs_kv = 2 * hid * 2;
  const bool in_rows = L->g_qkv.bias16 && L->g_kv.bias16 &&
                       ((int64_t)c.n + 128 * (int64_t)smax) * rs_qkv < ((int64_t)1 << 31) - (1 << 20);
  const T* pq = (const T*)L->P;
  const T* pk = (const T*)L->P2;
  if (in_rows) {
    if (!layer_gemm_bias(L, L->g_qkv, X, w->w_qkv, w->b_qkv, L->P, stream) ||
        !layer_gemm_bias(L, L->g_kv, X, wg + hid, (const T*)w->b_g + hid, L->P2, stream))
      return LWATTN_E_DEVICE;
  } else {
    if (!project(L->g_qkv, w->w_qkv, (const T*)w->b_qkv, t[0], t[1], t[2], 3)) return LWATTN_E_DEVICE;
    if (!project(L->g_kv, wg + hid, (const T*)w->b_g + hid, t[4], t[5], t[5], 2)) return LWATTN_E_DEVICE;
  }
  if (side && !hip_ok(hipStreamWaitEvent(stream, L->join, 0), "hipStreamWaitEvent")) return LWATTN_E_DEVICE;
  if (!hip_ok(hipGetLastError(), "hipGetLastError")) return LWATTN_E_DEVICE;
  // 2. the attention, its output rows written token-major ([M, hid]: the
  // heads merged) when a head's rows span less than 2^31 bytes
  const bool tok = (int64_t)c.n * hid * 2 < ((int64_t)1 << 31);
  InRows rows;
  rows.rs_qkv = rs_qkv;
  rows.rs_kv = rs_kv;
  lwattn_status st =
      in_rows ? forward_impl(p, pq, pq + hid, pq + 2 * hid, L->qkv[3], pk, pk + hid, lmask, gmask, tok ? L->Am : L->A,
                             tok, &rows, stream)
              : forward_impl(p, L->qkv[0], L->qkv[1], L->qkv[2], L->qkv[3], L->qkv[4], L->qkv[5], lmask, gmask,
                             tok ? L->Am : L->A, tok, nullptr, stream);
  if (st != LWATTN_OK) return st;
  // 3. output projection, bias, residual, LayerNorm
  if (!tok)
    hipLaunchKernelGGL(ly::merge_heads<T>, blocks(M * hid / 8), dim3(ly::LNT), 0, stream, (const T*)L->A, (T*)L->Am,
                       c.B, c.n, H);
  // (with the 16-bit bias epilogue the GEMM adds the bias and rounds its
  // result to the storage type, which the LayerNorm reads)
  auto project_out = [&](const LtGemm& g, const void* A, const void* W, const void* bias) {
    return g.bias16 ? layer_gemm_bias(L, g, A, W, bias, L->P, stream) : layer_gemm(L, g, dt, A, W, L->P, stream);
  };
  if (!project_out(L->g_o, L->Am, w->w_o, w->b_o)) return LWATTN_E_DEVICE;
  if (!layernorm<T>(H, L->P, L->g_o.bias16, w->b_o, X, w->ln1_g, w->ln1_b, L->eps, L->H1, M, stream))
    return LWATTN_E_UNSUPPORTED;
  // 4. FFN: intermediate GEMM, bias, GELU; output GEMM, bias, residual, LayerNorm
  if (L->g_f1.bias16) {
    // the bias in the GEMM's epilogue, the 16-bit result straight into F
    if (!layer_gemm_bias(L, L->g_f1, L->H1, w->w_1, w->b_1, L->F, stream)) return LWATTN_E_DEVICE;
    hipLaunchKernelGGL(ly::gelu16<T>, blocks(M * inter / 8), dim3(ly::LNT), 0, stream, (T*)L->F, M * inter / 8);
  } else {
    if (!layer_gemm(L, L->g_f1, dt, L->H1, w->w_1, L->P, stream)) return LWATTN_E_DEVICE;
    hipLaunchKernelGGL(ly::bias_gelu<T>, blocks(M * inter / 8), dim3(ly::LNT), 0, stream, L->P, (const T*)w->b_1,
                       (T*)L->F, M, (int)inter);
  }
  if (!project_out(L->g_f2, L->F, w->w_2, w->b_2)) return LWATTN_E_DEVICE;
  if (!layernorm<T>(H, L->P, L->g_f2.bias16, w->b_2, L->H1, w->ln2_g, w->ln2_b, L->eps, Y, M, stream))
    return LWATTN_E_UNSUPPORTED;
  if (!hip_ok(hipGetLastError(), "hipGetLastError")) return LWATTN_E_DEVICE;
  return LWATTN_OK;
}
}  // extern "C++"

lwattn_status lwattn_layer_forward(lwattn_layer_t L, const void* X, const lwattn_layer_weights* w,
                                   const float* lmask, const float* gmask, void* Y, hipStream_t stream) {
  if (!L || !w) return LWATTN_E_INVALID;
  lwattn_plan_t p = L->attn;
  const lwattn_config& c = p->cfg;
  if ((int64_t)c.B * c.n == 0) return LWATTN_OK;
  const void* ptrs[] = {X, Y, w->w_qkv, w->b_qkv, w->w_g, w->b_g, w->w_o, w->b_o, w->ln1_g, w->ln1_b,
                        w->w_1, w->b_1, w->w_2, w->b_2, w->ln2_g, w->ln2_b};
  for (const void* q : ptrs)
    if (!q || !aligned16(q)) return LWATTN_E_INVALID;
  if (!lmask || !gmask || ((uintptr_t)lmask & 3u) || ((uintptr_t)gmask & 3u)) return LWATTN_E_INVALID;
  if (!hip_ok(hipSetDevice(p->device), "hipSetDevice")) return LWATTN_E_DEVICE;
  if (rocblas_set_stream(L->blas, stream) != rocblas_status_success) return LWATTN_E_DEVICE;
  if (c.dtype == LWATTN_F16) return layer_forward<_Float16>(L, rocblas_datatype_f16_r, X, w, lmask, gmask, Y, stream);
  return layer_forward<__bf16>(L, rocblas_datatype_bf16_r, X, w, lmask, gmask, Y, stream);
}

lwattn_status lwattn_layer_destroy(lwattn_layer_t L) {
  free_layer(L);
  return LWATTN_OK;
}

lwattn_status lwattn_timing_read_backward(lwattn_plan_t p, float* ms, int32_t cap, int32_t* nkernels,
                                          int32_t* ncalls) {
  if (!p || !nkernels || !ncalls || (cap > 0 && !ms)) return LWATTN_E_INVALID;
  if (!hip_ok(hipSetDevice(p->device), "hipSetDevice")) return LWATTN_E_DEVICE;
  float tot[kNumBwKernels] = {};
  for (int call = 0; call < p->bw_calls; ++call) {
    hipEvent_t* ev = &p->bw_events[(size_t)call * 2 * kNumBwKernels];
    // the dK/dV kernel ends every backward
    if (!hip_ok(hipEventSynchronize(ev[2 * kNumBwKernels - 1]), "hipEventSynchronize")) return LWATTN_E_DEVICE;
    for (int k = 0; k < kNumBwKernels; ++k) {
      // only the pairs of kernels this call launched were recorded
      if (!((p->bw_launched[(size_t)call] >> k) & 1u)) continue;
      float t = 0.f;
      if (!hip_ok(hipEventElapsedTime(&t, ev[2 * k], ev[2 * k + 1]), "hipEventElapsedTime"))
        return LWATTN_E_DEVICE;
      tot[k] += t;
    }
  }
  for (int k = 0; k < kNumBwKernels && k < cap; ++k) ms[k] = tot[k];
  *nkernels = kNumBwKernels;
  *ncalls = p->bw_calls;
  return LWATTN_OK;
}


lwattn_status lwattn_probe_mfma(int32_t iters, float* out, hipStream_t stream) {
  if (iters < 0 || !out || ((uintptr_t)out & 3u)) return LWATTN_E_INVALID;
  hipLaunchKernelGGL(lwk::probe::mfma_probe_kernel, dim3(lwk::probe::MFMA_BLOCKS), dim3(lwk::probe::MFMA_THREADS), 0,
                     stream, (int)iters, 1.0f / 1024.0f, out);
  if (!hip_ok(hipGetLastError(), "hipGetLastError")) return LWATTN_E_DEVICE;
  return LWATTN_OK;
}

lwattn_status lwattn_probe_read(const void* buf, int64_t bytes, float* out, hipStream_t stream) {
  if (!buf || !out || bytes < 0 || ((uintptr_t)buf & 15u) || ((uintptr_t)out & 3u)) return LWATTN_E_INVALID;
  hipLaunchKernelGGL(lwk::probe::read_probe_kernel, dim3(lwk::probe::READ_BLOCKS), dim3(lwk::probe::READ_THREADS), 0,
                     stream, (const uint4*)buf, bytes / 16, out);
  if (!hip_ok(hipGetLastError(), "hipGetLastError")) return LWATTN_E_DEVICE;
  return LWATTN_OK;
}


lwattn_status lwattn_forward_noalloc(const lwattn_config* cfg, int hip_device, const void* Q, const void* K,
                                     const void* V, const void* Qg, const void* Kg, const void* Vg,
                                     const float* lmask, const float* gmask, void* O, int32_t* status,
                                     hipStream_t stream) {
  lwattn_status st = lwattn_check_config(cfg);
  if (st != LWATTN_OK) return st;
  const lwattn_config& c = *cfg;
  if (hip_device < 0 || hip_device >= kMaxDevices) return LWATTN_E_INVALID;
  if (status && ((uintptr_t)status & 3u)) return LWATTN_E_INVALID;
  bool empty = false;
  st = forward_args(c, Q, K, V, Qg, Kg, Vg, lmask, gmask, O, &empty);
  if (st != LWATTN_OK || empty) return st;
  // the head tables travel by value in the kernel arguments
  if (c.H > lwk::MAXH_ARG) return LWATTN_E_UNSUPPORTED;
  int32_t gap[lwk::MAXH_ARG], stride[lwk::MAXH_ARG], blk[lwk::MAXH_ARG + 1];
  for (int h = 0; h < c.H; ++h) gap[h] = c.dilation ? c.dilation[h] : 0;
  if (!hip_ok(hipSetDevice(hip_device), "hipSetDevice")) return LWATTN_E_DEVICE;
  uint8_t* base = (uint8_t*)scratch_of(hip_device);
  if (!base) return LWATTN_E_DEVICE;
  FwdGeom g;
  if (!forward_geometry(c, gap, g_scratch_ncu[hip_device], g, stride, blk)) return LWATTN_E_INVALID;

  // layout: the words that must start at zero (ready [B], fault, status [B],
  // gcnt [B], merge counters [B H nqt], band part counters), then the flags,
  // the global index, the global rows' partials and the band blocks' key
  // parts, each 256-byte aligned
  const size_t B = (size_t)c.B, n = (size_t)c.n;
  const size_t ntile = B * c.H * (size_t)(g.nqt > 0 ? g.nqt : 1);
  const size_t nzero = 3 * B + 1 + ntile + bcnt_words(g);
  const size_t nparts = fwd_parts(c, g);
  const size_t off_flags = align256(nzero * 4);
  const size_t off_gidx = off_flags + align256(B * n);
  const size_t off_po = off_gidx + align256(B * n * 4);
  const size_t off_pml = off_po + align256(nparts * lwk::D * 4);
  const size_t off_bpo = off_pml + align256(nparts * 2 * 4);
  const size_t off_bpml = off_bpo + align256(bpart_o_floats(g) * 4);
  const size_t total = off_bpml + align256(bpart_ml_floats(g) * 4);
  if (total > kScratchBytes || nzero > (size_t)INT32_MAX) return LWATTN_E_SCRATCH;

  FwdWork w;
  int32_t* ctrl = (int32_t*)base;
  w.ready = ctrl;
  w.fault = ctrl + B;
  w.status = ctrl + B + 1;
  w.gcnt = ctrl + 2 * B + 1;
  w.tile_cnt = ctrl + 3 * B + 1;
  w.bcnt = ctrl + 3 * B + 1 + ntile;
  w.bpart_o = (float*)(base + off_bpo);
  w.bpart_ml = (float*)(base + off_bpml);
  w.flags = base + off_flags;
  w.gidx = (int32_t*)(base + off_gidx);
  w.part_o = (float*)(base + off_po);
  w.part_ml = (float*)(base + off_pml);
  w.head_stride = nullptr;
  w.head_blk = nullptr;
  lwk::Params prm;
  // the readiness words start at zero on every call, so every call is forward 1
  forward_params(prm, c, g, w, stride, blk, Q, K, V, Qg, Kg, Vg, lmask, gmask, O, 1);
  const int zblocks = (int)std::min<size_t>((nzero + 255) / 256, 1024);
  hipLaunchKernelGGL(zero_words_kernel, dim3(zblocks), dim3(256), 0, stream, ctrl, (int)nzero);
  if (!hip_ok(hipGetLastError(), "hipGetLastError")) return LWATTN_E_DEVICE;
  if (!launch_forward(c, g, prm, stream, nullptr, nullptr)) return LWATTN_E_DEVICE;
  if (status) {
    // [0]: the fault word, [1 + b]: batch row b had more than max_global globals
    if (!hip_ok(hipMemcpyAsync(status, w.fault, (B + 1) * 4, hipMemcpyDeviceToDevice, stream), "hipMemcpyAsync"))
      return LWATTN_E_DEVICE;
  }
  return LWATTN_OK;
}

}  // extern "C"
