// lwattn.hip -- host runtime and C ABI of the Longformer window + global
// attention forward (declared in include/lwattn.h).
//
// A plan validates the configuration once, derives the launch geometry and
// owns the device workspace; a forward only enqueues three kernels on the
// caller's stream (see kernels.hpp) and never allocates or synchronizes.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "kernels.hpp"
#include "backward.hpp"
#include "causal.hpp"
#include "blocksparse.hpp"
#include "layer.hpp"

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
  // workspace
  uint8_t* flags = nullptr;
  int32_t* gidx = nullptr;
  int32_t* gcnt = nullptr;
  int32_t* status = nullptr;
  float* part_o = nullptr;
  float* part_ml = nullptr;
  int32_t* tile_cnt = nullptr;
  int32_t* ready = nullptr;   // [B] epoch of the last compaction of each batch row
  int32_t* fault = nullptr;   // sticky: a workgroup gave up waiting for its row
  int32_t epoch = 0;          // forwards launched (kept in 1 .. INT32_MAX - 1)
  bool inject_timeout = false; // fault test: the next forward's waits give up
  int32_t* head_stride = nullptr;
  int32_t* head_blk = nullptr;
  // backward: 64-row blocks per head (all residue classes), per-row statistics
  int32_t* head_blk64 = nullptr;
  int blocks64_per_b = 0;
  float2* stats = nullptr;
  // bf16 backward: the global rows' and global keys' sums over position chunks
  int gsplit = 0, gchunk = 0;
  float* gq = nullptr;
  float* gk = nullptr;
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
  (void)hipFree(p->ready);
  (void)hipFree(p->fault);
  (void)hipFree(p->head_stride);
  (void)hipFree(p->head_blk);
  (void)hipFree(p->head_blk64);
  (void)hipFree(p->stats);
  (void)hipFree(p->gq);
  (void)hipFree(p->gk);
  for (hipEvent_t e : p->events) (void)hipEventDestroy(e);
  for (hipEvent_t e : p->bw_events) (void)hipEventDestroy(e);
  delete p;
}

static int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }


// ---------------------------------------------------------------------------
// Encoder layer around the attention (bf16 storage): the plan gives B, H, n,
// the window, dilation and globals; the layer object owns the intermediate
// buffers and a rocBLAS handle.
struct lwattn_layer_s {
  lwattn_plan_t attn = nullptr;   // not owned
  int32_t inter = 0;
  float eps = 0.f;
  rocblas_handle blas = nullptr;
  float* P = nullptr;                  // [M, max(3 hid, inter)] fp32 GEMM results
  __bf16* qkv[6] = {};                 // Q, K, V, Qg, Kg, Vg [B, H, n, 64]
  __bf16* A = nullptr;                 // attention output [B, H, n, 64]
  __bf16* Am = nullptr;                // [M, hid]
  __bf16* H1 = nullptr;                // [M, hid]
  __bf16* F = nullptr;                 // [M, inter]
};

static void free_layer(lwattn_layer_t L) {
  if (!L) return;
  if (L->attn) (void)hipSetDevice(L->attn->device);
  (void)hipFree(L->P);
  for (auto* q : L->qkv) (void)hipFree(q);
  (void)hipFree(L->A);
  (void)hipFree(L->Am);
  (void)hipFree(L->H1);
  (void)hipFree(L->F);
  if (L->blas) (void)rocblas_destroy_handle(L->blas);
  delete L;
}

// Row-major Y[M, N] (fp32) = X[M, K] W[K, N] (bf16), as the column-major
// product Y^T = W^T X^T.
static bool gemm_rm(rocblas_handle h, int64_t M, int64_t N, int64_t K, const void* X, const void* W, float* Y) {
  const float one = 1.0f, zero = 0.0f;
  const rocblas_status st = rocblas_gemm_ex(h, rocblas_operation_none, rocblas_operation_none, (rocblas_int)N,
                                            (rocblas_int)M, (rocblas_int)K, &one, W, rocblas_datatype_bf16_r,
                                            (rocblas_int)N, X, rocblas_datatype_bf16_r, (rocblas_int)K, &zero, Y,
                                            rocblas_datatype_f32_r, (rocblas_int)N, Y, rocblas_datatype_f32_r,
                                            (rocblas_int)N, rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
  if (st != rocblas_status_success) {
    std::fprintf(stderr, "lwattn: rocblas_gemm_ex failed (%d)\n", (int)st);
    return false;
  }
  return true;
}

template <int PER>
static void launch_ln(const float* G, const void* b, const __bf16* R, const void* g, const void* be, float eps,
                      __bf16* Y, int64_t M, hipStream_t stream) {
  hipLaunchKernelGGL(lwk::layer::bias_residual_layernorm<PER>, dim3((uint32_t)((M + 3) / 4)),
                     dim3(lwk::layer::LNT), 0, stream, G, (const __bf16*)b, R, (const __bf16*)g,
                     (const __bf16*)be, eps, Y, M);
}

static bool layernorm(int H, const float* G, const void* b, const __bf16* R, const void* g, const void* be,
                      float eps, __bf16* Y, int64_t M, hipStream_t stream) {
  switch (H) {
    case 8: launch_ln<8>(G, b, R, g, be, eps, Y, M, stream); return true;
    case 16: launch_ln<16>(G, b, R, g, be, eps, Y, M, stream); return true;
    case 24: launch_ln<24>(G, b, R, g, be, eps, Y, M, stream); return true;
    case 32: launch_ln<32>(G, b, R, g, be, eps, Y, M, stream); return true;
    case 48: launch_ln<48>(G, b, R, g, be, eps, Y, M, stream); return true;
    case 64: launch_ln<64>(G, b, R, g, be, eps, Y, M, stream); return true;
    default: return false;
  }
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
  }
  return "unknown status";
}

lwattn_status lwattn_check_config(const lwattn_config* c) {
  if (!c) return LWATTN_E_INVALID;
  if (c->B < 0 || c->H < 0 || c->n < 0 || c->d <= 0) return LWATTN_E_INVALID;
  if (c->window < 0 || (c->window & 1)) return LWATTN_E_INVALID;
  if (c->max_global < 0) return LWATTN_E_INVALID;
  if (!(c->scale > 0.0f) || !std::isfinite(c->scale)) return LWATTN_E_INVALID;
  if (c->dtype != LWATTN_F32 && c->dtype != LWATTN_BF16) return LWATTN_E_INVALID;
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

  // band geometry: per head, sum over residue classes of ceil(n_rho / 128)
  // (forward) and of ceil(n_rho / 64) (backward)
  std::vector<int32_t> stride(H), blk(H + 1, 0), blk64(H + 1, 0);
  for (int h = 0; h < H; ++h) {
    const int s = p->gap[h] + 1;
    stride[h] = s;
    int64_t nb = 0, nb64 = 0;
    for (int rho = 0; rho < s && rho < n; ++rho) {
      const int64_t nr = ((int64_t)n - rho + s - 1) / s;
      nb += (nr + lwk::ROWS_WG - 1) / lwk::ROWS_WG;
      nb64 += (nr + lwk::bw::T - 1) / lwk::bw::T;
    }
    blk[h + 1] = blk[h] + (int32_t)nb;
    blk64[h + 1] = blk64[h] + (int32_t)nb64;
  }
  p->blocks64_per_b = blk64[H];
  p->blocks_per_b = blk[H];
  p->stride_host = stride;
  p->blk_host = blk;
  bool uni = H > 0;
  for (int h = 1; h < H; ++h) uni = uni && stride[h] == stride[0];
  p->uni_stride = uni ? stride[0] : 0;
  p->blocks_per_head = uni ? blk[1] : 0;
  const int64_t nband = (int64_t)B * blk[H];
  // band workgroups may take the bf16 fast path when every subsequence key
  // they stage has a byte offset that fits in 32 bits
  int smax = 1;
  for (int h = 0; h < H; ++h) smax = std::max(smax, stride[h]);
  p->band_fast = (cfg->dtype == LWATTN_BF16 && (int64_t)n + 128 * (int64_t)smax < ((int64_t)1 << 24)) ? 1 : 0;
  // compaction workgroups lead the grid, padded to a multiple of 8 so that the
  // band workgroups behind them keep their XCD placement
  const int64_t ncomp = ((int64_t)B + 7) / 8 * 8;
  // global-row geometry: the key slices are sized so that the global-row
  // workgroups fill what the compaction and band workgroups leave of the last
  // round of workgroup slots (two per compute unit), with at least 64 of them.
  // When that round is nearly empty (under a quarter used), a full round of
  // global-row workgroups would run behind the band ones with long merges of
  // many slices: a quarter of the slots serves them better (measured at
  // B=1, H=16, n=4096, 64 globals: 47 instead of 105 us; B=4: 114 instead of
  // 134 us)
  int ncu = 256;
  {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, hip_device) == hipSuccess && prop.multiProcessorCount > 0)
      ncu = prop.multiProcessorCount;
  }
  const int64_t slots = 2 * (int64_t)ncu;
  p->nqt = ceil_div(cfg->max_global, 32);
  p->nqg = ceil_div(p->nqt, lwk::NW);
  int64_t nglob = 0;
  if (p->nqt > 0 && n > 0 && B > 0 && H > 0) {
    const int64_t units = (int64_t)B * H * p->nqg;
    const int64_t used = (ncomp + nband) % slots;
    int64_t target = used < slots / 4 ? slots / 4 : slots - used;
    if (target < 64) target = 64;
    int64_t want = (target + units - 1) / units;
    const int64_t maxs = (n + 127) / 128;
    if (want > maxs) want = maxs;
    if (want < 1) want = 1;
    // but no slice longer than 4096 keys, so that no global-row workgroup
    // outlasts the band ones on long sequences
    if (want < (n + 4095) / 4096) want = (n + 4095) / 4096;
    p->ksplit = ceil_div(ceil_div(n, want), 64) * 64;   // whole 64-key steps
    p->nsplit = ceil_div(n, p->ksplit);
    nglob = units * p->nsplit;
  }
  const int64_t nglob_pad = (nglob + 7) / 8 * 8;
  if (ncomp + nband + nglob_pad > INT32_MAX) {
    free_plan(p);
    return LWATTN_E_INVALID;
  }
  p->n_comp_wg = (int)ncomp;
  p->n_band_wg = (int)nband;
  p->n_glob_wg = (int)nglob_pad;
  p->smem = cfg->dtype == LWATTN_BF16 ? lwk::smem_bytes<true>() : lwk::smem_bytes<false>();

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
  const size_t nparts = (size_t)B * H * p->nqt * (p->nsplit > 0 ? p->nsplit : 0) * 32;
  alloc((void**)&p->part_o, nparts * lwk::D * 4);
  alloc((void**)&p->part_ml, nparts * 2 * 4);
  alloc((void**)&p->tile_cnt, (size_t)B * H * (p->nqt > 0 ? p->nqt : 1) * 4);
  alloc((void**)&p->ready, (size_t)B * 4);
  alloc((void**)&p->fault, 4);
  alloc((void**)&p->head_stride, (size_t)H * 4);
  alloc((void**)&p->head_blk, (size_t)(H + 1) * 4);
  alloc((void**)&p->head_blk64, (size_t)(H + 1) * 4);
  alloc((void**)&p->stats, (size_t)B * H * n * sizeof(float2));
  if (cfg->dtype == LWATTN_BF16 && cfg->max_global > 0 && n > 0 && B > 0 && H > 0) {
    // the positions of a head are cut into chunks of whole 64-row tiles, as
    // many as bring the workgroups of the chunk sums (one per batch row, head,
    // 64 global rows and chunk) to about 1024
    const int64_t ntile = ((int64_t)n + lwk::bw::T - 1) / lwk::bw::T;
    const int64_t units = (int64_t)B * H * ceil_div(cfg->max_global, lwk::bw::T);
    const int64_t want = std::max<int64_t>(1, std::min<int64_t>(ntile, (1024 + units - 1) / units));
    const int64_t tiles = (ntile + want - 1) / want;
    p->gchunk = (int)(tiles * lwk::bw::T);
    p->gsplit = (int)((ntile + tiles - 1) / tiles);
    const size_t rows = (size_t)B * H * cfg->max_global * p->gsplit;
    alloc((void**)&p->gq, rows * 68 * 4);
    alloc((void**)&p->gk, rows * 128 * 4);
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
      !hip_ok(hipMemset(p->fault, 0, 4), "hipMemset") ||
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

static bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

lwattn_status lwattn_forward(lwattn_plan_t p, const void* Q, const void* K, const void* V,
                             const void* Qg, const void* Kg, const void* Vg,
                             const float* lmask, const float* gmask, void* O, hipStream_t stream) {
  if (!p) return LWATTN_E_INVALID;
  const lwattn_config& c = p->cfg;
  if ((int64_t)c.B * c.H * c.n == 0) return LWATTN_OK;   // empty problem
  const void* ptrs[] = {Q, K, V, Qg, Kg, Vg, O};
  for (const void* q : ptrs)
    if (!q || !aligned16(q)) return LWATTN_E_INVALID;
  if (!lmask || !gmask || ((uintptr_t)lmask & 3u) || ((uintptr_t)gmask & 3u)) return LWATTN_E_INVALID;
  if (!hip_ok(hipSetDevice(p->device), "hipSetDevice")) return LWATTN_E_DEVICE;

  lwk::Params prm;
  prm.Q = (const uint8_t*)Q;
  prm.K = (const uint8_t*)K;
  prm.V = (const uint8_t*)V;
  prm.Qg = (const uint8_t*)Qg;
  prm.Kg = (const uint8_t*)Kg;
  prm.Vg = (const uint8_t*)Vg;
  prm.O = (uint8_t*)O;
  prm.lmask = lmask;
  prm.gmask = gmask;
  prm.flags = p->flags;
  prm.gidx = p->gidx;
  prm.gcnt = p->gcnt;
  prm.status = p->status;
  prm.part_o = p->part_o;
  prm.part_ml = p->part_ml;
  prm.tile_cnt = p->tile_cnt;
  prm.ready = p->ready;
  prm.fault = p->fault;
  p->epoch = p->epoch >= INT32_MAX - 1 ? 1 : p->epoch + 1;
  prm.epoch = p->epoch;
  prm.publish = p->epoch;
  prm.spin_limit = (1 << 18) + (int32_t)(c.n >> 2);
  if (p->inject_timeout) {
    // the rows are published under another number and nobody waits long:
    // every waiting workgroup gives up, sets the fault word and skips its work
    p->inject_timeout = false;
    prm.publish = -1;
    prm.spin_limit = 64;
  }
  prm.n_comp_wg = p->n_comp_wg;
  prm.head_stride = p->head_stride;
  prm.head_blk = p->head_blk;
  prm.B = c.B;
  prm.H = c.H;
  prm.n = c.n;
  prm.r = (int)std::min<int64_t>(c.window / 2, c.n);
  prm.max_global = c.max_global;
  prm.nqt = p->nqt;
  prm.nqg = p->nqg;
  prm.nsplit = p->nsplit;
  prm.ksplit = p->ksplit;
  prm.n_glob_wg = p->n_glob_wg;
  prm.n_band_wg = p->n_band_wg;
  prm.blocks_per_b = p->blocks_per_b;
  prm.c = c.scale * 1.4426950408889634f;
  prm.mask_vec = ((((uintptr_t)lmask | (uintptr_t)gmask) & 15u) == 0 && (c.n % 4) == 0) ? 1 : 0;
  prm.uni_stride = p->uni_stride;
  prm.blocks_per_head = p->blocks_per_head;
  prm.band_fast = p->band_fast;
  for (int h = 0; h < lwk::MAXH_ARG; ++h) prm.hs[h] = h < c.H ? p->stride_host[h] : 0;
  for (int h = 0; h <= lwk::MAXH_ARG; ++h) prm.hb[h] = h <= c.H ? p->blk_host[h] : 0;

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
  const int grid = p->n_comp_wg + p->n_band_wg + p->n_glob_wg;
  if (c.dtype == LWATTN_BF16)
    hipExtLaunchKernelGGL(lwk::attn_kernel<true>, dim3(grid), dim3(lwk::NT), (uint32_t)p->smem, stream,
                          ev0, ev1, 0u, prm);
  else
    hipExtLaunchKernelGGL(lwk::attn_kernel<false>, dim3(grid), dim3(lwk::NT), (uint32_t)p->smem, stream,
                          ev0, ev1, 0u, prm);
  if (!hip_ok(hipGetLastError(), "hipGetLastError")) return LWATTN_E_DEVICE;

  if (timed) ++p->timing_calls;
  return LWATTN_OK;
}

lwattn_status lwattn_forward_causal(lwattn_plan_t p, const void* Q, const void* K, const void* V,
                                    const float* lmask, void* O, hipStream_t stream) {
  if (!p) return LWATTN_E_INVALID;
  const lwattn_config& c = p->cfg;
  if ((int64_t)c.B * c.H * c.n == 0) return LWATTN_OK;   // empty problem
  if (c.dtype != LWATTN_BF16) return LWATTN_E_UNSUPPORTED;
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
  (void)hipFuncSetAttribute((const void*)lwk::cz::causal_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                            lwk::cz::SMEM);
  hipLaunchKernelGGL(lwk::cz::causal_kernel, dim3((uint32_t)grid), dim3(lwk::bw::NTH), lwk::cz::SMEM, stream, cp);
  if (!hip_ok(hipGetLastError(), "hipGetLastError")) return LWATTN_E_DEVICE;
  return LWATTN_OK;
}

lwattn_status lwattn_backward_causal(lwattn_plan_t p, const void* Q, const void* K, const void* V,
                                     const float* lmask, const void* O, const void* dO, void* dQ, void* dK,
                                     void* dV, hipStream_t stream) {
  if (!p) return LWATTN_E_INVALID;
  const lwattn_config& c = p->cfg;
  if ((int64_t)c.B * c.H * c.n == 0) return LWATTN_OK;   // empty problem
  if (c.dtype != LWATTN_BF16) return LWATTN_E_UNSUPPORTED;
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
  (void)hipFuncSetAttribute((const void*)lwk::cz::causal_dq_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                            lwk::cz::BW_DQ_SMEM);
  (void)hipFuncSetAttribute((const void*)lwk::cz::causal_dkv_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                            lwk::cz::BW_DKV_SMEM);
  // dQ and the rows' statistics first; dK, dV read those statistics
  hipLaunchKernelGGL(lwk::cz::causal_dq_kernel, dim3((uint32_t)grid), dim3(lwk::bw::NTH), lwk::cz::BW_DQ_SMEM,
                     stream, bp);
  hipLaunchKernelGGL(lwk::cz::causal_dkv_kernel, dim3((uint32_t)grid), dim3(lwk::bw::NTH), lwk::cz::BW_DKV_SMEM,
                     stream, bp);
  if (!hip_ok(hipGetLastError(), "hipGetLastError")) return LWATTN_E_DEVICE;
  return LWATTN_OK;
}

lwattn_status lwattn_forward_blocksparse(lwattn_plan_t p, const void* Q, const void* K, const void* V,
                                         const float* lmask, const int32_t* rowptr, const int32_t* cols,
                                         int32_t causal, void* O, hipStream_t stream) {
  if (!p) return LWATTN_E_INVALID;
  const lwattn_config& c = p->cfg;
  if ((int64_t)c.B * c.H * c.n == 0) return LWATTN_OK;   // empty problem
  if (c.dtype != LWATTN_BF16) return LWATTN_E_UNSUPPORTED;
  // tiles are read through 32-bit buffer offsets over a head's n rows; the
  // column list of a query block lives in LDS
  const int64_t nb = ((int64_t)c.n + 63) / 64;
  if ((int64_t)c.n * 128 >= lwk::OOB_OFF || nb > 4096) return LWATTN_E_UNSUPPORTED;
  const void* ptrs[] = {Q, K, V, O};
  for (const void* q : ptrs)
    if (!q || !aligned16(q)) return LWATTN_E_INVALID;
  if (!lmask || ((uintptr_t)lmask & 3u) || !rowptr || ((uintptr_t)rowptr & 3u) || !cols ||
      ((uintptr_t)cols & 3u))
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
  bp.scale = c.scale;
  const int64_t grid = (int64_t)c.B * c.H * nb;
  if (grid > INT32_MAX) return LWATTN_E_UNSUPPORTED;
  const uint32_t smem = (uint32_t)(lwk::bsp::SMEM_BASE + 4 * nb);
  (void)hipFuncSetAttribute((const void*)lwk::bsp::blocksparse_kernel,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  hipLaunchKernelGGL(lwk::bsp::blocksparse_kernel, dim3((uint32_t)grid), dim3(lwk::bw::NTH), smem, stream, bp);
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
  //    next forward's waits still see a new number)
  lwk::Params cp;
  std::memset(&cp, 0, sizeof(cp));
  cp.lmask = lmask;
  cp.gmask = gmask;
  cp.flags = p->flags;
  cp.gidx = p->gidx;
  cp.gcnt = p->gcnt;
  cp.status = p->status;
  cp.ready = p->ready;
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
  hipExtLaunchKernelGGL(lwk::bw::compact_kernel, dim3(c.B), dim3(lwk::NT), (uint32_t)(lwk::NW * 4), stream,
                        ev(0, 0), ev(0, 1), 0u, cp);
  if (!hip_ok(hipGetLastError(), "hipGetLastError")) return LWATTN_E_DEVICE;

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
  if (c.dtype == LWATTN_BF16) {
    // 2. dQ, dQg (zero) and the local rows' statistics; 3. the chunk sums of
    // the global rows and keys; 4. their merge: dQg, the global rows'
    // statistics, the global keys' dK, dV; 5. dK, dV (window), dKg, dVg
    namespace mk = lwk::bw::mk;
    const int64_t nblk = (int64_t)c.B * p->blocks64_per_b;
    const int64_t nchunk = (int64_t)c.B * c.H * bp.ntg * p->gsplit;
    const int64_t nmerge = ((int64_t)c.B * c.H * c.max_global + 3) / 4;
    // tiles are read through 32-bit buffer offsets over a head's n rows
    if (nchunk > INT32_MAX || nmerge > INT32_MAX || (int64_t)c.n * 128 >= lwk::OOB_OFF)
      return LWATTN_E_UNSUPPORTED;
    (void)hipFuncSetAttribute((const void*)mk::dq_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, mk::DQ_SMEM);
    (void)hipFuncSetAttribute((const void*)mk::dkv_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, mk::DKV_SMEM);
    (void)hipFuncSetAttribute((const void*)mk::global_chunk_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                              mk::GS_SMEM);
    hipExtLaunchKernelGGL(mk::dq_kernel, dim3((uint32_t)nblk), dim3(lwk::bw::NTH), mk::DQ_SMEM, stream, ev(1, 0),
                          ev(1, 1), 0u, bp);
    if (nchunk > 0) {
      hipExtLaunchKernelGGL(mk::global_chunk_kernel, dim3((uint32_t)nchunk), dim3(lwk::bw::NTH), mk::GS_SMEM,
                            stream, ev(2, 0), ev(2, 1), 0u, bp);
      hipExtLaunchKernelGGL(mk::global_merge_kernel, dim3((uint32_t)nmerge), dim3(lwk::bw::NTH), 0, stream,
                            ev(3, 0), ev(3, 1), 0u, bp);
    }
    hipExtLaunchKernelGGL(mk::dkv_kernel, dim3((uint32_t)nblk), dim3(lwk::bw::NTH), mk::DKV_SMEM, stream,
                          ev(4, 0), ev(4, 1), 0u, bp);
  } else {
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
  if (c.dtype != LWATTN_BF16 || !(H == 8 || H == 16 || H == 24 || H == 32 || H == 48 || H == 64))
    return LWATTN_E_UNSUPPORTED;
  const int64_t M = (int64_t)c.B * c.n, hid = (int64_t)H * 64;
  if (M * std::max<int64_t>(3 * hid, inter) >= ((int64_t)1 << 31)) return LWATTN_E_UNSUPPORTED;
  if (!hip_ok(hipSetDevice(p->device), "hipSetDevice")) return LWATTN_E_DEVICE;
  lwattn_layer_t L = new (std::nothrow) lwattn_layer_s;
  if (!L) return LWATTN_E_NOMEM;
  L->attn = p;
  L->inter = inter;
  L->eps = eps;
  bool ok = true;
  auto alloc = [&](void** ptr, size_t bytes) {
    if (!ok) return;
    if (bytes == 0) bytes = 16;
    if (!hip_ok(hipMalloc(ptr, bytes), "hipMalloc")) { ok = false; *ptr = nullptr; }
  };
  alloc((void**)&L->P, (size_t)M * std::max<int64_t>(3 * hid, inter) * 4);
  for (auto*& q : L->qkv) alloc((void**)&q, (size_t)M * hid * 2);
  alloc((void**)&L->A, (size_t)M * hid * 2);
  alloc((void**)&L->Am, (size_t)M * hid * 2);
  alloc((void**)&L->H1, (size_t)M * hid * 2);
  alloc((void**)&L->F, (size_t)M * inter * 2);
  if (ok && rocblas_create_handle(&L->blas) != rocblas_status_success) ok = false;
  if (!ok) {
    free_layer(L);
    return LWATTN_E_NOMEM;
  }
  *out = L;
  return LWATTN_OK;
}

lwattn_status lwattn_layer_forward(lwattn_layer_t L, const void* X, const lwattn_layer_weights* w,
                                   const float* lmask, const float* gmask, void* Y, hipStream_t stream) {
  if (!L || !w) return LWATTN_E_INVALID;
  lwattn_plan_t p = L->attn;
  const lwattn_config& c = p->cfg;
  const int H = c.H;
  const int64_t M = (int64_t)c.B * c.n, hid = (int64_t)H * 64, inter = L->inter;
  if (M == 0) return LWATTN_OK;
  const void* ptrs[] = {X, Y, w->w_qkv, w->b_qkv, w->w_g, w->b_g, w->w_o, w->b_o, w->ln1_g, w->ln1_b,
                        w->w_1, w->b_1, w->w_2, w->b_2, w->ln2_g, w->ln2_b};
  for (const void* q : ptrs)
    if (!q || !aligned16(q)) return LWATTN_E_INVALID;
  if (!lmask || !gmask || ((uintptr_t)lmask & 3u) || ((uintptr_t)gmask & 3u)) return LWATTN_E_INVALID;
  if (!hip_ok(hipSetDevice(p->device), "hipSetDevice")) return LWATTN_E_DEVICE;
  if (rocblas_set_stream(L->blas, stream) != rocblas_status_success) return LWATTN_E_DEVICE;
  namespace ly = lwk::layer;
  auto blocks = [](int64_t threads) { return dim3((uint32_t)((threads + ly::LNT - 1) / ly::LNT)); };
  // 1. projections: Q, K, V then Qg, Kg, Vg, bias added while splitting heads
  if (!gemm_rm(L->blas, M, 3 * hid, hid, X, w->w_qkv, L->P)) return LWATTN_E_DEVICE;
  hipLaunchKernelGGL(ly::split_heads, blocks(M * 3 * hid / 8), dim3(ly::LNT), 0, stream, L->P,
                     (const __bf16*)w->b_qkv, L->qkv[0], L->qkv[1], L->qkv[2], c.B, c.n, H);
  if (!gemm_rm(L->blas, M, 3 * hid, hid, X, w->w_g, L->P)) return LWATTN_E_DEVICE;
  hipLaunchKernelGGL(ly::split_heads, blocks(M * 3 * hid / 8), dim3(ly::LNT), 0, stream, L->P,
                     (const __bf16*)w->b_g, L->qkv[3], L->qkv[4], L->qkv[5], c.B, c.n, H);
  if (!hip_ok(hipGetLastError(), "hipGetLastError")) return LWATTN_E_DEVICE;
  // 2. the attention
  lwattn_status st = lwattn_forward(p, L->qkv[0], L->qkv[1], L->qkv[2], L->qkv[3], L->qkv[4], L->qkv[5],
                                    lmask, gmask, L->A, stream);
  if (st != LWATTN_OK) return st;
  // 3. output projection, bias, residual, LayerNorm
  hipLaunchKernelGGL(ly::merge_heads, blocks(M * hid / 8), dim3(ly::LNT), 0, stream, L->A, L->Am, c.B, c.n, H);
  if (!gemm_rm(L->blas, M, hid, hid, L->Am, w->w_o, L->P)) return LWATTN_E_DEVICE;
  if (!layernorm(H, L->P, w->b_o, (const __bf16*)X, w->ln1_g, w->ln1_b, L->eps, L->H1, M, stream))
    return LWATTN_E_UNSUPPORTED;
  // 4. FFN: intermediate GEMM, bias, GELU; output GEMM, bias, residual, LayerNorm
  if (!gemm_rm(L->blas, M, inter, hid, L->H1, w->w_1, L->P)) return LWATTN_E_DEVICE;
  hipLaunchKernelGGL(ly::bias_gelu, blocks(M * inter / 8), dim3(ly::LNT), 0, stream, L->P,
                     (const __bf16*)w->b_1, L->F, M, (int)inter);
  if (!gemm_rm(L->blas, M, hid, inter, L->F, w->w_2, L->P)) return LWATTN_E_DEVICE;
  if (!layernorm(H, L->P, w->b_2, L->H1, w->ln2_g, w->ln2_b, L->eps, (__bf16*)Y, M, stream))
    return LWATTN_E_UNSUPPORTED;
  if (!hip_ok(hipGetLastError(), "hipGetLastError")) return LWATTN_E_DEVICE;
  return LWATTN_OK;
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

}  // extern "C"
