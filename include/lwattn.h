/*
 * lwattn.h -- Longformer self-attention forward (sliding window, per-head
 * dilation, task-driven global attention) on AMD Instinct MI355X (gfx950).
 *
 * What one forward computes, per batch row b, head h and query position i
 * (the pages' definition; the readings of what they leave open are spelled
 * out on each argument):
 *
 *   valid(j)  = local_attn_mask[b][j] != 0          (0.0 marks padding)
 *   global(j) = valid(j) && global_attn_mask[b][j] != 0
 *
 *   padded row  (!valid(i)) : O[b,h,i,:] = 0 exactly.
 *   global row  (global(i)) : softmax over every valid key j of
 *                             scale * <Qg_i, Kg_j>, weights applied to Vg_j.
 *   local row   (otherwise) : softmax over the window keys
 *                             { i + k*(dilation[h]+1) : |k| <= window/2,
 *                               0 <= key < n, valid, not global }
 *                             together with every global key (each key once)
 *                             of scale * <Q_i, K_j>, weights applied to V_j.
 *
 * Sources:
 *   "LongFormer: The Long-Document Transformer" notes (coding-zuo.github.io),
 *   sections "Sliding Window" (w/2 keys each side), "Dilated Sliding Window"
 *   (gapped taps, per-head dilation) and "Global Attention" (symmetric global
 *   tokens, separate Qg/Kg/Vg projections, banded Q.K^T).
 *   FasterTransformer Longformer encoder guide (hnwysp.cn): inputs
 *   local_attn_mask / global_attn_mask [batch, seq] with 1.0 = attends, the
 *   [batch, head, seq, dim] multi-head layout, head dim 64, the global-index
 *   partition (global_idx, global_token_nums), the masked softmax (local rows
 *   over window + globals, global rows over the whole sequence, padded query
 *   rows zeroed) and the float / half / bf16 instantiations.
 *
 * Conventions for every function: plain C, never throws, never aborts; every
 * failure is a status code.  Device pointers are HIP device allocations on the
 * plan's device.  The caller owns every tensor; a plan owns its workspace.
 */
#ifndef LWATTN_H_
#define LWATTN_H_

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct lwattn_plan_s* lwattn_plan_t;

/* Storage type of Q, K, V, Qg, Kg, Vg and O (FasterTransformer Longformer
 * encoder guide, implementation scope: the float, half and bfloat16
 * instantiations).  Scores, softmax and the output accumulation are always
 * float32; with 16-bit storage the matrix cores take the probabilities rounded
 * to the storage type.  LWATTN_F16 (IEEE half) runs the forwards
 * (lwattn_forward, lwattn_forward_noalloc, lwattn_forward_causal,
 * lwattn_forward_blocksparse), the backwards and the encoder layer. */
typedef enum { LWATTN_F32 = 0, LWATTN_BF16 = 1, LWATTN_F16 = 2 } lwattn_dtype;

typedef enum {
  LWATTN_OK = 0,
  LWATTN_E_INVALID = 1,           /* bad argument: null/misaligned pointer, bad config */
  LWATTN_E_UNSUPPORTED = 2,       /* valid but not implemented (d != 64) */
  LWATTN_E_NOMEM = 3,             /* workspace allocation failed */
  LWATTN_E_DEVICE = 4,            /* a HIP call failed */
  LWATTN_E_TOO_MANY_GLOBALS = 5,  /* a batch row had more than max_global global tokens */
  LWATTN_E_SCRATCH = 6            /* lwattn_forward_noalloc: the problem needs more workspace
                                     than its static buffer holds */
} lwattn_status;

typedef struct {
  int32_t B, H, n, d;     /* batch, heads, sequence length, head dim.  d must be 64
                             (the FasterTransformer guide states the same limit).
                             B, H or n equal to 0 is an empty problem: the forward
                             launches nothing and returns LWATTN_OK. */
  int32_t window;         /* w >= 0 and even: w/2 taps on each side of the query
                             ("Sliding Window").  w = 0 keeps the query itself. */
  const int32_t* dilation;/* host array [H] (copied by lwattn_plan): gap per head,
                             >= 0; taps are dilation+1 positions apart ("Dilated
                             Sliding Window").  NULL means 0 for every head. */
  int32_t max_global;     /* bound on global tokens per batch row (the guide's
                             max_global_token_num).  Sizes the workspace; more
                             global tokens in a row is reported by
                             lwattn_sync_status as LWATTN_E_TOO_MANY_GLOBALS. */
  float scale;            /* > 0, finite: multiplies every q.k (the guide's
                             attn_scaler); 1/sqrt(d) for the usual attention. */
  int32_t dtype;          /* lwattn_dtype */
} lwattn_config;

/* Validates a configuration without touching any device.  Returns LWATTN_OK,
 * LWATTN_E_INVALID (null cfg, negative sizes, odd or negative window, negative
 * dilation, max_global < 0, scale not > 0 and finite, unknown dtype, or
 * B*H*n*d beyond 2^40 elements, B*n beyond 2^31-1, n beyond 2^23) or
 * LWATTN_E_UNSUPPORTED (d != 64). */
lwattn_status lwattn_check_config(const lwattn_config* cfg);

/* Validates cfg, selects HIP device `hip_device`, allocates the plan and its
 * device workspace (flags and index lists of size B*n, per-row status, and the
 * split-softmax partials of the global rows, about
 * B*H*ceil(max_global/32)*nsplit*32*66*4 bytes).  On success *out owns them;
 * release with lwattn_destroy.  On failure *out is NULL. */
lwattn_status lwattn_plan(const lwattn_config* cfg, int hip_device, lwattn_plan_t* out);

/* Enqueues one forward on `stream` (asynchronous; no allocation, no host sync).
 *   Q, K, V, Qg, Kg, Vg : device, [B,H,n,d] contiguous, dtype; 16-byte aligned.
 *                         Only Qg rows at global positions and Q rows at local
 *                         positions are read.
 *   local_attn_mask     : device float32 [B,n]; != 0 marks a real token.
 *   global_attn_mask    : device float32 [B,n]; != 0 marks a global token.
 *   O                   : device, [B,H,n,d], dtype, 16-byte aligned; every row
 *                         is written.  Must not overlap any input.
 * Returns LWATTN_E_INVALID before launching anything if the plan or a pointer
 * is null or misaligned, LWATTN_E_DEVICE if a launch fails.  Data-dependent
 * errors (too many global tokens) are reported by lwattn_sync_status; O is
 * then undefined.  One plan serves one stream at a time: its workspace
 * (flags, global-index lists, per-row readiness words, merge counters) is
 * shared by all its forwards, so forwards of one plan that overlap on two
 * streams race.  The forward is a single kernel launch. */
lwattn_status lwattn_forward(lwattn_plan_t plan,
                             const void* Q, const void* K, const void* V,
                             const void* Qg, const void* Kg, const void* Vg,
                             const float* local_attn_mask, const float* global_attn_mask,
                             void* O, hipStream_t stream);

/* Causal variant of the window attention ("LongFormer: The Long-Document
 * Transformer" notes, section Implementation: an autoregressive language model
 * uses the dilated sliding window, its size chosen per layer, with no global
 * attention; "Longformer模型深度解析与应用指南": a local mask intersected with a causal
 * mask).  Row i of head h (stride s = dilation[h] + 1, reach r = window / 2 of
 * the plan) attends to the taps i - k*s, 0 <= k <= r, whose lmask is nonzero;
 * softmax of scale <Q_i, K_j> over them, O_i = sum_j p_j V_j; a row with
 * lmask 0 gets O_i = 0.  The plan's max_global and any global mask play no
 * part.  Per-layer window sizes: one plan per window size.
 * Q, K, V, O: [B][H][n][64] in the plan's 16-bit storage type (bf16 or fp16),
 * 16-byte aligned, device memory; lmask float32 [B][n], 4-byte aligned.  Every
 * element of O is written.  Enqueued on
 * `stream` (one kernel launch, no allocation, no host sync); it uses no plan
 * workspace, so it may overlap other calls of the same plan.
 * Errors: LWATTN_E_INVALID for a null plan or pointer or a misaligned one;
 * LWATTN_E_UNSUPPORTED for fp32 storage or n * 128 >= 2^31 - 256;
 * LWATTN_E_DEVICE if the launch fails. */
lwattn_status lwattn_forward_causal(lwattn_plan_t plan, const void* Q, const void* K, const void* V,
                                    const float* lmask, void* O, hipStream_t stream);

/* Backward of lwattn_forward_causal: the chain rule through its softmax,
 * the same derivation as lwattn_backward over the causal tap sets (dS_ij =
 * P_ij (dP_ij - D_i) with dP_ij = <dO_i, V_j> and D_i = <dO_i, O_i>;
 * dQ_i = scale sum_j dS_ij K_j, dK_j = scale sum_i dS_ij Q_i,
 * dV_j = sum_i P_ij dO_i).  O is the output of lwattn_forward_causal on the
 * same inputs.  Q, K, V, O, dO, dQ, dK, dV: [B][H][n][64] in the plan's 16-bit
 * storage type (bf16 or fp16), 16-byte aligned, device memory; lmask float32
 * [B][n].  Every element of dQ, dK, dV
 * is written (zero at rows and keys whose lmask is 0).  Enqueued on `stream`
 * (two kernel launches, no allocation, no host sync); it uses the plan's
 * per-row statistics buffer, so it must not overlap a backward of the same
 * plan.  Errors as lwattn_forward_causal. */
lwattn_status lwattn_backward_causal(lwattn_plan_t plan, const void* Q, const void* K, const void* V,
                                     const float* lmask, const void* O, const void* dO,
                                     void* dQ, void* dK, void* dV, hipStream_t stream);

/* Block-sparse attention over 64 x 64 blocks (xFormers' attention-mask notes:
 * a per-head layout over 64 x 64 blocks of the score matrix with block size
 * 64, and masks that compose by intersection, as a layout with a causal mask).
 * Row i of head h attends to key j when the layout holds block (i / 64,
 * j / 64) for h, lmask[b][j] != 0 and, if `causal` is nonzero, j <= i;
 * softmax of scale <Q_i, K_j> over those keys, O_i = sum_j p_j V_j.  A row with
 * lmask 0, or one that sees no key, gets O_i = 0.  The plan gives B, H, n,
 * scale and the storage type; its window, dilation and max_global play no part.
 * Layout, CSR over (head, query block), device memory, int32, 4-byte aligned:
 * the key blocks of query block qb of head h are cols[rowptr[h*nb + qb] ..
 * rowptr[h*nb + qb + 1]) with nb = ceil(n / 64); rowptr has H*nb + 1 entries
 * and cols holds nnz >= 0 entries.  Each listed key block is visited once per
 * listing (list a block once); a block index outside [0, nb) contributes no
 * key; a list longer than nb is cut to its first nb entries; offsets are
 * clamped into [0, nnz], so a malformed rowptr (negative, decreasing or past
 * nnz) never reads outside cols (its lists come out empty or cut).  Q, K, V, O: [B][H][n][64] in the
 * plan's 16-bit storage type (bf16 or fp16), 16-byte aligned;
 * lmask float32 [B][n].  Every element of O is written.  One kernel launch on
 * `stream`, no allocation, no host sync, no plan workspace.
 * Errors: LWATTN_E_INVALID for a null plan or pointer, a misaligned one or
 * nnz < 0; LWATTN_E_UNSUPPORTED for fp32 storage, n * 128 >= 2^31 - 256 or
 * nb > 4096; LWATTN_E_DEVICE if the launch fails. */
lwattn_status lwattn_forward_blocksparse(lwattn_plan_t plan, const void* Q, const void* K,
                                         const void* V, const float* lmask, const int32_t* rowptr,
                                         const int32_t* cols, int32_t nnz, int32_t causal, void* O,
                                         hipStream_t stream);

/* Encoder layer around the attention (FasterTransformer Longformer encoder
 * guide, compute flow; the plan's 16-bit storage, bf16 or fp16, with fp32
 * accumulation).  With M = B*n rows of hid = H*64 columns, X [M][hid] the
 * layer input:
 *   [Q | K | V]    = X w_qkv + b_qkv      (w_qkv [hid][3 hid], b_qkv [3 hid])
 *   [Qg | Kg | Vg] = X w_g + b_g          (same shapes); column h*64 + j of a
 *                    part is head h, element j; Qg is formed for the global
 *                    tokens' rows only (gathered, projected, scattered back),
 *                    the only rows the attention reads of it
 *   A  = the attention of the plan (as lwattn_forward) on those six tensors and
 *        the masks, heads merged back to [M][hid]
 *   H1 = LayerNorm(A w_o + b_o + X) * ln1_g + ln1_b
 *   F  = gelu(H1 w_1 + b_1), gelu(x) = x (1 + erf(x / sqrt 2)) / 2 (erf by
 *        Abramowitz-Stegun 7.1.26: absolute error of gelu below 2.2e-7)
 *   Y  = LayerNorm(F w_2 + b_2 + H1) * ln2_g + ln2_b
 * LayerNorm over each row: (x - mean) / sqrt(biased variance + eps).  All
 * weights row-major [in][out] in the storage type, 16-byte aligned device
 * memory; X and Y [M][hid] in the storage type.  The GEMMs run in hipBLASLt
 * (rocBLAS for a shape it has no algorithm for), adding the bias in their
 * epilogue where it has one; each GEMM result and every other intermediate
 * is rounded to the storage type once.  The attention reads Q, K, V, Kg, Vg
 * where the GEMMs left them and writes its rows already merged.
 * lwattn_layer_create(plan, inter, eps, &layer): plan with 16-bit storage and
 * H a multiple of 4 up to 64, inter a positive multiple of 8, eps > 0; the
 * layer keeps the plan (which must outlive it) and allocates its
 * intermediates, its GEMM handles and an internal stream.
 * lwattn_layer_forward enqueues the layer on `stream` (no allocation, no host
 * sync): the global rows' Qg chain runs on the layer's internal stream,
 * forked from `stream` at the start and joined back into it before the
 * attention, so the call stays ordered with the other work on `stream`.  It
 * uses the plan's workspace, so it must not overlap other calls of the plan or
 * of the same layer.
 * Errors: LWATTN_E_INVALID for null or misaligned arguments or a bad inter /
 * eps; LWATTN_E_UNSUPPORTED for fp32 storage, another H, or M * 3 hid or
 * M * inter >= 2^31; LWATTN_E_NOMEM; LWATTN_E_DEVICE if a launch or GEMM fails;
 * the attention's own errors as lwattn_forward reports them. */
typedef struct lwattn_layer_s* lwattn_layer_t;
typedef struct {
  const void *w_qkv, *b_qkv;   /* [hid][3 hid], [3 hid]: Q, K, V */
  const void *w_g, *b_g;       /* [hid][3 hid], [3 hid]: Qg, Kg, Vg */
  const void *w_o, *b_o;       /* [hid][hid], [hid] */
  const void *ln1_g, *ln1_b;   /* [hid] */
  const void *w_1, *b_1;       /* [hid][inter], [inter] */
  const void *w_2, *b_2;       /* [inter][hid], [hid] */
  const void *ln2_g, *ln2_b;   /* [hid] */
} lwattn_layer_weights;
lwattn_status lwattn_layer_create(lwattn_plan_t plan, int32_t inter, float eps, lwattn_layer_t* out);
lwattn_status lwattn_layer_forward(lwattn_layer_t layer, const void* X, const lwattn_layer_weights* w,
                                   const float* lmask, const float* gmask, void* Y, hipStream_t stream);
lwattn_status lwattn_layer_destroy(lwattn_layer_t layer);

/* Enqueues the backward of one forward on `stream` (asynchronous; no
 * allocation, no host sync): the gradients of a loss with respect to Q, K, V,
 * Qg, Kg, Vg, given dO = dLoss/dO.  It differentiates the operation that
 * lwattn_forward computes (LongFormer notes, sections "Sliding Window",
 * "Dilated Sliding Window" and "Global Attention"): with P the softmax of a
 * row over its allowed keys, dP_ij = <dO_i, v_j> and D_i = <dO_i, O_i>,
 *   dS_ij = P_ij (dP_ij - D_i),  dq_i = scale sum_j dS_ij k_j,
 *   dk_j = scale sum_i dS_ij q_i,  dv_j = sum_i P_ij dO_i,
 * over (Q, K, V) for a local row's window and global keys and (Qg, Kg, Vg) for
 * a global row.
 *   Q .. Vg, masks      : the forward's inputs (same layouts and rules).
 *   O                   : device [B,H,n,d], dtype: the forward's output for them.
 *   dO                  : device [B,H,n,d], dtype; rows of padded positions are
 *                         not read.
 *   dQ, dK, dV, dQg, dKg, dVg : device [B,H,n,d], dtype; every element is
 *                         written (zero where no path reaches it).  They must
 *                         not overlap each other or any input.
 * All pointers 16-byte aligned.  Arithmetic in fp32 (16-bit storage is widened
 * on load and rounded RNE on store).  16-bit storage (bf16 or fp16, on the
 * matrix cores): the global-index compaction
 * (inside the dQ launch, by its first B workgroups, when that grid fits one
 * round of workgroup slots), dQ (which leaves each row's log-sum-exp and D in
 * the plan's workspace), the chunk sums of the global rows and keys and their
 * merge (when max_global > 0; the merge inside the dK/dV launch when its last
 * round has spare slots for it), dK/dV/dKg/dVg.  fp32: three launches, the
 * compaction, dQ/dQg, then dK/dV/dKg/dVg.  Errors as for lwattn_forward; too many
 * global tokens is reported by lwattn_sync_status.  Shares the plan's
 * workspace with lwattn_forward: a forward and a backward of one plan must
 * not overlap (same stream, or ordered). */
lwattn_status lwattn_backward(lwattn_plan_t plan,
                              const void* Q, const void* K, const void* V,
                              const void* Qg, const void* Kg, const void* Vg,
                              const float* local_attn_mask, const float* global_attn_mask,
                              const void* O, const void* dO,
                              void* dQ, void* dK, void* dV, void* dQg, void* dKg, void* dVg,
                              hipStream_t stream);

/* Frees the plan and its workspace.  NULL is a no-op. */
lwattn_status lwattn_destroy(lwattn_plan_t plan);

/* Copies the global-index lists of the last forward on `stream` (stream-ordered,
 * asynchronous) into caller-owned device buffers:
 *   gidx [B,n] int32: ascending global positions of row b, then -1 to the end;
 *   gcnt [B]   int32: the number of global tokens of row b.
 * (The FasterTransformer guide's global_idx / global_token_nums.)  Returns
 * LWATTN_E_INVALID for a null plan or pointer, LWATTN_E_DEVICE if the copy
 * cannot be enqueued. */
lwattn_status lwattn_global_index(lwattn_plan_t plan, int32_t* gidx, int32_t* gcnt,
                                  hipStream_t stream);

/* Synchronizes `stream`, then reports the device-side status of the last
 * forward: LWATTN_E_TOO_MANY_GLOBALS if any row exceeded max_global, else
 * LWATTN_OK.  LWATTN_E_DEVICE if a HIP call failed, or if in any forward
 * since lwattn_plan a workgroup timed out waiting for the compaction of its
 * batch row (its output rows were then not written); that state is sticky
 * and the plan should be destroyed. */
lwattn_status lwattn_sync_status(lwattn_plan_t plan, hipStream_t stream);

/* Kernel timing for measurement.  While enabled, every forward's kernel is
 * launched with a pair of HIP events that its dispatch records at the start
 * and the end of the kernel's execution (hipExtLaunchKernel; up to
 * `max_calls` forwards are kept).  lwattn_timing_read synchronizes on the recorded events
 * and returns, per kernel of the forward, the summed duration in milliseconds
 * (ms[k] for k < *nkernels, at most `cap`) and the number of recorded forwards.
 * A forward is one kernel (*nkernels = 1): the global-index compaction, the
 * local rows and the global rows including the merge of their key slices. */
lwattn_status lwattn_timing_enable(lwattn_plan_t plan, int32_t max_calls);
/* Record the events of every `every`-th forward only (every >= 1; 1 after
 * lwattn_plan), so that recording adds little host work to a timed loop of
 * back-to-back forwards.  Counting restarts at lwattn_timing_enable.
 * LWATTN_E_INVALID for a null plan or every < 1. */
lwattn_status lwattn_timing_every(lwattn_plan_t plan, int32_t every);
lwattn_status lwattn_timing_read(lwattn_plan_t plan, float* ms, int32_t cap,
                                 int32_t* nkernels, int32_t* ncalls);
/* The same for backwards (recorded while timing is enabled, every `every`-th
 * backward, up to `max_calls`): per kernel slot, the summed duration in
 * milliseconds over the recorded backwards.  Slots (*nkernels = 5): the
 * global-index compaction, dQ, the chunk sums of the global rows and keys, their
 * merge, dK/dV; a slot whose kernel a backward did not launch counts zero
 * (fp32 launches slots 0, 1 and 4; 16-bit storage skips slot 0 when the compaction runs
 * inside dQ, slot 3 when the merge runs inside dK/dV, slots 2 and 3 without
 * global tokens). */
lwattn_status lwattn_timing_read_backward(lwattn_plan_t plan, float* ms, int32_t cap,
                                          int32_t* nkernels, int32_t* ncalls);
lwattn_status lwattn_timing_disable(lwattn_plan_t plan);

/* Testing aid for the failure path of the in-kernel wait (for test code only).
 * In the next forward of `plan` (or 16-bit backward, whichever comes first), the
 * row compactions publish a number the other workgroups do not wait for, and
 * their waits give up after 64 polls: every workgroup still exits normally,
 * the outputs are undefined, and lwattn_sync_status reports LWATTN_E_DEVICE
 * from then on (the plan is then to be destroyed).  A backward whose
 * compaction is a launch of its own has no such wait and is unaffected.
 * LWATTN_E_INVALID for a null plan. */
lwattn_status lwattn_test_inject_wait_timeout(lwattn_plan_t plan);

/* Allocation-free forward, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  It computes exactly what lwattn_forward computes for a plan
 * made from *cfg (same kernel, same launch geometry), without a plan: the
 * workspace is a static device buffer of 32 MiB per GPU, held from the first
 * call on that GPU until the process ends, and the call makes no hipMalloc,
 * hipFree or other allocating call, on the device or the host.
 * cfg: as for lwattn_plan, with H <= 32 (the head tables travel in the kernel
 * arguments).  hip_device: the GPU the tensors live on (< 64); it becomes the
 * current device.  Q .. O, lmask, gmask: as lwattn_forward.  status: NULL, or
 * device int32 [B + 1], written on `stream` after the forward: [0] nonzero if
 * a workgroup gave up waiting for its row's global index (O undefined), [1 + b]
 * = 1 if batch row b had more than max_global global tokens (its O undefined),
 * else 0.  Asynchronous on `stream`, no host sync.  Every call on one GPU
 * shares that GPU's buffer (the words that must start at zero are cleared by
 * a kernel at the start of each call): calls that may overlap on one GPU, on
 * different streams or from different threads, race and must be serialised
 * by the caller.  The workspace needed is about B n 5 bytes plus, for the
 * global rows, B H ceil(max_global / 32) nsplit 8448 bytes (nsplit <= 32
 * key slices); a problem that needs more than the buffer returns
 * LWATTN_E_SCRATCH before anything is launched.
 * Errors: as lwattn_check_config; LWATTN_E_INVALID for a null or misaligned
 * pointer or a bad hip_device; LWATTN_E_UNSUPPORTED for H > 32;
 * LWATTN_E_SCRATCH; LWATTN_E_DEVICE if a HIP call fails. */
lwattn_status lwattn_forward_noalloc(const lwattn_config* cfg, int hip_device, const void* Q, const void* K,
                                     const void* V, const void* Qg, const void* Kg, const void* Vg,
                                     const float* lmask, const float* gmask, void* O, int32_t* status,
                                     hipStream_t stream);

/* Measurement aids (bench and tests only): what the chip delivers, so that
 * roofline fractions can be stated against measured peaks as well as the
 * published ones.  Each enqueues one kernel on `stream` and returns at once.
 * lwattn_probe_mfma: 512 workgroups of 4 waves; every wave runs `iters`
 *   rounds of 8 independent v_mfma_f32_32x32x16_bf16 (32768 flops each), so a
 *   launch performs 512 * 4 * iters * 8 * 32768 flops; out: device float
 *   [2048], one value per wave (written so that nothing is optimised away).
 * lwattn_probe_read: reads `bytes` (rounded down to 16) of device memory at
 *   `buf` (16-byte aligned) once, 16-byte loads in a grid-stride stream;
 *   out: device float [4096], one value per workgroup.
 * Errors: LWATTN_E_INVALID for null or misaligned pointers or negative
 * sizes; LWATTN_E_DEVICE if the launch fails. */
lwattn_status lwattn_probe_mfma(int32_t iters, float* out, hipStream_t stream);
lwattn_status lwattn_probe_read(const void* buf, int64_t bytes, float* out, hipStream_t stream);

/* Static description of a status code. */
const char* lwattn_strerror(lwattn_status s);

#ifdef __cplusplus
}
#endif
#endif /* LWATTN_H_ */
