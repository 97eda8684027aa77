/*
 * lwattn_oracle.c -- CPU oracle for the Longformer window + global attention
 * forward.  TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or helper with the HIP path under long_document_sparse_amd/.
 *
 * It is the plain definition of the method, computed directly in double
 * precision, one query row at a time, over an explicit list of allowed keys:
 *
 *   - "LongFormer: The Long-Document Transformer" notes (coding-zuo.github.io),
 *     section "Sliding Window": every token looks at w/2 tokens on each side.
 *   - same page, section "Dilated Sliding Window": the window has gaps, as in
 *     a dilated convolution; different heads may use different dilations.
 *   - same page, section "Global Attention": pre-selected tokens attend to every
 *     token and every token attends to them; the global scores use their own
 *     projections Qg, Kg, Vg, the window scores use Qs, Ks, Vs.
 *   - FasterTransformer Longformer encoder guide (hnwysp.cn), "compute flow":
 *     a local token's softmax spans its window plus the global tokens, a global
 *     token's softmax spans the whole sequence, and the output row of a padded
 *     query is zeroed; the global token indices are the stable partition of
 *     the global flags (global_idx, global_token_nums).
 *
 * Readings taken where the pages are silent:
 *   window  : keys i + k*s for -w/2 <= k <= w/2, with s = gap + 1 (the dilation
 *             value is the number of skipped positions between taps); keys
 *             outside [0, n) do not exist.
 *   padding : lmask[j] == 0 makes j a padded position: it is never a key, its
 *             output row is exactly zero, and it is never global ("padding
 *             wins" over the global flag).
 *   masks   : a mask value counts as set when it compares != 0.0f.
 *   globals : a local row uses Q.K and V both for its window keys and for the
 *             global keys; a global row uses Qg.Kg and Vg over all valid keys.
 *             A global key inside a local row's window is counted once.
 *   masking : excluded keys are left out of the softmax (no additive bias).
 *   softmax : two passes -- the maximum over the allowed set, then
 *             p_j = exp(x_j - max) / sum_k exp(x_k - max).
 *
 * The causal variant (problem.causal != 0) follows the same notes, section
 * "Implementation": an autoregressive language model uses the dilated sliding
 * window, with window sizes that may differ from layer to layer, and no global
 * attention; and "Longformer模型深度解析与应用指南" (bmjup.com), where a local mask
 * and a causal mask are combined by intersection.  Reading: row i's keys are
 * the window's taps at or before i, i - k*s for 0 <= k <= w/2, that are
 * valid; the global mask is not read.
 *
 * Block-sparse layouts (lwo_rows_blocksparse) follow xFormers' attention-mask
 * notes (gitcode xformers page): a per-head layout over 64 x 64 blocks of the
 * score matrix says which query block sees which key block, and masks compose
 * by intersection (a layout and a causal mask).  Reading: row i of head h sees
 * key j when layout[h][i/64][j/64] is set, j is valid, and (causal) j <= i; a
 * padded row, or a row that sees no key, has output zero.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC (see oracle/__init__.py).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define LWO_PADDED 0
#define LWO_GLOBAL 1
#define LWO_LOCAL 2

typedef struct {
  int32_t B, H, n, d;
  int32_t window;        /* w; reach w/2 on each side */
  const int32_t* gap;    /* [H] dilation gap per head (stride = gap + 1) */
  double scale;          /* multiplies q.k */
  const float *Q, *K, *V, *Qg, *Kg, *Vg; /* [B,H,n,d] */
  const float* lmask;    /* [B,n] */
  const float* gmask;    /* [B,n] */
  int32_t causal;        /* nonzero: the causal variant (window taps at or before i, no globals) */
} lwo_problem;

static int is_valid(const float* lm, int64_t j) { return lm[j] != 0.0f; }
static int is_global(const float* lm, const float* gm, int64_t j) {
  return lm[j] != 0.0f && gm[j] != 0.0f;
}

/* Global-index compaction: for every batch row, the ascending positions of the
 * global tokens (valid and flagged), then -1 up to n; and their count. */
int lwo_compact(const float* lmask, const float* gmask, int32_t B, int32_t n,
                int32_t* gidx, int32_t* gcnt) {
  for (int32_t b = 0; b < B; ++b) {
    const float* lm = lmask + (int64_t)b * n;
    const float* gm = gmask + (int64_t)b * n;
    int32_t* out = gidx + (int64_t)b * n;
    int32_t count = 0;
    for (int32_t j = 0; j < n; ++j)
      if (is_global(lm, gm, j)) out[count++] = j;
    for (int32_t k = count; k < n; ++k) out[k] = -1;
    gcnt[b] = count;
  }
  return 0;
}

/* The allowed key set of query row i of one batch row, ascending within each
 * part (window keys first, then the global keys).  Writes the keys to `keys`
 * (capacity n), the row kind to *kind, and returns the number of keys. */
int64_t lwo_allowed(const float* lm, const float* gm, int32_t n, int32_t window,
                    int32_t gap, int32_t i, int32_t* keys, int32_t* kind) {
  int64_t cnt = 0;
  if (!is_valid(lm, i)) {
    *kind = LWO_PADDED;
    return 0;
  }
  if (is_global(lm, gm, i)) {
    *kind = LWO_GLOBAL;
    for (int32_t j = 0; j < n; ++j)
      if (is_valid(lm, j)) keys[cnt++] = j;
    return cnt;
  }
  *kind = LWO_LOCAL;
  const int64_t s = (int64_t)gap + 1;
  const int64_t r = window / 2;
  /* taps k with 0 <= i + k*s <= n-1, limited to |k| <= r */
  int64_t klo = -((int64_t)i / s);
  int64_t khi = ((int64_t)n - 1 - i) / s;
  if (klo < -r) klo = -r;
  if (khi > r) khi = r;
  for (int64_t k = klo; k <= khi; ++k) {
    int64_t j = (int64_t)i + k * s;
    if (is_valid(lm, j) && !is_global(lm, gm, j)) keys[cnt++] = (int32_t)j;
  }
  for (int32_t j = 0; j < n; ++j)
    if (is_global(lm, gm, j)) keys[cnt++] = j;
  return cnt;
}

/* Causal variant: the valid taps i - k*s, 0 <= k <= w/2, in ascending position
 * order; 0 keys for a padded row (kind LWO_PADDED), else kind LWO_LOCAL. */
int64_t lwo_allowed_causal(const float* lm, int32_t n, int32_t window, int32_t gap, int32_t i,
                           int32_t* keys, int32_t* kind) {
  int64_t cnt = 0;
  (void)n;
  if (!is_valid(lm, i)) {
    *kind = LWO_PADDED;
    return 0;
  }
  *kind = LWO_LOCAL;
  const int64_t s = (int64_t)gap + 1;
  const int64_t r = window / 2;
  int64_t kmax = (int64_t)i / s;   /* taps at position >= 0 */
  if (kmax > r) kmax = r;
  for (int64_t k = kmax; k >= 0; --k) {
    const int64_t j = (int64_t)i - k * s;
    if (is_valid(lm, j)) keys[cnt++] = (int32_t)j;
  }
  return cnt;
}

/* One output row (b, h, i) into out[0..d). keys/p are scratch of size n. */
static void lwo_row(const lwo_problem* p, int32_t b, int32_t h, int32_t i,
                    int32_t* keys, double* prob, double* out) {
  const int32_t n = p->n, d = p->d;
  const float* lm = p->lmask + (int64_t)b * n;
  const float* gm = p->gmask + (int64_t)b * n;
  int32_t kind;
  int64_t cnt = p->causal ? lwo_allowed_causal(lm, n, p->window, p->gap[h], i, keys, &kind)
                          : lwo_allowed(lm, gm, n, p->window, p->gap[h], i, keys, &kind);
  for (int32_t c = 0; c < d; ++c) out[c] = 0.0;
  if (kind == LWO_PADDED) return;

  const int64_t head = ((int64_t)b * p->H + h) * (int64_t)n * d;
  const float* q = (kind == LWO_GLOBAL ? p->Qg : p->Q) + head + (int64_t)i * d;
  const float* kmat = (kind == LWO_GLOBAL ? p->Kg : p->K) + head;
  const float* vmat = (kind == LWO_GLOBAL ? p->Vg : p->V) + head;

  /* scores x_t = scale * <q, k_j> and their maximum */
  double mx = -INFINITY;
  for (int64_t t = 0; t < cnt; ++t) {
    const float* kr = kmat + (int64_t)keys[t] * d;
    double dot = 0.0;
    for (int32_t c = 0; c < d; ++c) dot += (double)q[c] * (double)kr[c];
    prob[t] = p->scale * dot;
    if (prob[t] > mx) mx = prob[t];
  }
  /* softmax over the allowed set */
  double sum = 0.0;
  for (int64_t t = 0; t < cnt; ++t) {
    prob[t] = exp(prob[t] - mx);
    sum += prob[t];
  }
  for (int64_t t = 0; t < cnt; ++t) prob[t] /= sum;
  /* weighted sum of the value rows */
  for (int64_t t = 0; t < cnt; ++t) {
    const float* vr = vmat + (int64_t)keys[t] * d;
    for (int32_t c = 0; c < d; ++c) out[c] += prob[t] * (double)vr[c];
  }
}

/* Selected rows: rows[t] is the flat index (b*H + h)*n + i; out is [nrows, d].
 * Rows are independent, so they are spread over `threads` OpenMP threads. */
int lwo_rows(const lwo_problem* p, const int64_t* rows, int64_t nrows,
             double* out, int32_t threads) {
  const int64_t total = (int64_t)p->B * p->H * p->n;
  for (int64_t t = 0; t < nrows; ++t)
    if (rows[t] < 0 || rows[t] >= total) return 1;
  if (threads < 1) threads = 1;
  int err = 0;
#pragma omp parallel num_threads(threads)
  {
    int32_t* keys = (int32_t*)malloc(sizeof(int32_t) * (size_t)(p->n > 0 ? p->n : 1));
    double* prob = (double*)malloc(sizeof(double) * (size_t)(p->n > 0 ? p->n : 1));
    if (!keys || !prob) {
#pragma omp atomic write
      err = 2;
    } else {
#pragma omp for schedule(dynamic, 64)
      for (int64_t t = 0; t < nrows; ++t) {
        int64_t f = rows[t];
        int32_t i = (int32_t)(f % p->n);
        int64_t bh = f / p->n;
        int32_t h = (int32_t)(bh % p->H);
        int32_t b = (int32_t)(bh / p->H);
        lwo_row(p, b, h, i, keys, prob, out + t * p->d);
      }
    }
    free(keys);
    free(prob);
  }
  return err;
}

/* Every row: out is [B,H,n,d]. */
int lwo_forward(const lwo_problem* p, double* out, int32_t threads) {
  const int64_t total = (int64_t)p->B * p->H * p->n;
  if (threads < 1) threads = 1;
  int err = 0;
#pragma omp parallel num_threads(threads)
  {
    int32_t* keys = (int32_t*)malloc(sizeof(int32_t) * (size_t)(p->n > 0 ? p->n : 1));
    double* prob = (double*)malloc(sizeof(double) * (size_t)(p->n > 0 ? p->n : 1));
    if (!keys || !prob) {
#pragma omp atomic write
      err = 2;
    } else {
#pragma omp for schedule(dynamic, 64)
      for (int64_t f = 0; f < total; ++f) {
        int32_t i = (int32_t)(f % p->n);
        int64_t bh = f / p->n;
        lwo_row(p, (int32_t)(bh / p->H), (int32_t)(bh % p->H), i, keys, prob,
                out + f * p->d);
      }
    }
    free(keys);
    free(prob);
  }
  return err;
}

/* Gradient of the forward with respect to Q, K, V, Qg, Kg, Vg, given dO, the
 * gradient of a scalar loss with respect to the output (all [B,H,n,d]).
 *
 * It is the chain rule through the definition above, row by row.  For a
 * non-padded row i with allowed keys t (the same set lwo_allowed gives the
 * forward), scores x_t = scale <q_i, k_t> and probabilities p_t = softmax(x)_t,
 * the output O_i = sum_t p_t v_t gives, with e_t = <dO_i, v_t> and
 * D = sum_t p_t e_t:
 *   dx_t  = p_t (e_t - D)                  (softmax Jacobian)
 *   dq_i  = scale * sum_t dx_t k_t         (into dQ for a local row, dQg for a global row)
 *   dk_t += scale * dx_t q_i               (into dK, or dKg for a global row)
 *   dv_t += p_t dO_i                       (into dV, or dVg for a global row)
 * A local row's window keys and its global keys both use (q, k, v) = (Q, K, V);
 * a global row uses (Qg, Kg, Vg).  Padded rows contribute nothing, and every
 * entry no row touches stays zero.  (b, h) pairs are independent (one OpenMP
 * task each); within a pair the rows are summed in order. */
int lwo_backward(const lwo_problem* p, const float* dO, double* dQ, double* dK, double* dV,
                 double* dQg, double* dKg, double* dVg, int32_t threads) {
  const int32_t n = p->n, d = p->d;
  const int64_t pairs = (int64_t)p->B * p->H;
  const int64_t per = (int64_t)n * d;
  if (threads < 1) threads = 1;
  int err = 0;
#pragma omp parallel num_threads(threads)
  {
    int32_t* keys = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
    double* prob = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    double* dx = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    if (!keys || !prob || !dx) {
#pragma omp atomic write
      err = 2;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t bh = 0; bh < pairs; ++bh) {
        const int32_t b = (int32_t)(bh / p->H), h = (int32_t)(bh % p->H);
        const int64_t head = bh * per;
        for (int64_t e = 0; e < per; ++e) {
          dQ[head + e] = 0.0; dK[head + e] = 0.0; dV[head + e] = 0.0;
          dQg[head + e] = 0.0; dKg[head + e] = 0.0; dVg[head + e] = 0.0;
        }
        const float* lm = p->lmask + (int64_t)b * n;
        const float* gm = p->gmask + (int64_t)b * n;
        for (int32_t i = 0; i < n; ++i) {
          int32_t kind;
          const int64_t cnt = p->causal ? lwo_allowed_causal(lm, n, p->window, p->gap[h], i, keys, &kind)
                                        : lwo_allowed(lm, gm, n, p->window, p->gap[h], i, keys, &kind);
          if (kind == LWO_PADDED || cnt == 0) continue;
          const int glob = kind == LWO_GLOBAL;
          const float* q = (glob ? p->Qg : p->Q) + head + (int64_t)i * d;
          const float* kmat = (glob ? p->Kg : p->K) + head;
          const float* vmat = (glob ? p->Vg : p->V) + head;
          const float* go = dO + head + (int64_t)i * d;
          double* gq = (glob ? dQg : dQ) + head + (int64_t)i * d;
          double* gk = (glob ? dKg : dK) + head;
          double* gv = (glob ? dVg : dV) + head;
          /* probabilities, as in the forward */
          double mx = -INFINITY;
          for (int64_t t = 0; t < cnt; ++t) {
            const float* kr = kmat + (int64_t)keys[t] * d;
            double dot = 0.0;
            for (int32_t c = 0; c < d; ++c) dot += (double)q[c] * (double)kr[c];
            prob[t] = p->scale * dot;
            if (prob[t] > mx) mx = prob[t];
          }
          double sum = 0.0;
          for (int64_t t = 0; t < cnt; ++t) {
            prob[t] = exp(prob[t] - mx);
            sum += prob[t];
          }
          for (int64_t t = 0; t < cnt; ++t) prob[t] /= sum;
          /* e_t = <dO_i, v_t>, D = sum_t p_t e_t, dx_t = p_t (e_t - D) */
          double D = 0.0;
          for (int64_t t = 0; t < cnt; ++t) {
            const float* vr = vmat + (int64_t)keys[t] * d;
            double e = 0.0;
            for (int32_t c = 0; c < d; ++c) e += (double)go[c] * (double)vr[c];
            dx[t] = e;
            D += prob[t] * e;
          }
          for (int64_t t = 0; t < cnt; ++t) dx[t] = prob[t] * (dx[t] - D);
          for (int64_t t = 0; t < cnt; ++t) {
            const int64_t j = keys[t];
            const float* kr = kmat + j * d;
            for (int32_t c = 0; c < d; ++c) {
              gq[c] += p->scale * dx[t] * (double)kr[c];
              gk[j * d + c] += p->scale * dx[t] * (double)q[c];
              gv[j * d + c] += prob[t] * (double)go[c];
            }
          }
        }
      }
    }
    free(keys);
    free(prob);
    free(dx);
  }
  return err;
}

/* Block-sparse layout: rows[t] is the flat index (b*H + h)*n + i; out is
 * [nrows, d].  layout is uint8 [H][nb][nb], nb = ceil(n / 64). */
int lwo_rows_blocksparse(int32_t B, int32_t H, int32_t n, int32_t d, double scale, const float* Q,
                         const float* K, const float* V, const float* lmask, const uint8_t* layout,
                         int32_t causal, const int64_t* rows, int64_t nrows, double* out,
                         int32_t threads) {
  const int64_t nb = ((int64_t)n + 63) / 64;
  if (threads < 1) threads = 1;
  int err = 0;
#pragma omp parallel num_threads(threads)
  {
    int32_t* keys = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
    double* prob = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    if (!keys || !prob) {
#pragma omp atomic write
      err = 1;
    } else {
#pragma omp for schedule(dynamic, 16)
      for (int64_t t = 0; t < nrows; ++t) {
        const int64_t f = rows[t];
        const int32_t i = (int32_t)(f % n);
        const int64_t bh = f / n;
        const int32_t b = (int32_t)(bh / H), h = (int32_t)(bh % H);
        const float* lm = lmask + (int64_t)b * n;
        double* o = out + t * d;
        for (int32_t c = 0; c < d; ++c) o[c] = 0.0;
        if (!is_valid(lm, i)) continue;
        /* the allowed keys */
        int64_t cnt = 0;
        const uint8_t* lrow = layout + ((int64_t)h * nb + i / 64) * nb;
        for (int32_t j = 0; j < n; ++j)
          if (lrow[j / 64] && is_valid(lm, j) && (!causal || j <= i)) keys[cnt++] = j;
        if (cnt == 0) continue;
        const int64_t head = bh * (int64_t)n * d;
        const float* q = Q + head + (int64_t)i * d;
        double mx = -INFINITY;
        for (int64_t u = 0; u < cnt; ++u) {
          const float* kr = K + head + (int64_t)keys[u] * d;
          double dot = 0.0;
          for (int32_t c = 0; c < d; ++c) dot += (double)q[c] * (double)kr[c];
          prob[u] = scale * dot;
          if (prob[u] > mx) mx = prob[u];
        }
        double sum = 0.0;
        for (int64_t u = 0; u < cnt; ++u) {
          prob[u] = exp(prob[u] - mx);
          sum += prob[u];
        }
        for (int64_t u = 0; u < cnt; ++u) {
          const float* vr = V + head + (int64_t)keys[u] * d;
          const double pu = prob[u] / sum;
          for (int32_t c = 0; c < d; ++c) o[c] += pu * (double)vr[c];
        }
      }
    }
    free(keys);
    free(prob);
  }
  return err;
}
