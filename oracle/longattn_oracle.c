/*
 * fp64 CPU oracle for the forward pass of banded sparse self-attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the plain, slow, obviously correct definition that the
 * GPU library is checked against.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg load it.  It shares no code, header, table or helper with the HIP library,
 * and the HIP library never calls it.
 *
 * What it computes.  Attention restricted to a sparse key set is exact masked softmax
 * attention; nothing is approximated.  The pages describe the pattern as a directed graph
 * whose edges are the allowed (query, key) pairs (Big Bird reading notes, section 3.1), built
 * as the union of a local window, global tokens and random keys (same notes, section 3.3).
 * For batch b, head h and query row i:
 *
 *   1. Allowed set A.
 *      - If i is a global token of sample b, A = every position: a global token attends the
 *        whole sequence (Longformer hub page, section 2; Big Bird notes, section 3.2.3).
 *      - Otherwise A is the union of
 *          Band(i)  = { i + dil[h]*t : t in [-win_left, win_right] }, cut to [0, n)
 *                     (window around the query, Big Bird notes section 3.2.1; the window
 *                     skips tokens like a dilated convolution when dil > 1, Longformer hub
 *                     page section 2),
 *          G_b      = the global tokens, which every position attends,
 *          Layout   = every key of the blocks listed for (h, block of i) in the block
 *                     layout (random and sliding blocks, Big Bird notes section 3.2.2).
 *        win_left = win_right = -1 switches the band off.
 *   2. Padded keys are removed: S = A minus { j : key_pad[b][j] != 0 } (the Longformer hub
 *      page, section 5: mask value 0 marks padding).  A key is counted once even when it is
 *      in several of the sets (a graph edge exists or not).
 *   3. E += |S| (the number of useful score entries).
 *   4. If S is empty: out = 0 and lse = -infinity.
 *   5. s_j = scale * sum_c q[i][c] * k[j][c] for j in S, ascending c, in fp64.
 *   6. m = max s_j, w_j = exp(s_j - m), l = sum w_j, out = (sum_j w_j v[j]) / l and
 *      lse = m + log(l); sums run over S in ascending key order.
 *
 * Backward pass (longattn_oracle_backward).  The forward output is a differentiable function
 * of q, k and v, and training with this attention needs its gradient (the Longformer hub page,
 * section 3, keeps training a converted model on long documents; the SWA/Hybrid-RoPE blog,
 * section 1, fine-tunes at 16K+ tokens).  Given the
 * gradient dO of a loss with respect to out, the oracle writes the exact gradients dQ, dK, dV of
 * that loss, from the chain rule through steps 5 and 6 with the same sets S:
 *
 *   P_j   = exp(s_j - lse)                    (the softmax weights of row i, j in S)
 *   dP_j  = sum_c dO[i][c] * v[j][c]          (gradient of the loss w.r.t. P_j)
 *   Drow  = sum_j P_j * dP_j                  (= sum_c dO[i][c] * out[i][c])
 *   dS_j  = P_j * (dP_j - Drow)               (through the softmax normalisation)
 *   dQ[i] = scale * sum_j dS_j * k[j],   dK[j] += scale * dS_j * q[i],   dV[j] += P_j * dO[i].
 *
 * Rows with an empty S contribute nothing (their output is the constant 0).  Each (b, h) is
 * handled by one thread, rows in ascending order, so the sums into dK and dV run in a fixed
 * order.
 *
 * Layout of every tensor: contiguous [batch][heads][n][d] (q, k, v, out, dO, dQ, dK, dV) and
 * [batch][heads][n] (lse).  All pointers are host pointers.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_OK = 0, ORACLE_BAD_ARG = -1, ORACLE_NO_MEMORY = -2 };

static int cmp_i32(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

static int64_t floor_div(int64_t a, int64_t b) { /* b > 0 */
  int64_t q = a / b;
  if ((a % b != 0) && (a < 0)) q -= 1;
  return q;
}

typedef struct {
  int64_t B, H, n, d;
  int64_t win_left, win_right;
  const int32_t* dilation;
  const int32_t* global_idx;
  int64_t n_global;
  const uint8_t* key_pad;
  const int32_t* layout;
  int64_t block, max_kb;
} problem;

static int check(const problem* p) {
  if (p->B < 0 || p->H < 0 || p->n < 0 || p->d < 0 || p->n_global < 0) return ORACLE_BAD_ARG;
  int band_off = (p->win_left == -1 && p->win_right == -1);
  if (!band_off && (p->win_left < 0 || p->win_right < 0)) return ORACLE_BAD_ARG;
  if (p->dilation)
    for (int64_t h = 0; h < p->H; ++h)
      if (p->dilation[h] < 1) return ORACLE_BAD_ARG;
  if (p->n_global > 0) {
    if (!p->global_idx) return ORACLE_BAD_ARG;
    for (int64_t t = 0; t < p->B * p->n_global; ++t)
      if (p->global_idx[t] < 0 || p->global_idx[t] >= p->n) return ORACLE_BAD_ARG;
  }
  if (p->layout) {
    if (p->block < 1 || p->max_kb < 0 || (p->n % p->block) != 0) return ORACLE_BAD_ARG;
    int64_t nb = p->n / p->block;
    for (int64_t t = 0; t < p->H * nb * p->max_kb; ++t)
      if (p->layout[t] < -1 || p->layout[t] >= nb) return ORACLE_BAD_ARG;
  }
  return ORACLE_OK;
}

/* Per-thread scratch: an epoch-stamped marker per position so a key in several sets is
 * listed once, the key list itself and its scores. */
typedef struct {
  int64_t* mark;
  int64_t epoch;
  int32_t* keys;
  int64_t cnt;
  double* s;
} scratch;

static void add_key(scratch* w, const problem* p, int64_t b, int64_t j) {
  if (w->mark[j] == w->epoch) return;
  w->mark[j] = w->epoch;
  if (p->key_pad && p->key_pad[b * p->n + j]) return; /* padded keys are never attended */
  w->keys[w->cnt++] = (int32_t)j;
}

/* Builds S(b, h, i) in w->keys (ascending).  is_global[b*n + i] marks global rows. */
static void build_set(scratch* w, const problem* p, const uint8_t* is_global, int64_t b,
                      int64_t h, int64_t i) {
  w->epoch += 1;
  w->cnt = 0;
  if (is_global && is_global[b * p->n + i]) {
    for (int64_t j = 0; j < p->n; ++j) add_key(w, p, b, j);
    return; /* already ascending */
  }
  if (!(p->win_left == -1 && p->win_right == -1)) {
    int64_t dil = p->dilation ? p->dilation[h] : 1;
    /* keys i + dil*t with t in [-win_left, win_right] that fall inside [0, n) */
    int64_t t_lo = -p->win_left, t_hi = p->win_right;
    int64_t t_min_in = -floor_div(i, dil);           /* smallest t with i + dil*t >= 0 */
    int64_t t_max_in = floor_div(p->n - 1 - i, dil); /* largest t with i + dil*t <= n-1 */
    if (t_lo < t_min_in) t_lo = t_min_in;
    if (t_hi > t_max_in) t_hi = t_max_in;
    for (int64_t t = t_lo; t <= t_hi; ++t) add_key(w, p, b, i + dil * t);
  }
  for (int64_t c = 0; c < p->n_global; ++c) add_key(w, p, b, p->global_idx[b * p->n_global + c]);
  if (p->layout) {
    int64_t nb = p->n / p->block;
    const int32_t* row = p->layout + (h * nb + i / p->block) * p->max_kb;
    for (int64_t s = 0; s < p->max_kb; ++s) {
      if (row[s] < 0) continue;
      for (int64_t j = (int64_t)row[s] * p->block; j < ((int64_t)row[s] + 1) * p->block; ++j)
        add_key(w, p, b, j);
    }
  }
  qsort(w->keys, (size_t)w->cnt, sizeof(int32_t), cmp_i32);
}

static int run(const problem* p, double scale, const double* q, const double* k,
               const double* v, double* out, double* lse, int64_t* E_out, int nthreads) {
  int rc = check(p);
  if (rc != ORACLE_OK) return rc;
  int64_t rows = p->B * p->H * p->n;
  uint8_t* is_global = NULL;
  if (p->n_global > 0 && p->B * p->n > 0) {
    is_global = (uint8_t*)calloc((size_t)(p->B * p->n), 1);
    if (!is_global) return ORACLE_NO_MEMORY;
    for (int64_t b = 0; b < p->B; ++b)
      for (int64_t c = 0; c < p->n_global; ++c)
        is_global[b * p->n + p->global_idx[b * p->n_global + c]] = 1;
  }
  if (nthreads <= 0) nthreads = omp_get_max_threads();
  int64_t E = 0;
  int failed = 0;
#pragma omp parallel num_threads(nthreads) reduction(+ : E) reduction(| : failed)
  {
    scratch w;
    size_t cap = (size_t)(p->n > 0 ? p->n : 1);
    w.mark = (int64_t*)malloc(cap * sizeof(int64_t));
    w.keys = (int32_t*)malloc(cap * sizeof(int32_t));
    w.s = (double*)malloc(cap * sizeof(double));
    w.epoch = 0;
    if (!w.mark || !w.keys || !w.s) failed = 1;
    if (!failed) {
      for (size_t j = 0; j < cap; ++j) w.mark[j] = 0;
    }
#pragma omp for schedule(dynamic, 32)
    for (int64_t r = 0; r < rows; ++r) {
      if (failed) continue;
      int64_t i = r % p->n, bh = r / p->n, h = bh % p->H, b = bh / p->H;
      build_set(&w, p, is_global, b, h, i);
      E += w.cnt;
      if (!q) continue; /* counting only */
      const double* qi = q + r * p->d;
      double* oi = out + r * p->d;
      const double* kb = k + bh * p->n * p->d;
      const double* vb = v + bh * p->n * p->d;
      if (w.cnt == 0) {
        for (int64_t c = 0; c < p->d; ++c) oi[c] = 0.0;
        if (lse) lse[r] = -INFINITY;
        continue;
      }
      double m = -INFINITY;
      for (int64_t t = 0; t < w.cnt; ++t) {
        const double* kj = kb + (int64_t)w.keys[t] * p->d;
        double dot = 0.0;
        for (int64_t c = 0; c < p->d; ++c) dot += qi[c] * kj[c];
        w.s[t] = scale * dot;
        if (w.s[t] > m) m = w.s[t];
      }
      double l = 0.0;
      for (int64_t c = 0; c < p->d; ++c) oi[c] = 0.0;
      for (int64_t t = 0; t < w.cnt; ++t) {
        double wt = exp(w.s[t] - m);
        l += wt;
        const double* vj = vb + (int64_t)w.keys[t] * p->d;
        for (int64_t c = 0; c < p->d; ++c) oi[c] += wt * vj[c];
      }
      for (int64_t c = 0; c < p->d; ++c) oi[c] /= l;
      if (lse) lse[r] = m + log(l);
    }
    free(w.mark);
    free(w.keys);
    free(w.s);
  }
  free(is_global);
  if (failed) return ORACLE_NO_MEMORY;
  if (E_out) *E_out = E;
  return ORACLE_OK;
}

/* Forward pass.  q, k, v, out: [B][H][n][d] fp64; lse: [B][H][n] fp64 or NULL.
 * dilation: [H] or NULL (all 1).  global_idx: [B][n_global], each in [0, n).
 * key_pad: [B][n] (nonzero = padded key) or NULL.  layout: [H][n/block][max_kb] block ids,
 * -1 = unused slot, or NULL.  E_out: receives the number of useful score entries.
 * nthreads <= 0 uses OpenMP's default.  Returns 0, or a negative code on bad arguments. */
int longattn_oracle_forward(int64_t B, int64_t H, int64_t n, int64_t d, double scale,
                            int64_t win_left, int64_t win_right, const int32_t* dilation,
                            const int32_t* global_idx, int64_t n_global, const uint8_t* key_pad,
                            const int32_t* layout, int64_t block, int64_t max_kb,
                            const double* q, const double* k, const double* v, double* out,
                            double* lse, int64_t* E_out, int nthreads) {
  problem p = {B, H, n, d, win_left, win_right, dilation, global_idx, n_global,
               key_pad, layout, block, max_kb};
  if (!q || !k || !v || !out) return ORACLE_BAD_ARG;
  return run(&p, scale, q, k, v, out, lse, E_out, nthreads);
}

/* Number of useful score entries E = sum over (b, h, i) of |S(b, h, i)|, no arithmetic. */
int longattn_oracle_count(int64_t B, int64_t H, int64_t n, int64_t win_left, int64_t win_right,
                          const int32_t* dilation, const int32_t* global_idx, int64_t n_global,
                          const uint8_t* key_pad, const int32_t* layout, int64_t block,
                          int64_t max_kb, int64_t* E_out, int nthreads) {
  problem p = {B, H, n, 0, win_left, win_right, dilation, global_idx, n_global,
               key_pad, layout, block, max_kb};
  return run(&p, 0.0, NULL, NULL, NULL, NULL, NULL, E_out, nthreads);
}

/* The allowed key set of one query row, ascending, written to keys_out (capacity n).
 * Returns the set size, or a negative code on bad arguments. */
int64_t longattn_oracle_row_set(int64_t B, int64_t H, int64_t n, int64_t win_left,
                                int64_t win_right, const int32_t* dilation,
                                const int32_t* global_idx, int64_t n_global,
                                const uint8_t* key_pad, const int32_t* layout, int64_t block,
                                int64_t max_kb, int64_t b, int64_t h, int64_t i,
                                int32_t* keys_out) {
  problem p = {B, H, n, 0, win_left, win_right, dilation, global_idx, n_global,
               key_pad, layout, block, max_kb};
  int rc = check(&p);
  if (rc != ORACLE_OK) return rc;
  if (b < 0 || b >= B || h < 0 || h >= H || i < 0 || i >= n) return ORACLE_BAD_ARG;
  uint8_t* is_global = NULL;
  if (n_global > 0) {
    is_global = (uint8_t*)calloc((size_t)(B * n), 1);
    if (!is_global) return ORACLE_NO_MEMORY;
    for (int64_t bb = 0; bb < B; ++bb)
      for (int64_t c = 0; c < n_global; ++c) is_global[bb * n + global_idx[bb * n_global + c]] = 1;
  }
  scratch w;
  w.mark = (int64_t*)calloc((size_t)n, sizeof(int64_t));
  w.keys = keys_out;
  w.s = NULL;
  w.epoch = 0;
  if (!w.mark) {
    free(is_global);
    return ORACLE_NO_MEMORY;
  }
  build_set(&w, &p, is_global, b, h, i);
  free(w.mark);
  free(is_global);
  return w.cnt;
}

/* Backward pass: gradients of sum(dout * out) with respect to q, k and v (see the header).
 * dout, dq, dk, dv: [B][H][n][d] fp64; dq, dk, dv are overwritten.  Returns 0, or a negative
 * code on bad arguments. */
int longattn_oracle_backward(int64_t B, int64_t H, int64_t n, int64_t d, double scale,
                             int64_t win_left, int64_t win_right, const int32_t* dilation,
                             const int32_t* global_idx, int64_t n_global,
                             const uint8_t* key_pad, const int32_t* layout, int64_t block,
                             int64_t max_kb, const double* q, const double* k, const double* v,
                             const double* dout, double* dq, double* dk, double* dv,
                             int nthreads) {
  problem p = {B, H, n, d, win_left, win_right, dilation, global_idx, n_global,
               key_pad, layout, block, max_kb};
  if (!q || !k || !v || !dout || !dq || !dk || !dv) return ORACLE_BAD_ARG;
  int rc = check(&p);
  if (rc != ORACLE_OK) return rc;
  uint8_t* is_global = NULL;
  if (n_global > 0 && B * n > 0) {
    is_global = (uint8_t*)calloc((size_t)(B * n), 1);
    if (!is_global) return ORACLE_NO_MEMORY;
    for (int64_t b = 0; b < B; ++b)
      for (int64_t c = 0; c < n_global; ++c) is_global[b * n + global_idx[b * n_global + c]] = 1;
  }
  memset(dq, 0, (size_t)(B * H * n * d) * sizeof(double));
  memset(dk, 0, (size_t)(B * H * n * d) * sizeof(double));
  memset(dv, 0, (size_t)(B * H * n * d) * sizeof(double));
  if (nthreads <= 0) nthreads = omp_get_max_threads();
  int failed = 0;
#pragma omp parallel num_threads(nthreads) reduction(| : failed)
  {
    scratch w;
    size_t cap = (size_t)(n > 0 ? n : 1);
    w.mark = (int64_t*)calloc(cap, sizeof(int64_t));
    w.keys = (int32_t*)malloc(cap * sizeof(int32_t));
    w.s = (double*)malloc(cap * sizeof(double));
    double* dp = (double*)malloc(cap * sizeof(double));
    w.epoch = 0;
    if (!w.mark || !w.keys || !w.s || !dp) failed = 1;
#pragma omp for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < B * H; ++bh) {
      if (failed) continue;
      const int64_t b = bh / H, h = bh % H;
      const double* kb = k + bh * n * d;
      const double* vb = v + bh * n * d;
      double* dkb = dk + bh * n * d;
      double* dvb = dv + bh * n * d;
      for (int64_t i = 0; i < n; ++i) {
        build_set(&w, &p, is_global, b, h, i);
        if (w.cnt == 0) continue;
        const int64_t r = bh * n + i;
        const double* qi = q + r * d;
        const double* doi = dout + r * d;
        double* dqi = dq + r * d;
        /* scores and the log-normaliser of row i, as in the forward pass */
        double m = -INFINITY;
        for (int64_t t = 0; t < w.cnt; ++t) {
          const double* kj = kb + (int64_t)w.keys[t] * d;
          double dot = 0.0;
          for (int64_t c = 0; c < d; ++c) dot += qi[c] * kj[c];
          w.s[t] = dot * scale;
          if (w.s[t] > m) m = w.s[t];
        }
        double l = 0.0;
        for (int64_t t = 0; t < w.cnt; ++t) l += exp(w.s[t] - m);
        const double lse = m + log(l);
        /* P_j, dP_j and Drow */
        double drow = 0.0;
        for (int64_t t = 0; t < w.cnt; ++t) {
          const double* vj = vb + (int64_t)w.keys[t] * d;
          double dot = 0.0;
          for (int64_t c = 0; c < d; ++c) dot += doi[c] * vj[c];
          w.s[t] = exp(w.s[t] - lse); /* P_j from here on */
          dp[t] = dot;
          drow += w.s[t] * dot;
        }
        /* dS_j and the three gradients */
        for (int64_t t = 0; t < w.cnt; ++t) {
          const int64_t j = w.keys[t];
          const double ds = w.s[t] * (dp[t] - drow);
          const double* kj = kb + j * d;
          for (int64_t c = 0; c < d; ++c) {
            dqi[c] += scale * ds * kj[c];
            dkb[j * d + c] += scale * ds * qi[c];
            dvb[j * d + c] += w.s[t] * doi[c];
          }
        }
      }
    }
    free(w.mark);
    free(w.keys);
    free(w.s);
    free(dp);
  }
  free(is_global);
  return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/* ------------------------------------------------------------------------------------------
 * LongT5 Transient-Global attention (LongT5 guide, sections on TGlobal attention, the block and
 * side helpers, and relative position encoding).
 *
 * Global tokens.  The sequence is cut into fixed blocks of `blk` tokens (k = 16 by default); a
 * token's block id is i / blk, except that the trailing incomplete block (if any) merges into
 * the block before it, so there are G = max(1, n / blk) global tokens and block(i) =
 * min(i / blk, G - 1); padded tokens belong to no block.  Global token g of sample b is the sum
 * of the embeddings x of the non-padded tokens of block g, RMS-normalised (y = s / sqrt(mean(s^2)
 * + eps) * gamma, the T5 layer norm), then projected with the attention's key and value
 * weights: side_k[b, h, g] = y . Wk[:, h*d : (h+1)*d], side_v likewise.  A block without any
 * non-padded token gives no global token (side_valid = 0).
 *
 * Attention.  Query i (head h) attends
 *   the local keys j with |i - j| <= radius that are not padded, score scale * q_i . k_j +
 *   bias_local[bucket(j - i)][h], and
 *   every valid global token g, score scale * q_i . side_k[g] + bias_side[bucket(g - block(i))][h],
 * all in one softmax (the side keys join the local keys); out = sum of weights times the local
 * values and the side values; lse as in the forward pass.  E counts the (query, key) pairs:
 * O(n (r + n/k)) (the guide's cost law).
 *
 * Relative position buckets (T5's bidirectional scheme, as the guide describes it): half of the
 * buckets are for positive distances (key after query), half for the rest; within a half,
 * distances below half/2 get one bucket each, larger ones share log-spaced buckets up to
 * max_distance, and everything farther falls in the half's last bucket:
 *   h = nb / 2; base = (rel > 0) ? h : 0; a = |rel|; e = h / 2;
 *   a < e:  base + a;  else base + min(h - 1, e + floor(log(a / e) / log(md / e) * (h - e))).
 * fp64 throughout.
 * ------------------------------------------------------------------------------------------ */
int64_t longattn_oracle_t5_bucket(int64_t rel, int64_t num_buckets, int64_t max_distance) {
  const int64_t half = num_buckets / 2;
  const int64_t base = rel > 0 ? half : 0;
  const int64_t a = rel < 0 ? -rel : rel;
  const int64_t exact = half / 2;
  if (a < exact) return base + a;
  const double x = log((double)a / (double)exact) / log((double)max_distance / (double)exact) *
                   (double)(half - exact);
  int64_t off = exact + (int64_t)floor(x);
  if (off > half - 1) off = half - 1;
  return base + off;
}

static int64_t tg_num_global(int64_t n, int64_t blk) {
  int64_t G = n / blk;
  return G < 1 ? 1 : G;
}

/* Global tokens.  x: [B][n][dm]; gamma: [dm]; wk, wv: [dm][H*d]; key_pad: [B][n] or NULL.
 * side_k, side_v: [B][H][G][d]; side_valid: [B][G] (1 = the block has a non-padded token). */
int longattn_oracle_tglobal_side(int64_t B, int64_t n, int64_t dm, int64_t H, int64_t d,
                                 int64_t blk, double eps, const double* x, const double* gamma,
                                 const double* wk, const double* wv, const uint8_t* key_pad,
                                 double* side_k, double* side_v, uint8_t* side_valid) {
  if (B < 0 || n < 1 || dm < 1 || H < 1 || d < 1 || blk < 1 || !(eps >= 0.0)) return ORACLE_BAD_ARG;
  if (!x || !gamma || !wk || !wv || !side_k || !side_v || !side_valid) return ORACLE_BAD_ARG;
  const int64_t G = tg_num_global(n, blk);
  double* s = (double*)malloc((size_t)dm * sizeof(double));
  double* y = (double*)malloc((size_t)dm * sizeof(double));
  if (!s || !y) {
    free(s);
    free(y);
    return ORACLE_NO_MEMORY;
  }
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t g = 0; g < G; ++g) {
      /* sum of the block's non-padded token embeddings (the merged tail included) */
      for (int64_t c = 0; c < dm; ++c) s[c] = 0.0;
      int any = 0;
      for (int64_t i = 0; i < n; ++i) {
        int64_t bi = i / blk;
        if (bi > G - 1) bi = G - 1;
        if (bi != g) continue;
        if (key_pad && key_pad[b * n + i]) continue;
        any = 1;
        for (int64_t c = 0; c < dm; ++c) s[c] += x[(b * n + i) * dm + c];
      }
      side_valid[b * G + g] = (uint8_t)any;
      /* RMS normalisation */
      double ms = 0.0;
      for (int64_t c = 0; c < dm; ++c) ms += s[c] * s[c];
      ms /= (double)dm;
      const double inv = 1.0 / sqrt(ms + eps);
      for (int64_t c = 0; c < dm; ++c) y[c] = s[c] * inv * gamma[c];
      /* projections */
      for (int64_t h = 0; h < H; ++h)
        for (int64_t c = 0; c < d; ++c) {
          double ak = 0.0, av = 0.0;
          for (int64_t m = 0; m < dm; ++m) {
            ak += y[m] * wk[m * (H * d) + h * d + c];
            av += y[m] * wv[m * (H * d) + h * d + c];
          }
          side_k[((b * H + h) * G + g) * d + c] = ak;
          side_v[((b * H + h) * G + g) * d + c] = av;
        }
    }
  }
  free(s);
  free(y);
  return ORACLE_OK;
}

/* Attention.  q, k, v, out: [B][H][n][d]; side_k, side_v: [B][H][G][d]; side_valid: [B][G];
 * key_pad: [B][n] or NULL; bias_local, bias_side: [num_buckets][H]; lse: [B][H][n] or NULL. */
int longattn_oracle_tglobal_forward(int64_t B, int64_t H, int64_t n, int64_t d, int64_t radius,
                                    int64_t blk, int64_t num_buckets, int64_t max_distance,
                                    double scale, const double* q, const double* k,
                                    const double* v, const double* side_k, const double* side_v,
                                    const uint8_t* side_valid, const uint8_t* key_pad,
                                    const double* bias_local, const double* bias_side,
                                    double* out, double* lse, int64_t* E_out, int nthreads) {
  if (B < 0 || H < 1 || n < 1 || d < 1 || radius < 0 || blk < 1 || num_buckets < 4 ||
      max_distance < 1)
    return ORACLE_BAD_ARG;
  if (!q || !k || !v || !side_k || !side_v || !side_valid || !bias_local || !bias_side || !out)
    return ORACLE_BAD_ARG;
  const int64_t G = tg_num_global(n, blk);
  if (nthreads <= 0) nthreads = omp_get_max_threads();
  int64_t E = 0;
  int failed = 0;
  const int64_t rows = B * H * n;
#pragma omp parallel num_threads(nthreads) reduction(+ : E) reduction(| : failed)
  {
    const size_t cap = (size_t)(2 * radius + 1 + G);
    double* sc = (double*)malloc(cap * sizeof(double));
    const double** vr = (const double**)malloc(cap * sizeof(double*));
    if (!sc || !vr) failed = 1;
#pragma omp for schedule(dynamic, 64)
    for (int64_t r = 0; r < rows; ++r) {
      if (failed) continue;
      const int64_t i = r % n, bh = r / n, h = bh % H, b = bh / H;
      const double* qi = q + r * d;
      int64_t cnt = 0;
      /* local keys */
      const int64_t j0 = i - radius < 0 ? 0 : i - radius;
      const int64_t j1 = i + radius > n - 1 ? n - 1 : i + radius;
      for (int64_t j = j0; j <= j1; ++j) {
        if (key_pad && key_pad[b * n + j]) continue;
        const double* kj = k + (bh * n + j) * d;
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c) dot += qi[c] * kj[c];
        sc[cnt] = scale * dot + bias_local[longattn_oracle_t5_bucket(j - i, num_buckets, max_distance) * H + h];
        vr[cnt] = v + (bh * n + j) * d;
        ++cnt;
      }
      /* global tokens */
      int64_t bi = i / blk;
      if (bi > G - 1) bi = G - 1;
      for (int64_t g = 0; g < G; ++g) {
        if (!side_valid[b * G + g]) continue;
        const double* kg = side_k + (bh * G + g) * d;
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c) dot += qi[c] * kg[c];
        sc[cnt] = scale * dot + bias_side[longattn_oracle_t5_bucket(g - bi, num_buckets, max_distance) * H + h];
        vr[cnt] = side_v + (bh * G + g) * d;
        ++cnt;
      }
      E += cnt;
      double* oi = out + r * d;
      for (int64_t c = 0; c < d; ++c) oi[c] = 0.0;
      if (cnt == 0) {
        if (lse != NULL) lse[r] = -INFINITY;
        continue;
      }
      double m = -INFINITY;
      for (int64_t t = 0; t < cnt; ++t)
        if (sc[t] > m) m = sc[t];
      double l = 0.0;
      for (int64_t t = 0; t < cnt; ++t) {
        const double w = exp(sc[t] - m);
        l += w;
        for (int64_t c = 0; c < d; ++c) oi[c] += w * vr[t][c];
      }
      for (int64_t c = 0; c < d; ++c) oi[c] /= l;
      if (lse != NULL) lse[r] = m + log(l);
    }
    free(sc);
    free(vr);
  }
  if (failed) return ORACLE_NO_MEMORY;
  if (E_out) *E_out = E;
  return ORACLE_OK;
}

/* ------------------------------------------------------------------------------------------
 * Output gates of gated attention (SWA/Hybrid-RoPE blog, section 3: Gated Attention).
 *
 * Elementwise: each head's output is multiplied, dimension by dimension, by a sigmoid gate:
 *   gated[b][h][i][c] = out[b][h][i][c] * sigmoid(gate[b][h][i][c]),
 * gate being the pre-sigmoid logits the model computes for that token (an input here).
 * LowRank (bottleneck r, 128 on the page): the token's attention output over all heads,
 * o = out[b][:][i][:] flattened head-major (H*d values), is projected to r dimensions and back,
 * and the result gates o:  gated = o * sigmoid(W_up (W_down o)), W_down: [r][H*d],
 * W_up: [H*d][r].  sigmoid(x) = 1 / (1 + exp(-x)).  fp64.
 * ------------------------------------------------------------------------------------------ */
int longattn_oracle_gate_elementwise(int64_t count, const double* out, const double* gate,
                                     double* gated) {
  if (count < 0 || !out || !gate || !gated) return ORACLE_BAD_ARG;
  for (int64_t e = 0; e < count; ++e) gated[e] = out[e] / (1.0 + exp(-gate[e]));
  return ORACLE_OK;
}

int longattn_oracle_gate_lowrank(int64_t B, int64_t H, int64_t n, int64_t d, int64_t r,
                                 const double* out, const double* w_down, const double* w_up,
                                 double* gated) {
  if (B < 0 || H < 1 || n < 0 || d < 1 || r < 1 || !out || !w_down || !w_up || !gated)
    return ORACLE_BAD_ARG;
  const int64_t hd = H * d;
  double* o = (double*)malloc((size_t)hd * sizeof(double));
  double* z = (double*)malloc((size_t)r * sizeof(double));
  if (!o || !z) {
    free(o);
    free(z);
    return ORACLE_NO_MEMORY;
  }
  for (int64_t b = 0; b < B; ++b)
    for (int64_t i = 0; i < n; ++i) {
      for (int64_t h = 0; h < H; ++h)
        for (int64_t c = 0; c < d; ++c) o[h * d + c] = out[((b * H + h) * n + i) * d + c];
      for (int64_t t = 0; t < r; ++t) {
        double acc = 0.0;
        for (int64_t e = 0; e < hd; ++e) acc += w_down[t * hd + e] * o[e];
        z[t] = acc;
      }
      for (int64_t h = 0; h < H; ++h)
        for (int64_t c = 0; c < d; ++c) {
          const int64_t e = h * d + c;
          double acc = 0.0;
          for (int64_t t = 0; t < r; ++t) acc += w_up[e * r + t] * z[t];
          gated[((b * H + h) * n + i) * d + c] = o[e] / (1.0 + exp(-acc));
        }
    }
  free(o);
  free(z);
  return ORACLE_OK;
}
