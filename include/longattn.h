/*
 * longattn — forward pass of banded sparse self-attention on AMD MI355X (gfx950).
 *
 * What one call computes.  For every batch sample b, head h and query row i, the output row
 * is exact softmax attention of q[b,h,i] over the key set S(b,h,i), scaled by `scale`:
 *
 *   out[b,h,i] = sum_{j in S} softmax_j(scale * q_i . k_j) * v_j,
 *   lse[b,h,i] = log sum_{j in S} exp(scale * q_i . k_j)       (natural log)
 *
 * S is the union of (each key counted once), minus the padded keys of sample b:
 *   - the window i + dil[h]*t, t in [-win_left, win_right], cut to [0, n): a sliding window
 *     around the query, symmetric as in Longformer or causal (win_right = 0) as in
 *     sliding-window decoders (Longformer hub page, section 2; Big Bird reading notes,
 *     section 3.2.1; SWAN-GPT summary, section 3.3).  With dil > 1 the window skips tokens
 *     like a dilated convolution: the same number of keys over a span dil times wider
 *     (Longformer hub page, section 2);
 *   - the global tokens global_idx[b][*]: every position attends them, and a global token's
 *     own row attends the whole sequence (Longformer hub page, section 2; Big Bird notes,
 *     section 3.2.3, the ITC form that marks existing tokens as global);
 *   - the key blocks listed for (h, block of i) in block_layout: BigBird's random and sliding
 *     blocks (Big Bird notes, sections 3.2.2 and 3.3).
 * Padded keys are never attended (Longformer hub page, section 5: a 0 in the attention mask
 * marks padding).  A query row whose set is empty gets out = 0 and lse = -inf.
 *
 * Layout.  q, k, v, out: contiguous [batch][heads][n][d] (row-major, "BHND"), all of `dtype`.
 * lse: contiguous fp32 [batch][heads][n].  bf16 values are stored as raw 16-bit patterns.
 *
 * Ownership.  Every tensor pointer is DEVICE memory allocated and owned by the caller, except
 * `dilation`, which is a HOST array read during the call.  The library allocates no device
 * memory and keeps no state between calls; scratch space comes from the caller's workspace.
 * Calls are asynchronous on `stream` (a hipStream_t; NULL = the default stream): results are
 * valid once the stream has been synchronised.  Concurrent calls on different streams must
 * use different workspaces.
 *
 * Errors.  A call that returns anything but LONGATTN_OK has launched nothing (except
 * LONGATTN_ERR_HIP, which reports a failed launch).  No exception crosses this interface.
 * With the environment variable LONGATTN_DEBUG=1 the library also copies global_idx and
 * block_layout to the host and checks their contents (sorted, distinct, in range).
 */
#ifndef LONGATTN_H
#define LONGATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum longattn_status {
  LONGATTN_OK = 0,
  LONGATTN_ERR_INVALID_ARG = 1, /* a size, window, dilation, index or pointer is out of range */
  LONGATTN_ERR_UNSUPPORTED = 2, /* valid, but the library has no kernel for it (see below)    */
  LONGATTN_ERR_ALIGNMENT = 3,   /* q, k, v or out is not 16-byte aligned                       */
  LONGATTN_ERR_WORKSPACE = 4,   /* workspace missing or smaller than longattn_workspace_size  */
  LONGATTN_ERR_HIP = 5          /* the HIP runtime reported an error while launching           */
} longattn_status;

typedef enum longattn_dtype { LONGATTN_BF16 = 0, LONGATTN_F32 = 1 } longattn_dtype;

typedef struct longattn_desc {
  int32_t batch, heads, n, d; /* each >= 0; d >= 1                                             */
  int32_t dtype;              /* longattn_dtype of q, k, v and out                             */
  float scale;                /* > 0 and finite; 1/sqrt(d) for standard attention            */
  int32_t win_left;           /* one-sided inclusive extents in dilated steps, >= 0;          */
  int32_t win_right;          /*   win_left = win_right = -1 switches the window off          */
  const int32_t* dilation;    /* HOST [heads], each >= 1; NULL = 1 for every head              */
  const int32_t* global_idx;  /* DEVICE [batch][n_global]: per sample ascending, distinct,
                                 each in [0, n)                                               */
  int32_t n_global;           /* 0 = no global tokens; n_global <= n                           */
  const uint8_t* key_pad;     /* DEVICE [batch][n], nonzero = padded key; NULL = no padding    */
  const int32_t* block_layout; /* DEVICE [heads][n/block][max_kb] key-block ids, distinct per
                                  row, -1 = unused slot; NULL = no block layout               */
  int32_t block;              /* layout block size: n % block == 0                             */
  int32_t max_kb;             /* slots per layout row                                          */
} longattn_desc;

/*
 * What the GPU kernels implement (anything else valid returns LONGATTN_ERR_UNSUPPORTED):
 *   bf16: d in {64, 128}; n * d * 2 < 2^31 (one head's K or V under 2 GiB); either the window
 *         or the block layout (not both at once); layout block in {64, 128}, max_kb <= 256;
 *         n_global <= 256; if the heads' dilations differ, each is <= 255 and heads <= 256.
 *   fp32: 1 <= d <= 256; every combination of window, dilation, globals, padding and layout.
 */

/* Bytes of device workspace longattn_forward needs for this descriptor (0 if none).
 * The answer depends only on the descriptor's sizes and dtype. */
longattn_status longattn_workspace_size(const longattn_desc* desc, size_t* bytes);

/* One forward pass.  q, k, v: DEVICE [B][H][n][d] inputs; out: DEVICE [B][H][n][d] output;
 * lse: DEVICE fp32 [B][H][n] output or NULL; workspace: DEVICE scratch of at least
 * longattn_workspace_size bytes (may be NULL when that size is 0). */
longattn_status longattn_forward(const longattn_desc* desc, const void* q, const void* k,
                                 const void* v, void* out, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* The same pass, with caller-created hipEvent_t handles that time each kernel: marks[0] and
 * marks[1] record the start and end of the attention kernel (every non-global row plus the
 * global rows' per-chunk partials, one launch), marks[2] and marks[3] those of the global-row
 * combine kernel.  The events are attached to the kernels' own dispatches; when the combine does
 * not run, marks[2] and marks[3] are recorded back to back on `stream` after the attention
 * kernel.  n_marks must be 0 (no marks, same as longattn_forward) or LONGATTN_N_MARKS. */
#define LONGATTN_N_MARKS 4
longattn_status longattn_forward_marked(const longattn_desc* desc, const void* q, const void* k,
                                        const void* v, void* out, float* lse, void* workspace,
                                        size_t workspace_bytes, void* stream,
                                        void* const* marks, int32_t n_marks);

/* The forward pass of gated attention with an elementwise output gate (SWA/Hybrid-RoPE blog,
 * section 3, Gated Attention: a per-dimension sigmoid gate on each head's output), fused into
 * the kernels' epilogues: out = attention(q, k, v) * sigmoid(gate), elementwise.  gate: DEVICE
 * [B][H][n][d] pre-sigmoid logits in desc->dtype (not NULL, 16-byte aligned); lse is that of the
 * attention before the gate.  Everything else as longattn_forward. */
longattn_status longattn_forward_gated(const longattn_desc* desc, const void* q, const void* k,
                                       const void* v, const void* gate, void* out, float* lse,
                                       void* workspace, size_t workspace_bytes, void* stream);

/* Low-rank output gate of gated attention (SWA/Hybrid-RoPE blog, section 3: the attention output
 * is projected to a bottleneck, 128 dimensions on the page, and then gates): for every token,
 * o = its outputs over all heads (H*d values, head-major), and
 *   out = o * sigmoid(w_up (w_down o)),
 * written in place.  out: DEVICE bf16 [B][H][n][d]; w_down: DEVICE bf16 [rank][H*d]; w_up:
 * DEVICE bf16 [H*d][rank]; 16-byte aligned.  Kernels: d % 16 == 0, H*d % 32 == 0 and
 * H*d <= 16384, rank in {32, 64, 128, 256}; other valid sizes return UNSUPPORTED. */
typedef struct {
  int32_t batch, heads, n, d;
  int32_t rank;
} longattn_gate_desc;
longattn_status longattn_gate_lowrank(const longattn_gate_desc* desc, void* out,
                                      const void* w_down, const void* w_up, void* stream);

/* The forward pass without a caller workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments and result as longattn_forward without the workspace; allocates nothing.  The
 * scratch it needs (the global rows' partial results) lives in a device array of the library's
 * own, LONGATTN_NOALLOC_SCRATCH_BYTES bytes, one per GPU, held until the process ends.  A
 * descriptor whose longattn_workspace_size exceeds that returns LONGATTN_ERR_WORKSPACE and
 * launches nothing.  Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (different streams, or host threads) race and must be serialised by the caller; calls in
 * order on one stream are safe (each pass writes every partial it reads).  The first call on
 * each GPU resolves the array's device address (a runtime query, no allocation); make it before
 * capturing a graph.  LONGATTN_DEBUG checks are not run by this entry point. */
#define LONGATTN_NOALLOC_SCRATCH_BYTES (32u << 20)
longattn_status longattn_forward_noalloc(const longattn_desc* desc, const void* q,
                                         const void* k, const void* v, void* out, float* lse,
                                         void* stream);

/* Useful score entries, counted on the GPU: entries_out is a DEVICE int64[2] that receives
 * [0] E = sum over all (b, h, i) of |S(b, h, i)| and [1] the part of E in global-token rows
 * (asynchronous on `stream`).  4 * d * E is the useful floating-point work of one forward pass
 * (2d for the score dot product and 2d for the weighted value sum of each entry). */
longattn_status longattn_count_entries(const longattn_desc* desc, int64_t* entries_out,
                                       void* stream);

/* ---------------------------------------------------------------------------------------
 * Backward pass.
 *
 * Gradients of a loss through the forward pass above, for training with this attention (the
 * Longformer hub page, section 3: a converted model keeps training on long documents; the
 * SWA/Hybrid-RoPE blog, section 1: a 16K+ fine-tuning stage).  Given dout = dLoss/dout, it writes
 * dq, dk, dv = dLoss/dq, dLoss/dk, dLoss/dv of the same descriptor's attention:
 *   P_ij = exp(scale * q_i . k_j - lse_i) for j in S(b, h, i),  Drow_i = dout_i . out_i,
 *   dS_ij = P_ij * (dout_i . v_j - Drow_i),
 *   dq_i = scale * sum_j dS_ij k_j,  dk_j = scale * sum_i dS_ij q_i,  dv_j = sum_i P_ij dout_i.
 * Rows with an empty key set (lse = -inf) contribute nothing.  out and lse must be the forward
 * pass's outputs for the same q, k, v and descriptor (the saved log-normaliser replaces the
 * softmax recomputation).
 *
 * q, k, v, out, dout: DEVICE [B][H][n][d] inputs (desc->dtype); lse: DEVICE fp32 [B][H][n];
 * dq, dk, dv: DEVICE [B][H][n][d] outputs (desc->dtype), overwritten, not aliasing any input.
 * Every (b, h) position gets a value (0 where no edge touches it).  workspace: DEVICE scratch of
 * at least longattn_backward_workspace_size bytes.  Kernels: bf16 with d in {64, 128} and no
 * block layout runs on matrix cores (bf16 operands, fp32 accumulation; within the forward's
 * bf16 limits); every other pattern with d <= 256, in both dtypes, on per-row kernels with fp32
 * arithmetic.  Status rules as longattn_forward.
 * --------------------------------------------------------------------------------------- */
longattn_status longattn_backward_workspace_size(const longattn_desc* desc, size_t* bytes);
longattn_status longattn_backward(const longattn_desc* desc, const void* q, const void* k,
                                  const void* v, const void* out, const float* lse,
                                  const void* dout, void* dq, void* dk, void* dv,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* The same pass with caller-created hipEvent_t handles that time its phases.  Matrix-core path
 * (attached to the kernels' dispatches): marks[0..1] the start and end of the dQ kernel (which
 * also prepares each row's Drow), marks[2..3] of the dK/dV kernel, marks[4..5] of the global-
 * token combine (recorded back to back when there are no global tokens).  Per-row path:
 * marks[0..1] bracket the Drow kernel and marks[2..5] the dQ and dK/dV kernels together.
 * n_marks: 0 or LONGATTN_BWD_N_MARKS. */
#define LONGATTN_BWD_N_MARKS 6
longattn_status longattn_backward_marked(const longattn_desc* desc, const void* q,
                                         const void* k, const void* v, const void* out,
                                         const float* lse, const void* dout, void* dq, void* dk,
                                         void* dv, void* workspace, size_t workspace_bytes,
                                         void* stream, void* const* marks, int32_t n_marks);

/* ---------------------------------------------------------------------------------------
 * LongT5 Transient-Global attention (LongT5 guide: Transient-Global attention, the block and
 * side helpers, relative position encoding).
 *
 * Global tokens: the sequence is cut into blocks of `block` tokens (k = 16 by default); the
 * trailing incomplete block merges into the one before it, so there are G = max(1, n / block)
 * global tokens and token i belongs to block min(i / block, G - 1).  Global token g of sample b
 * is the sum of the embeddings x of the block's non-padded tokens, RMS-normalised
 * (y = s / sqrt(mean(s^2) + eps) * gamma) and projected with the attention's key and value
 * weights: side_k[b][h][g] = y . wk[:, h*d : (h+1)*d], side_v likewise.  side_valid[b][g] = 0
 * when the block has no non-padded token.
 *
 * Attention: query i of head h attends the local keys j with |i - j| <= radius (not padded),
 * score scale * q_i . k_j + bias_local[bucket(j - i)][h], and every valid global token g, score
 * scale * q_i . side_k[g] + bias_side[bucket(g - block(i))][h], all in one softmax; out and lse
 * as in longattn_forward.  bucket() is T5's bidirectional relative-position bucket with
 * num_buckets buckets and max_distance (half the buckets per direction, exact below a quarter
 * of num_buckets, log-spaced up to max_distance, saturated beyond).
 *
 * Tensors (DEVICE): x [B][n][d_model] bf16; gamma fp32 [d_model]; wk, wv bf16 [d_model][H*d];
 * q, k, v, out bf16 [B][H][n][d]; side_k, side_v bf16 [B][H][G][d] (written by
 * longattn_tglobal_side, read by longattn_tglobal_forward); side_valid uint8 [B][G]; bias
 * tables fp32 [num_buckets][H]; lse fp32 [B][H][n] or NULL.  Kernels: bf16, d in {64, 128},
 * radius <= 512, max_distance <= 512, num_buckets even in [4, 256], d_model a multiple of 64
 * and <= 4096 (the normalised global inputs are rounded to bf16 before the projections); other
 * valid values return LONGATTN_ERR_UNSUPPORTED.  Workspace: longattn_tglobal_workspace_size
 * bytes (covers both calls), 16-byte aligned (else LONGATTN_ERR_ALIGNMENT).
 * --------------------------------------------------------------------------------------- */
typedef struct {
  int32_t batch, heads, n, d;
  int32_t d_model;
  float scale;                 /* > 0 and finite                                                 */
  int32_t radius;              /* local radius r >= 0                                            */
  int32_t block;               /* global block length k >= 1                                     */
  int32_t num_buckets;         /* even, >= 4                                                     */
  int32_t max_distance;        /* >= 1                                                           */
  float eps;                   /* RMS-norm epsilon, >= 0                                         */
  const uint8_t* key_pad;      /* DEVICE [batch][n], nonzero = padded token; NULL = none         */
} longattn_tglobal_desc;

longattn_status longattn_tglobal_workspace_size(const longattn_tglobal_desc* desc, size_t* bytes);
longattn_status longattn_tglobal_side(const longattn_tglobal_desc* desc, const void* x,
                                      const float* gamma, const void* wk, const void* wv,
                                      void* side_k, void* side_v, uint8_t* side_valid,
                                      void* workspace, size_t workspace_bytes, void* stream);
longattn_status longattn_tglobal_forward(const longattn_tglobal_desc* desc, const void* q,
                                         const void* k, const void* v, const void* side_k,
                                         const void* side_v, const uint8_t* side_valid,
                                         const float* bias_local, const float* bias_side,
                                         void* out, float* lse, void* workspace,
                                         size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * Sliding-window decode over a key/value cache.
 *
 * The incremental form of the causal sliding window used by the SWA decoder layers (SWAN-GPT
 * summary, section on the SWA-RoPE layers; SWA/Hybrid-RoPE blog, section 3: a 512-key window
 * and a cost of O(n*w) because each token looks at its last w keys only).  Sample b brings m new
 * query rows at absolute positions t0_b, t0_b + 1, ..., t0_b + m - 1; the row at position t
 * attends the keys at positions max(0, t - window + 1) .. t, which must already be in the cache:
 *
 *   out[b,h,j] = sum_{p in P(t)} softmax_p(scale * q[b,h,j] . k(p)) * v(p),   t = t0_b + j,
 *   lse[b,h,j] = log sum_{p in P(t)} exp(scale * q[b,h,j] . k(p)),
 *
 * which is exactly the forward pass above with win_left = window - 1, win_right = 0, no global
 * tokens and no padding, restricted to those rows.  Position p lives in cache slot
 *   p                  (linear cache, ring = 0; requires t0_b + m - 1 < cache_len), or
 *   p mod cache_len    (rolling buffer, ring = 1; requires window + m - 1 <= cache_len so the
 *                      slots of every needed position still hold it).
 *
 * q: DEVICE [B][H][m][d]; k_cache, v_cache: DEVICE [B][H][cache_len][d]; out: DEVICE
 * [B][H][m][d]; lse: DEVICE fp32 [B][H][m] or NULL; positions: DEVICE int32 [B] (t0_b >= 0, read
 * by the kernels; values that break the cache requirement above give keys outside the cache
 * window no weight but are not otherwise reported unless LONGATTN_DEBUG=1).  bf16 and fp32,
 * 1 <= d <= 256 with d % 8 == 0, 1 <= m <= 16.  Same alignment and error rules as
 * longattn_forward.  The workspace holds per-chunk partial results when the library splits a
 * window over several workgroups; its size depends on the shape (0 when one workgroup covers
 * each window; then it may be NULL), so ask longattn_decode_workspace_size.
 * --------------------------------------------------------------------------------------- */
typedef struct {
  int32_t batch, heads, d;
  int32_t dtype;               /* longattn_dtype of q, the caches and out                      */
  float scale;                 /* > 0 and finite                                                 */
  int32_t window;              /* keys per row, >= 1 (the row itself and window - 1 before it)  */
  int32_t n_queries;           /* m, new rows per sample                                         */
  int32_t cache_len;           /* slots per (b, h) in the caches                                 */
  int32_t ring;                /* 0: linear cache, 1: rolling buffer                             */
  const int32_t* positions;    /* DEVICE [batch]: position of each sample's first new row        */
} longattn_decode_desc;

longattn_status longattn_decode_workspace_size(const longattn_decode_desc* desc, size_t* bytes);
longattn_status longattn_decode(const longattn_decode_desc* desc, const void* q,
                                const void* k_cache, const void* v_cache, void* out, float* lse,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Static, human-readable name of a status code. */
const char* longattn_status_string(longattn_status status);

#ifdef __cplusplus
}
#endif

#endif /* LONGATTN_H */
