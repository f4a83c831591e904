/*
 * hstu.h -- C ABI of the MI355X (gfx950) HSTU layer forward library (libhstu.so).
 *
 * The layer is the one written in "Actions Speak Louder than Words" as retold on
 * chenhuiyu.github.io ("生成式推荐 16: HSTU", section "HSTU Layer 到底改了什么",
 * equations 1-3):
 *
 *     U, V, Q, K = Split(SiLU(f1(X)))                                   (1)
 *     A(X)V      = SiLU(Q K^T + rab^{p,t}) V      pointwise, no softmax  (2)
 *     Y          = f2(LayerNorm(A(X)V) * U)                              (3)
 *
 * computed on jagged batches at their true lengths (same page, section "另外三块拼图",
 * item 1) under a causal mask, or under the M-FALCON candidate mask (same section,
 * item 3; ltzyclt.github.io section 5.2).
 *
 * Conventions for every entry point
 *  - Pointers marked (device) are HIP device pointers; everything else is host memory
 *    read during the call only.  bf16 and fp16 tensors are passed as uint16_t bit
 *    patterns.
 *  - Precision: X, Y, w1 and w2 are bf16; the f1 output U|V|Q|K and the attention
 *    weights A are fp16 (same MFMA rate on gfx950, 3 more mantissa bits, which the layer
 *    needs to stay within 2e-2 / 2e-3 of an fp64 reference); every product accumulates
 *    in fp32.  f1 outputs saturate at +-65504.  A is rounded to fp16 as A / -ln 2 (the
 *    kernel's scaled domain), so a weight above 65504 ln 2 (about 45403) saturates at
 *    that value instead of overflowing.  The forward layer's f2 runs in fp16 as well:
 *    each head's attention output leaves the attention kernel normalised by that head's
 *    mean and standard deviation (fp16, magnitude at most sqrt(dv)), the f2 GEMM forms
 *    G = LayerNorm(AV) * U in fp16 while staging it (saturating at +-65504) and
 *    multiplies it by an fp16 copy of w2 made on each call (w2 entries below 2^-14 keep
 *    fewer significant bits there, entries above 65504 saturate).  hstu_layer_bwd forms
 *    its own G in bf16.
 *  - Row-major layouts.  Weights are "out x in": f1(X) = X w1^T + b1, f2(G) = G w2^T + b2.
 *  - U|V|Q|K layout of the f1 output: columns [0,H*dv) = U, [H*dv,2H*dv) = V,
 *    then H*dqk columns of Q and H*dqk of K; head h owns columns [h*dh,(h+1)*dh) of
 *    each block.
 *  - rab^{p,t}(i,j) = rab_pos[r][min(i-j, pos_buckets-1)]
 *                   + rab_time[r][min(time_buckets-1, floor(log2(1 + max(0, ts_i-ts_j))))]
 *    with r = h if rab_heads == num_heads else 0; the bias is added before SiLU.  The
 *    time gap is taken over the full int32 range without overflow.
 *  - Ownership: the caller owns every buffer.  The library allocates no device memory
 *    and keeps no pointer after a call returns; scratch memory comes from the caller's
 *    workspace (hstu_attn_fwd_noalloc: from a fixed static array, see there).  Calls are
 *    asynchronous on `stream` (a hipStream_t, NULL = default stream) and never
 *    synchronise, except hstu_validate_jagged.
 *  - Errors: host-checkable problems return a status before anything is launched and
 *    leave all outputs untouched; a failed launch returns HSTU_ERR_HIP and the HIP
 *    error code is available from hstu_last_hip_error().  No exception crosses the ABI.
 *  - Device-side jagged offsets are a precondition (0 = off[0] <= ... <= off[B] = T,
 *    max length <= max_seq_len); they are not re-validated on the hot path.  Use
 *    hstu_validate_jagged when in doubt.  Zero-length sequences are legal.
 *  - Token capacity: the forward entry points (hstu_layer_fwd, hstu_layer_fwd_train,
 *    hstu_layer_fwd_mfalcon, hstu_stack_fwd, hstu_stack_fwd_mfalcon, hstu_attn_fwd,
 *    hstu_attn_fwd_noalloc) also
 *    accept total_tokens above off[B], as a capacity: row buffers and workspaces are then
 *    sized for total_tokens rows, the kernels take the true count off[B] from the device,
 *    and output rows from off[B] on are left as they were.  A batch built on the device
 *    (hstu_stochastic_length) thus feeds a layer with no copy to the host: pass the raw
 *    token count as total_tokens and the raw max_seq_len (or the subsample length, if
 *    larger) as max_seq_len.  Work scales with off[B], not with the capacity.  The
 *    backward entry points need total_tokens == off[B].
 *  - Supported shapes: dqk == dv in {32, 64, 128}; 1 <= pos_buckets <= 1024;
 *    1 <= time_buckets <= 64; rab_heads 1 or num_heads.  The layer entry points also
 *    need d_model and num_heads*dv to be multiples of 64, d_model <= 2^21 and
 *    num_heads*dv <= 2048 (hstu_attn_fwd ignores d_model).
 */
#ifndef HSTU_H_
#define HSTU_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HSTU_OK = 0,
  HSTU_ERR_INVALID_ARG = 1, /* null pointer, negative size, inconsistent sizes        */
  HSTU_ERR_UNSUPPORTED = 2, /* shape outside the supported set listed above           */
  HSTU_ERR_WORKSPACE = 3,   /* workspace pointer null or smaller than required        */
  HSTU_ERR_HIP = 4          /* a HIP call or kernel launch failed                     */
} hstu_status_t;

typedef enum {
  /* Query i of a sequence (position n_p + i) sees every prefix key (positions
   * 0..n_p-1) and its own sequence's keys j <= i (positions n_p + j).             */
  HSTU_MASK_CAUSAL = 0,
  /* M-FALCON candidates: every query sits at position n_p, sees every prefix key
   * (the user's history) and itself (position gap 0, time gap 0), nothing else.   */
  HSTU_MASK_SELF_ONLY = 1
} hstu_mask_t;

typedef struct {
  int32_t d_model;      /* d: width of X and Y                                      */
  int32_t num_heads;    /* H                                                        */
  int32_t dqk;          /* per-head width of Q and K                                */
  int32_t dv;           /* per-head width of V and U                                */
  int32_t pos_buckets;  /* entries per row of rab_pos (64 in the configs)           */
  int32_t time_buckets; /* entries per row of rab_time (32 in the configs)          */
  int32_t rab_heads;    /* rows of each rab table: 1 (shared) or num_heads          */
  float ln_eps;         /* LayerNorm epsilon (1e-5)                                 */
} hstu_dims_t;

typedef struct {
  const uint16_t *w1;      /* (device) bf16 [2H(dv+dqk)][d]                         */
  const float *b1;         /* (device) [2H(dv+dqk)] or NULL (no bias)               */
  const uint16_t *w2;      /* (device) bf16 [d][H*dv]                               */
  const float *b2;         /* (device) [d] or NULL                                  */
  const float *ln_gamma;   /* (device) [H*dv] or NULL (= 1)                          */
  const float *ln_beta;    /* (device) [H*dv] or NULL (= 0)                          */
  const float *rab_pos;    /* (device) [rab_heads][pos_buckets] or NULL (no term)   */
  const float *rab_time;   /* (device) [rab_heads][time_buckets] or NULL (no term)  */
} hstu_weights_t;

typedef struct {
  int32_t batch;              /* B >= 0                                                */
  int32_t total_tokens;       /* T = seq_offsets[B] (host copy), or a capacity above   */
                              /* it for the forward entry points (see above)           */
  int32_t max_seq_len;        /* upper bound on every sequence length (host)           */
  const int32_t *seq_offsets; /* (device) [B+1], non-decreasing, off[0] = 0            */
  const int32_t *timestamps;  /* (device) [T] or NULL (time term off)                  */
} hstu_jagged_t;

/* Keys that precede each sequence's own tokens: the M-FALCON user history.  Sequence
 * b of the query batch sees rows [seq->seq_offsets[b], seq->seq_offsets[b+1]) of k/v. */
typedef struct {
  const hstu_jagged_t *seq;   /* same batch size as the query batch                   */
  const uint16_t *k;          /* (device) fp16, row r at k + r*row_stride               */
  const uint16_t *v;          /* (device) fp16, row r at v + r*row_stride               */
  int64_t row_stride;         /* elements between consecutive rows; must equal the     */
                              /* candidates' row_stride (else HSTU_ERR_UNSUPPORTED)    */
} hstu_prefix_t;

/* Workspace (bytes) needed by hstu_layer_fwd / hstu_layer_fwd_mfalcon for this batch;
 * 0 when the arguments are invalid.  Alignment: 256 bytes.                           */
size_t hstu_layer_workspace_bytes(const hstu_dims_t *dims, const hstu_jagged_t *seq);

/* Workspace (bytes) needed by hstu_layer_fwd_mfalcon for this history and candidate
 * micro-batch; 0 when the arguments are invalid.                                    */
size_t hstu_mfalcon_workspace_bytes(const hstu_dims_t *dims, const hstu_jagged_t *hist,
                                    const hstu_jagged_t *cand);

/* Workspace (bytes) needed by hstu_attn_fwd (jagged tile schedule and key-block
 * timestamp ranges); prefix_seq is the prefix batch or NULL.                        */
size_t hstu_attn_workspace_bytes(const hstu_dims_t *dims, const hstu_jagged_t *seq,
                                 const hstu_jagged_t *prefix_seq);

/* One HSTU layer, equations (1)-(3), causal mask.
 *   x    (device) bf16 [T][d]                       input rows
 *   y    (device) bf16 [T][d]                       output rows (may not alias x)
 *   uvqk (device) fp16 [T][2H(dv+dqk)]              f1 output, written; the caller may
 *                                                   keep it as the K/V cache of an
 *                                                   M-FALCON history
 *   ws   (device) workspace of ws_bytes >= hstu_layer_workspace_bytes(dims, seq)    */
hstu_status_t hstu_layer_fwd(const hstu_dims_t *dims, const hstu_weights_t *w,
                             const hstu_jagged_t *seq, const uint16_t *x, uint16_t *y,
                             uint16_t *uvqk, void *ws, size_t ws_bytes, void *stream);

/* M-FALCON candidate micro-batch (ltzyclt.github.io section 5.2): f1 on the candidate
 * rows, then each candidate of user b attends to the cached K/V of that user's history
 * (hist_uvqk, the uvqk buffer written by hstu_layer_fwd on the history batch `hist`)
 * and to itself only, then LayerNorm, gate and f2.  cand->timestamps are the
 * candidates' request times.  The results of one candidate do not depend on which
 * other candidates share its micro-batch.
 *   hist_uvqk (device) fp16 [T_hist][2H(dv+dqk)]
 *   x_cand    (device) bf16 [T_cand][d];   y_cand (device) bf16 [T_cand][d]
 *   uvqk_cand (device) fp16 [T_cand][2H(dv+dqk)]
 *   ws        >= hstu_mfalcon_workspace_bytes(dims, hist, cand)                      */
hstu_status_t hstu_layer_fwd_mfalcon(const hstu_dims_t *dims, const hstu_weights_t *w,
                                     const hstu_jagged_t *hist, const uint16_t *hist_uvqk,
                                     const hstu_jagged_t *cand, const uint16_t *x_cand,
                                     uint16_t *y_cand, uint16_t *uvqk_cand, void *ws,
                                     size_t ws_bytes, void *stream);

/* Workspace (bytes) of hstu_stack_fwd / hstu_stack_fwd_mfalcon: a layer's workspace
 * plus one [T][d] bf16 activation buffer; 0 when the arguments are invalid.          */
size_t hstu_stack_workspace_bytes(const hstu_dims_t *dims, const hstu_jagged_t *seq);
size_t hstu_stack_mfalcon_workspace_bytes(const hstu_dims_t *dims, const hstu_jagged_t *hist,
                                          const hstu_jagged_t *cand);

/* A stack of n_layers causal layers (the deep configurations of chenhuiyu.github.io,
 * section on experiments, go to 24 layers): layer l maps X_l to X_{l+1} with its own
 * weights w[l]; X_0 = x and the last layer's output is written to y.  Every layer is
 * computed exactly as hstu_layer_fwd would (the results are bit-identical to n_layers
 * such calls); the batch's tile schedule and key-block timestamp ranges are built once.
 *   w           (host) array of n_layers weight sets
 *   x, y        (device) bf16 [T][d]; y may not alias x (x is not written)
 *   uvqk        (device) fp16: [T][2H(dv+dqk)] reused by every layer when keep_caches is
 *               0, or [n_layers][T][2H(dv+dqk)] keeping every layer's U|V|Q|K when it is
 *               1 (the per-layer K/V caches of an M-FALCON history)
 *   ws          >= hstu_stack_workspace_bytes(dims, seq)                              */
hstu_status_t hstu_stack_fwd(const hstu_dims_t *dims, int32_t n_layers, const hstu_weights_t *w,
                             const hstu_jagged_t *seq, const uint16_t *x, uint16_t *y,
                             uint16_t *uvqk, int32_t keep_caches, void *ws, size_t ws_bytes,
                             void *stream);

/* M-FALCON serving through a stack (chenhuiyu.github.io, section "另外三块拼图", item 3;
 * ltzyclt.github.io section 5.2): a candidate micro-batch goes through all n_layers
 * layers, each attending to that layer's cached history K/V and to itself.  Layer l is
 * computed exactly as hstu_layer_fwd_mfalcon would with hist_uvqk + l*T_hist*2H(dv+dqk).
 *   hist_uvqk   (device) fp16 [n_layers][T_hist][2H(dv+dqk)], written by hstu_stack_fwd on
 *               the history batch with keep_caches = 1 and the same weights
 *   x_cand, y_cand (device) bf16 [T_cand][d], no aliasing
 *   uvqk_cand   (device) fp16 [T_cand][2H(dv+dqk)] scratch
 *   ws          >= hstu_stack_mfalcon_workspace_bytes(dims, hist, cand)                */
hstu_status_t hstu_stack_fwd_mfalcon(const hstu_dims_t *dims, int32_t n_layers,
                                     const hstu_weights_t *w, const hstu_jagged_t *hist,
                                     const uint16_t *hist_uvqk, const hstu_jagged_t *cand,
                                     const uint16_t *x_cand, uint16_t *y_cand, uint16_t *uvqk_cand,
                                     void *ws, size_t ws_bytes, void *stream);

/* Equation (2) alone: out[t][h*dv + f] = sum_j SiLU(q_t.k_j + rab(t,j)) v_j[f] over the
 * keys allowed by `mask` (see hstu_mask_t), fp32, no normalisation.
 *   q, k, v (device) fp16; row t of head h at q + t*row_stride + h*dqk (same for k,v
 *           with dqk / dv)
 *   prefix  NULL or the keys preceding each sequence (required for SELF_ONLY)
 *   out     (device) fp32 [T][H*dv], every row below off[B] written
 *   ws      >= hstu_attn_workspace_bytes(dims, seq, prefix ? prefix->seq : NULL)     */
hstu_status_t hstu_attn_fwd(const hstu_dims_t *dims, const float *rab_pos,
                            const float *rab_time, const hstu_jagged_t *seq,
                            const uint16_t *q, const uint16_t *k, const uint16_t *v,
                            int64_t row_stride, const hstu_prefix_t *prefix,
                            hstu_mask_t mask, float *out, void *ws, size_t ws_bytes,
                            void *stream);

/* For callers that cannot allocate memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): hstu_attn_fwd with the same
 * arguments and results (the same kernels, bit for bit) but no workspace argument.
 * Its scratch (the jagged tile schedule and the key-block timestamp ranges) lives in a
 * static device array of hstu_attn_noalloc_max_scratch_bytes() bytes (16 MiB), one copy
 * per GPU, held from its first use until the process ends; the call uses the copy of
 * the current device (the stream must belong to it).  It calls no hipMalloc, hipFree
 * or allocating routine.  A batch whose scratch, hstu_attn_workspace_bytes(dims, seq,
 * prefix seq), exceeds that size returns HSTU_ERR_WORKSPACE before any launch (about
 * two million tokens, batch and prefix together).  Every call on one GPU shares that
 * GPU's array and rewrites it before reading it: calls that overlap in time on one GPU
 * (for instance on two streams) race and must not be issued.                        */
size_t hstu_attn_noalloc_max_scratch_bytes(void);
hstu_status_t hstu_attn_fwd_noalloc(const hstu_dims_t *dims, const float *rab_pos,
                                    const float *rab_time, const hstu_jagged_t *seq,
                                    const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                    int64_t row_stride, const hstu_prefix_t *prefix,
                                    hstu_mask_t mask, float *out, void *stream);

/* Workspace (bytes) needed by hstu_stochastic_length for this raw batch (256-byte
 * aligned); 0 when the batch description is invalid.                               */
size_t hstu_sl_workspace_bytes(const hstu_jagged_t *raw);

/* Stochastic Length (ltzyclt.github.io section 5.1; chenhuiyu.github.io section
 * "另外三块拼图", item 2): subsamples each user's raw sequence before the layer.
 * With L = floor(n_target^(alpha/2)) (fp64), user b of length n keeps all n tokens when
 * n <= L or u_keep[b] < n_target^alpha / n^2 (fp64 compare); otherwise it keeps the L
 * tokens whose (keys[t], position) pairs are smallest, in time order.  The random draws
 * are inputs, so the result is a deterministic function of them.
 *   raw          the raw batch (raw->timestamps may be NULL unless new_ts is given)
 *   u_keep       (device) fp64 [B], uniform draws in [0, 1), one per user (may be
 *                NULL when B == 0)
 *   keys         (device) uint32 [T_raw], one priority per raw token
 *   n_target     N >= 1 (4096 in the configs); alpha > 0 (1.6)
 *   kept         (device) int32 [T_raw]: written with the raw indices of the kept tokens
 *                in batch order, entries [0, new_offsets[B]); later entries untouched
 *   new_offsets  (device) int32 [B+1], written (new_offsets[0] = 0)
 *   new_ts       (device) int32 [T_raw] or NULL: timestamps of the kept tokens
 *   x_raw, x_out (device) both NULL, or raw rows [T_raw][row_elems] and kept rows
 *                [T_raw][row_elems] (16-bit values, copied bit for bit); row_elems a
 *                multiple of 8, both 16-byte aligned, no aliasing
 *   ws           >= hstu_sl_workspace_bytes(raw) (may be NULL when B == 0)
 * The new batch's total token count is new_offsets[B] on the device; its longest
 * sequence is at most max(L, raw->max_seq_len).  Invalid arguments (including N^alpha
 * or L outside fp64 / int32 range, L < 1) return HSTU_ERR_INVALID_ARG before any
 * launch.                                                                          */
hstu_status_t hstu_stochastic_length(const hstu_jagged_t *raw, const double *u_keep,
                                     const uint32_t *keys, int32_t n_target, double alpha,
                                     int32_t *kept, int32_t *new_offsets, int32_t *new_ts,
                                     const uint16_t *x_raw, uint16_t *x_out, int64_t row_elems,
                                     void *ws, size_t ws_bytes, void *stream);

/* Workspace (bytes) of hstu_attn_bwd: hstu_attn_bwd_workspace_bytes for the faster path,
 * which keeps dS (fp16, 2 KB per 32 x 32 block of each causal triangle and head: 4.3 GB
 * at 8 x 8192 tokens and 8 heads) so that dQ needs no second pass over the scores; it
 * equals the minimum when that buffer would exceed 32 GiB.  A workspace of at least
 * hstu_attn_bwd_min_workspace_bytes but less than the first runs the path that forms
 * dS twice.  Both give the same results to rounding.  0 when the arguments are invalid. */
size_t hstu_attn_bwd_workspace_bytes(const hstu_dims_t *dims, const hstu_jagged_t *seq);
size_t hstu_attn_bwd_min_workspace_bytes(const hstu_dims_t *dims, const hstu_jagged_t *seq);

/* Gradients of equation (2) (the causal attention computed by hstu_attn_fwd without a
 * prefix) for the upstream gradient d_out of its output:
 *     dA = dO V^T, dS = dA * SiLU'(S) on allowed pairs (0 elsewhere), dQ = dS K,
 *     dK = dS^T Q, dV = A^T dO,  with S = Q K^T + rab, A = SiLU(S).
 * With d_rab_pos / d_rab_time (device fp32, the shape of the table: [rab_heads][buckets]),
 * the tables' gradients too: the sum of dS over the allowed pairs of each bucket (over
 * all heads when the table is shared).  Either may be NULL (not formed); each must be
 * NULL when its table is.  An empty batch sets them to 0.  Every row of dq, dk and dv is
 * written.  dq, dk and dv are deterministic (fixed summation orders); the tables' sums
 * add per wave in LDS with atomics, so their order between a wave's lanes is the
 * hardware's and two calls agree to rounding, not necessarily bit for bit.
 *   q, k, v    (device) fp16, as for hstu_attn_fwd (row_stride elements between rows)
 *   d_out      (device) fp32 [T][H*dv]; rounded to fp16 for the matrix products
 *   dq, dk, dv (device) fp32 [T][H*dqk], [T][H*dqk], [T][H*dv]
 *   ws         >= hstu_attn_bwd_min_workspace_bytes(dims, seq); with
 *              hstu_attn_bwd_workspace_bytes(dims, seq) bytes the faster path runs
 * The caller owns every buffer.  HSTU_ERR_INVALID_ARG for a null or misaligned pointer,
 * an output equal to another output or to an input, or row_stride < H*dqk or not a
 * multiple of 8; HSTU_ERR_UNSUPPORTED for dqk != dv or dqk not in {32, 64, 128};
 * HSTU_ERR_WORKSPACE for a workspace below the minimum or misaligned.  An empty batch
 * launches nothing but the zeroing of the table gradients.                          */
hstu_status_t hstu_attn_bwd(const hstu_dims_t *dims, const float *rab_pos,
                            const float *rab_time, const hstu_jagged_t *seq,
                            const uint16_t *q, const uint16_t *k, const uint16_t *v,
                            int64_t row_stride, const float *d_out, float *dq, float *dk,
                            float *dv, float *d_rab_pos, float *d_rab_time, void *ws,
                            size_t ws_bytes, void *stream);

/* Gradients of the layer's parameters: device fp32 buffers owned by the caller, in the
 * layouts of hstu_weights_t.  A NULL entry is not formed.                            */
typedef struct {
  float *w1;        /* [2H(dv+dqk)][d], required                                       */
  float *b1;        /* [2H(dv+dqk)]: gradient of a bias added after f1 (also when the  */
                    /* weights have none) or NULL                                      */
  float *w2;        /* [d][H*dv], required                                             */
  float *b2;        /* [d] or NULL, likewise                                           */
  float *ln_gamma;  /* [H*dv] or NULL; must be NULL when the weights have no ln_gamma  */
  float *ln_beta;   /* [H*dv] or NULL; must be NULL when the weights have no ln_beta   */
  float *rab_pos;   /* [rab_heads][pos_buckets] or NULL; NULL when the table is        */
  float *rab_time;  /* [rab_heads][time_buckets] or NULL; likewise                     */
} hstu_layer_grads_t;

/* Workspace (bytes) of hstu_layer_bwd, as for hstu_attn_bwd: the first enables the
 * stored-dS path of the attention gradient, the second is the minimum.  0 when the
 * arguments are invalid.                                                              */
size_t hstu_layer_bwd_workspace_bytes(const hstu_dims_t *dims, const hstu_jagged_t *seq);
size_t hstu_layer_bwd_min_workspace_bytes(const hstu_dims_t *dims, const hstu_jagged_t *seq);

/* Backward of one causal layer (equations 1-3) for the upstream gradient d_y of its
 * output: dX and the parameter gradients, by the chain rule through f2, the U gate,
 * LayerNorm, the pointwise attention (as hstu_attn_bwd), SiLU and f1.  The forward
 * pieces it needs (Z = X w1^T + b1, U|V|Q|K, the attention output) are recomputed from
 * x, so the forward keeps no activations for it.  Matrix products take bf16 operands
 * (dY, G = LayerNorm(O) U and dZ rounded to bf16; the attention's as in hstu_attn_bwd)
 * with fp32 accumulation; every result is fp32 and repeats bit for bit, except the
 * bias-table gradients, which repeat to rounding only (as in hstu_attn_bwd).
 *   x    (device) bf16 [T][d], the layer input
 *   d_y  (device) fp32 [T][d];   d_x (device) fp32 [T][d]
 *   grads: see hstu_layer_grads_t; an empty batch sets every formed gradient to 0.
 * HSTU_ERR_INVALID_ARG for a null or misaligned pointer, d_x equal to another buffer,
 * a required gradient missing or a gradient asked for a parameter the weights lack;
 * otherwise the shape rules and errors of hstu_layer_fwd.                            */
hstu_status_t hstu_layer_bwd(const hstu_dims_t *dims, const hstu_weights_t *w,
                             const hstu_jagged_t *seq, const uint16_t *x, const float *d_y,
                             float *d_x, const hstu_layer_grads_t *grads, void *ws,
                             size_t ws_bytes, void *stream);

/* The forward of hstu_layer_fwd for training (same arguments, results and errors), which
 * also hands the caller what hstu_layer_bwd_saved reuses instead of recomputing: the
 * attention output of equation 2 for each row and head, as it enters the LayerNorm of
 * equation 3 ("Actions Speak Louder than Words" as retold on chenhuiyu.github.io,
 * section "HSTU Layer 到底改了什么"), in the parts the layer itself keeps.
 *   cn    (device) fp16 [T][H*dv]: each head's dv outputs standardised over that head,
 *                  (o - mean) / sqrt(var) (0 when var = 0), |value| <= sqrt(dv)
 *   stats (device) fp32 [T][H][2]: (mean, biased variance) of those dv outputs, so that
 *                  o = cn * sqrt(var) + mean
 * cn, stats may not alias y, uvqk or each other (HSTU_ERR_INVALID_ARG).            */
hstu_status_t hstu_layer_fwd_train(const hstu_dims_t *dims, const hstu_weights_t *w,
                                   const hstu_jagged_t *seq, const uint16_t *x, uint16_t *y,
                                   uint16_t *uvqk, uint16_t *cn, float *stats, void *ws,
                                   size_t ws_bytes, void *stream);

/* hstu_layer_bwd with the activations that hstu_layer_fwd_train wrote for the same x,
 * weights and batch (uvqk, cn, stats as documented there): U|V|Q|K and the attention
 * output are read instead of recomputed; only Z = X w1^T + b1 (for SiLU') is formed
 * again.  The gradients are those of the forward as it ran (its fp16 U|V|Q|K and
 * standardised output), so they differ from hstu_layer_bwd's, which rebuilds both from
 * x, by rounding only.  Same workspace, other arguments and errors as hstu_layer_bwd;
 * uvqk, cn, stats may not alias d_x or a gradient (HSTU_ERR_INVALID_ARG).            */
hstu_status_t hstu_layer_bwd_saved(const hstu_dims_t *dims, const hstu_weights_t *w,
                                   const hstu_jagged_t *seq, const uint16_t *x,
                                   const uint16_t *uvqk, const uint16_t *cn, const float *stats,
                                   const float *d_y, float *d_x, const hstu_layer_grads_t *grads,
                                   void *ws, size_t ws_bytes, void *stream);

/* Debug check of device offsets: off[0] == 0, non-decreasing, off[B] <= total_tokens
 * (equal, unless total_tokens is meant as a capacity), every length <= max_seq_len.
 * Synchronises the stream.  Returns HSTU_OK or HSTU_ERR_INVALID_ARG.                  */
hstu_status_t hstu_validate_jagged(const hstu_jagged_t *seq, void *stream);

/* Static description of a status code.                                              */
const char *hstu_status_str(hstu_status_t status);

/* HIP error code of the last HSTU_ERR_HIP returned on this thread (0 if none).       */
int hstu_last_hip_error(void);

/* Optional per-kernel timing with HIP events on the launch stream (off by default).
 * `on` is a bitmask of kernel ids (bit k: kernel id k; -1: all, 0: none).  Every launch
 * of a selected kernel is bracketed by two events on its stream; the durations are
 * collected by hstu_profile_collect, which synchronises the events.  Each event pair adds
 * a little time between launches, so a timed run can select only the kernel it reports.
 * Kernel ids: 0 schedule and key-block timestamp ranges, 1 f1 GEMM (with the f2 operand
 * preparation, w2, gamma and beta to fp16, that runs in the same launch or right after
 * it), 2 attention, 3 reserved (no launch records under it), 4 f2 GEMM with the
 * LayerNorm and the U gate formed in its operand staging.                            */
void hstu_profile_enable(int on);
void hstu_profile_reset(void);
/* Adds up finished records: total_ms[k] and launches[k] for k in [0, 5).           */
hstu_status_t hstu_profile_collect(double *total_ms, int64_t *launches);
const char *hstu_kernel_name(int kernel_id);
/* Average shader (core) clock in GHz over the lifetimes of the first 64 workgroups of
 * every attention launch that ran inside a layer while the attention (id 2) was profiled
 * since the last hstu_profile_reset (the core clock counter against the 100 MHz real-time
 * counter, both added up over those launches), 0 if none.  The sums are plain adds: two
 * profiled attention launches running at once on different streams may lose samples.
 * Synchronises the device.                                                            */
hstu_status_t hstu_profile_clock_ghz(double *ghz);

#ifdef __cplusplus
}
#endif

#endif /* HSTU_H_ */
