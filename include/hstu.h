/*
 * hstu.h — C ABI of libhstu: the HSTU layer forward over jagged sequences on
 * AMD MI355X (gfx950).
 *
 * What is computed (sources cited by page title and section):
 *   [SRM] "4.4 Scaling Recommendation Models", section "Generative
 *         Recommenders and HSTU" — the layer's three equations:
 *           U, V, Q, K = Split(SiLU(f1(X)))
 *           AV         = SiLU(Q K^T + rab^{p,t}) V      (pointwise, no softmax)
 *           Y          = f2(Norm(AV) * U)
 *         the bullets under them (SiLU weights with a constant normaliser such
 *         as the sequence length; bias from position and time difference), the
 *         "Efficiency tricks" paragraph (variable-length sequences; candidates
 *         appended to the history see the history but not one another), and
 *         section "Code" (LayerNorm before f1, u|v|q|k chunk order, lower
 *         triangular mask with the diagonal, division by n, LayerNorm over the
 *         merged heads, gate by u, f2, residual add).
 *   [FRC] "HSTU: The First Exploration of the Scaling Law", 7.1.4 Innovations
 *         1-2 (LayerNorm(AV) * U; bias on p_i - p_j and t_i - t_j) and 7.1.5
 *         M-FALCON layer 1 (batched candidates under a mask).
 *
 * Per sequence b with L_b tokens whose last m_b are candidates
 * (n_b = L_b - m_b history tokens), local query i, key j:
 *   x~      = LayerNorm_in(x)                   if HSTU_INPUT_NORM, else x
 *   u|v|q|k = SiLU(x~ W1^T + b1)                split in that order; head h owns
 *                                               columns h*dh .. h*dh+dh-1 of a block
 *   M_ij    = (j <= i) && (j < n_b || j == i)
 *   p(i)    = min(i, n_b) if HSTU_CAND_SHARED_POS else i
 *   bp      = clamp(p(i) - p(j), -R, R) + R,     R = (pos_buckets - 1) / 2
 *   dt      = ts[i] - ts[j]  (int64 seconds, two's-complement wrap)
 *   bt      = dt <= 0 ? 0 : min(NB - 1, 1 + (k << s) + sub),  k = floor(log2 dt),
 *             sub = the s = time_sub_bits bits right below dt's leading one
 *   rab     = pos[h][bp] + time[h][bt] (+ type[h][ty(i)][ty(j)] if num_types > 0)
 *   AV_i^h  = (1/N_b) sum_j M_ij SiLU(q_i^h . k_j^h + rab) v_j^h
 *             N_b = L_b, or norm_len when norm_len > 0 (no 1/sqrt(d) scale)
 *   Z       = LayerNorm_av(concat_h AV^h) * u   (over H*dv, biased variance)
 *   Y       = Z W2^T + b2 (+ x if HSTU_RESIDUAL)
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller; the library keeps
 *     none after returning and allocates no device memory (scratch comes from
 *     the caller's workspace).
 *   - Work is enqueued on `stream` and runs asynchronously.  The returned status
 *     covers host-side validation and launch errors only; faults inside kernels
 *     surface at the caller's next synchronisation.
 *   - Errors: a non-HSTU_OK status leaves every output untouched (validation
 *     happens before any launch); hstu_last_error() returns a thread-local
 *     message describing the last failure on the calling thread.
 *   - Thread-safe and stateless: concurrent calls on different streams with
 *     disjoint outputs and workspaces are independent.
 *   - Floating tensors (x, out, weights, LayerNorm parameters, bias tables) all
 *     have the layer dtype; offsets and timestamps are int64, candidate counts
 *     int32.  Floating tensors must be 16-byte aligned, int64 arrays 8-byte,
 *     int32 arrays 4-byte.
 *   - Device-side robustness: offsets are clamped to [0, T] and made
 *     non-decreasing, candidate counts to [0, L_b], so malformed metadata
 *     cannot cause out-of-bounds accesses (the result is then unspecified).
 *     HSTU_VALIDATE checks them exactly instead (it synchronises the stream).
 */
#ifndef HSTU_H_
#define HSTU_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hstu_stream_t; /* a hipStream_t; NULL = default stream */

typedef enum {
  HSTU_OK = 0,
  HSTU_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size, bad metadata */
  HSTU_ERR_UNSUPPORTED = 2, /* a dimension or dtype this build has no kernel for */
  HSTU_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
  HSTU_ERR_DEVICE = 4       /* a HIP launch or copy returned an error */
} hstu_status;

typedef enum { HSTU_F32 = 0, HSTU_BF16 = 1 } hstu_dtype;

enum {
  HSTU_INPUT_NORM = 1u << 0,      /* LayerNorm on x before f1 ([SRM] "Code")        */
  HSTU_RESIDUAL = 1u << 1,        /* Y += x ([SRM] "Code")                           */
  HSTU_CAND_SHARED_POS = 1u << 2, /* candidates all take position n_b (M-FALCON)     */
  HSTU_VALIDATE = 1u << 3,        /* copy metadata to the host, check, synchronise   */
  HSTU_REUSE_PLAN = 1u << 4,      /* attention plan already in the workspace (below) */
  HSTU_SAVED_FWD = 1u << 5        /* hstu_layer_bwd: forward activations already in the
                                     workspace, from hstu_layer_fwd_train (below)     */
};

/* HSTU_REUSE_PLAN: the attention work list and the per-key-block timestamp
 * summary in the workspace depend only on seq_offsets, num_candidates,
 * timestamps, batch and total_tokens.  With this flag hstu_layer_fwd and
 * hstu_attn_fwd skip rebuilding them: the caller asserts that an earlier call
 * enqueued on the same stream, with the same workspace and the same metadata,
 * built them (e.g. every layer after the first of a stack).  With other
 * metadata the results are wrong but every access stays in bounds.          */

typedef struct {
  int32_t d_model;       /* model width d; multiple of 32, 32..8192            */
  int32_t num_heads;     /* H; 1..64                                           */
  int32_t dqk;           /* query/key width per head: 32, 64 or 128            */
  int32_t dv;            /* value width per head: 32, 64 or 128                */
  int32_t pos_buckets;   /* P, odd, 1..2047; R = (P-1)/2                        */
  int32_t time_buckets;  /* NB, 1..2048                                         */
  int32_t time_sub_bits; /* s, 0..4                                             */
  hstu_dtype dtype;      /* arithmetic/storage type of every floating tensor    */
  uint32_t flags;        /* HSTU_* bits                                         */
  float ln_eps;          /* LayerNorm epsilon (> 0), e.g. 1e-5                  */
  int32_t norm_len;      /* 0: divide by L_b; > 0: divide by this constant      */
  int32_t num_types;     /* 0: no token-type term; 1..16: token types (below)  */
} hstu_desc;

/* Layer parameters, nn.Linear layouts (row n of W is output feature n).      */
typedef struct {
  const void* w1;      /* [2H(dqk+dv), d]: rows U | V | Q | K, heads contiguous */
  const void* b1;      /* [2H(dqk+dv)]                                          */
  const void* w2;      /* [d, H*dv]                                             */
  const void* b2;      /* [d]                                                   */
  const void* ln_in_g; /* [d]    gain of the input LayerNorm (HSTU_INPUT_NORM)  */
  const void* ln_in_b; /* [d]    offset of the input LayerNorm                  */
  const void* ln_av_g; /* [H*dv] gain of the LayerNorm over the merged heads    */
  const void* ln_av_b; /* [H*dv] offset                                         */
} hstu_weights;

/* Relative-attention-bias tables.  Entry (h, idx) is at ptr[h*stride + idx];
 * a head stride of 0 shares one table across heads.
 *
 * Token-type term ([FRC] 7.1.4 Innovation 2: the bias also depends on the
 * two tokens' types, e.g. content and action tokens), used when
 * desc->num_types = NT > 0: the bias gains type[h*type_head_stride + a*NT + b]
 * for a query of type a and a key of type b.  token_types gives each row's
 * type (uint8, values >= NT are taken as NT - 1); in hstu_cand_fwd it holds
 * the candidates' types and hist_types the cached history rows' types.  All
 * type fields are ignored when num_types = 0.                               */
typedef struct {
  const void* pos;   /* >= [P]  position-difference table                      */
  const void* time;  /* >= [NB] log-bucketed time-difference table             */
  int32_t pos_head_stride;
  int32_t time_head_stride;
  const void* type;  /* >= [NT * NT] token-type table (layer dtype)            */
  int32_t type_head_stride;       /* 0, or >= NT * NT                          */
  int32_t reserved;               /* must be 0                                 */
  const uint8_t* token_types;     /* [T] (query rows)                          */
  const uint8_t* hist_types;      /* [Th] hstu_cand_fwd only                   */
} hstu_bias_tables;

/* Intermediate activations, the hand-off between the three stages.          */
typedef struct {
  void* u;         /* [T, H*dv]  gate                                          */
  void* v;         /* [H, T, dv] values, head-major                            */
  void* q;         /* [H, T, dqk]                                              */
  void* k;         /* [H, T, dqk]                                              */
  void* av;        /* [T, H*dv]  AV^h minus its mean over dv (per row, head)   */
  float* av_stats; /* [T, H, 2]  fp32 mean over dv and sum of squared
                      deviations over dv of AV^h, per (row, head)             */
} hstu_activations;

/* Bytes of workspace hstu_layer_fwd needs for T tokens in B sequences.       */
size_t hstu_workspace_size(const hstu_desc* desc, int64_t total_tokens, int32_t batch);

/* The layer forward ([SRM] three equations, "Code" sketch; [FRC] 7.1.4-7.1.5).
 *   x               [T, d]   input rows, sequences packed back to back
 *   seq_offsets     [B+1]    int64; sequence b owns rows off[b] .. off[b+1]-1,
 *                            off[0] = 0, off[B] = T; empty sequences allowed
 *   timestamps      [T]      int64 seconds
 *   num_candidates  [B]      int32 trailing candidate tokens per sequence, or
 *                            NULL for none (pure causal)
 *   out             [T, d]   may alias x
 *   workspace       >= hstu_workspace_size(desc, T, B) bytes, 256-aligned
 * Returns HSTU_OK after enqueuing all kernels on `stream`.                    */
hstu_status hstu_layer_fwd(const hstu_desc* desc, const void* x, const int64_t* seq_offsets,
                           int32_t batch, int64_t total_tokens, const int64_t* timestamps,
                           const int32_t* num_candidates, const hstu_weights* weights,
                           const hstu_bias_tables* tables, void* out, void* workspace,
                           size_t workspace_bytes, hstu_stream_t stream);

/* hstu_layer_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels on the same arguments, with the workspace taken from a
 * library-owned device array of HSTU_NOALLOC_SCRATCH_BYTES per GPU instead of
 * a caller buffer.  The array is found once per device, on the first call with
 * that device current, and is held until the process ends.  Calls with
 * hstu_workspace_size(desc, T, B) above the limit return HSTU_ERR_WORKSPACE;
 * HSTU_VALIDATE (which copies to the host and synchronises) is rejected with
 * HSTU_ERR_INVALID_ARG.  Nothing is allocated.  All calls on one GPU share
 * that GPU's array: calls whose work overlaps on one GPU (two streams, two
 * threads) race and give wrong results; calls enqueued one after another on
 * one stream are safe.  HSTU_REUSE_PLAN reuses the plan of the previous call
 * on the same GPU.                                                          */
#define HSTU_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
hstu_status hstu_layer_fwd_noalloc(const hstu_desc* desc, const void* x, const int64_t* seq_offsets,
                                   int32_t batch, int64_t total_tokens, const int64_t* timestamps,
                                   const int32_t* num_candidates, const hstu_weights* weights,
                                   const hstu_bias_tables* tables, void* out, hstu_stream_t stream);

/* Stage 1 ([SRM] first equation and the "Code" LayerNorm before f1): input
 * LayerNorm, f1, SiLU, split into acts->u, v, q, k.  Needs
 * hstu_proj_workspace_size() bytes of workspace (the normalised x).          */
size_t hstu_proj_workspace_size(const hstu_desc* desc, int64_t total_tokens);
hstu_status hstu_proj_fwd(const hstu_desc* desc, const void* x, int64_t total_tokens,
                          const hstu_weights* weights, const hstu_activations* acts,
                          void* workspace, size_t workspace_bytes, hstu_stream_t stream);

/* Stage 2 ([SRM] second equation and bullets; [FRC] 7.1.4 Innovations 1-2,
 * 7.1.5 candidate mask): reads acts->q, k, v; writes acts->av and
 * acts->av_stats.  Needs hstu_attn_workspace_size() bytes (the work list and
 * a per-key-block summary of the timestamps), 256-aligned.                   */
size_t hstu_attn_workspace_size(const hstu_desc* desc, int64_t total_tokens, int32_t batch);
hstu_status hstu_attn_fwd(const hstu_desc* desc, const int64_t* seq_offsets, int32_t batch,
                          int64_t total_tokens, const int64_t* timestamps,
                          const int32_t* num_candidates, const hstu_bias_tables* tables,
                          const hstu_activations* acts, void* workspace, size_t workspace_bytes,
                          hstu_stream_t stream);

/* Stage 3a ([SRM] third equation, "Code" LayerNorm over the merged heads
 * then multiplication by u; [FRC] 7.1.4 LayerNorm(AV) * U): reads acts->u,
 * av, av_stats and weights->ln_av_g / ln_av_b; writes
 * z = (LayerNorm(AV) * ln_av_g + ln_av_b) * U, [T, H*dv] in the layer dtype,
 * row-major, caller-owned device memory, 16-byte aligned.                    */
hstu_status hstu_gate_fwd(const hstu_desc* desc, int64_t total_tokens, const hstu_weights* weights,
                          const hstu_activations* acts, void* z, hstu_stream_t stream);

/* Stage 3 ([SRM] third equation, "Code" LayerNorm over merged heads, gate,
 * f2, residual; [FRC] 7.1.4 LayerNorm(AV) * U): reads acts->u, av, av_stats
 * (and x for the residual); writes the gated normalised tensor
 * z [T, H*dv] (layer dtype, row-major, caller-owned device memory, 16-byte
 * aligned, required: it is the f2 GEMM's operand and stays readable
 * afterwards) and out [T, d].  out may alias x; z must not overlap any other
 * argument.                                                                  */
hstu_status hstu_out_fwd(const hstu_desc* desc, const void* x, int64_t total_tokens,
                         const hstu_weights* weights, const hstu_activations* acts, void* out,
                         void* z, hstu_stream_t stream);

/* Candidate pass against cached history ([FRC] 7.1.5 M-FALCON; [SRM]
 * "Efficiency tricks": candidates see the history and themselves, not one
 * another).  A candidate's output row depends only on its own row, the
 * history's K and V and its metadata, so a caller scores m_b candidates in
 * micro-batches: the history's K/V come once from hstu_proj_fwd over the
 * history rows alone (acts->k, acts->v of that call), and each micro-batch
 * runs stage 1 on its candidates only and stage 2 with queries = those
 * candidates, keys = cached history + the candidate itself.  Each output row
 * equals the candidate's row of hstu_layer_fwd over history + all m_b
 * candidates (same weights, HSTU_CAND_SHARED_POS) up to rounding order.
 *   x_cand         [Tc, d]   candidate rows of this micro-batch, packed per
 *                            sequence (sequence b owns cand_offsets[b] ..
 *                            cand_offsets[b+1]-1; empty allowed)
 *   cand_offsets   [B+1]     int64, cand_offsets[0] = 0, [B] = Tc
 *   cand_ts        [Tc]      int64 candidate timestamps
 *   num_candidates [B]       int32 m_b: the sequence's candidates over ALL
 *                            micro-batches (N_b = n_b + m_b; values below the
 *                            micro-batch's own count are raised to it)
 *   hist_offsets   [B+1]     int64 history rows of the cache, [B] = Th
 *   hist_ts        [Th]      int64 history timestamps
 *   hist_k         [H, Th, dqk], hist_v [H, Th, dv]: the cache, layer dtype
 *                            (hist_k, hist_v, hist_ts may be NULL when Th = 0)
 *   out            [Tc, d]   may alias x_cand
 *   workspace      >= hstu_cand_workspace_size(desc, Tc, Th, B), 256-aligned;
 *                            besides the stage buffers it holds the fp32
 *                            partial AV of up to 8 history chunks per
 *                            candidate row (32 * Tc * H * dv bytes)
 * Requires HSTU_CAND_SHARED_POS (a candidate's position is then n_b whatever
 * micro-batch it is in); without it returns HSTU_ERR_UNSUPPORTED.
 * HSTU_REUSE_PLAN applies as in hstu_layer_fwd (same micro-batch metadata).  */
size_t hstu_cand_workspace_size(const hstu_desc* desc, int64_t cand_tokens, int64_t hist_tokens,
                                int32_t batch);
hstu_status hstu_cand_fwd(const hstu_desc* desc, const void* x_cand, const int64_t* cand_offsets,
                          int32_t batch, int64_t cand_tokens, const int64_t* cand_ts,
                          const int32_t* num_candidates, const int64_t* hist_offsets,
                          int64_t hist_tokens, const int64_t* hist_ts, const void* hist_k,
                          const void* hist_v, const hstu_weights* weights,
                          const hstu_bias_tables* tables, void* out, void* workspace,
                          size_t workspace_bytes, hstu_stream_t stream);

/* Gradients of one layer's parameters (fp32, overwritten), each laid out
 * like its parameter: w1 [N1, d], b1 [N1], w2 [d, H*dv], b2 [d], the four
 * LayerNorm vectors, pos [H][P] and time [H][NB] ([P] / [NB] when the table's
 * head stride is 0: the heads' gradients summed).  A NULL pointer skips
 * nothing: every field is required.                                          */
typedef struct {
  float* w1;
  float* b1;
  float* w2;
  float* b2;
  float* ln_in_g;  /* zeros without HSTU_INPUT_NORM */
  float* ln_in_b;
  float* ln_av_g;
  float* ln_av_b;
  float* pos;
  float* time;
} hstu_grads;

/* The layer backward (training; [SRM] "Reported results" and [FRC] 7.1.5
 * Stochastic Length train this layer): given dy = dL/dy [T, d] (layer
 * dtype), writes dx = dL/dx [T, d] (layer dtype; may not alias dy or x) and
 * every parameter gradient, for the layer defined above.  The forward
 * activations are recomputed into the workspace, unless desc->flags has
 * HSTU_SAVED_FWD: then the caller asserts that hstu_layer_fwd_train ran just
 * before with the same arguments and workspace (with other contents the
 * gradients are wrong but every access stays in bounds).  Supported: dqk = dv in {32, 64, 128} for bf16, {32, 64} for
 * fp32, num_types = 0, pos_buckets + time_buckets <= 2048, d_model <= 2048
 * and num_heads * dv <= 2048; else HSTU_ERR_UNSUPPORTED.  Results are reproducible bit for bit.  Weight gradients come from
 * GEMMs over the token dimension in the layer dtype with fp32 accumulation.
 * The SiLU derivative of f1 is taken at the forward's pre-activation
 * x W1^T + b1 as stored in the workspace, in the layer dtype.
 *   workspace >= hstu_bwd_workspace_size(desc, T, B) bytes, 256-aligned     */
size_t hstu_bwd_workspace_size(const hstu_desc* desc, int64_t total_tokens, int32_t batch);

/* The layer forward of a training step: the same computation and result as
 * hstu_layer_fwd (bit for bit), run in a backward workspace whose forward part
 * it leaves filled (x after the input LayerNorm, U, V, Q, K, the
 * pre-activation x W1^T + b1, AV and its statistics, the attention plan, and
 * Z = LN(AV) * U), so that a following
 * hstu_layer_bwd with HSTU_SAVED_FWD, on the same stream, with the same
 * arguments and workspace, skips its forward recompute.  Limits as
 * hstu_layer_bwd.  HSTU_SAVED_FWD in desc is ignored here.
 *   workspace >= hstu_bwd_workspace_size(desc, T, B) bytes, 256-aligned     */
hstu_status hstu_layer_fwd_train(const hstu_desc* desc, const void* x, const int64_t* seq_offsets, int32_t batch,
                                 int64_t total_tokens, const int64_t* timestamps, const int32_t* num_candidates,
                                 const hstu_weights* weights, const hstu_bias_tables* tables, void* out,
                                 void* workspace, size_t workspace_bytes, hstu_stream_t stream);
hstu_status hstu_layer_bwd(const hstu_desc* desc, const void* x, const int64_t* seq_offsets, int32_t batch,
                           int64_t total_tokens, const int64_t* timestamps, const int32_t* num_candidates,
                           const hstu_weights* weights, const hstu_bias_tables* tables, const void* dy,
                           void* dx, const hstu_grads* grads, void* workspace, size_t workspace_bytes,
                           hstu_stream_t stream);

/* The attention stage of the backward alone ([SRM] second layer equation;
 * the gradient of AV = sum_j a_ij v_j, a_ij = M_ij SiLU(S_ij) / N_b): reads
 * acts->q, k, v and dav = dL/dAV [T, H*dv] (layer dtype, row-major), writes
 * dqkv [T, N1] fp32 in the columns of the u|v|q|k split: dL/dv, dL/dq and
 * dL/dk (the u block is left untouched), and the position / time table
 * gradients (fp32, laid out like the tables' gradients in hstu_grads).
 * Limits as hstu_layer_bwd; HSTU_REUSE_PLAN as in hstu_attn_fwd.
 *   workspace >= hstu_attn_bwd_workspace_size(desc, T, B) bytes, 256-aligned */
size_t hstu_attn_bwd_workspace_size(const hstu_desc* desc, int64_t total_tokens, int32_t batch);
hstu_status hstu_attn_bwd(const hstu_desc* desc, const int64_t* seq_offsets, int32_t batch, int64_t total_tokens,
                          const int64_t* timestamps, const int32_t* num_candidates, const hstu_bias_tables* tables,
                          const hstu_activations* acts, const void* dav, float* dqkv, float* dpos, float* dtime,
                          void* workspace, size_t workspace_bytes, hstu_stream_t stream);

/* Stochastic length ([FRC] 7.1.5 "Stochastic Length"), the training-time
 * input sampler: with N = max_len, a sequence of n > N^(alpha/2) tokens is,
 * when u[b] < 1 - N^alpha / n^2 (float64), replaced by k = floor(N^(alpha/2))
 * of its tokens: those with the k smallest (keys[row], row) pairs, kept in
 * their original order; other sequences are kept whole.  alpha = 2 keeps
 * every sequence of at most N tokens.  The random draws are the caller's:
 *   u            [B]    float32 uniforms in [0, 1), one per sequence
 *   keys         [T]    uint32, one per token (uniform keys give a uniform
 *                       subset; the page's feature weighting is not modelled)
 *   out_offsets  [B+1]  int64: the sampled batch's offsets (out_offsets[B] =
 *                       the kept token count, on the device)
 *   out_rows     [T]    int64: flat source row of every kept token, in order
 *                       (entries past out_offsets[B] are left untouched)
 *   workspace    >= hstu_sl_workspace_size(B) bytes, 256-aligned
 * alpha must lie in (0, 2] and max_len >= 1.  Re-pack the per-token tensors
 * with hstu_gather_rows (num_rows = out_offsets + B).                       */
size_t hstu_sl_workspace_size(int32_t batch);
hstu_status hstu_sl_sample(const int64_t* seq_offsets, int32_t batch, int64_t total_tokens, int32_t max_len,
                           float alpha, const float* u, const uint32_t* keys, int64_t* out_offsets,
                           int64_t* out_rows, void* workspace, size_t workspace_bytes,
                           hstu_stream_t stream);

/* Jagged re-packing: dst row r = src row rows[r] (row_bytes bytes each) for
 * r < min(*num_rows, max_rows), where num_rows points to DEVICE memory (e.g.
 * out_offsets + B of hstu_sl_sample), so no synchronisation is needed; rows
 * outside [0, src_rows) are clamped into it.  16-, 8- or 4-byte words are
 * used when src, dst and row_bytes allow.                                    */
hstu_status hstu_gather_rows(const void* src, int64_t src_rows, int64_t row_bytes, const int64_t* rows,
                             const int64_t* num_rows, int64_t max_rows, void* dst, hstu_stream_t stream);

/* Integer indexing used by stage 2, for inspection: for each flat pair
 * (query row, key row) in pairs[n_pairs][2] (int64, device) writes
 * out[n][0..5] = {b, i, j, bp, bt, mask} (int64, device) with the definitions
 * above; pairs whose key lies outside the query's sequence get b = -1 and
 * zeros.  Out-of-range rows are an HSTU_ERR_INVALID_ARG only under
 * HSTU_VALIDATE; otherwise they yield b = -1.                                */
hstu_status hstu_debug_indices(const hstu_desc* desc, const int64_t* seq_offsets, int32_t batch,
                               int64_t total_tokens, const int64_t* timestamps,
                               const int32_t* num_candidates, const int64_t* pairs,
                               int64_t n_pairs, int64_t* out, hstu_stream_t stream);

/* The attention kernel's own bias, for inspection ([SRM] second equation and
 * the bullets under it: the relative-position and time-bucket bias added to
 * q.k per head; [FRC] 7.1.4 Innovation 1).  Runs the
 * forward attention kernel's block enumeration, its per-(wave, key block)
 * weight-mode classification and its per-pair bias selection -- the code the
 * forward runs -- without the matrix products, and for every query row r
 * with 0 <= slot[r] < n_slots writes, for each key j < min(L_b, max_len) of
 * r's sequence that the kernel visits:
 *   out[(h * n_slots + slot[r]) * max_len + j]
 *     = -log2(e) * (pos[h][bp(i, j)] + time[h][bt(i, j)])   (float32, as the
 *       kernel holds it: each table entry widened to fp32 and scaled, then added)
 * or NaN where the pair is masked.  Entries the kernel does not visit (key
 * blocks it skips as wholly masked for a wave's rows) are left as they were.
 *   slot [T] int32 (device), out [H * n_slots * max_len] float32 (device)
 *   workspace >= hstu_attn_workspace_size(desc, T, B) bytes, 256-aligned
 * Token types are not supported (num_types must be 0).                     */
hstu_status hstu_debug_attn_bias(const hstu_desc* desc, const int64_t* seq_offsets, int32_t batch,
                                 int64_t total_tokens, const int64_t* timestamps,
                                 const int32_t* num_candidates, const hstu_bias_tables* tables,
                                 const int32_t* slot, int32_t n_slots, int32_t max_len, float* out,
                                 void* workspace, size_t workspace_bytes, hstu_stream_t stream);

const char* hstu_status_str(hstu_status status);
const char* hstu_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HSTU_H_ */
