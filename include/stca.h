/*
 * stca.h -- C ABI of the STCA forward library for MI355X (gfx950).
 *
 * The library computes the forward hot path of Stacked Target-to-History
 * Cross Attention (STCA) over ragged user histories, with Request Level
 * Batching (every target of a user reads that user's keys and values once
 * per layer) and, on the fused path, the embedding gather fused with the
 * attention ("lookup while computing").
 *
 * Pages this interface follows (cited by title and section):
 *   [Notes]    "超长序列建模 —— STCA 精读笔记": §STCA (layer definition:
 *              history FFN+LN feeding W_K/W_V, query from the target, heads
 *              concatenated then W_O), §Request Level Batching.
 *   [Review]   "Make It Long, Keep It Fast: End-to-End 10K Long User Behavior
 *              Sequence Modeling for Billion-Scale Douyin Recommendation"
 *              (paper review): architecture tree and 核心公式 (alpha, o,
 *              fusion q^(i+1), final z).
 *   [WeChat]   "视频号推荐超长序列技术演进：从端到端到 Cross-Mask Transformer":
 *              §1.1 显存优化 (lookup fused with target attention, no [B,L,D]
 *              KV tensor), §1.2 (ReLU-activated target attention, active keys
 *              are those with score > 0), §2.2.3 (context similarity added
 *              to the target-attention score), §3.2-3.3 (Cross-Mask masks and
 *              shared attention maps).
 *   [HyFormer] "HyFormer：重新审视序列建模和特征交互在 CTR 预测中的作用":
 *              eq. (7)-(9) and (16) (per-layer SwiGLU encoding without LN,
 *              multi-query cross attention), §3.7 (one query set per sequence).
 *
 * Conventions
 *   - Row vectors: y = x W with W stored [in, out] row-major.
 *   - Every data pointer below is a DEVICE pointer unless marked "host".
 *     The caller allocates and owns every buffer, including the workspace;
 *     the library keeps no pointer after a call returns.
 *   - Calls are asynchronous on the given HIP stream (hipStream_t passed as
 *     void*; NULL = the null stream).  The library never synchronises.
 *   - bf16 arrays hold raw bf16 bits (uint16).  fp32 arrays are IEEE float.
 *   - All device pointers must be 16-byte aligned.
 *
 * Errors
 *   Host-side validation is synchronous: a negative stca_status is returned,
 *   nothing is enqueued, and stca_last_error() gives a thread-local message.
 *   Conditions only visible on the device (inconsistent CSR offsets, a user
 *   with more targets than max_tgt_per_user, ids outside [0, table_rows))
 *   never cause an out-of-bounds access: the offending rows are treated as
 *   zero rows / empty users, and if outputs->dev_status is non-NULL a nonzero
 *   bit mask (STCA_DEV_*) is OR-ed into it; the caller reads it after the
 *   stream has completed.  No exception crosses the ABI and nothing aborts.
 */
#ifndef STCA_H_
#define STCA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  STCA_OK = 0,
  STCA_ERR_INVALID_ARG = -1,   /* null/misaligned pointer, bad size or mode   */
  STCA_ERR_UNSUPPORTED = -2,   /* valid request this build does not implement */
  STCA_ERR_WORKSPACE = -3,     /* workspace missing or smaller than required  */
  STCA_ERR_HIP = -4            /* a HIP launch or runtime call failed         */
} stca_status;

enum { STCA_F32 = 0, STCA_BF16 = 1 };                  /* stca_config.dtype  */
enum { STCA_SCORE_SOFTMAX = 0, STCA_SCORE_RELU = 1 };  /* stca_config.score  */
enum { STCA_Q_FUSION = 0, STCA_Q_LINEAR = 1,          /* stca_config.qmode  */
       STCA_Q_HYFORMER = 2 };
/* STCA_Q_HYFORMER ([HyFormer] §3.3.2 eq. (3)-(4), §3.5 eq. (10)-(15), §3.6
 * eq. (16)-(17)): every user has exactly m = max_tgt_per_user queries
 * (tgt_offsets[u] = u m), generated from the user's non-sequence tokens F
 * (batch->ns_feats) and the mean of its raw history rows:
 *   g_u = [F_u,1 | .. | F_u,n_ns | MeanPool(rows)],  q_u,n = FFN_n(g_u);
 * each layer decodes them (multi-head cross attention, W_O) into o and boosts
 * Q = [o_u,1..m | F_u,1..n_ns] (T = m + n_ns tokens, T divides d): every token
 * is cut into T subspaces of width d / T, mixed token h concatenates every
 * token's h-th subspace, Q_boost = Q + [FFN'_1(mixed 1) | .. | FFN'_T(mixed T)]
 * position by position; the first m boosted tokens are the next queries and,
 * after the last layer, z.  Every FFN is SwiGLU without LN, hidden width
 * cfg->q_hidden.  bf16, staged path; the history side is HyFormer's
 * eq. (7)-(8) encoding as in STCA_Q_LINEAR. */
enum { STCA_PATH_STAGED = 0, STCA_PATH_FUSED = 1 };    /* stca_config.path   */
enum { STCA_ENC_SWIGLU = 0, STCA_ENC_LONGER = 1 };     /* stca_config.encoder */
/* History (sequence) encoding of every layer:
 *  STCA_ENC_SWIGLU: Xt = [LN](SwiGLU(X)) of the raw rows X ([Notes] §STCA;
 *    [HyFormer] eq. (7)), K = Xt W_K, V = Xt W_V.
 *  STCA_ENC_LONGER ([HyFormer] §3.4.1 (ii), eq. (6) then (8)): per layer
 *    H_l = CrossAttn(S_short, S, S), the multi-head softmax cross attention
 *    (scale 1/sqrt(d_h), the layer's own enc_wq / enc_wk / enc_wv / enc_wo,
 *    no residual, no LN) from the user's last min(L_u, l_short) history rows
 *    (S_short) to all of its rows (S); then K = H_l W_K, V = H_l W_V, and the
 *    targets attend over these min(L_u, l_short) rows.  bf16, staged path,
 *    softmax scores; not with STCA_FLAG_DEDUP, Cross-Mask, x_dump, kv_dump or
 *    stca_backward.  The history FFN weights (layer.kv) are not read, and
 *    STCA_FLAG_KV_LN is ignored. */
enum {                                                 /* stca_config.flags  */
  STCA_FLAG_KV_LN = 1,  /* LN after the history FFN (STCA); clear for HyFormer eq. (7) */
  STCA_FLAG_Z_LN = 2,   /* LN on the final z ([Notes] wording); default is [Review]'s z */
  STCA_FLAG_DEDUP = 4   /* encode each distinct history id of the batch once and copy its
                           K/V to every token carrying it (a row's encoding depends on its
                           id alone, [Notes] §STCA); results are bit-identical to the plain
                           path.  bf16, staged path only; not with x_dump. */
};
enum {                                                 /* dev_status bits     */
  STCA_DEV_BAD_HIST_OFFSETS = 1,  /* hist_offsets not monotone / not ending at n_hist: all users empty */
  STCA_DEV_BAD_TGT_OFFSETS = 2,   /* tgt_offsets inconsistent or m_u > max_tgt_per_user: no targets  */
  STCA_DEV_BAD_ID = 4             /* an id outside [0, table_rows): that row reads as zeros           */
};

/* Model and launch configuration (host struct). */
typedef struct {
  int32_t B;            /* users in the batch                                     */
  int32_t d;            /* model width; bf16: 128, 256 or 512; fp32: 32..512 (x32) */
  int32_t H;            /* heads; d_h = d / H must be 32 or 64                    */
  int32_t hidden;       /* SwiGLU hidden width h; multiple of 128 (bf16) / 32     */
  int32_t M;            /* stacked layers, 1..16                                  */
  int64_t table_rows;   /* rows N of the embedding table                          */
  int32_t dtype;        /* STCA_F32 or STCA_BF16: table, weights, K/V, queries    */
  int32_t score;        /* STCA_SCORE_*                                           */
  int32_t qmode;        /* STCA_Q_*                                               */
  int32_t path;         /* STCA_PATH_*.  STCA_PATH_FUSED ([WeChat] §1.1): per layer
                           one kernel gathers, encodes and attends 64 keys at a time
                           and no K/V tensor is kept; bf16 only, d = 256 (d_h 32
                           or 64) or d = 128 (d_h 32), STCA_FLAG_KV_LN set, at most
                           64 targets per user; otherwise STCA_ERR_UNSUPPORTED     */
  int32_t flags;        /* STCA_FLAG_*                                            */
  int32_t chunk_keys;   /* keys per split-L chunk (multiple of 32); 0 = automatic  */
  int32_t n_ns;         /* STCA_Q_HYFORMER: non-sequence feature tokens per user   */
  int32_t q_hidden;     /* STCA_Q_HYFORMER: hidden width of the query FFNs (x32)   */
  const int32_t *head_map; /* host [H] or NULL: Cross-Mask shared attention maps
                           ([WeChat] §3.3.1, several heads share one attention map
                           under different masks): head h scores with the Q / K
                           columns of head head_map[h] (values in [0, H)); its V
                           columns and output slice stay its own.  Staged bf16 only */
  int32_t encoder;      /* STCA_ENC_* (0: the SwiGLU encoding)                    */
  int32_t l_short;      /* STCA_ENC_LONGER: short-sequence length L_H, 1..4096     */
} stca_config;

/* One batch of requests: ragged histories and targets in CSR form.
 * User u owns history tokens [hist_offsets[u], hist_offsets[u+1]) and targets
 * [tgt_offsets[u], tgt_offsets[u+1]) ([Notes] §RLB: the targets of one request
 * share the user's encoding).  Histories may be empty. */
typedef struct {
  const int32_t *hist_offsets;  /* [B+1], hist_offsets[0] = 0, last = n_hist       */
  const int32_t *hist_ids;      /* [n_hist] table rows of the history items         */
  const int32_t *tgt_offsets;   /* [B+1], tgt_offsets[0] = 0, last = n_tgt          */
  const int32_t *tgt_ids;       /* [n_tgt] table rows of the targets (STCA_Q_FUSION) */
  const void *q0;               /* [n_tgt, d] first-layer queries (STCA_Q_LINEAR)   */
  const void *table;            /* [table_rows, d] embedding table                  */
  int64_t n_hist;               /* host: total history tokens, < 2^31               */
  int64_t n_tgt;                /* host: total targets, < 2^31                      */
  int32_t max_tgt_per_user;     /* host: upper bound on any m_u, 1..4096            */
  const void *ns_feats;         /* [B, n_ns, d] non-sequence tokens (STCA_Q_HYFORMER) */
  const uint32_t *key_mask;     /* [n_hist] or NULL: Cross-Mask vertical masks ([WeChat]
                                   §3.2): bit h set = history item j is visible to head h
                                   (its feature-domain condition holds, e.g. "action =
                                   complete"); softmax and ReLU then run over the visible
                                   items only, a head with none gives 0.  Staged bf16 only */
  const float *score_bias;      /* [n_hist, H] fp32 or NULL: context-similarity score bias
                                   ([WeChat] §2.2.3, 上下文利用: the context similarity of two
                                   videos fine-tunes the target-attention score; the page
                                   gives no formula, the values are the caller's).  Every
                                   layer's score of item j and head h becomes
                                   s_j = q . k_j / sqrt(d_h) + score_bias[j, h] for every
                                   target of the user, before the softmax or the ReLU (the
                                   active count is then #{j : s_j > 0}).  With a head map,
                                   head h adds its own bias column.  Staged bf16 only, not
                                   with STCA_ENC_LONGER; read once per call (a blocked copy
                                   in the workspace) */
} stca_batch;

/* SwiGLU FFN d -> h -> d, optionally followed by LayerNorm (eps 1e-5):
 * y = (SiLU(x W1) * (x W3)) W2;  LN(y) = (y - mean) / sqrt(var + eps) * ln_g + ln_b.
 * Matrices in the config dtype; ln_g / ln_b are always fp32 [d]. */
typedef struct {
  const void *w1;     /* [d, h] */
  const void *w3;     /* [d, h] */
  const void *w2;     /* [h, d] */
  const float *ln_g;  /* [d] (NULL when the LN is not applied) */
  const float *ln_b;  /* [d] */
} stca_ffn;

/* Weights of layer i (0-based).  Heads are column slices of width d_h of
 * W_Q, W_K, W_V; W_O acts on the concatenated heads ([Notes] §STCA). */
typedef struct {
  stca_ffn kv;        /* history FFN (+LN if STCA_FLAG_KV_LN): Xt = LN(SwiGLU(X))   */
  stca_ffn q;         /* query FFN+LN (STCA_Q_FUSION): q1 = LN(SwiGLU(x_t)) at i = 0,
                         q_{i+1} = LN(SwiGLU([o_1|..|o_i|x_t] W_C)) at i > 0          */
  const void *wk, *wv, *wq, *wo;   /* [d, d] each                                   */
  const void *wc;     /* [(i+1) d, d] fusion matrix (STCA_Q_FUSION, i > 0; else NULL) */
  const void *r;      /* [d, d] next-query map Q_{i+1} = O_i R_i (STCA_Q_LINEAR,
                         i < M-1; else ignored)                                      */
  const void *boost_w1, *boost_w3;  /* [T, d, q_hidden] per-token boosting FFNs      */
  const void *boost_w2;             /* [T, q_hidden, d]   (STCA_Q_HYFORMER)           */
  const void *enc_wq, *enc_wk, *enc_wv, *enc_wo;  /* [d, d] each: the cross attention of
                                                     STCA_ENC_LONGER (NULL otherwise) */
} stca_layer;

typedef struct {
  const stca_layer *layers;  /* host array [M]                                      */
  stca_ffn z;                /* final SwiGLU (+LN with STCA_FLAG_Z_LN), STCA_Q_FUSION */
  const void *wz;            /* [(M+1) d, d] final concat map, STCA_Q_FUSION          */
  /* STCA_Q_HYFORMER query generation: FFN_n for n < m */
  const void *qgen_w1, *qgen_w3;  /* [m, (n_ns+1) d, q_hidden]                         */
  const void *qgen_w2;            /* [m, q_hidden, d]                                  */
} stca_weights;

typedef struct {
  float *z;            /* [n_tgt, d] z (fusion) or O_M (linear); required if n_tgt > 0 */
  float *o_layers;     /* [M, n_tgt, d] optional: o^(i) after W_O                    */
  float *attn;         /* [M, n_tgt, d] optional: heads concatenated, before W_O     */
  int32_t *active;     /* [M, n_tgt, H] optional, STCA_SCORE_RELU: #{j : s_j > 0}    */
  void *q_dump;        /* [M, n_tgt, d] optional: query rows as the attention reads
                          them (after W_Q and the 1/sqrt(d_h) scale), config dtype   */
  void *kv_dump;       /* [M, 2, n_hist, d] optional: K then V rows of every layer as
                          the attention reads them, config dtype (staged path only)  */
  void *x_dump;        /* [n_hist, d] optional: gathered history rows (table dtype).
                          Fused path: written with layer 0's encoding            */
  int32_t *dev_status; /* optional: STCA_DEV_* bits OR-ed in on the device           */
  /* Optional stage timing: host array of caller-created hipEvent_t handles.  The
   * library records (hipEventRecord on the call's stream, no synchronisation) up
   * to n_stage_events of these boundaries, in this order:
   *   0            start of the call
   *   1            weights prepared and batch planned
   *   2 + i        history encoding (gather, FFN, LN, W_K|W_V) of layer i done, i < M
   *                (bf16 staged at d <= 256: one launch encodes every layer,
   *                so all M are recorded after it and 2 + 0 spans it all;
   *                fused path: all M recorded right after event 1, the
   *                encoding being part of each layer's attention partials)
   *   2 + M + 4i   query of layer i done
   *   3 + M + 4i   attention partials of layer i done
   *   4 + M + 4i   partial merge of layer i done
   *   5 + M + 4i   output projection (and next-query map) of layer i done
   *   2 + 5M       final z done                     (5M + 3 events in all)
   * With STCA_ENC_LONGER the span 0..1 also holds the encoding pre-pass, whose
   * boundaries follow (9M + 4 events in all):
   *   3 + 5M       encoder weights packed, short sequences and raw plan built
   *   4 + 5M + 4i  encoder K/V (S W'_K | S W'_V, raw rows) of layer i done
   *   5 + 5M + 4i  encoder queries (S_short W'_Q) of layer i done
   *   6 + 5M + 4i  encoder attention (partials and merge) of layer i done
   *   7 + 5M + 4i  H_l = attention W'_O of layer i done */
  void *const *stage_events;
  int32_t n_stage_events;
  float *lse;          /* [M, n_tgt, H] optional, STCA_SCORE_SOFTMAX: log of each (target,
                          head)'s softmax denominator, ln sum_j exp(s_j) (the max plus the
                          log of the rescaled sum; 0 for an empty history).  The backward
                          recomputes the weights exp(s_j - lse) from it. */
  uint64_t *clock_probe; /* [8][4] optional measurement aid, bf16 staged path at
                          d = 128 or 256: workgroups 0..7 of the history-encoding launch (one
                          per XCD under round-robin dispatch) write, from their first
                          wave, {shader-clock counter (s_memtime), 100 MHz counter
                          (s_memrealtime)} at their start and at their end.  The
                          ratio of the differences x 0.1 GHz is the shader clock the
                          chip held during the launch.  Rows of workgroups that do not
                          exist are left untouched.                                */
} stca_outputs;

/* Workspace bytes stca_forward needs for this configuration and batch.
 * With STCA_PATH_FUSED the size does not grow with n_hist * d (no K/V buffer). */
int stca_workspace_size(const stca_config *cfg, const stca_batch *batch, size_t *bytes);

/* The full forward: every layer's history encoding (gather, SwiGLU FFN, LN,
 * W_K/W_V), the query chain, the m-target multi-head cross attention of every
 * user, W_O, the fusion update and z.  Returns STCA_OK once everything is
 * enqueued on `hip_stream`. */
int stca_forward(const stca_config *cfg, const stca_batch *batch, const stca_weights *w,
                 const stca_outputs *out, void *workspace, size_t ws_bytes, void *hip_stream);

/* stca_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same forward, its workspace taken from a static device array of
 * STCA_NOALLOC_SCRATCH_BYTES that the library holds on each device it runs on
 * until the process ends.  The caller still passes every input and output.
 * A batch whose stca_workspace_size exceeds the array is rejected with
 * STCA_ERR_WORKSPACE before anything is enqueued.  The device is the one
 * current on the calling thread (hip_stream must belong to it).  Every call
 * on a device shares that device's array: calls that overlap on one device
 * (other streams, other threads) race and must be serialised by the caller.
 * Allocates nothing: no hipMalloc, hipFree or allocating library routine. */
#define STCA_NOALLOC_SCRATCH_BYTES (128u << 20)
int stca_forward_noalloc(const stca_config *cfg, const stca_batch *batch, const stca_weights *w,
                         const stca_outputs *out, void *hip_stream);

/* The attention core alone on caller-provided operands ([Review] formula for
 * alpha and o; [WeChat] §1.2 for the ReLU form): for every user u, target t of
 * u and head eta,
 *   s_j = q_t[eta] . k_j[eta]                (q rows already carry 1/sqrt(d_h))
 *   softmax: attn_t[eta] = sum_j exp(s_j - max) v_j[eta] / sum_j exp(s_j - max)
 *   relu:    attn_t[eta] = sum_j max(0, s_j) v_j[eta], active = #{j : s_j > 0}
 * over the user's history rows j (plus score_bias[j, eta] when given).  An
 * empty history gives zeros. */
typedef struct {
  int32_t B, d, H;          /* host                                                  */
  int32_t dtype;            /* STCA_F32 / STCA_BF16 for q, k, v                       */
  int32_t score;            /* STCA_SCORE_*                                           */
  int32_t chunk_keys;       /* as in stca_config                                      */
  const int32_t *hist_offsets;  /* [B+1] */
  const int32_t *tgt_offsets;   /* [B+1] */
  int64_t n_hist, n_tgt;    /* host */
  int32_t max_tgt_per_user; /* host */
  const void *q;            /* [n_tgt, d] */
  const void *k, *v;        /* [n_hist, d] each */
  float *attn;              /* [n_tgt, d] output */
  int32_t *active;          /* [n_tgt, H] output, ReLU only (optional) */
  int32_t *dev_status;      /* optional */
  const uint32_t *key_mask; /* [n_hist] or NULL, as stca_batch.key_mask (bf16 only) */
  const int32_t *head_map;  /* host [H] or NULL, as stca_config.head_map (bf16 only) */
  const float *score_bias;  /* [n_hist, H] or NULL, as stca_batch.score_bias: added to
                               s_j (bf16 only) */
} stca_attn_args;

int stca_attention_workspace_size(const stca_attn_args *a, size_t *bytes);
int stca_attention(const stca_attn_args *a, void *workspace, size_t ws_bytes, void *hip_stream);

/* ---------------------------------------------------------------- training step
 * Gradients of a loss through z.  The pages train the same model as they serve
 * ([Review] 核心公式, "RLB 损失函数": the per-user loss is the mean BCE over the
 * user's m targets, L_u = (1/m) sum_k BCE(y_hat(u, t_k), y_k); [Notes]
 * "短序列训练，长序列推理": training runs on shorter, Beta-sampled lengths).  The
 * head from z to y_hat (RankMixer, sigmoid) is not part of this library: the
 * caller passes dz = dL/dz and receives the gradient of every STCA weight and of
 * every embedding row the forward read, by the chain rule through the forward
 * of stca_forward (recomputed inside the call from the same inputs: nothing is
 * kept between calls).  Supported: bf16, STCA_Q_FUSION, d_h 32 or 64,
 * max_tgt_per_user <= 64, softmax or ReLU scores, with or without the history
 * and z LayerNorms.  cfg->path is ignored (the recompute runs the staged path).
 * STCA_FLAG_DEDUP is honoured: the recompute encodes each distinct history id
 * once, and the history side's backward runs once per distinct id on the sum
 * of its items' dK | dV (fixed item order); grads->d_hist (a per-item output)
 * is then rejected with STCA_ERR_UNSUPPORTED.  Cross-Mask masks and maps and
 * the score bias are rejected (STCA_ERR_UNSUPPORTED).
 *
 * Weight gradients are fp32, shaped like the weights ([in, out] row-major), and
 * ACCUMULATED (+=) into the caller's buffers: zero them for a fresh step.  The
 * ReLU score takes derivative 0 at s = 0.  Rows read through an id outside the
 * table get no gradient. */
typedef struct {
  float *w1, *w3;     /* [d, h] */
  float *w2;          /* [h, d] */
  float *ln_g, *ln_b; /* [d]; required where the forward applies that LN */
} stca_ffn_grad;

typedef struct {
  stca_ffn_grad kv, q;
  float *wk, *wv, *wq, *wo;  /* [d, d] */
  float *wc;                 /* [(i+1) d, d]; NULL at i = 0 */
} stca_layer_grad;

typedef struct {
  const stca_layer_grad *layers;  /* host array [M]; every pointer required */
  stca_ffn_grad z;
  float *wz;           /* [(M+1) d, d] */
  float *table;        /* [table_rows, d] optional: += the gradient of every row read by a
                          history item or a target (atomic adds: the summation order of a
                          row shared by several items is not fixed) */
  float *d_hist;       /* [n_hist, d] optional: gradient per history item (overwritten) */
  float *d_tgt;        /* [n_tgt, d] optional: gradient per target row x_t (overwritten) */
  float *z_out;        /* [n_tgt, d] optional: z of the recomputed forward */
  float *dq_dump;      /* [M, n_tgt, d] optional: gradient w.r.t. each layer's query rows
                          as the attention reads them (after the 1/sqrt(d_h) scale) */
  float *da_dump;      /* [M, n_tgt, d] optional: gradient w.r.t. each layer's attention
                          output (heads concatenated, before W_O) */
  void *dkv_dump;      /* [M, n_hist, 2d] optional, bf16: each layer's dK | dV rows */
  int32_t *dev_status; /* optional: STCA_DEV_* bits, as for stca_forward */
  /* Optional stage timing, as for stca_forward: up to n_stage_events of
   *   0            start of the call
   *   1            forward recompute done
   *   2            z head, history-row gather and (dedup) unique-row sort done
   *   3 + 5j       layer i = M-1-j: output projection and attention backward done
   *   4 + 5j       layer i: query side done
   *   5 + 5j       layer i: (dedup) dK | dV summed per unique row
   *   6 + 5j       layer i: history side's row pass done (recompute, dX; at d = 256
   *                one fused launch, otherwise recorded with the next event)
   *   7 + 5j       layer i: history side done (weight gradients)
   *   3 + 5M       row gradients added to the table     (5M + 4 events in all) */
  void *const *stage_events;
  int32_t n_stage_events;
  /* Nonzero: skip the forward recompute.  The caller has run
   * stca_forward_for_backward with the same config, batch and weights on this
   * workspace, and nothing has written the workspace since; its activations
   * are used as they are (events 0 and 1 are recorded back to back).  z_out
   * must then be NULL (z is that call's output). */
  int32_t saved_forward;
} stca_grads;

int stca_backward_workspace_size(const stca_config *cfg, const stca_batch *batch, size_t *bytes);

/* dz: [n_tgt, d] fp32 device array, the upstream gradient of z. */
int stca_backward(const stca_config *cfg, const stca_batch *batch, const stca_weights *w, const float *dz,
                  const stca_grads *grads, void *workspace, size_t ws_bytes, void *hip_stream);

/* The forward of a training step, keeping its activations for the backward
 * instead of having stca_backward recompute them: the same computation as
 * stca_backward's recompute (the staged path, STCA_FLAG_DEDUP honoured, the
 * same checks and the same results bit for bit), writing z [n_tgt, d] (fp32,
 * required when n_tgt > 0) and leaving each layer's o, attention output,
 * scaled Q, K/V rows and softmax lse in `workspace` (stca_backward's, of
 * stca_backward_workspace_size bytes).  Then stca_backward with
 * grads->saved_forward = 1 on the same workspace skips its recompute.  A
 * training step saves the recompute this way at the cost of keeping the
 * workspace between the two calls.  dev_status (optional): STCA_DEV_* bits. */
int stca_forward_for_backward(const stca_config *cfg, const stca_batch *batch, const stca_weights *w, float *z,
                              int32_t *dev_status, void *workspace, size_t ws_bytes, void *hip_stream);

/* Measurement aid, not a step of the method: `blocks` workgroups of 256
 * threads, every wave doing `iters` rounds of 8 independent dense bf16
 * 32x32x16 MFMA products from registers (blocks * 4 * iters * 8 * 32768
 * flop), writing one checksum per wave to out[blocks * 4] (device, fp32).
 * Timed by the caller on `hip_stream`, it gives the matrix cores' attainable
 * rate at the clock the chip holds under that load.  The operands are fixed
 * low-entropy values; with iters < 0 the kernel runs |iters| rounds on
 * operands whose signs, exponents and mantissas vary like real data (four
 * random A and B fragments per lane, a different pair for consecutive
 * products): the chip's clock under MFMA load depends on how many operand
 * bits switch, so this is the attainable rate for realistic operands.  clock
 * (device, optional, [4]): workgroup 0's {s_memtime, s_memrealtime} at its
 * start and end, as for stca_outputs.clock_probe.  Enqueued only; returns
 * STCA_ERR_INVALID_ARG for blocks <= 0, iters = 0 or a NULL out. */
int stca_peak_mfma_bf16(int32_t blocks, int32_t iters, float *out, uint64_t *clock, void *hip_stream);

/* Measurement aid, not a step of the method: `blocks` workgroups of 256
 * threads stream `bytes` (a multiple of 16) of device memory at buf once with
 * 16-byte non-temporal loads, the access the attention uses for K/V, and
 * write one word to out[0] (device) only if the data XOR to a sentinel (so
 * the loads are live).  Timed by the caller over a buffer larger than the
 * memory-side cache, it gives the attainable HBM read rate.  Enqueued only;
 * STCA_ERR_INVALID_ARG for non-positive sizes, a size not a multiple of 16,
 * or NULL pointers. */
int stca_peak_hbm_read(const void *buf, int64_t bytes, int32_t blocks, uint32_t *out, void *hip_stream);

const char *stca_status_string(int status);
/* Detail of the last failure on the calling thread ("" if none). */
const char *stca_last_error(void);
/* Library version, major * 10000 + minor * 100 + patch. */
int stca_version(void);

#ifdef __cplusplus
}
#endif
#endif /* STCA_H_ */
