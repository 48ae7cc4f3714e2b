/*
 * lcsr.h — long-context sparse prefill with DCA and YaRN RoPE on MI355X.
 *
 * C ABI of the library liblcsr.so (gfx950).  One prefill chunk of one
 * attention layer at a time: rotate the chunk's keys into the KV cache,
 * estimate the vertical-slash pattern from the chunk's last queries, and run
 * the sparse causal attention of the chunk's queries over the cache.
 *
 * Sources (cited by page and section):
 *  [Qwen2.5-1M explainer] "論文解説: Qwen2.5-1M — 100万トークンコンテキストを実現する
 *     長文脈LLMの設計と推論最適化" (0h-n0.github.io): 推論フレームワーク,
 *     Length Extrapolation (DCA, YaRN attention scaling), 疎アテンション,
 *     Chunked Prefill (last-64 estimate, attention recall, refinement),
 *     アルゴリズム: DCAと疎アテンションの統合 (pseudocode of the chunk loop).
 *  [long-context blog] "大規模モデル長文脈最適化実践" (toolsku.com): RoPE原理の復習,
 *     YaRN実装.
 *  [architecture overview] deepseekmodel.com long-context architecture page:
 *     §2.4 code (inv_freq, rotate_half), §3.2 (online softmax), §4.2
 *     (vertical-slash), §4.6 (GQA head mapping).
 *
 * Conventions shared by every call
 *  - Every pointer is DEVICE memory unless marked (host).  The caller owns
 *    every buffer, including the workspace; the library allocates no device
 *    memory and keeps no pointer after a call returns.  Host structs are read
 *    during the call only.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream).  No call synchronises the device or reads device data back.
 *  - Tensors are row-major with the last dimension (head_dim) contiguous;
 *    strides are in elements.  Device pointers must be 16-byte aligned and
 *    row strides multiples of 8 elements.
 *  - Status: 0 on success, else a negative LCSR_E* code.  Arguments are
 *    validated before anything is launched, so an error return other than
 *    LCSR_EHIP has written nothing.  lcsr_last_error() gives a message for
 *    the last failing call of the calling thread.  No exception crosses the
 *    ABI; calls are thread-safe.
 *  - Precision.  Inputs (queries, keys, values) are bf16 (fp32 queries are
 *    rounded to bf16 on entry).  RoPE angles are formed in fp64 from the
 *    integer position and the rotation in fp32.  QK^T runs on the matrix
 *    cores with fp16 operands, the rotated keys of the K cache and the
 *    rotated queries, each rounded to nearest; PV with bf16 operands (the V
 *    cache and the probabilities); every product accumulates in fp32.
 *    Rotated keys and queries must lie within the fp16 range (|x| < 65504).
 */
#ifndef LCSR_H
#define LCSR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define LCSR_OK 0
#define LCSR_EINVAL (-1)     /* bad shape, stride, alignment, pointer or value  */
#define LCSR_ENOTSUP (-2)    /* valid but unsupported (head_dim, DCA period...) */
#define LCSR_EWORKSPACE (-3) /* workspace smaller than lcsr_workspace_bytes()   */
#define LCSR_EHIP (-4)       /* a HIP launch failed                             */

/* Zero-length calls.  chunk_len 0 (or n_rows 0 for the recall checks) is a
 * valid call that launches nothing and writes nothing; output pointers may
 * then be NULL. */

/* ---- element types ----------------------------------------------------- */
#define LCSR_BF16 0
#define LCSR_FP32 1
#define LCSR_FP16 2

/* ---- flags ------------------------------------------------------------- */
#define LCSR_ROPE_YARN_FREQ 0x1u  /* lcsr_rope_t.flags: YaRN frequency blend  */
#define LCSR_ROPE_NO_ROTATE 0x2u  /* rope_yarn_apply: convert/scale only      */
#define LCSR_ROPE_OUT_FP16 0x4u   /* rope_yarn_apply: store fp16, not bf16    */
#define LCSR_EST_SELECT_ONLY 0x1u /* estimate: scores are inputs, select only */
#define LCSR_ATTN_DENSE 0x1u      /* attention: every causal key (no pattern) */
#define LCSR_BS_SELECT_ONLY 0x1u  /* block estimate: scores are inputs        */

/* ---- workspace kinds --------------------------------------------------- */
#define LCSR_WS_ESTIMATE 0
#define LCSR_WS_ATTN 1
#define LCSR_WS_RECALL 2
#define LCSR_WS_DECODE 3
#define LCSR_WS_BLOCK_EST 4
#define LCSR_WS_BLOCK_ATTN 5

/* Rotary embedding setup ([architecture overview] §2.4 code; YaRN from
 * [Qwen2.5-1M explainer] Length Extrapolation and [long-context blog]
 * YaRN実装).  theta_p = base^(-2p/D).  With LCSR_ROPE_YARN_FREQ and
 * yarn_factor s > 1, theta_p is blended as YaRN's NTK-by-parts:
 * r_p = orig_max_pos * theta_p / (2 pi), g_p = clamp((r_p - beta_slow) /
 * (beta_fast - beta_slow), 0, 1), theta_p <- theta_p ((1 - g_p)/s + g_p).
 * The YaRN temperature is not applied here: the attention calls take it
 * in sm_scale (lcsr_softmax_scale). */
typedef struct lcsr_rope {
  double base;          /* RoPE base, e.g. 1e4 or 1e7                       */
  double yarn_factor;   /* s = inference length / training length; <=1 off */
  int64_t orig_max_pos; /* training length for the frequency blend          */
  double beta_fast;     /* 32 in the published YaRN                         */
  double beta_slow;     /* 1                                                */
  uint32_t flags;       /* LCSR_ROPE_YARN_FREQ                              */
} lcsr_rope_t;

/* Dual Chunk Attention ([Qwen2.5-1M explainer] Length Extrapolation).
 * chunk = C, the largest position + 1 (the training length); local = W, the
 * successive-chunk local window; keys repeat with period S = C - W.
 * P_k(j) = j mod S; query positions: intra i mod S, succ S + (i mod S) if
 * (i mod S) < W else C - 1, inter C - 1; the pair (i, j) uses intra / succ /
 * inter when floor(i/S) - floor(j/S) is 0 / 1 / >= 2.  chunk = 0: DCA off. */
typedef struct lcsr_dca {
  int64_t chunk;
  int64_t local;
} lcsr_dca_t;

/* One prefill chunk of one layer: query rows [chunk_start, chunk_start +
 * chunk_len) against the KV cache rows [0, chunk_start + chunk_len).
 * Grouped-query attention: query head h reads KV head h / (H / H_kv)
 * ([architecture overview] §4.6).  Supported: head_dim 64 or 128,
 * n_heads <= 64, n_heads % n_kv_heads == 0, n_heads / n_kv_heads <= 16.
 * With DCA on, S = C - W >= 64 and chunk_start % 64 == 0 (any chunk_start
 * for lcsr_attn_decode); lcsr_vs_sparse_attn_prefill takes S % 32 == 0 (its
 * 32-query-row blocks stay inside one DCA chunk); the other calls take any
 * S. */
typedef struct lcsr_problem {
  const void* q;       /* [H, chunk_len, D] pre-RoPE queries of the chunk   */
  int32_t q_dtype;     /* LCSR_BF16 or LCSR_FP32 (fp32 is rounded to bf16)  */
  int64_t q_stride_h;
  int64_t q_stride_t;
  const void* k_cache; /* fp16 [H_kv, >= chunk_start + chunk_len, D], keys
                          rotated at P_k(j) (lcsr_rope_yarn_apply with
                          LCSR_ROPE_OUT_FP16)                              */
  const void* v_cache; /* bf16, same layout; unused by the estimate        */
  int64_t kv_stride_h;
  int64_t kv_stride_t;
  int32_t n_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int64_t chunk_start;
  int64_t chunk_len;
  lcsr_rope_t rope;
  lcsr_dca_t dca;
  float sm_scale;      /* 1 / (t sqrt(D)), the YaRN temperature folded in
                          (lcsr_softmax_scale gives it from rope)          */
} lcsr_problem_t;

/* Vertical-slash pattern of every head.  vert_idx[h, :vert_cnt[h]] are key
 * columns j and slash_idx[h, :slash_cnt[h]] diagonal offsets o = i - j, both
 * strictly ascending, the rest padded with -1.  The critical set of query
 * row i is { v <= i } U { i - o : o <= i } (each key once). */
typedef struct lcsr_pattern {
  int32_t* vert_idx;  /* [H, max_vert]  */
  int32_t* vert_cnt;  /* [H]            */
  int32_t max_vert;
  int32_t* slash_idx; /* [H, max_slash] */
  int32_t* slash_cnt; /* [H]            */
  int32_t max_slash;
} lcsr_pattern_t;

/* Bytes of workspace a call needs.  which = LCSR_WS_*; n_ctx = chunk_start +
 * chunk_len (keys visible to the chunk); max_vert/max_slash as in the
 * pattern.  Returns 0 for invalid arguments. */
size_t lcsr_workspace_bytes(int which, const lcsr_problem_t* p,
                            int32_t max_vert, int32_t max_slash);

/* Message of the last failing call on this thread ("" if none). */
const char* lcsr_last_error(void);

/* lcsr_softmax_scale — the logit scale every attention call takes in
 * lcsr_problem_t.sm_scale: 1 / (t sqrt(head_dim)) with the YaRN attention
 * temperature sqrt(1/t) = 0.1 ln(s) + 1, s = rope->yarn_factor
 * ([Qwen2.5-1M explainer] Length Extrapolation, YaRN Attention Scaling);
 * s <= 1 means no temperature, 1 / sqrt(head_dim).  Formed in double and
 * returned rounded to float.  Host only; launches nothing.
 * Errors: returns 0 (message in lcsr_last_error) for a NULL rope,
 * head_dim <= 0 or a yarn_factor that is NaN or infinite. */
float lcsr_softmax_scale(const lcsr_rope_t* rope, int32_t head_dim);

/* lcsr_rope_yarn_apply — y[h, t, :] = scale * R(pos[t]) x[h, t, :], stored
 * bf16 (or fp16).  Rotation pairs (x_p, x_{p+D/2}) turn by pos[t] * theta_p
 * (rotate_half, [architecture overview] §2.4 code; relative-position
 * property, [long-context blog] RoPE原理の復習).  In the chunk loop, pos is
 * P_k of the chunk's tokens and y is the chunk's rows of the K cache
 * (fp16).
 *   x      [n_heads, n_tok, head_dim], x_dtype LCSR_BF16 or LCSR_FP32
 *   y      bf16 (fp16 with LCSR_ROPE_OUT_FP16) [n_heads, n_tok, head_dim],
 *          rounded to nearest; may equal x (in place) only when x is bf16
 *          with the same strides
 *   pos    int32 [n_tok] (device), positions >= 0
 *   rope   (host) frequency setup; scale multiplies the result (1 = none)
 *   flags  LCSR_ROPE_NO_ROTATE: y = scale * x (a dtype conversion/copy,
 *          used to fill the V cache); pos may then be NULL.
 *          LCSR_ROPE_OUT_FP16: y is fp16 (the K cache of the attention
 *          calls).
 * Errors: LCSR_EINVAL for null pointers, odd head_dim, head_dim > 256,
 * misalignment; LCSR_EHIP if the launch fails. */
int lcsr_rope_yarn_apply(const void* x, int32_t x_dtype, int64_t x_stride_h,
                         int64_t x_stride_t, void* y, int64_t y_stride_h,
                         int64_t y_stride_t, int64_t n_heads, int64_t n_tok,
                         int64_t head_dim, const int32_t* pos,
                         const lcsr_rope_t* rope, float scale, uint32_t flags,
                         void* stream);

/* lcsr_pattern_fill_a_shape — the A-shape head pattern (attention sinks plus
 * a sliding window, [architecture overview] §4.1; one pattern per head,
 * §4.2) written into the rows of `pat` whose head_mask entry is non-zero
 * (every row if head_mask is NULL): verticals 0 .. min(n_sink, n_ctx) - 1,
 * slash offsets 0 .. min(n_local, n_ctx) - 1, ascending, the rest of each
 * row -1, and the counts.  Under the vertical-slash rule row i then attends
 * to every j <= i with j < n_sink or i - j < n_local.  Other rows are left
 * as they are, so one pattern can hold A-shape heads beside heads filled by
 * lcsr_vs_pattern_estimate (with the complementary head_mask).
 *   pat        (host struct, device arrays) as for lcsr_vs_pattern_estimate
 *   n_heads    rows of the pattern arrays, 1 .. 64
 *   head_mask  (host) int32 [n_heads] or NULL
 *   n_sink     0 .. pat->max_vert;  n_local 0 .. pat->max_slash
 *   n_ctx      keys visible to the chunk (chunk_start + chunk_len)
 * Asynchronous on `stream`.  Errors: LCSR_EINVAL for a NULL or inconsistent
 * pattern, n_heads out of range, negative sizes or sizes beyond the pattern's
 * row lengths (nothing written); LCSR_EHIP if the launch fails. */
int lcsr_pattern_fill_a_shape(const lcsr_pattern_t* pat, int32_t n_heads,
                              const int32_t* head_mask, int32_t n_sink, int32_t n_local,
                              int64_t n_ctx, void* stream);

/* lcsr_block_sparse_estimate — the block-sparse head pattern of one prefill
 * chunk.  [architecture overview] §4.2 lists a block pattern among the
 * stable head patterns and §4.3 selectors that score whole key blocks per
 * query; [Qwen2.5-1M explainer] アルゴリズム: selection at continuous
 * positions.  Blocks are 64 tokens aligned to the token index; query block
 * qb holds chunk rows [64 qb, 64 qb + 64) and its diagonal key block is
 * diag = chunk_start / 64 + qb.
 *   score[h][qb][kb] = sm_scale <mean_i R(i) q_i, mean_j R(j) k_j>   (kb <= diag)
 * over the block's queries i and keys j (partial last blocks: the mean of
 * the tokens present; keys are read from the K cache at P_k and turned to
 * continuous positions).  Each query block keeps its diagonal and the
 * k - 1 best key blocks kb < diag by (score desc, index asc), with
 * k = min(n_blocks[h], diag + 1).
 *   p            as for the other calls; chunk_start % 64 == 0; at most
 *                32768 key blocks (2M keys); p->v_cache unused
 *   n_blocks     (host) int32 [H], 1 .. max_blocks, kept blocks per query block
 *   head_mask    (host) int32 [H] or NULL; other heads are not touched
 *   blk_idx      int32 [H][n_qb][max_blocks], n_qb = ceil(chunk_len / 64):
 *                kept key blocks ascending, -1 after the count
 *   blk_cnt      int32 [H][n_qb]
 *   scores       fp32 [H][n_qb][n_kb] (n_kb = ceil((chunk_start + chunk_len)
 *                / 64)) or NULL: written with the scores at or below each
 *                diagonal; with LCSR_BS_SELECT_ONLY an input (only the
 *                selection runs)
 *   ws           lcsr_workspace_bytes(LCSR_WS_BLOCK_EST, ...) bytes (not
 *                needed with LCSR_BS_SELECT_ONLY)
 * Asynchronous on `stream`.  Errors: LCSR_EINVAL (shapes, NULL arrays,
 * budgets, chunk_start alignment), LCSR_ENOTSUP (head_dim, context beyond
 * the block limit), LCSR_EWORKSPACE, LCSR_EHIP. */
int lcsr_block_sparse_estimate(const lcsr_problem_t* p, const int32_t* n_blocks,
                               const int32_t* head_mask, int32_t max_blocks, int32_t* blk_idx,
                               int32_t* blk_cnt, float* scores, uint32_t flags, void* ws,
                               size_t ws_bytes, void* stream);

/* lcsr_block_sparse_attn_prefill — attention of the chunk's rows over their
 * query block's kept key blocks: row i attends to every key j <= i inside a
 * listed block, with the DCA logits and temperature of
 * lcsr_vs_sparse_attn_prefill ([Qwen2.5-1M explainer] Length
 * Extrapolation).  out_i = softmax over that set times V; lse_i natural
 * log.  blk_idx / blk_cnt as written by lcsr_block_sparse_estimate (any
 * ascending lists of distinct blocks <= each diagonal are accepted).
 *   out      [H, chunk_len, D] with strides (o_stride_h, o_stride_t),
 *            out_dtype LCSR_FP32 or LCSR_BF16
 *   lse      fp32 [H, chunk_len] (dense) or NULL
 *   stats    int64 [2] or NULL: adds (pairs multiplied on whole 64 x 32
 *            tiles, pairs in the sets)
 *   ws       lcsr_workspace_bytes(LCSR_WS_BLOCK_ATTN, ...) bytes
 * Errors as for lcsr_block_sparse_estimate; LCSR_EINVAL also for a NULL or
 * mistyped output. */
int lcsr_block_sparse_attn_prefill(const lcsr_problem_t* p, const int32_t* blk_idx,
                                   const int32_t* blk_cnt, int32_t max_blocks,
                                   const int32_t* head_mask, void* out, int32_t out_dtype,
                                   int64_t o_stride_h, int64_t o_stride_t, float* lse,
                                   int64_t* stats, void* ws, size_t ws_bytes, void* stream);

/* lcsr_dca_positions — DCA position maps of tokens [tok_start, tok_start +
 * n_tok) ([Qwen2.5-1M explainer] Length Extrapolation, see lcsr_dca_t).
 * Each output is int32 [n_tok] or NULL (not written).  With DCA off every
 * map is the token index.  Errors: LCSR_EINVAL for negative sizes, local
 * outside [0, chunk), or positions beyond int32. */
int lcsr_dca_positions(int64_t tok_start, int64_t n_tok, const lcsr_dca_t* dca,
                       int32_t* pk, int32_t* pq_intra, int32_t* pq_succ,
                       int32_t* pq_inter, void* stream);

/* lcsr_vs_pattern_estimate — choose each head's verticals and slashes for
 * one chunk ([Qwen2.5-1M explainer] 疎アテンション and Chunked Prefill: the
 * chunk's last `last_q` (64) queries attend to all keys; アルゴリズム: with
 * continuous relative positions).  Rows r in [max(c0, c1 - last_q), c1),
 * keys j in [0, c1) with j <= r, c1 = chunk_start + chunk_len;
 * A = row softmax of sm_scale <R(r) q_r, R(j) k_j>; vertical score
 * v_j = sum_r A[r, j], slash score s_o = sum_r A[r, r - o].  Head h keeps
 * the min(n_vert[h], c1) largest v and min(n_slash[h], c1) largest s,
 * ties to the lower index, written ascending into `pat`.  Sums are done in
 * a fixed order, so results are bitwise reproducible.
 *   n_vert, n_slash (host) int32 [H] budgets, <= pat->max_vert/max_slash
 *   head_mask       (host) int32 [H] or NULL; heads with 0 are not touched
 *   vert_score      fp32 [H, c1] or NULL; written (or read, with
 *   slash_score     LCSR_EST_SELECT_ONLY) scores
 *   flags           LCSR_EST_SELECT_ONLY: skip the scores, select from the
 *                   given arrays (both must then be non-NULL)
 *   ws, ws_bytes    workspace >= lcsr_workspace_bytes(LCSR_WS_ESTIMATE)
 * Errors: LCSR_EINVAL, LCSR_ENOTSUP, LCSR_EWORKSPACE, LCSR_EHIP. */
int lcsr_vs_pattern_estimate(const lcsr_problem_t* p, int32_t last_q,
                             const int32_t* n_vert, const int32_t* n_slash,
                             const int32_t* head_mask, const lcsr_pattern_t* pat,
                             float* vert_score, float* slash_score,
                             uint32_t flags, void* ws, size_t ws_bytes,
                             void* stream);

/* lcsr_vs_sparse_attn_prefill — sparse causal attention of the chunk's rows
 * ([Qwen2.5-1M explainer] 疎アテンション: attention over the critical tokens
 * only; アルゴリズム: weights with the DCA positions; temperature from
 * YaRN attention scaling).  For row i: C_i = {v <= i} U {i - o : o <= i};
 * l_ij = sm_scale <R(P_q(i, j)) q_i, R(P_k(j)) k_j>; out_i =
 * softmax(l_i.) over C_i times V; lse_i = log sum exp (natural log).  An
 * empty C_i gives out_i = 0 and lse_i = -inf.
 *   pat        the pattern (e.g. from lcsr_vs_pattern_estimate)
 *   head_mask  (host) int32 [H] or NULL
 *   out        [H, chunk_len, D], out_dtype LCSR_FP32 or LCSR_BF16
 *   lse        fp32 [H, chunk_len] or NULL
 *   stats      int64 [2] or NULL: adds (query, key) pairs multiplied on the
 *              matrix cores (padding included) and pairs in the critical
 *              sets (the algorithmic work)
 *   flags      LCSR_ATTN_DENSE: every causal key (pattern ignored)
 *   ws         workspace >= lcsr_workspace_bytes(LCSR_WS_ATTN)
 * Errors: LCSR_EINVAL, LCSR_ENOTSUP, LCSR_EWORKSPACE, LCSR_EHIP. */
int lcsr_vs_sparse_attn_prefill(const lcsr_problem_t* p, const lcsr_pattern_t* pat,
                                const int32_t* head_mask, void* out,
                                int32_t out_dtype, int64_t o_stride_h,
                                int64_t o_stride_t, float* lse, int64_t* stats,
                                uint32_t flags, void* ws, size_t ws_bytes,
                                void* stream);

/* lcsr_attn_decode — decode-step attention: the sequence's newest rows,
 * tokens i = chunk_start .. chunk_start + chunk_len - 1 (their K and V
 * already in the caches), against every key j <= i, with the same DCA logits
 * and temperature as the prefill ([Qwen2.5-1M explainer] Length
 * Extrapolation: intra / successive / inter relations; アルゴリズム: weights
 * with the DCA positions).  Dense (no pattern): a decode step reads the whole
 * K/V prefix once and is bound by HBM bandwidth (long-context engineering
 * page, §7.1).  out_i = softmax(l_i.) over j <= i times V; lse_i natural log.
 *   p          chunk_start may be any token (no 64-token alignment with
 *              DCA); (n_heads / n_kv_heads) x chunk_len <= 32
 *   out        [H, chunk_len, D] with strides o_stride_h / o_stride_t,
 *              out_dtype LCSR_FP32 or LCSR_BF16, 16-byte aligned
 *   lse        fp32 [H, chunk_len] or NULL
 *   ws         workspace >= lcsr_workspace_bytes(LCSR_WS_DECODE)
 * Results are bitwise reproducible (the key splits merge in a fixed order).
 * Errors: LCSR_EINVAL, LCSR_ENOTSUP, LCSR_EWORKSPACE, LCSR_EHIP. */
int lcsr_attn_decode(const lcsr_problem_t* p, void* out, int32_t out_dtype,
                     int64_t o_stride_h, int64_t o_stride_t, float* lse, void* ws,
                     size_t ws_bytes, void* stream);

/* lcsr_attn_decode_noalloc — lcsr_attn_decode without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops that forbid allocation).  Same arguments, results
 * and errors as lcsr_attn_decode; the workspace is a static device array of
 * the library (8 MiB per GPU, held until the process ends), which bounds
 * every problem lcsr_attn_decode accepts (LCSR_ENOTSUP otherwise).  The call
 * allocates nothing and launches the same kernels.  Calls on one GPU share
 * that array: calls that may overlap on one GPU (different streams) race and
 * must be serialised by the caller.  Asynchronous on `stream`. */
int lcsr_attn_decode_noalloc(const lcsr_problem_t* p, void* out, int32_t out_dtype,
                             int64_t o_stride_h, int64_t o_stride_t, float* lse,
                             void* stream);

/* lcsr_block_sparse_recall_check — attention recall of sampled rows for a
 * block-sparse pattern ([Qwen2.5-1M explainer] Chunked Prefill), C_i being
 * every key j <= i inside the kept blocks of i's query block (the set of
 * lcsr_block_sparse_attn_prefill), same logits.  The blocks come from
 * blk_idx / blk_cnt as written by lcsr_block_sparse_estimate; entries
 * outside [0, the row's block] are ignored.
 *   rows       int32 [n_rows], offsets within the chunk
 *   lse_full, lse_sparse, recall   fp32 [H, n_rows]
 * No workspace.  Errors: LCSR_EINVAL, LCSR_ENOTSUP, LCSR_EHIP. */
int lcsr_block_sparse_recall_check(const lcsr_problem_t* p, const int32_t* blk_idx,
                                   const int32_t* blk_cnt, int32_t max_blocks,
                                   const int32_t* head_mask, const int32_t* rows,
                                   int32_t n_rows, float* lse_full, float* lse_sparse,
                                   float* recall, void* stream);

/* lcsr_attn_recall_check — attention recall of sampled rows
 * ([Qwen2.5-1M explainer] Chunked Prefill: lse_full over every j <= i,
 * lse_sparse over C_i, recall = exp(lse_sparse - lse_full)), with the same
 * DCA logits and temperature as the attention.
 *   rows       int32 [n_rows], offsets within the chunk (0 <= r < chunk_len)
 *   lse_full, lse_sparse, recall   fp32 [H, n_rows]
 *   ws         workspace >= lcsr_workspace_bytes(LCSR_WS_RECALL)
 * Errors: LCSR_EINVAL, LCSR_ENOTSUP, LCSR_EWORKSPACE, LCSR_EHIP. */
int lcsr_attn_recall_check(const lcsr_problem_t* p, const lcsr_pattern_t* pat,
                           const int32_t* head_mask, const int32_t* rows,
                           int32_t n_rows, float* lse_full, float* lse_sparse,
                           float* recall, void* ws, size_t ws_bytes,
                           void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LCSR_H */
