// C-ABI entry points: argument validation, workspace sizing, dispatch.
#include <cmath>
#include <cstdarg>
#include <cstring>

#include "lcsr_internal.h"

namespace lcsr {

namespace {
thread_local char g_err[512] = "";
}

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(LCSR_EHIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return LCSR_OK;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

EstimateLayout estimate_layout(const lcsr_problem_t& p) {
  EstimateLayout L{};
  const int64_t H = p.n_heads, D = p.head_dim;
  L.n_ctx = p.chunk_start + p.chunk_len;
  L.n_tiles = (L.n_ctx + kTileK - 1) / kTileK;
  const int64_t period = p.dca.chunk > 0 ? p.dca.chunk - p.dca.local : 0;
  L.n_kc = period ? (L.n_ctx + period - 1) / period : 1;
  // key-range splits per KV head: about 1024 workgroups in total
  int64_t want = (1024 + p.n_kv_heads - 1) / p.n_kv_heads;
  L.n_split = want < L.n_tiles ? want : L.n_tiles;
  if (L.n_split < 1) L.n_split = 1;
  L.q_est = align256((size_t)L.n_kc * H * kEstRows * D * 2);
  // one partial per key split, plus one for the keys past DCA chunk edges
  // inside 64-key tiles (scored apart, with the next chunk's query rows)
  L.part = align256((size_t)H * (L.n_split + 1) * kEstRows * 2 * sizeof(float));
  L.lse = align256((size_t)H * kEstRows * sizeof(float));
  L.vscore = align256((size_t)H * L.n_ctx * sizeof(float));
  L.sscore = L.vscore;
  // slash-score parts at the key-split boundaries: five per lane of 32
  L.bnd = align256((size_t)H * L.n_split * 5 * 32 * sizeof(float));
  L.topk = align256(topk_workspace(L.n_ctx, (int)H));
  L.total = L.q_est + L.part + L.lse + L.vscore + L.sscore + L.bnd + L.topk;
  return L;
}

AttnLayout attn_layout(const lcsr_problem_t& p, int32_t max_vert, int32_t max_slash,
                       bool attention) {
  AttnLayout L{};
  const int64_t H = p.n_heads, D = p.head_dim;
  const int64_t G = p.n_kv_heads > 0 ? p.n_heads / p.n_kv_heads : 1;
  L.n_ctx = p.chunk_start + p.chunk_len;
  L.n_words = (L.n_ctx + 31) / 32 + 2 * kBitPad;   // per-head stride, zero words at both ends
  L.n_var = p.dca.chunk > 0 ? 3 : 1;
  L.n_rb = (p.chunk_len + kRowBlock - 1) / kRowBlock;
  L.n_sub = (G + kMaxAttnWaves - 1) / kMaxAttnWaves;
  L.nw = (G + L.n_sub - 1) / L.n_sub;
  L.n_wgg = p.n_kv_heads * L.n_sub;
  L.ubw = (L.n_ctx + 32 * kGranule - 1) / (32 * kGranule);
  L.with_plan = attention;
  if (max_vert < 1) max_vert = 1;
  if (max_slash < 1) max_slash = 1;
  size_t off = 0;
  L.o_q_rot = off;
  off += attention ? align256((size_t)L.n_var * H * p.chunk_len * D * 2) : 0;
  L.o_off_bits = off;
  off += align256((size_t)H * L.n_words * 4);
  L.o_col_bits = off;
  off += align256((size_t)H * L.n_words * 4);
  L.o_runs = off;
  off += align256((size_t)H * max_slash * 2 * 4);
  L.o_run_cnt = off;
  off += align256((size_t)H * 4);
  L.o_union = off;
  off += attention ? align256((size_t)L.n_wgg * L.n_rb * L.ubw * 4) : 0;
  L.o_first = off;  // 4 bits per granule: first pair key of each marked granule
  off += attention ? align256((size_t)L.n_wgg * L.n_rb * L.ubw * 16) : 0;
  L.o_vl = off;
  off += attention ? align256((size_t)H * L.n_rb * max_vert * 4) : 0;
  L.o_vl_cnt = off;
  off += attention ? align256((size_t)H * L.n_rb * 4) : 0;
  L.total = off;
  return L;
}

// Decode workspace: the rows' query variants, then per (KV head, key split)
// the partial O [32][D] and (m, l) [32][2] of the 32 matrix rows.
DecodeLayout decode_layout(const lcsr_problem_t& p) {
  DecodeLayout L{};
  const int64_t H = p.n_heads, D = p.head_dim;
  L.n_ctx = p.chunk_start + p.chunk_len;
  L.n_tiles = (L.n_ctx + kTileK - 1) / kTileK;
  L.n_var = p.dca.chunk > 0 ? 3 : 1;
  // one workgroup per compute unit (256) over the KV heads
  const int64_t want = (kMaxDecSplit + p.n_kv_heads - 1) / (p.n_kv_heads > 0 ? p.n_kv_heads : 1);
  L.n_split = want < L.n_tiles ? want : L.n_tiles;
  if (L.n_split < 1) L.n_split = 1;
  size_t off = 0;
  L.o_q_rot = off;
  off += align256((size_t)L.n_var * H * (p.chunk_len > 0 ? p.chunk_len : 1) * D * 2);
  L.o_part_o = off;
  off += align256((size_t)p.n_kv_heads * L.n_split * 32 * D * 4);
  L.o_part_ml = off;
  off += align256((size_t)p.n_kv_heads * L.n_split * 32 * 2 * 4);
  L.total = off;
  return L;
}

}  // namespace lcsr

using namespace lcsr;

namespace {

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

// any_start: the rows may start anywhere (decode); otherwise, with DCA, the
// chunk must start on a 64-token tile.  period_align: the DCA key period S =
// chunk - local must be a multiple of it (32 for the vertical-slash
// attention, whose 32-row blocks share one query variant; 1 elsewhere).
// Every call takes S >= 64, so a 64-key tile meets at most one edge.
int validate_problem(const lcsr_problem_t* p, bool need_v, bool any_start = false,
                     int64_t period_align = 1) {
  if (!p) return fail(LCSR_EINVAL, "problem is NULL");
  // an empty chunk reads no query (its pointer may be NULL)
  if ((!p->q && p->chunk_len > 0) || !p->k_cache || (need_v && !p->v_cache))
    return fail(LCSR_EINVAL, "q/k_cache/v_cache pointer is NULL");
  if (!aligned16(p->q) || !aligned16(p->k_cache) || (need_v && !aligned16(p->v_cache)))
    return fail(LCSR_EINVAL, "q/k_cache/v_cache must be 16-byte aligned");
  if (p->q_dtype != LCSR_BF16 && p->q_dtype != LCSR_FP32)
    return fail(LCSR_EINVAL, "q_dtype must be LCSR_BF16 or LCSR_FP32");
  if (p->n_heads <= 0 || p->n_kv_heads <= 0 || p->n_heads % p->n_kv_heads)
    return fail(LCSR_EINVAL, "n_heads %d must be a positive multiple of n_kv_heads %d",
                p->n_heads, p->n_kv_heads);
  if (p->n_heads > kMaxHeads || p->n_heads / p->n_kv_heads > kMaxGroup)
    return fail(LCSR_ENOTSUP, "n_heads <= %d and n_heads/n_kv_heads <= %d supported",
                kMaxHeads, kMaxGroup);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(LCSR_ENOTSUP, "head_dim %d not supported (64 or 128)", p->head_dim);
  if (p->chunk_start < 0 || p->chunk_len < 0)
    return fail(LCSR_EINVAL, "chunk_start and chunk_len must be >= 0");
  const int64_t n_ctx = p->chunk_start + p->chunk_len;
  if (n_ctx > (int64_t)1 << 30)
    return fail(LCSR_ENOTSUP, "contexts beyond 2^30 tokens are not supported");
  const int64_t D = p->head_dim;
  if (p->q_stride_t < D || p->q_stride_h < D || p->kv_stride_t < D || p->kv_stride_h < D)
    return fail(LCSR_EINVAL, "strides must be >= head_dim");
  if (p->q_stride_t % 8 || p->q_stride_h % 8 || p->kv_stride_t % 8 || p->kv_stride_h % 8)
    return fail(LCSR_EINVAL, "strides must be multiples of 8 elements");
  if (p->dca.chunk < 0) return fail(LCSR_EINVAL, "dca.chunk must be >= 0");
  if (p->dca.chunk > 0) {
    if (p->dca.local < 0 || p->dca.local >= p->dca.chunk)
      return fail(LCSR_EINVAL, "dca.local must be in [0, dca.chunk)");
    const int64_t period = p->dca.chunk - p->dca.local;
    if (period < kTileK || period % period_align)
      return fail(LCSR_ENOTSUP, "with DCA, chunk - local (%lld) must be >= %d and a multiple "
                  "of %lld for this call", (long long)period, kTileK, (long long)period_align);
    if (!any_start && p->chunk_start % kTileK)
      return fail(LCSR_ENOTSUP, "with DCA, chunk_start must be a multiple of %d", kTileK);
    if (p->dca.chunk > ((int64_t)1 << 30))
      return fail(LCSR_ENOTSUP, "dca.chunk beyond 2^30");
  }
  if (!(p->sm_scale > 0.0f) || !std::isfinite(p->sm_scale))
    return fail(LCSR_EINVAL, "sm_scale must be finite and > 0");
  return LCSR_OK;
}

int head_mask_bits(const lcsr_problem_t* p, const int32_t* head_mask, uint64_t* bits) {
  uint64_t m = 0;
  for (int h = 0; h < p->n_heads; ++h)
    if (!head_mask || head_mask[h]) m |= (uint64_t)1 << h;
  *bits = m;
  return LCSR_OK;
}

int validate_pattern(const lcsr_problem_t* p, const lcsr_pattern_t* pat, bool write) {
  if (!pat) return fail(LCSR_EINVAL, "pattern is NULL");
  if (pat->max_vert < 0 || pat->max_slash < 0)
    return fail(LCSR_EINVAL, "max_vert / max_slash must be >= 0");
  if (!pat->vert_cnt || !pat->slash_cnt)
    return fail(LCSR_EINVAL, "vert_cnt / slash_cnt must not be NULL");
  if ((pat->max_vert > 0 && !pat->vert_idx) || (pat->max_slash > 0 && !pat->slash_idx))
    return fail(LCSR_EINVAL, "vert_idx / slash_idx must not be NULL");
  if (pat->max_vert > (1 << 24) || pat->max_slash > (1 << 24))
    return fail(LCSR_ENOTSUP, "max_vert / max_slash beyond 2^24");
  (void)p;
  (void)write;
  return LCSR_OK;
}

}  // namespace

extern "C" {

const char* lcsr_last_error(void) { return g_err; }

float lcsr_softmax_scale(const lcsr_rope_t* rope, int32_t head_dim) {
  if (!rope) {
    set_error("rope is NULL");
    return 0.0f;
  }
  if (head_dim <= 0) {
    set_error("head_dim must be > 0, got %d", head_dim);
    return 0.0f;
  }
  const double s = rope->yarn_factor;
  if (!std::isfinite(s)) {
    set_error("yarn_factor must be finite");
    return 0.0f;
  }
  // sqrt(1/t) = 0.1 ln s + 1 for s > 1; no temperature otherwise
  const double m = s > 1.0 ? 0.1 * std::log(s) + 1.0 : 1.0;
  return (float)(m * m / std::sqrt((double)head_dim));
}

size_t lcsr_workspace_bytes(int which, const lcsr_problem_t* p, int32_t max_vert,
                            int32_t max_slash) {
  const int64_t align = which == LCSR_WS_ATTN ? kRowBlock : 1;
  if (!p || validate_problem(p, false, which == LCSR_WS_DECODE, align) != LCSR_OK) return 0;
  switch (which) {
    case LCSR_WS_ESTIMATE: return estimate_layout(*p).total;
    case LCSR_WS_ATTN: return attn_layout(*p, max_vert, max_slash, true).total;
    case LCSR_WS_RECALL: return attn_layout(*p, max_vert, max_slash, false).total;
    case LCSR_WS_DECODE: return decode_layout(*p).total;
    case LCSR_WS_BLOCK_EST: return block_layout(*p).est_total;
    case LCSR_WS_BLOCK_ATTN: return block_layout(*p).attn_total;
    default: set_error("unknown workspace kind %d", which); return 0;
  }
}

int lcsr_rope_yarn_apply(const void* x, int32_t x_dtype, int64_t x_stride_h,
                         int64_t x_stride_t, void* y, int64_t y_stride_h,
                         int64_t y_stride_t, int64_t n_heads, int64_t n_tok,
                         int64_t head_dim, const int32_t* pos,
                         const lcsr_rope_t* rope, float scale, uint32_t flags,
                         void* stream) {
  const bool rotate = !(flags & LCSR_ROPE_NO_ROTATE);
  if (!x || !y) return fail(LCSR_EINVAL, "x / y is NULL");
  if (rotate && !pos) return fail(LCSR_EINVAL, "pos is NULL");
  if (x_dtype != LCSR_BF16 && x_dtype != LCSR_FP32)
    return fail(LCSR_EINVAL, "x_dtype must be LCSR_BF16 or LCSR_FP32");
  if (n_heads < 0 || n_tok < 0) return fail(LCSR_EINVAL, "negative size");
  if (head_dim <= 0 || head_dim % 2 || head_dim > 2 * kMaxRopeHalf)
    return fail(LCSR_EINVAL, "head_dim must be even and <= %d", 2 * kMaxRopeHalf);
  if (x_stride_t < head_dim || y_stride_t < head_dim ||
      (n_heads > 1 && (x_stride_h < head_dim || y_stride_h < head_dim)))
    return fail(LCSR_EINVAL, "strides must be >= head_dim");
  if (x == y && (x_dtype != LCSR_BF16 || x_stride_h != y_stride_h || x_stride_t != y_stride_t))
    return fail(LCSR_EINVAL, "in-place needs bf16 x with the same strides");
  if (!std::isfinite(scale)) return fail(LCSR_EINVAL, "scale must be finite");
  FreqTable ft;
  int rc = build_freq_table(rope, head_dim, &ft);
  if (rc) return rc;
  RotateArgs a{};
  a.src = x;
  a.src_dtype = x_dtype;
  a.src_sh = x_stride_h;
  a.src_st = x_stride_t;
  a.dst = static_cast<uint16_t*>(y);
  a.dst_dtype = (flags & LCSR_ROPE_OUT_FP16) ? LCSR_FP16 : LCSR_BF16;
  a.dst_sh = y_stride_h;
  a.dst_st = y_stride_t;
  a.n_heads = n_heads;
  a.n_tok = n_tok;
  a.head_dim = head_dim;
  a.pos = pos;
  a.mode = rotate ? kPosArray : kNoRotate;
  a.scale = scale;
  return launch_rotate(a, ft, static_cast<hipStream_t>(stream));
}

int lcsr_dca_positions(int64_t tok_start, int64_t n_tok, const lcsr_dca_t* dca,
                       int32_t* pk, int32_t* pq_intra, int32_t* pq_succ,
                       int32_t* pq_inter, void* stream) {
  if (!dca) return fail(LCSR_EINVAL, "dca is NULL");
  if (tok_start < 0 || n_tok < 0) return fail(LCSR_EINVAL, "negative token range");
  if (dca->chunk < 0 || (dca->chunk > 0 && (dca->local < 0 || dca->local >= dca->chunk)))
    return fail(LCSR_EINVAL, "need chunk >= 0 and 0 <= local < chunk");
  if (tok_start + n_tok > ((int64_t)1 << 31) - 1)
    return fail(LCSR_EINVAL, "positions beyond int32");
  return launch_dca_positions(tok_start, n_tok, make_dca(dca), pk, pq_intra, pq_succ,
                              pq_inter, static_cast<hipStream_t>(stream));
}

int lcsr_pattern_fill_a_shape(const lcsr_pattern_t* pat, int32_t n_heads,
                              const int32_t* head_mask, int32_t n_sink, int32_t n_local,
                              int64_t n_ctx, void* stream) {
  int rc = validate_pattern(nullptr, pat, true);
  if (rc) return rc;
  if (n_heads < 1 || n_heads > kMaxHeads)
    return fail(LCSR_EINVAL, "n_heads must be in [1, %d]", kMaxHeads);
  if (n_sink < 0 || n_local < 0 || n_ctx < 0)
    return fail(LCSR_EINVAL, "n_sink, n_local and n_ctx must be >= 0");
  if (n_sink > pat->max_vert || n_local > pat->max_slash)
    return fail(LCSR_EINVAL, "n_sink %d / n_local %d exceed max_vert %d / max_slash %d", n_sink,
                n_local, pat->max_vert, pat->max_slash);
  uint64_t mask = 0;
  for (int h = 0; h < n_heads; ++h)
    if (!head_mask || head_mask[h]) mask |= (uint64_t)1 << h;
  const int32_t nv = (int32_t)std::min<int64_t>(n_sink, n_ctx);
  const int32_t ns = (int32_t)std::min<int64_t>(n_local, n_ctx);
  return launch_fill_a_shape(*pat, n_heads, mask, nv, ns, static_cast<hipStream_t>(stream));
}

int lcsr_vs_pattern_estimate(const lcsr_problem_t* p, int32_t last_q,
                             const int32_t* n_vert, const int32_t* n_slash,
                             const int32_t* head_mask, const lcsr_pattern_t* pat,
                             float* vert_score, float* slash_score, uint32_t flags,
                             void* ws, size_t ws_bytes, void* stream) {
  int rc = validate_problem(p, false);
  if (rc) return rc;
  rc = validate_pattern(p, pat, true);
  if (rc) return rc;
  const bool select_only = flags & LCSR_EST_SELECT_ONLY;
  if (select_only && (!vert_score || !slash_score))
    return fail(LCSR_EINVAL, "LCSR_EST_SELECT_ONLY needs both score arrays");
  if (last_q < 1 || last_q > kEstRows)
    return fail(LCSR_EINVAL, "last_q must be in [1, %d]", kEstRows);
  if (!n_vert || !n_slash) return fail(LCSR_EINVAL, "budgets are NULL");
  HeadSet hs{};
  head_mask_bits(p, head_mask, &hs.mask);
  for (int h = 0; h < p->n_heads; ++h) {
    if (n_vert[h] < 0 || n_vert[h] > pat->max_vert || n_slash[h] < 0 ||
        n_slash[h] > pat->max_slash)
      return fail(LCSR_EINVAL, "head %d budget (%d, %d) outside [0, max]", h, n_vert[h],
                  n_slash[h]);
    hs.n_vert[h] = n_vert[h];
    hs.n_slash[h] = n_slash[h];
  }
  if ((vert_score && !aligned16(vert_score)) || (slash_score && !aligned16(slash_score)))
    return fail(LCSR_EINVAL, "score arrays must be 16-byte aligned");
  const EstimateLayout L = estimate_layout(*p);
  if (!ws || ws_bytes < L.total || !aligned16(ws))
    return fail(LCSR_EWORKSPACE, "estimate needs %zu workspace bytes (16-byte aligned), got %zu",
                L.total, ws_bytes);
  if (p->chunk_len == 0) return LCSR_OK;
  return run_estimate(*p, last_q, hs, *pat, vert_score, slash_score, select_only,
                      static_cast<char*>(ws), static_cast<hipStream_t>(stream));
}

int lcsr_vs_sparse_attn_prefill(const lcsr_problem_t* p, const lcsr_pattern_t* pat,
                                const int32_t* head_mask, void* out, int32_t out_dtype,
                                int64_t o_stride_h, int64_t o_stride_t, float* lse,
                                int64_t* stats, uint32_t flags, void* ws,
                                size_t ws_bytes, void* stream) {
  int rc = validate_problem(p, true, false, kRowBlock);
  if (rc) return rc;
  const bool dense = flags & LCSR_ATTN_DENSE;
  if (!dense) {
    rc = validate_pattern(p, pat, false);
    if (rc) return rc;
  }
  if (p->chunk_len > 0 && (!out || !aligned16(out)))
    return fail(LCSR_EINVAL, "out must be non-NULL and 16-byte aligned");
  if (out_dtype != LCSR_FP32 && out_dtype != LCSR_BF16)
    return fail(LCSR_EINVAL, "out_dtype must be LCSR_FP32 or LCSR_BF16");
  if (o_stride_t < p->head_dim || o_stride_h < p->head_dim || o_stride_t % 8 || o_stride_h % 8)
    return fail(LCSR_EINVAL, "output strides must be >= head_dim and multiples of 8");
  uint64_t hm;
  head_mask_bits(p, head_mask, &hm);
  lcsr_pattern_t empty{};
  const lcsr_pattern_t& P = (dense && !pat) ? empty : *pat;
  const AttnLayout L = attn_layout(*p, dense ? 1 : P.max_vert, dense ? 1 : P.max_slash, true);
  if (!ws || ws_bytes < L.total || !aligned16(ws))
    return fail(LCSR_EWORKSPACE, "attention needs %zu workspace bytes (16-byte aligned), got %zu",
                L.total, ws_bytes);
  if (p->chunk_len == 0) return LCSR_OK;
  return run_attention(*p, P, hm, out, out_dtype, o_stride_h, o_stride_t, lse, stats, dense,
                       static_cast<char*>(ws), static_cast<hipStream_t>(stream));
}

static int validate_blocks(const lcsr_problem_t* p, int32_t max_blocks) {
  if (p->chunk_start % 64)
    return fail(LCSR_EINVAL, "block-sparse calls need chunk_start %% 64 == 0");
  if (max_blocks < 1) return fail(LCSR_EINVAL, "max_blocks must be >= 1");
  const int64_t n_kb = (p->chunk_start + p->chunk_len + 63) / 64;
  if (n_kb > kMaxKeyBlocks)
    return fail(LCSR_ENOTSUP, "block-sparse context limited to %d key blocks of 64",
                kMaxKeyBlocks);
  return LCSR_OK;
}

int lcsr_block_sparse_estimate(const lcsr_problem_t* p, const int32_t* n_blocks,
                               const int32_t* head_mask, int32_t max_blocks, int32_t* blk_idx,
                               int32_t* blk_cnt, float* scores, uint32_t flags, void* ws,
                               size_t ws_bytes, void* stream) {
  int rc = validate_problem(p, false);
  if (rc) return rc;
  rc = validate_blocks(p, max_blocks);
  if (rc) return rc;
  if ((!blk_idx || !blk_cnt) && p->chunk_len > 0)
    return fail(LCSR_EINVAL, "blk_idx / blk_cnt must not be NULL");
  if (!n_blocks) return fail(LCSR_EINVAL, "n_blocks is NULL");
  const bool select_only = flags & LCSR_BS_SELECT_ONLY;
  if (select_only && !scores) return fail(LCSR_EINVAL, "LCSR_BS_SELECT_ONLY needs the scores");
  uint64_t hm;
  head_mask_bits(p, head_mask, &hm);
  for (int h = 0; h < p->n_heads; ++h)
    if (((hm >> h) & 1ull) && (n_blocks[h] < 1 || n_blocks[h] > max_blocks))
      return fail(LCSR_EINVAL, "n_blocks[%d] = %d outside [1, max_blocks %d]", h, n_blocks[h],
                  max_blocks);
  const BlockLayout L = block_layout(*p);
  const size_t need = select_only ? 0 : (scores ? L.o_scores : L.est_total);
  if (need && (!ws || ws_bytes < need || !aligned16(ws)))
    return fail(LCSR_EWORKSPACE, "block estimate needs %zu workspace bytes (16-byte aligned), "
                "got %zu", need, ws_bytes);
  if (p->chunk_len == 0) return LCSR_OK;
  return run_block_estimate(*p, n_blocks, hm, max_blocks, blk_idx, blk_cnt, scores, select_only,
                            static_cast<char*>(ws), static_cast<hipStream_t>(stream));
}

int lcsr_block_sparse_attn_prefill(const lcsr_problem_t* p, const int32_t* blk_idx,
                                   const int32_t* blk_cnt, int32_t max_blocks,
                                   const int32_t* head_mask, void* out, int32_t out_dtype,
                                   int64_t o_stride_h, int64_t o_stride_t, float* lse,
                                   int64_t* stats, void* ws, size_t ws_bytes, void* stream) {
  int rc = validate_problem(p, true);
  if (rc) return rc;
  rc = validate_blocks(p, max_blocks);
  if (rc) return rc;
  if ((!blk_idx || !blk_cnt) && p->chunk_len > 0)
    return fail(LCSR_EINVAL, "blk_idx / blk_cnt must not be NULL");
  if (!out && p->chunk_len > 0) return fail(LCSR_EINVAL, "out must not be NULL");
  if (out_dtype != LCSR_FP32 && out_dtype != LCSR_BF16)
    return fail(LCSR_EINVAL, "out_dtype must be LCSR_FP32 or LCSR_BF16");
  if (o_stride_t < p->head_dim || o_stride_h < p->head_dim)
    return fail(LCSR_EINVAL, "output strides must be >= head_dim");
  uint64_t hm;
  head_mask_bits(p, head_mask, &hm);
  const BlockLayout L = block_layout(*p);
  if (!ws || ws_bytes < L.attn_total || !aligned16(ws))
    return fail(LCSR_EWORKSPACE, "block attention needs %zu workspace bytes (16-byte aligned), "
                "got %zu", L.attn_total, ws_bytes);
  if (p->chunk_len == 0) return LCSR_OK;
  return run_block_attention(*p, blk_idx, blk_cnt, max_blocks, hm, out, out_dtype, o_stride_h,
                             o_stride_t, lse, stats, static_cast<char*>(ws),
                             static_cast<hipStream_t>(stream));
}

int lcsr_attn_decode(const lcsr_problem_t* p, void* out, int32_t out_dtype,
                     int64_t o_stride_h, int64_t o_stride_t, float* lse, void* ws,
                     size_t ws_bytes, void* stream) {
  int rc = validate_problem(p, true, true);
  if (rc) return rc;
  const int G = p->n_heads / p->n_kv_heads;
  if ((int64_t)G * p->chunk_len > 32)
    return fail(LCSR_ENOTSUP, "decode takes (n_heads / n_kv_heads) x chunk_len <= 32 rows, got "
                "%d x %lld", G, (long long)p->chunk_len);
  if (p->chunk_len > 0 && (!out || !aligned16(out)))
    return fail(LCSR_EINVAL, "out must be non-NULL and 16-byte aligned");
  if (out_dtype != LCSR_FP32 && out_dtype != LCSR_BF16)
    return fail(LCSR_EINVAL, "out_dtype must be LCSR_FP32 or LCSR_BF16");
  if (o_stride_t < p->head_dim || o_stride_h < p->head_dim)
    return fail(LCSR_EINVAL, "output strides must be >= head_dim");
  const DecodeLayout L = decode_layout(*p);
  if (!ws || ws_bytes < L.total || !aligned16(ws))
    return fail(LCSR_EWORKSPACE, "decode needs %zu workspace bytes (16-byte aligned), got %zu",
                L.total, ws_bytes);
  if (p->chunk_len == 0) return LCSR_OK;
  return run_decode(*p, out, out_dtype, o_stride_h, o_stride_t, lse, static_cast<char*>(ws),
                    static_cast<hipStream_t>(stream));
}

int lcsr_attn_recall_check(const lcsr_problem_t* p, const lcsr_pattern_t* pat,
                           const int32_t* head_mask, const int32_t* rows, int32_t n_rows,
                           float* lse_full, float* lse_sparse, float* recall, void* ws,
                           size_t ws_bytes, void* stream) {
  int rc = validate_problem(p, false);
  if (rc) return rc;
  rc = validate_pattern(p, pat, false);
  if (rc) return rc;
  if (n_rows < 0) return fail(LCSR_EINVAL, "n_rows must be >= 0");
  if (n_rows > 0 && (!rows || !lse_full || !lse_sparse || !recall))
    return fail(LCSR_EINVAL, "rows and the three outputs must be non-NULL");
  uint64_t hm;
  head_mask_bits(p, head_mask, &hm);
  const AttnLayout L = attn_layout(*p, pat->max_vert, pat->max_slash, false);
  if (!ws || ws_bytes < L.total || !aligned16(ws))
    return fail(LCSR_EWORKSPACE, "recall needs %zu workspace bytes (16-byte aligned), got %zu",
                L.total, ws_bytes);
  if (n_rows == 0 || p->chunk_len == 0) return LCSR_OK;
  return run_recall(*p, *pat, hm, rows, n_rows, lse_full, lse_sparse, recall,
                    static_cast<char*>(ws), static_cast<hipStream_t>(stream));
}

int lcsr_block_sparse_recall_check(const lcsr_problem_t* p, const int32_t* blk_idx,
                                   const int32_t* blk_cnt, int32_t max_blocks,
                                   const int32_t* head_mask, const int32_t* rows,
                                   int32_t n_rows, float* lse_full, float* lse_sparse,
                                   float* recall, void* stream) {
  int rc = validate_problem(p, false);
  if (rc) return rc;
  rc = validate_blocks(p, max_blocks);
  if (rc) return rc;
  if ((!blk_idx || !blk_cnt) && p->chunk_len > 0)
    return fail(LCSR_EINVAL, "blk_idx / blk_cnt must not be NULL");
  if (n_rows < 0) return fail(LCSR_EINVAL, "n_rows must be >= 0");
  if (n_rows > 0 && (!rows || !lse_full || !lse_sparse || !recall))
    return fail(LCSR_EINVAL, "rows and the three outputs must be non-NULL");
  uint64_t hm;
  head_mask_bits(p, head_mask, &hm);
  if (n_rows == 0 || p->chunk_len == 0) return LCSR_OK;
  return run_block_recall(*p, blk_idx, blk_cnt, max_blocks, hm, rows, n_rows, lse_full,
                          lse_sparse, recall, static_cast<hipStream_t>(stream));
}

}  // extern "C"
