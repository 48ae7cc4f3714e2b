// Attention recall of sampled rows (page: "論文解説: Qwen2.5-1M"
// (0h-n0.github.io), Chunked Prefill: softmax_lse_full over every causal
// key, softmax_lse_sparse over the critical set C, recall =
// exp(lse_sparse - lse_full)), with the DCA logits and YaRN temperature of
// the attention itself.  Off the timed path: one workgroup per (row, head),
// a plain fp32 dot product per key on the vector ALUs, an independent check
// of the matrix-core attention.
#include <cmath>

#include "lcsr_internal.h"

namespace lcsr {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kRecallThreads = 256;

struct RecallArgs {
  const void* q;
  int32_t q_dtype;
  int64_t q_sh, q_st;
  const uint16_t* k;      // K cache (fp16)
  int64_t kv_sh, kv_st;
  int32_t H, G, D;
  int64_t c0, L, n_ctx;
  DcaParams dca;
  FreqTable ft;
  float scale_log2;
  const uint32_t* off_bits;
  const uint32_t* col_bits;
  int64_t n_words;
  uint64_t head_mask;
  const int32_t* rows;
  int32_t n_rows;
  // block-sparse sets instead of the bitmaps (blk_idx != nullptr): the kept
  // 64-key blocks of each (head, 64-row query block)
  const int32_t* blk_idx;
  const int32_t* blk_cnt;
  int32_t max_blocks;
  int64_t n_qb;
  float* lse_full;
  float* lse_sparse;
  float* recall;
};

__device__ __forceinline__ bool bit_at(const uint32_t* bm, int64_t pos) {
  return pos >= 0 && ((bm[pos >> 5] >> (pos & 31)) & 1u);
}

__device__ __forceinline__ void lse_merge(float& m, float& l, float m2, float l2) {
  const float mm = fmaxf(m, m2);
  if (mm == -INFINITY) return;
  l = l * exp2f(m - mm) + l2 * exp2f(m2 - mm);
  m = mm;
}

__global__ void __launch_bounds__(kRecallThreads) recall_kernel(RecallArgs a) {
  const int k = blockIdx.x, h = blockIdx.y;
  if (!((a.head_mask >> h) & 1)) return;
  __shared__ float qv[3][128];
  __shared__ float red[4][kRecallThreads / 64];
  __shared__ uint32_t kept[kMaxKeyBlocks / 32];
  const int64_t out_i = (int64_t)h * a.n_rows + k;
  const int32_t t = a.rows[k];
  if (t < 0 || t >= a.L) {  // row outside the chunk: NaN results
    if (threadIdx.x == 0) {
      a.lse_full[out_i] = NAN;
      a.lse_sparse[out_i] = NAN;
      a.recall[out_i] = NAN;
    }
    return;
  }
  const int64_t i = a.c0 + t;
  const int half = a.D / 2;
  const int n_var = a.dca.period ? 3 : 1;
  // rotated query variants, rounded to fp16 as the matrix-core path feeds them
  for (int x = threadIdx.x; x < n_var * half; x += kRecallThreads) {
    const int v = x / half, p = x % half;
    const int64_t pos = dca_query_pos(i, v, a.dca);
    float c, s;
    rope_cos_sin(pos, a.ft.inv_freq[p], &c, &s);
    const int64_t off = h * a.q_sh + (int64_t)t * a.q_st;
    float x1, x2;
    if (a.q_dtype == LCSR_FP32) {
      x1 = static_cast<const float*>(a.q)[off + p];
      x2 = static_cast<const float*>(a.q)[off + p + half];
    } else {
      x1 = bf16_to_f32(static_cast<const uint16_t*>(a.q)[off + p]);
      x2 = bf16_to_f32(static_cast<const uint16_t*>(a.q)[off + p + half]);
    }
    x1 = bf16_to_f32(f32_to_bf16(x1));
    x2 = bf16_to_f32(f32_to_bf16(x2));
    qv[v][p] = f16_to_f32(f32_to_f16(x1 * c - x2 * s));
    qv[v][p + half] = f16_to_f32(f32_to_f16(x2 * c + x1 * s));
  }
  const bool blocks = a.blk_idx != nullptr;
  if (blocks) {
    // this row's kept key blocks as a bitmap (blocks past the diagonal or
    // negative are ignored, like the attention kernel's guard keeps loads in
    // bounds; they hold no key j <= i)
    const int64_t nw = (i / 64) / 32 + 1;
    for (int64_t x = threadIdx.x; x < nw; x += kRecallThreads) kept[x] = 0u;
    __syncthreads();
    const int64_t qb = t / 64;
    const int32_t* list = a.blk_idx + ((int64_t)h * a.n_qb + qb) * a.max_blocks;
    int n = a.blk_cnt[(int64_t)h * a.n_qb + qb];
    n = n < a.max_blocks ? n : a.max_blocks;
    for (int x = threadIdx.x; x < n; x += kRecallThreads) {
      const int32_t b = list[x];
      if (b >= 0 && b <= i / 64) atomicOr(&kept[b >> 5], 1u << (b & 31));
    }
  }
  __syncthreads();
  const int g = h / a.G;
  const uint16_t* kb = a.k + (int64_t)g * a.kv_sh;
  const uint32_t* ob = a.off_bits + (int64_t)h * a.n_words + kBitPad;
  const uint32_t* cb = a.col_bits + (int64_t)h * a.n_words + kBitPad;
  const int64_t qc = a.dca.period ? i / a.dca.period : 0;
  float mf = -INFINITY, lf = 0.f, ms = -INFINITY, ls = 0.f;
  for (int64_t j = threadIdx.x; j <= i; j += kRecallThreads) {
    const int64_t kc = a.dca.period ? j / a.dca.period : 0;
    const int64_t rel = qc - kc;
    const int v = n_var == 1 ? 0 : (rel >= 2 ? 2 : (int)rel);
    const uint16_t* kr = kb + j * a.kv_st;
    float dot = 0.f;
    for (int d = 0; d < a.D; d += 8) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(kr + d);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dot += qv[v][d + 2 * e] * f16_to_f32((uint16_t)(w[e] & 0xFFFFu));
        dot += qv[v][d + 2 * e + 1] * f16_to_f32((uint16_t)(w[e] >> 16));
      }
    }
    const float x = dot * a.scale_log2;
    lse_merge(mf, lf, x, 1.f);
    const bool in_set = blocks ? ((kept[j >> 11] >> ((j >> 6) & 31)) & 1u)
                               : (bit_at(cb, j) || bit_at(ob, i - j));
    if (in_set) lse_merge(ms, ls, x, 1.f);
  }
  // block reduction in a fixed order
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int off = 32; off > 0; off >>= 1) {
    lse_merge(mf, lf, __shfl_xor(mf, off), __shfl_xor(lf, off));
    lse_merge(ms, ls, __shfl_xor(ms, off), __shfl_xor(ls, off));
  }
  if (lane == 0) {
    red[0][w] = mf;
    red[1][w] = lf;
    red[2][w] = ms;
    red[3][w] = ls;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float Mf = -INFINITY, Lf = 0.f, Ms = -INFINITY, Ls = 0.f;
    for (int x = 0; x < kRecallThreads / 64; ++x) {
      lse_merge(Mf, Lf, red[0][x], red[1][x]);
      lse_merge(Ms, Ls, red[2][x], red[3][x]);
    }
    const float full = Lf > 0.f ? (Mf + log2f(Lf)) * kLn2 : -INFINITY;
    const float sparse = Ls > 0.f ? (Ms + log2f(Ls)) * kLn2 : -INFINITY;
    a.lse_full[out_i] = full;
    a.lse_sparse[out_i] = sparse;
    a.recall[out_i] = Ls > 0.f ? expf(sparse - full) : 0.f;
  }
}

}  // namespace

int run_recall(const lcsr_problem_t& p, const lcsr_pattern_t& pat, uint64_t head_mask,
               const int32_t* rows, int32_t n_rows, float* lse_full, float* lse_sparse,
               float* recall, char* ws, hipStream_t s) {
  const AttnLayout L = attn_layout(p, pat.max_vert, pat.max_slash, false);
  int rc = build_pattern_aux(p, pat, head_mask, false, L, ws, s);
  if (rc) return rc;
  RecallArgs a{};
  rc = build_freq_table(&p.rope, p.head_dim, &a.ft);
  if (rc) return rc;
  a.q = p.q;
  a.q_dtype = p.q_dtype;
  a.q_sh = p.q_stride_h;
  a.q_st = p.q_stride_t;
  a.k = static_cast<const uint16_t*>(p.k_cache);
  a.kv_sh = p.kv_stride_h;
  a.kv_st = p.kv_stride_t;
  a.H = p.n_heads;
  a.G = p.n_heads / p.n_kv_heads;
  a.D = p.head_dim;
  a.c0 = p.chunk_start;
  a.L = p.chunk_len;
  a.n_ctx = L.n_ctx;
  a.dca = make_dca(&p.dca);
  a.scale_log2 = p.sm_scale * kLog2e;
  a.off_bits = reinterpret_cast<const uint32_t*>(ws + L.o_off_bits);
  a.col_bits = reinterpret_cast<const uint32_t*>(ws + L.o_col_bits);
  a.n_words = L.n_words;
  a.head_mask = head_mask;
  a.rows = rows;
  a.n_rows = n_rows;
  a.lse_full = lse_full;
  a.lse_sparse = lse_sparse;
  a.recall = recall;
  hipLaunchKernelGGL(recall_kernel, dim3((unsigned)n_rows, (unsigned)p.n_heads),
                     dim3(kRecallThreads), 0, s, a);
  return check_launch("recall");
}

int run_block_recall(const lcsr_problem_t& p, const int32_t* idx, const int32_t* cnt,
                     int32_t max_blocks, uint64_t head_mask, const int32_t* rows,
                     int32_t n_rows, float* lse_full, float* lse_sparse, float* recall,
                     hipStream_t s) {
  RecallArgs a{};
  int rc = build_freq_table(&p.rope, p.head_dim, &a.ft);
  if (rc) return rc;
  a.q = p.q;
  a.q_dtype = p.q_dtype;
  a.q_sh = p.q_stride_h;
  a.q_st = p.q_stride_t;
  a.k = static_cast<const uint16_t*>(p.k_cache);
  a.kv_sh = p.kv_stride_h;
  a.kv_st = p.kv_stride_t;
  a.H = p.n_heads;
  a.G = p.n_heads / p.n_kv_heads;
  a.D = p.head_dim;
  a.c0 = p.chunk_start;
  a.L = p.chunk_len;
  a.n_ctx = p.chunk_start + p.chunk_len;
  a.dca = make_dca(&p.dca);
  a.scale_log2 = p.sm_scale * kLog2e;
  a.head_mask = head_mask;
  a.rows = rows;
  a.n_rows = n_rows;
  a.lse_full = lse_full;
  a.lse_sparse = lse_sparse;
  a.recall = recall;
  a.blk_idx = idx;
  a.blk_cnt = cnt;
  a.max_blocks = max_blocks;
  a.n_qb = (p.chunk_len + 63) / 64;
  hipLaunchKernelGGL(recall_kernel, dim3((unsigned)n_rows, (unsigned)p.n_heads),
                     dim3(kRecallThreads), 0, s, a);
  return check_launch("block recall");
}

}  // namespace lcsr
