// Block-sparse pattern estimate (gfx950): block scores from pooled queries
// and keys, then per (head, query block) the diagonal key block plus the best
// earlier key blocks.
//
// [architecture overview] §4.2 names a block pattern among the stable head
// patterns; §4.3 describes selectors that score whole KV blocks per query and
// attend only inside the chosen ones.  [Qwen2.5-1M explainer] アルゴリズム:
// the selection uses continuous relative positions.
//
// Blocks are 64 tokens, aligned to the token index.  The score of (query
// block qb, key block kb) is sm_scale <mean_i R(i) q_i, mean_j R(j) k_j>.
// The K cache holds R(P_k(j)) k_j with P_k(j) = j - S c(j), so the mean of a
// key block is taken from the cache as it is and the query mean is turned
// back by R(-S c) for key chunk c: <R(-S c) Q, mean R(j - S c) k_j> =
// <Q, mean R(j) k_j>.  A block's chunk c is that of its first key; keys of a
// block after a chunk edge (S need not be a multiple of 64) are turned by
// R(S) into the frame of chunk c before they are averaged.
#include "lcsr_internal.h"

namespace lcsr {
namespace {

constexpr int kBlk = 64;
constexpr int kScoreQb = 4;      // query blocks per score workgroup
constexpr int kScoreSpan = 1024;  // key blocks per score workgroup (grid.z splits the rest)

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

__device__ __forceinline__ float load_q(const void* q, int32_t dtype, int64_t idx) {
  if (dtype == LCSR_FP32) {
    // fp32 inputs are taken at their bf16 value, as every other call does
    return bf16_to_f32(f32_to_bf16(static_cast<const float*>(q)[idx]));
  }
  return bf16_to_f32(static_cast<const uint16_t*>(q)[idx]);
}

// grid (n_kb, H_kv), 64 threads (one rotation pair (p, p + D/2) each): mean
// of each 64-key block of the (fp16) cache in the frame of its first key's
// DCA chunk, stored as float4 [H_kv][D / 4][n_kb] so that lanes of the score
// kernel (one key block each) read consecutive addresses.
__global__ void __launch_bounds__(64) bs_pool_keys(const uint16_t* __restrict__ k, int64_t kv_sh,
                                                   int64_t kv_st, int64_t n_ctx, int D,
                                                   int64_t n_kb, int64_t period, FreqTable ft,
                                                   float* __restrict__ pk) {
  const int64_t kb = blockIdx.x;
  const int g = blockIdx.y;
  const int half = D / 2, p = threadIdx.x;
  if (p >= half) return;
  const int64_t j0 = kb * kBlk;
  const int64_t j1 = j0 + kBlk < n_ctx ? j0 + kBlk : n_ctx;
  // first key of the next DCA chunk, if inside the block
  int64_t edge = j1;
  if (period) {
    const int64_t next = (j0 / period + 1) * period;
    edge = next < j1 ? next : j1;
  }
  const float inv = 1.0f / (float)(j1 - j0);
  const uint16_t* src = k + g * kv_sh;
  float s1 = 0.f, s2 = 0.f;
#pragma unroll 8
  for (int64_t j = j0; j < edge; ++j) {
    s1 += f16_to_f32(src[j * kv_st + p]);
    s2 += f16_to_f32(src[j * kv_st + p + half]);
  }
  if (edge < j1) {
    float c, sn;
    rope_cos_sin(period, ft.inv_freq[p], &c, &sn);
    for (int64_t j = edge; j < j1; ++j) {
      const float x1 = f16_to_f32(src[j * kv_st + p]), x2 = f16_to_f32(src[j * kv_st + p + half]);
      s1 += x1 * c - x2 * sn;
      s2 += x2 * c + x1 * sn;
    }
  }
  pk[(((int64_t)g * (D / 4) + p / 4) * n_kb + kb) * 4 + p % 4] = s1 * inv;
  pk[(((int64_t)g * (D / 4) + (p + half) / 4) * n_kb + kb) * 4 + (p + half) % 4] = s2 * inv;
}

// grid (n_qb, H), 64 threads (one rotation pair each): the block mean of
// R(i) q_i, then turned by R(-S c) for each key chunk c < n_kc:
// pq[c][h][qb][D].
struct PoolQArgs {
  const void* q;
  int32_t q_dtype;
  int64_t q_sh, q_st;
  int64_t c0, L, period;
  int32_t H, D, n_kc;
  int64_t n_qb;
  float* pq;
};

__global__ void __launch_bounds__(64) bs_pool_queries(PoolQArgs a, FreqTable ft) {
  const int64_t qb = blockIdx.x;
  const int h = blockIdx.y;
  const int half = a.D / 2;
  const int p = threadIdx.x;
  if (p >= half) return;
  const int64_t i0 = a.c0 + qb * kBlk;
  const int64_t i1 = i0 + kBlk < a.c0 + a.L ? i0 + kBlk : a.c0 + a.L;
  float s1 = 0.f, s2 = 0.f;
  for (int64_t i = i0; i < i1; ++i) {
    const int64_t base = h * a.q_sh + (i - a.c0) * a.q_st;
    const float x1 = load_q(a.q, a.q_dtype, base + p);
    const float x2 = load_q(a.q, a.q_dtype, base + p + half);
    float c, s;
    rope_cos_sin(i, ft.inv_freq[p], &c, &s);
    s1 += x1 * c - x2 * s;
    s2 += x2 * c + x1 * s;
  }
  const float inv = 1.0f / (float)(i1 - i0);
  s1 *= inv;
  s2 *= inv;
  for (int kc = 0; kc < a.n_kc; ++kc) {
    float c = 1.f, s = 0.f;
    if (kc) rope_cos_sin(-a.period * kc, ft.inv_freq[p], &c, &s);
    float* dst = a.pq + (((int64_t)kc * a.H + h) * a.n_qb + qb) * a.D;
    dst[p] = s1 * c - s2 * s;
    dst[p + half] = s2 * c + s1 * s;
  }
}

// grid (ceil(n_qb / kScoreQb), H_kv, key-block spans), 256 threads, one key
// block per thread and pass: the scores of the G query heads x kScoreQb query
// blocks against the key blocks of span z (kScoreSpan blocks) up to the
// workgroup's last diagonal, key chunk by key chunk (the matching query means
// sit in LDS).  Blocks above a query block's diagonal are not written.
struct ScoreArgs {
  const float* pk;  // float4 [H_kv][D / 4][n_kb]
  const float* pq;  // [n_kc][H][n_qb][D]
  float* scores;    // [H][n_qb][n_kb]
  int64_t c0, period, n_qb, n_kb;
  int32_t H, G, D, n_kc;
  uint64_t head_mask;
  float sm_scale;
};

template <int D, int NV>
__global__ void __launch_bounds__(256) bs_score(ScoreArgs a) {
  __shared__ float4 qv[NV][D / 4];
  const int g = blockIdx.y;
  const int64_t qb0 = (int64_t)blockIdx.x * kScoreQb;
  const int nq = (int)(a.n_qb - qb0 < kScoreQb ? a.n_qb - qb0 : kScoreQb);
  const int nv = a.G * nq;  // vectors: v = hh * nq + b
  const int64_t diag0 = a.c0 / kBlk + qb0;        // diagonal of the first block
  const int64_t kb_end = diag0 + nq;              // one past the last diagonal
  const int64_t z0 = (int64_t)blockIdx.z * kScoreSpan;
  const int64_t z1 = z0 + kScoreSpan < kb_end ? z0 + kScoreSpan : kb_end;
  if (z0 >= z1) return;
  for (int kc = 0; kc < a.n_kc; ++kc) {
    // the key blocks whose first key lies in chunk kc
    int64_t kb_lo = a.period ? (kc * a.period + kBlk - 1) / kBlk : 0;
    int64_t kb_hi = a.period ? ((kc + 1) * a.period + kBlk - 1) / kBlk : kb_end;
    kb_hi = kb_hi < kb_end ? kb_hi : kb_end;
    if (kb_lo >= kb_hi) break;
    kb_lo = kb_lo > z0 ? kb_lo : z0;
    kb_hi = kb_hi < z1 ? kb_hi : z1;
    if (kb_lo >= kb_hi) continue;
    __syncthreads();
    for (int e = threadIdx.x; e < nv * (D / 4); e += 256) {
      const int vv = e / (D / 4), d4 = e % (D / 4);
      const int hh = vv / nq, b = vv % nq;
      const int h = g * a.G + hh;
      qv[vv][d4] = reinterpret_cast<const float4*>(
          a.pq + (((int64_t)kc * a.H + h) * a.n_qb + qb0 + b) * D)[d4];
    }
    __syncthreads();
    for (int64_t kb = kb_lo + threadIdx.x; kb < kb_hi; kb += 256) {
      const float4* kp = reinterpret_cast<const float4*>(a.pk) + (int64_t)g * (D / 4) * a.n_kb + kb;
      float acc[NV];
#pragma unroll
      for (int vv = 0; vv < NV; ++vv) acc[vv] = 0.f;
#pragma unroll 2
      for (int d4 = 0; d4 < D / 4; ++d4) {
        const float4 k4 = kp[(int64_t)d4 * a.n_kb];
#pragma unroll
        for (int vv = 0; vv < NV; ++vv) {
          if (vv < nv) {
            const float4 q4 = qv[vv][d4];
            acc[vv] += k4.x * q4.x + k4.y * q4.y + k4.z * q4.z + k4.w * q4.w;
          }
        }
      }
#pragma unroll
      for (int vv = 0; vv < NV; ++vv) {
        if (vv < nv) {
          const int hh = vv / nq, b = vv % nq;
          const int h = g * a.G + hh;
          if (((a.head_mask >> h) & 1ull) && kb <= diag0 + b)
            a.scores[((int64_t)h * a.n_qb + qb0 + b) * a.n_kb + kb] = acc[vv] * a.sm_scale;
        }
      }
    }
  }
}

// fp32 -> uint32 whose unsigned order is the float order (-0 taken as +0).
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over the 256 threads of a workgroup (wave scans with
// lane shuffles, then the four wave totals); also returns the total.
__device__ __forceinline__ uint32_t block_scan_excl(uint32_t v, uint32_t* wave_tot,
                                                    uint32_t* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wave_tot[w] = x;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint32_t t = wave_tot[u];
    before += u < w ? t : 0u;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

// grid (n_qb, H), 256 threads: per query block, the k - 1 best of the key
// blocks 0 .. diag - 1 (order: score desc, index asc) and the diagonal, in
// ascending order; -1 after the count.  Keys sit in LDS (dynamic, n_kb
// words); a radix select over 11, 11 and 10 key bits (2048-bin histograms,
// so that keys of one magnitude spread over many bins, with prefix sums
// across the workgroup to find the bin) gives the k-1-th key, then an
// ordered compaction writes the indices.
struct SelectArgs {
  const float* scores;  // [H][n_qb][n_kb]
  int32_t* idx;         // [H][n_qb][max_blocks]
  int32_t* cnt;         // [H][n_qb]
  int32_t budget[kMaxHeads];  // kept blocks per query block, per head
  int64_t c0, n_qb, n_kb;
  int32_t max_blocks;
  uint64_t head_mask;
};

constexpr int kSelBins = 2048;

__global__ void __launch_bounds__(256) bs_select(SelectArgs a) {
  extern __shared__ uint32_t keys[];
  __shared__ uint32_t hist[kSelBins];
  __shared__ uint32_t wave_tot[4];
  __shared__ uint32_t sh_prefix, sh_need;
  const int64_t qb = blockIdx.x;
  const int h = blockIdx.y;
  if (!((a.head_mask >> h) & 1ull)) return;
  const int tid = threadIdx.x;
  const int64_t diag = a.c0 / kBlk + qb;
  const int n = (int)diag;  // candidates 0 .. diag - 1
  int kk = a.budget[h];
  if (kk > n + 1) kk = n + 1;
  kk -= 1;  // earlier blocks to keep
  int32_t* out = a.idx + ((int64_t)h * a.n_qb + qb) * a.max_blocks;
  const float* sc = a.scores + ((int64_t)h * a.n_qb + qb) * a.n_kb;
  // the row's scores as order keys: 16-byte loads, several in flight per
  // thread, when the row start is 16-byte aligned
  if ((((uintptr_t)sc) & 15u) == 0) {
    const int n4 = n / 4;
    const float4* sc4 = reinterpret_cast<const float4*>(sc);
#pragma unroll 4
    for (int i = tid; i < n4; i += 256) {
      const float4 x = sc4[i];
      keys[4 * i] = order_key(x.x);
      keys[4 * i + 1] = order_key(x.y);
      keys[4 * i + 2] = order_key(x.z);
      keys[4 * i + 3] = order_key(x.w);
    }
    for (int i = 4 * n4 + tid; i < n; i += 256) keys[i] = order_key(sc[i]);
  } else {
#pragma unroll 8
    for (int i = tid; i < n; i += 256) keys[i] = order_key(sc[i]);
  }
  __syncthreads();
  uint32_t prefix = 0, mask = 0, need = (uint32_t)kk;
  const bool partial = kk > 0 && kk < n;  // uniform
  if (partial) {
    const int shifts[3] = {21, 10, 0};
    const int widths[3] = {11, 11, 10};
    for (int r = 0; r < 3; ++r) {
      const int shift = shifts[r];
      const uint32_t dmask = (1u << widths[r]) - 1u;
      const int nb = 1 << widths[r];
      for (int b = tid; b < nb; b += 256) hist[b] = 0;
      __syncthreads();
      for (int i = tid; i < n; i += 256) {
        const uint32_t u = keys[i];
        if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & dmask], 1u);
      }
      __syncthreads();
      // thread t owns bins [t * per, (t + 1) * per), counted from the top
      // bin down: thread 0 the highest bins
      const int per = nb / 256;
      const int top = nb - 1 - tid * per;
      uint32_t own = 0;
      for (int b = 0; b < per; ++b) own += hist[top - b];
      uint32_t total;
      const uint32_t above = block_scan_excl(own, wave_tot, &total);
      if (above < need && above + own >= need) {
        uint32_t cum = above;
        int b = top;
        for (; b > top - per + 1; --b) {
          if (cum + hist[b] >= need) break;
          cum += hist[b];
        }
        sh_prefix = prefix | ((uint32_t)b << shift);
        sh_need = need - cum;
      }
      __syncthreads();
      prefix = sh_prefix;
      need = sh_need;
      mask |= dmask << shift;
    }
  }
  // keep: key > T, or key == T among the first `need` ties by index; with
  // kk == n every candidate is kept, with kk == 0 none
  const uint32_t T = prefix;
  const int seg = (n + 255) / 256;
  const int b0 = tid * seg < n ? tid * seg : n;
  const int b1 = b0 + seg < n ? b0 + seg : n;
  uint32_t eq = 0, gt = 0;
  if (partial)
    for (int i = b0; i < b1; ++i) {
      eq += keys[i] == T;
      gt += keys[i] > T;
    }
  uint32_t tot;
  const uint32_t eq_before0 = block_scan_excl(eq, wave_tot, &tot);
  uint32_t sel;
  if (kk >= n) sel = (uint32_t)(b1 - b0);
  else if (kk == 0) sel = 0;
  else {
    // ties of this segment that are kept: those ranked below `need`
    const uint32_t lo = eq_before0 < need ? need - eq_before0 : 0u;
    sel = gt + (eq < lo ? eq : lo);
  }
  uint32_t pos = block_scan_excl(sel, wave_tot, &tot);
  uint32_t eq_before = eq_before0;
  for (int i = b0; i < b1; ++i) {
    bool keep;
    if (kk >= n) keep = true;
    else if (kk == 0) keep = false;
    else {
      const uint32_t u = keys[i];
      keep = u > T || (u == T && eq_before < need);
      eq_before += u == T;
    }
    if (keep) out[pos++] = i;
  }
  if (tid == 0) {
    out[kk] = (int32_t)diag;
    a.cnt[(int64_t)h * a.n_qb + qb] = kk + 1;
  }
  for (int i = kk + 1 + tid; i < a.max_blocks; i += 256) out[i] = -1;
}

}  // namespace

BlockLayout block_layout(const lcsr_problem_t& p) {
  BlockLayout L{};
  L.n_ctx = p.chunk_start + p.chunk_len;
  L.n_qb = (p.chunk_len + kBlk - 1) / kBlk;
  L.n_kb = (L.n_ctx + kBlk - 1) / kBlk;
  const int64_t period = p.dca.chunk > 0 ? p.dca.chunk - p.dca.local : 0;
  L.n_kc = period ? (L.n_ctx + period - 1) / period : 1;
  L.n_var = p.dca.chunk > 0 ? 3 : 1;
  const int64_t H = p.n_heads, D = p.head_dim;
  size_t off = 0;
  L.o_pk = off;
  off += align256((size_t)p.n_kv_heads * L.n_kb * D * 4);
  L.o_pq = off;
  off += align256((size_t)L.n_kc * H * L.n_qb * D * 4);
  L.o_scores = off;
  off += align256((size_t)H * L.n_qb * L.n_kb * 4);
  L.est_total = off;
  // attention: the chunk's rotated query variants
  L.o_q_rot = 0;
  L.attn_total = align256((size_t)L.n_var * H * (p.chunk_len > 0 ? p.chunk_len : 1) * D * 2);
  return L;
}

int run_block_estimate(const lcsr_problem_t& p, const int32_t* budgets_host, uint64_t head_mask,
                       int32_t max_blocks, int32_t* idx, int32_t* cnt, float* scores,
                       bool select_only, char* ws, hipStream_t s) {
  const BlockLayout L = block_layout(p);
  if (L.n_qb == 0 || !head_mask) return LCSR_OK;
  const DcaParams d = make_dca(&p.dca);
  const int64_t period = d.period;
  float* sc = scores ? scores : reinterpret_cast<float*>(ws + L.o_scores);
  int rc;
  if (!select_only) {
    FreqTable ft;
    rc = build_freq_table(&p.rope, p.head_dim, &ft);
    if (rc) return rc;
    float* pk = reinterpret_cast<float*>(ws + L.o_pk);
    float* pq = reinterpret_cast<float*>(ws + L.o_pq);
    hipLaunchKernelGGL(bs_pool_keys, dim3((unsigned)L.n_kb, (unsigned)p.n_kv_heads), dim3(64), 0,
                       s, static_cast<const uint16_t*>(p.k_cache), p.kv_stride_h, p.kv_stride_t,
                       L.n_ctx, (int)p.head_dim, L.n_kb, period, ft, pk);
    rc = check_launch("block pool keys");
    if (rc) return rc;
    PoolQArgs qa{};
    qa.q = p.q;
    qa.q_dtype = p.q_dtype;
    qa.q_sh = p.q_stride_h;
    qa.q_st = p.q_stride_t;
    qa.c0 = p.chunk_start;
    qa.L = p.chunk_len;
    qa.period = period;
    qa.H = p.n_heads;
    qa.D = (int)p.head_dim;
    qa.n_kc = (int)L.n_kc;
    qa.n_qb = L.n_qb;
    qa.pq = pq;
    hipLaunchKernelGGL(bs_pool_queries, dim3((unsigned)L.n_qb, (unsigned)p.n_heads), dim3(64), 0,
                       s, qa, ft);
    rc = check_launch("block pool queries");
    if (rc) return rc;
    ScoreArgs sa{};
    sa.pk = pk;
    sa.pq = pq;
    sa.scores = sc;
    sa.c0 = p.chunk_start;
    sa.period = period;
    sa.n_qb = L.n_qb;
    sa.n_kb = L.n_kb;
    sa.H = p.n_heads;
    sa.G = p.n_heads / p.n_kv_heads;
    sa.D = (int)p.head_dim;
    sa.n_kc = (int)L.n_kc;
    sa.head_mask = head_mask;
    sa.sm_scale = p.sm_scale;
    const dim3 grid((unsigned)((L.n_qb + kScoreQb - 1) / kScoreQb), (unsigned)p.n_kv_heads,
                    (unsigned)((L.n_kb + kScoreSpan - 1) / kScoreSpan));
    // accumulators for G x kScoreQb query means, rounded up to a power of two
    const int nv = sa.G * kScoreQb;
#define LCSR_BS_SCORE(DD, NV) hipLaunchKernelGGL((bs_score<DD, NV>), grid, dim3(256), 0, s, sa)
    if (p.head_dim == 128) {
      if (nv <= 4) LCSR_BS_SCORE(128, 4);
      else if (nv <= 8) LCSR_BS_SCORE(128, 8);
      else if (nv <= 16) LCSR_BS_SCORE(128, 16);
      else if (nv <= 32) LCSR_BS_SCORE(128, 32);
      else LCSR_BS_SCORE(128, 64);
    } else {
      if (nv <= 4) LCSR_BS_SCORE(64, 4);
      else if (nv <= 8) LCSR_BS_SCORE(64, 8);
      else if (nv <= 16) LCSR_BS_SCORE(64, 16);
      else if (nv <= 32) LCSR_BS_SCORE(64, 32);
      else LCSR_BS_SCORE(64, 64);
    }
#undef LCSR_BS_SCORE
    rc = check_launch("block scores");
    if (rc) return rc;
  }
  SelectArgs ka{};
  for (int h = 0; h < p.n_heads; ++h) ka.budget[h] = budgets_host[h];
  ka.scores = sc;
  ka.idx = idx;
  ka.cnt = cnt;
  ka.c0 = p.chunk_start;
  ka.n_qb = L.n_qb;
  ka.n_kb = L.n_kb;
  ka.max_blocks = max_blocks;
  ka.head_mask = head_mask;
  const size_t lds = (size_t)(L.n_kb > 0 ? L.n_kb : 1) * 4;
  hipLaunchKernelGGL(bs_select, dim3((unsigned)L.n_qb, (unsigned)p.n_heads), dim3(256), lds, s,
                     ka);
  return check_launch("block select");
}

}  // namespace lcsr
