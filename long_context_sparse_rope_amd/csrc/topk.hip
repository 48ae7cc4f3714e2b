// Deterministic top-k of a score row, ties to the lower index, written in
// ascending index order (page: "論文解説: Qwen2.5-1M" (0h-n0.github.io),
// 疎アテンション: critical vertical and slash lines are chosen dynamically;
// the order and the tie rule are ours: score descending, index ascending).
//
// One workgroup of 16 waves per head.  Scores are mapped to order-preserving
// unsigned keys; a 4-round 8-bit radix select finds the exact key T of the
// k-th largest score and how many ties at T are needed; then each wave
// compacts one contiguous segment of the row with ballots, so the output is
// ascending and every decision is integer-exact.
#include "lcsr_internal.h"

namespace lcsr {

namespace {

constexpr int kTopkWaves = 16;

struct TopkArgs {
  const float* scores;
  int64_t n, stride;
  uint64_t head_mask;
  int32_t budget[kMaxHeads];
  int32_t* idx;
  int32_t max_k;
  int32_t* cnt;
};

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0 ranks as +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__global__ void __launch_bounds__(64 * kTopkWaves) topk_kernel(TopkArgs a) {
  const int h = blockIdx.x;
  if (!((a.head_mask >> h) & 1)) return;
  const float* sc = a.scores + (int64_t)h * a.stride;
  int32_t* out = a.idx + (int64_t)h * a.max_k;
  const int64_t n = a.n;
  const int64_t k = a.budget[h] < n ? a.budget[h] : n;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int nthr = blockDim.x;

  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_prefix, s_rem;
  __shared__ uint32_t s_gt[kTopkWaves], s_eq[kTopkWaves];

  if (k >= n) {  // every index is selected
    for (int64_t i = tid; i < n; i += nthr) out[i] = (int32_t)i;
    for (int64_t i = n + tid; i < a.max_k; i += nthr) out[i] = -1;
    if (tid == 0) a.cnt[h] = (int32_t)n;
    return;
  }
  if (k == 0) {
    for (int64_t i = tid; i < a.max_k; i += nthr) out[i] = -1;
    if (tid == 0) a.cnt[h] = 0;
    return;
  }

  uint32_t prefix = 0, pmask = 0, rem = (uint32_t)k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = tid; b < 256; b += nthr) hist[b] = 0;
    __syncthreads();
    for (int64_t i = tid; i < n; i += nthr) {
      const uint32_t key = order_key(sc[i]);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t cum = 0, digit = 0;
      for (int b = 255; b >= 0; --b) {
        if (cum + hist[b] >= rem) {
          digit = (uint32_t)b;
          break;
        }
        cum += hist[b];
      }
      s_rem = rem - cum;
      s_prefix = prefix | (digit << shift);
    }
    __syncthreads();
    rem = s_rem;
    prefix = s_prefix;
    pmask |= 0xFFu << shift;
    __syncthreads();
  }
  const uint32_t T = prefix;      // key of the k-th largest score
  const uint32_t need_eq = rem;   // ties at T to keep, lowest indices first

  // contiguous segment of the row for this wave (multiple of 64 long)
  const int64_t seg = ((n + kTopkWaves - 1) / kTopkWaves + 63) / 64 * 64;
  const int64_t s0 = (int64_t)w * seg;
  const int64_t s1 = s0 + seg < n ? s0 + seg : n;
  uint32_t gt = 0, eq = 0;
  for (int64_t base = s0; base < s1; base += 64) {
    const int64_t i = base + lane;
    const uint32_t key = i < s1 ? order_key(sc[i]) : 0u;
    const bool valid = i < s1;
    gt += __popcll(__ballot(valid && key > T));
    eq += __popcll(__ballot(valid && key == T));
  }
  if (lane == 0) {
    s_gt[w] = gt;
    s_eq[w] = eq;
  }
  __syncthreads();
  uint32_t eq_before = 0, out_base = 0;
  for (int v = 0; v < w; ++v) {
    const uint32_t take = need_eq > eq_before ? (need_eq - eq_before < s_eq[v] ? need_eq - eq_before
                                                                               : s_eq[v])
                                              : 0u;
    out_base += s_gt[v] + take;
    eq_before += s_eq[v];
  }
  uint32_t eq_seen = 0, sel_seen = 0;
  for (int64_t base = s0; base < s1; base += 64) {
    const int64_t i = base + lane;
    const bool valid = i < s1;
    const uint32_t key = valid ? order_key(sc[i]) : 0u;
    const bool is_eq = valid && key == T;
    const uint64_t eq_mask = __ballot(is_eq);
    const uint32_t rank = eq_before + eq_seen + lanes_below(eq_mask);
    const bool sel = valid && (key > T || (is_eq && rank < need_eq));
    const uint64_t sel_mask = __ballot(sel);
    if (sel) out[out_base + sel_seen + lanes_below(sel_mask)] = (int32_t)i;
    eq_seen += __popcll(eq_mask);
    sel_seen += __popcll(sel_mask);
  }
  for (int64_t i = k + tid; i < a.max_k; i += nthr) out[i] = -1;
  if (tid == 0) a.cnt[h] = (int32_t)k;
}

}  // namespace

int launch_topk(const float* scores, int64_t n, int64_t score_stride, int n_heads,
                uint64_t head_mask, const int32_t* budget, int32_t* idx, int32_t max_k,
                int32_t* cnt, hipStream_t s) {
  TopkArgs a{};
  a.scores = scores;
  a.n = n;
  a.stride = score_stride;
  a.head_mask = head_mask;
  for (int h = 0; h < n_heads; ++h) a.budget[h] = budget[h];
  a.idx = idx;
  a.max_k = max_k;
  a.cnt = cnt;
  hipLaunchKernelGGL(topk_kernel, dim3(n_heads), dim3(64 * kTopkWaves), 0, s, a);
  return check_launch("topk");
}

}  // namespace lcsr
