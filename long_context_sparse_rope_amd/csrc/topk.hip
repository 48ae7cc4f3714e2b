// Deterministic top-k of score rows, ties to the lower index, written in
// ascending index order (page: "論文解説: Qwen2.5-1M" (0h-n0.github.io),
// 疎アテンション: critical vertical and slash lines are chosen dynamically;
// the order and the tie rule are ours: score descending, index ascending).
//
// Whole-chip radix select over every row at once (the vertical and the slash
// scores of every head).  Scores map to order-preserving unsigned keys and
// each row is cut into slices of kSlice keys, one workgroup per slice:
//   hist(l), l = 0, 1, 2   keys that match the prefix found so far are
//                          counted by their next 12, 12, 8 bits in LDS; the
//                          non-zero bins are added to the row's histogram;
//   pick(l)                one workgroup per row finds the bin that holds the
//                          k-th largest key and extends the prefix;
//   count                  per slice: keys above T and equal to T, where T is
//                          the exact key of the k-th largest score;
//   compact                each slice writes its selected indices after those
//                          of the slices before it, in ascending order; ties
//                          at T are taken from the lowest indices.
// Every decision is on integers, so the result does not depend on timing.
#include "lcsr_internal.h"

namespace lcsr {

namespace {

constexpr int kSlice = 16384;                 // keys per workgroup
constexpr int kThreads = 256;
constexpr int kPerThread = kSlice / kThreads;  // 64
constexpr int kBins = 4096;
constexpr int kLevels = 3;

enum : uint32_t { kModeSelect = 0, kModeAll = 1, kModeNone = 2 };

struct TopkSet {
  const float* scores;  // [H][stride]
  int32_t* idx;         // [H][max_k]
  int32_t* cnt;         // [H]
  int32_t max_k;
  int32_t budget[kMaxHeads];
};

struct TopkArgs {
  TopkSet set[2];
  int64_t n, stride;
  uint64_t head_mask;
  int32_t n_heads, n_slices;
  uint32_t* hist;    // [2][H][kLevels][kBins]
  uint32_t* state;   // [2][H][4]: prefix, prefix mask, remaining, mode | k << 2
  uint32_t* counts;  // [2][H][n_slices][2]: above T, equal to T
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

// Keys of indices first + u * step (u = 0..7), all eight loads issued
// before the first is used; indices past last read index last (their keys
// are ignored by the callers).
__device__ __forceinline__ void load_keys8(const float* sc, int64_t first, int64_t step,
                                           int64_t last, uint32_t (&key)[8]) {
  float f[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int64_t i = first + u * step;
    f[u] = sc[i < last ? i : last];
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) key[u] = order_key(f[u]);
}

__device__ __forceinline__ int level_shift(int l) { return l == 0 ? 20 : (l == 1 ? 8 : 0); }
__device__ __forceinline__ uint32_t level_mask(int l) { return l == 2 ? 0xFFu : 0xFFFu; }

__device__ __forceinline__ int64_t row_k(const TopkArgs& a, int set, int h) {
  const int64_t b = a.set[set].budget[h];
  return b < a.n ? (b > 0 ? b : 0) : a.n;
}

__device__ __forceinline__ bool row_live(const TopkArgs& a, int h) {
  return (a.head_mask >> h) & 1;
}

// ------------------------------------------------------------- histogram
__global__ void __launch_bounds__(kThreads) topk_hist(TopkArgs a, int level) {
  const int slice = blockIdx.x, h = blockIdx.y, set = blockIdx.z;
  if (!row_live(a, h)) return;
  const int64_t row = (int64_t)set * a.n_heads + h;
  uint32_t prefix = 0, pmask = 0;
  if (level == 0) {
    const int64_t k = row_k(a, set, h);
    if (k == 0 || k >= a.n) return;
  } else {
    const uint32_t* st = a.state + row * 4;
    if ((st[3] & 3u) != kModeSelect) return;
    prefix = st[0];
    pmask = st[1];
  }
  __shared__ uint32_t hist[kBins];
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < kBins / kThreads; ++j) hist[j * kThreads + tid] = 0;
  __syncthreads();
  const int shift = level_shift(level);
  const uint32_t bmask = level_mask(level);
  const float* sc = a.set[set].scores + h * a.stride;
  const int64_t s0 = (int64_t)slice * kSlice;
  const int64_t s1 = s0 + kSlice < a.n ? s0 + kSlice : a.n;
  // eight loads in flight per thread
  for (int j0 = 0; j0 < kPerThread; j0 += 8) {
    uint32_t key[8];
    load_keys8(sc, s0 + (int64_t)j0 * kThreads + tid, kThreads, s1 - 1, key);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t i = s0 + (int64_t)(j0 + u) * kThreads + tid;
      if (i < s1 && (key[u] & pmask) == prefix) atomicAdd(&hist[(key[u] >> shift) & bmask], 1u);
    }
  }
  __syncthreads();
  uint32_t* hg = a.hist + (row * kLevels + level) * kBins;
#pragma unroll
  for (int j = 0; j < kBins / kThreads; ++j) {
    const int b = j * kThreads + tid;
    if (hist[b]) atomicAdd(&hg[b], hist[b]);
  }
}

// ------------------------------------------------------------- pick a bin
// Thread t owns the 16 bins [kBins - 16 (t + 1), kBins - 16 t): thread 0 the
// largest keys.  An exclusive scan over threads gives the count above each
// range; the thread whose range holds the rem-th largest key walks it.
__global__ void __launch_bounds__(kThreads) topk_pick(TopkArgs a, int level) {
  const int h = blockIdx.x, set = blockIdx.y;
  if (!row_live(a, h)) return;
  const int64_t row = (int64_t)set * a.n_heads + h;
  uint32_t* st = a.state + row * 4;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  uint32_t prefix = 0, pmask = 0, rem;
  if (level == 0) {
    const int64_t k = row_k(a, set, h);
    const uint32_t mode = k == 0 ? kModeNone : (k >= a.n ? kModeAll : kModeSelect);
    if (mode != kModeSelect) {
      if (tid == 0) {
        st[0] = 0;
        st[1] = 0;
        st[2] = 0;
        st[3] = mode | ((uint32_t)k << 2);
      }
      return;
    }
    rem = (uint32_t)k;
  } else {
    if ((st[3] & 3u) != kModeSelect) return;
    prefix = st[0];
    pmask = st[1];
    rem = st[2];
  }
  const uint32_t* hg = a.hist + (row * kLevels + level) * kBins;
  constexpr int kPer = kBins / kThreads;
  const int top = kBins - kPer * tid;  // bins [top - kPer, top)
  uint32_t v[kPer];
  uint32_t sum = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    v[j] = hg[top - 1 - j];
    sum += v[j];
  }
  // inclusive scan within the wave, then over the four waves
  uint32_t inc = sum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t o = __shfl_up(inc, d);
    if (lane >= d) inc += o;
  }
  __shared__ uint32_t wsum[kThreads / 64];
  if (lane == 63) wsum[w] = inc;
  __syncthreads();
  uint32_t above = inc - sum;
  for (int u = 0; u < w; ++u) above += wsum[u];
  if (above < rem && above + sum >= rem) {
    uint32_t cum = above, digit = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (cum + v[j] >= rem) {
        digit = (uint32_t)(top - 1 - j);
        break;
      }
      cum += v[j];
    }
    const int shift = level_shift(level);
    st[0] = prefix | (digit << shift);
    st[1] = pmask | (level_mask(level) << shift);
    st[2] = rem - cum;
    if (level == 0) st[3] = kModeSelect | ((uint32_t)row_k(a, set, h) << 2);
  }
}

// ------------------------------------------------------------- count
__global__ void __launch_bounds__(kThreads) topk_count(TopkArgs a) {
  const int slice = blockIdx.x, h = blockIdx.y, set = blockIdx.z;
  if (!row_live(a, h)) return;
  const int64_t row = (int64_t)set * a.n_heads + h;
  const uint32_t* st = a.state + row * 4;
  if ((st[3] & 3u) != kModeSelect) return;
  const uint32_t T = st[0];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float* sc = a.set[set].scores + h * a.stride;
  const int64_t s0 = (int64_t)slice * kSlice;
  const int64_t s1 = s0 + kSlice < a.n ? s0 + kSlice : a.n;
  uint32_t gt = 0, eq = 0;
  for (int j0 = 0; j0 < kPerThread; j0 += 8) {
    uint32_t key[8];
    load_keys8(sc, s0 + (int64_t)j0 * kThreads + tid, kThreads, s1 - 1, key);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool valid = s0 + (int64_t)(j0 + u) * kThreads + tid < s1;
      gt += __popcll(__ballot(valid && key[u] > T));
      eq += __popcll(__ballot(valid && key[u] == T));
    }
  }
  __shared__ uint32_t wc[kThreads / 64][2];
  if (lane == 0) {
    wc[w][0] = gt;
    wc[w][1] = eq;
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t g = 0, e = 0;
    for (int u = 0; u < kThreads / 64; ++u) {
      g += wc[u][0];
      e += wc[u][1];
    }
    uint32_t* c = a.counts + (row * a.n_slices + slice) * 2;
    c[0] = g;
    c[1] = e;
  }
}

__device__ __forceinline__ uint32_t take_eq(uint32_t need, uint32_t before, uint32_t eq) {
  if (need <= before) return 0u;
  return need - before < eq ? need - before : eq;
}

// ------------------------------------------------------------- compact
// Wave w of the slice owns keys [s0 + 4096 w, s0 + 4096 (w + 1)), lane-
// interleaved in steps of 64: read once to count them and again (from L2)
// to write the selected indices.  (Holding the 64 keys of a lane in
// registers between the two took 157 VGPRs and spilled SGPRs.)
__global__ void __launch_bounds__(kThreads) topk_compact(TopkArgs a) {
  const int slice = blockIdx.x, h = blockIdx.y, set = blockIdx.z;
  if (!row_live(a, h)) return;
  const int64_t row = (int64_t)set * a.n_heads + h;
  const TopkSet& S = a.set[set];
  const uint32_t* st = a.state + row * 4;
  const uint32_t mode = st[3] & 3u;
  const int64_t k = st[3] >> 2;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int32_t* out = S.idx + (int64_t)h * S.max_k;
  const int64_t s0 = (int64_t)slice * kSlice;
  const int64_t s1 = s0 + kSlice < a.n ? s0 + kSlice : a.n;
  if (slice == 0) {
    for (int64_t i = k + tid; i < S.max_k; i += kThreads) out[i] = -1;
    if (tid == 0) S.cnt[h] = (int32_t)k;
  }
  if (mode == kModeNone) return;
  if (mode == kModeAll) {
    for (int64_t i = s0 + tid; i < s1; i += kThreads) out[i] = (int32_t)i;
    return;
  }
  const uint32_t T = st[0], need_eq = st[2];
  // selected keys and ties at T in the slices before this one: keys above T
  // plus the first need_eq ties (integer sums over the slices, in parallel)
  const uint32_t* cnts = a.counts + row * a.n_slices * 2;
  uint32_t gs = 0, es = 0;
  for (int u = tid; u < slice; u += kThreads) {
    gs += cnts[u * 2];
    es += cnts[u * 2 + 1];
  }
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) {
    gs += __shfl_xor(gs, d);
    es += __shfl_xor(es, d);
  }
  __shared__ uint32_t before[kThreads / 64][2];
  if (lane == 0) {
    before[w][0] = gs;
    before[w][1] = es;
  }
  __syncthreads();
  uint32_t g_before = 0, eq_before = 0;
  for (int u = 0; u < kThreads / 64; ++u) {
    g_before += before[u][0];
    eq_before += before[u][1];
  }
  uint32_t base = g_before + (eq_before < need_eq ? eq_before : need_eq);
  constexpr int kPerWave = kSlice / (kThreads / 64);
  constexpr int kSteps = kPerWave / 64;
  const int64_t w0 = s0 + (int64_t)w * kPerWave;
  const float* sc = S.scores + h * a.stride;
  uint32_t gt = 0, eq = 0;
  for (int j0 = 0; j0 < kSteps; j0 += 8) {
    uint32_t key[8];
    load_keys8(sc, w0 + j0 * 64 + lane, 64, s1 - 1, key);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool valid = w0 + (j0 + u) * 64 + lane < s1;
      gt += __popcll(__ballot(valid && key[u] > T));
      eq += __popcll(__ballot(valid && key[u] == T));
    }
  }
  __shared__ uint32_t wc[kThreads / 64][2];
  if (lane == 0) {
    wc[w][0] = gt;
    wc[w][1] = eq;
  }
  __syncthreads();
  for (int u = 0; u < w; ++u) {
    base += wc[u][0] + take_eq(need_eq, eq_before, wc[u][1]);
    eq_before += wc[u][1];
  }
  uint32_t eq_seen = 0, sel_seen = 0;
  for (int j0 = 0; j0 < kSteps; j0 += 8) {
    uint32_t key[8];
    load_keys8(sc, w0 + j0 * 64 + lane, 64, s1 - 1, key);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t i = w0 + (j0 + u) * 64 + lane;
      const bool valid = i < s1;
      const bool is_eq = valid && key[u] == T;
      const uint64_t eq_mask = __ballot(is_eq);
      const uint32_t rank = eq_before + eq_seen + lanes_below(eq_mask);
      const bool sel = valid && (key[u] > T || (is_eq && rank < need_eq));
      const uint64_t sel_mask = __ballot(sel);
      if (sel) out[base + sel_seen + lanes_below(sel_mask)] = (int32_t)i;
      eq_seen += __popcll(eq_mask);
      sel_seen += __popcll(sel_mask);
    }
  }
}

}  // namespace

size_t topk_workspace(int64_t n, int n_heads) {
  const int64_t n_slices = (n + kSlice - 1) / kSlice;
  const size_t hist = (size_t)2 * n_heads * kLevels * kBins * 4;
  const size_t state = (size_t)2 * n_heads * 4 * 4;
  const size_t counts = (size_t)2 * n_heads * (n_slices > 0 ? n_slices : 1) * 2 * 4;
  return ((hist + 255) & ~(size_t)255) + ((state + 255) & ~(size_t)255) +
         ((counts + 255) & ~(size_t)255);
}

int launch_topk(const TopkRequest& r, hipStream_t s) {
  TopkArgs a{};
  for (int z = 0; z < 2; ++z) {
    a.set[z].scores = r.scores[z];
    a.set[z].idx = r.idx[z];
    a.set[z].cnt = r.cnt[z];
    a.set[z].max_k = r.max_k[z];
    for (int h = 0; h < r.n_heads; ++h) a.set[z].budget[h] = r.budget[z][h];
  }
  a.n = r.n;
  a.stride = r.stride;
  a.head_mask = r.head_mask;
  a.n_heads = r.n_heads;
  const int64_t n_slices = (r.n + kSlice - 1) / kSlice;
  if (n_slices > 65535) return fail(LCSR_ENOTSUP, "top-k over more than %lld scores",
                                    (long long)65535 * kSlice);
  a.n_slices = (int32_t)(n_slices > 0 ? n_slices : 1);
  char* cur = static_cast<char*>(r.ws);
  const size_t hist = (size_t)2 * r.n_heads * kLevels * kBins * 4;
  a.hist = reinterpret_cast<uint32_t*>(cur);
  cur += (hist + 255) & ~(size_t)255;
  a.state = reinterpret_cast<uint32_t*>(cur);
  cur += ((size_t)2 * r.n_heads * 4 * 4 + 255) & ~(size_t)255;
  a.counts = reinterpret_cast<uint32_t*>(cur);
  int rc = launch_fill_zero(a.hist, hist, s);  // a kernel: capturable
  if (rc) return rc;
  const dim3 rows((unsigned)a.n_slices, (unsigned)r.n_heads, 2u);
  const dim3 pick((unsigned)r.n_heads, 2u);
  for (int l = 0; l < kLevels; ++l) {
    hipLaunchKernelGGL(topk_hist, rows, dim3(kThreads), 0, s, a, l);
    hipLaunchKernelGGL(topk_pick, pick, dim3(kThreads), 0, s, a, l);
  }
  hipLaunchKernelGGL(topk_count, rows, dim3(kThreads), 0, s, a);
  hipLaunchKernelGGL(topk_compact, rows, dim3(kThreads), 0, s, a);
  return check_launch("topk");
}

}  // namespace lcsr
