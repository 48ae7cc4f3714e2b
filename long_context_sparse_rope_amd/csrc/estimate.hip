// Vertical-slash pattern estimate (the chunk's last queries against every
// key), on the matrix cores.
//
// Page: "論文解説: Qwen2.5-1M" (0h-n0.github.io), 疎アテンション and Chunked
// Prefill: the last 64 queries of each chunk attend to all keys and the
// critical vertical / slash lines are chosen from that attention;
// "アルゴリズム: DCAと疎アテンションの統合": selection uses continuous relative
// positions.  The keys in the cache are rotated at P_k(j) = j mod S, so the
// estimate rows are rotated at (r - S * c) for the DCA chunk c of the key
// tile, which gives the continuous relative position r - j.
//
// Pass 1: row max / sum of exp2 per key split (online, in-lane).
// Combine: row logsumexp (log2 units of the scaled logits).
// Pass 2: probabilities, vertical sums (per key, in-lane over rows) and
// diagonal sums of every 32x32 block (through a wave-private LDS scratch),
// all in a fixed order: the scores are bitwise reproducible.
// Reduce: slash score per offset from the <= 2 diagonal records covering it.
#include <cmath>

#include "lcsr_internal.h"

namespace lcsr {

namespace {

struct EstArgs {
  const uint16_t* k;      // K cache, rotated at P_k
  int64_t kv_sh, kv_st;
  const uint16_t* q_est;  // [n_kc][H][64][D]
  int32_t H, G;
  int64_t n_ctx;          // c1
  int64_t row0;           // first estimate row
  int32_t n_rows;         // <= 64
  int64_t period;         // S, 0 = DCA off
  int64_t n_tiles, tiles_per_split;
  int32_t n_split;
  float scale_log2;       // sm_scale * log2(e)
  float* part;            // [H][n_split][64][2]
  float* lse2;            // [H][64]
  float* vscore;          // [H][n_ctx]
  float* sscore;          // [H][n_ctx]
  float* diag;            // [H][n_diag][2][64]
  int64_t n_diag;
  uint64_t head_mask;
};

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxEstGroup = 8;  // one wave per query head of a KV group

template <int D>
struct KTile {
  static constexpr int kStride = D + 8;  // bf16 elements per LDS row (16 B pad)
};

// Cooperative load of the 64-key tile starting at key k0 into LDS (rows past
// n_ctx are zero).  Every thread of the block takes part.
template <int D>
__device__ __forceinline__ void load_k_tile(const EstArgs& a, int g, int64_t k0,
                                            uint16_t* ks) {
  constexpr int kChunks = D / 8;  // 16-byte chunks per key row
  const int nthr = blockDim.x;
  const uint16_t* base = a.k + (int64_t)g * a.kv_sh;
  for (int c = threadIdx.x; c < kTileK * kChunks; c += nthr) {
    const int r = c / kChunks, col = (c % kChunks) * 8;
    const int64_t key = k0 + r;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (key < a.n_ctx) v = *reinterpret_cast<const u32x4*>(base + key * a.kv_st + col);
    *reinterpret_cast<u32x4*>(ks + r * KTile<D>::kStride + col) = v;
  }
}

template <int D>
__device__ __forceinline__ void load_q_frags(const EstArgs& a, int h, int64_t c,
                                             bf16x8 (&qf)[2][D / 16]) {
  const int lane = threadIdx.x & 63;
  const uint16_t* base = a.q_est + (((int64_t)c * a.H + h) * kEstRows) * D;
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      qf[b][s] = *reinterpret_cast<const bf16x8*>(
          base + (int64_t)(b * 32 + (lane & 31)) * D + s * 16 + 8 * (lane >> 5));
}

template <int D>
__device__ __forceinline__ bf16x8 k_frag(const uint16_t* ks, int kb, int s) {
  const int lane = threadIdx.x & 63;
  return *reinterpret_cast<const bf16x8*>(ks + (kb * 32 + (lane & 31)) * KTile<D>::kStride +
                                          s * 16 + 8 * (lane >> 5));
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ------------------------------------------------------------------ pass 1
template <int D>
__global__ void __launch_bounds__(512) est_pass1(EstArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t ks[kTileK * KTile<D>::kStride];
  const int g = blockIdx.y, split = blockIdx.x;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = g * a.G + w;
  const bool active = (a.head_mask >> h) & 1;
  const int64_t t_begin = (int64_t)split * a.tiles_per_split;
  const int64_t t_end = t_begin + a.tiles_per_split < a.n_tiles ? t_begin + a.tiles_per_split
                                                                 : a.n_tiles;
  bf16x8 qf[2][D / 16];
  int64_t cur_c = -1;
  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
  const int half = lane >> 5;
  for (int64_t t = t_begin; t < t_end; ++t) {
    const int64_t k0 = t * kTileK;
    __syncthreads();
    load_k_tile<D>(a, g, k0, ks);
    __syncthreads();
    if (!active) continue;
    const int64_t c = a.period ? k0 / a.period : 0;
    if (c != cur_c) {
      load_q_frags<D>(a, h, c, qf);
      cur_c = c;
    }
    // the tile needs masking only at the causal edge or past n_ctx
    const bool edge = (k0 + kTileK - 1 > a.row0);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      f32x16 acc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        acc[kb] = (f32x16){};
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
          acc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_frag<D>(ks, kb, s), qf[b][s],
                                                            acc[kb], 0, 0, 0);
      }
      const int64_t row = a.row0 + b * 32 + (lane & 31);
      float x[2][16];
      float mx = m[b];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = acc[kb][r] * a.scale_log2;
          if (edge) {
            const int64_t key = k0 + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            if (key > row || key >= a.n_ctx) v = -INFINITY;
          }
          x[kb][r] = v;
          mx = fmaxf(mx, v);
        }
      if (mx == -INFINITY) continue;
      float sum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sum += exp2f(x[kb][r] - mx);
      l[b] = l[b] * exp2f(m[b] - mx) + sum;
      m[b] = mx;
    }
  }
  if (!active) return;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const float mo = __shfl_xor(m[b], 32);
    const float lo = __shfl_xor(l[b], 32);
    const float mm = fmaxf(m[b], mo);
    float ll = 0.f;
    if (mm != -INFINITY) {
      // combine the two halves in a fixed order (lower half first)
      const float la = half ? lo : l[b], ma = half ? mo : m[b];
      const float lb = half ? l[b] : lo, mb = half ? m[b] : mo;
      ll = la * exp2f(ma - mm) + lb * exp2f(mb - mm);
    }
    if (half == 0) {
      float* dst = a.part + (((int64_t)h * a.n_split + split) * kEstRows + b * 32 + lane) * 2;
      dst[0] = mm;
      dst[1] = ll;
    }
  }
}

__global__ void est_combine(EstArgs a) {
  const int h = blockIdx.x, r = threadIdx.x;
  if (!((a.head_mask >> h) & 1) || r >= kEstRows) return;
  const float* p = a.part + ((int64_t)h * a.n_split * kEstRows + r) * 2;
  float mm = -INFINITY;
  for (int z = 0; z < a.n_split; ++z) mm = fmaxf(mm, p[(int64_t)z * kEstRows * 2]);
  float ll = 0.f;
  if (mm != -INFINITY)
    for (int z = 0; z < a.n_split; ++z)
      ll += p[(int64_t)z * kEstRows * 2 + 1] * exp2f(p[(int64_t)z * kEstRows * 2] - mm);
  a.lse2[h * kEstRows + r] = (r < a.n_rows && ll > 0.f) ? mm + log2f(ll) : INFINITY;
}

// ------------------------------------------------------------------ pass 2
// Diagonal sums of a 32x32 block held in the S = Q K^T layout (lane -> key
// column n = lane % 32, register r -> query row 8(r/4) + 4(lane/32) + r%4):
// out[d + 31] = sum_m X[m][m - d], d in [-31, 31], m ascending.
__device__ __forceinline__ void diag_record(const float (&x)[16], float* scratch,
                                            float* dst) {
  const int lane = threadIdx.x & 63;
  const int n = lane & 31, half = lane >> 5;
#pragma unroll
  for (int r = 0; r < 16; ++r) scratch[(8 * (r >> 2) + 4 * half + (r & 3)) * 33 + n] = x[r];
  wave_lds_sync();
  if (lane < 63) {
    const int d = lane - 31;
    const int m0 = d > 0 ? d : 0, m1 = d < 0 ? 31 + d : 31;
    float s = 0.f;
    for (int mm = m0; mm <= m1; ++mm) s += scratch[mm * 33 + (mm - d)];
    dst[lane] = s;
  } else {
    dst[63] = 0.f;
  }
  wave_lds_sync();
}

template <int D>
__global__ void __launch_bounds__(512) est_pass2(EstArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t ks[kTileK * KTile<D>::kStride];
  __shared__ float scratch_all[kMaxEstGroup][32 * 33];
  const int g = blockIdx.y, split = blockIdx.x;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = g * a.G + w;
  const bool active = (a.head_mask >> h) & 1;
  const int half = lane >> 5;
  float* scratch = scratch_all[w];
  const int64_t t_begin = (int64_t)split * a.tiles_per_split;
  const int64_t t_end = t_begin + a.tiles_per_split < a.n_tiles ? t_begin + a.tiles_per_split
                                                                 : a.n_tiles;
  bf16x8 qf[2][D / 16];
  int64_t cur_c = -1;
  // log2-sum-exp of this lane's rows (INFINITY for padding rows -> p = 0)
  float lse[2][16];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      lse[b][r] = active ? a.lse2[h * kEstRows + b * 32 + 8 * (r >> 2) + 4 * half + (r & 3)]
                         : INFINITY;
  float* vout = a.vscore + (int64_t)h * a.n_ctx;
  float* drec = a.diag + (int64_t)h * a.n_diag * 2 * 64;
  for (int64_t t = t_begin; t < t_end; ++t) {
    const int64_t k0 = t * kTileK;
    __syncthreads();
    load_k_tile<D>(a, g, k0, ks);
    __syncthreads();
    if (!active) continue;
    const int64_t c = a.period ? k0 / a.period : 0;
    if (c != cur_c) {
      load_q_frags<D>(a, h, c, qf);
      cur_c = c;
    }
    const bool edge = (k0 + kTileK - 1 > a.row0);
    float p[2][2][16];  // [kb][b][r]
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        f32x16 acc = {};
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[b][s], k_frag<D>(ks, kb, s), acc,
                                                        0, 0, 0);
        const int64_t key = k0 + kb * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = exp2f(acc[r] * a.scale_log2 - lse[b][r]);
          if (edge) {
            const int64_t row = a.row0 + b * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            if (key > row || key >= a.n_ctx) v = 0.f;
          }
          p[kb][b][r] = v;
        }
      }
    // vertical scores: fixed order (b = 0 rows, then b = 1 rows; lower half first)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float s = 0.f;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += p[kb][b][r];
      const float o = __shfl_xor(s, 32);
      const float tot = half ? o + s : s + o;
      const int64_t key = k0 + kb * 32 + (lane & 31);
      if (half == 0 && key < a.n_ctx) vout[key] = tot;
    }
    // diagonal records: e = 2t (blocks (0,0) + (1,1)), e = 2t + 1 (b=0, kb=1,
    // slot 0), e = 2t - 1 (b=1, kb=0, slot 1); record index e + 1
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = p[0][0][r] + p[1][1][r];
    diag_record(x, scratch, drec + ((2 * t + 1) * 2 + 0) * 64);
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = p[1][0][r];
    diag_record(x, scratch, drec + ((2 * t + 2) * 2 + 0) * 64);
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = p[0][1][r];
    diag_record(x, scratch, drec + ((2 * t) * 2 + 1) * 64);
  }
}

// s_o = sum over the diagonal records covering offset o (fixed order).
__global__ void est_slash_reduce(EstArgs a) {
  const int h = blockIdx.y;
  const int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (!((a.head_mask >> h) & 1) || o >= a.n_ctx) return;
  const float* drec = a.diag + (int64_t)h * a.n_diag * 2 * 64;
  // o = row0 - 32 e + d, |d| <= 31  =>  e in [(row0 - o - 31) / 32, (row0 - o + 31) / 32]
  const int64_t num = a.row0 - o;
  const int64_t lo = num - 31;
  const int64_t e_lo = lo >= 0 ? lo / 32 : -((-lo + 31) / 32);  // floor(lo / 32)
  float s = 0.f;
  for (int64_t e = e_lo; e <= e_lo + 2; ++e) {
    if (e < -1 || e > 2 * a.n_tiles - 1) continue;
    const int64_t d = o - a.row0 + 32 * e;
    if (d < -31 || d > 31) continue;
    const float* rec = drec + (e + 1) * 2 * 64;
    if ((e & 1) == 0) {
      s += rec[d + 31];
    } else {
      if ((e - 1) / 2 >= 0 && e >= 1) s += rec[d + 31];                 // slot 0 (tile (e-1)/2)
      if ((e + 1) / 2 < a.n_tiles) s += rec[64 + d + 31];              // slot 1 (tile (e+1)/2)
    }
  }
  a.sscore[(int64_t)h * a.n_ctx + o] = s;
}

}  // namespace

int run_estimate(const lcsr_problem_t& p, int32_t last_q, const HeadSet& hs,
                 const lcsr_pattern_t& pat, float* vscore, float* sscore,
                 bool select_only, char* ws, hipStream_t s) {
  const EstimateLayout L = estimate_layout(p);
  char* cur = ws;
  uint16_t* q_est = reinterpret_cast<uint16_t*>(cur);
  cur += L.q_est;
  float* part = reinterpret_cast<float*>(cur);
  cur += L.part;
  float* lse2 = reinterpret_cast<float*>(cur);
  cur += L.lse;
  float* vs_ws = reinterpret_cast<float*>(cur);
  cur += L.vscore;
  float* ss_ws = reinterpret_cast<float*>(cur);
  cur += L.sscore;
  float* diag = reinterpret_cast<float*>(cur);
  cur += L.diag;
  void* topk_ws = cur;
  float* vsc = vscore ? vscore : vs_ws;
  float* ssc = sscore ? sscore : ss_ws;
  const int64_t c1 = L.n_ctx;
  if (!select_only && p.n_heads / p.n_kv_heads > kMaxEstGroup)
    return fail(LCSR_ENOTSUP, "the estimate supports n_heads / n_kv_heads <= %d", kMaxEstGroup);
  if (!select_only) {
    FreqTable ft;
    int rc = build_freq_table(&p.rope, p.head_dim, &ft);
    if (rc) return rc;
    const DcaParams d = make_dca(&p.dca);
    const int64_t row0 = c1 - last_q > p.chunk_start ? c1 - last_q : p.chunk_start;
    const int n_rows = (int)(c1 - row0);
    EstArgs a{};
    a.k = static_cast<const uint16_t*>(p.k_cache);
    a.kv_sh = p.kv_stride_h;
    a.kv_st = p.kv_stride_t;
    a.q_est = q_est;
    a.H = p.n_heads;
    a.G = p.n_heads / p.n_kv_heads;
    a.n_ctx = c1;
    a.row0 = row0;
    a.n_rows = n_rows;
    a.period = d.period;
    a.n_tiles = L.n_tiles;
    a.n_split = (int32_t)L.n_split;
    a.tiles_per_split = (L.n_tiles + L.n_split - 1) / L.n_split;
    a.scale_log2 = p.sm_scale * kLog2e;
    a.part = part;
    a.lse2 = lse2;
    a.vscore = vsc;
    a.sscore = ssc;
    a.diag = diag;
    a.n_diag = L.n_diag;
    a.head_mask = hs.mask;
    // padding rows of the estimate Q (rows >= n_rows) never reach a result
    // but must be finite: clear the buffer (a kernel, not a memset node)
    rc = launch_fill_zero(q_est, L.q_est, s);
    if (rc) return rc;
    rc = launch_rotate_q_estimate(p, ft, d, row0, n_rows, (int)L.n_kc, q_est, s);
    if (rc) return rc;
    const dim3 grid((unsigned)L.n_split, (unsigned)p.n_kv_heads);
    const dim3 block((unsigned)(64 * a.G));
    if (p.head_dim == 128) hipLaunchKernelGGL(est_pass1<128>, grid, block, 0, s, a);
    else hipLaunchKernelGGL(est_pass1<64>, grid, block, 0, s, a);
    rc = check_launch("estimate pass 1");
    if (rc) return rc;
    hipLaunchKernelGGL(est_combine, dim3(p.n_heads), dim3(64), 0, s, a);
    rc = check_launch("estimate combine");
    if (rc) return rc;
    if (p.head_dim == 128) hipLaunchKernelGGL(est_pass2<128>, grid, block, 0, s, a);
    else hipLaunchKernelGGL(est_pass2<64>, grid, block, 0, s, a);
    rc = check_launch("estimate pass 2");
    if (rc) return rc;
    hipLaunchKernelGGL(est_slash_reduce, dim3((unsigned)((c1 + 255) / 256), p.n_heads),
                       dim3(256), 0, s, a);
    rc = check_launch("estimate slash reduce");
    if (rc) return rc;
  }
  TopkRequest r{};
  r.scores[0] = vsc;
  r.scores[1] = ssc;
  r.idx[0] = pat.vert_idx;
  r.idx[1] = pat.slash_idx;
  r.cnt[0] = pat.vert_cnt;
  r.cnt[1] = pat.slash_cnt;
  r.max_k[0] = pat.max_vert;
  r.max_k[1] = pat.max_slash;
  r.budget[0] = hs.n_vert;
  r.budget[1] = hs.n_slash;
  r.n = c1;
  r.stride = c1;
  r.n_heads = (int)p.n_heads;
  r.head_mask = hs.mask;
  r.ws = topk_ws;
  return launch_topk(r, s);
}

}  // namespace lcsr
