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
// Pass 1: row sum of exp2 per key split against a running reference
// (online, in-lane).
// Combine: row logsumexp (log2 units of the scaled logits).
// Pass 2: probabilities, vertical sums (per key, in-lane over rows) and
// diagonal sums of every 32x32 block (through a wave-private LDS scratch),
// all in a fixed order: the scores are bitwise reproducible.
// Reduce: slash score per offset from the <= 2 diagonal records covering it.
// DCA key periods need not be multiples of the 64-key tile: in a tile that
// meets a chunk edge the passes count only the keys before it, and the edge
// kernels score the keys after it with the next chunk's query rows (a
// partial of its own in pass 1; vertical scores and diagonal sums added
// after pass 2).
#include <cmath>

#include "lcsr_internal.h"

namespace lcsr {

namespace {

struct EstArgs {
  const uint16_t* k;      // K cache (fp16), rotated at P_k
  int64_t kv_sh, kv_st;
  const uint16_t* q_est;  // [n_kc][H][64][D] fp16
  int32_t H, G;
  int64_t n_ctx;          // c1
  int64_t row0;           // first estimate row
  int32_t n_rows;         // <= 64
  int64_t period;         // S, 0 = DCA off
  int64_t n_tiles, tiles_per_split;
  int32_t n_split;
  int32_t n_part;         // partials per head: n_split, + 1 when a tile meets a DCA edge
  float scale_log2;       // sm_scale * log2(e)
  float* part;            // [H][n_part][64][2]
  float* lse2;            // [H][64]
  float* vscore;          // [H][n_ctx]
  float* sscore;          // [H][n_ctx]
  float* diag;            // [H][n_diag][2][64]
  int64_t n_diag;
  uint64_t head_mask;
  int32_t n_sub, nw;      // workgroups per KV head, query heads (waves) per workgroup
};

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxEstWaves = 7;  // query heads per workgroup (+1 loader wave)
constexpr int kEstStages = 4;    // LDS ring of key tiles

// A 64-key tile of K in LDS: 16-byte chunk c of row r sits at slot
// c ^ (r mod 16) of the row (no padding, bank-spread fragment reads).
template <int D>
struct KTile {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = D / 8;
  static constexpr int kBytes = kTileK * kRowBytes;
  static constexpr int kRowsPerInstr = 1024 / kRowBytes;  // rows one 64-lane load fills
  static constexpr int kInstr = kTileK / kRowsPerInstr;   // loads per tile
};

template <int D>
__device__ __forceinline__ int kslot(int chunk, int row) {
  return (chunk ^ (row & 15)) & (KTile<D>::kChunks - 1);
}

__device__ __forceinline__ uint32_t est_lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// global -> LDS, 16 bytes per lane; M0 holds the LDS byte address of lane 0's
// 16 bytes.  No register results, so nothing is left in flight in a VGPR.
__device__ __forceinline__ void est_dma16(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(lds) : "memory");
}

// s_waitcnt vmcnt(N), other counters untouched.
template <int N>
__device__ __forceinline__ void est_wait_vm() {
  constexpr int n = N > 63 ? 63 : N;
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier of the key ring: LDS reads and writes of this wave retire
// first (lgkmcnt(0)); no release fence (that would wait for every load in
// flight).  The loader waits for a tile's loads (vmcnt) before arriving.
__device__ __forceinline__ void est_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// Loader wave: streams the workgroup's key tiles [t_begin, t_end) of KV head
// g into the ring (tile i in stage i mod 4), two tiles ahead of the heads;
// rows past n_ctx repeat the last key (those keys are masked).  Arrives at
// one barrier before the first tile and one after each tile, like the heads.
template <int D>
__device__ void est_loader(const EstArgs& a, int g, int64_t t_begin, int64_t t_end,
                           char* ring, int lane) {
  using T = KTile<D>;
  constexpr int R = T::kRowsPerInstr;
  const char* kg = reinterpret_cast<const char*>(a.k + (int64_t)g * a.kv_sh);
  const uint32_t kvst_b = (uint32_t)(a.kv_st * 2);
  const uint32_t ring0 = est_lds_addr(ring);
  const int sub = lane / T::kChunks, cl = lane % T::kChunks;
  auto issue = [&](int64_t i) {
    const int64_t t = t_begin + i;
    if (t >= t_end) return;
    const int64_t k0 = t * kTileK;
    const int32_t n = (int32_t)(a.n_ctx - k0 < kTileK ? a.n_ctx - k0 : kTileK);
    const char* kb = kg + k0 * kvst_b;
    const uint32_t dst = ring0 + (uint32_t)((i & (kEstStages - 1)) * T::kBytes);
#pragma unroll
    for (int gi = 0; gi < T::kInstr; ++gi) {
      const int row = gi * R + sub;
      const uint32_t rr = (uint32_t)(row < n ? row : n - 1);
      est_dma16(kb, rr * kvst_b + (uint32_t)kslot<D>(cl, row) * 16u, dst + gi * 1024);
    }
  };
  auto land = [&](int64_t ahead) {  // only tile `ahead` may still be in flight
    if (t_begin + ahead < t_end) est_wait_vm<T::kInstr>();
    else est_wait_vm<0>();
  };
  issue(0);
  issue(1);
  land(1);
  est_barrier();
  for (int64_t i = 0; t_begin + i < t_end; ++i) {
    issue(i + 2);
    land(i + 2);
    est_barrier();
  }
}

template <int D>
__device__ __forceinline__ void load_q_frags(const EstArgs& a, int h, int64_t c,
                                             f16x8 (&qf)[2][D / 16]) {
  const int lane = threadIdx.x & 63;
  const uint16_t* base = a.q_est + (((int64_t)c * a.H + h) * kEstRows) * D;
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      qf[b][s] = *reinterpret_cast<const f16x8*>(
          base + (int64_t)(b * 32 + (lane & 31)) * D + s * 16 + 8 * (lane >> 5));
}

// First key of the next DCA chunk if the 64-key tile at k0 (in chunk c)
// meets a chunk edge, else k0 + 64 (never, without DCA).  A tile meets at
// most one edge: the period is at least 64 keys.
__device__ __forceinline__ int64_t straddle_edge(const EstArgs& a, int64_t k0, int64_t c) {
  const int64_t next = (c + 1) * a.period;
  return (a.period && next < k0 + kTileK && next < a.n_ctx) ? next : k0 + kTileK;
}

// K fragment s of key block kb: lane -> key row 32 kb + lane % 32, chunk
// 2 s + lane / 32.
template <int D>
__device__ __forceinline__ f16x8 k_frag(const char* ks, int kb, int s) {
  const int lane = threadIdx.x & 63;
  const int row = kb * 32 + (lane & 31);
  return *reinterpret_cast<const f16x8*>(ks + row * KTile<D>::kRowBytes +
                                          kslot<D>(2 * s + (lane >> 5), row) * 16);
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ------------------------------------------------------------------ pass 1
template <int D>
__global__ void __launch_bounds__(64 * (kMaxEstWaves + 1)) est_pass1(EstArgs a) {
  __shared__ __attribute__((aligned(16))) char ring[kEstStages][KTile<D>::kBytes];
  const int split = blockIdx.x;
  const int g = blockIdx.y / a.n_sub, sub = blockIdx.y % a.n_sub;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n_here = min(a.nw, a.G - sub * a.nw);
  const int64_t t_begin = (int64_t)split * a.tiles_per_split;
  const int64_t t_end = t_begin + a.tiles_per_split < a.n_tiles ? t_begin + a.tiles_per_split
                                                                 : a.n_tiles;
  if (w == a.nw) {
    est_loader<D>(a, g, t_begin, t_end, &ring[0][0], lane);
    return;
  }
  const int h = g * a.G + sub * a.nw + w;
  const bool active = w < n_here && ((a.head_mask >> h) & 1);
  f16x8 qf[2][D / 16];
  int64_t cur_c = -1;
  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
  const int half = lane >> 5;
  est_barrier();  // the first tile is in its stage
  for (int64_t i = 0; t_begin + i < t_end; ++i) {
    const int64_t t = t_begin + i;
    const int64_t k0 = t * kTileK;
    const char* ks = ring[i & (kEstStages - 1)];
    if (active) {
    const int64_t c = a.period ? k0 / a.period : 0;
    if (c != cur_c) {
      load_q_frags<D>(a, h, c, qf);
      cur_c = c;
    }
    // the tile needs masking only at the causal edge, past n_ctx or past a
    // DCA chunk edge inside it (those keys are the edge kernel's)
    const int64_t kedge = straddle_edge(a, k0, c);
    const bool edge = (k0 + kTileK - 1 > a.row0) || kedge < k0 + kTileK;
    // key block kb: its K fragments are read once and serve both row blocks
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f16x8 kf[D / 16];
#pragma unroll
      for (int s = 0; s < D / 16; ++s) kf[s] = k_frag<D>(ks, kb, s);
      f32x16 acc[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        acc[b] = (f32x16){};
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
          acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[s], qf[b][s], acc[b], 0, 0, 0);
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        if (edge) {
          const int64_t row = a.row0 + b * 32 + (lane & 31);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int64_t key = k0 + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            if (key > row || key >= a.n_ctx || key >= kedge) acc[b][r] = -INFINITY;
          }
        }
        // The row sum is kept against a reference m that need not be the
        // row max: 2^(x - m) is exact for any m.  The block's own max is
        // taken only for a row's first keys or when the block's sum leaves
        // 2^64 (then l is rescaled to the new m).  Exponentials below 2^-126
        // flush to zero (v_exp_f32), far below the precision of the row sum.
        // Four interleaved partial sums (fixed order) keep the chains short.
        auto block_sum = [&](float mref) {
          float sp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int r = 0; r < 16; ++r)
            sp[r & 3] += __builtin_amdgcn_exp2f(fmaf(acc[b][r], a.scale_log2, -mref));
          return (sp[0] + sp[1]) + (sp[2] + sp[3]);
        };
        float sum = block_sum(m[b] == -INFINITY ? 0.f : m[b]);
        const bool slow = m[b] == -INFINITY || !(sum <= 0x1p64f);
        if (__builtin_expect(__ballot(slow) != 0ull, 0) && slow) {
          float mx = -INFINITY;
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[b][r]);
          mx *= a.scale_log2;
          if (mx > m[b]) {
            l[b] = m[b] == -INFINITY ? 0.f : l[b] * exp2f(m[b] - mx);
            m[b] = mx;
            sum = block_sum(mx);
          }
        }
        l[b] += sum;
      }
    }
    }
    est_barrier();  // tile i done, tile i + 1 in its stage
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
      float* dst = a.part + (((int64_t)h * a.n_part + split) * kEstRows + b * 32 + lane) * 2;
      dst[0] = mm;
      dst[1] = ll;
    }
  }
}

// Row logsumexp from the split partials: thread (part, r) reduces splits
// part, part + 4, ... of row r; the four parts are then merged in order.
__global__ void __launch_bounds__(256) est_combine(EstArgs a) {
  const int h = blockIdx.x, r = threadIdx.x & 63, part = threadIdx.x >> 6;
  if (!((a.head_mask >> h) & 1)) return;
  __shared__ float pm[4][kEstRows], pl[4][kEstRows];
  const float* p = a.part + ((int64_t)h * a.n_part * kEstRows + r) * 2;
  float mm = -INFINITY;
  for (int z = part; z < a.n_part; z += 4) mm = fmaxf(mm, p[(int64_t)z * kEstRows * 2]);
  float ll = 0.f;
  if (mm != -INFINITY)
    for (int z = part; z < a.n_part; z += 4)
      ll += p[(int64_t)z * kEstRows * 2 + 1] * exp2f(p[(int64_t)z * kEstRows * 2] - mm);
  pm[part][r] = mm;
  pl[part][r] = ll;
  __syncthreads();
  if (part != 0) return;
  float M = pm[0][r];
  for (int u = 1; u < 4; ++u) M = fmaxf(M, pm[u][r]);
  float L = 0.f;
  if (M != -INFINITY)
    for (int u = 0; u < 4; ++u)
      if (pm[u][r] != -INFINITY) L += pl[u][r] * exp2f(pm[u][r] - M);
  a.lse2[h * kEstRows + r] = (r < a.n_rows && L > 0.f) ? M + log2f(L) : INFINITY;
}

// ------------------------------------------------------------------ pass 2
// Diagonal sums of a 32x32 block held in the S = Q K^T layout (lane -> key
// column n = lane % 32, register r -> query row m = 8(r/4) + 4(lane/32) +
// r%4): dst[d + 31] = sum_m X[m][m - d], d in [-31, 31] (dst[63] = 0).
// Lane t of each half pulls, for each of its half's rows m, the value of
// diagonal t (key n = m - t) or of diagonal t - 32 (key n = m - t + 32) with a
// lane permute; the two halves are then added, lower half first.  The order
// of the sums is fixed, so the records are reproducible.
__device__ __forceinline__ void diag_record(const float (&x)[16], float* dst) {
  const int lane = threadIdx.x & 63;
  const int t = lane & 31, half = lane >> 5;
  float pos = 0.f, neg = 0.f;  // diagonal t, diagonal t - 32
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = 8 * (r >> 2) + 4 * half + (r & 3);
    const int src = (half << 5) | ((m - t) & 31);
    const float v =
        __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(x[r])));
    if (m >= t) pos += v;
    else neg += v;
  }
  const float pos_o = __shfl_xor(pos, 32), neg_o = __shfl_xor(neg, 32);
  if (half == 0) {
    dst[t + 31] = pos + pos_o;
    if (t > 0) dst[t - 1] = neg + neg_o;
    else dst[63] = 0.f;
  }
}

template <int D>
__global__ void __launch_bounds__(64 * (kMaxEstWaves + 1)) est_pass2(EstArgs a) {
  __shared__ __attribute__((aligned(16))) char ring[kEstStages][KTile<D>::kBytes];
  __shared__ __attribute__((aligned(16))) float lse_all[kMaxEstWaves][kEstRows];
  const int split = blockIdx.x;
  const int g = blockIdx.y / a.n_sub, sub = blockIdx.y % a.n_sub;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n_here = min(a.nw, a.G - sub * a.nw);
  const int64_t t_begin = (int64_t)split * a.tiles_per_split;
  const int64_t t_end = t_begin + a.tiles_per_split < a.n_tiles ? t_begin + a.tiles_per_split
                                                                 : a.n_tiles;
  if (w == a.nw) {
    est_loader<D>(a, g, t_begin, t_end, &ring[0][0], lane);
    return;
  }
  const int h = g * a.G + sub * a.nw + w;
  const bool active = w < n_here && ((a.head_mask >> h) & 1);
  const int half = lane >> 5;
  f16x8 qf[2][D / 16];
  int64_t cur_c = -1;
  // log2-sum-exp of the wave's 64 rows (INFINITY for padding rows -> p = 0),
  // kept in LDS: rows 8 j + 4 half .. + 3 of block b are one 16-byte read
  float* lse = lse_all[w];
  lse[lane] = active ? a.lse2[h * kEstRows + lane] : INFINITY;
  float* vout = a.vscore + (int64_t)h * a.n_ctx;
  float* drec = a.diag + (int64_t)h * a.n_diag * 2 * 64;
  est_barrier();  // the first tile is in its stage
  for (int64_t i = 0; t_begin + i < t_end; ++i) {
    const int64_t t = t_begin + i;
    const int64_t k0 = t * kTileK;
    const char* ks = ring[i & (kEstStages - 1)];
    if (active) {
    const int64_t c = a.period ? k0 / a.period : 0;
    if (c != cur_c) {
      load_q_frags<D>(a, h, c, qf);
      cur_c = c;
    }
    const int64_t kedge = straddle_edge(a, k0, c);
    const bool edge = (k0 + kTileK - 1 > a.row0) || kedge < k0 + kTileK;
    // probabilities of the 32x32 block (row block b, key block kb)
    auto block_p = [&](int kb, int b, float (&pp)[16]) {
      f32x16 acc = {};
#pragma unroll
      for (int s = 0; s < D / 16; ++s)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(qf[b][s], k_frag<D>(ks, kb, s), acc, 0,
                                                      0, 0);
      const int64_t key = k0 + kb * 32 + (lane & 31);
      float lr[16];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<float4*>(&lr[4 * j]) =
            *reinterpret_cast<const float4*>(lse + b * 32 + 8 * j + 4 * half);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // probabilities below 2^-126 flush to zero (v_exp_f32): their sum
        // over the estimate rows stays below 2^-120
        float v = __builtin_amdgcn_exp2f(acc[r] * a.scale_log2 - lr[r]);
        if (edge) {
          const int64_t row = a.row0 + b * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (key > row || key >= a.n_ctx || key >= kedge) v = 0.f;
        }
        pp[r] = v;
      }
    };
    // vertical score of key block kb from this lane's partial row sum s:
    // the two halves' rows, lower half first
    auto vertical = [&](int kb, float s) {
      const float o = __shfl_xor(s, 32);
      const float tot = half ? o + s : s + o;
      const int64_t key = k0 + kb * 32 + (lane & 31);
      if (half == 0 && key < a.n_ctx) vout[key] = tot;
    };
    // The four 32x32 blocks (key block kb, row block b) in the order that
    // keeps at most two of them live: (0,0) and (1,1) first (their sum is one
    // diagonal record), then (kb 0, b 1) and (kb 1, b 0).  Vertical sums in a
    // fixed order: key block 0 adds its b = 0 rows then its b = 1 rows, key
    // block 1 its b = 1 rows then its b = 0 rows.  Diagonal records (index
    // e + 1): e = 2t holds blocks (0,0) + (1,1), e = 2t + 1 slot 0 the block
    // (b 0, kb 1), e = 2t - 1 slot 1 the block (b 1, kb 0).
    float pa[16], pb[16];
    block_p(0, 0, pa);
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s0 += pa[r];
    __builtin_amdgcn_sched_barrier(0);
    block_p(1, 1, pb);
#pragma unroll
    for (int r = 0; r < 16; ++r) s1 += pb[r];
#pragma unroll
    for (int r = 0; r < 16; ++r) pa[r] += pb[r];
    diag_record(pa, drec + ((2 * t + 1) * 2 + 0) * 64);
    __builtin_amdgcn_sched_barrier(0);
    block_p(0, 1, pa);
#pragma unroll
    for (int r = 0; r < 16; ++r) s0 += pa[r];
    vertical(0, s0);
    diag_record(pa, drec + ((2 * t) * 2 + 1) * 64);
    __builtin_amdgcn_sched_barrier(0);
    block_p(1, 0, pb);
#pragma unroll
    for (int r = 0; r < 16; ++r) s1 += pb[r];
    vertical(1, s1);
    diag_record(pb, drec + ((2 * t + 2) * 2 + 0) * 64);
    }
    est_barrier();  // tile i done, tile i + 1 in its stage
  }
}

// ------------------------------------------------------------ DCA edges
// Keys after a DCA chunk edge inside a 64-key tile (edge e = c S not a
// multiple of 64; keys e .. the tile's end), which the passes leave out:
// they meet the query rows rotated for chunk c.  Scores on the vector units,
// fp32 sums of the fp16 products (the operands of the matrix-core passes).

// Whether chunk c's first key e = c S lies inside a 64-key tile (and inside
// the context); e_end: one past the tile's last key.
__device__ __forceinline__ bool edge_tile(const EstArgs& a, int64_t c, int64_t& e,
                                          int64_t& e_end) {
  e = c * a.period;
  if (e >= a.n_ctx || (e % kTileK) == 0) return false;
  const int64_t k_end = (e / kTileK + 1) * kTileK;
  e_end = k_end < a.n_ctx ? k_end : a.n_ctx;
  return true;
}

// sm_scale <q_est[c][h][r], K[j]> in log2 units
template <int D>
__device__ __forceinline__ float edge_logit(const EstArgs& a, int h, int g, int64_t c, int r,
                                            int64_t j) {
  const uint16_t* q = a.q_est + (((int64_t)c * a.H + h) * kEstRows + r) * D;
  const uint16_t* k = a.k + (int64_t)g * a.kv_sh + j * a.kv_st;
  float acc = 0.f;
#pragma unroll 8
  for (int d = 0; d < D; ++d) acc = fmaf(f16_to_f32(q[d]), f16_to_f32(k[d]), acc);
  return acc * a.scale_log2;
}

// Pass 1 for the edge keys: one thread per estimate row, the edges in
// ascending order, an online max / sum into the head's last partial.
template <int D>
__global__ void __launch_bounds__(kEstRows) est_edge1(EstArgs a) {
  const int h = blockIdx.x, r = threadIdx.x;
  if (!((a.head_mask >> h) & 1)) return;
  const int g = h / a.G;
  const int64_t row = a.row0 + r;
  const int64_t n_kc = (a.n_ctx + a.period - 1) / a.period;
  float m = -INFINITY, l = 0.f;
  for (int64_t c = 1; c < n_kc; ++c) {
    int64_t e, e_end;
    if (!edge_tile(a, c, e, e_end)) continue;
    for (int64_t j = e; j < e_end && j <= row; ++j) {
      const float v = edge_logit<D>(a, h, g, c, r, j);
      if (v > m) {
        l = l * exp2f(m - v) + 1.f;
        m = v;
      } else {
        l += exp2f(v - m);
      }
    }
  }
  float* dst = a.part + (((int64_t)h * a.n_part + a.n_split) * kEstRows + r) * 2;
  dst[0] = m;
  dst[1] = l;
}

// Pass 2 for the edge keys, after est_pass2: the probabilities of the tile's
// 64 rows x 64 keys (zero outside the edge keys) in LDS, then the vertical
// scores of the edge keys (rows in ascending order) and the diagonal sums of
// the tile's four 32 x 32 blocks, added to the records pass 2 wrote (same
// record layout: blocks (0,0) + (1,1) in record 2t + 1 slot 0, block (row 1,
// key 0) in record 2t slot 1, block (row 0, key 1) in record 2t + 2 slot 0).
template <int D>
__global__ void __launch_bounds__(256) est_edge2(EstArgs a) {
  __shared__ float P[kEstRows][kTileK + 1];
  const int h = blockIdx.x, tid = threadIdx.x;
  if (!((a.head_mask >> h) & 1)) return;
  const int g = h / a.G;
  const int64_t n_kc = (a.n_ctx + a.period - 1) / a.period;
  float* drec = a.diag + (int64_t)h * a.n_diag * 2 * 64;
  for (int64_t c = 1; c < n_kc; ++c) {
    int64_t e, e_end;
    if (!edge_tile(a, c, e, e_end)) continue;
    const int64_t k0 = e / kTileK * kTileK, t = k0 / kTileK;
    for (int x = tid; x < kEstRows * kTileK; x += 256) {
      const int r = x / kTileK, n = x % kTileK;
      const int64_t j = k0 + n, row = a.row0 + r;
      float p = 0.f;
      if (j >= e && j < e_end && j <= row)
        p = exp2f(edge_logit<D>(a, h, g, c, r, j) - a.lse2[h * kEstRows + r]);
      P[r][n] = p;
    }
    __syncthreads();
    if (tid < kTileK) {
      const int64_t j = k0 + tid;
      if (j >= e && j < e_end) {
        float v = 0.f;
        for (int r = 0; r < kEstRows; ++r) v += P[r][tid];
        a.vscore[(int64_t)h * a.n_ctx + j] = v;
      }
    }
    // diagonal d = m - n' of a 32 x 32 block, d in [-31, 31]
    if (tid < 3 * 63) {
      const int target = tid / 63, d = tid % 63 - 31;
      float sum = 0.f;
      for (int blk = 0; blk < 2; ++blk) {
        int b, kb;
        if (target == 0) { b = blk; kb = blk; }           // (0,0) + (1,1)
        else if (target == 1) { if (blk) break; b = 1; kb = 0; }
        else { if (blk) break; b = 0; kb = 1; }
        for (int mm = 0; mm < 32; ++mm) {
          const int n = mm - d;
          if (n >= 0 && n < 32) sum += P[32 * b + mm][32 * kb + n];
        }
      }
      const int64_t rec = target == 0 ? ((2 * t + 1) * 2 + 0)
                        : target == 1 ? ((2 * t) * 2 + 1) : ((2 * t + 2) * 2 + 0);
      drec[rec * 64 + d + 31] += sum;
    }
    __syncthreads();
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
    // a DCA chunk edge inside a 64-key tile: its later keys take the edge
    // kernels and a partial of their own
    bool edges = false;
    for (int64_t c = 1; d.period && c * d.period < c1 && !edges; ++c)
      edges = (c * d.period) % kTileK != 0;
    a.n_part = a.n_split + (edges ? 1 : 0);
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
    // a workgroup = up to kMaxEstWaves query heads of one KV head + a loader
    a.n_sub = (a.G + kMaxEstWaves - 1) / kMaxEstWaves;
    a.nw = (a.G + a.n_sub - 1) / a.n_sub;
    const dim3 grid((unsigned)L.n_split, (unsigned)(p.n_kv_heads * a.n_sub));
    const dim3 block((unsigned)(64 * (a.nw + 1)));
    if (p.head_dim == 128) hipLaunchKernelGGL(est_pass1<128>, grid, block, 0, s, a);
    else hipLaunchKernelGGL(est_pass1<64>, grid, block, 0, s, a);
    rc = check_launch("estimate pass 1");
    if (rc) return rc;
    if (edges) {
      if (p.head_dim == 128) hipLaunchKernelGGL(est_edge1<128>, dim3(p.n_heads), dim3(kEstRows), 0, s, a);
      else hipLaunchKernelGGL(est_edge1<64>, dim3(p.n_heads), dim3(kEstRows), 0, s, a);
      rc = check_launch("estimate edge pass 1");
      if (rc) return rc;
    }
    hipLaunchKernelGGL(est_combine, dim3(p.n_heads), dim3(256), 0, s, a);
    rc = check_launch("estimate combine");
    if (rc) return rc;
    if (p.head_dim == 128) hipLaunchKernelGGL(est_pass2<128>, grid, block, 0, s, a);
    else hipLaunchKernelGGL(est_pass2<64>, grid, block, 0, s, a);
    rc = check_launch("estimate pass 2");
    if (rc) return rc;
    if (edges) {
      if (p.head_dim == 128) hipLaunchKernelGGL(est_edge2<128>, dim3(p.n_heads), dim3(256), 0, s, a);
      else hipLaunchKernelGGL(est_edge2<64>, dim3(p.n_heads), dim3(256), 0, s, a);
      rc = check_launch("estimate edge pass 2");
      if (rc) return rc;
    }
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
