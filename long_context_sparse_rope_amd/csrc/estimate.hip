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
// diagonal sums of every 32x32 block (lane permutes), all in a fixed order:
// the scores are bitwise reproducible.  A slash score gathers the diagonal
// sums of two consecutive tiles; a wave carries the previous tile's sums and
// writes each slash score once both tiles are done.  At the first tile of a
// key split the two tiles belong to two workgroups: both write their parts
// to a small boundary buffer and est_slash_fix adds them in the same order.
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
  float* bnd;             // [H][n_split][5][32] slash sums at key-split boundaries
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

// Row logsumexp from the split partials: one wave per (head, row); lane j
// merges partials j, j + 64, ... online in ascending order, then the lanes
// are merged pairwise over a fixed butterfly (lane distance 1, 2, ..., 32),
// so the result does not depend on timing.
__device__ __forceinline__ void merge_ml(float& m, float& l, float mv, float lv) {
  if (mv == -INFINITY) return;
  if (mv > m) {
    l = (m == -INFINITY ? 0.f : l * exp2f(m - mv)) + lv;
    m = mv;
  } else {
    l += lv * exp2f(mv - m);
  }
}

__global__ void __launch_bounds__(256) est_combine(EstArgs a) {
  const int h = blockIdx.y, r = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (!((a.head_mask >> h) & 1)) return;
  const float* p = a.part + ((int64_t)h * a.n_part * kEstRows + r) * 2;
  float m = -INFINITY, l = 0.f;
  for (int z = lane; z < a.n_part; z += 64)
    merge_ml(m, l, p[(int64_t)z * kEstRows * 2], p[(int64_t)z * kEstRows * 2 + 1]);
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const float mo = __shfl_xor(m, d), lo = __shfl_xor(l, d);
    // the lower lane's state first, in both lanes of the pair
    float ma = m, la = l, mb = mo, lb = lo;
    if (lane & d) {
      ma = mo;
      la = lo;
      mb = m;
      lb = l;
    }
    merge_ml(ma, la, mb, lb);
    m = ma;
    l = la;
  }
  if (lane == 0) a.lse2[h * kEstRows + r] = (r < a.n_rows && l > 0.f) ? m + log2f(l) : INFINITY;
}

// ------------------------------------------------------------------ pass 2
// Diagonal sums of a 32x32 block held in the S = Q K^T layout (lane -> key
// column n = lane % 32, register r -> query row m = 8(r/4) + 4(lane/32) +
// r%4): pos = sum_m X[m][m - t] (diagonal t) and neg = sum_m X[m][m - t +
// 32] (diagonal t - 32, zero for t = 0), t = lane % 32, in every lane.
// Lane t of each half pulls, for each of its half's rows m, the value of
// diagonal t or t - 32 with a lane permute; the two halves are then added,
// lower half first.  The order of the sums is fixed, so they are
// reproducible.
__device__ __forceinline__ void diag_pair(const float (&x)[16], float& pos_out, float& neg_out) {
  const int lane = threadIdx.x & 63;
  const int t = lane & 31, half = lane >> 5;
  // The rows m of registers r = 0..15 ascend, so the values of diagonal
  // t - 32 (m < t) come first: one running sum, saved as neg and restarted
  // at the first register with m >= t, adds each diagonal's values in
  // register order.
  float acc = 0.f, neg = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = 8 * (r >> 2) + 4 * half + (r & 3);
    const int mp = r ? 8 * ((r - 1) >> 2) + 4 * half + ((r - 1) & 3) : -1;
    const int src = (half << 5) | ((m - t) & 31);
    const float v =
        __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(x[r])));
    const bool start = m >= t && mp < t;  // first register of diagonal t
    neg = start ? acc : neg;
    acc = (start ? 0.f : acc) + v;
  }
  // every row below t: all values belong to diagonal t - 32
  float pos = acc;
  if (8 * 3 + 4 * half + 3 < t) {
    neg = acc;
    pos = 0.f;
  }
  const float pos_o = __shfl_xor(pos, 32), neg_o = __shfl_xor(neg, 32);
  pos_out = half ? pos_o + pos : pos + pos_o;
  neg_out = half ? neg_o + neg : neg + neg_o;
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
  float* sout = a.sscore + (int64_t)h * a.n_ctx;
  float* bnd = a.bnd + ((int64_t)h * a.n_split + split) * 5 * 32;
  const int lt = lane & 31;
  // Diagonal group E of the tiles holds the offsets o = row0 - 32 E + lt
  // (lt = lane % 32).  Tile t adds (row block b, key block kb) to group
  // 2t + kb - b: its diagonal t part (pos) to offset row0 - 32 E + lt and
  // its diagonal t - 32 part (neg) to offset row0 - 32 (E + 1) + lt.  So
  // the slash score of group E is neg(E - 1) + pos(E), and groups 2t - 1 and
  // 2t are complete after tile t.  Carried from the previous tile: neg of
  // its group 2t (c_na), pos and neg of its block (b 0, kb 1) (c_pb0, c_nb0).
  float c_na = 0.f, c_pb0 = 0.f, c_nb0 = 0.f;
  auto put = [&](int64_t E, float v) {
    const int64_t o = a.row0 - 32 * E + lt;
    if (half == 0 && o >= 0 && o < a.n_ctx) sout[o] = v;
  };
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
    // diagonal group), then (kb 0, b 1) and (kb 1, b 0).  Vertical sums in a
    // fixed order: key block 0 adds its b = 0 rows then its b = 1 rows, key
    // block 1 its b = 1 rows then its b = 0 rows.  Diagonal groups: A = (0,0)
    // + (1,1) is group 2t, B1 = (b 1, kb 0) group 2t - 1, B0 = (b 0, kb 1)
    // group 2t + 1.  Group 2t - 1 = (group 2t - 2's neg + group 2t - 1's pos
    // of the previous tile) + its pos of this tile (B1); group 2t = (group
    // 2t - 1's neg of the previous tile + that of B1) + A's pos.  At the
    // first tile of a split the carried parts are zero, so the boundary
    // buffer takes B1's own parts and A's pos.
    const bool first = i == 0 && t_begin > 0;
    float pa[16], pb[16];
    float s0 = 0.f, s1 = 0.f;
    float p_a, n_a;
    block_p(0, 0, pa);
#pragma unroll
    for (int r = 0; r < 16; ++r) s0 += pa[r];
    __builtin_amdgcn_sched_barrier(0);
    block_p(1, 1, pb);
#pragma unroll
    for (int r = 0; r < 16; ++r) s1 += pb[r];
#pragma unroll
    for (int r = 0; r < 16; ++r) pa[r] += pb[r];
    diag_pair(pa, p_a, n_a);  // A
    __builtin_amdgcn_sched_barrier(0);
    block_p(0, 1, pa);
#pragma unroll
    for (int r = 0; r < 16; ++r) s0 += pa[r];
    vertical(0, s0);
    {
      float p, n;
      diag_pair(pa, p, n);  // B1
      const float v1 = (c_na + c_pb0) + p;
      const float w = c_nb0 + n;
      if (first) {
        if (half == 0) {
          bnd[2 * 32 + lt] = v1;
          bnd[3 * 32 + lt] = w;
          bnd[4 * 32 + lt] = p_a;
        }
      } else {
        put(2 * t - 1, v1);
        put(2 * t, w + p_a);
      }
      c_na = n_a;
    }
    __builtin_amdgcn_sched_barrier(0);
    block_p(1, 0, pb);
#pragma unroll
    for (int r = 0; r < 16; ++r) s1 += pb[r];
    vertical(1, s1);
    diag_pair(pb, c_pb0, c_nb0);  // B0
    }
    est_barrier();  // tile i done, tile i + 1 in its stage
  }
  if (!active || t_begin >= t_end) return;
  if (t_end == a.n_tiles) {
    // the last tile of the context: groups 2t + 1 and 2t + 2 have no later tile
    const int64_t t = t_end - 1;
    put(2 * t + 1, c_na + c_pb0);
    put(2 * t + 2, c_nb0);
  } else if (half == 0) {
    bnd[0 * 32 + lt] = c_na + c_pb0;
    bnd[1 * 32 + lt] = c_nb0;
  }
}

// Slash scores of the two diagonal groups at each key-split boundary: the
// previous split's parts, then the next split's, in pass 2's order.
__global__ void __launch_bounds__(256) est_slash_fix(EstArgs a) {
  const int h = blockIdx.y;
  const int z = blockIdx.x * 8 + (threadIdx.x >> 5), lt = threadIdx.x & 31;
  if (!((a.head_mask >> h) & 1) || z < 1 || z >= a.n_split) return;
  const int64_t tb = (int64_t)z * a.tiles_per_split;
  if (tb >= a.n_tiles) return;
  const float* x = a.bnd + ((int64_t)h * a.n_split + z - 1) * 5 * 32;
  const float* y = x + 5 * 32;
  float* sout = a.sscore + (int64_t)h * a.n_ctx;
  const int64_t o1 = a.row0 - 32 * (2 * tb - 1) + lt, o2 = o1 - 32;
  if (o1 >= 0 && o1 < a.n_ctx) sout[o1] = x[0 * 32 + lt] + y[2 * 32 + lt];
  if (o2 >= 0 && o2 < a.n_ctx) sout[o2] = (x[1 * 32 + lt] + y[3 * 32 + lt]) + y[4 * 32 + lt];
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

// Pass 2 for the edge keys, after est_pass2 and est_slash_fix: the
// probabilities of the tile's 64 rows x 64 keys (zero outside the edge keys)
// in LDS, then the vertical scores of the edge keys (rows in ascending order)
// and, per offset row0 + r - (k0 + n) met in the tile, the sum over its rows
// (ascending), added to the slash score pass 2 wrote.  One thread per offset,
// and the edge tiles in ascending order, so the sums are reproducible.
template <int D>
__global__ void __launch_bounds__(256) est_edge2(EstArgs a) {
  __shared__ float P[kEstRows][kTileK + 1];
  const int h = blockIdx.x, tid = threadIdx.x;
  if (!((a.head_mask >> h) & 1)) return;
  const int g = h / a.G;
  const int64_t n_kc = (a.n_ctx + a.period - 1) / a.period;
  for (int64_t c = 1; c < n_kc; ++c) {
    int64_t e, e_end;
    if (!edge_tile(a, c, e, e_end)) continue;
    const int64_t k0 = e / kTileK * kTileK;
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
    // offset o = row0 - k0 + dr, dr = r - n in [-63, 63]
    if (tid < 2 * kTileK - 1) {
      const int dr = tid - (kTileK - 1);
      const int64_t o = a.row0 - k0 + dr;
      if (o >= 0 && o < a.n_ctx) {
        float sum = 0.f;
        for (int r = 0; r < kEstRows; ++r) {
          const int n = r - dr;
          if (n >= 0 && n < kTileK) sum += P[r][n];
        }
        a.sscore[(int64_t)h * a.n_ctx + o] += sum;
      }
    }
    __syncthreads();
  }
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
  float* bnd = reinterpret_cast<float*>(cur);
  cur += L.bnd;
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
    a.bnd = bnd;
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
    hipLaunchKernelGGL(est_combine, dim3(kEstRows / 4, p.n_heads), dim3(256), 0, s, a);
    rc = check_launch("estimate combine");
    if (rc) return rc;
    if (p.head_dim == 128) hipLaunchKernelGGL(est_pass2<128>, grid, block, 0, s, a);
    else hipLaunchKernelGGL(est_pass2<64>, grid, block, 0, s, a);
    rc = check_launch("estimate pass 2");
    if (rc) return rc;
    if (a.n_split > 1) {
      hipLaunchKernelGGL(est_slash_fix, dim3((unsigned)((a.n_split + 7) / 8), p.n_heads),
                         dim3(256), 0, s, a);
      rc = check_launch("estimate slash boundaries");
      if (rc) return rc;
    }
    if (edges) {
      if (p.head_dim == 128) hipLaunchKernelGGL(est_edge2<128>, dim3(p.n_heads), dim3(256), 0, s, a);
      else hipLaunchKernelGGL(est_edge2<64>, dim3(p.n_heads), dim3(256), 0, s, a);
      rc = check_launch("estimate edge pass 2");
      if (rc) return rc;
    }
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
