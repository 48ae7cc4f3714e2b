// Vertical-slash sparse prefill attention with DCA positions, on the
// matrix cores.
//
// Page: "論文解説: Qwen2.5-1M" (0h-n0.github.io): 疎アテンション (attention over
// the critical tokens only), Length Extrapolation (DCA intra / successive /
// inter patterns, YaRN temperature) and "アルゴリズム: DCAと疎アテンションの統合"
// (weights with the DCA positions).  Blocked attention with an online
// softmax: deepseekmodel.com long-context architecture page, §3.2.
//
// Work decomposition (our design; the pages give no kernel):
//  * a workgroup = one query head x 128 query rows (4 waves x 32 rows);
//  * slash offsets are merged into runs (consecutive offsets closer than
//    128); for the tile, run [oa, ob] covers the key span
//    [r0 - ob, r0 + 127 - oa], cut at DCA chunk edges into 64-key tiles;
//  * verticals not inside any span are gathered into 64-key tiles;
//  * per (wave, key tile) the pair mask is: key <= row and (offset bit or
//    column bit); tiles a wave does not touch are skipped, tiles it fully
//    covers run without a mask;
//  * S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_bf16: each lane
//    owns one query row, so the softmax max / sum and the O rescale are
//    in-lane (one exchange between the two lane halves per tile);
//  * the DCA relation of a (wave, tile) pair picks one of three pre-rotated
//    query variants (intra / successive / inter).
#include <cmath>

#include "lcsr_internal.h"

namespace lcsr {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kVBatch = kThreads;  // verticals examined per batch

struct AttnArgs {
  const uint16_t* q_rot;   // [n_var][H][L][D]
  const uint16_t* k;       // K cache (rotated at P_k)
  const uint16_t* v;       // V cache
  int64_t kv_sh, kv_st;
  int32_t H, G, n_var;
  int64_t c0, L, n_ctx;
  int64_t period;          // S (0: DCA off)
  int64_t n_qt;            // query tiles
  int64_t n_blocks;        // H * n_qt
  float scale_log2;
  const uint32_t* off_bits;  // [H][n_words]
  const uint32_t* col_bits;  // [H][n_words]
  int64_t n_words;
  const int32_t* runs;       // [H][max_slash][2]
  const int32_t* run_cnt;    // [H]
  int32_t max_runs;
  const int32_t* vert_idx;   // [H][max_vert]
  const int32_t* vert_cnt;   // [H]
  int32_t max_vert;
  int32_t dense;
  uint64_t head_mask;
  void* out;
  int32_t out_dtype;
  int64_t o_sh, o_st;
  float* lse;
  unsigned long long* stats;
};

// bits [pos, pos + 64) of a bitmap; bits at negative positions are 0 (the
// bitmap carries zero words past its end).
__device__ __forceinline__ uint64_t get64(const uint32_t* bm, int64_t pos) {
  if (pos <= -64) return 0;
  const int64_t wi = pos >> 5;
  const int sh = (int)(pos & 31);
  const uint32_t w0 = wi >= 0 ? bm[wi] : 0u;
  const uint32_t w1 = wi + 1 >= 0 ? bm[wi + 1] : 0u;
  const uint32_t w2 = wi + 2 >= 0 ? bm[wi + 2] : 0u;
  const uint64_t lo = ((uint64_t)w1 << 32) | w0;
  return sh ? (lo >> sh) | ((uint64_t)w2 << (64 - sh)) : lo;
}

__device__ __forceinline__ uint64_t low_bits(int64_t n) {  // n in [0, 64]
  return n >= 64 ? ~0ull : (n <= 0 ? 0ull : ((1ull << n) - 1));
}

// any / all bits set in [a, b] (a > b: empty -> any false, all true)
__device__ __forceinline__ bool any_bits(const uint32_t* bm, int64_t a, int64_t b) {
  for (int64_t p = a; p <= b; p += 64) {
    const uint64_t w = get64(bm, p) & low_bits(b - p + 1);
    if (w) return true;
  }
  return false;
}
__device__ __forceinline__ bool all_bits(const uint32_t* bm, int64_t a, int64_t b) {
  for (int64_t p = a; p <= b; p += 64) {
    const uint64_t m = low_bits(b - p + 1);
    if ((get64(bm, p) & m) != m) return false;
  }
  return true;
}

__device__ __forceinline__ uint64_t bitrev64(uint64_t x) {
  const uint32_t lo = __builtin_bitreverse32((uint32_t)x);
  const uint32_t hi = __builtin_bitreverse32((uint32_t)(x >> 32));
  return ((uint64_t)lo << 32) | hi;
}

template <int D>
struct Smem {
  static constexpr int kKStride = D + 8;       // bf16 per K row
  static constexpr int kVStride = kTileK + 8;  // bf16 per V^T row
  uint16_t ks[kTileK * kKStride];
  uint16_t vt[D * kVStride];
  int32_t vlist[kVBatch];
  int32_t wave_cnt[kWaves];
  unsigned long long stat[2];
};

// Position of key k (0..63) of a tile in the V^T rows: bits 2 and 3 swapped,
// so that the 8 keys one lane half feeds to a 16-key MFMA step are contiguous.
__device__ __forceinline__ int vt_pos(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

// Load one 64-key tile of K (row-major) and V (transposed) into LDS.  Keys
// come from [ks, ks + n) (gather == false) or from vlist[s0 .. s0 + n)
// (gather == true); missing rows are zero.
template <int D>
__device__ __forceinline__ void load_tile(const AttnArgs& a, int g, Smem<D>& sm, bool gather,
                                          int64_t ks, int s0, int n) {
  const int t = threadIdx.x;
  const uint16_t* kb = a.k + (int64_t)g * a.kv_sh;
  const uint16_t* vb = a.v + (int64_t)g * a.kv_sh;
  constexpr int kChunks = D / 8;           // 16-byte chunks per row
  constexpr int kRowsPerPass = kThreads / kChunks;
  // K: thread -> (row, chunk), rows strided by kRowsPerPass
  {
    const int cc = t % kChunks;
    for (int r = t / kChunks; r < kTileK; r += kRowsPerPass) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (r < n) {
        const int64_t key = gather ? (int64_t)sm.vlist[s0 + r] : ks + r;
        v = *reinterpret_cast<const u32x4*>(kb + key * a.kv_st + cc * 8);
      }
      *reinterpret_cast<u32x4*>(sm.ks + r * Smem<D>::kKStride + cc * 8) = v;
    }
  }
  // V: thread -> (4 consecutive keys, 8 consecutive d); transposed store
  for (int unit = t; unit < (kTileK / 4) * kChunks; unit += kThreads) {
    const int dc = unit % kChunks, kg = unit / kChunks;
    u32x4 rows[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = kg * 4 + j;
      rows[j] = (u32x4){0u, 0u, 0u, 0u};
      if (r < n) {
        const int64_t key = gather ? (int64_t)sm.vlist[s0 + r] : ks + r;
        rows[j] = *reinterpret_cast<const u32x4*>(vb + key * a.kv_st + dc * 8);
      }
    }
    const int p0 = vt_pos(kg * 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {  // dword e holds d = 8dc + 2e (lo) and 2e + 1 (hi)
      const uint32_t lo01 = __builtin_amdgcn_perm(rows[1][e], rows[0][e], 0x05040100u);
      const uint32_t lo23 = __builtin_amdgcn_perm(rows[3][e], rows[2][e], 0x05040100u);
      const uint32_t hi01 = __builtin_amdgcn_perm(rows[1][e], rows[0][e], 0x07060302u);
      const uint32_t hi23 = __builtin_amdgcn_perm(rows[3][e], rows[2][e], 0x07060302u);
      uint16_t* d0 = sm.vt + (dc * 8 + 2 * e) * Smem<D>::kVStride + p0;
      *reinterpret_cast<uint2*>(d0) = make_uint2(lo01, lo23);
      *reinterpret_cast<uint2*>(d0 + Smem<D>::kVStride) = make_uint2(hi01, hi23);
    }
  }
}

template <int D>
struct WaveState {
  bf16x8 q[D / 16];
  f32x16 o[D / 32];
  float m, l;
  int var;
  unsigned long long exec, sel;
};

template <int D>
__device__ __forceinline__ void load_q(const AttnArgs& a, int h, int64_t i0, int var,
                                       WaveState<D>& st) {
  const int lane = threadIdx.x & 63;
  const int64_t t = i0 - a.c0 + (lane & 31);
  const uint16_t* base = a.q_rot + (((int64_t)var * a.H + h) * a.L + t) * D + 8 * (lane >> 5);
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    if (t < a.L) st.q[s] = *reinterpret_cast<const bf16x8*>(base + s * 16);
    else st.q[s] = (bf16x8){};
  }
  st.var = var;
}

// One (wave, key tile) step.  mask_mode: 0 none, 1 span mask, 2 vertical.
template <int D>
__device__ __forceinline__ void wave_tile(const AttnArgs& a, Smem<D>& sm, WaveState<D>& st,
                                          int mask_mode, uint64_t mword) {
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;
  f32x16 acc[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    acc[kb] = (f32x16){};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(
          sm.ks + (kb * 32 + (lane & 31)) * Smem<D>::kKStride + s * 16 + 8 * half);
      acc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, st.q[s], acc[kb], 0, 0, 0);
    }
  }
  // scale (log2 domain) and mask; register r of block kb holds key
  // 32 kb + 8 (r / 4) + 4 half + r % 4 of the tile
  const uint64_t mh = mword >> (4 * half);
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float x = acc[kb][r] * a.scale_log2;
      if (mask_mode) {
        const int bit = 32 * kb + 8 * (r >> 2) + (r & 3);
        if (!((mh >> bit) & 1ull)) x = -INFINITY;
      }
      acc[kb][r] = x;
      mx = fmaxf(mx, x);
    }
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float m_new = fmaxf(st.m, mx);
  // rescale the running sums when the row max grew
  if (__ballot(m_new > st.m) != 0ull) {
    const float alpha = (st.m == -INFINITY) ? 0.f : exp2f(st.m - m_new);
    st.l *= alpha;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o[db][r] *= alpha;
    st.m = m_new;
  }
  const float msub = (st.m == -INFINITY) ? 0.f : st.m;
  bf16x8 pf[4];
  float psum = 0.f;
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // the row sum adds the bf16-rounded weights the PV product uses, so
      // the output is an exact convex combination of those weights
      const __bf16 pb = (__bf16)exp2f(acc[s >> 1][8 * (s & 1) + e] - msub);
      psum += (float)pb;
      pf[s][e] = pb;
    }
  st.l += psum;
  // O^T += V^T P^T
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8 vf = *reinterpret_cast<const bf16x8*>(
          sm.vt + (db * 32 + (lane & 31)) * Smem<D>::kVStride + 16 * s + 8 * half);
      st.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[s], st.o[db], 0, 0, 0);
    }
}

template <int D>
__global__ void __launch_bounds__(kThreads) attn_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) Smem<D> sm;
  // XCD-aware order: consecutive logical blocks (same KV group and query
  // tile, then the next tile) land on one XCD, sharing its L2.
  const int64_t nb = a.n_blocks;
  const int64_t per_xcd = (nb + 7) / 8;
  const int64_t logical = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (logical >= nb) return;
  const int64_t gq = logical / a.G;  // (g, qt)
  const int hh = (int)(logical % a.G);
  const int g = (int)(gq / a.n_qt);
  const int64_t qt = gq % a.n_qt;
  const int h = g * a.G + hh;
  if (!((a.head_mask >> h) & 1)) return;

  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, half = lane >> 5;
  const int64_t r0 = a.c0 + qt * kTileQ;
  const int64_t c1 = a.n_ctx;
  const int64_t rlast = (r0 + kTileQ - 1 < c1 - 1) ? r0 + kTileQ - 1 : c1 - 1;
  const int64_t i0 = r0 + 32 * w;          // first row of this wave
  const bool wave_live = i0 <= rlast;
  const int64_t my_row = i0 + (lane & 31);
  const int64_t qchunk = a.period ? i0 / a.period : 0;
  const uint32_t* offb = a.off_bits + (int64_t)h * a.n_words;
  const uint32_t* colb = a.col_bits + (int64_t)h * a.n_words;

  WaveState<D> st;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) st.o[db] = (f32x16){};
  st.m = -INFINITY;
  st.l = 0.f;
  st.var = -1;
  st.exec = 0;
  st.sel = 0;
  if (threadIdx.x < 2) sm.stat[threadIdx.x] = 0;
  __syncthreads();

  // per (wave, tile) decision and step; kchunk = DCA chunk of the tile
  auto step = [&](bool gather, int64_t ks, int n, int s0, int64_t kchunk) {
    if (!wave_live) return;
    int64_t kmax;  // largest key of the tile
    if (gather) kmax = sm.vlist[s0 + n - 1];
    else kmax = ks + n - 1;
    const int64_t kmin = gather ? (int64_t)sm.vlist[s0] : ks;
    if (kmin > i0 + 31) return;  // whole tile in the future of this wave
    int mode;
    uint64_t mword = 0;
    if (!gather) {
      const int64_t olo = i0 - kmax, ohi = i0 + 31 - ks;
      const bool any_off = any_bits(offb, olo > 0 ? olo : 0, ohi);
      const bool any_col = (get64(colb, ks) & low_bits(n)) != 0ull;
      if (!any_off && !any_col) return;
      const bool full = (n == kTileK) && (kmax <= i0) && all_bits(offb, olo, ohi);
      mode = full ? 0 : 1;
      if (mode) {
        // offsets of my row: key ks + m <-> offset my_row - ks - m
        const uint64_t w_off = get64(offb, my_row - ks - 63);
        const uint64_t w_col = get64(colb, ks) & low_bits(n);
        mword = (bitrev64(w_off) | w_col) & low_bits(my_row - ks + 1) & low_bits(n);
      }
    } else {
      mode = (n == kTileK && kmax <= i0) ? 0 : 2;
      if (mode) {
        // count of gathered keys <= my_row (keys ascending)
        int lo = 0, hi = n;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if ((int64_t)sm.vlist[s0 + mid] <= my_row) lo = mid + 1;
          else hi = mid;
        }
        mword = low_bits(lo);
      }
    }
    const int64_t rel = qchunk - kchunk;
    const int var = a.n_var == 1 ? 0 : (rel >= 2 ? 2 : (int)rel);
    if (var != st.var) load_q<D>(a, h, i0, var, st);
    wave_tile<D>(a, sm, st, mode, mword);
    // statistics: multiplied pairs and pairs of the critical sets
    st.exec += 32ull * kTileK;
    if (half == 0 && my_row <= rlast)
      st.sel += mode ? (unsigned long long)__popcll(mword) : (unsigned long long)n;
  };

  // ---------------- spans from the slash runs
  const int n_runs = a.dense ? 1 : min(a.run_cnt[h], a.max_runs);
  const int32_t* runs = a.runs + (int64_t)h * a.max_runs * 2;
  for (int ru = 0; ru < n_runs; ++ru) {
    const int64_t oa = a.dense ? 0 : runs[2 * ru];
    const int64_t ob = a.dense ? c1 - 1 : runs[2 * ru + 1];
    if (oa > r0 + kTileQ - 1) break;
    const int64_t lo = r0 - ob > 0 ? r0 - ob : 0;
    const int64_t hi = (r0 + kTileQ - 1 - oa < rlast) ? r0 + kTileQ - 1 - oa : rlast;
    for (int64_t ks = lo; ks <= hi;) {
      int64_t ke = ks + kTileK < hi + 1 ? ks + kTileK : hi + 1;
      const int64_t kchunk = a.period ? ks / a.period : 0;
      if (a.period && ke > (kchunk + 1) * a.period) ke = (kchunk + 1) * a.period;
      __syncthreads();
      load_tile<D>(a, g, sm, false, ks, 0, (int)(ke - ks));
      __syncthreads();
      step(false, ks, (int)(ke - ks), 0, kchunk);
      ks = ke;
    }
  }

  // ---------------- verticals outside every span, gathered
  if (!a.dense) {
    const int vcnt = min(a.vert_cnt[h], a.max_vert);
    const int32_t* verts = a.vert_idx + (int64_t)h * a.max_vert;
    for (int vb = 0; vb < vcnt; vb += kVBatch) {
      if (verts[vb] > rlast) break;  // ascending: nothing further is causal
      const int i = vb + threadIdx.x;
      bool keep = false;
      if (i < vcnt) {
        const int64_t v = verts[i];
        if (v >= 0 && v <= rlast) {
          const int64_t olo = r0 - v > 0 ? r0 - v : 0;
          keep = !any_bits(offb, olo, r0 + kTileQ - 1 - v);
        }
      }
      const uint64_t bal = __ballot(keep);
      __syncthreads();  // previous batch's tiles are done with vlist
      if (lane == 0) sm.wave_cnt[w] = __popcll(bal);
      __syncthreads();
      int base = 0, total = 0;
      for (int x = 0; x < kWaves; ++x) {
        if (x < w) base += sm.wave_cnt[x];
        total += sm.wave_cnt[x];
      }
      if (keep) {
        const uint32_t below = __builtin_amdgcn_mbcnt_hi(
            (uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
        sm.vlist[base + below] = verts[i];
      }
      __syncthreads();
      for (int s0 = 0; s0 < total;) {
        const int64_t kchunk = a.period ? (int64_t)sm.vlist[s0] / a.period : 0;
        int s1 = s0 + kTileK < total ? s0 + kTileK : total;
        if (a.period) {
          int x = s0 + 1;
          while (x < s1 && (int64_t)sm.vlist[x] / a.period == kchunk) ++x;
          s1 = x;
        }
        __syncthreads();
        load_tile<D>(a, g, sm, true, 0, s0, s1 - s0);
        __syncthreads();
        step(true, 0, s1 - s0, s0, kchunk);
        s0 = s1;
      }
    }
  }

  // ---------------- epilogue
  if (wave_live) {
    const float l_tot = st.l + __shfl_xor(st.l, 32);
    const bool row_ok = my_row <= rlast;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (row_ok) {
      const int64_t t = my_row - a.c0;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d = 32 * db + 8 * i4 + 4 * half;
          const float v0 = st.o[db][4 * i4 + 0] * inv, v1 = st.o[db][4 * i4 + 1] * inv;
          const float v2 = st.o[db][4 * i4 + 2] * inv, v3 = st.o[db][4 * i4 + 3] * inv;
          if (a.out_dtype == LCSR_FP32) {
            float* o = static_cast<float*>(a.out) + h * a.o_sh + t * a.o_st + d;
            *reinterpret_cast<float4*>(o) = make_float4(v0, v1, v2, v3);
          } else {
            uint16_t* o = static_cast<uint16_t*>(a.out) + h * a.o_sh + t * a.o_st + d;
            *reinterpret_cast<uint2*>(o) = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
          }
        }
      if (a.lse && half == 0)
        a.lse[(int64_t)h * a.L + t] = l_tot > 0.f ? (st.m + log2f(l_tot)) * kLn2 : -INFINITY;
    }
  }
  if (a.stats) {
    unsigned long long ex = st.exec, se = st.sel;
    if (lane != 0) ex = 0;  // exec is wave-uniform
    for (int off = 32; off > 0; off >>= 1) se += __shfl_xor(se, off);
    if (lane == 0) {
      atomicAdd(&sm.stat[0], ex);
      atomicAdd(&sm.stat[1], se);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      atomicAdd(&a.stats[0], sm.stat[0]);
      atomicAdd(&a.stats[1], sm.stat[1]);
    }
  }
}

// ---------------------------------------------------------------- aux
struct AuxArgs {
  const int32_t* vert_idx;
  const int32_t* vert_cnt;
  int32_t max_vert;
  const int32_t* slash_idx;
  const int32_t* slash_cnt;
  int32_t max_slash;
  int64_t n_ctx, n_words;
  uint32_t* off_bits;
  uint32_t* col_bits;
  int32_t* runs;
  int32_t* run_cnt;
  int32_t dense;
  uint64_t head_mask;
};

constexpr int kAuxThreads = 1024;

// Per head: offset / column bitmaps and the slash runs (consecutive offsets
// at most 128 apart).  Indices outside [0, n_ctx) are ignored; indices must
// be ascending.
__global__ void __launch_bounds__(kAuxThreads) aux_kernel(AuxArgs a) {
  const int h = blockIdx.x;
  if (!((a.head_mask >> h) & 1)) return;
  uint32_t* ob = a.off_bits + (int64_t)h * a.n_words;
  uint32_t* cb = a.col_bits + (int64_t)h * a.n_words;
  const int tid = threadIdx.x;
  for (int64_t wi = tid; wi < a.n_words; wi += kAuxThreads) {
    uint32_t v = 0;
    if (a.dense) {
      const int64_t b0 = wi * 32;
      if (b0 + 32 <= a.n_ctx) v = 0xFFFFFFFFu;
      else if (b0 < a.n_ctx) v = (1u << (a.n_ctx - b0)) - 1u;
    }
    ob[wi] = v;
    cb[wi] = 0u;
  }
  if (a.dense) {
    if (tid == 0) a.run_cnt[h] = 1;
    return;
  }
  __syncthreads();
  const int ns = min(a.slash_cnt[h], a.max_slash), nv = min(a.vert_cnt[h], a.max_vert);
  const int32_t* so = a.slash_idx + (int64_t)h * a.max_slash;
  const int32_t* vo = a.vert_idx + (int64_t)h * a.max_vert;
  for (int i = tid; i < ns; i += kAuxThreads) {
    const int32_t o = so[i];
    if (o >= 0 && o < a.n_ctx) atomicOr(&ob[o >> 5], 1u << (o & 31));
  }
  for (int i = tid; i < nv; i += kAuxThreads) {
    const int32_t v = vo[i];
    if (v >= 0 && v < a.n_ctx) atomicOr(&cb[v >> 5], 1u << (v & 31));
  }
  // runs: a run starts at the first valid offset and wherever the gap to the
  // previous valid offset exceeds the query tile height
  __shared__ int s_wave[kAuxThreads / 64];
  __shared__ int s_carry;
  __shared__ int s_last;  // previous valid offset carried across batches
  if (tid == 0) {
    s_carry = 0;
    s_last = -1;
  }
  __syncthreads();
  int32_t* rr = a.runs + (int64_t)h * a.max_slash * 2;
  const int lane = tid & 63, w = tid >> 6;
  for (int b0 = 0; b0 < ns; b0 += kAuxThreads) {
    const int i = b0 + tid;
    const int32_t o = i < ns ? so[i] : -1;
    const bool valid = o >= 0 && o < a.n_ctx;
    // previous valid offset: offsets are ascending, so it is so[i - 1] when
    // valid (invalid entries sit only at the ends)
    int32_t prev = -1;
    if (valid) {
      if (i == b0) prev = s_last;
      else {
        const int32_t pv = so[i - 1];
        prev = (pv >= 0 && pv < a.n_ctx) ? pv : -1;
      }
    }
    const bool start = valid && (prev < 0 || o - prev > kTileQ);
    const uint64_t bal = __ballot(start);
    if (lane == 0) s_wave[w] = __popcll(bal);
    __syncthreads();
    int base = s_carry;
    for (int x = 0; x < w; ++x) base += s_wave[x];
    const int below = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
    if (start) rr[2 * (base + below)] = o;
    __syncthreads();
    if (tid == 0) {
      int tot = 0;
      for (int x = 0; x < kAuxThreads / 64; ++x) tot += s_wave[x];
      s_carry += tot;
      int last = s_last;
      const int end = b0 + kAuxThreads < ns ? b0 + kAuxThreads : ns;
      for (int x = end - 1; x >= b0; --x) {
        if (so[x] >= 0 && so[x] < a.n_ctx) {
          last = so[x];
          break;
        }
      }
      s_last = last;
    }
    __syncthreads();
  }
  // run ends: the run r ends at the last valid offset before run r + 1 starts
  const int nr = s_carry;
  for (int b0 = 0; b0 < ns; b0 += kAuxThreads) {
    const int i = b0 + tid;
    if (i < ns) {
      const int32_t o = so[i];
      const bool valid = o >= 0 && o < a.n_ctx;
      // o ends a run if it is valid and the next valid offset starts a new
      // run (or there is none)
      if (valid) {
        int32_t nx = -1;
        if (i + 1 < ns) {
          const int32_t q = so[i + 1];
          nx = (q >= 0 && q < a.n_ctx) ? q : -1;
        }
        if (nx < 0 || nx - o > kTileQ) {
          // find the run index: runs are ordered, binary search on starts
          int lo = 0, hi = nr - 1;
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (rr[2 * mid] <= o) lo = mid;
            else hi = mid - 1;
          }
          rr[2 * lo + 1] = o;
        }
      }
    }
  }
  if (tid == 0) a.run_cnt[h] = nr;
}

}  // namespace

int build_pattern_aux(const lcsr_problem_t& p, const lcsr_pattern_t& pat, uint64_t head_mask,
                      bool dense, const AttnLayout& L, char* ws, hipStream_t s) {
  char* cur = ws + L.q_rot;
  AuxArgs a{};
  a.vert_idx = pat.vert_idx;
  a.vert_cnt = pat.vert_cnt;
  a.max_vert = pat.max_vert;
  a.slash_idx = pat.slash_idx;
  a.slash_cnt = pat.slash_cnt;
  a.max_slash = pat.max_slash;
  a.n_ctx = L.n_ctx;
  a.n_words = L.n_words;
  a.off_bits = reinterpret_cast<uint32_t*>(cur);
  cur += L.off_bits;
  a.col_bits = reinterpret_cast<uint32_t*>(cur);
  cur += L.col_bits;
  a.runs = reinterpret_cast<int32_t*>(cur);
  cur += L.runs;
  a.run_cnt = reinterpret_cast<int32_t*>(cur);
  a.dense = dense ? 1 : 0;
  a.head_mask = head_mask;
  hipLaunchKernelGGL(aux_kernel, dim3(p.n_heads), dim3(kAuxThreads), 0, s, a);
  return check_launch("pattern aux");
}

int run_attention(const lcsr_problem_t& p, const lcsr_pattern_t& pat, uint64_t head_mask,
                  void* out, int32_t out_dtype, int64_t o_sh, int64_t o_st, float* lse,
                  int64_t* stats, bool dense, char* ws, hipStream_t s) {
  const AttnLayout L = attn_layout(p, dense ? 1 : pat.max_slash, true);
  FreqTable ft;
  int rc = build_freq_table(&p.rope, p.head_dim, &ft);
  if (rc) return rc;
  const DcaParams d = make_dca(&p.dca);
  uint16_t* q_rot = reinterpret_cast<uint16_t*>(ws);
  rc = launch_rotate_q_variants(p, ft, d, q_rot, (int)L.n_var, s);
  if (rc) return rc;
  rc = build_pattern_aux(p, pat, head_mask, dense, L, ws, s);
  if (rc) return rc;
  char* cur = ws + L.q_rot;
  AttnArgs a{};
  a.q_rot = q_rot;
  a.k = static_cast<const uint16_t*>(p.k_cache);
  a.v = static_cast<const uint16_t*>(p.v_cache);
  a.kv_sh = p.kv_stride_h;
  a.kv_st = p.kv_stride_t;
  a.H = p.n_heads;
  a.G = p.n_heads / p.n_kv_heads;
  a.n_var = (int32_t)L.n_var;
  a.c0 = p.chunk_start;
  a.L = p.chunk_len;
  a.n_ctx = L.n_ctx;
  a.period = d.period;
  a.n_qt = (p.chunk_len + kTileQ - 1) / kTileQ;
  a.n_blocks = (int64_t)p.n_heads * a.n_qt;
  a.scale_log2 = p.sm_scale * kLog2e;
  a.off_bits = reinterpret_cast<const uint32_t*>(cur);
  cur += L.off_bits;
  a.col_bits = reinterpret_cast<const uint32_t*>(cur);
  cur += L.col_bits;
  a.runs = reinterpret_cast<const int32_t*>(cur);
  cur += L.runs;
  a.run_cnt = reinterpret_cast<const int32_t*>(cur);
  a.n_words = L.n_words;
  a.max_runs = dense ? 1 : pat.max_slash;
  a.vert_idx = pat.vert_idx;
  a.vert_cnt = pat.vert_cnt;
  a.max_vert = pat.max_vert;
  a.dense = dense ? 1 : 0;
  a.head_mask = head_mask;
  a.out = out;
  a.out_dtype = out_dtype;
  a.o_sh = o_sh;
  a.o_st = o_st;
  a.lse = lse;
  a.stats = reinterpret_cast<unsigned long long*>(stats);
  const int64_t grid = (a.n_blocks + 7) / 8 * 8;
  if (p.head_dim == 128) hipLaunchKernelGGL(attn_kernel<128>, dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL(attn_kernel<64>, dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return check_launch("sparse attention");
}

}  // namespace lcsr
