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
//  * a workgroup = one query head x 128 query rows (4 waves x 32 rows), two
//    workgroups per CU;
//  * slash offsets are merged into runs (consecutive offsets at most 128
//    apart); run [oa, ob] covers the key span [r0 - ob, r0 + 127 - oa] of the
//    tile, cut at DCA chunk edges into 64-key tiles;
//  * verticals outside every span of the tile are listed per (head, tile)
//    by a pre-kernel and gathered 64 at a time;
//  * K and V tiles go straight from HBM to LDS (global_load_lds_dwordx4,
//    16-byte chunks XOR-swizzled by row), double buffered: the next tile is
//    in flight while the current one is multiplied;
//  * per (wave, key tile) the pair mask is: key <= row and (offset bit or
//    column bit); tiles a wave does not touch are skipped, tiles it fully
//    covers run without a mask;
//  * S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_bf16 (V^T read
//    with the LDS transpose load ds_read_b64_tr_b16): each lane owns one
//    query row, so the softmax max / sum and the O rescale are in-lane; the
//    row max is only raised when it grows by more than 2^8 (the exponent
//    bound keeps p <= 256), and the row sum adds the bf16 weights the PV
//    product uses (v_dot2_f32_bf16);
//  * the DCA relation of a (wave, tile) pair picks one of three pre-rotated
//    query variants (intra / successive / inter).
#include <cmath>
#include <type_traits>

#include "lcsr_internal.h"

namespace lcsr {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kRescaleSlack = 8.0f;  // log2 units

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;

struct AttnArgs {
  const uint16_t* __restrict__ q_rot;   // [n_var][H][L][D]
  const uint16_t* __restrict__ k;       // K cache (rotated at P_k)
  const uint16_t* __restrict__ v;       // V cache
  int64_t kv_sh, kv_st;
  int32_t H, G, n_var;
  int64_t c0, L, n_ctx;
  int64_t period;          // S (0: DCA off)
  int64_t n_qt;            // query tiles
  int64_t n_blocks;        // H * n_qt
  float scale_log2;
  const uint32_t* __restrict__ off_bits;  // [H][n_words]
  const uint32_t* __restrict__ col_bits;  // [H][n_words]
  int64_t n_words;
  const int32_t* __restrict__ runs;       // [H][max_runs][2]
  const int32_t* __restrict__ run_cnt;    // [H]
  int32_t max_runs;
  const int32_t* __restrict__ vl;         // [H][n_qt][max_vert] leftover verticals
  const int32_t* __restrict__ vl_cnt;     // [H][n_qt]
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

__device__ __forceinline__ uint64_t low_bits(int64_t n) {  // n clamped to [0, 64]
  return n >= 64 ? ~0ull : (n <= 0 ? 0ull : ((1ull << n) - 1));
}

// any / all bits set in [a, b] (a > b: empty -> any false, all true)
__device__ __forceinline__ bool any_bits(const uint32_t* bm, int64_t a, int64_t b) {
  for (int64_t p = a; p <= b; p += 64) {
    if (get64(bm, p) & low_bits(b - p + 1)) return true;
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

// 128 bitmap bits [base, base + 128) loaded with uniform (scalar) loads.
struct Win {
  uint32_t w0, w1, w2, w3;
  int32_t base;
};

__device__ __forceinline__ Win load_win(const uint32_t* bm, int32_t pos) {
  // floor(pos / 32); the bitmaps carry kBitPad zero words before bit 0
  const int32_t wi = pos >= 0 ? pos >> 5 : -((31 - pos) >> 5);
  // constant address space: uniform loads become scalar loads, which do not
  // wait behind the tile loads in flight
  typedef const __attribute__((address_space(4))) uint32_t cu32;
  cu32* p = (cu32*)(bm + wi);
  return Win{p[0], p[1], p[2], p[3], wi * 32};
}

// 64 bits starting at bit `rel` of the window (rel in [0, 127]; bits past
// 128 read as 0).
__device__ __forceinline__ uint64_t bits_at(const Win& W, int rel) {
  const uint64_t lo = ((uint64_t)W.w1 << 32) | W.w0;
  const uint64_t hi = ((uint64_t)W.w3 << 32) | W.w2;
  if (rel >= 64) return hi >> (rel - 64);
  if (rel == 0) return lo;
  return (lo >> rel) | (hi << (64 - rel));
}

// Any / all bits of [a, b] inside the window (uniform; a - base and b - base
// in [0, 127]).
__device__ __forceinline__ bool win_any(const Win& W, int32_t a, int32_t b) {
  if (a > b) return false;
  const int32_t n = b - a + 1, r = a - W.base;
  if (bits_at(W, r) & low_bits(n)) return true;
  return n > 64 && (bits_at(W, r + 64) & low_bits(n - 64));
}
__device__ __forceinline__ bool win_all(const Win& W, int32_t a, int32_t b) {
  if (a > b) return true;
  const int32_t n = b - a + 1, r = a - W.base;
  const uint64_t m0 = low_bits(n), m1 = low_bits(n - 64);
  if ((bits_at(W, r) & m0) != m0) return false;
  return n <= 64 || (bits_at(W, r + 64) & m1) == m1;
}

__device__ __forceinline__ uint64_t bitrev64(uint64_t x) {
  const uint32_t lo = __builtin_bitreverse32((uint32_t)x);
  const uint32_t hi = __builtin_bitreverse32((uint32_t)(x >> 32));
  return ((uint64_t)lo << 32) | hi;
}

// One 64-key tile: keys [ks, ks + n) (gather == 0) or vl[ks .. ks + n).
// W / C: the offset window of this wave and the column window of the tile,
// loaded one iteration ahead so that they are ready with the tile itself.
struct Tile {
  int32_t ks;      // first key (span) / slot of the first key (gather)
  int32_t n;
  int32_t gather;
  int32_t kchunk;  // DCA chunk of the tile's keys
  int32_t kmin, kmax;
  Win W, C;
};

// Scalar walk over the tile list of one workgroup: the spans of the slash
// runs, then the leftover verticals.  Every thread computes the same thing.
struct TileWalk {
  int32_t phase;   // 0 spans, 1 verticals, 2 done
  int32_t ru;      // next run
  int32_t ks, hi;  // current span position / end (inclusive)
  int32_t s0;      // next vertical slot
};

__device__ __forceinline__ bool next_tile(const AttnArgs& a, int32_t r0, int32_t rlast,
                                          int32_t period, const int32_t* runs, int n_runs,
                                          const int32_t* vl, int32_t vcnt, TileWalk& w,
                                          Tile& t) {
  while (w.phase == 0) {
    if (w.ks <= w.hi) {
      int32_t ke = w.ks + kTileK < w.hi + 1 ? w.ks + kTileK : w.hi + 1;
      const int32_t kc = period ? w.ks / period : 0;
      if (period && ke > (kc + 1) * period) ke = (kc + 1) * period;
      t.ks = w.ks;
      t.n = ke - w.ks;
      t.gather = 0;
      t.kchunk = kc;
      t.kmin = w.ks;
      t.kmax = ke - 1;
      w.ks = ke;
      return true;
    }
    if (w.ru >= n_runs) {
      w.phase = 1;
      break;
    }
    const int32_t oa = a.dense ? 0 : runs[2 * w.ru];
    const int32_t ob = a.dense ? (int32_t)a.n_ctx - 1 : runs[2 * w.ru + 1];
    ++w.ru;
    if (oa > r0 + kTileQ - 1) {
      w.phase = 1;
      break;
    }
    w.ks = r0 - ob > 0 ? r0 - ob : 0;
    w.hi = (r0 + kTileQ - 1 - oa < rlast) ? r0 + kTileQ - 1 - oa : rlast;
  }
  if (w.phase == 1) {
    if (a.dense || w.s0 >= vcnt) {
      w.phase = 2;
      return false;
    }
    const int32_t s0 = w.s0;
    int32_t s1 = s0 + kTileK < vcnt ? s0 + kTileK : vcnt;
    const int32_t k0 = vl[s0];
    const int32_t kc = period ? k0 / period : 0;
    if (period && vl[s1 - 1] / period != kc) {
      // first slot of the next DCA chunk (keys ascending)
      int lo = s0 + 1, hi = s1 - 1;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (vl[mid] / period != kc) hi = mid;
        else lo = mid + 1;
      }
      s1 = lo;
    }
    t.ks = s0;
    t.n = s1 - s0;
    t.gather = 1;
    t.kchunk = kc;
    t.kmin = k0;
    t.kmax = vl[s1 - 1];
    w.s0 = s1;
    return true;
  }
  return false;
}

// LDS layout of one buffer: K rows then V rows, 64 rows of D bf16 each.  The
// 16-byte chunk c of K row r sits at slot c ^ (r & 15) and of V row r at slot
// c ^ 4 (r & 3) (both mod the chunks per row): the K fragment reads (one
// chunk of 32 consecutive rows) and the V transpose reads (two chunks of four
// consecutive rows per 16 lanes) then hit distinct banks.
template <int D>
struct Buf {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = D / 8;
  static constexpr int kKBytes = kTileK * kRowBytes;
  static constexpr int kBytes = 2 * kKBytes;
};

template <int D>
__device__ __forceinline__ int swz_k(int chunk, int row) {
  return (chunk ^ (row & 15)) & (Buf<D>::kChunks - 1);
}
template <int D>
__device__ __forceinline__ int swz_v(int chunk, int row) {
  return (chunk ^ ((row & 3) << 2)) & (Buf<D>::kChunks - 1);
}

// Per-lane constants of the tile pipeline, computed once per workgroup.
template <int D>
struct LaneConst {
  static constexpr int kCh = Buf<D>::kChunks;
  static constexpr int kRowsPerInstr = 64 / kCh;   // rows one wave fills per load
  static constexpr int kInstr = kTileK / (kWaves * kRowsPerInstr);
  int32_t row[kInstr];      // tile row this lane loads in load i
  int32_t k_chunk[kInstr];  // global chunk it loads for K / V
  int32_t v_chunk[kInstr];
  int32_t k_rd[D / 16];     // LDS byte offset of the K fragment of step s (kb = 0)
  int32_t v_rd[D / 32];     // LDS byte offset of the V^T fragment of block db (s = 0)
};

template <int D>
__device__ __forceinline__ void lane_consts(LaneConst<D>& c, int w, int lane) {
  constexpr int kCh = Buf<D>::kChunks, RB = Buf<D>::kRowBytes;
#pragma unroll
  for (int i = 0; i < LaneConst<D>::kInstr; ++i) {
    const int row = (i * kWaves + w) * LaneConst<D>::kRowsPerInstr + lane / kCh;
    c.row[i] = row;
    c.k_chunk[i] = swz_k<D>(lane % kCh, row);  // the XOR swizzles are involutions
    c.v_chunk[i] = swz_v<D>(lane % kCh, row);
  }
  const int half = lane >> 5;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const int row = lane & 31;
    c.k_rd[s] = row * RB + swz_k<D>(2 * s + half, row) * 16;
  }
  // V^T transpose reads: lane j of each 16-lane group addresses key
  // 4 half + j / 4 (+16 s, +8 for the second load) at d = d0 + 4 (j % 4)
  const int j = lane & 15;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const int key = 4 * half + (j >> 2);
    const int d = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
    c.v_rd[db] = Buf<D>::kKBytes + key * RB + swz_v<D>(d >> 3, key) * 16 + 8 * ((d >> 2) & 1);
  }
}

// Toggle the LDS read offsets between the two buffers.
template <int D>
__device__ __forceinline__ void flip_buffers(LaneConst<D>& c) {
#pragma unroll
  for (int s = 0; s < D / 16; ++s) c.k_rd[s] ^= Buf<D>::kBytes;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) c.v_rd[db] ^= Buf<D>::kBytes;
}

// Issue the direct-to-LDS loads of one tile into the buffer at byte `buf`.
// Padding rows (past t.n) repeat the tile's last key, so every value is finite.
template <int D>
__device__ __forceinline__ void issue_tile(const AttnArgs& a, int g, const int32_t* vl,
                                           const Tile& t, int buf, const LaneConst<D>& c,
                                           int32_t* keys_lds, int w, int lane) {
  constexpr int kCh = Buf<D>::kChunks, RB = Buf<D>::kRowBytes;
  const uint32_t kvst_b = (uint32_t)(a.kv_st * 2);
  const char* kbase = reinterpret_cast<const char*>(a.k + (int64_t)g * a.kv_sh);
  const char* vbase = reinterpret_cast<const char*>(a.v + (int64_t)g * a.kv_sh);
  if (!t.gather) {
    kbase += (int64_t)t.ks * kvst_b;
    vbase += (int64_t)t.ks * kvst_b;
  }
#pragma unroll
  for (int i = 0; i < LaneConst<D>::kInstr; ++i) {
    const int rr = c.row[i] < t.n ? c.row[i] : t.n - 1;
    int64_t roff;
    if (t.gather) roff = (int64_t)vl[t.ks + rr] * kvst_b;
    else roff = (uint32_t)rr * kvst_b;
    const int lds = buf + (i * kWaves + w) * LaneConst<D>::kRowsPerInstr * RB;
    __builtin_amdgcn_global_load_lds(kbase + roff + c.k_chunk[i] * 16, (lds_void*)(lds), 16,
                                     0, 0);
    __builtin_amdgcn_global_load_lds(vbase + roff + c.v_chunk[i] * 16,
                                     (lds_void*)(lds + Buf<D>::kKBytes), 16, 0, 0);
    if (t.gather && (lane % kCh) == 0)
      keys_lds[c.row[i]] = c.row[i] < t.n ? vl[t.ks + c.row[i]] : INT32_MAX;
  }
}

template <int D>
struct WaveState {
  bf16x8 q[D / 16];
  f32x16 o[D / 32];
  float m, l;
  int var;
  uint32_t sel;   // critical-set pairs of this lane's row
};

template <int D>
__device__ __forceinline__ void load_q(const AttnArgs& a, int h, int32_t i0, int var,
                                       WaveState<D>& st) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)i0 - a.c0 + (lane & 31);
  const uint16_t* base = a.q_rot + (((int64_t)var * a.H + h) * a.L + t) * D + 8 * (lane >> 5);
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    if (t < a.L) st.q[s] = *reinterpret_cast<const bf16x8*>(base + s * 16);
    else st.q[s] = (bf16x8){};
  }
  st.var = var;
}

// One (wave, key tile) step on the current buffer (offsets in `c`).  With
// `masked`, mword is the 64-bit key mask of this lane's row.
template <int D>
__device__ __forceinline__ void wave_tile(const AttnArgs& a, const char* smem,
                                          const LaneConst<D>& c, WaveState<D>& st,
                                          bool masked, uint64_t mword, int half) {
  constexpr int RB = Buf<D>::kRowBytes;
  constexpr int KS = D / 16;  // k-steps of the QK product
  constexpr int DB = D / 32;  // 32-row blocks of O^T
  // every K fragment of the tile is requested before the first product, so
  // the LDS latency is paid once per tile, not once per MFMA
  bf16x8 kf[2][KS];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int s = 0; s < KS; ++s)
      kf[kb][s] = *reinterpret_cast<const bf16x8*>(smem + c.k_rd[s] + kb * 32 * RB);
  __builtin_amdgcn_sched_barrier(0);  // keep every K read ahead of the products
  f32x16 acc[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) acc[kb] = (f32x16){};
#pragma unroll
  for (int s = 0; s < KS; ++s)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      acc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kb][s], st.q[s], acc[kb], 0, 0, 0);
  // V^T fragments of the first two 16-key steps, in flight during the softmax;
  // each lane receives V[16 s + 4 half + r][d0 + j] (r = 0..3 for the first
  // load, +8 for the second), the k-order of its P fragment
  auto load_v = [&](int s, int db) {
    const char* p = smem + c.v_rd[db] + 16 * s * RB;
    const v4i16 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
    const v4i16 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + 8 * RB));
    const v4i16 vv[2] = {va, vb};
    bf16x8 vf;
    __builtin_memcpy(&vf, vv, 16);
    return vf;
  };
  bf16x8 vf[2][DB];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int db = 0; db < DB; ++db) vf[s][db] = load_v(s, db);
  __builtin_amdgcn_sched_barrier(0);  // V reads in flight before the softmax
  // key k of the tile sits in register r of block kb: k = 32 kb + 8 (r / 4)
  // + 4 half + r % 4
  if (__builtin_expect(masked, 0)) {
    const uint64_t mh = mword >> (4 * half);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int bit = 32 * kb + 8 * (r >> 2) + (r & 3);
        if (!((mh >> bit) & 1ull)) acc[kb][r] = -INFINITY;
      }
  }
  // row max of the raw scores (the scale is positive)
  float mx = fmaxf(acc[0][0], acc[1][0]);
#pragma unroll
  for (int r = 1; r < 16; ++r) mx = fmaxf(fmaxf(mx, acc[0][r]), acc[1][r]);
  mx = fmaxf(mx, __shfl_xor(mx, 32)) * a.scale_log2;
  if (__builtin_expect(__ballot(mx > st.m + kRescaleSlack) != 0ull, 0)) {
    const float m_new = fmaxf(st.m, mx);
    const float alpha = (st.m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(st.m - m_new);
    st.l *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o[db][r] *= alpha;
    st.m = m_new;
  }
  const float msub = (st.m == -INFINITY) ? 0.f : st.m;
  bf16x8 pf[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      pf[s][e] = (__bf16)__builtin_amdgcn_exp2f(
          fmaf(acc[s >> 1][8 * (s & 1) + e], a.scale_log2, -msub));
  // row sum of the bf16 weights the PV product uses
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  float psum = 0.f;
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const bf16x2 pr = {pf[s][e], pf[s][e + 1]};
      psum = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, psum, false);
    }
  st.l += psum;
  // O^T += V^T P^T: steps 0, 1 from the fragments in flight, 2, 3 after
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int db = 0; db < DB; ++db)
      st.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[s][db], pf[s], st.o[db], 0, 0, 0);
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int db = 0; db < DB; ++db) vf[s][db] = load_v(s + 2, db);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int db = 0; db < DB; ++db)
      st.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[s][db], pf[s + 2], st.o[db], 0, 0,
                                                         0);
}

template <int D>
constexpr size_t attn_smem_bytes() {
  return 2 * Buf<D>::kBytes + 2 * kTileK * sizeof(int32_t) + 2 * sizeof(unsigned long long);
}

// Per (wave, tile) decision: false = skip; masked + mword otherwise.
__device__ __forceinline__ bool tile_mask(const Tile& t, int32_t i0, int32_t my_row, int lane,
                                          const int32_t* keys_lds, bool& masked,
                                          uint64_t& mword) {
  masked = false;
  mword = 0;
  if (!t.gather) {
    const int32_t wlo = i0 - t.ks - 63;
    const uint64_t wcol = bits_at(t.C, t.ks - t.C.base) & low_bits(t.n);
    const int32_t olo = i0 - t.kmax, ohi = i0 + 31 - t.ks;
    if (!wcol && !win_any(t.W, olo > 0 ? olo : 0, ohi)) return false;
    if (!(t.n == kTileK && t.kmax <= i0 && win_all(t.W, olo, ohi))) {
      masked = true;
      // this lane's 64 offsets start at wlo + lane % 32
      const uint64_t woff = bits_at(t.W, wlo - t.W.base + (lane & 31));
      mword = (bitrev64(woff) | wcol) & low_bits(my_row - t.ks + 1) & low_bits(t.n);
    }
  } else if (!(t.n == kTileK && t.kmax <= i0)) {
    masked = true;
    int lo = 0, hi = t.n;  // keys <= my_row (keys ascending)
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (keys_lds[mid] <= my_row) lo = mid + 1;
      else hi = mid;
    }
    mword = low_bits(lo);
  }
  return true;
}

template <int D>
__global__ void __launch_bounds__(kThreads, 2) attn_kernel(AttnArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  int32_t* keys_lds = reinterpret_cast<int32_t*>(smem + 2 * Buf<D>::kBytes);  // [2][64]
  unsigned long long* stat_lds = reinterpret_cast<unsigned long long*>(keys_lds + 2 * kTileK);
  // XCD-aware order: consecutive logical blocks (same KV group and query
  // tile, then the next tile) land on one XCD, sharing its L2.
  const int32_t nb = (int32_t)a.n_blocks;
  const int32_t per_xcd = (nb + 7) / 8;
  const int32_t logical = (int32_t)(blockIdx.x % 8) * per_xcd + (int32_t)(blockIdx.x / 8);
  if (logical >= nb) return;
  const int32_t gq = logical / a.G;
  const int hh = logical % a.G;
  const int g = gq / (int32_t)a.n_qt;
  const int32_t qt = gq % (int32_t)a.n_qt;
  const int h = g * a.G + hh;
  if (!((a.head_mask >> h) & 1)) return;

  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, half = lane >> 5;
  const int32_t c0 = (int32_t)a.c0, c1 = (int32_t)a.n_ctx, period = (int32_t)a.period;
  const int32_t r0 = c0 + qt * kTileQ;
  const int32_t rlast = (r0 + kTileQ - 1 < c1 - 1) ? r0 + kTileQ - 1 : c1 - 1;
  const int32_t i0 = r0 + 32 * w;
  const bool wave_live = i0 <= rlast;
  const int32_t my_row = i0 + (lane & 31);
  const int32_t qchunk = period ? i0 / period : 0;
  const uint32_t* offb = a.off_bits + (int64_t)h * a.n_words + kBitPad;
  const uint32_t* colb = a.col_bits + (int64_t)h * a.n_words + kBitPad;
  const int32_t* runs = a.runs + (int64_t)h * a.max_runs * 2;
  const int n_runs = a.dense ? 1 : min(a.run_cnt[h], a.max_runs);
  const int32_t* vl = a.vl + ((int64_t)h * a.n_qt + qt) * a.max_vert;
  const int32_t vcnt = a.dense ? 0 : min(a.vl_cnt[(int64_t)h * a.n_qt + qt], a.max_vert);

  LaneConst<D> lc;
  lane_consts<D>(lc, w, lane);
  WaveState<D> st;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) st.o[db] = (f32x16){};
  st.m = -INFINITY;
  st.l = 0.f;
  st.var = -1;
  st.sel = 0;
  uint32_t exec_tiles = 0;
  if (threadIdx.x < 2) stat_lds[threadIdx.x] = 0;

  // offset / column windows of a span tile for this wave (offsets the wave
  // can meet: [i0 - kmax, i0 + 31 - ks]; lane windows [my_row - ks - 63,
  // my_row - ks] all sit in the 128 bits from i0 - ks - 63)
  auto load_windows = [&](Tile& t) {
    if (!t.gather && wave_live) {
      t.W = load_win(offb, i0 - t.ks - 63);
      t.C = load_win(colb, t.ks);
    }
  };
  TileWalk walk{0, 0, 0, -1, 0};
  Tile cur, nxt;
  bool have = next_tile(a, r0, rlast, period, runs, n_runs, vl, vcnt, walk, cur);
  if (have) {
    load_windows(cur);
    issue_tile<D>(a, g, vl, cur, 0, lc, keys_lds, w, lane);
  }
  int b = 0;
  while (have) {
    const bool have_next = next_tile(a, r0, rlast, period, runs, n_runs, vl, vcnt, walk, nxt);
    if (have_next) load_windows(nxt);
    __syncthreads();  // tile `cur` landed in buffer b; buffer b ^ 1 is free
    if (have_next)
      issue_tile<D>(a, g, vl, nxt, (b ^ 1) * Buf<D>::kBytes, lc, keys_lds + (b ^ 1) * kTileK,
                    w, lane);
    bool masked;
    uint64_t mword;
    if (wave_live && cur.kmin <= i0 + 31 &&
        tile_mask(cur, i0, my_row, lane, keys_lds + b * kTileK, masked, mword)) {
      const int32_t rel = qchunk - cur.kchunk;
      const int var = a.n_var == 1 ? 0 : (rel >= 2 ? 2 : rel);
      if (var != st.var) load_q<D>(a, h, i0, var, st);
      wave_tile<D>(a, smem, lc, st, masked, mword, half);
      ++exec_tiles;
      if (half == 0 && my_row <= rlast) st.sel += masked ? (uint32_t)__popcll(mword) : cur.n;
    }
    flip_buffers<D>(lc);
    cur = nxt;
    have = have_next;
    b ^= 1;
  }

  // ---------------- epilogue
  if (wave_live) {
    const float l_tot = st.l + __shfl_xor(st.l, 32);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (my_row <= rlast) {
      const int64_t t = my_row - c0;
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
    __syncthreads();
    unsigned long long se = st.sel;
    for (int off = 32; off > 0; off >>= 1) se += __shfl_xor(se, off);
    if (lane == 0) {
      atomicAdd(&stat_lds[0], (unsigned long long)exec_tiles * 32ull * kTileK);
      atomicAdd(&stat_lds[1], se);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      atomicAdd(&a.stats[0], stat_lds[0]);
      atomicAdd(&a.stats[1], stat_lds[1]);
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
  int32_t* vl;
  int32_t* vl_cnt;
  int64_t c0, n_qt;
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
  uint32_t* ob_raw = a.off_bits + (int64_t)h * a.n_words;
  uint32_t* cb_raw = a.col_bits + (int64_t)h * a.n_words;
  uint32_t* ob = ob_raw + kBitPad;
  uint32_t* cb = cb_raw + kBitPad;
  const int tid = threadIdx.x;
  for (int64_t wi = tid; wi < a.n_words; wi += kAuxThreads) {
    uint32_t v = 0;
    const int64_t b0 = (wi - kBitPad) * 32;
    if (a.dense && b0 >= 0) {
      if (b0 + 32 <= a.n_ctx) v = 0xFFFFFFFFu;
      else if (b0 < a.n_ctx) v = (1u << (a.n_ctx - b0)) - 1u;
    }
    ob_raw[wi] = v;
    cb_raw[wi] = 0u;
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
      if (o >= 0 && o < a.n_ctx) {
        int32_t nx = -1;
        if (i + 1 < ns) {
          const int32_t q = so[i + 1];
          nx = (q >= 0 && q < a.n_ctx) ? q : -1;
        }
        if (nx < 0 || nx - o > kTileQ) {
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

constexpr int kVlThreads = 256;

// Per (query tile, head): the verticals v <= the tile's last row that no
// slash span of the tile covers (no selected offset in [r0 - v, r0 + 127 -
// v]), ascending.
__global__ void __launch_bounds__(kVlThreads) vert_list_kernel(AuxArgs a) {
  const int64_t qt = blockIdx.x;
  const int h = blockIdx.y;
  if (!((a.head_mask >> h) & 1) || a.dense) return;
  const int64_t r0 = a.c0 + qt * kTileQ;
  const int64_t rlast = r0 + kTileQ - 1 < a.n_ctx - 1 ? r0 + kTileQ - 1 : a.n_ctx - 1;
  const int nv = min(a.vert_cnt[h], a.max_vert);
  const int32_t* vo = a.vert_idx + (int64_t)h * a.max_vert;
  const uint32_t* ob = a.off_bits + (int64_t)h * a.n_words + kBitPad;
  int32_t* out = a.vl + ((int64_t)h * a.n_qt + qt) * a.max_vert;
  __shared__ int s_wave[kVlThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int total = 0;
  for (int b0 = 0; b0 < nv; b0 += kVlThreads) {
    if (vo[b0] > rlast) break;
    const int i = b0 + tid;
    bool keep = false;
    int32_t v = 0;
    if (i < nv) {
      v = vo[i];
      if (v >= 0 && v <= rlast) {
        const int64_t olo = r0 - v > 0 ? r0 - v : 0;
        keep = !any_bits(ob, olo, r0 + kTileQ - 1 - v);
      }
    }
    const uint64_t bal = __ballot(keep);
    __syncthreads();
    if (lane == 0) s_wave[w] = __popcll(bal);
    __syncthreads();
    int base = total, tot = 0;
    for (int x = 0; x < kVlThreads / 64; ++x) {
      if (x < w) base += s_wave[x];
      tot += s_wave[x];
    }
    if (keep) {
      const int below = (int)__builtin_amdgcn_mbcnt_hi(
          (uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
      out[base + below] = v;
    }
    total += tot;
  }
  if (tid == 0) a.vl_cnt[(int64_t)h * a.n_qt + qt] = total;
}

}  // namespace

int build_pattern_aux(const lcsr_problem_t& p, const lcsr_pattern_t& pat, uint64_t head_mask,
                      bool dense, const AttnLayout& L, char* ws, hipStream_t s) {
  AuxArgs a{};
  a.vert_idx = pat.vert_idx;
  a.vert_cnt = pat.vert_cnt;
  a.max_vert = pat.max_vert;
  a.slash_idx = pat.slash_idx;
  a.slash_cnt = pat.slash_cnt;
  a.max_slash = pat.max_slash;
  a.n_ctx = L.n_ctx;
  a.n_words = L.n_words;
  a.off_bits = reinterpret_cast<uint32_t*>(ws + L.o_off_bits);
  a.col_bits = reinterpret_cast<uint32_t*>(ws + L.o_col_bits);
  a.runs = reinterpret_cast<int32_t*>(ws + L.o_runs);
  a.run_cnt = reinterpret_cast<int32_t*>(ws + L.o_run_cnt);
  a.vl = reinterpret_cast<int32_t*>(ws + L.o_vl);
  a.vl_cnt = reinterpret_cast<int32_t*>(ws + L.o_vl_cnt);
  a.c0 = p.chunk_start;
  a.n_qt = L.n_qt;
  a.dense = dense ? 1 : 0;
  a.head_mask = head_mask;
  hipLaunchKernelGGL(aux_kernel, dim3(p.n_heads), dim3(kAuxThreads), 0, s, a);
  int rc = check_launch("pattern aux");
  if (rc || dense || !L.with_vl) return rc;
  hipLaunchKernelGGL(vert_list_kernel, dim3((unsigned)L.n_qt, p.n_heads), dim3(kVlThreads), 0,
                     s, a);
  return check_launch("vertical lists");
}

int run_attention(const lcsr_problem_t& p, const lcsr_pattern_t& pat, uint64_t head_mask,
                  void* out, int32_t out_dtype, int64_t o_sh, int64_t o_st, float* lse,
                  int64_t* stats, bool dense, char* ws, hipStream_t s) {
  const AttnLayout L = attn_layout(p, dense ? 1 : pat.max_vert, dense ? 1 : pat.max_slash, true);
  FreqTable ft;
  int rc = build_freq_table(&p.rope, p.head_dim, &ft);
  if (rc) return rc;
  const DcaParams d = make_dca(&p.dca);
  uint16_t* q_rot = reinterpret_cast<uint16_t*>(ws + L.o_q_rot);
  rc = launch_rotate_q_variants(p, ft, d, q_rot, (int)L.n_var, s);
  if (rc) return rc;
  rc = build_pattern_aux(p, pat, head_mask, dense, L, ws, s);
  if (rc) return rc;
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
  a.n_qt = L.n_qt;
  a.n_blocks = (int64_t)p.n_heads * a.n_qt;
  a.scale_log2 = p.sm_scale * kLog2e;
  a.off_bits = reinterpret_cast<const uint32_t*>(ws + L.o_off_bits);
  a.col_bits = reinterpret_cast<const uint32_t*>(ws + L.o_col_bits);
  a.n_words = L.n_words;
  a.runs = reinterpret_cast<const int32_t*>(ws + L.o_runs);
  a.run_cnt = reinterpret_cast<const int32_t*>(ws + L.o_run_cnt);
  a.max_runs = dense ? 1 : pat.max_slash;
  a.vl = reinterpret_cast<const int32_t*>(ws + L.o_vl);
  a.vl_cnt = reinterpret_cast<const int32_t*>(ws + L.o_vl_cnt);
  a.max_vert = dense ? 1 : pat.max_vert;
  a.dense = dense ? 1 : 0;
  a.head_mask = head_mask;
  a.out = out;
  a.out_dtype = out_dtype;
  a.o_sh = o_sh;
  a.o_st = o_st;
  a.lse = lse;
  a.stats = reinterpret_cast<unsigned long long*>(stats);
  const int64_t grid = (a.n_blocks + 7) / 8 * 8;
  // more than 64 KB of dynamic LDS per workgroup must be allowed explicitly
  static const hipError_t attr_rc[2] = {
      hipFuncSetAttribute(reinterpret_cast<const void*>(attn_kernel<64>),
                          hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)attn_smem_bytes<64>()),
      hipFuncSetAttribute(reinterpret_cast<const void*>(attn_kernel<128>),
                          hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)attn_smem_bytes<128>())};
  if (attr_rc[p.head_dim == 128 ? 1 : 0] != hipSuccess)
    return fail(LCSR_EHIP, "cannot raise the LDS limit of the attention kernel: %s",
                hipGetErrorString(attr_rc[p.head_dim == 128 ? 1 : 0]));
  if (p.head_dim == 128) {
    hipLaunchKernelGGL(attn_kernel<128>, dim3((unsigned)grid), dim3(kThreads),
                       attn_smem_bytes<128>(), s, a);
  } else {
    hipLaunchKernelGGL(attn_kernel<64>, dim3((unsigned)grid), dim3(kThreads),
                       attn_smem_bytes<64>(), s, a);
  }
  return check_launch("sparse attention");
}

}  // namespace lcsr
