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
//  * a workgroup = the query heads of one KV head (up to 7, one wave each)
//    x one block of 32 query rows; every wave multiplies the same K/V tiles,
//    so a tile is read from HBM once for all heads of the group;
//  * a planning kernel marks, per (KV group, row block), the 16-key granules
//    that any head's slash runs reach (run [oa, ob] reaches keys
//    [r0 - ob, rlast - oa]); the attention walks the marked granules in
//    64-key tiles (each from the first key a pair reaches, cut at DCA chunk
//    edges), and lists per head the verticals in unmarked granules, which
//    are gathered 64 at a time;
//  * K and V tiles go straight from HBM to LDS (global_load_lds_dwordx4,
//    16-byte chunks XOR-swizzled by row) through a ring of four stages: two
//    tiles are multiplied per step while the next two are loaded, one after
//    the other (dense calls: one tile per step, two loading);
//  * per (wave, key tile) the pair mask is: key <= row and (offset bit of the
//    wave's head or column bit in a marked granule); tiles a head does not
//    touch are skipped by its wave, tiles it fully covers run unmasked;
//  * S^T = K Q^T on v_mfma_f32_32x32x16_f16 (fp16 rotated keys and queries)
//    and O^T += V^T P^T on v_mfma_f32_32x32x16_bf16 (V^T read
//    with the LDS transpose load ds_read_b64_tr_b16): each lane owns one
//    query row, so the softmax max / sum and the O rescale are in-lane; a
//    tile's own max is taken only when a row has none yet or its weights sum
//    above 2^64 (weights are exact for any running max; it only guards the
//    range), and the row sum adds the bf16 weights the PV product uses
//    (v_dot2_f32_bf16);
//  * the DCA relation of the row block and a tile picks one of three
//    pre-rotated query variants (intra / successive / inter).
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "lcsr_internal.h"

namespace lcsr {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kStages = 4;             // LDS ring of K/V tiles
constexpr int kRunGap = kRowBlock;     // offsets at most this far apart share a run
constexpr int kGranPerChunk = 64 * 32; // granules covered by one 64-word bitmap chunk

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
  float scale_log2;
  const uint32_t* __restrict__ off_bits;  // [H][n_words]
  const uint32_t* __restrict__ col_bits;  // [H][n_words]
  int64_t n_words;
  const uint32_t* __restrict__ ubits;     // [n_wgg][n_rb][ubw] granule bitmaps
  const uint32_t* __restrict__ first;     // [n_wgg][n_rb][4 ubw] first pair key per granule, or null
  int64_t ubw;
  const int32_t* __restrict__ vl;         // [H][n_rb][max_vert] leftover verticals
  const int32_t* __restrict__ vl_cnt;     // [H][n_rb]
  int32_t max_vert;
  int32_t n_rb, n_sub, nw, n_wgg;
  int32_t dense;
  uint64_t head_mask;
  void* out;
  int32_t out_dtype;
  int64_t o_sh, o_st;
  float* lse;
  unsigned long long* stats;
};

__device__ __forceinline__ uint64_t low_bits(int64_t n) {  // n clamped to [0, 64]
  return n >= 64 ? ~0ull : (n <= 0 ? 0ull : ((1ull << n) - 1));
}

// Uniform read through the constant address space: it becomes a scalar load
// (the direct-to-LDS loads count as memory writes for the compiler, which
// would otherwise turn later uniform reads into vector loads that wait behind
// the tile loads in flight).
__device__ __forceinline__ int32_t ld_uniform(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)p;
}

// 128 bitmap bits [base, base + 128) loaded with uniform (scalar) loads.
struct Win {
  uint32_t w0, w1, w2, w3;
  int32_t base;
};

__device__ __forceinline__ Win load_win(const uint32_t* bm, int32_t pos) {
  // floor(pos / 32); the bitmaps carry kBitPad zero words before bit 0
  const int32_t wi = pos >= 0 ? pos >> 5 : -((31 - pos) >> 5);
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

// s_waitcnt vmcnt(N), other counters untouched: at most N of this wave's
// vector-memory operations are still in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
  constexpr int n = N > 63 ? 63 : N;
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// One 64-key tile.  Span tiles (wave < 0): keys [ks, ks + n), marked bits of
// granules ks/16 .. ks/16 + 4 in `gran` (ks need not be a granule start).
// Gathered tiles: wave `wave` only (its head's leftover list), keys
// list[ks .. ks + n).
struct Tile {
  int32_t ks;      // first key (span) / first slot (gather)
  int32_t n;
  int32_t wave;    // -1: span tile; else the wave whose head owns the list
  int32_t kchunk;  // DCA chunk of the tile's keys
  int32_t kmax;    // last key
  int32_t gran;    // span tile: marked bits of granules ks/16 .. ks/16 + 4
};

// The walk over one workgroup's tiles, identical in every wave: marked
// granules in ascending key order, then each head's leftover verticals.
struct Walk {
  int32_t phase;   // 0 spans, 1 verticals, 2 done
  int32_t pos;     // first key not covered yet
  int32_t chunk;   // bitmap chunk held in the lanes' `cw` (-1: none)
  uint64_t nz;     // non-zero words of that chunk
  int32_t kc;      // DCA chunk of pos
  int32_t edge;    // first key of the next DCA chunk
  int32_t gw;      // verticals: wave (head) being listed
  int32_t s0;      // next slot of that list
  int32_t vcnt;    // its length
};

struct WalkConst {
  int32_t rlast, period, glast, nwords, n_here, rb, h_first;
  const uint32_t* ub;     // LDS bitmap
  const uint32_t* first;  // first pair key of each granule (4 bits), or null
};

__device__ __forceinline__ bool next_tile(const AttnArgs& a, const WalkConst& c, Walk& w,
                                          uint32_t& cw, uint4& nf, Tile& t) {
  const int lane = threadIdx.x & 63;
  if (w.phase == 0) {
    // Next tile: 64 keys from the first marked granule that holds keys >=
    // pos (the granule holding pos itself when a tile ended inside it),
    // starting at pos or at the granule's first key that a pair of the row
    // block reaches, whichever is later; cut at a DCA chunk edge and after
    // rlast.  No key a pair reaches is skipped: the granules in between are
    // unmarked, and the granule's keys before its first reached key have no
    // pair.  Starting there rather than at the granule's first key leaves
    // fewer key halves with pairs (an isolated diagonal of a 32-row block
    // then often fits one half).
    const int32_t p = w.pos;
    int32_t g = p / kGranule;
    {
      bool found = false;
      while (g <= c.glast) {
        const int32_t ch = g / kGranPerChunk;
        if (ch != w.chunk) {
          const int32_t wi = ch * 64 + lane;
          cw = wi < c.nwords ? c.ub[wi] : 0u;
          w.nz = __ballot(cw != 0u);
          w.chunk = ch;
          // the chunk's first-key nibbles, 32 granules per lane: a vector
          // load, waited for at once (with any tile loads in flight, once per
          // 2,048 granules), so that no wait for it is left at its uses
          if (c.first) {
            nf = wi < c.nwords ? reinterpret_cast<const uint4*>(c.first)[wi]
                               : make_uint4(0u, 0u, 0u, 0u);
            wait_vm<0>();
          }
        }
        const int32_t wl = (g >> 5) & 63;
        const uint32_t word =
            (uint32_t)__builtin_amdgcn_readlane(cw, wl) & (0xFFFFFFFFu << (g & 31));
        if (word) {
          g = (g & ~31) + __builtin_ctz(word);
          found = true;
          break;
        }
        const uint64_t rest = wl == 63 ? 0ull : (w.nz & (~0ull << (wl + 1)));
        g = rest ? ch * kGranPerChunk + 32 * __builtin_ctzll(rest) : (ch + 1) * kGranPerChunk;
      }
      int32_t ks = g * kGranule;
      if (found && c.first) {
        const int32_t wl = (g >> 5) & 63, sel = (g >> 3) & 3;
        const uint32_t fw = sel == 0 ? nf.x : (sel == 1 ? nf.y : (sel == 2 ? nf.z : nf.w));
        ks += (int32_t)(((uint32_t)__builtin_amdgcn_readlane(fw, wl) >> (4 * (g & 7))) & 15u);
      }
      if (ks < p) ks = p;
      if (!found || g > c.glast || ks > c.rlast) goto spans_done;
      int32_t ke = ks + kTileK < c.rlast + 1 ? ks + kTileK : c.rlast + 1;
      if (c.period) {
        while (ks >= w.edge) {
          ++w.kc;
          w.edge += c.period;
        }
        if (ke > w.edge) ke = w.edge;
      }
      // marked bits of the five granules from g (they may straddle a word)
      const int32_t wl = (g >> 5) & 63, sh = g & 31;
      // (readlane returns int: shift the word as unsigned)
      uint32_t gb = (uint32_t)__builtin_amdgcn_readlane(cw, wl) >> sh;
      if (sh > 27) {
        const int32_t nwi = (g >> 5) + 1;
        const uint32_t nx =
            wl < 63 ? (uint32_t)__builtin_amdgcn_readlane(cw, wl + 1)
                    : (nwi < c.nwords ? (uint32_t)__builtin_amdgcn_readfirstlane(c.ub[nwi]) : 0u);
        gb |= nx << (32 - sh);
      }
      t.ks = ks;
      t.n = ke - ks;
      t.wave = -1;
      t.kchunk = w.kc;
      t.kmax = ke - 1;
      t.gran = (int32_t)(gb & 31u);
      w.pos = ke;
      return true;
    }
  spans_done:
    w.phase = 1;
    w.gw = -1;
    w.s0 = 0;
    w.vcnt = 0;
  }
  if (w.phase == 1) {
    while (w.s0 >= w.vcnt) {
      ++w.gw;
      if (w.gw >= c.n_here) {
        w.phase = 2;
        return false;
      }
      const int h = c.h_first + w.gw;
      w.s0 = 0;
      w.vcnt = (a.dense || !((a.head_mask >> h) & 1))
                   ? 0
                   : min(ld_uniform(a.vl_cnt + (int64_t)h * a.n_rb + c.rb), a.max_vert);
    }
    const int h = c.h_first + w.gw;
    const int32_t* vl = a.vl + ((int64_t)h * a.n_rb + c.rb) * a.max_vert;
    const int32_t s0 = w.s0;
    int32_t s1 = s0 + kTileK < w.vcnt ? s0 + kTileK : w.vcnt;
    const int32_t k0 = ld_uniform(vl + s0);
    const int32_t kc = c.period ? k0 / c.period : 0;
    if (c.period && ld_uniform(vl + s1 - 1) / c.period != kc) {
      // first slot of the next DCA chunk (keys ascending)
      int lo = s0 + 1, hi = s1 - 1;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (ld_uniform(vl + mid) / c.period != kc) hi = mid;
        else lo = mid + 1;
      }
      s1 = lo;
    }
    t.ks = s0;
    t.n = s1 - s0;
    t.wave = w.gw;
    t.kchunk = kc;
    t.kmax = ld_uniform(vl + s1 - 1);
    t.gran = 0;
    w.s0 = s1;
    return true;
  }
  return false;
}

// LDS layout of one stage: K rows, V rows (64 rows of D bf16 each), then the
// 64 keys of a gathered tile.  The 16-byte chunk c of K row r sits at slot
// c ^ (r & 15) and of V row r at slot c ^ 4 (r & 3) (both mod the chunks per
// row): the K fragment reads (one chunk of 32 consecutive rows) and the V
// transpose reads (two chunks of four consecutive rows per 16 lanes) then hit
// distinct banks.
template <int D>
struct Buf {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = D / 8;
  static constexpr int kKBytes = kTileK * kRowBytes;
  static constexpr int kKeyOff = 2 * kKBytes;
  static constexpr int kBytes = 2 * kKBytes + kTileK * 4;
  static constexpr int kRowsPerInstr = 1024 / kRowBytes;  // rows one 64-lane load fills
  static constexpr int kInstrPerMat = kTileK / kRowsPerInstr;
  static constexpr int kInstr = 2 * kInstrPerMat;         // loads per tile (K and V)
};

template <int D>
__device__ __forceinline__ int swz_k(int chunk, int row) {
  return (chunk ^ (row & 15)) & (Buf<D>::kChunks - 1);
}
template <int D>
__device__ __forceinline__ int swz_v(int chunk, int row) {
  return (chunk ^ ((row & 3) << 2)) & (Buf<D>::kChunks - 1);
}

// Per-lane LDS read offsets, computed once per workgroup.
template <int D>
struct LaneConst {
  int32_t k_rd[D / 16];  // K fragment of step s (kb = 0)
  int32_t v_rd[D / 32];  // V^T fragment of block db (s = 0)
};

template <int D>
__device__ __forceinline__ void lane_consts(LaneConst<D>& c, int lane) {
  constexpr int RB = Buf<D>::kRowBytes;
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

// Direct-to-LDS loads written as inline assembly: the compiler then does not
// see LDS writes in flight, so it adds no waits before reading the other
// stages (the kernel waits for its own loads explicitly).  They have no
// register results.  M0 holds the LDS byte address of lane 0's 16 bytes.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}
__device__ __forceinline__ void dma16_s(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void dma16_v(const void* addr, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(addr), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void dma4_v(const void* addr, uint32_t lds) {
  asm volatile("global_load_lds_dword %0, off" ::"v"(addr), "{m0}"(lds) : "memory");
}

// Every direct-to-LDS load of one tile, issued by the walker wave into the
// stage at LDS address `dst`: load i fills rows (i mod M) * R .. + R - 1 of K
// (i < M) or V (M = loads per matrix, R rows per load); padding rows past
// t.n repeat the last key.  For gathered tiles the keys of each load's rows
// come from scalar loads, and one more load copies the tile's keys into the
// stage (for the masks); span tiles issue the same count (the extra load
// copies 256 bytes of the first K row there), so the walker can wait for a
// tile with a fixed vmcnt.
template <int D>
struct Issue {
  static constexpr int kPerTile = Buf<D>::kInstr + 1;
};

template <int D>
__device__ __forceinline__ void issue_tile(const char* kg, const char* vg, uint32_t kvst_b,
                                           const Tile& t, const int32_t* vl, uint32_t dst,
                                           int lane) {
  using B = Buf<D>;
  constexpr int M = B::kInstrPerMat, R = B::kRowsPerInstr;
  const int sub = lane / B::kChunks;  // row within a load
  const int cl = lane % B::kChunks;   // LDS slot of this lane's 16 bytes
  if (t.wave < 0) {
    const char* kb = kg + (int64_t)t.ks * kvst_b;
    const char* vb = vg + (int64_t)t.ks * kvst_b;
#pragma unroll
    for (int gi = 0; gi < B::kInstr; ++gi) {
      const bool isv = gi >= M;
      const int gm = isv ? gi - M : gi;
      const int row = gm * R + sub;
      const uint32_t rr = (uint32_t)(row < t.n ? row : t.n - 1);
      const int chunk = isv ? swz_v<D>(cl, row) : swz_k<D>(cl, row);
      dma16_s(isv ? vb : kb, rr * kvst_b + (uint32_t)chunk * 16u,
              dst + (isv ? B::kKBytes : 0) + gm * 1024);
    }
    dma4_v(kb + (lane & (D / 2 - 1)) * 4, dst + B::kKeyOff);
  } else {
#pragma unroll
    for (int gi = 0; gi < B::kInstr; ++gi) {
      const bool isv = gi >= M;
      const int gm = isv ? gi - M : gi;
      // keys of the R rows of this load (uniform), then this lane's one
      int32_t key = 0;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int row = gm * R + r;
        const int32_t kr = ld_uniform(vl + t.ks + (row < t.n ? row : t.n - 1));
        key = sub == r ? kr : key;
      }
      const int row = gm * R + sub;
      const int chunk = isv ? swz_v<D>(cl, row) : swz_k<D>(cl, row);
      dma16_v((isv ? vg : kg) + (int64_t)key * kvst_b + chunk * 16,
              dst + (isv ? B::kKBytes : 0) + gm * 1024);
    }
    dma4_v(vl + t.ks + (lane < t.n ? lane : t.n - 1), dst + B::kKeyOff);
  }
}

template <int D>
struct WaveState {
  f16x8 q[D / 16];   // rotated query rows, the fp16 operand of QK^T
  f32x16 o[D / 32];
  float m, l;
};

// Query variant `var` of this wave's 32 rows (rows past the chunk read the
// chunk's last row; their outputs are not written).
template <int D>
__device__ __forceinline__ void load_q(const AttnArgs& a, int h, int32_t i0, int var,
                                       WaveState<D>& st) {
  const int lane = threadIdx.x & 63;
  int64_t t = (int64_t)i0 - a.c0 + (lane & 31);
  if (t > a.L - 1) t = a.L - 1;
  const uint16_t* base = a.q_rot + (((int64_t)var * a.H + h) * a.L + t) * D + 8 * (lane >> 5);
#pragma unroll
  for (int s = 0; s < D / 16; ++s) st.q[s] = *reinterpret_cast<const f16x8*>(base + s * 16);
}

// max / sum of this lane's value and the value of lane l ^ 32
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Scores of one (wave, key tile) step on the stage `smem`, into the bf16
// weights pf of the tile's PV product.  With `masked`, mword is the 64-bit key
// mask of this lane's row.  act0 / act1: the wave has pairs in key half 0 / 1
// of the tile; an empty half skips its QK product and its softmax (its
// weights are zero).  `mid` runs once the QK products are issued (a wave that
// multiplies the previous tile's PV product there overlaps those MFMAs with
// this tile's softmax; a rescale of O for this tile's row max then applies
// after that product, as the online softmax requires).  `after_qk` runs next
// (scalar loads issued there land during the softmax).
template <int D, typename M, typename F>
__device__ __forceinline__ void wave_scores(float scale_log2, const char* smem,
                                            const LaneConst<D>& c, WaveState<D>& st,
                                            bool act0, bool act1, bool masked, uint64_t mword,
                                            int half, bf16x8 (&pf)[4], M&& mid,
                                            F&& after_qk) {
  constexpr int RB = Buf<D>::kRowBytes;
  constexpr int KS = D / 16;  // k-steps of the QK product
  constexpr int DB = D / 32;  // 32-row blocks of O^T
  const bool act[2] = {act0, act1};
  f32x16 acc[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    if (!act[kb]) continue;
    f16x8 kf[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s)
      kf[s] = *reinterpret_cast<const f16x8*>(smem + c.k_rd[s] + kb * 32 * RB);
    // keep the reads ahead of the products (else the scheduler waits for each
    // read next to its MFMA)
    __builtin_amdgcn_sched_barrier(0);
    acc[kb] = (f32x16){};
#pragma unroll
    for (int s = 0; s < KS; ++s)
      acc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[s], st.q[s], acc[kb], 0, 0, 0);
  }
  mid();
  after_qk();
  // key k of the tile sits in register r of block kb: k = 32 kb + 8 (r / 4)
  // + 4 half + r % 4
  if (__builtin_expect(masked, 0)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (!act[kb]) continue;
      const uint32_t word = (uint32_t)((mword >> (4 * half)) >> (32 * kb));
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // all ones where the key is kept, zero where it is masked
        const uint32_t keep =
            (uint32_t)__builtin_amdgcn_sbfe((int)word, 8 * (r >> 2) + (r & 3), 1);
        acc[kb][r] =
            __uint_as_float((__float_as_uint(acc[kb][r]) & keep) | (0xFF800000u & ~keep));
      }
    }
  }
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  // weights 2^(l - m) against the row's running max m and their sum
  auto weights = [&](float msub, float& psum) {
    psum = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (act[s >> 1]) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          pf[s][e] = (__bf16)__builtin_amdgcn_exp2f(
              fmaf(acc[s >> 1][8 * (s & 1) + e], scale_log2, -msub));
        // row sum of the bf16 weights the PV product uses
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const bf16x2 pr = {pf[s][e], pf[s][e + 1]};
          psum = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, psum, false);
        }
      } else {
        pf[s] = (bf16x8){};
      }
    }
  };
  // The running max only guards the range: a weight is exact for any m, so
  // the tile's own max is needed only when a row has no max yet (its first
  // keys) or a weight may be far above 1 (sum above 2^64, well inside the
  // range of fp32 and bf16).
  float psum;
  weights(st.m == -INFINITY ? 0.f : st.m, psum);
  const bool has_key = mword != 0ull;
  if (__builtin_expect(__ballot((st.m == -INFINITY && has_key) || !(psum <= 0x1p64f)) != 0ull,
                       0)) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (!act[kb]) continue;
#pragma unroll
      for (int r = 0; r < 16; r += 2) mx = fmaxf(fmaxf(mx, acc[kb][r]), acc[kb][r + 1]);
    }
    mx = max_halves(mx) * scale_log2;
    if (mx > st.m) {
      const float alpha = (st.m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(st.m - mx);
      st.l *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.o[db][r] *= alpha;
      st.m = mx;
    }
    weights(st.m == -INFINITY ? 0.f : st.m, psum);
  }
  st.l += psum;
}

// The PV product of one tile: O^T += V^T P^T over the key halves with pairs.
template <int D>
__device__ __forceinline__ void wave_pv(const char* smem, const LaneConst<D>& c,
                                        WaveState<D>& st, const bf16x8 (&pf)[4], bool act0,
                                        bool act1) {
  constexpr int RB = Buf<D>::kRowBytes;
  constexpr int DB = D / 32;
  const bool act[2] = {act0, act1};
  // O^T += V^T P^T; each lane receives V[16 s + 4 half + r][d0 + j] (r = 0..3
  // for the first transpose load, +8 for the second), the k-order of its P
  // fragment
  auto load_v = [&](int s, int db) {
    const char* p = smem + c.v_rd[db] + 16 * s * RB;
    const v4i16 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
    const v4i16 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + 8 * RB));
    const v4i16 vv[2] = {va, vb};
    bf16x8 vf;
    __builtin_memcpy(&vf, vv, 16);
    return vf;
  };
  // each key half with pairs: its two k-steps, V fragments read together
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    if (!act[kb]) continue;
    bf16x8 vf[2][DB];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int db = 0; db < DB; ++db) vf[j][db] = load_v(2 * kb + j, db);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int db = 0; db < DB; ++db)
        st.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[j][db], pf[2 * kb + j], st.o[db],
                                                           0, 0, 0);
  }
}

// 16 copies of each of the four low bits of g
__device__ __forceinline__ uint64_t granule_keys(int32_t g) {
  uint64_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if ((g >> i) & 1) m |= 0xFFFFull << (16 * i);
  return m;
}

// Key mask of this lane's row for one tile and this wave's head (bit k: key
// k of the tile is critical for the row).  Span tiles: the pair (row, key)
// is critical when its offset row - key is a slash of the head or the key is
// a vertical of the head in a marked granule (verticals elsewhere are
// gathered); keys <= row.  W / C: the head's offset bits from word
// floor((i0 - ks - 63) / 32) (they hold [row - ks - 63, row - ks] for every
// row) and column bits from word ks / 32.  Straight-line vector code: only
// the 64-bit window shift depends on the lane.
__device__ __forceinline__ uint64_t span_mask(const Tile& t, const Win& W, const Win& C,
                                              int32_t i0, int32_t row, int r) {
  // keys of the tile in marked granules (the tile may start inside a granule)
  const int32_t gs = t.ks & (kGranule - 1);
  uint64_t gk = granule_keys(t.gran);
  if (gs) gk = (gk >> gs) | (((t.gran >> 4) & 1) ? (~0ull << (64 - gs)) : 0ull);
  gk &= low_bits(t.n);
  const int cs = t.ks - C.base;  // 0 .. 31
  const uint64_t c01 = ((uint64_t)C.w1 << 32) | C.w0;
  const uint64_t wcol = (cs ? (c01 >> cs) | ((uint64_t)C.w2 << (64 - cs)) : c01) & gk;
  const uint64_t lo = ((uint64_t)W.w1 << 32) | W.w0;
  const uint64_t hi = ((uint64_t)W.w3 << 32) | W.w2;
  const uint32_t rel = (uint32_t)(i0 - t.ks - 63 - W.base + r);  // 0 .. 62
  const uint64_t woff = rel ? (lo >> rel) | (hi << (64 - rel)) : lo;
  return (bitrev64(woff) | wcol) & low_bits(row - t.ks + 1) & low_bits(t.n);
}

// Gathered tile: the keys of the list (in the stage, ascending) that are <=
// the row.
__device__ __forceinline__ uint64_t gather_mask(const Tile& t, const int32_t* keys,
                                                int32_t row) {
  int lo = 0, hi = t.n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (keys[mid] <= row) lo = mid + 1;
    else hi = mid;
  }
  return low_bits(lo);
}


// Workgroup barrier of the tile ring.  It carries no release fence: a fenced
// barrier waits for every load in flight (vmcnt(0)), which would drain the
// ring.  A stage is visible to all waves because the producer waits for its
// loads of that stage (wait_vm) before arriving; the lgkmcnt(0) wait retires
// this wave's LDS reads and writes (stage reads, descriptor writes) before
// the barrier.  The empty asm statements keep the compiler from moving memory
// accesses across.
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// The head waves' barrier at the end of a step: every LDS read they issued
// has been consumed by then (the products waited for it), so only scalar
// loads of the next tile's windows can be outstanding, and those need not
// land before the barrier.  A stage is refilled two barriers after the step
// that reads it, so reads that the compiler moves past this barrier still
// complete in time.
__device__ __forceinline__ void step_barrier() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

constexpr int kRing = 8;  // tile descriptors in LDS (producer -> consumers)

// Descriptor: {ks, n | (wave + 1) << 8 | gran << 16, kchunk, kmax}; n = 0
// ends the walk.
__device__ __forceinline__ int4 pack_desc(const Tile& t) {
  return make_int4(t.ks, t.n | ((t.wave + 1) << 8) | (t.gran << 16), t.kchunk, t.kmax);
}
__device__ __forceinline__ Tile read_desc(const int4* slot) {
  const int4 d = *slot;
  Tile t;
  t.ks = __builtin_amdgcn_readfirstlane(d.x);
  const int32_t info = __builtin_amdgcn_readfirstlane(d.y);
  t.kchunk = __builtin_amdgcn_readfirstlane(d.z);
  t.kmax = __builtin_amdgcn_readfirstlane(d.w);
  t.n = info & 0xFF;
  t.wave = ((info >> 8) & 0xFF) - 1;
  t.gran = (info >> 16) & 0x1F;
  return t;
}

// Waves 0 .. NW - 1 compute (one query head each) and issue the tile loads
// between them; wave NW walks the tiles and publishes a descriptor per tile
// four tiles ahead.  Tile i sits in stage i mod 4; its loads are issued three
// tiles ahead.  One barrier per tile.
// kPair: one barrier per pair of tiles (sparse calls: the heads' uneven
// work per tile evens out over two); else one per tile, with the second
// wave of each SIMD a whole tile late (dense calls: every head has the same
// work, and the de-phasing is worth more).
template <int D, int NW, bool kPair>
__global__ void __launch_bounds__(64 * (NW + 1), 1) attn_kernel(AttnArgs a) {
  using B = Buf<D>;
  constexpr int kPerTile = Issue<D>::kPerTile;  // walker loads per tile
  __shared__ __attribute__((aligned(16))) char stage[kStages][B::kBytes];
  __shared__ int4 ring[kRing];
  __shared__ unsigned long long sstat[2];
  extern __shared__ uint32_t ub_lds[];  // granule bitmap of this row block

  // XCD-aware order: consecutive logical blocks (same KV group, next row
  // block) land on one XCD, sharing its L2.
  const int32_t nb = a.n_wgg * a.n_rb;
  const int32_t per_xcd = (nb + 7) / 8;
  const int32_t logical = (int32_t)(blockIdx.x % 8) * per_xcd + (int32_t)(blockIdx.x / 8);
  if (logical >= nb) return;
  const int32_t wgg = logical / a.n_rb;
  const int32_t rb = logical % a.n_rb;
  const int g = wgg / a.n_sub;
  const int sub = wgg % a.n_sub;
  const int h_first = g * a.G + sub * a.nw;
  const int n_here = min(a.nw, a.G - sub * a.nw);
  const uint64_t wg_heads = ((n_here >= 64 ? ~0ull : ((1ull << n_here) - 1)) << h_first);
  if (!(a.head_mask & wg_heads)) return;

  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, half = lane >> 5;
  const int32_t c0 = (int32_t)a.c0, c1 = (int32_t)a.n_ctx, period = (int32_t)a.period;
  const int32_t r0 = c0 + rb * kRowBlock;
  const int32_t rlast = (r0 + kRowBlock - 1 < c1 - 1) ? r0 + kRowBlock - 1 : c1 - 1;
  const int32_t i0 = r0;

  // the row block's granule bitmap into LDS
  const int32_t glast = rlast / kGranule;
  const int32_t nwords = glast / 32 + 1;
  {
    const uint32_t* src = a.ubits + ((int64_t)wgg * a.n_rb + rb) * a.ubw;
    for (int i = threadIdx.x; i < nwords; i += 64 * (NW + 1)) ub_lds[i] = src[i];
  }
  if (threadIdx.x < 2) sstat[threadIdx.x] = 0;
  __syncthreads();

  uint32_t exec_tiles = 0, sel = 0;
  if (w == NW) {
    // ---------------- walker: publishes tile j during step j - 4
    const uint32_t* first =
        a.first ? a.first + ((int64_t)wgg * a.n_rb + rb) * a.ubw * 4 : nullptr;
    const WalkConst wc{rlast, period, glast, nwords, n_here, rb, h_first, ub_lds, first};
    Walk walk;
    walk.phase = 0;
    walk.pos = 0;
    walk.chunk = -1;
    walk.nz = 0;
    walk.kc = 0;
    walk.edge = period;
    walk.gw = -1;
    walk.s0 = 0;
    walk.vcnt = 0;
    uint32_t cw = 0;
    uint4 nf = make_uint4(0u, 0u, 0u, 0u);
    Tile t;
    int n_tiles = -1;  // known once the walk ends
    auto publish = [&](int j) {
      const bool e = n_tiles < 0 && next_tile(a, wc, walk, cw, nf, t);
      if (!e && n_tiles < 0) n_tiles = j;
      if (lane == 0) ring[j & (kRing - 1)] = e ? pack_desc(t) : make_int4(0, 0, 0, 0);
    };
    // K / V of every tile, issued ahead of the step that multiplies it (one
    // tile per step: tile i + 2 while tile i is multiplied, into the stage of
    // tile i - 2; pairs: tiles 2j + 2, 2j + 3 during step j, into the stages
    // of step j - 1).  Two tiles are 66 loads: past the 63 the vmcnt counter
    // holds, the wave's next load issue waits for the oldest to return.
    const char* kg = reinterpret_cast<const char*>(a.k + (int64_t)g * a.kv_sh);
    const char* vg = reinterpret_cast<const char*>(a.v + (int64_t)g * a.kv_sh);
    const uint32_t kvst_b = (uint32_t)(a.kv_st * 2);
    const uint32_t stage0 = lds_addr(&stage[0][0]);
    auto issue = [&](const Tile& tt, int j) {
      if (tt.n > 0) {
        const int32_t* vl =
            a.vl + ((int64_t)(h_first + (tt.wave < 0 ? 0 : tt.wave)) * a.n_rb + rb) * a.max_vert;
        issue_tile<D>(kg, vg, kvst_b, tt, vl,
                      stage0 + (uint32_t)((j & (kStages - 1)) * B::kBytes), lane);
      }
    };
    // wait until only the loads of tile `ahead` may still be in flight
    auto land = [&](const Tile& ahead) {
      if (ahead.n > 0) wait_vm<kPerTile>();
      else wait_vm<0>();
    };
    if constexpr (kPair) {
      for (int j = 0; j < 6; ++j) publish(j);
      {
        const Tile ta = read_desc(&ring[0]), tb = read_desc(&ring[1]);
        issue(ta, 0);
        issue(tb, 1);
        wait_vm<0>();
      }
      ring_barrier();  // descriptors 0 .. 5 published, tiles 0 and 1 in their stages
      for (int j = 0; n_tiles < 0 || 2 * j < n_tiles; ++j) {
        // the consumers multiply tiles 2j and 2j + 1; tiles 2j + 2 and 2j + 3
        // go into the stages of step j - 1, whose products are done
        const Tile ta = read_desc(&ring[(2 * j + 2) & (kRing - 1)]);
        const Tile tb = read_desc(&ring[(2 * j + 3) & (kRing - 1)]);
        // One tile's loads in flight at a time: the second tile's loads go
        // out once the first tile's have landed, and a walk step runs while
        // each tile is in flight.  Against issuing both tiles back to back
        // this halved the HBM traffic of a 1M-token call (fewer lines evicted
        // from L2 before the other row blocks of the XCD read them), and it
        // is faster.
        issue(ta, 2 * j + 2);
        publish(2 * j + 6);
        wait_vm<0>();
        issue(tb, 2 * j + 3);
        publish(2 * j + 7);
        wait_vm<0>();
        ring_barrier();  // tiles 2j, 2j + 1 done; 2j + 2, 2j + 3 in their stages
      }
    } else {
      for (int j = 0; j < 4; ++j) publish(j);
      {
        const Tile ta = read_desc(&ring[0]), tb = read_desc(&ring[1]);
        issue(ta, 0);
        issue(tb, 1);
        land(tb);
      }
      ring_barrier();  // descriptors 0 .. 3 published, tile 0 in its stage
      for (int i = 0; n_tiles < 0 || i < n_tiles; ++i) {
        // the consumers multiply tile i
        const Tile tn = read_desc(&ring[(i + 2) & (kRing - 1)]);
        issue(tn, i + 2);
        publish(i + 4);
        land(tn);
        ring_barrier();  // tile i done, tile i + 1 in its stage
      }
    }
  } else {
    // ---------------- consumers: wave w multiplies for head h
    const int h = h_first + w;
    const bool live = w < n_here && ((a.head_mask >> h) & 1);
    const int32_t my_row = i0 + (lane & 31);
    const int32_t qchunk = period ? i0 / period : 0;
    LaneConst<D> lc;
    lane_consts<D>(lc, lane);
    WaveState<D> st;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) st.o[db] = (f32x16){};
    st.m = -INFINITY;
    st.l = 0.f;
    const uint32_t* offb = a.off_bits + (int64_t)(live ? h : 0) * a.n_words + kBitPad;
    const uint32_t* colb = a.col_bits + (int64_t)(live ? h : 0) * a.n_words + kBitPad;
    // offset / column windows of a span tile for this head (scalar loads)
    auto load_windows = [&](const Tile& tt, Win& W, Win& C) {
      if (tt.n > 0 && tt.wave < 0 && live && !a.dense) {
        W = load_win(offb, i0 - tt.ks - 63);
        C = load_win(colb, tt.ks);
      }
    };
    if constexpr (kPair) {
      ring_barrier();  // descriptors 0 .. 5 published, tiles 0 and 1 in their stages
      // DCA relation of a tile (the same for every wave and row: the period is
      // a multiple of 32, so a 32-row block lies inside one DCA chunk)
      auto var_of = [&](const Tile& tt) {
        const int32_t rel = qchunk - tt.kchunk;
        return a.n_var == 1 ? 0 : (rel >= 2 ? 2 : rel);
      };
      // Tiles come in runs of one DCA relation (keys ascend, so it changes at
      // most twice per walk): the query variant is reloaded only when it
      // changes.
      int cur_var = -1;
      auto use_var = [&](const Tile& tt) {
        const int var = var_of(tt);
        if (live && var != cur_var) {
          load_q<D>(a, h, i0, var, st);
          wait_vm<0>();
        }
        cur_var = var;
      };
      // This wave's key mask for a tile: pairs (row, key) of its head.
      auto mask_of = [&](const Tile& tt, const Win& W, const Win& C, const char* bc) {
        uint64_t m = 0;
        if (live && tt.wave < 0)
          m = span_mask(tt, W, C, i0, my_row, lane & 31);
        else if (live && tt.wave == w)
          m = gather_mask(tt, reinterpret_cast<const int32_t*>(bc + B::kKeyOff), my_row);
        return my_row <= rlast ? m : 0ull;
      };
      // Scores of one tile into pf; `mid` runs once its QK products are
      // issued, `next` requests the windows of the tile after it.
      auto scores = [&](const Tile& tt, const Win& W, const Win& C, const char* bc,
                        bf16x8 (&pf)[4], bool& act0, bool& act1, auto&& mid, auto&& next) {
        use_var(tt);
        const uint64_t mword = mask_of(tt, W, C, bc);
        act0 = __ballot((uint32_t)mword != 0u) != 0;
        act1 = __ballot((uint32_t)(mword >> 32) != 0u) != 0;
        const bool masked = __ballot(mword == ~0ull) != ~0ull;
        wave_scores<D>(a.scale_log2, bc, lc, st, act0, act1, masked, mword, half, pf, mid, next);
        if (act0 || act1) {
          ++exec_tiles;
          if (half == 0) sel += (uint32_t)__popcll(mword);
        }
      };
      // One step per pair of tiles (tile i in stage i mod 4), then one barrier:
      // the step lasts as long as its slowest wave's two tiles, which evens out
      // the heads' work better than a barrier per tile.  The second wave on a
      // SIMD (waves 4 .. 6 share SIMDs with waves 0 .. 2) multiplies the first
      // tile's PV product during the second tile's softmax, so the two waves of
      // a SIMD alternate between the matrix cores and the vector ALUs.
      auto run = [&](auto lag) {
        constexpr bool kLate = decltype(lag)::value;
        Tile ta = read_desc(&ring[0]);
        Win W0{}, C0{}, W1{}, C1{};
        if (ta.n > 0 && ta.wave < 0 && live) {
          W0 = load_win(offb, i0 - ta.ks - 63);
          C0 = load_win(colb, ta.ks);
        }
        for (int i = 0; ta.n > 0; i += 2) {
          const Tile tb = read_desc(&ring[(i + 1) & (kRing - 1)]);
          const Tile tc = read_desc(&ring[(i + 2) & (kRing - 1)]);
          const char* ba = stage[i & (kStages - 1)];
          const char* bb = stage[(i + 1) & (kStages - 1)];
          bf16x8 pa[4];
          bool a0, a1;
          scores(ta, W0, C0, ba, pa, a0, a1, [] {}, [&] { load_windows(tb, W1, C1); });
          if (!kLate || tb.n == 0) wave_pv<D>(ba, lc, st, pa, a0, a1);
          if (tb.n > 0) {
            bf16x8 pb[4];
            bool b0, b1;
            if constexpr (kLate)
              scores(tb, W1, C1, bb, pb, b0, b1, [&] { wave_pv<D>(ba, lc, st, pa, a0, a1); },
                     [&] { load_windows(tc, W0, C0); });
            else
              scores(tb, W1, C1, bb, pb, b0, b1, [] {}, [&] { load_windows(tc, W0, C0); });
            wave_pv<D>(bb, lc, st, pb, b0, b1);
          }
          // tiles i, i + 1 done; both stages are refilled right after the
          // barrier, and every LDS read of this step has been consumed by a
          // product or a mask by then
          step_barrier();
          ta = tc;
        }
      };
      if (w >= 4) run(std::true_type{});
      else run(std::false_type{});
    } else {
      ring_barrier();  // descriptors 0 .. 3 published, tile 0 in its stage
      Tile t0 = read_desc(&ring[0]);
      // DCA relation of a tile (the same for every wave and row: the period is
      // a multiple of 32, so a 32-row block lies inside one DCA chunk)
      auto var_of = [&](const Tile& tt) {
        const int32_t rel = qchunk - tt.kchunk;
        return a.n_var == 1 ? 0 : (rel >= 2 ? 2 : rel);
      };
      Win W0{}, C0{}, W1{}, C1{};
      load_windows(t0, W0, C0);
      int i = 0;
      // The second wave on a SIMD (waves 4 .. 6 share SIMDs with waves 0 .. 2)
      // multiplies each tile's PV product one step late, during its next
      // tile's softmax: the two waves of a SIMD then alternate between the
      // matrix cores and the vector ALUs instead of contending for the same
      // unit at the same time.  The previous tile's stage is intact during the
      // step (it is refilled after the step's barrier).
      bf16x8 pf_prev[4];
  #pragma unroll
      for (int s = 0; s < 4; ++s) pf_prev[s] = (bf16x8){};
      bool pa0 = false, pa1 = false;
      const char* bc_prev = stage[0];
      // one step per tile (tile i in stage i mod 4), then the step's barrier
      auto step = [&](auto lag) {
        constexpr bool kLag = decltype(lag)::value;
        const Tile t1 = read_desc(&ring[(i + 1) & (kRing - 1)]);
        const char* bc = stage[i & (kStages - 1)];
        // this wave's key mask for the tile; act: any pair, full: all 64 x 32
        uint64_t mword = 0;
        // dense calls select every offset, so the span mask is the causal
        // one: no bitmap windows
        if (live && t0.wave < 0)
          mword = a.dense ? low_bits(my_row - t0.ks + 1) & low_bits(t0.n)
                          : span_mask(t0, W0, C0, i0, my_row, lane & 31);
        else if (live && t0.wave == w)
          mword = gather_mask(t0, reinterpret_cast<const int32_t*>(bc + B::kKeyOff), my_row);
        const bool row_ok = my_row <= rlast;
        if (!row_ok) mword = 0;
        const bool act0 = __ballot((uint32_t)mword != 0u) != 0;
        const bool act1 = __ballot((uint32_t)(mword >> 32) != 0u) != 0;
        const bool act = act0 || act1;
        const bool masked = __ballot(mword == ~0ull) != ~0ull;
        // the next tile's windows are requested during this tile's softmax
        bf16x8 pf[4];
        if constexpr (kLag) {
          wave_scores<D>(a.scale_log2, bc, lc, st, act0, act1, masked, mword, half, pf,
                         [&] { wave_pv<D>(bc_prev, lc, st, pf_prev, pa0, pa1); },
                         [&] { load_windows(t1, W1, C1); });
  #pragma unroll
          for (int s = 0; s < 4; ++s) pf_prev[s] = pf[s];
          pa0 = act0;
          pa1 = act1;
          bc_prev = bc;
        } else {
          wave_scores<D>(a.scale_log2, bc, lc, st, act0, act1, masked, mword, half, pf, [] {},
                         [&] { load_windows(t1, W1, C1); });
          wave_pv<D>(bc, lc, st, pf, act0, act1);
        }
        if (act) {
          ++exec_tiles;
          if (half == 0 && row_ok) sel += (uint32_t)__popcll(mword);
        }
        // tile i done, tile i + 1 in its stage; a late wave's reads of the
        // previous stage retire before the barrier (that stage is refilled
        // right after it)
        if constexpr (kLag) ring_barrier();
        else step_barrier();
        t0 = t1;
        W0 = W1;
        C0 = C1;
        ++i;
      };
      // tiles come in runs of one DCA relation (keys ascend, so it changes at
      // most twice per walk); the query variant is loaded once per run, outside
      // the inner loop
      auto run = [&](auto lag) {
        while (t0.n > 0) {
          const int var = var_of(t0);
          if (live) {
            load_q<D>(a, h, i0, var, st);
            wait_vm<0>();
          }
          do {
            step(lag);
          } while (t0.n > 0 && var_of(t0) == var);
        }
        // a late wave's last PV product (the last stage is not refilled)
        if constexpr (decltype(lag)::value) wave_pv<D>(bc_prev, lc, st, pf_prev, pa0, pa1);
      };
      if (w >= 4) run(std::true_type{});
      else run(std::false_type{});
    }

    // ---------------- epilogue
    if (live) {
      const float l_tot = sum_halves(st.l);
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      if (my_row <= rlast) {
        const int64_t tr = my_row - c0;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int d = 32 * db + 8 * i4 + 4 * half;
            const float v0 = st.o[db][4 * i4 + 0] * inv, v1 = st.o[db][4 * i4 + 1] * inv;
            const float v2 = st.o[db][4 * i4 + 2] * inv, v3 = st.o[db][4 * i4 + 3] * inv;
            if (a.out_dtype == LCSR_FP32) {
              float* o = static_cast<float*>(a.out) + h * a.o_sh + tr * a.o_st + d;
              *reinterpret_cast<float4*>(o) = make_float4(v0, v1, v2, v3);
            } else {
              uint16_t* o = static_cast<uint16_t*>(a.out) + h * a.o_sh + tr * a.o_st + d;
              *reinterpret_cast<uint2*>(o) =
                  make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
            }
          }
        if (a.lse && half == 0)
          a.lse[(int64_t)h * a.L + tr] = l_tot > 0.f ? (st.m + log2f(l_tot)) * kLn2 : -INFINITY;
      }
    }
  }
  if (a.stats) {
    __syncthreads();
    unsigned long long se = sel;
    for (int off = 32; off > 0; off >>= 1) se += __shfl_xor(se, off);
    if (lane == 0) {
      atomicAdd(&sstat[0], (unsigned long long)exec_tiles * 32ull * kTileK);
      atomicAdd(&sstat[1], se);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      atomicAdd(&a.stats[0], sstat[0]);
      atomicAdd(&a.stats[1], sstat[1]);
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
// at most kRunGap apart).  Indices outside [0, n_ctx) are ignored; indices
// must be ascending.
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
  // previous valid offset exceeds kRunGap
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
    const bool start = valid && (prev < 0 || o - prev > kRunGap);
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
        if (nx < 0 || nx - o > kRunGap) {
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

struct PlanArgs {
  const int32_t* vert_idx;
  const int32_t* vert_cnt;
  int32_t max_vert;
  const int32_t* runs;
  const int32_t* run_cnt;
  int32_t max_runs;
  int64_t n_ctx, c0;
  int32_t n_rb, n_sub, nw, G;
  int64_t ubw;
  uint32_t* ubits;
  uint32_t* first;  // [n_wgg][n_rb][4 ubw] first pair key of each granule, or null
  int32_t* vl;
  int32_t* vl_cnt;
  int32_t dense;
  uint64_t head_mask;
};

constexpr int kPlanThreads = 256;

// Set bits [g0, g1] of an LDS bitmap.
__device__ __forceinline__ void set_bits(uint32_t* bm, int32_t g0, int32_t g1) {
  for (int32_t wi = g0 >> 5; wi <= (g1 >> 5); ++wi) {
    const int32_t lo = max(g0, wi * 32) - wi * 32, hi = min(g1, wi * 32 + 31) - wi * 32;
    const uint32_t m = (hi == 31 ? 0xFFFFFFFFu : ((1u << (hi + 1)) - 1u)) & ~((1u << lo) - 1u);
    atomicOr(&bm[wi], m);
  }
}

// Lower nibble g of an LDS nibble array to at most v.
__device__ __forceinline__ void nib_min(uint32_t* nib, int32_t g, uint32_t v) {
  uint32_t* w = &nib[g >> 3];
  const int sh = 4 * (g & 7);
  uint32_t old = *reinterpret_cast<volatile uint32_t*>(w);
  while (((old >> sh) & 15u) > v) {
    const uint32_t prev = atomicCAS(w, old, (old & ~(15u << sh)) | (v << sh));
    if (prev == old) break;
    old = prev;
  }
}

// Per (row block, KV sub-group): the granules any of its heads' slash runs
// reach in the row block, and per head the verticals (<= the block's last
// row) in unmarked granules, ascending.  With `first`, also the first key of
// each marked granule that a pair of the row block reaches, as an offset
// 0..15 in the granule (4 bits per granule): the start of a run's key span
// [r0 - ob, rlast - oa] inside the granule, 0 when a span covers the
// granule's first key, or a vertical of a head in the granule.
__global__ void __launch_bounds__(kPlanThreads) plan_kernel(PlanArgs a) {
  extern __shared__ uint32_t bm[];
  const int rb = blockIdx.x, wgg = blockIdx.y;
  const int g = wgg / a.n_sub, sub = wgg % a.n_sub;
  const int h_first = g * a.G + sub * a.nw;
  const int n_here = min(a.nw, a.G - sub * a.nw);
  const int64_t r0 = a.c0 + (int64_t)rb * kRowBlock;
  const int64_t rlast = r0 + kRowBlock - 1 < a.n_ctx - 1 ? r0 + kRowBlock - 1 : a.n_ctx - 1;
  const int32_t glast = (int32_t)(rlast / kGranule);
  const int32_t nwords = glast / 32 + 1;
  const int tid = threadIdx.x;
  // with first: [ubw] marked granules, [ubw] granules whose first key a span
  // covers, [4 ubw] first-key nibbles
  const bool with_first = a.first != nullptr && !a.dense;
  uint32_t* cov = bm + a.ubw;
  uint32_t* nib = bm + 2 * a.ubw;
  for (int i = tid; i < nwords; i += kPlanThreads) bm[i] = 0u;
  if (with_first) {
    for (int i = tid; i < nwords; i += kPlanThreads) cov[i] = 0u;
    for (int i = tid; i < 4 * nwords; i += kPlanThreads) nib[i] = 0xFFFFFFFFu;
  }
  __syncthreads();
  for (int hh = 0; hh < n_here; ++hh) {
    const int h = h_first + hh;
    if (!((a.head_mask >> h) & 1)) continue;
    if (a.dense) {
      const uint32_t last = glast % 32 == 31 ? 0xFFFFFFFFu : (1u << (glast % 32 + 1)) - 1u;
      for (int i = tid; i < nwords; i += kPlanThreads)
        atomicOr(&bm[i], i < nwords - 1 ? 0xFFFFFFFFu : last);
      continue;
    }
    const int nr = min(a.run_cnt[h], a.max_runs);
    const int2* rr = reinterpret_cast<const int2*>(a.runs + (int64_t)h * a.max_runs * 2);
    // four runs per thread loaded before the first is used (indices past the
    // list read its last run and are skipped)
    for (int i0 = tid; i0 < nr; i0 += 4 * kPlanThreads) {
      int2 run[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u * kPlanThreads;
        run[u] = rr[i < nr ? i : nr - 1];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t oa = run[u].x, ob = run[u].y;
        if (i0 + u * kPlanThreads >= nr || oa > rlast) continue;
        const int64_t lo = r0 - ob > 0 ? r0 - ob : 0, hi = rlast - oa;
        set_bits(bm, (int32_t)(lo / kGranule), (int32_t)(hi / kGranule));
        if (with_first) {
          const int32_t gc = (int32_t)((lo + kGranule - 1) / kGranule);
          const int32_t gh = (int32_t)(hi / kGranule);
          if (gc <= gh) set_bits(cov, gc, gh);
          if (lo % kGranule) nib_min(nib, (int32_t)(lo / kGranule), (uint32_t)(lo % kGranule));
        }
      }
    }
  }
  __syncthreads();
  uint32_t* dst = a.ubits + ((int64_t)wgg * a.n_rb + rb) * a.ubw;
  for (int i = tid; i < nwords; i += kPlanThreads) dst[i] = bm[i];
  if (a.dense) {
    for (int hh = tid; hh < n_here; hh += kPlanThreads)
      a.vl_cnt[(int64_t)(h_first + hh) * a.n_rb + rb] = 0;
    return;
  }
  __shared__ int s_wave[kPlanThreads / 64];
  const int lane = tid & 63, w = tid >> 6;
  for (int hh = 0; hh < n_here; ++hh) {
    const int h = h_first + hh;
    if (!((a.head_mask >> h) & 1)) continue;
    const int nv = min(a.vert_cnt[h], a.max_vert);
    const int32_t* vo = a.vert_idx + (int64_t)h * a.max_vert;
    int32_t* out = a.vl + ((int64_t)h * a.n_rb + rb) * a.max_vert;
    int total = 0;
    for (int b0 = 0; b0 < nv; b0 += kPlanThreads) {
      const int i = b0 + tid;
      // this thread's vertical and the batch's first, loaded together
      const int32_t vi = vo[i < nv ? i : nv - 1];
      if (vo[b0] > rlast) break;
      bool keep = false;
      int32_t v = 0;
      if (i < nv) {
        v = vi;
        if (v >= 0 && v <= rlast) {
          const int32_t gi = v / kGranule;
          keep = !((bm[gi >> 5] >> (gi & 31)) & 1u);
          // a vertical in a marked granule is a span-tile key
          if (!keep && with_first) nib_min(nib, gi, (uint32_t)(v % kGranule));
        }
      }
      const uint64_t bal = __ballot(keep);
      __syncthreads();
      if (lane == 0) s_wave[w] = __popcll(bal);
      __syncthreads();
      int base = total, tot = 0;
      for (int x = 0; x < kPlanThreads / 64; ++x) {
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
    if (tid == 0) a.vl_cnt[(int64_t)h * a.n_rb + rb] = total;
  }
  if (with_first) {
    __syncthreads();
    uint32_t* fd = a.first + ((int64_t)wgg * a.n_rb + rb) * a.ubw * 4;
    for (int i = tid; i < 4 * nwords; i += kPlanThreads) {
      // nibble word i holds granules 8i .. 8i + 7: zero where a span covers
      // the granule's first key
      const uint32_t cb = (cov[i >> 2] >> (8 * (i & 3))) & 0xFFu;
      uint32_t clear = 0u;
#pragma unroll
      for (int b = 0; b < 8; ++b)
        if ((cb >> b) & 1u) clear |= 15u << (4 * b);
      fd[i] = nib[i] & ~clear;
    }
  }
}

template <int D, int NW>
int launch_attn(const AttnArgs& a, int64_t grid, size_t dyn_lds, hipStream_t s) {
  if (a.dense)
    hipLaunchKernelGGL((attn_kernel<D, NW, false>), dim3((unsigned)grid), dim3(64 * (NW + 1)),
                       dyn_lds, s, a);
  else
    hipLaunchKernelGGL((attn_kernel<D, NW, true>), dim3((unsigned)grid), dim3(64 * (NW + 1)),
                       dyn_lds, s, a);
  return check_launch("sparse attention");
}

template <int D>
int launch_attn_nw(const AttnArgs& a, int nw, int64_t grid, size_t dyn_lds, hipStream_t s) {
  switch (nw) {
    case 1: return launch_attn<D, 1>(a, grid, dyn_lds, s);
    case 2: return launch_attn<D, 2>(a, grid, dyn_lds, s);
    case 3: return launch_attn<D, 3>(a, grid, dyn_lds, s);
    case 4: return launch_attn<D, 4>(a, grid, dyn_lds, s);
    case 5: return launch_attn<D, 5>(a, grid, dyn_lds, s);
    case 6: return launch_attn<D, 6>(a, grid, dyn_lds, s);
    case 7: return launch_attn<D, 7>(a, grid, dyn_lds, s);
    default: return fail(LCSR_ENOTSUP, "%d query heads per workgroup", nw);
  }
}

// ---------------------------------------------------------------- decode
// Decode-step attention: the newest rows of the sequence (tokens c0 .. c0 +
// n_q - 1, whose keys are already in the cache) against every causal key,
// dense, with the DCA logits of the prefill (Length Extrapolation: intra /
// successive / inter relations; blocked online softmax: deepseekmodel.com
// §3.2).  The step reads the whole K/V prefix once, so the work is split
// over the keys: workgroup (split, KV head) streams its key range through a
// four-stage K/V ring in LDS and multiplies it with the G x n_q (head, row)
// pairs of the KV group on the 32 rows of the matrix products, and writes
// the unnormalised partial (m, l, O) of every pair; decode_combine merges
// the splits in a fixed order.
struct DecArgs {
  const uint16_t* __restrict__ q_rot;  // [n_var][H][n_q][D]
  const uint16_t* __restrict__ k;
  const uint16_t* __restrict__ v;
  int64_t kv_sh, kv_st;
  int32_t H, G, n_var, n_q, n_split;
  int64_t c0, n_ctx, period, n_tiles, tiles_per_split;
  float scale_log2;
  float* part_o;   // [H_kv][n_split][32][D]
  float* part_ml;  // [H_kv][n_split][32][2]
};

constexpr int kDecStages = 5;

// Workgroup: waves 0 and 1 multiply, wave 0 the first and wave 1 the second
// 32-key half of every tile, each with an online softmax state of its own;
// wave 2 loads the K tiles and wave 3 the V tiles of the key range
// (direct-to-LDS, 16 loads per tile each; four tiles in flight are 64 loads,
// one past what the vmcnt counter holds, so the last issue waits for the
// oldest load to return).  A stage holds K then V of one tile (no key
// list: 32 KB at D 128, so five stages fill the 160 KB of LDS).  Tile i of
// the range sits in stage i mod 5; at barrier i tile i has landed and the
// products of tile i - 1 are done, so tile i + 4 then refills that stage.
// At the end the two states are merged in a fixed order (wave 0's, then
// wave 1's), so the partial does not depend on timing.
constexpr int kDecThreads = 256;

template <int D>
__global__ void __launch_bounds__(kDecThreads, 1) decode_kernel(DecArgs a) {
  using B = Buf<D>;
  constexpr int M = B::kInstrPerMat;  // loads per matrix and tile
  constexpr int R = B::kRowsPerInstr;
  constexpr int kStageBytes = 2 * B::kKBytes;
  __shared__ __attribute__((aligned(16))) char stage[kDecStages][kStageBytes];
  const int split = blockIdx.x, g = blockIdx.y;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, half = lane >> 5;
  const int64_t t_begin = (int64_t)split * a.tiles_per_split;
  const int64_t t_end =
      t_begin + a.tiles_per_split < a.n_tiles ? t_begin + a.tiles_per_split : a.n_tiles;
  const int n_local = t_end > t_begin ? (int)(t_end - t_begin) : 0;
  auto tile_of = [&](int64_t t) {
    Tile x;
    x.ks = (int32_t)(t * kTileK);
    x.n = (int32_t)(a.n_ctx - x.ks < kTileK ? a.n_ctx - x.ks : kTileK);
    x.wave = -1;
    x.kchunk = a.period ? (int32_t)(x.ks / a.period) : 0;
    x.kmax = x.ks + x.n - 1;
    x.gran = 15;
    return x;
  };
  if (w >= 2) {
    // ---------------- loaders: wave 2 K, wave 3 V
    const bool isv = w == 3;
    const char* src = reinterpret_cast<const char*>((isv ? a.v : a.k) + (int64_t)g * a.kv_sh);
    const uint32_t kvst_b = (uint32_t)(a.kv_st * 2);
    const uint32_t base = lds_addr(&stage[0][0]) + (isv ? B::kKBytes : 0);
    const int sub = lane / B::kChunks, cl = lane % B::kChunks;
    auto issue = [&](int i) {
      const Tile x = tile_of(t_begin + i);
      const char* sb = src + (int64_t)x.ks * kvst_b;
      const uint32_t dst = base + (uint32_t)((i % kDecStages) * kStageBytes);
#pragma unroll
      for (int gm = 0; gm < M; ++gm) {
        const int row = gm * R + sub;
        const uint32_t rr = (uint32_t)(row < x.n ? row : x.n - 1);
        const int chunk = isv ? swz_v<D>(cl, row) : swz_k<D>(cl, row);
        dma16_s(sb, rr * kvst_b + (uint32_t)chunk * 16u, dst + gm * 1024);
      }
    };
    for (int i = 0; i < kDecStages - 1 && i < n_local; ++i) issue(i);
    for (int i = 0; i < n_local; ++i) {
      // tile i has landed: only tiles i + 1 .. i + 3 may still be in flight
      const int ahead = n_local - 1 - i;
      if (ahead >= 3) wait_vm<3 * M>();
      else if (ahead == 2) wait_vm<2 * M>();
      else if (ahead == 1) wait_vm<M>();
      else wait_vm<0>();
      step_barrier();
      if (i + kDecStages - 1 < n_local) issue(i + kDecStages - 1);
    }
    __syncthreads();  // the products are done: stage 0 takes wave 1's state
    __syncthreads();  // wave 0 has read it
    return;
  }
  // ---------------- waves 0 and 1: the products of key half w
  // this lane's matrix row: (head, row) pair rho; rows past G x n_q repeat a
  // live pair's query and are never written
  const int rho = lane & 31;
  const bool live = rho < a.G * a.n_q;
  const int hh = live ? rho / a.n_q : 0, r = live ? rho % a.n_q : 0;
  const int h = g * a.G + hh;
  const int64_t pos = a.c0 + r;
  const int64_t qchunk = a.period ? pos / a.period : 0;
  LaneConst<D> lc;
  lane_consts<D>(lc, lane);
  WaveState<D> st;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) st.o[db] = (f32x16){};
  st.m = -INFINITY;
  st.l = 0.f;
  int cur_var = -1;
  // One iteration per (tile, key chunk) pass: a tile meets at most one DCA
  // chunk edge (the period is at least 64 keys), and the keys on either side
  // take the query variant of their own chunk.  The products run on every
  // iteration (a product that a branch may skip would merge two copies of
  // the accumulators); the barrier comes with each new tile.
  // the key chunk of the current tile and the first key of the next chunk,
  // kept up to date as the tiles ascend (the period is at least one tile)
  int32_t kc0 = a.period ? (int32_t)(t_begin * kTileK / a.period) : 0;
  int64_t next_edge = a.period ? (int64_t)(kc0 + 1) * a.period : INT64_MAX;
  int64_t ks = 0;
  int32_t tn = 0;
  uint64_t causal = 0;
  int64_t edge = kTileK;  // first key of the later chunk in the tile
  int seg = 0;
  for (int i = 0; i < n_local;) {
    if (seg == 0) {
      step_barrier();  // tile i in its stage; the stage of tile i - 1 is released
      ks = (t_begin + i) * kTileK;
      tn = (int32_t)(a.n_ctx - ks < kTileK ? a.n_ctx - ks : kTileK);
      if (ks >= next_edge) {
        ++kc0;
        next_edge += a.period;
      }
      // keys <= this row's token; the other rows see the whole tile
      const int64_t lim = live ? pos - ks + 1 : kTileK;
      causal = low_bits(lim < tn ? lim : tn);
      edge = next_edge - ks < tn ? next_edge - ks : kTileK;
    }
    const int32_t kc = kc0 + seg;
    // the query variant of this lane's row against the key chunk.  Rows of
    // one call may straddle a chunk edge: an earlier row then meets keys of
    // the next chunk (rel < 0), which all lie after it and are masked; it
    // takes variant 0 there, so the query load stays inside the variants
    const int64_t rel = qchunk - kc;
    const int var = a.n_var == 1 ? 0 : (rel >= 2 ? 2 : (rel <= 0 ? 0 : (int)rel));
    if (__ballot(var != cur_var) != 0ull) {
      const uint16_t* qb = a.q_rot + (((int64_t)var * a.H + h) * a.n_q + r) * D + 8 * half;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) st.q[s] = *reinterpret_cast<const f16x8*>(qb + s * 16);
      wait_vm<0>();
      cur_var = var;
    }
    const uint64_t mword = causal & (seg ? ~low_bits(edge) : low_bits(edge));
    const bool act0 = w == 0 && __ballot((uint32_t)mword != 0u) != 0;
    const bool act1 = w == 1 && __ballot((uint32_t)(mword >> 32) != 0u) != 0;
    const bool masked = __ballot(mword == ~0ull) != ~0ull;
    const char* bc = stage[i % kDecStages];
    bf16x8 pf[4];
    wave_scores<D>(a.scale_log2, bc, lc, st, act0, act1, masked, mword, half, pf, [] {}, [] {});
    wave_pv<D>(bc, lc, st, pf, act0, act1);
    if (seg == 0 && edge < kTileK) {
      seg = 1;
    } else {
      seg = 0;
      ++i;
    }
  }
  // wave 1's state through LDS (stage 0, lane-major: conflict-free), merged
  // into wave 0's: M = max(m0, m1), l and O weighted by 2^(m - M)
  constexpr int NO = D / 32 * 16;  // O values per lane
  float* xs = reinterpret_cast<float*>(&stage[0][0]);
  __syncthreads();
  if (w == 1) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 16; ++i4) xs[(db * 16 + i4) * 64 + lane] = st.o[db][i4];
    xs[NO * 64 + lane] = st.m;
    xs[(NO + 1) * 64 + lane] = st.l;
  }
  __syncthreads();
  if (w == 1) return;
  {
    const float m1 = xs[NO * 64 + lane], l1 = xs[(NO + 1) * 64 + lane];
    const float mm = fmaxf(st.m, m1);
    const float a0 = st.m == -INFINITY ? 0.f : exp2f(st.m - mm);
    const float a1 = m1 == -INFINITY ? 0.f : exp2f(m1 - mm);
    st.l = st.l * a0 + l1 * a1;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 16; ++i4)
        st.o[db][i4] = st.o[db][i4] * a0 + xs[(db * 16 + i4) * 64 + lane] * a1;
    st.m = mm;
  }
  // the split's partial for every live pair: O unnormalised, m in log2 units
  if (live) {
    const float l_tot = sum_halves(st.l);
    const int64_t slot = ((int64_t)g * a.n_split + split) * 32 + rho;
    if (half == 0) {
      a.part_ml[slot * 2] = st.m;
      a.part_ml[slot * 2 + 1] = l_tot;
    }
    float* po = a.part_o + slot * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = 32 * db + 8 * i4 + 4 * half;
        *reinterpret_cast<float4*>(po + d) =
            make_float4(st.o[db][4 * i4], st.o[db][4 * i4 + 1], st.o[db][4 * i4 + 2],
                        st.o[db][4 * i4 + 3]);
      }
  }
}

// One (head, row) pair per workgroup of 256 threads (grid G x n_q, H_kv):
// out = sum_s O_s 2^(m_s - M) / L and lse = (M + log2 L) ln 2, with
// L = sum_s l_s 2^(m_s - M) and M the largest m_s.  One thread per split
// forms its weight; the O rows are summed by D/4 float4 columns x 256/(D/4)
// split groups, then the group sums are added in group order, so the result
// does not depend on timing.
template <int D>
__global__ void __launch_bounds__(256) decode_combine(DecArgs a, void* out, int32_t out_dtype,
                                                      int64_t o_sh, int64_t o_st, float* lse) {
  constexpr int C = D / 4;     // float4 columns of a row
  constexpr int NG = 256 / C;  // split groups
  __shared__ float wsplit[kMaxDecSplit];
  __shared__ float wmax[4], wsum[4];
  __shared__ float4 gsum[NG][C];
  const int rho = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int hh = rho / a.n_q, r = rho % a.n_q, h = g * a.G + hh;
  const int64_t base = (int64_t)g * a.n_split * 32 + rho;
  const float ms = tid < a.n_split ? a.part_ml[(base + (int64_t)tid * 32) * 2] : -INFINITY;
  const float ls = tid < a.n_split ? a.part_ml[(base + (int64_t)tid * 32) * 2 + 1] : 0.f;
  float mx = ms;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if (lane == 0) wmax[wv] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float w = ms == -INFINITY ? 0.f : exp2f(ms - M);
  wsplit[tid] = w;
  float lw = ls * w;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) lw += __shfl_xor(lw, off);
  if (lane == 0) wsum[wv] = lw;
  __syncthreads();
  const float L = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
  // a split without keys for this row holds O = 0 and weight 0
  const int c = tid % C, grp = tid / C;
  const float4* po = reinterpret_cast<const float4*>(a.part_o + base * D) + c;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
  for (int s = grp; s < a.n_split; s += NG) {
    const float4 x = po[(int64_t)s * 32 * C];
    const float ww = wsplit[s];
    acc.x += ww * x.x;
    acc.y += ww * x.y;
    acc.z += ww * x.z;
    acc.w += ww * x.w;
  }
  gsum[grp][c] = acc;
  __syncthreads();
  if (tid < C) {
    float4 t = gsum[0][tid];
#pragma unroll
    for (int k = 1; k < NG; ++k) {
      const float4 y = gsum[k][tid];
      t.x += y.x;
      t.y += y.y;
      t.z += y.z;
      t.w += y.w;
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const float o[4] = {t.x * inv, t.y * inv, t.z * inv, t.w * inv};
    const int64_t ob = h * o_sh + r * o_st + 4 * tid;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (out_dtype == LCSR_FP32)
        static_cast<float*>(out)[ob + e] = o[e];
      else
        static_cast<uint16_t*>(out)[ob + e] = f32_to_bf16(o[e]);
    }
  }
  if (lse && tid == 0) lse[(int64_t)h * a.n_q + r] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
}

// ------------------------------------------------------------ block sparse
// Attention over whole 64-key blocks: the 64 rows of query block qb of head h
// attend to the key blocks listed for it, causally inside the diagonal
// block.  The decode step's scheme with two consumers: waves 0 and 1 multiply
// (rows 0-31 and 32-63 of the block, sharing every tile), wave 2 streams the
// K tiles and wave 3 the V tiles of the list into a ring of kStages stages.
// Each lane takes the query variant of its own row; a key block that meets a
// DCA chunk edge runs as two passes, one per key chunk.
struct BsArgs {
  const uint16_t* __restrict__ q_rot;  // [n_var][H][L][D]
  const uint16_t* __restrict__ k;
  const uint16_t* __restrict__ v;
  int64_t kv_sh, kv_st;
  int32_t H, G, n_var, max_blocks;
  int64_t c0, L, n_ctx, period, n_qb;
  const int32_t* blk_idx;  // [H][n_qb][max_blocks]
  const int32_t* blk_cnt;  // [H][n_qb]
  uint64_t head_mask;
  float scale_log2;
  void* out;
  int32_t out_dtype;
  int64_t o_sh, o_st;
  float* lse;
  unsigned long long* stats;  // [2]: (executed, selected) pairs
};

constexpr int kBsStages = 2;  // ring stages (two workgroups per CU at D 128)

template <int M, int S>
__device__ __forceinline__ void wait_tiles_ahead(int ahead) {
  // `ahead` tiles after the one that must have landed are still allowed in
  // flight (at most S - 2)
  if (S >= 5 && ahead >= 3) wait_vm<3 * M>();
  else if (S >= 4 && ahead >= 2) wait_vm<2 * M>();
  else if (S >= 3 && ahead >= 1) wait_vm<M>();
  else wait_vm<0>();
}

template <int D, int kStages>
__global__ void __launch_bounds__(256) bs_attn_kernel(BsArgs a) {
  using B = Buf<D>;
  constexpr int M = B::kInstrPerMat;
  constexpr int R = B::kRowsPerInstr;
  constexpr int kStageBytes = 2 * B::kKBytes;
  __shared__ __attribute__((aligned(16))) char stage[kStages][kStageBytes];
  const int64_t qb = blockIdx.x;
  const int h = blockIdx.y;
  if (!((a.head_mask >> h) & 1ull)) return;
  const int g = h / a.G;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, half = lane >> 5;
  const int32_t* list = a.blk_idx + ((int64_t)h * a.n_qb + qb) * a.max_blocks;
  const int cnt_in = __builtin_amdgcn_readfirstlane(a.blk_cnt[(int64_t)h * a.n_qb + qb]);
  const int n_local = cnt_in < a.max_blocks ? cnt_in : a.max_blocks;
  // a listed block outside [0, diagonal] is taken as the diagonal: no load
  // leaves the keys the chunk can see, whatever the lists hold
  const int32_t diag = (int32_t)(a.c0 / kTileK + qb);
  auto tile_of = [&](int i) {
    int32_t kb = __builtin_amdgcn_readfirstlane(list[i]);
    kb = kb < 0 || kb > diag ? diag : kb;
    Tile x;
    x.ks = kb * kTileK;
    x.n = (int32_t)(a.n_ctx - x.ks < kTileK ? a.n_ctx - x.ks : kTileK);
    x.wave = -1;
    x.kchunk = a.period ? (int32_t)(x.ks / a.period) : 0;
    x.kmax = x.ks + x.n - 1;
    x.gran = 15;
    return x;
  };
  if (w >= 2) {
    const bool isv = w == 3;
    const char* src = reinterpret_cast<const char*>((isv ? a.v : a.k) + (int64_t)g * a.kv_sh);
    const uint32_t kvst_b = (uint32_t)(a.kv_st * 2);
    const uint32_t base = lds_addr(&stage[0][0]) + (isv ? B::kKBytes : 0);
    const int sub = lane / B::kChunks, cl = lane % B::kChunks;
    auto issue = [&](int i) {
      const Tile x = tile_of(i);
      const char* sb = src + (int64_t)x.ks * kvst_b;
      const uint32_t dst = base + (uint32_t)((i % kStages) * kStageBytes);
#pragma unroll
      for (int gm = 0; gm < M; ++gm) {
        const int row = gm * R + sub;
        const uint32_t rr = (uint32_t)(row < x.n ? row : x.n - 1);
        const int chunk = isv ? swz_v<D>(cl, row) : swz_k<D>(cl, row);
        dma16_s(sb, rr * kvst_b + (uint32_t)chunk * 16u, dst + gm * 1024);
      }
    };
    for (int i = 0; i < kStages - 1 && i < n_local; ++i) issue(i);
    for (int i = 0; i < n_local; ++i) {
      const int ahead = n_local - 1 - i;
      wait_tiles_ahead<M, kStages>(ahead);
      step_barrier();
      if (i + kStages - 1 < n_local) issue(i + kStages - 1);
    }
    return;
  }
  // ---------------- waves 0 and 1: the products; lane rows rho = lane & 31
  const int rho = lane & 31;
  const int64_t row = a.c0 + (qb * 2 + w) * kRowBlock + rho;
  const bool live = row < a.c0 + a.L;
  const int64_t my_row = live ? row : a.c0 + a.L - 1;
  const int64_t qchunk = a.period ? my_row / a.period : 0;
  LaneConst<D> lc;
  lane_consts<D>(lc, lane);
  WaveState<D> st;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) st.o[db] = (f32x16){};
  st.m = -INFINITY;
  st.l = 0.f;
  int cur_var = -1;
  unsigned long long sel = 0;
  // One iteration per (block, key chunk) pass: a block meets at most one DCA
  // chunk edge (the period is at least 64 keys), and its keys on either side
  // take the query variant of their own chunk; the barrier comes with each
  // new block.
  Tile tt{};
  int64_t edge = kTileK;  // first key of the later chunk in the block
  int seg = 0;
  for (int i = 0; i < n_local;) {
    if (seg == 0) {
      step_barrier();
      tt = tile_of(i);
      const int64_t next = (int64_t)(tt.kchunk + 1) * a.period - tt.ks;
      edge = (a.period && next < tt.n) ? next : kTileK;
    }
    // rel >= 0 here (kept blocks lie at or before the diagonal) except for a
    // row before an edge inside its own block; clamped all the same, so that
    // the query load can never leave the variants
    const int64_t rel = qchunk - (tt.kchunk + seg);
    const int var = a.n_var == 1 ? 0 : (rel >= 2 ? 2 : (rel <= 0 ? 0 : (int)rel));
    if (__ballot(var != cur_var) != 0ull) {
      const uint16_t* qp =
          a.q_rot + (((int64_t)var * a.H + h) * a.L + (my_row - a.c0)) * D + 8 * half;
#pragma unroll
      for (int s2 = 0; s2 < D / 16; ++s2) st.q[s2] = *reinterpret_cast<const f16x8*>(qp + s2 * 16);
      wait_vm<0>();
      cur_var = var;
    }
    const int64_t lim = my_row - tt.ks + 1;
    const uint64_t mword =
        low_bits(lim < tt.n ? lim : tt.n) & (seg ? ~low_bits(edge) : low_bits(edge));
    if (live && half == 0) sel += __popcll(mword);
    const bool act0 = __ballot((uint32_t)mword != 0u) != 0;
    const bool act1 = __ballot((uint32_t)(mword >> 32) != 0u) != 0;
    const bool masked = __ballot(mword == ~0ull) != ~0ull;
    const char* bc = stage[i % kStages];
    bf16x8 pf[4];
    wave_scores<D>(a.scale_log2, bc, lc, st, act0, act1, masked, mword, half, pf, [] {}, [] {});
    wave_pv<D>(bc, lc, st, pf, act0, act1);
    if (seg == 0 && edge < kTileK) {
      seg = 1;
    } else {
      seg = 0;
      ++i;
    }
  }
  const float l_tot = sum_halves(st.l);
  if (live) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int64_t tr = row - a.c0;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = 32 * db + 8 * i4 + 4 * half;
        const float v0 = st.o[db][4 * i4 + 0] * inv, v1 = st.o[db][4 * i4 + 1] * inv;
        const float v2 = st.o[db][4 * i4 + 2] * inv, v3 = st.o[db][4 * i4 + 3] * inv;
        if (a.out_dtype == LCSR_FP32) {
          float* o = static_cast<float*>(a.out) + h * a.o_sh + tr * a.o_st + d;
          o[0] = v0;
          o[1] = v1;
          o[2] = v2;
          o[3] = v3;
        } else {
          uint16_t* o = static_cast<uint16_t*>(a.out) + h * a.o_sh + tr * a.o_st + d;
          o[0] = f32_to_bf16(v0);
          o[1] = f32_to_bf16(v1);
          o[2] = f32_to_bf16(v2);
          o[3] = f32_to_bf16(v3);
        }
      }
    if (a.lse && half == 0)
      a.lse[(int64_t)h * a.L + tr] = l_tot > 0.f ? (st.m + log2f(l_tot)) * kLn2 : -INFINITY;
  }
  if (a.stats) {
    unsigned long long se = sel;
    for (int off = 32; off > 0; off >>= 1) se += __shfl_xor(se, off);
    if (lane == 0) {
      atomicAdd(&a.stats[0], (unsigned long long)n_local * 32ull * kTileK);
      atomicAdd(&a.stats[1], se);
    }
  }
}

// Block-sparse attention with the tiles shared by the heads of a KV group:
// one workgroup per (KV head g, 32-row block rb) holds one wave per query
// head of the group (NW <= 7) and one loader wave.  The heads' lists for the
// row block's query block are turned into per-head block bitmaps in LDS,
// their union is compacted into an ascending tile list with a per-tile head
// mask, and every union tile is streamed once (K then V, 32 loads) into a
// three-stage ring; a head wave multiplies only the tiles its own list holds.
// With the 7B grouping and 100 blocks per head, about 120 union tiles replace
// 700 per-head ones per query block.
constexpr int kBsgStages = 3;
constexpr int kBsgMaxList = 2048;  // union tiles per workgroup (NW x max_blocks bound)

template <int D, int NW>
__global__ void __launch_bounds__(64 * (NW + 1)) bs_attn_gqa_kernel(BsArgs a) {
  using B = Buf<D>;
  constexpr int M = B::kInstrPerMat;
  constexpr int R = B::kRowsPerInstr;
  constexpr int kStageBytes = 2 * B::kKBytes;
  __shared__ __attribute__((aligned(16))) char stage[kBsgStages][kStageBytes];
  __shared__ uint16_t tile_kb[kBsgMaxList];
  __shared__ uint8_t tile_heads[kBsgMaxList];
  __shared__ uint32_t n_tiles_sh;
  extern __shared__ uint32_t bits[];  // [NW + 1][nw]: head bitmaps, then the union
  const int rb = blockIdx.x, g = blockIdx.y;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, half = lane >> 5;
  const int64_t qb = rb >> 1;
  const int32_t diag = (int32_t)(a.c0 / kTileK + qb);
  const int nw = diag / 32 + 1;
  uint32_t* ubits = bits + NW * nw;
  // ---------------- the union tile list
  for (int x = threadIdx.x; x < (NW + 1) * nw; x += 64 * (NW + 1)) bits[x] = 0u;
  __syncthreads();
  if (w < NW) {
    const int h = g * a.G + w;
    if ((a.head_mask >> h) & 1ull) {
      const int32_t* list = a.blk_idx + ((int64_t)h * a.n_qb + qb) * a.max_blocks;
      int n = a.blk_cnt[(int64_t)h * a.n_qb + qb];
      n = n < a.max_blocks ? n : a.max_blocks;
      for (int x = lane; x < n; x += 64) {
        int32_t kb = list[x];
        kb = kb < 0 || kb > diag ? diag : kb;  // out-of-range entries: the diagonal
        atomicOr(&bits[w * nw + (kb >> 5)], 1u << (kb & 31));
      }
    }
  }
  __syncthreads();
  for (int x = threadIdx.x; x < nw; x += 64 * (NW + 1)) {
    uint32_t u = 0;
#pragma unroll
    for (int hh = 0; hh < NW; ++hh) u |= bits[hh * nw + x];
    ubits[x] = u;
  }
  __syncthreads();
  if (w == NW) {
    // ordered compaction of the union bitmap, 64 words per pass
    uint32_t base = 0;
    for (int x0 = 0; x0 < nw; x0 += 64) {
      const int x = x0 + lane;
      const uint32_t u = x < nw ? ubits[x] : 0u;
      const uint32_t cnt = __popc(u);
      uint32_t incl = cnt;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
      uint32_t pos = base + incl - cnt;
      uint32_t rest = u;
      while (rest) {
        const int b = __ffs(rest) - 1;
        rest &= rest - 1;
        if (pos < (uint32_t)kBsgMaxList) {
          const int kb = x * 32 + b;
          uint32_t hm = 0;
#pragma unroll
          for (int hh = 0; hh < NW; ++hh) hm |= ((bits[hh * nw + x] >> b) & 1u) << hh;
          tile_kb[pos] = (uint16_t)kb;
          tile_heads[pos] = (uint8_t)hm;
        }
        ++pos;
      }
      base += __shfl(incl, 63);
    }
    if (lane == 0) n_tiles_sh = base < (uint32_t)kBsgMaxList ? base : (uint32_t)kBsgMaxList;
  }
  __syncthreads();
  const int n_local = (int)__builtin_amdgcn_readfirstlane(n_tiles_sh);
  auto tile_of = [&](int i) {
    const int32_t kb = (int32_t)__builtin_amdgcn_readfirstlane(tile_kb[i]);
    Tile x;
    x.ks = kb * kTileK;
    x.n = (int32_t)(a.n_ctx - x.ks < kTileK ? a.n_ctx - x.ks : kTileK);
    x.wave = -1;
    x.kchunk = a.period ? (int32_t)(x.ks / a.period) : 0;
    x.kmax = x.ks + x.n - 1;
    x.gran = 15;
    return x;
  };
  if (w == NW) {
    // ---------------- loader: K then V of each union tile
    const char* kbase = reinterpret_cast<const char*>(a.k + (int64_t)g * a.kv_sh);
    const char* vbase = reinterpret_cast<const char*>(a.v + (int64_t)g * a.kv_sh);
    const uint32_t kvst_b = (uint32_t)(a.kv_st * 2);
    const uint32_t base = lds_addr(&stage[0][0]);
    const int sub = lane / B::kChunks, cl = lane % B::kChunks;
    auto issue = [&](int i) {
      const Tile x = tile_of(i);
      const int64_t off = (int64_t)x.ks * kvst_b;
      const uint32_t dst = base + (uint32_t)((i % kBsgStages) * kStageBytes);
#pragma unroll
      for (int gm = 0; gm < M; ++gm) {
        const int row = gm * R + sub;
        const uint32_t rr = (uint32_t)(row < x.n ? row : x.n - 1);
        dma16_s(kbase + off, rr * kvst_b + (uint32_t)swz_k<D>(cl, row) * 16u, dst + gm * 1024);
      }
#pragma unroll
      for (int gm = 0; gm < M; ++gm) {
        const int row = gm * R + sub;
        const uint32_t rr = (uint32_t)(row < x.n ? row : x.n - 1);
        dma16_s(vbase + off, rr * kvst_b + (uint32_t)swz_v<D>(cl, row) * 16u,
                dst + B::kKBytes + gm * 1024);
      }
    };
    for (int i = 0; i < kBsgStages - 1 && i < n_local; ++i) issue(i);
    for (int i = 0; i < n_local; ++i) {
      // tile i has landed; tile i + 1 may still be in flight
      if (n_local - 1 - i >= 1) wait_vm<2 * M>();
      else wait_vm<0>();
      step_barrier();
      if (i + kBsgStages - 1 < n_local) issue(i + kBsgStages - 1);
    }
    return;
  }
  // ---------------- head waves
  const int hh = w;
  const int h = g * a.G + hh;
  const bool head_on = (a.head_mask >> h) & 1ull;
  const int rho = lane & 31;
  const int64_t row = a.c0 + (int64_t)rb * kRowBlock + rho;
  const bool live = row < a.c0 + a.L;
  const int64_t my_row = live ? row : a.c0 + a.L - 1;
  const int64_t qchunk = a.period ? my_row / a.period : 0;
  LaneConst<D> lc;
  lane_consts<D>(lc, lane);
  WaveState<D> st;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) st.o[db] = (f32x16){};
  st.m = -INFINITY;
  st.l = 0.f;
  int cur_var = -1;
  unsigned long long sel = 0, exe = 0;
  // One iteration per (tile, key chunk) pass, as in bs_attn_kernel.
  Tile tt{};
  int64_t edge = kTileK;  // first key of the later chunk in the tile
  uint32_t heads = 0;
  int seg = 0;
  for (int i = 0; i < n_local;) {
    if (seg == 0) {
      step_barrier();
      heads = __builtin_amdgcn_readfirstlane(tile_heads[i]);
      tt = tile_of(i);
      const int64_t next = (int64_t)(tt.kchunk + 1) * a.period - tt.ks;
      edge = (a.period && next < tt.n) ? next : kTileK;
    }
    if (head_on && ((heads >> hh) & 1u)) {
      const int64_t rel = qchunk - (tt.kchunk + seg);
      const int var = a.n_var == 1 ? 0 : (rel >= 2 ? 2 : (rel <= 0 ? 0 : (int)rel));
      if (__ballot(var != cur_var) != 0ull) {
        const uint16_t* qp =
            a.q_rot + (((int64_t)var * a.H + h) * a.L + (my_row - a.c0)) * D + 8 * half;
#pragma unroll
        for (int s2 = 0; s2 < D / 16; ++s2)
          st.q[s2] = *reinterpret_cast<const f16x8*>(qp + s2 * 16);
        wait_vm<0>();
        cur_var = var;
      }
      const int64_t lim = my_row - tt.ks + 1;
      const uint64_t mword =
          low_bits(lim < tt.n ? lim : tt.n) & (seg ? ~low_bits(edge) : low_bits(edge));
      if (live && half == 0) sel += __popcll(mword);
      if (seg == 0) ++exe;
      const bool act0 = __ballot((uint32_t)mword != 0u) != 0;
      const bool act1 = __ballot((uint32_t)(mword >> 32) != 0u) != 0;
      const bool masked = __ballot(mword == ~0ull) != ~0ull;
      const char* bc = stage[i % kBsgStages];
      bf16x8 pf[4];
      wave_scores<D>(a.scale_log2, bc, lc, st, act0, act1, masked, mword, half, pf, [] {},
                     [] {});
      wave_pv<D>(bc, lc, st, pf, act0, act1);
    }
    if (seg == 0 && edge < kTileK) {
      seg = 1;
    } else {
      seg = 0;
      ++i;
    }
  }
  if (!head_on) return;
  const float l_tot = sum_halves(st.l);
  if (live) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int64_t tr = row - a.c0;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = 32 * db + 8 * i4 + 4 * half;
        const float v0 = st.o[db][4 * i4 + 0] * inv, v1 = st.o[db][4 * i4 + 1] * inv;
        const float v2 = st.o[db][4 * i4 + 2] * inv, v3 = st.o[db][4 * i4 + 3] * inv;
        if (a.out_dtype == LCSR_FP32) {
          float* o = static_cast<float*>(a.out) + h * a.o_sh + tr * a.o_st + d;
          o[0] = v0;
          o[1] = v1;
          o[2] = v2;
          o[3] = v3;
        } else {
          uint16_t* o = static_cast<uint16_t*>(a.out) + h * a.o_sh + tr * a.o_st + d;
          o[0] = f32_to_bf16(v0);
          o[1] = f32_to_bf16(v1);
          o[2] = f32_to_bf16(v2);
          o[3] = f32_to_bf16(v3);
        }
      }
    if (a.lse && half == 0)
      a.lse[(int64_t)h * a.L + tr] = l_tot > 0.f ? (st.m + log2f(l_tot)) * kLn2 : -INFINITY;
  }
  if (a.stats) {
    unsigned long long se = sel;
    for (int off = 32; off > 0; off >>= 1) se += __shfl_xor(se, off);
    if (lane == 0) {
      atomicAdd(&a.stats[0], exe * 32ull * kTileK);
      atomicAdd(&a.stats[1], se);
    }
  }
}

template <int D>
int launch_block_attn_gqa(const BsArgs& a, int nw, int64_t n_rb, int n_kv, hipStream_t s) {
  const int64_t words = (a.c0 / kTileK + (n_rb - 1) / 2) / 32 + 1;  // of the last row block
  const dim3 grid((unsigned)n_rb, (unsigned)n_kv);
#define LCSR_BSG(NW)                                                                      \
  hipLaunchKernelGGL((bs_attn_gqa_kernel<D, NW>), grid, dim3(64 * ((NW) + 1)),             \
                     (size_t)((NW) + 1) * words * 4, s, a)
  switch (nw) {
    case 1: LCSR_BSG(1); break;
    case 2: LCSR_BSG(2); break;
    case 3: LCSR_BSG(3); break;
    case 4: LCSR_BSG(4); break;
    case 5: LCSR_BSG(5); break;
    case 6: LCSR_BSG(6); break;
    default: LCSR_BSG(7); break;
  }
#undef LCSR_BSG
  return check_launch("block-sparse attention (shared tiles)");
}

template <int D>
int launch_block_attn(const BsArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((bs_attn_kernel<D, kBsStages>), dim3((unsigned)a.n_qb, (unsigned)a.H),
                     dim3(256), 0, s, a);
  return check_launch("block-sparse attention");
}

template <int D>
int launch_decode(const DecArgs& a, void* out, int32_t out_dtype, int64_t o_sh, int64_t o_st,
                  float* lse, int n_kv, hipStream_t s) {
  hipLaunchKernelGGL(decode_kernel<D>, dim3((unsigned)a.n_split, (unsigned)n_kv),
                     dim3(kDecThreads), 0, s, a);
  int rc = check_launch("decode attention");
  if (rc) return rc;
  hipLaunchKernelGGL(decode_combine<D>, dim3((unsigned)(a.G * a.n_q), (unsigned)n_kv), dim3(256),
                     0, s, a, out, out_dtype, o_sh, o_st, lse);
  return check_launch("decode combine");
}

}  // namespace

// Largest context the attention supports: the row block's granule bitmap
// shares the 160 KB of LDS with the four K/V stages.
int64_t attn_max_context(int64_t head_dim) {
  const int64_t stages = kStages * (head_dim == 128 ? Buf<128>::kBytes : Buf<64>::kBytes);
  const int64_t rings = kRing * 16;  // descriptors
  const int64_t words = (160 * 1024 - stages - rings - 64) / 4;
  return words * 32 * kGranule;
}

// The DCA period as the attention kernels see it: a DCA chunk longer than the
// context changes nothing (every key and query is in chunk 0); capping it
// keeps the chunk edges inside int32.
static int64_t attn_period(const DcaParams& d, int64_t n_ctx) {
  return d.period ? std::min<int64_t>(d.period, (n_ctx + kTileK) / kTileK * kTileK) : 0;
}

// Whether the plan records each granule's first pair key (sparse calls whose
// plan bitmaps fit 160 KB of LDS six times over; else tiles start at granule
// starts).
static bool attn_first_keys(const AttnLayout& L, bool dense) {
  return !dense && L.ubw * 4 * 6 <= 160 * 1024;
}

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
  a.dense = dense ? 1 : 0;
  a.head_mask = head_mask;
  hipLaunchKernelGGL(aux_kernel, dim3(p.n_heads), dim3(kAuxThreads), 0, s, a);
  int rc = check_launch("pattern aux");
  if (rc || !L.with_plan) return rc;
  PlanArgs b{};
  b.vert_idx = pat.vert_idx;
  b.vert_cnt = pat.vert_cnt;
  b.max_vert = dense ? 1 : pat.max_vert;
  b.runs = a.runs;
  b.run_cnt = a.run_cnt;
  b.max_runs = dense ? 1 : pat.max_slash;
  b.n_ctx = L.n_ctx;
  b.c0 = p.chunk_start;
  b.n_rb = (int32_t)L.n_rb;
  b.n_sub = (int32_t)L.n_sub;
  b.nw = (int32_t)L.nw;
  b.G = p.n_heads / p.n_kv_heads;
  b.ubw = L.ubw;
  b.ubits = reinterpret_cast<uint32_t*>(ws + L.o_union);
  b.first = attn_first_keys(L, dense) ? reinterpret_cast<uint32_t*>(ws + L.o_first) : nullptr;
  b.vl = reinterpret_cast<int32_t*>(ws + L.o_vl);
  b.vl_cnt = reinterpret_cast<int32_t*>(ws + L.o_vl_cnt);
  b.dense = dense ? 1 : 0;
  b.head_mask = head_mask;
  hipLaunchKernelGGL(plan_kernel, dim3((unsigned)L.n_rb, (unsigned)L.n_wgg), dim3(kPlanThreads),
                     (size_t)L.ubw * 4 * (b.first ? 6 : 1), s, b);
  return check_launch("attention plan");
}

int run_attention(const lcsr_problem_t& p, const lcsr_pattern_t& pat, uint64_t head_mask,
                  void* out, int32_t out_dtype, int64_t o_sh, int64_t o_st, float* lse,
                  int64_t* stats, bool dense, char* ws, hipStream_t s) {
  const AttnLayout L = attn_layout(p, dense ? 1 : pat.max_vert, dense ? 1 : pat.max_slash, true);
  if (L.n_ctx > attn_max_context(p.head_dim))
    return fail(LCSR_ENOTSUP, "attention supports contexts up to %lld tokens at head_dim %d",
                (long long)attn_max_context(p.head_dim), p.head_dim);
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
  a.period = attn_period(d, L.n_ctx);
  a.scale_log2 = p.sm_scale * kLog2e;
  a.off_bits = reinterpret_cast<const uint32_t*>(ws + L.o_off_bits);
  a.col_bits = reinterpret_cast<const uint32_t*>(ws + L.o_col_bits);
  a.n_words = L.n_words;
  a.ubits = reinterpret_cast<const uint32_t*>(ws + L.o_union);
  a.first =
      attn_first_keys(L, dense) ? reinterpret_cast<const uint32_t*>(ws + L.o_first) : nullptr;
  a.ubw = L.ubw;
  a.vl = reinterpret_cast<const int32_t*>(ws + L.o_vl);
  a.vl_cnt = reinterpret_cast<const int32_t*>(ws + L.o_vl_cnt);
  a.max_vert = dense ? 1 : pat.max_vert;
  a.n_rb = (int32_t)L.n_rb;
  a.n_sub = (int32_t)L.n_sub;
  a.nw = (int32_t)L.nw;
  a.n_wgg = (int32_t)L.n_wgg;
  a.dense = dense ? 1 : 0;
  a.head_mask = head_mask;
  a.out = out;
  a.out_dtype = out_dtype;
  a.o_sh = o_sh;
  a.o_st = o_st;
  a.lse = lse;
  a.stats = reinterpret_cast<unsigned long long*>(stats);
  const int64_t nb = L.n_wgg * L.n_rb;
  const int64_t grid = (nb + 7) / 8 * 8;
  const size_t dyn = (size_t)L.ubw * 4;
  if (p.head_dim == 128) return launch_attn_nw<128>(a, (int)L.nw, grid, dyn, s);
  return launch_attn_nw<64>(a, (int)L.nw, grid, dyn, s);
}

int run_decode(const lcsr_problem_t& p, void* out, int32_t out_dtype, int64_t o_sh,
               int64_t o_st, float* lse, char* ws, hipStream_t s) {
  const DecodeLayout L = decode_layout(p);
  FreqTable ft;
  int rc = build_freq_table(&p.rope, p.head_dim, &ft);
  if (rc) return rc;
  const DcaParams d = make_dca(&p.dca);
  uint16_t* q_rot = reinterpret_cast<uint16_t*>(ws + L.o_q_rot);
  rc = launch_rotate_q_variants(p, ft, d, q_rot, (int)L.n_var, s, true);
  if (rc) return rc;
  DecArgs a{};
  a.q_rot = q_rot;
  a.k = static_cast<const uint16_t*>(p.k_cache);
  a.v = static_cast<const uint16_t*>(p.v_cache);
  a.kv_sh = p.kv_stride_h;
  a.kv_st = p.kv_stride_t;
  a.H = p.n_heads;
  a.G = p.n_heads / p.n_kv_heads;
  a.n_var = (int32_t)L.n_var;
  a.n_q = (int32_t)p.chunk_len;
  a.n_split = (int32_t)L.n_split;
  a.c0 = p.chunk_start;
  a.n_ctx = L.n_ctx;
  a.period = attn_period(d, L.n_ctx);
  a.n_tiles = L.n_tiles;
  a.tiles_per_split = (L.n_tiles + L.n_split - 1) / L.n_split;
  a.scale_log2 = p.sm_scale * kLog2e;
  a.part_o = reinterpret_cast<float*>(ws + L.o_part_o);
  a.part_ml = reinterpret_cast<float*>(ws + L.o_part_ml);
  if (p.head_dim == 128) return launch_decode<128>(a, out, out_dtype, o_sh, o_st, lse, p.n_kv_heads, s);
  return launch_decode<64>(a, out, out_dtype, o_sh, o_st, lse, p.n_kv_heads, s);
}

int run_block_attention(const lcsr_problem_t& p, const int32_t* idx, const int32_t* cnt,
                        int32_t max_blocks, uint64_t head_mask, void* out, int32_t out_dtype,
                        int64_t o_sh, int64_t o_st, float* lse, int64_t* stats, char* ws,
                        hipStream_t s) {
  const BlockLayout L = block_layout(p);
  if (p.chunk_len == 0 || !head_mask) return LCSR_OK;
  FreqTable ft;
  int rc = build_freq_table(&p.rope, p.head_dim, &ft);
  if (rc) return rc;
  const DcaParams d = make_dca(&p.dca);
  uint16_t* q_rot = reinterpret_cast<uint16_t*>(ws + L.o_q_rot);
  rc = launch_rotate_q_variants(p, ft, d, q_rot, (int)L.n_var, s);
  if (rc) return rc;
  BsArgs a{};
  a.q_rot = q_rot;
  a.k = static_cast<const uint16_t*>(p.k_cache);
  a.v = static_cast<const uint16_t*>(p.v_cache);
  a.kv_sh = p.kv_stride_h;
  a.kv_st = p.kv_stride_t;
  a.H = p.n_heads;
  a.G = p.n_heads / p.n_kv_heads;
  a.n_var = (int32_t)L.n_var;
  a.max_blocks = max_blocks;
  a.c0 = p.chunk_start;
  a.L = p.chunk_len;
  a.n_ctx = L.n_ctx;
  a.period = d.period;
  a.n_qb = L.n_qb;
  a.blk_idx = idx;
  a.blk_cnt = cnt;
  a.head_mask = head_mask;
  a.scale_log2 = p.sm_scale * kLog2e;
  a.out = out;
  a.out_dtype = out_dtype;
  a.o_sh = o_sh;
  a.o_st = o_st;
  a.lse = lse;
  a.stats = reinterpret_cast<unsigned long long*>(stats);
  // tiles shared across the heads of a group when the union list fits in
  // LDS; else one workgroup per (head, query block)
  const int G = a.G;
  const int64_t n_rb = (p.chunk_len + kRowBlock - 1) / kRowBlock;
  if (G <= 7 && (int64_t)G * max_blocks <= kBsgMaxList)
    return p.head_dim == 128 ? launch_block_attn_gqa<128>(a, G, n_rb, p.n_kv_heads, s)
                             : launch_block_attn_gqa<64>(a, G, n_rb, p.n_kv_heads, s);
  return p.head_dim == 128 ? launch_block_attn<128>(a, s) : launch_block_attn<64>(a, s);
}

}  // namespace lcsr
