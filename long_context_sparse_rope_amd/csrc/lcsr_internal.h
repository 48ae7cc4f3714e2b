// Internal declarations shared by the HIP sources of liblcsr (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <string>

#include "lcsr.h"

namespace lcsr {

// ---------------------------------------------------------------- errors
void set_error(const char* fmt, ...);
int fail(int code, const char* fmt, ...);
int check_launch(const char* what);

// ---------------------------------------------------------------- vectors
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxHeads = 64;
constexpr int kMaxHalfDim = 64;          // head_dim <= 128 for attention
constexpr int kMaxRopeHalf = 128;        // head_dim <= 256 for rope_yarn_apply
constexpr int kMaxGroup = 16;            // n_heads / n_kv_heads
constexpr int kRowBlock = 32;            // query rows per attention workgroup
constexpr int kTileK = 64;               // keys per tile (attention, estimate)
constexpr int kGranule = 16;             // keys per bit of a row block's key-span bitmap
constexpr int kMaxAttnWaves = 7;         // query heads per attention workgroup (+1 loader wave)
constexpr int kEstRows = 64;             // largest last_q
constexpr int kBitPad = 8;               // zero words before and after each head's bitmap
constexpr int kMaxDecSplit = 256;        // key splits of the decode step per KV head
constexpr int kMaxKeyBlocks = 32768;     // 64-key blocks of a block-sparse context (2M keys)

// fp64 inverse frequencies, built on the host from lcsr_rope_t.
struct FreqTable {
  double inv_freq[kMaxRopeHalf];
};
int build_freq_table(const lcsr_rope_t* rope, int64_t head_dim, FreqTable* out);

// DCA parameters as the kernels see them (period == 0: DCA off).
struct DcaParams {
  int64_t chunk;   // C
  int64_t local;   // W
  int64_t period;  // S = C - W, or 0
};
DcaParams make_dca(const lcsr_dca_t* dca);

__device__ __forceinline__ int64_t dca_chunk_of(int64_t t, const DcaParams& d) {
  return d.period ? t / d.period : 0;
}
__device__ __forceinline__ int64_t dca_key_pos(int64_t t, const DcaParams& d) {
  return d.period ? t % d.period : t;
}
// Query position for the pair relation rel = chunk(i) - chunk(j) (0, 1, >= 2).
__device__ __forceinline__ int64_t dca_query_pos(int64_t i, int64_t rel,
                                                 const DcaParams& d) {
  if (!d.period) return i;
  int64_t ip = i % d.period;
  if (rel <= 0) return ip;
  if (rel == 1) return ip < d.local ? d.period + ip : d.chunk - 1;
  return d.chunk - 1;
}

// bf16 <-> fp32 (round to nearest even on the way down).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) |
         (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// fp16 <-> fp32 (round to nearest even on the way down).  The QK^T
// operands (rotated keys in the K cache, rotated queries) are fp16: for the
// unit-scale activations of attention its 11-bit significand rounds 8x finer
// than bf16's 8 bits at the same matrix-core rate.
__device__ __forceinline__ float f16_to_f32(uint16_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, b));
}
__device__ __forceinline__ uint16_t f32_to_f16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_f16(lo)) | (static_cast<uint32_t>(f32_to_f16(hi)) << 16);
}
// Round to the destination type (LCSR_BF16 or LCSR_FP16).
__device__ __forceinline__ uint16_t f32_to_16(float f, int32_t dtype) {
  return dtype == LCSR_FP16 ? f32_to_f16(f) : f32_to_bf16(f);
}
__device__ __forceinline__ uint32_t pack_16x2(float lo, float hi, int32_t dtype) {
  return dtype == LCSR_FP16 ? pack_f16x2(lo, hi) : pack_bf16x2(lo, hi);
}

// Angle pos * theta in fp64, reduced to [-pi, pi], then cos/sin.
__device__ __forceinline__ void rope_cos_sin(int64_t pos, double inv_freq,
                                             float* c, float* s) {
  const double two_pi = 6.283185307179586476925286766559;
  double a = static_cast<double>(pos) * inv_freq;
  a -= two_pi * rint(a / two_pi);
  double sd, cd;
  sincos(a, &sd, &cd);
  *c = static_cast<float>(cd);
  *s = static_cast<float>(sd);
}

// ---------------------------------------------------------------- launches
// Rotate rows of a [H, n_tok, D] tensor into a bf16 or fp16 destination.
// Position of token t (0-based within the call):
//   kPosArray:   pos[t]
//   kPosAffine:  t + pos_offset
//   kPosDca:     dca_query_pos(t + pos_offset, v) for the n_var variants
//                v = 0 .. n_var - 1, written at dst + v * dst_vs
//   kNoRotate:   no rotation (conversion and scale only)
enum PosMode : int32_t { kPosArray = 0, kPosAffine = 1, kPosDca = 2, kNoRotate = 3 };
struct RotateArgs {
  const void* src;
  int32_t src_dtype;
  int64_t src_sh, src_st;
  uint16_t* dst;
  int32_t dst_dtype;   // LCSR_BF16 or LCSR_FP16
  int64_t dst_vs, dst_sh, dst_st;
  int64_t n_heads, n_tok, head_dim;
  const int32_t* pos;
  int64_t pos_offset;
  int32_t mode;
  int32_t n_var;
  DcaParams dca;
  float scale;
};
int launch_rotate(const RotateArgs& a, const FreqTable& ft, hipStream_t s);

int launch_fill_zero(void* ptr, size_t bytes, hipStream_t s);

int launch_dca_positions(int64_t tok_start, int64_t n_tok, const DcaParams& d,
                         int32_t* pk, int32_t* pi, int32_t* ps, int32_t* pn,
                         hipStream_t s);

// Queries of the chunk rotated for the attention: variant v (0 intra,
// 1 succ, 2 inter; only 0 = plain position without DCA) written to
// dst[v][h][t][D] fp16 (the QK^T operand type).
int launch_rotate_q_variants(const lcsr_problem_t& p, const FreqTable& ft,
                             const DcaParams& d, uint16_t* dst, int n_var,
                             hipStream_t s, bool decode = false);

// Estimate rows rotated at continuous positions for each key DCA chunk c:
// dst[c][h][r][D] fp16 with position (row - c * S).
int launch_rotate_q_estimate(const lcsr_problem_t& p, const FreqTable& ft,
                             const DcaParams& d, int64_t row0, int n_rows,
                             int n_kc, uint16_t* dst, hipStream_t s);

}  // namespace lcsr

namespace lcsr {

// ---------------------------------------------------------------- workspace
// Byte layout of the caller's workspace for each call (host side).
struct EstimateLayout {
  int64_t n_ctx, n_tiles, n_kc, n_split;
  size_t q_est, part, lse, vscore, sscore, bnd, topk, total;
};
struct AttnLayout {
  int64_t n_ctx, n_words, n_var;
  int64_t n_rb;      // query row blocks of kRowBlock rows
  int64_t n_sub;     // workgroups per KV group (heads split into groups of <= 8)
  int64_t nw;        // query heads (waves) per workgroup
  int64_t n_wgg;     // KV head x sub-group
  int64_t ubw;       // 32-bit words of one row block's granule bitmap
  bool with_plan;    // attention: union bitmaps and leftover vertical lists
  size_t o_q_rot, o_off_bits, o_col_bits, o_runs, o_run_cnt, o_union, o_first, o_vl, o_vl_cnt,
      total;
};
struct DecodeLayout {
  int64_t n_ctx, n_tiles, n_var, n_split;
  size_t o_q_rot, o_part_o, o_part_ml, total;
};
// Block-sparse pattern: 64-token blocks; estimate workspace (pooled keys,
// pooled query variants, scores) and attention workspace (rotated queries).
struct BlockLayout {
  int64_t n_ctx, n_qb, n_kb, n_kc, n_var;
  size_t o_pk, o_pq, o_scores, est_total;
  size_t o_q_rot, attn_total;
};
BlockLayout block_layout(const lcsr_problem_t& p);
EstimateLayout estimate_layout(const lcsr_problem_t& p);
DecodeLayout decode_layout(const lcsr_problem_t& p);
AttnLayout attn_layout(const lcsr_problem_t& p, int32_t max_vert, int32_t max_slash,
                       bool attention);

// ---------------------------------------------------------------- kernels
struct HeadSet {
  uint64_t mask;              // bit h set: head h is processed
  int32_t n_vert[kMaxHeads];  // budgets (estimate)
  int32_t n_slash[kMaxHeads];
};

// Top-k of the vertical (set 0) and slash (set 1) score rows of every head.
struct TopkRequest {
  const float* scores[2];  // [n_heads][stride]
  int32_t* idx[2];         // [n_heads][max_k[set]]
  int32_t* cnt[2];         // [n_heads]
  int32_t max_k[2];
  const int32_t* budget[2];  // host arrays of n_heads budgets
  int64_t n, stride;
  int n_heads;
  uint64_t head_mask;
  void* ws;                // topk_workspace(n, n_heads) bytes
};
size_t topk_workspace(int64_t n, int n_heads);
int launch_topk(const TopkRequest& r, hipStream_t s);

int run_estimate(const lcsr_problem_t& p, int32_t last_q, const HeadSet& hs,
                 const lcsr_pattern_t& pat, float* vscore, float* sscore,
                 bool select_only, char* ws, hipStream_t s);

int run_attention(const lcsr_problem_t& p, const lcsr_pattern_t& pat,
                  uint64_t head_mask, void* out, int32_t out_dtype,
                  int64_t o_sh, int64_t o_st, float* lse, int64_t* stats,
                  bool dense, char* ws, hipStream_t s);

int run_block_estimate(const lcsr_problem_t& p, const int32_t* budgets_host, uint64_t head_mask,
                       int32_t max_blocks, int32_t* idx, int32_t* cnt, float* scores,
                       bool select_only, char* ws, hipStream_t s);

int run_block_attention(const lcsr_problem_t& p, const int32_t* idx, const int32_t* cnt,
                        int32_t max_blocks, uint64_t head_mask, void* out, int32_t out_dtype,
                        int64_t o_sh, int64_t o_st, float* lse, int64_t* stats, char* ws,
                        hipStream_t s);

int run_block_recall(const lcsr_problem_t& p, const int32_t* idx, const int32_t* cnt,
                     int32_t max_blocks, uint64_t head_mask, const int32_t* rows,
                     int32_t n_rows, float* lse_full, float* lse_sparse, float* recall,
                     hipStream_t s);

int run_decode(const lcsr_problem_t& p, void* out, int32_t out_dtype, int64_t o_sh,
               int64_t o_st, float* lse, char* ws, hipStream_t s);

// A-shape rows (verticals 0 .. nv - 1, slashes 0 .. ns - 1) for the heads
// of `mask`.
int launch_fill_a_shape(const lcsr_pattern_t& pat, int32_t n_heads, uint64_t mask,
                        int32_t nv, int32_t ns, hipStream_t s);

int run_recall(const lcsr_problem_t& p, const lcsr_pattern_t& pat,
               uint64_t head_mask, const int32_t* rows, int32_t n_rows,
               float* lse_full, float* lse_sparse, float* recall, char* ws,
               hipStream_t s);

// Pattern bitmaps (offset bits and column bits per head) and slash runs,
// shared by the attention and the recall check.
int build_pattern_aux(const lcsr_problem_t& p, const lcsr_pattern_t& pat,
                      uint64_t head_mask, bool dense, const AttnLayout& L,
                      char* ws, hipStream_t s);

}  // namespace lcsr
