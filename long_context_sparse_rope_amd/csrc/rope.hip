// RoPE / YaRN rotation, DCA position maps and the query pre-rotations.
//
// Rotation: rotate_half convention (deepseekmodel.com long-context
// architecture page, §2.4 code): the pair (x_p, x_{p+D/2}) turns by
// pos * theta_p.  The angle is formed in fp64 from the integer position and
// reduced to [-pi, pi] before sin/cos, so positions up to 2^31 keep full
// fp32 accuracy; the rotation itself is fp32 and the store bf16 or fp16
// (RNE): fp16 for the QK^T operands (K cache, query variants), bf16 for
// the V cache copy.
#include <cmath>

#include "lcsr_internal.h"

namespace lcsr {

DcaParams make_dca(const lcsr_dca_t* dca) {
  DcaParams d{0, 0, 0};
  if (dca && dca->chunk > 0) {
    d.chunk = dca->chunk;
    d.local = dca->local;
    d.period = dca->chunk - dca->local;
  }
  return d;
}

int build_freq_table(const lcsr_rope_t* rope, int64_t head_dim, FreqTable* out) {
  if (!rope) return fail(LCSR_EINVAL, "rope is NULL");
  if (head_dim <= 0 || head_dim % 2 || head_dim / 2 > kMaxRopeHalf)
    return fail(LCSR_EINVAL, "head_dim %lld must be even and <= %d",
                (long long)head_dim, 2 * kMaxRopeHalf);
  if (!(rope->base > 1.0))
    return fail(LCSR_EINVAL, "rope base must be > 1");
  const bool blend = (rope->flags & LCSR_ROPE_YARN_FREQ) && rope->yarn_factor > 1.0;
  if (blend && (rope->orig_max_pos <= 0 || !(rope->beta_fast > rope->beta_slow)))
    return fail(LCSR_EINVAL, "YaRN blend needs orig_max_pos > 0 and beta_fast > beta_slow");
  const int64_t half = head_dim / 2;
  const double two_pi = 6.283185307179586476925286766559;
  for (int64_t p = 0; p < half; ++p) {
    double theta = std::pow(rope->base, -2.0 * (double)p / (double)head_dim);
    if (blend) {
      // YaRN NTK-by-parts: r = turns of the pair over the training length.
      double r = (double)rope->orig_max_pos * theta / two_pi;
      double g = (r - rope->beta_slow) / (rope->beta_fast - rope->beta_slow);
      g = g < 0.0 ? 0.0 : (g > 1.0 ? 1.0 : g);
      theta = theta * ((1.0 - g) / rope->yarn_factor + g);
    }
    out->inv_freq[p] = theta;
  }
  for (int64_t p = half; p < kMaxRopeHalf; ++p) out->inv_freq[p] = 0.0;
  return LCSR_OK;
}

namespace {

// fp32 inputs are rounded to bf16 on entry, like every input of the library
__device__ __forceinline__ float load_elem(const void* base, int32_t dtype, int64_t off) {
  if (dtype == LCSR_FP32) return bf16_to_f32(f32_to_bf16(static_cast<const float*>(base)[off]));
  return bf16_to_f32(static_cast<const uint16_t*>(base)[off]);
}

// One thread per (token, pair); the angle is shared by every head.  In
// kPosDca mode the thread writes the n_var DCA query variants of its pair
// (intra, successive, inter) from one read of the input.  kTag only names
// the launch site in profiles: 0 the RoPE call, 1 the attention's query
// variants, 2 the estimate rows.
template <int kTag>
__global__ void __launch_bounds__(256) rotate_kernel(RotateArgs a, FreqTable ft, int hpb) {
  const int64_t half = a.head_dim / 2;
  const int64_t tok_per_block = 256 / half;
  const int64_t t = (int64_t)blockIdx.x * tok_per_block + threadIdx.x / half;
  const int64_t p = threadIdx.x % half;
  if (threadIdx.x >= tok_per_block * half || t >= a.n_tok) return;
  const int nv = a.mode == kPosDca ? a.n_var : 1;
  float c[3] = {1.0f, 1.0f, 1.0f}, s[3] = {0.0f, 0.0f, 0.0f};
  if (a.mode != kNoRotate) {
    for (int v = 0; v < nv; ++v) {
      int64_t pos;
      if (a.mode == kPosArray) pos = a.pos[t];
      else if (a.mode == kPosAffine) pos = t + a.pos_offset;
      else pos = dca_query_pos(t + a.pos_offset, v, a.dca);
      rope_cos_sin(pos, ft.inv_freq[p], &c[v], &s[v]);
    }
  }
  const int64_t h0 = (int64_t)blockIdx.y * hpb;
  const int64_t h1 = h0 + hpb < a.n_heads ? h0 + hpb : a.n_heads;
  for (int64_t h = h0; h < h1; ++h) {
    const int64_t so = h * a.src_sh + t * a.src_st;
    const float x1 = load_elem(a.src, a.src_dtype, so + p);
    const float x2 = load_elem(a.src, a.src_dtype, so + p + half);
    for (int v = 0; v < nv; ++v) {
      const float y1 = (x1 * c[v] - x2 * s[v]) * a.scale;
      const float y2 = (x2 * c[v] + x1 * s[v]) * a.scale;
      uint16_t* d = a.dst + v * a.dst_vs + h * a.dst_sh + t * a.dst_st;
      d[p] = f32_to_16(y1, a.dst_dtype);
      d[p + half] = f32_to_16(y2, a.dst_dtype);
    }
  }
}

// The same rotation, four pairs per thread with 8-byte loads and stores (bf16
// input, 8-byte aligned rows): pairs p0 .. p0 + 3 of one token.
template <int kTag>
__global__ void __launch_bounds__(256) rotate4_kernel(RotateArgs a, FreqTable ft, int hpb) {
  const int64_t half = a.head_dim / 2;
  const int64_t groups = half / 4;  // pair groups per token
  const int64_t tok_per_block = 256 / groups;
  const int64_t t = (int64_t)blockIdx.x * tok_per_block + threadIdx.x / groups;
  const int64_t p0 = (threadIdx.x % groups) * 4;
  if (threadIdx.x >= tok_per_block * groups || t >= a.n_tok) return;
  const int nv = a.mode == kPosDca ? a.n_var : 1;
  float c[3][4], s[3][4];
#pragma unroll
  for (int v = 0; v < 3; ++v)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      c[v][j] = 1.0f;
      s[v][j] = 0.0f;
    }
  if (a.mode != kNoRotate) {
    for (int v = 0; v < nv; ++v) {
      int64_t pos;
      if (a.mode == kPosArray) pos = a.pos[t];
      else if (a.mode == kPosAffine) pos = t + a.pos_offset;
      else pos = dca_query_pos(t + a.pos_offset, v, a.dca);
#pragma unroll
      for (int j = 0; j < 4; ++j) rope_cos_sin(pos, ft.inv_freq[p0 + j], &c[v][j], &s[v][j]);
    }
  }
  const uint16_t* src = static_cast<const uint16_t*>(a.src);
  const int64_t h0 = (int64_t)blockIdx.y * hpb;
  const int64_t h1 = h0 + hpb < a.n_heads ? h0 + hpb : a.n_heads;
  for (int64_t h = h0; h < h1; ++h) {
    const int64_t so = h * a.src_sh + t * a.src_st + p0;
    const uint2 u1 = *reinterpret_cast<const uint2*>(src + so);
    const uint2 u2 = *reinterpret_cast<const uint2*>(src + so + half);
    const float x1[4] = {__uint_as_float(u1.x << 16), __uint_as_float(u1.x & 0xFFFF0000u),
                         __uint_as_float(u1.y << 16), __uint_as_float(u1.y & 0xFFFF0000u)};
    const float x2[4] = {__uint_as_float(u2.x << 16), __uint_as_float(u2.x & 0xFFFF0000u),
                         __uint_as_float(u2.y << 16), __uint_as_float(u2.y & 0xFFFF0000u)};
    for (int v = 0; v < nv; ++v) {
      float y1[4], y2[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        y1[j] = (x1[j] * c[v][j] - x2[j] * s[v][j]) * a.scale;
        y2[j] = (x2[j] * c[v][j] + x1[j] * s[v][j]) * a.scale;
      }
      uint16_t* d = a.dst + v * a.dst_vs + h * a.dst_sh + t * a.dst_st + p0;
      const int32_t dt = a.dst_dtype;
      *reinterpret_cast<uint2*>(d) =
          make_uint2(pack_16x2(y1[0], y1[1], dt), pack_16x2(y1[2], y1[3], dt));
      *reinterpret_cast<uint2*>(d + half) =
          make_uint2(pack_16x2(y2[0], y2[1], dt), pack_16x2(y2[2], y2[3], dt));
    }
  }
}

__global__ void dca_positions_kernel(int64_t tok_start, int64_t n_tok, DcaParams d,
                                     int32_t* pk, int32_t* pi, int32_t* ps, int32_t* pn) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n_tok) return;
  const int64_t i = tok_start + t;
  if (pk) pk[t] = (int32_t)dca_key_pos(i, d);
  if (pi) pi[t] = (int32_t)dca_query_pos(i, 0, d);
  if (ps) ps[t] = (int32_t)dca_query_pos(i, 1, d);
  if (pn) pn[t] = (int32_t)dca_query_pos(i, 2, d);
}

__global__ void fill_zero_kernel(u32x4* p, int64_t n16) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n16) p[i] = (u32x4){0u, 0u, 0u, 0u};
}

}  // namespace

int launch_fill_zero(void* ptr, size_t bytes, hipStream_t s) {
  // callers pass 256-byte aligned workspace slices whose size is a multiple of 16
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return LCSR_OK;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, s,
                     static_cast<u32x4*>(ptr), n16);
  return check_launch("fill_zero");
}

namespace {
template <int kTag>
int launch_rotate_tagged(const RotateArgs& a, const FreqTable& ft, hipStream_t s) {
  if (a.n_tok == 0 || a.n_heads == 0) return LCSR_OK;
  if (a.mode == kPosDca && (a.n_var < 1 || a.n_var > 3))
    return fail(LCSR_EINVAL, "rotate: 1 to 3 DCA query variants");
  const int64_t half = a.head_dim / 2;
  // 8-byte accesses when every row start is 8-byte aligned
  const bool wide = a.src_dtype == LCSR_BF16 && a.head_dim % 8 == 0 && a.head_dim <= 256 &&
                    ((uintptr_t)a.src & 7) == 0 && ((uintptr_t)a.dst & 7) == 0 &&
                    a.src_sh % 4 == 0 && a.src_st % 4 == 0 && a.dst_sh % 4 == 0 &&
                    a.dst_st % 4 == 0 && a.dst_vs % 4 == 0;
  const int64_t tok_per_block = wide ? 256 / (half / 4) : 256 / half;
  const int64_t blocks = (a.n_tok + tok_per_block - 1) / tok_per_block;
  // heads spread over grid.y until about 2048 workgroups: a block shares its
  // cos/sin over its heads, and few tokens (a decode step) still fill the chip
  int64_t hy = (2048 + blocks - 1) / blocks;
  if (hy > a.n_heads) hy = a.n_heads;
  const int hpb = (int)((a.n_heads + hy - 1) / hy);
  hy = (a.n_heads + hpb - 1) / hpb;
  const dim3 grid((unsigned)blocks, (unsigned)hy);
  if (wide)
    hipLaunchKernelGGL(rotate4_kernel<kTag>, grid, dim3(256), 0, s, a, ft, hpb);
  else
    hipLaunchKernelGGL(rotate_kernel<kTag>, grid, dim3(256), 0, s, a, ft, hpb);
  return check_launch("rotate");
}
}  // namespace

int launch_rotate(const RotateArgs& a, const FreqTable& ft, hipStream_t s) {
  return launch_rotate_tagged<0>(a, ft, s);
}

int launch_dca_positions(int64_t tok_start, int64_t n_tok, const DcaParams& d,
                         int32_t* pk, int32_t* pi, int32_t* ps, int32_t* pn,
                         hipStream_t s) {
  if (n_tok == 0) return LCSR_OK;
  const int64_t blocks = (n_tok + 255) / 256;
  hipLaunchKernelGGL(dca_positions_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     tok_start, n_tok, d, pk, pi, ps, pn);
  return check_launch("dca_positions");
}

int launch_rotate_q_variants(const lcsr_problem_t& p, const FreqTable& ft,
                             const DcaParams& d, uint16_t* dst, int n_var,
                             hipStream_t s, bool decode) {
  const int64_t D = p.head_dim, L = p.chunk_len, H = p.n_heads;
  RotateArgs a{};
  a.src = p.q;
  a.src_dtype = p.q_dtype;
  a.src_sh = p.q_stride_h;
  a.src_st = p.q_stride_t;
  a.dst = dst;
  a.dst_dtype = LCSR_FP16;
  a.dst_vs = H * L * D;
  a.dst_sh = L * D;
  a.dst_st = D;
  a.n_heads = H;
  a.n_tok = L;
  a.head_dim = D;
  a.pos_offset = p.chunk_start;
  a.mode = kPosDca;
  a.n_var = n_var;
  a.dca = d;
  a.scale = 1.0f;
  // a separate instantiation for the decode step keeps the two apart in traces
  return decode ? launch_rotate_tagged<3>(a, ft, s) : launch_rotate_tagged<1>(a, ft, s);
}

int launch_rotate_q_estimate(const lcsr_problem_t& p, const FreqTable& ft,
                             const DcaParams& d, int64_t row0, int n_rows,
                             int n_kc, uint16_t* dst, hipStream_t s) {
  const int64_t D = p.head_dim, H = p.n_heads;
  const int64_t t0 = row0 - p.chunk_start;
  for (int c = 0; c < n_kc; ++c) {
    RotateArgs a{};
    a.src = (p.q_dtype == LCSR_FP32)
                ? (const void*)((const float*)p.q + t0 * p.q_stride_t)
                : (const void*)((const uint16_t*)p.q + t0 * p.q_stride_t);
    a.src_dtype = p.q_dtype;
    a.src_sh = p.q_stride_h;
    a.src_st = p.q_stride_t;
    a.dst = dst + (int64_t)c * H * kEstRows * D;
    a.dst_dtype = LCSR_FP16;
    a.dst_sh = (int64_t)kEstRows * D;
    a.dst_st = D;
    a.n_heads = H;
    a.n_tok = n_rows;
    a.head_dim = D;
    a.pos_offset = row0 - (int64_t)c * d.period;
    a.mode = kPosAffine;
    a.scale = 1.0f;
    int rc = launch_rotate_tagged<2>(a, ft, s);
    if (rc) return rc;
  }
  return LCSR_OK;
}

}  // namespace lcsr
