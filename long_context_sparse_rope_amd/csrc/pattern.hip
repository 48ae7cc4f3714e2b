// Fixed head patterns written into a vertical-slash pattern (gfx950).
//
// [architecture overview] §4.1: a StreamingLLM head keeps the first few
// tokens (attention sinks) and a window of the most recent ones; MInference
// names this head pattern "A-shape".  Under the vertical-slash rule the
// sinks are the vertical columns 0 .. n_sink - 1 and the window is the slash
// offsets 0 .. n_local - 1, so these heads run through the same estimate-free
// attention as the others.
#include "lcsr_internal.h"

namespace lcsr {
namespace {

// grid (ceil(max(max_vert, max_slash) / 256), n_heads); a block of an
// unselected head returns at once.
__global__ void __launch_bounds__(256) fill_a_shape_kernel(lcsr_pattern_t pat, uint64_t mask,
                                                           int32_t nv, int32_t ns) {
  const int h = blockIdx.y;
  if (!((mask >> h) & 1ull)) return;
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t < pat.max_vert) pat.vert_idx[(int64_t)h * pat.max_vert + t] = t < nv ? t : -1;
  if (t < pat.max_slash) pat.slash_idx[(int64_t)h * pat.max_slash + t] = t < ns ? t : -1;
  if (t == 0) {
    pat.vert_cnt[h] = nv;
    pat.slash_cnt[h] = ns;
  }
}

}  // namespace

int launch_fill_a_shape(const lcsr_pattern_t& pat, int32_t n_heads, uint64_t mask,
                        int32_t nv, int32_t ns, hipStream_t s) {
  if (!mask) return LCSR_OK;
  const int32_t width = pat.max_vert > pat.max_slash ? pat.max_vert : pat.max_slash;
  const unsigned bx = (unsigned)((width + 255) / 256 > 0 ? (width + 255) / 256 : 1);
  hipLaunchKernelGGL(fill_a_shape_kernel, dim3(bx, (unsigned)n_heads), dim3(256), 0, s, pat,
                     mask, nv, ns);
  return check_launch("fill a-shape");
}

}  // namespace lcsr
