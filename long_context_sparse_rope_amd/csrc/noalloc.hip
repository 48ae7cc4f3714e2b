// The decode step on a library-owned scratch buffer: lcsr_attn_decode for
// callers that cannot allocate device memory (code under HIP graph capture,
// serving loops that forbid allocation).
//
// The workspace of lcsr_attn_decode (rotated query variants, per-split
// partial outputs and (m, l) pairs) lives in one file-scope device array per
// GPU.  Its size bounds every valid decode problem: with G x n_q <= 32 matrix
// rows per KV head, n_heads <= 64 and head_dim <= 128, the partials of at
// most 256 + H_kv - 1 <= 319 (KV head, split) workgroups take 319 x 32 x
// (128 + 2) x 4 bytes and the three query variants of at most 32 x H_kv <=
// 2048 rows take 3 x 2048 x 128 x 2 bytes, under 7 MB in all.
//
// The device address of the array is looked up once per device with
// hipGetSymbolAddress (the array's name in host code is only a stand-in) and
// kept for later calls.  Every split writes every partial it owns before the
// combine reads it, so nothing needs clearing between calls.  Calls on one
// GPU share the array: calls that may overlap on one GPU (different streams)
// race on it and must be serialised by the caller.
#include <mutex>

#include "lcsr_internal.h"

namespace lcsr {

namespace {

constexpr size_t kScratchBytes = size_t(8) << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address (looked up on its first use).
int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(LCSR_EHIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(LCSR_ENOTSUP, "device %d beyond the %d supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(LCSR_EHIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return LCSR_OK;
}

}  // namespace

}  // namespace lcsr

using namespace lcsr;

extern "C" int lcsr_attn_decode_noalloc(const lcsr_problem_t* p, void* out, int32_t out_dtype,
                                        int64_t o_stride_h, int64_t o_stride_t, float* lse,
                                        void* stream) {
  // validation only: without a workspace lcsr_attn_decode returns its own
  // status for an invalid problem, else LCSR_EWORKSPACE, before any launch
  int rc = lcsr_attn_decode(p, out, out_dtype, o_stride_h, o_stride_t, lse, nullptr, 0, stream);
  if (rc != LCSR_EWORKSPACE) return rc;
  const size_t need = lcsr_workspace_bytes(LCSR_WS_DECODE, p, 0, 0);
  if (need == 0 || need > kScratchBytes)
    return fail(LCSR_ENOTSUP, "decode needs %zu bytes of scratch; the static scratch holds %zu",
                need, kScratchBytes);
  void* ws = nullptr;
  rc = scratch_address(&ws);
  if (rc) return rc;
  return lcsr_attn_decode(p, out, out_dtype, o_stride_h, o_stride_t, lse, ws, kScratchBytes,
                          stream);
}
