// fa_noalloc.hip -- fa_bwd_noalloc: fa_bwd with the library's own static
// device scratch in place of a caller-provided workspace, for callers that
// cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid allocation).
//
// The scratch is one file-scope __device__ array per GPU, held until the
// process ends.  In host code its name is only a handle for the runtime: its
// device address on the current GPU comes from hipGetSymbolAddress, taken
// once per device and kept, and only that address is ever passed to kernels.
// Every call on one GPU shares that GPU's array: calls that overlap on one
// GPU (other streams, other threads) race on it.  Nothing in it has to start
// at zero: Delta and the FP32 partial sums are fully written before they are
// read within each call.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fa.h"
#include "fa_launch.hpp"

namespace {

constexpr size_t kScratchBytes = FA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of this GPU's scratch array; `dev` is current on entry.
int scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return FA_ERR_HIP;
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess || g_scratch_ptr[dev] == nullptr) return FA_ERR_HIP;
  *out = g_scratch_ptr[dev];
  return FA_OK;
}

}  // namespace

extern "C" int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                              const void* dout, void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t N,
                              int64_t D, int causal, float scale, int dtype, void* stream) {
  int st = fa::check_bwd_args(q, k, v, o, lse, dout, dq, dk, dv, B, H, H, N, D, causal, scale, dtype);
  if (st != FA_OK) return st;
  const size_t need = fa_bwd_workspace_bytes(B, H, N, D, causal, dtype);
  if (need > kScratchBytes) return FA_ERR_SCRATCH_LIMIT;
  // The scratch of the GPU the stream belongs to (the current one for the
  // null stream), looked up with that GPU current.
  int cur = 0, dev = 0;
  if (hipGetDevice(&cur) != hipSuccess) return FA_ERR_HIP;
  dev = cur;
  if (stream != nullptr && hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) != hipSuccess)
    return FA_ERR_HIP;
  void* ws = nullptr;
  if (dev != cur) {
    if (hipSetDevice(dev) != hipSuccess) return FA_ERR_HIP;
    st = scratch_address(dev, &ws);
    if (hipSetDevice(cur) != hipSuccess) return FA_ERR_HIP;
  } else {
    st = scratch_address(dev, &ws);
  }
  if (st != FA_OK) return st;
  return fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, D, causal, scale, dtype, ws, kScratchBytes, stream);
}
