// rlk_linear_logp_noalloc: the fused forward for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).  The kernels and results are those of
// rlk_linear_logp; only the workspace differs: the chunk partials and target
// logits live in `scratch`, a file-scope device array of fixed size.
//
// Each GPU the library runs on holds its own copy of `scratch` until the
// process ends.  In host code the name is a stand-in for the symbol, not a
// device address: the address is looked up once per device with
// hipGetSymbolAddress (that device current) and kept, and only that address
// is handed to the kernels.  Every call on a GPU shares its copy, so calls
// that overlap in time on one GPU race; nothing in it needs clearing between
// calls, since every byte the kernels read is written earlier in the same
// call.  No hipMalloc, hipFree or allocating routine is called here.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "rlk.h"
#include "rlk_internal.hpp"

namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;  // 32 MiB per GPU
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, or null if the lookup
// fails; looked up on the first call on each device.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" int rlk_linear_logp_noalloc(const void* hidden, int64_t ld_h, const void* weight,
                                       int64_t ld_w, const int64_t* targets, const uint8_t* mask,
                                       int64_t N, int64_t V, int64_t H, float* logp, float* lse,
                                       hipStream_t stream) {
  const int st = rlk::check_linear_logp_args(hidden, ld_h, weight, ld_w, targets, logp, N, V, H);
  if (st != RLK_OK || N == 0) return st;
  if (rlk::linear_workspace_bytes(N, V) > kScratchBytes) return RLK_ERR_UNSUPPORTED;
  void* ws = device_scratch();
  if (ws == nullptr) return RLK_ERR_LAUNCH;
  const hipError_t e = rlk::launch_linear_logp(
      static_cast<const uint16_t*>(hidden), ld_h, static_cast<const uint16_t*>(weight), ld_w,
      targets, mask, N, static_cast<int>(V), static_cast<int>(H), logp, lse, nullptr, 0, ws, stream);
  return e == hipSuccess ? RLK_OK : RLK_ERR_LAUNCH;
}
