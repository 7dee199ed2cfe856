// q4_awq_search_static: the activation-aware search of q4_awq_search with its device scratch in
// a file-scope device array instead of a caller's workspace, for callers that cannot allocate
// (code under stream capture, serving loops that forbid allocation).  No allocation happens on
// any call: the array is part of the library's code object, one copy per GPU, held until the
// process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: its device address is
// taken once per device with hipGetSymbolAddress (with that device current) and only that
// address is handed to the kernels.  The search writes every scratch word it reads in the same
// call (partial sums included), so nothing needs clearing between calls; calls that overlap on
// one GPU share the array and race.
#include "../../include/q4.h"
#include "q4_device.h"
#include "q4_internal.h"

#include <mutex>

namespace q4 {
namespace {

constexpr int64_t kScratchBytes = int64_t(64) << 20;       // 64 MiB per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`, or nullptr if HIP cannot name it.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    scratch_ptr[dev] = p;
  }
  return scratch_ptr[dev];
}

}  // namespace
}  // namespace q4

extern "C" int64_t q4_awq_static_scratch_bytes(void) { return q4::kScratchBytes; }

extern "C" int q4_awq_search_static(const void* X, int64_t M, const void* Yref, const void* W, int64_t N,
                                    int64_t K, int32_t g, int32_t mode, int32_t n_alpha, void* s_out,
                                    void* packed, void* scales, void* zeros, void* errors, void* best,
                                    void* stream) {
  const int64_t need = q4_awq_workspace_bytes(M, N, K, g, n_alpha);
  if (need < 0) return (int)need;                       // the shape errors of q4_awq_search
  if (need > q4::kScratchBytes) return Q4_ERR_SCRATCH;  // checked before any HIP call
  void* p = q4::scratch_on_current_device();
  if (p == nullptr) return Q4_ERR_HIP;
  return q4_awq_search(X, M, Yref, W, N, K, g, mode, n_alpha, p, q4::kScratchBytes, s_out, packed, scales,
                       zeros, errors, best, stream);
}
