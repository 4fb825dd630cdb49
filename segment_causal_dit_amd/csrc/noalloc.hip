// Allocation-free form of the packed-form attention backward, for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).
//
// The backward needs one scratch buffer beside its inputs and outputs: delta,
// fp32 [n_heads][n], written by the first kernel and read by the other two.
// Here it lives in a file-scope device array of kScratchFloats entries
// (32 MiB), which each GPU the library runs on holds until the process ends.
// Its device address is taken once per device, with that device current, on
// the entry point's first call there; the kernels then receive that address.
// Every call on a GPU shares the GPU's array, so calls that overlap on one GPU
// (other streams, other host threads) race; the array needs no clearing:
// delta is written in full before it is read.
#include <mutex>

#include "internal.h"

namespace {

constexpr int64_t kScratchFloats = (int64_t)1 << 23;   // delta entries: n x n_heads <= 2^23
constexpr int kMaxDevices = 64;

std::mutex g_mutex;
float* g_scratch[kMaxDevices] = {};   // device address of `scratch`, per device

}  // namespace

static __device__ __align__(256) float scratch[kScratchFloats];

extern "C" int segcausal_joint_attn_bwd_noalloc(const segc_attn_bwd_args* a, void* stream) {
  if (!a) return segc::report(SEGC_EINVAL, "args is NULL");
  // n <= 0: refused (n < 0) or a no-op, by the shared checks, before any device access
  if (a->n <= 0) return segc::attn_bwd_checked(a, nullptr, stream);
  if (a->n > 0 && a->n_heads > 0 && a->n * (int64_t)a->n_heads > kScratchFloats)
    return segc::report(SEGC_EINVAL,
                        "n x n_heads exceeds the 2^23 delta entries of the allocation-free scratch");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return segc::report(SEGC_EHIP, hipGetErrorString(e));
  }
  if (dev < 0 || dev >= kMaxDevices) return segc::report(SEGC_EUNSUPPORTED, "device index beyond 63");
  float* ptr = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_scratch[dev]) {
      void* sym = nullptr;
      e = hipGetSymbolAddress(&sym, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !sym) {
        (void)hipGetLastError();
        return segc::report(SEGC_EHIP, e != hipSuccess ? hipGetErrorString(e) : "scratch has no device address");
      }
      g_scratch[dev] = (float*)sym;
    }
    ptr = g_scratch[dev];
  }
  return segc::attn_bwd_checked(a, ptr, stream);
}
