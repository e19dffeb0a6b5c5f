// The library's own device scratch for callers that cannot allocate (code
// under graph capture, tight serving loops, harnesses that forbid
// allocation): a fixed-size array in the code object's device memory,
// taking the place of a caller-provided workspace.
//
// Each GPU the library runs on holds its own copy of the array, at its own
// address, from module load until the process ends.  Host code never uses
// the array's name as an address (that is a host-side stand-in); it uses
// the device address hipGetSymbolAddress returns, fetched once per device
// with that device current and kept per device.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kq_launch.hpp"

static __device__ __align__(256) char scratch[kq::kScratchBytes];

namespace kq {

void* scratch_address(hipError_t* err) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *err = e != hipSuccess ? e : hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return nullptr;
    }
    addr[dev] = p;
  }
  *err = hipSuccess;
  return addr[dev];
}

}  // namespace kq
