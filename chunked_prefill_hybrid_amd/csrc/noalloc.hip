// The fixed device scratch of the no-allocation layer forward.
//
// The array below lives in every GPU's copy of the library's code object from the moment the module
// is loaded until the process ends; a forward that may not allocate (a caller capturing a graph, a
// serving loop or a harness that forbids device allocation) uses it as its workspace.  In host code
// the array's name is only a host-side stand-in: its device address is looked up once per device,
// with that device current, and only that address is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "kernels.h"

namespace sarathi {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_mutex;

}  // namespace

hipError_t noalloc_scratch(int device, void **out) {
  *out = nullptr;
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  void *p = g_scratch[device].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch[device].load(std::memory_order_relaxed);
    if (!p) {
      int current = -1;
      hipError_t e = hipGetDevice(&current);
      if (e != hipSuccess) return e;
      if (current != device) return hipErrorInvalidDevice;   // each device's copy is found with it current
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch[device].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace sarathi
