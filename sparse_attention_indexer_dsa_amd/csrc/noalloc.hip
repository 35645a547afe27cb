// Fixed device scratch for the scoring + selection entry point that allocates nothing
// (dsa_index_score_topk_noalloc).
//
// The score rows that dsa_index_score_topk keeps in the caller's workspace live here in a
// file-scope device array of kNoAllocScratchBytes per GPU, held from the time the library's
// code object is loaded on a device until the process ends. Host code never passes the
// array's name to a kernel or a copy (in host code the name is only a stand-in, not a device
// address): on the first call on a device, with that device current, its address is looked
// up once and kept per device, and that address is what the kernels receive.
//
// Every call on a GPU shares that GPU's array, which keeps the last call's contents. Nothing
// in it needs to start at zero: the scoring kernel writes every candidate slot of a row
// before the selection kernel (ordered after it on the same stream) reads it, and the
// selection reads no other slot. Calls that overlap on one GPU (on different streams, or
// from different host threads without ordering) race on the array.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"

static __device__ __align__(256) uint8_t scratch[dsa::kNoAllocScratchBytes];

namespace dsa {

hipError_t noalloc_scratch(void** out) {
  constexpr int kDevices = 64;
  static std::mutex mu;
  static void* addr[kDevices] = {};
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return e;
  if (device < 0 || device >= kDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[device] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[device] = p;
  }
  *out = addr[device];
  return hipSuccess;
}

}  // namespace dsa
