// The static device scratch behind mla_decode_mxfp4_noalloc: plan words and
// split-K partials of that entry point live in one file-scope device array
// instead of a caller-supplied workspace, for callers that cannot allocate.
//
// Each device that loads the library holds its own copy of the array, at
// its own address, until the process ends. Host code never passes the
// array's name to a kernel (on the host it only stands for the symbol):
// the device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and that address is what
// the planner and decode kernels receive.
#include <hip/hip_runtime.h>

#include <mutex>
#include <unordered_map>

#include "mla_internal.h"

namespace mla {
namespace {

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
std::unordered_map<int, void*> g_scratch_ptr;   // device -> address of its copy of `scratch`

}  // namespace

int noalloc_scratch(int device, void** ptr) {
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  auto it = g_scratch_ptr.find(device);
  if (it != g_scratch_ptr.end()) {
    *ptr = it->second;
    return (int)hipSuccess;
  }
  // the caller has made `device` current
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return (int)e;
  if (p == nullptr || ((uintptr_t)p % kAlignBytes) != 0) return (int)hipErrorInvalidSymbol;
  g_scratch_ptr[device] = p;
  *ptr = p;
  return (int)hipSuccess;
}

}  // namespace mla
