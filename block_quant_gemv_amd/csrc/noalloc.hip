// Fixed device scratch for the entry point that allocates nothing.
//
// Callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc) still need the GEMV
// workspace: the quantized activations, their scales and block sums, and
// for the batched path the token-tiled codes and K-split partial sums. This
// file holds that workspace as one file-scope device array. Every GPU the
// library runs on holds its own copy of the array for the life of the
// process; the host reaches it only through the address hipGetSymbolAddress
// returns with that device current (the array's name in host code is a
// host-side stand-in, not a device address).
//
// Every call on one GPU shares that GPU's array and leaves its contents
// behind; nothing in it needs to start at zero (each region is fully written
// before it is read within a call). Calls that overlap on one GPU (two
// streams, two threads) race on the array.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>

#include "internal.h"

namespace qg {

namespace {

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

struct ScratchTable {
  std::mutex mu;
  std::map<int, void*> ptr;  // device -> address of that device's copy of `scratch`
};

ScratchTable& table() {
  static ScratchTable t;
  return t;
}

}  // namespace

hipError_t noalloc_scratch(void** out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  ScratchTable& t = table();
  std::lock_guard<std::mutex> g(t.mu);
  auto it = t.ptr.find(dev);
  if (it != t.ptr.end()) {
    *out = it->second;
    return hipSuccess;
  }
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with `dev` current: its copy
  if (e != hipSuccess) return e;
  if (!p) return hipErrorInvalidSymbol;
  t.ptr[dev] = p;
  *out = p;
  return hipSuccess;
}

}  // namespace qg
