// Static device workspace of muon_step_noalloc, the entry point for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).
//
// `scratch` is a file-scope device array of MUON_STATIC_WORKSPACE_BYTES; each
// GPU that uses it holds its own copy until the process ends. In host code
// its name is only a stand-in for the symbol, not a device address: the
// address is taken once per device with hipGetSymbolAddress (with that
// device current) and kept, and only that address is ever passed to kernels.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>

#include "kernels.h"
#include "muon.h"

namespace muon {
namespace {

static __device__ __align__(256) unsigned char scratch[MUON_STATIC_WORKSPACE_BYTES];

std::mutex g_mu;
std::map<int, void*> g_ptr;   // device -> address of that device's scratch

}  // namespace

hipError_t static_workspace(void** ptr, size_t* bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_ptr.find(dev);
  if (it == g_ptr.end()) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    it = g_ptr.emplace(dev, p).first;
  }
  *ptr = it->second;
  *bytes = MUON_STATIC_WORKSPACE_BYTES;
  return hipSuccess;
}

}  // namespace muon
