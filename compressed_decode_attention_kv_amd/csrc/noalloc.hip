// Library-owned decode workspace for tq_decode_attention_static: callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation) get the decode's workspace from a
// file-scope device array instead of a buffer of their own.
//
// Each device that loads the library holds its own copy of the array, at its
// own address, until the process ends.  Host code never passes the array's
// name to a kernel or a copy: on the host that name is only a stand-in.  The
// device address comes from hipGetSymbolAddress, taken once per device (with
// that device current) on the entry point's first call there, and kept.
#include <map>
#include <mutex>

#include "internal.h"

namespace tq {
namespace {

constexpr size_t kStaticScratchBytes = size_t(64) << 20;

static __device__ __align__(256) char scratch[kStaticScratchBytes];

std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_ptr;  // device -> address of that device's copy

}  // namespace

size_t static_scratch_bytes() { return kStaticScratchBytes; }

hipError_t static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it != g_scratch_ptr.end()) {
    *out = it->second;
    return hipSuccess;
  }
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  g_scratch_ptr[dev] = p;
  *out = p;
  return hipSuccess;
}

}  // namespace tq
