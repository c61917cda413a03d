// noalloc.hip -- decode attention for callers that cannot allocate device
// memory (work under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  milo_attn_decode_noalloc is milo_attn_decode with the
// split-K partials of its work units in a library-owned static device buffer
// instead of the caller's workspace; the kernels are the same.
//
// The buffer is a file-scope __device__ array: every GPU the library runs on
// holds its own copy, at its own address, from the code object's load until
// the process ends.  In host code the array's name is only a stand-in for
// the symbol, so its device address is resolved with hipGetSymbolAddress
// once per device (on the entry point's first call with that device
// current) and that address is what the kernels receive.  Every call on a
// GPU uses that GPU's one copy: calls that overlap on one GPU (concurrent
// streams, or threads) race on it.  Nothing in it needs clearing: the merge
// reads exactly the partial records the decode kernel writes in the same
// call.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"
#include "milo_attn.h"

namespace {

constexpr size_t kScratchBytes = MILO_NOALLOC_SCRATCH_BYTES;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device

// The current device's copy of `scratch` (resolved on first use).
milo_status current_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MILO_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return MILO_ERR_DEVICE;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MILO_OK;
}

}  // namespace

extern "C" milo_status milo_attn_decode_noalloc(const milo_attn_args* a, void* hip_stream) {
  size_t need = 0;
  milo_status st = milo::decode_check(a, &need);
  if (st != MILO_OK) return st;
  if (a->batch == 0) return MILO_OK;
  if (need > kScratchBytes) return MILO_ERR_WORKSPACE;
  void* ws = nullptr;
  st = current_scratch(&ws);
  if (st != MILO_OK) return st;
  return milo::decode_launch(a, ws, hip_stream);
}
