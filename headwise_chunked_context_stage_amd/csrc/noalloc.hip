// noalloc.hip -- the forward without a workspace argument, for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).
//
// The stage buffers live in `scratch`, a static device array of kScratchBytes
// that each GPU the library runs on holds until the process ends.  Host code
// never passes the array's name to a kernel (on the host it is a stand-in,
// not a device address): the first call on a device takes the address of
// that device's copy with hipGetSymbolAddress, with the device current, and
// every call passes that address on as the workspace of upipe_fwd, which then
// runs exactly the kernels it runs with a caller's workspace.
//
// Nothing in the forward's workspace has to start at zero: every region is
// written by the stage's projection before the attention reads it, so the
// contents a previous call left are never read.  All calls on one GPU share
// its array: calls that overlap in time on one GPU (two streams, two host
// threads) race on it.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>

#include "upipe_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(256) << 20;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_ptr;  // device -> its copy of `scratch`

// Address of the current device's copy of `scratch` (taken once per device).
hipError_t scratch_on(int dev, void** out) {
  std::lock_guard<std::mutex> g(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it != g_scratch_ptr.end()) {
    *out = it->second;
    return hipSuccess;
  }
  void* ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (ptr == nullptr) return hipErrorInvalidSymbol;
  g_scratch_ptr[dev] = ptr;
  *out = ptr;
  return hipSuccess;
}

}  // namespace

extern "C" {

size_t upipe_noalloc_max_bytes(void) { return kScratchBytes; }

int upipe_fwd_noalloc(const upipe_plan* h, const void* X, const void* Wq, const void* Wk,
                      const void* Wv, void* O, float* LSE, void* stream) {
  if (!h) return UPIPE_ERR_ARG;
  const upipe::Plan& p = h->p;
  if (p.pipeline) return UPIPE_ERR_ARG;  // its helper stream and events are created on demand
  if (p.ws.fwd_bytes > kScratchBytes) return UPIPE_ERR_WORKSPACE;
  if (p.S == 0) return UPIPE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int dev = -1, sdev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return UPIPE_ERR_HIP;
  // the scratch address is the current device's: the stream must be on it
  if (s != nullptr) {
    if (hipStreamGetDevice(s, &sdev) != hipSuccess) return UPIPE_ERR_HIP;
    if (sdev != dev) return UPIPE_ERR_ARG;
  }
  void* ws = nullptr;
  if (scratch_on(dev, &ws) != hipSuccess) return UPIPE_ERR_HIP;
  return upipe_fwd(h, X, Wq, Wk, Wv, O, LSE, ws, kScratchBytes, stream);
}

}  // extern "C"
