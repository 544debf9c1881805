// Library-held scratch memory of qa_decode_noalloc.
//
// For callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc), decode's
// split-K partials and in-launch merge counters live in one file-scope
// device array per GPU instead of a caller workspace.  In host code the
// array's name is only a host-side stand-in, so its device address is looked
// up once per device with hipGetSymbolAddress and that address is what the
// kernels receive.  On that first use the array is cleared with the fill
// kernel (the merge counters must start at zero; every decode call returns
// them to zero).  All calls on one GPU share its array: calls that overlap
// on one GPU race.
#include <mutex>

#include "qa_device.h"

namespace qa {

constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
constexpr int kNoAllocMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
std::mutex g_mu;
void* g_ptr[kNoAllocMaxDevices];
}  // namespace

size_t noalloc_scratch_bytes() { return kNoAllocScratchBytes; }

// The current device's scratch address.  Until a clear has run eagerly on
// that device, each call enqueues the fill kernel on its stream first: a
// call captured into a graph then carries the clear with it, and the first
// eager call clears the array once for good.
hipError_t noalloc_scratch(void** out, hipStream_t s) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kNoAllocMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(s, &cap);
    if (e != hipSuccess) return e;
    e = launch_fill_zero(p, kNoAllocScratchBytes, s);
    if (e != hipSuccess) return e;
    if (cap != hipStreamCaptureStatusNone) {
      *out = p;
      return hipSuccess;
    }
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace qa
