// static_scratch.hip - the workspace of the allocation-free entry point.
//
// verify_attn_run_static serves callers that cannot allocate device memory (code under stream
// capture, tight serving loops, harnesses that forbid it). Its workspace is the file-scope
// array below: it is part of the library's code object, so the library neither allocates nor
// frees it, and every GPU the library runs on holds its own copy until the process ends.
//
// Host code never uses the array's name as a device address (on the host it names a stand-in
// object). On its first call on a device, with that device current, static_scratch() asks the
// runtime for the array's address on that device (hipGetSymbolAddress) and keeps it; every
// launch then takes that address.
//
// Every call on one GPU shares that GPU's array, which keeps the previous call's contents:
// the kernels rewrite every partial they read in the same call, and the only region that must
// hold zeros (the row that unusable keys load, in the header) is never written by a kernel.
// Calls that overlap in time on one GPU race on the array.
#include <atomic>
#include <mutex>

#include "va_internal.h"

namespace va {
namespace {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device
std::mutex g_setup_mutex;

// Zeroes n words: clears the header (status words and the zero row) once per device. A kernel
// rather than a memset, so that a first call recorded into a graph records an ordinary node.
__global__ void __launch_bounds__(256) clear_words(uint32_t *p, int n) {
  for (int i = int(threadIdx.x); i < n; i += int(blockDim.x)) p[i] = 0u;
}

}  // namespace

hipError_t static_scratch(hipStream_t stream, void **base) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_setup_mutex);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      static_assert(kHeaderBytes % 4 == 0, "the header is whole words");
      hipLaunchKernelGGL(clear_words, dim3(1), dim3(256), 0, stream, static_cast<uint32_t *>(p),
                         int(kHeaderBytes / 4));
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *base = p;
  return hipSuccess;
}

}  // namespace va
