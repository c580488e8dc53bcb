// Scratch for the allocation-free entry point (topk_ragged_noalloc): a
// file-scope device array that stands in for the caller's workspace, for
// callers that cannot allocate device memory.  Each GPU the library runs on
// holds its own copy of the array until the process ends.
//
// In host code the array's name is only a host-side stand-in for the
// symbol; the device address of each GPU's copy comes from
// hipGetSymbolAddress, called once per device with that device current, and
// only that address is ever handed to kernels.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <mutex>

#include "topk_internal.h"

namespace rrt {

static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

struct ScratchSlot {
  std::atomic<void*> ptr{nullptr};  // device address of this device's copy, once set up
};

ScratchSlot g_slots[kMaxDevices];
std::mutex g_setup_mu;

}  // namespace

// Device address of `dev`'s scratch.  The first call for a device looks the
// address up (with that device current) and queues a fill kernel that zeroes
// the whole array on `stream`, ahead of the caller's launch on the same
// stream; kernels leave the array all-zero again when they end.  No
// allocation.  Returns 0 or a HIP error code; *msg names the failing step.
int noalloc_scratch(int dev, hipStream_t stream, void** out, const char** msg) {
  *msg = "";
  if (dev < 0 || dev >= kMaxDevices) {
    *msg = "device ordinal beyond the scratch table";
    return (int)hipErrorInvalidDevice;
  }
  void* p = g_slots[dev].ptr.load(std::memory_order_acquire);
  if (p != nullptr) {
    *out = p;
    return 0;
  }
  std::lock_guard<std::mutex> lk(g_setup_mu);
  p = g_slots[dev].ptr.load(std::memory_order_relaxed);
  if (p == nullptr) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    void* addr = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (cur >= 0 && cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || addr == nullptr) {
      *msg = "hipGetSymbolAddress of the scratch array failed";
      return e != hipSuccess ? (int)e : (int)hipErrorInvalidSymbol;
    }
    // One-time zero fill (a kernel, not a memset node), ordered before the
    // caller's launch on the same stream.
    uint32_t* words = static_cast<uint32_t*>(addr);
    uint64_t n = kNoallocScratchBytes / 4;
    void* args[] = {&words, &n};
    e = hipLaunchKernel(zero_kernel_ptr(), dim3(1024), dim3(256), args, 0, stream);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) {
      *msg = "zeroing the scratch array failed";
      return (int)e;
    }
    p = addr;
    g_slots[dev].ptr.store(p, std::memory_order_release);
  }
  *out = p;
  return 0;
}

}  // namespace rrt
