// Fixed device buffer of the allocation-free descriptor builder
// (pva_seg_desc_build_noalloc): the work list and per-row key limits of the
// most recent such descriptor of each device live in a file-scope device
// array instead of a hipMalloc'ed buffer, for callers that cannot allocate.
//
// In host code the array's name stands for a host-side shadow, not a device
// address: its device address is taken once per device with
// hipGetSymbolAddress (that device current) and only that address is handed
// to copies and kernels. Each device holds its own copy of the array at its
// own address until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "pva_internal.h"

namespace pva {

namespace {

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;

struct DeviceScratch {
  void* ptr = nullptr;      // device address of `scratch` on this device
  uint64_t generation = 0;  // bumped by every acquisition; 0: never used
};

std::mutex g_mu;
DeviceScratch g_devices[kMaxDevices];

}  // namespace

int scratch_acquire(int device, size_t bytes, void** ptr, uint64_t* generation, std::string* err) {
  if (device < 0 || device >= kMaxDevices) {
    *err = "device index " + std::to_string(device) + " out of range for the no-alloc buffer";
    return PVA_ERR_UNSUPPORTED;
  }
  if (bytes > kNoAllocScratchBytes) {
    *err = "the work list and key limits need " + std::to_string(bytes) + " bytes; the no-alloc buffer holds " +
           std::to_string(kNoAllocScratchBytes) + " (PVA_NOALLOC_SCRATCH_BYTES): use pva_seg_desc_build";
    return PVA_ERR_INVALID_ARG;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceScratch& d = g_devices[device];
  if (d.ptr == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      *err = std::string("hipGetSymbolAddress of the no-alloc buffer: ") + hipGetErrorString(e);
      return PVA_ERR_HIP;
    }
    d.ptr = p;
  }
  *ptr = d.ptr;
  *generation = ++d.generation;
  return PVA_OK;
}

bool scratch_is_current(int device, uint64_t generation) {
  if (device < 0 || device >= kMaxDevices) return false;
  std::lock_guard<std::mutex> lock(g_mu);
  return g_devices[device].generation == generation;
}

}  // namespace pva
