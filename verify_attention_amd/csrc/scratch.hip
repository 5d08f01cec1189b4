// The library-owned scratch array of the allocation-free entry points
// (spec_accept_static): a fixed-size device array, one copy per GPU, kept for
// the life of the process. Every call on a GPU shares that GPU's copy, so
// calls that overlap on one GPU (unordered streams) race on it; nothing in it
// has to start at zero (the accept's first kernel writes every entry its
// second kernel reads).
#include <mutex>

#include "specattn.h"
#include "kernels.h"

namespace specattn {

namespace {

__device__ __align__(256) unsigned char scratch[SPEC_ACCEPT_STATIC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;

struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t status = hipSuccess;
};
ScratchSlot g_slots[kMaxScratchDevices];

}  // namespace

// Device address of the current GPU's copy of `scratch`, looked up once per
// device with that device current. In host code the array's name is only a
// host-side handle, never a device address: kernels are given this pointer.
hipError_t scratch_on_current_device(void** out, size_t* bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  ScratchSlot& slot = g_slots[dev];
  std::call_once(slot.once, [&slot] {
    slot.status = hipGetSymbolAddress(&slot.ptr, HIP_SYMBOL(scratch));
    if (slot.status == hipSuccess && !slot.ptr) slot.status = hipErrorInvalidSymbol;
  });
  if (slot.status != hipSuccess) return slot.status;
  *out = slot.ptr;
  *bytes = sizeof(scratch);
  return hipSuccess;
}

}  // namespace specattn
