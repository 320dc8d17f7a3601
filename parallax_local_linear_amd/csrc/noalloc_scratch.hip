// Fixed device scratch of the allocation-free decode entry point
// (parallax_decode_noalloc): the split records of one call live in a
// file-scope device array instead of a caller or library workspace.  Every
// device the library runs on holds its own copy of the array for the life of
// the process.  In host code the array's name only stands for the symbol; the
// device address of the current device's copy comes from hipGetSymbolAddress,
// looked up once per device with that device current and kept.

#include <hip/hip_runtime.h>

#include <mutex>

namespace plx {

constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_slots[kMaxDevices];
}  // namespace

size_t noalloc_scratch_bytes() { return kNoAllocScratchBytes; }

// Device address of the current device's scratch in *ptr.  hipErrorInvalidDevice
// for a device index past those tracked; the lookup's own error otherwise.
hipError_t noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  ScratchSlot& sl = g_slots[dev];
  std::call_once(sl.once, [&sl]() {
    void* p = nullptr;
    sl.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (sl.err == hipSuccess) sl.ptr = p;
  });
  if (!sl.ptr) return sl.err != hipSuccess ? sl.err : hipErrorUnknown;
  *ptr = sl.ptr;
  return hipSuccess;
}

}  // namespace plx
