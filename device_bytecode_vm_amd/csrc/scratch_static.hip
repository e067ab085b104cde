// A fixed reduce-all scratch area in device memory, for callers that cannot
// allocate (code under HIP graph capture, serving loops, harnesses that
// forbid hipMalloc): dvm_launch_noalloc runs reduce-all programs on it.
//
// The area is a file-scope device array: each GPU the library runs on holds
// its own copy, at its own address, until the process ends.  Host code never
// passes the array's name to a kernel (on the host that name is only a
// stand-in); it looks the device address up once per device, with that device
// current, and passes that address instead.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

// the per-workgroup partials from byte 256 (the first 256 bytes are spare):
// 65536 of them
constexpr size_t DVM_STATIC_SCRATCH_BYTES = 256 + 4 * 65536;

static __device__ __align__(256) unsigned char scratch[DVM_STATIC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void* g_ptr[MAX_DEVICES];
hipError_t g_err[MAX_DEVICES];
bool g_done[MAX_DEVICES];
}  // namespace

// Device address of the array on `device`, which must be the current device.
// Looked up once per device; later calls return the cached address.
extern "C" hipError_t dvm_static_scratch_init(int device, void** ptr, size_t* bytes) {
  *ptr = nullptr;
  *bytes = DVM_STATIC_SCRATCH_BYTES;
  if (device < 0 || device >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_done[device]) {
    void* p = nullptr;
    g_err[device] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[device] = g_err[device] == hipSuccess ? p : nullptr;
    g_done[device] = true;
  }
  *ptr = g_ptr[device];
  return g_err[device];
}
