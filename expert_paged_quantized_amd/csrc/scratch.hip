// Static device scratch of the no-allocation forward (strata_moe_forward_noalloc):
// one file-scope array in the library's code object, so a forward can run
// without any device allocation.  Each GPU the library is loaded on holds its
// own copy of the array until the process ends.  Host code never uses the
// array's name as an address (on the host it is only a stand-in for the
// symbol): the device address of each GPU's copy is looked up once per device
// with hipGetSymbolAddress and kept here.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

namespace strata {

constexpr uint64_t kScratchBytes = uint64_t(64) << 20;
constexpr int kScratchDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

static std::mutex g_scratch_mu;
static void* g_scratch_dev[kScratchDevices] = {};

uint64_t scratch_bytes() { return kScratchBytes; }

// Looks up `device`'s copy of the array (once; later calls return at once).
// Makes `device` current for the lookup and restores the caller's device.
hipError_t scratch_init(int device) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (device < 0 || device >= kScratchDevices) return hipErrorInvalidDevice;
  if (g_scratch_dev[device]) return hipSuccess;
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return e;
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (cur != device) (void)hipSetDevice(cur);
  if (e != hipSuccess) return e;
  if (!p) return hipErrorInvalidSymbol;
  g_scratch_dev[device] = p;
  return hipSuccess;
}

// The device address of `device`'s copy, or nullptr before scratch_init.
void* scratch_ptr(int device) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return (device >= 0 && device < kScratchDevices) ? g_scratch_dev[device] : nullptr;
}

}  // namespace strata
