// oscar_decode_attn_noalloc: decode_attn with its scratch in a library-owned
// static device array instead of a caller workspace, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// The array is a file-scope __device__ symbol: every GPU the library runs on
// holds its own copy, at its own address, until the process ends.  Host code
// never passes the symbol itself to a kernel (on the host it is only a
// stand-in); the device address is looked up once per device with
// hipGetSymbolAddress and cached.  The kernels are the ones oscar_decode_attn
// launches; nothing in the scratch needs to start at zero (every record is
// written before it is read within one call).  Calls that overlap in time on
// one GPU share the array and race.
#include <mutex>

#include "../../include/oscar.h"
#include "kernels.h"

static_assert(OSCAR_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) uint8_t scratch[OSCAR_NOALLOC_SCRATCH_BYTES];

namespace oscar {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

// Device address of this device's copy of `scratch` (looked up once per device,
// with that device current).  Returns hipSuccess or the lookup's error.
hipError_t noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p || reinterpret_cast<uintptr_t>(p) % 256 != 0) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace oscar
