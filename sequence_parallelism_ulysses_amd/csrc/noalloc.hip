// attn_bwd without a caller-provided workspace, for callers that cannot
// allocate device memory (code under graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// The workspace is a file-scope device array, one copy per GPU the library
// runs on, held until the process ends. Host code never passes the array's
// name to a kernel (on the host it is only a stand-in for the symbol): the
// first call on a device asks the runtime for that device's address of the
// array, with the device current, and every later call on the device uses
// that address. All calls on one GPU share the array, which keeps the last
// call's contents; the backward clears what it needs zeroed itself. Calls
// that overlap in time on one GPU (several streams or host threads) race.
#include <mutex>

#include "internal.hpp"

namespace uly {
namespace {

static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Address of this device's copy of `scratch`, looked up once per device.
hipError_t scratch_address(int device, void** ptr) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch_ptr[device] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[device] = p;
  }
  *ptr = g_scratch_ptr[device];
  return hipSuccess;
}

}  // namespace

hipError_t launch_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                                   const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                   const AttnDesc& desc, hipStream_t stream, size_t* need) {
  AttnDesc d = desc;
  d.splits = 1;  // no partial dK/dV sums
  *need = bwd_workspace_bytes(d);
  if (*need > kNoAllocScratchBytes) return hipErrorInvalidValue;
  int device = -1;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return e;
  if (stream != nullptr) {
    // the stream's device must be the current one, whose copy is looked up
    int sdev = -1;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return e;
    if (sdev != device) return hipErrorInvalidDevice;
  }
  void* ws = nullptr;
  e = scratch_address(device, &ws);
  if (e != hipSuccess) return e;
  return launch_attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, ws, d, d.dt, stream);
}

}  // namespace uly
