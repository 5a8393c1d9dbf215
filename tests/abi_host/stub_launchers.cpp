// Host-only stand-ins for the kernel launchers and the few HIP runtime calls
// the C ABI layer (api.cpp) makes, so that the argument checks can be built
// with AddressSanitizer and run on a machine without a GPU. Each launcher
// records that it was reached and touches every host array it is given (so
// that an array shorter than the ABI promises is an out-of-bounds read).
#include <cstdio>

#include "internal.hpp"

int g_launches = 0;

extern "C" const char* hipGetErrorString(hipError_t) { return "stub HIP error"; }

namespace uly {

hipError_t launch_pack(const void* const* const* shards, void* const* out, const PermuteDesc& d, hipStream_t) {
  volatile uintptr_t x = 0;
  for (int s = 0; s < d.nseg; ++s) {
    x = x + reinterpret_cast<uintptr_t>(out[s]);
    for (int j = 0; j < d.P; ++j) x = x + reinterpret_cast<uintptr_t>(shards[s][j]);
  }
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_unpack(const void* const* in, void* const* const* shards, const PermuteDesc& d, hipStream_t) {
  volatile uintptr_t x = 0;
  for (int s = 0; s < d.nseg; ++s) {
    x = x + reinterpret_cast<uintptr_t>(in[s]);
    for (int j = 0; j < d.P; ++j) x = x + reinterpret_cast<uintptr_t>(shards[s][j]);
  }
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_attn_fwd(const void*, const void*, const void*, void*, float*, const AttnDesc&, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_attn_fwd_from_shards(const void* const* q, const void* const* k, const void* const* v, int P,
                                       int64_t, int, int, int, void*, float*, const AttnDesc&, hipStream_t) {
  volatile uintptr_t x = 0;
  for (int j = 0; j < P; ++j)
    x = x + reinterpret_cast<uintptr_t>(q[j]) + reinterpret_cast<uintptr_t>(k[j]) + reinterpret_cast<uintptr_t>(v[j]);
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_attn_merge(const void* const* o_parts, const float* const* lse_parts, int nparts, int64_t, int,
                             int, uly_dtype, void*, float*, hipStream_t) {
  volatile uintptr_t x = 0;
  for (int c = 0; c < nparts; ++c)
    x = x + reinterpret_cast<uintptr_t>(o_parts[c]) + reinterpret_cast<uintptr_t>(lse_parts[c]);
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_attn_bwd(const void*, const void*, const void*, const void*, const void*, const float*, void*,
                           void*, void*, void*, const AttnDesc&, uly_dtype, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_attn_bwd_noalloc(const void*, const void*, const void*, const void*, const void*, const float*,
                                   void*, void*, void*, const AttnDesc& d, hipStream_t, size_t* need) {
  AttnDesc one = d;
  one.splits = 1;
  *need = bwd_workspace_bytes(one);
  ++g_launches;
  return hipSuccess;
}

}  // namespace uly
