// Attention backward: not yet implemented (placeholder so the library links).
#include "internal.hpp"

namespace uly {

size_t bwd_workspace_bytes(const AttnDesc& d) { return size_t(4) * d.hq * d.N; }

hipError_t launch_attn_bwd(const void*, const void*, const void*, const void*, const void*, const float*,
                           void*, void*, void*, void*, const AttnDesc&, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace uly
