// attn_bwd.hip -- 8-bit attention backward (dQ, dK, dV).
#include "sage_device.hpp"
#include "sage_launch.hpp"

namespace sage {

size_t attn_bwd_ws_bytes(const Shape&) { return 0; }

hipError_t launch_attn_bwd(const Shape&, const void*, const void*, const void*, const void*, const void*,
                           const float*, void*, void*, void*, void*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace sage
