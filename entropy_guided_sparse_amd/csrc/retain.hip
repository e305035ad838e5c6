// K6/K7/K8: decode-time KV retention and decode attention (being written).
#include "egs_device.h"
#include "egs_launch.h"

namespace egs {
size_t retain_workspace_bytes(const DecodeDims&) { return 256; }
hipError_t launch_kv_retain(const DecodeDims&, const egs_retain_params&, const void*, const void*,
                            const void*, const float*, int32_t*, void*, void*, float*, float*,
                            void*, hipStream_t) {
  return hipErrorNotSupported;
}
size_t decode_attn_workspace_bytes(const DecodeDims&, int) { return 256; }
hipError_t launch_decode_attn(const DecodeDims&, const void*, const void*, const void*, int,
                              void*, void*, hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace egs
