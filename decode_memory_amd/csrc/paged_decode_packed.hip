// paged_decode for packed pools (K8/V8, K8/V4, K4/V4).
#include "device_common.h"
#include "internal.h"

namespace pagedkv {

bool packed_decode_available() { return false; }

hipError_t launch_paged_decode_packed(const DecodeArgs&, int32_t, int32_t, hipStream_t) {
  return hipErrorInvalidValue;
}

}  // namespace pagedkv
