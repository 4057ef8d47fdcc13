// Division by a launch-time constant as one high multiply, for kernels whose
// per-element index math would otherwise be dominated by integer divisions.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pagedkv {

// ceil(2^32 / d) for d >= 2; 0 stands for d = 1.
inline uint32_t reciprocal_u32(uint32_t d) {
  return d <= 1 ? 0u : static_cast<uint32_t>(((uint64_t{1} << 32) + d - 1) / d);
}

// n / d given m = reciprocal_u32(d).  With m = ceil(2^32 / d) = (2^32 + e) / d,
// 0 <= e < d, the high product is floor(n / d + n e / (d 2^32)), which is
// exact while n < 2^32 / d: the caller checks that bound for every index.
__device__ __forceinline__ uint32_t div_by(uint32_t n, uint32_t m) {
  return m ? __umulhi(n, m) : n;
}

}  // namespace pagedkv
