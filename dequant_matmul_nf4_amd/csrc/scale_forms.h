// The block scale with its form fixed at compile time, for kernels that
// stream scales next to other loads.
#pragma once

#include "nf4_device.h"

namespace nf4i {

// block_scale with the scale form fixed at compile time (no runtime branch,
// so no table load behind one): plain absmax, or the double-quantized form
// with int8 (kF8 = false) or float8 codes.
template <bool kDQ, bool kF8>
__device__ __forceinline__ float block_scale_t(const Scales& sc, int64_t b, float mean) {
  if constexpr (!kDQ) {
    return sc.absmax[b];
  } else {
    const float t = code_ratio(sc.q[b], kF8 ? 1 : 0);
    const float u = t * sc.absmax2[b >> 8];
    return u + mean;
  }
}

}  // namespace nf4i
