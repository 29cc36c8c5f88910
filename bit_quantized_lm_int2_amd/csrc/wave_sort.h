// The block emit's ranking of one block row across a wave (gfx950, wave64).
#pragma once
#include "device_util.h"

namespace i2h {

// Descending bitonic sort across the wave of (value, column); better = larger value, then lower
// column. Afterwards lane r holds the r-th best.
__device__ __forceinline__ void wave_sort_vc(float& v, int& c, int lane) {
#pragma unroll
  for (int size = 2; size <= kWave; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const float ov = __shfl_xor(v, stride);
      const int oc = __shfl_xor(c, stride);
      const bool lower = (lane & stride) == 0;
      const bool desc = (lane & size) == 0;
      const bool other_better = (ov > v) || (ov == v && oc < c);
      if ((lower == desc) == other_better) {
        v = ov;
        c = oc;
      }
    }
  }
}

}  // namespace i2h
