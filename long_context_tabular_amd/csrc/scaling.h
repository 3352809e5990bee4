// Device helpers of the shared-length query scaling, used by the scaling
// kernels and by the projection epilogue so that both produce the same bits
// ("Fuse shared-length query scaling during inference", Solution: every eager
// fp16 rounding boundary is kept).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "internal.h"

namespace sdm {

// Correctly rounded double -> fp16: round to odd into float (the sticky bit
// keeps the information a second rounding needs; float has >= 2 more bits than
// fp16), then round to nearest even into fp16.
__device__ inline _Float16 f64_to_f16(double d) {
  float f = (float)d;
  const double df = (double)f;
  if (df != d) {
    uint32_t b = __float_as_uint(f);
    if (fabs(df) > fabs(d)) b -= 1u;  // step one ulp towards zero (f != 0 here)
    f = __uint_as_float(b | 1u);
  }
  return (_Float16)f;
}

// fp16(1 + fp16(tanh g)) as a float, with fp16(tanh g) correctly rounded.
// Fast path: the float32 tanhf is accurate to a few float32 ulps, far inside
// 2^-19 relative, so when t * (1 - 2^-19) and t * (1 + 2^-19) round to the
// same fp16 value, that value is the correctly rounded fp16 of tanh g.
// Otherwise (tanh g lies next to an fp16 rounding boundary) tanh is taken in
// double.  Exhaustively equal, over every finite fp16 gate, to rounding the
// double tanh.
__device__ inline float gate_factor(_Float16 g) {
  const float t32 = tanhf((float)g);
  _Float16 t = (_Float16)t32;
  const _Float16 lo = (_Float16)(t32 * (1.0f - 0x1p-19f));
  const _Float16 hi = (_Float16)(t32 * (1.0f + 0x1p-19f));
  if (lo != t || hi != t) t = f64_to_f16(tanh((double)g));
  return (float)(_Float16)(1.0f + (float)t);
}

// One element of q~: NONE q, LOG fp16(q*k), GATED fp16(fp16(q*k)*u).  The
// fp16 x fp16 products are exact in float32, so each step rounds once.
template <int MODE>
__device__ inline _Float16 scale_elem(_Float16 q, float kh, float u) {
  if constexpr (MODE == kScaleNone) {
    return q;
  } else {
    const _Float16 qk = (_Float16)((float)q * kh);
    if constexpr (MODE == kScaleLog) return qk;
    return (_Float16)((float)qk * u);
  }
}

}  // namespace sdm
