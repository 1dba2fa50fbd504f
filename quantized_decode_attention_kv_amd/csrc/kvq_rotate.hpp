// Key-only rotation (KVQ_KEY_ROTATION): the orthonormal Walsh-Hadamard transform
// of a key row or query, in float32, as butterflies h = 1, 2, 4, ..., n/2 (the
// entries j and j + h of every 2h-block become a + b and a - b) and one multiply
// by the transform's scale ("Quantize What Counts", technical summary:
// contributions, orthogonality and integration; results, rotation integration).
// The steps are fixed, so every implementation that takes them gets the same bits.
#pragma once

#include <hip/hip_runtime.h>

namespace kvq {

// float32 scale 2^(-m/2) of the width-2^m transform; for odd m the float32 of
// sqrt(1/2) times 2^(-(m-1)/2) (a power of two, so the product is exact)
__host__ __device__ inline float rotation_scale(int m) {
  const float p = ldexpf(1.0f, -(m / 2));
  return (m & 1) ? 0.70710677f * p : p;
}

// x times the scale, rounded to float32 on its own.  Left visible, a multiply
// whose result is next converted to fp16 may be folded into one mixed-precision
// instruction that rounds the exact product once, straight to fp16, which differs
// from rounding to float32 first whenever the float32 product is an fp16 tie; the
// empty asm hands the compiler an opaque float32 value.
__device__ __forceinline__ float rotation_scaled(float x, float scale) {
  float y = x * scale;
  asm("" : "+v"(y));
  return y;
}

// One butterfly of an element held apart from its partner (the element h away):
// the lower element of the pair becomes self + partner, the upper partner - self.
__device__ __forceinline__ float butterfly(float self, float partner, bool upper) {
  return upper ? partner - self : self + partner;
}

// Butterflies h = 1, 2, 4 inside 8 consecutive entries held by one thread.
__device__ __forceinline__ void butterflies8(float (&x)[8]) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if ((k & h) == 0) {
        const float a = x[k], b = x[k + h];
        x[k] = a + b;
        x[k + h] = a - b;
      }
    }
  }
}

}  // namespace kvq
