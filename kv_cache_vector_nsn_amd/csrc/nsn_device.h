// Device helpers shared by the encode, append and dequantize kernels.
//
// Token layout inside a wavefront ("pair layout"): a 64-lane wave holds two
// tokens of d = 128 channels; lanes 0-31 hold token 0, lanes 32-63 token 1,
// and lane p of a half holds channels 4p .. 4p+3.  A global load of 4 fp16
// channels per lane is then one coalesced 512-byte access per wave.
#pragma once

#include "nsn_internal.h"

namespace nsn {

// Sum over the 32 lanes of a half-wave (xor butterflies stay inside a half).
__device__ __forceinline__ float half_wave_sum(float v) {
#pragma unroll
  for (int m = 1; m < 32; m <<= 1) v += __shfl_xor(v, m);
  return v;
}

// Unnormalised Walsh-Hadamard transform (Sylvester, natural order) of the 128
// channels held in pair layout: H[i][j] = (-1)^popcount(i & j), so the
// butterfly (a, b) -> (a + b, a - b) on pairs at distance 1, 2, ..., 64 gives
// H v.  Distances 1 and 2 are inside a lane, 4 .. 64 are lane distances 1 .. 16.
__device__ __forceinline__ void fwht128_pair(float v[4], int p) {
  float a0 = v[0] + v[1], a1 = v[0] - v[1], a2 = v[2] + v[3], a3 = v[2] - v[3];
  v[0] = a0 + a2;
  v[1] = a1 + a3;
  v[2] = a0 - a2;
  v[3] = a1 - a3;
#pragma unroll
  for (int m = 1; m < 32; m <<= 1) {
    const bool upper = (p & m) != 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float o = __shfl_xor(v[c], m);
      v[c] = upper ? (o - v[c]) : (v[c] + o);
    }
  }
}

// Load 4 channels (4p .. 4p+3) of one token as fp32.
__device__ __forceinline__ void load4(const _Float16* __restrict__ row, int p, float v[4]) {
  const half4 h = *reinterpret_cast<const half4*>(row + 4 * p);
  v[0] = (float)h[0];
  v[1] = (float)h[1];
  v[2] = (float)h[2];
  v[3] = (float)h[3];
}
__device__ __forceinline__ void load4(const float* __restrict__ row, int p, float v[4]) {
  const float4 f = *reinterpret_cast<const float4*>(row + 4 * p);
  v[0] = f.x;
  v[1] = f.y;
  v[2] = f.z;
  v[3] = f.w;
}

__device__ __forceinline__ uint16_t f16_bits(float f) {
  _Float16 h = (_Float16)f;  // round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float f16_val(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

}  // namespace nsn
