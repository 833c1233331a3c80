// Dequantization of the NSNQuant cache.
//
// Reconstruction follows "1. Normalize-Shift-Normalize (NSN)" of the Technical
// Summary of the explainer "NSNQuant: A Double Normalization Approach for
// Calibration-Free Low-Bit Vector Quantization of KV Cache"
// (gist.science/paper/2505.18231): the byproducts (s1, o, s2) rebuild the
// tensor, x_hat = s1 (s2' H w_hat + o) (s1 (s2' D H w_hat + o) with the
// randomized transform's signs D).
#include "nsn_device.h"

namespace nsn {
namespace {

// Grid (ceil(L / 8), BH), 256 threads: each wave rebuilds a token pair.
template <int G>
__global__ __launch_bounds__(256) void k_dequant(const uint8_t* __restrict__ idx, const uint16_t* __restrict__ sc,
                                                 const float* __restrict__ o, const float* __restrict__ c32,
                                                 int L, int L_cap, float* __restrict__ xh, uint4 smask) {
  constexpr int M = kD / G;
  const int bh = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, p = lane & 31;
  const int t = blockIdx.x * 8 + wave * 2 + half;
  if (t >= L) return;  // whole half-wave leaves together: no shuffles below cross halves
  const size_t row = (size_t)bh * L_cap + t;
  const int sv = (G == 4) ? p : (p >> 1);
  const int off = (G == 4) ? 0 : 4 * (p & 1);
  const int k = idx[row * M + sv];
  float v[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) v[c] = c32[k * G + off + c];
  const uint32_t w = *reinterpret_cast<const uint32_t*>(sc + row * 2);
  const float s1 = f16_val((uint16_t)(w & 0xffffu)), s2 = f16_val((uint16_t)(w >> 16));
  fwht128_pair(v, p);
  flip4(v, lane_signs(smask, p));  // randomized rotation: D H w_hat
  const float rs = 0.08838834764831845f;  // 1/sqrt(128)
  float4 r;
  r.x = s1 * (s2 * (v[0] * rs) + o[(size_t)bh * kD + 4 * p + 0]);
  r.y = s1 * (s2 * (v[1] * rs) + o[(size_t)bh * kD + 4 * p + 1]);
  r.z = s1 * (s2 * (v[2] * rs) + o[(size_t)bh * kD + 4 * p + 2]);
  r.w = s1 * (s2 * (v[3] * rs) + o[(size_t)bh * kD + 4 * p + 3]);
  *reinterpret_cast<float4*>(xh + ((size_t)bh * L + t) * kD + 4 * p) = r;
}

}  // namespace

hipError_t launch_dequantize(const nsn_codebook* cb, const uint8_t* idx, const uint16_t* scales, const float* o,
                             int BH, int L, int L_cap, float* x_hat, hipStream_t st) {
  dim3 grid((L + 7) / 8, BH);
  const uint4 sm = make_uint4(cb->sgn[0], cb->sgn[1], cb->sgn[2], cb->sgn[3]);
  if (cb->g == 4)
    k_dequant<4><<<grid, 256, 0, st>>>(idx, scales, o, cb->d_c32, L, L_cap, x_hat, sm);
  else
    k_dequant<8><<<grid, 256, 0, st>>>(idx, scales, o, cb->d_c32, L, L_cap, x_hat, sm);
  return hipGetLastError();
}

}  // namespace nsn
