// Device helpers shared by the encode, append and dequantize kernels.
//
// Token layout inside a wavefront ("pair layout"): a 64-lane wave holds two
// tokens of d = 128 channels; lanes 0-31 hold token 0, lanes 32-63 token 1,
// and lane p of a half holds channels 4p .. 4p+3.  A global load of 4 fp16
// channels per lane is then one coalesced 512-byte access per wave.
#pragma once

#include "nsn_internal.h"

namespace nsn {

// Value of lane (i op DPP_CTRL) inside the 16-lane row (DPP; every lane active).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}

// Value of lane i ^ M inside the 32-lane half (ds_swizzle bit mode: and 0x1f, or 0,
// xor M).  It runs on the LDS crossbar without a memory access, so the exchange
// costs no vector-ALU slot.
template <int M>
__device__ __forceinline__ float swz_xor(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1F | (M << 10)));
}

// Sum over the 32 lanes of a half-wave, every lane gets the total.  Inside a
// 16-lane row: quad swaps 1 and 2, half-row mirror, row mirror (each pairs the
// partial sums of disjoint lane groups); then v_permlane16_swap adds the two
// rows of the half.
__device__ __forceinline__ float half_wave_sum(float v) {
  v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);  // row_half_mirror
  v += dpp_f<0x140>(v);  // row_mirror
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One radix-2 stage at lane distance M: (a, b) -> (a + b, a - b) where the lane
// without bit M holds a.  The upper lane forms partner - own, i.e.
// fma(sign, own, partner) with sign = -1 there.
template <int M>
__device__ __forceinline__ void fwht_stage(float v[4], int p) {
  const float sg = (p & M) ? -1.f : 1.f;
  float o[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) o[c] = swz_xor<M>(v[c]);
#pragma unroll
  for (int c = 0; c < 4; ++c) v[c] = fmaf(sg, v[c], o[c]);
}

// Unnormalised Walsh-Hadamard transform (Sylvester, natural order) of the 128
// channels held in pair layout: H[i][j] = (-1)^popcount(i & j), so the
// butterfly (a, b) -> (a + b, a - b) on pairs at distance 1, 2, ..., 64 gives
// H v.  Distances 1 and 2 are inside a lane, 4 .. 64 are lane distances 1 .. 16.
// Needs every lane of the half active.
__device__ __forceinline__ void fwht128_pair(float v[4], int p) {
  const float a0 = v[0] + v[1], a1 = v[0] - v[1], a2 = v[2] + v[3], a3 = v[2] - v[3];
  v[0] = a0 + a2;
  v[1] = a1 + a3;
  v[2] = a0 - a2;
  v[3] = a1 - a3;
  fwht_stage<1>(v, p);
  fwht_stage<2>(v, p);
  fwht_stage<4>(v, p);
  fwht_stage<8>(v, p);
  fwht_stage<16>(v, p);
}

// Value of lane i ^ M inside the 32-lane half through the vector ALU only (DPP
// inside a 16-lane row, v_permlane16_swap across the two rows of the half).  For
// code that has LDS-DMA loads in flight: an LDS-pipe exchange (ds_swizzle) carries
// no memory operand, so the compiler would first wait for every such load.
template <int M>
__device__ __forceinline__ float xor_valu(float v, int p) {
  if constexpr (M == 1) {
    return dpp_f<0xB1>(v);  // quad_perm [1,0,3,2]
  } else if constexpr (M == 2) {
    return dpp_f<0x4E>(v);  // quad_perm [2,3,0,1]
  } else if constexpr (M == 4) {
    // banks 0, 2 (bit 2 clear) read lane + 4 (row_shl:4); banks 1, 3 read lane - 4 (row_shr:4)
    int t = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x104, 0xf, 0x5, false);
    t = __builtin_amdgcn_update_dpp(t, __float_as_int(v), 0x114, 0xf, 0xa, false);
    return __int_as_float(t);
  } else if constexpr (M == 8) {
    return dpp_f<0x128>(v);  // row_ror:8
  } else {
    static_assert(M == 16, "lane distance 1..16");
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    // r[0] holds row 0 (2) in rows 0, 1 (2, 3); r[1] holds row 1 (3)
    return __uint_as_float((p & 16) ? r[0] : r[1]);
  }
}

template <int M>
__device__ __forceinline__ void fwht_stage_valu(float v[4], int p) {
  const float sg = (p & M) ? -1.f : 1.f;
#pragma unroll
  for (int c = 0; c < 4; ++c) v[c] = fmaf(sg, v[c], xor_valu<M>(v[c], p));
}

// fwht128_pair with vector-ALU exchanges only (same result).
__device__ __forceinline__ void fwht128_pair_valu(float v[4], int p) {
  const float a0 = v[0] + v[1], a1 = v[0] - v[1], a2 = v[2] + v[3], a3 = v[2] - v[3];
  v[0] = a0 + a2;
  v[1] = a1 + a3;
  v[2] = a0 - a2;
  v[3] = a1 - a3;
  fwht_stage_valu<1>(v, p);
  fwht_stage_valu<2>(v, p);
  fwht_stage_valu<4>(v, p);
  fwht_stage_valu<8>(v, p);
  fwht_stage_valu<16>(v, p);
}

// Randomized Hadamard: the rotation H D with D = diag(+-1) over the 128 channels,
// given as a 128-bit mask (bit c % 32 of word c / 32 set <=> channel c negated).
// lane_signs gives, for the channels 4p .. 4p+3 of pair-layout lane p, the bit
// to XOR into each fp32 value (bit 31 where the channel is negated, else 0).
struct Sign4 {
  uint32_t m[4];
};
__device__ __forceinline__ Sign4 lane_signs(uint4 mask, int p) {
  const uint32_t w = (p & 16) ? ((p & 8) ? mask.w : mask.z) : ((p & 8) ? mask.y : mask.x);
  const uint32_t nib = w >> (4 * (p & 7));
  Sign4 s;
#pragma unroll
  for (int c = 0; c < 4; ++c) s.m[c] = ((nib >> c) & 1u) << 31;
  return s;
}
__device__ __forceinline__ void flip4(float v[4], const Sign4& s) {
#pragma unroll
  for (int c = 0; c < 4; ++c) v[c] = __uint_as_float(__float_as_uint(v[c]) ^ s.m[c]);
}

// The same flips on 4 channels as loaded: fp16 (two sign bits per dword, so the
// halves stay packed for mixed-precision use) or fp32.
__device__ __forceinline__ half4 flip_raw(half4 r, const Sign4& s) {
  uint2 u = __builtin_bit_cast(uint2, r);
  u.x ^= (s.m[0] >> 16) | s.m[1];
  u.y ^= (s.m[2] >> 16) | s.m[3];
  return __builtin_bit_cast(half4, u);
}
__device__ __forceinline__ floatx4 flip_raw(floatx4 r, const Sign4& s) {
#pragma unroll
  for (int c = 0; c < 4; ++c) r[c] = __uint_as_float(__float_as_uint(r[c]) ^ s.m[c]);
  return r;
}

// floor(f) converted to int in one instruction (NaN -> 0, saturating).
__device__ __forceinline__ int cvt_flr(float f) {
  int r;
  asm("v_cvt_flr_i32_f32 %0, %1" : "=v"(r) : "v"(f));
  return r;
}

// The 4 channels 4p .. 4p+3 of one token as stored (8 bytes of fp16 or 16 of
// fp32), so that a load can be issued ahead of its use, and their fp32 values.
template <typename T> struct raw4;
template <> struct raw4<_Float16> { using type = half4; };
template <> struct raw4<float> { using type = floatx4; };
template <typename T>
__device__ __forceinline__ typename raw4<T>::type load_raw4(const T* __restrict__ row, int p) {
  return *reinterpret_cast<const typename raw4<T>::type*>(row + 4 * p);
}
// The same channels through a buffer descriptor over [base, base + bytes) at
// byte offset voff: a read past the end returns zeros, so a load for a token
// beyond the range needs no branch.  The loads are marked streaming
// (non-temporal, system coherence scope: nt sc1) so that the input, read once,
// does not push the encode kernel's candidate table out of the L2.  (The
// descriptor type exists only in the device compilation pass.)
template <typename T>
__device__ __forceinline__ typename raw4<T>::type buffer_raw4(const T* base, int bytes, uint32_t voff) {
  using V = typename raw4<T>::type;
#if defined(__HIP_DEVICE_COMPILE__)
  const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(base), (short)0, bytes, 0x00020000);
  if constexpr (sizeof(V) == 8)
    return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b64(rs, (int)voff, 0, 18));
  else
    return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)voff, 0, 18));
#else
  (void)base; (void)bytes; (void)voff;
  return V{};
#endif
}
// 16 bytes at byte offset voff of [base, base + bytes) (zeros past the end).
__device__ __forceinline__ uint4 buffer_load_u4(const void* base, int bytes, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)voff, 0, 0));
#else
  (void)base; (void)bytes; (void)voff;
  return uint4{};
#endif
}

// Stores through a buffer descriptor over [base, base + bytes): a store at an
// offset past the end is dropped, so lanes with nothing to write need no branch
// (and the compiler's wait for an earlier load is not widened by a join).
__device__ __forceinline__ void buffer_store_u8(uint8_t v, void* base, int bytes, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  const auto rs = __builtin_amdgcn_make_buffer_rsrc(base, (short)0, bytes, 0x00020000);
  __builtin_amdgcn_raw_buffer_store_b8(v, rs, (int)voff, 0, 0);
#else
  (void)v; (void)base; (void)bytes; (void)voff;
#endif
}
__device__ __forceinline__ void buffer_store_u32(uint32_t v, void* base, int bytes, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  const auto rs = __builtin_amdgcn_make_buffer_rsrc(base, (short)0, bytes, 0x00020000);
  __builtin_amdgcn_raw_buffer_store_b32(v, rs, (int)voff, 0, 0);
#else
  (void)v; (void)base; (void)bytes; (void)voff;
#endif
}
__device__ __forceinline__ void buffer_store_u64(uint2 v, void* base, int bytes, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  const auto rs = __builtin_amdgcn_make_buffer_rsrc(base, (short)0, bytes, 0x00020000);
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned int, v), rs,
                                        (int)voff, 0, 0);
#else
  (void)v; (void)base; (void)bytes; (void)voff;
#endif
}
template <typename V>
__device__ __forceinline__ void unpack4(V r, float v[4]) {
#pragma unroll
  for (int c = 0; c < 4; ++c) v[c] = (float)r[c];
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
