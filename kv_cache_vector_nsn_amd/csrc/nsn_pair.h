// Pair-layout encode pieces shared by the encode kernels and the decode step's
// append: NSN and the rotation of one token per half-wave, the double-quantized
// s1 grid, the exhaustive nearest-centroid search on the matrix cores, and the
// encode of a (K, V) token pair in one wave.
//
// Follows the Technical Summary of the explainer "NSNQuant: A Double
// Normalization Approach for Calibration-Free Low-Bit Vector Quantization of KV
// Cache" (gist.science/paper/2505.18231), sections "1. Normalize-Shift-Normalize
// (NSN)", "2. Hadamard Transform", "3. Vector Quantization and Codebook" and
// "4. Implementation Details" ("Residuals": a new token is quantized with the
// stored shift and appended).
#pragma once

#include "nsn_device.h"

namespace nsn {
namespace {

constexpr float kSqrtD = 11.313708498984761f;      // sqrt(128)
constexpr float kInvSqrtD = 0.08838834764831845f;  // 1 / sqrt(128)

// half_wave_sum with its last exchange (between the two 16-lane rows) through the
// LDS crossbar: ds_swizzle + add instead of a copy, v_permlane16_swap and an add,
// two vector-ALU instructions fewer in the VALU-bound per-token kernels (the sum
// is bitwise the same: the two rows' values are added either way).
__device__ __forceinline__ float half_sum_swz(float v) {
  v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);  // row_half_mirror
  v += dpp_f<0x140>(v);  // row_mirror
  return v + swz_xor<16>(v);
}

// Double quantization ([VQ] "Double Quantization"): the s1 grid of a tensor and
// the 4-bit o.  The grid is uniform over the fp16 bit pattern of s1: code 0 is a
// zero token, code c >= 1 the pattern base + (c - 1) stride (capped at the
// largest finite fp16); a token takes the nearest code (ties up), clamped to
// 1 .. 15.
struct DqS1 {
  uint32_t base = 0, stride = 1;
  float rstride = 1.f;  // 1 / stride (estimate; the floor is corrected exactly)
};

__device__ __forceinline__ DqS1 dq_s1_load(const nsn_dq_head* hd) {
  DqS1 q;
  q.base = hd->s1_base;
  q.stride = hd->s1_stride;
  q.rstride = 1.f / (float)q.stride;
  return q;
}

// Code of a non-zero s1 (fp32) and the fp16 pattern of its quantized value.
__device__ __forceinline__ uint32_t dq_s1_code(float s1, const DqS1& q) {
  const int off = max((int)f16_bits(s1) - (int)q.base, 0) + (int)(q.stride >> 1);
  int c = (int)((float)off * q.rstride);  // within one of floor(off / stride)
  c += ((c + 1) * (int)q.stride <= off) ? 1 : 0;
  c -= (c * (int)q.stride > off) ? 1 : 0;
  return 1u + (uint32_t)min(c, 14);
}
__device__ __forceinline__ uint32_t dq_s1_pattern(uint32_t code, const DqS1& q) {
  return min(q.base + (code - 1u) * q.stride, 0x7BFFu);
}

// o_q of channels 4p .. 4p+3 from the head record (codes in bytes 2p, 2p+1).
__device__ __forceinline__ void dq_o_load(const nsn_dq_head* hd, int p, float ov[4]) {
  const uint32_t b = *reinterpret_cast<const uint16_t*>(hd->o_codes + 2 * p);
  const float sc = hd->o_scale;
#pragma unroll
  for (int c = 0; c < 4; ++c) ov[c] = (float)((int)((b >> (4 * c)) & 15u) - 8) * sc;
}

// NSN and rotation of one token per half-wave (pair layout; every lane of the
// half must be active).  On return h holds channels 4p .. 4p+3 of H_sylvester z
// (unnormalised) and rz = 1 / ||z||, so that the rotated token is
// w = rz h = (H / sqrt(d)) u, u = (y - o) / s2, ||w||^2 = d; s1 = ||x|| / sqrt(d),
// s2 = ||z|| / sqrt(d) (0 when z is degenerate, then rz = 0 and w = 0).
// DQ: y = x / s1_q with s1_q the grid value of s1's code (returned in code;
// 0 for a zero token), and ov holds o_q.
template <bool DQ = false>
__device__ __forceinline__ void nsn_rotate(const float xv[4], int p, const float ov[4], float w[4], float& s1,
                                           float& s2, float& rz, bool& degen, const DqS1* dq = nullptr,
                                           uint32_t* code = nullptr) {
  const float ss = half_sum_swz(xv[0] * xv[0] + xv[1] * xv[1] + xv[2] * xv[2] + xv[3] * xv[3]);
  const float r1 = ss > 0.f ? __builtin_amdgcn_rsqf(ss) : 0.f;  // 1 / ||x||
  s1 = ss * r1 * kInvSqrtD;
  float inv1 = r1 * kSqrtD;  // 1 / s1 (0 for a zero token: y = 0)
  if constexpr (DQ) {
    const uint32_t c = ss > 0.f ? dq_s1_code(s1, *dq) : 0u;
    inv1 = c ? __builtin_amdgcn_rcpf(f16_val((uint16_t)dq_s1_pattern(c, *dq))) : 0.f;
    *code = c;
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) w[c] = fmaf(xv[c], inv1, -ov[c]);  // z = y - o
  const float zz = half_sum_swz(w[0] * w[0] + w[1] * w[1] + w[2] * w[2] + w[3] * w[3]);
  degen = !(zz > kEpsZ * kEpsZ * (float)kD);  // ||z|| <= kEpsZ sqrt(d)
  rz = degen ? 0.f : __builtin_amdgcn_rsqf(zz);  // 1 / ||z||
  s2 = zz * rz * kInvSqrtD;
  fwht128_pair(w, p);  // H_sylvester z
}

// (v0, v1) rounded to fp16 (nearest even), packed: one v_cvt_pk_f16_f32
__device__ __forceinline__ uint32_t hi_pair(float v0, float v1) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  typedef float f2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){v0, v1}, h2));
}

// The fp16 residues (v0 - hi0, v1 - hi1) of a pair whose rounded halves are packed in
// hi: two mixed-precision fmas that read the fp16 halves of hi in place and write
// the halves of the result (round to nearest even).
__device__ __forceinline__ uint32_t lo_pair(uint32_t hi, float v0, float v1) {
  uint32_t r;
  asm("v_fma_mixlo_f16 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=&v"(r) : "v"(hi), "v"(v0));
  asm("v_fma_mixhi_f16 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "+v"(r) : "v"(hi), "v"(v1));
  return r;
}

__device__ __forceinline__ float f16_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu)); }
__device__ __forceinline__ float f16_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

// Exhaustive argmin over the 256 centroids for the 32 columns of one MFMA set
// (g = 4 layout: lanes 0-31 hold B K-slots 0-7 of column lane % 32, lanes 32-63
// slots 8-15).  A fragments come from the codebook's prebuilt encode table.
// Returns, in both lanes of a column, the packed key (distance bits, index).
__device__ __forceinline__ int mfma_argmin_col4(const half8 B, const uint16_t* __restrict__ encA, int lane) {
  const int h = lane >> 5;
  int best = 0x7fffffff;
  // one tile at a time: this path is rare and must not raise the kernel's register count
#pragma unroll 1
  for (int tt = 0; tt < kTiles; ++tt) {
    const half8 A = *reinterpret_cast<const half8*>(encA + ((size_t)(tt * 2) * 64 + lane) * 8);
    floatx16 Z = {};
    const floatx16 D = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, B, Z, 0, 0, 0);
    // row of register r in this lane half: 8 (r / 4) + 4 h + r % 4 -> centroid 32 tt + row
    int tb = 0x7fffffff;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      // copy the element out first: a bit cast of a vector element
      // expression would read the vector's first element instead
      const float d0 = D[r], d1 = D[r + 1];
      const int key0 = (__float_as_int(d0) & ~0xff) | (8 * (r >> 2) + (r & 3));
      const int key1 = (__float_as_int(d1) & ~0xff) | (8 * ((r + 1) >> 2) + ((r + 1) & 3));
      tb = min(min(tb, key0), key1);
    }
    best = min(best, tb + 32 * tt);
  }
  best |= h << 2;
  const auto r = __builtin_amdgcn_permlane32_swap((uint32_t)best, (uint32_t)best, false, false);
  return min((int)r[0], (int)r[1]);
}


// H_sylvester on the matrix cores (16x16x32 fp16): row tile mt (rows 16 mt ..
// 16 mt + 15) times K step ks (columns 32 ks .. 32 ks + 31) as the A operand.  Lane
// l holds row i = l % 16 and columns 8 (l / 16) + j of the step; the sign of
// H[r][c] is the parity of r & c, which splits into a lane part (the bits of i and
// j, bit 3 of i with bit 0 of l / 16, bit 0 of mt with bit 1 of l / 16) and a part
// shared by the wave (bits 1-2 of mt with the bits of ks).  Four fragments per lane
// serve all 32 products: +-F_0 (mt even) and +-F_1 (mt odd), the sign from
// hsyl_neg(mt, ks).
// fp16 +-1 fragment of lane l (see above); neg flips every sign
__device__ __forceinline__ half8 hsyl_frag(int l, int f1, int neg) {
  const int l0 = l & 1, l1 = (l >> 1) & 1, l2 = (l >> 2) & 1, l3 = (l >> 3) & 1, l4 = (l >> 4) & 1, l5 = (l >> 5) & 1;
  uint32_t w[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t v = 0;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int j = 2 * d + e;
      const int sgn = (l3 & l4) ^ (l2 & (j >> 2)) ^ (l1 & ((j >> 1) & 1)) ^ (l0 & (j & 1)) ^ (f1 & l5) ^ neg;
      v |= (sgn ? 0xBC00u : 0x3C00u) << (16 * e);
    }
    w[d] = v;
  }
  return __builtin_bit_cast(half8, make_uint4(w[0], w[1], w[2], w[3]));
}

__device__ __forceinline__ bool hsyl_neg(int mt, int ks) {
  return ((((mt >> 2) & 1) & ((ks >> 1) & 1)) ^ (((mt >> 1) & 1) & (ks & 1))) != 0;
}

// Encode of one (K, V) token pair of a (batch, KV head) in one wave, one token
// per half-wave (half 0: K, half 1: V), with the stored channel means: NSN with
// that o, the rotation (H D with the handle's signs), the exhaustive nearest
// centroid on the matrix cores (exact products, fp32 sums, ties to the lowest
// index), alpha and the stored fp16 scale pair.  Every lane of the wave must be
// active.  Writes the half's token record (idx row, scale word) and returns, in
// lane p of the half, the channels 4p .. 4p+3 of the token's w_hat (centroid
// values, rotated domain) with the stored s1 and s2' as fp16-rounded floats.
// g = 8 needs 2 x 128 floats of LDS scratch (lds_w).
template <int G, bool RHT>
__device__ __forceinline__ void encode_pair(const _Float16* __restrict__ xh, const float* __restrict__ oh,
                                            const uint16_t* __restrict__ encA, const float* __restrict__ c32,
                                            uint4 smask, int lane, float* lds_w, uint8_t* idx_row,
                                            uint16_t* sc_row, float wq[4], float& s1q, float& s2q) {
  const int p = lane & 31, h = lane >> 5;
  // every load first (the A fragments of all 8 tiles, the token, o): one memory
  // latency instead of one per tile
  half8 A[kTiles], Ax[kTiles];
#pragma unroll
  for (int tt = 0; tt < kTiles; ++tt) {
    A[tt] = *reinterpret_cast<const half8*>(encA + ((size_t)(tt * 2 + 0) * 64 + lane) * 8);
    if constexpr (G == 8) Ax[tt] = *reinterpret_cast<const half8*>(encA + ((size_t)(tt * 2 + 1) * 64 + lane) * 8);
  }
  float xv[4], ov[4];
  load4(xh, p, xv);
#pragma unroll
  for (int c = 0; c < 4; ++c) ov[c] = oh[4 * p + c];
  if constexpr (RHT) {
    const Sign4 sg = lane_signs(smask, p);
    flip4(xv, sg);
    flip4(ov, sg);
  }
  float w[4], s1, s2, rz;
  bool degen;
  nsn_rotate<false>(xv, p, ov, w, s1, s2, rz, degen);
#pragma unroll
  for (int c = 0; c < 4; ++c) w[c] *= rz;  // ||w||^2 = d (0 for a degenerate token)
  int k4 = 0;  // g = 4: the index of sub-vector p; g = 8: the index of sub-vector p / 2
  if constexpr (G == 4) {
    // lane p of a half owns sub-vector p: B columns = the 32 sub-vectors of one token
    half8 Pf, Qf;
    const float nv = w[0] * w[0] + w[1] * w[1] + w[2] * w[2] + w[3] * w[3];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float m2 = -2.f * w[e];
      const _Float16 ah = (_Float16)m2;
      Pf[e] = ah;
      Pf[4 + e] = (_Float16)(m2 - (float)ah);
    }
    const _Float16 nh = (_Float16)nv;
    Qf[0] = (_Float16)1.f; Qf[1] = (_Float16)1.f; Qf[2] = nh; Qf[3] = (_Float16)(nv - (float)nh);
    Qf[4] = (_Float16)0.f; Qf[5] = (_Float16)0.f; Qf[6] = (_Float16)0.f; Qf[7] = (_Float16)0.f;
    const uint4 pw = __builtin_bit_cast(uint4, Pf), qw = __builtin_bit_cast(uint4, Qf);
    const uint32_t pa[4] = {pw.x, pw.y, pw.z, pw.w}, qa[4] = {qw.x, qw.y, qw.z, qw.w};
    uint32_t b0[4], b1[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const auto r = __builtin_amdgcn_permlane32_swap(pa[d], qa[d], false, false);
      b0[d] = r[0];  // token 0's columns: its P parts in lanes 0-31, its Q parts in 32-63
      b1[d] = r[1];  // token 1's columns
    }
    // both tokens' 32 columns against each 32-centroid tile; lane (column c, half h)
    // holds rows 8 (r / 4) + 4 h + r % 4 of the result, keys tagged with the row
    const half8 B0 = __builtin_bit_cast(half8, make_uint4(b0[0], b0[1], b0[2], b0[3]));
    const half8 B1 = __builtin_bit_cast(half8, make_uint4(b1[0], b1[1], b1[2], b1[3]));
    int best0 = 0x7fffffff, best1 = 0x7fffffff;
#pragma unroll
    for (int tt = 0; tt < kTiles; ++tt) {
      floatx16 Z = {};
      const floatx16 D0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[tt], B0, Z, 0, 0, 0);
      const floatx16 D1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[tt], B1, Z, 0, 0, 0);
      int t0 = 0x7fffffff, t1 = 0x7fffffff;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float d0 = D0[r], d1 = D1[r];
        const int tag = 8 * (r >> 2) + (r & 3);
        t0 = min(t0, (__float_as_int(d0) & ~0xff) | tag);
        t1 = min(t1, (__float_as_int(d1) & ~0xff) | tag);
      }
      best0 = min(best0, t0 + 32 * tt);
      best1 = min(best1, t1 + 32 * tt);
    }
    best0 |= h << 2;
    best1 |= h << 2;
    const auto r0 = __builtin_amdgcn_permlane32_swap((uint32_t)best0, (uint32_t)best0, false, false);
    const auto r1 = __builtin_amdgcn_permlane32_swap((uint32_t)best1, (uint32_t)best1, false, false);
    const int c0 = min((int)r0[0], (int)r0[1]), c1 = min((int)r1[0], (int)r1[1]);
    k4 = (h == 0 ? c0 : c1) & 0xff;
    idx_row[p] = (uint8_t)k4;
#pragma unroll
    for (int c = 0; c < 4; ++c) wq[c] = c32[k4 * 4 + c];
  } else {
    // column c = p: sub-vector c % 16 of token c / 16; the halves hold the hi and
    // lo parts of -2 w and complementary rows of the 32 x 32 result
#pragma unroll
    for (int c = 0; c < 4; ++c) lds_w[h * kD + 4 * p + c] = w[c];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int tok = p >> 4, sv = p & 15;
    float w8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) w8[e] = lds_w[tok * kD + sv * 8 + e];
    float wn = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) wn += w8[e] * w8[e];
    const _Float16 wn_hi = (_Float16)wn;
    const _Float16 wn_lo = (_Float16)(wn - (float)wn_hi);
    half8 Bf, Bx;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float a = -2.f * w8[e];
      const _Float16 ah = (_Float16)a;
      Bf[e] = h == 0 ? ah : (_Float16)(a - (float)ah);
    }
    Bx[0] = h == 0 ? (_Float16)1.f : (_Float16)0.f;
    Bx[1] = Bx[0];
    Bx[2] = h == 0 ? wn_hi : (_Float16)0.f;
    Bx[3] = h == 0 ? wn_lo : (_Float16)0.f;
    Bx[4] = (_Float16)0.f; Bx[5] = (_Float16)0.f; Bx[6] = (_Float16)0.f; Bx[7] = (_Float16)0.f;
    int best = 0x7fffffff;
#pragma unroll
    for (int tt = 0; tt < kTiles; ++tt) {
      floatx16 D = {};
      D = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[tt], Bf, D, 0, 0, 0);
      D = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ax[tt], Bx, D, 0, 0, 0);
      // row of register r in this lane half: 8 (r / 4) + 4 h + r % 4 -> centroid 32 tt + row
      int tb = 0x7fffffff;
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float d0 = D[r], d1 = D[r + 1];
        const int key0 = (__float_as_int(d0) & ~0xff) | (8 * (r >> 2) + (r & 3));
        const int key1 = (__float_as_int(d1) & ~0xff) | (8 * ((r + 1) >> 2) + ((r + 1) & 3));
        tb = min(min(tb, key0), key1);
      }
      best = min(best, tb + 32 * tt);
    }
    best |= h << 2;
    {
      const auto r = __builtin_amdgcn_permlane32_swap((uint32_t)best, (uint32_t)best, false, false);
      best = min((int)r[0], (int)r[1]);
    }
    const int kc = best & 0xff;  // index of column p (both halves)
    // pair layout: lane p of half h takes the index of (token h, sub-vector p / 2),
    // held by column 16 h + p / 2
    k4 = __builtin_amdgcn_ds_bpermute(4 * (16 * h + (p >> 1)), kc);
    if ((p & 1) == 0) idx_row[p >> 1] = (uint8_t)k4;
#pragma unroll
    for (int c = 0; c < 4; ++c) wq[c] = c32[k4 * 8 + 4 * (p & 1) + c];
  }
  // alpha = ||w||^2 / <w, w_hat> = d / <w, w_hat>
  float dot = w[0] * wq[0] + w[1] * wq[1] + w[2] * wq[2] + w[3] * wq[3];
  dot = half_sum_swz(dot);
  const float alpha = (!degen && dot > 0.f) ? (float)kD * __builtin_amdgcn_rcpf(dot) : 1.f;
  const uint16_t b1 = f16_bits(s1), b2 = f16_bits(s2 * alpha);
  if (p == 0) *reinterpret_cast<uint32_t*>(sc_row) = (uint32_t)b1 | ((uint32_t)b2 << 16);
  s1q = f16_val(b1);
  s2q = f16_val(b2);
}

}  // namespace
}  // namespace nsn
