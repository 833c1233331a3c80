// NSNQuant encode on gfx950: Normalize-Shift-Normalize, Hadamard rotation and
// nearest-centroid vector quantization with the scale adjustment.
//
// Follows the Technical Summary of the explainer "NSNQuant: A Double
// Normalization Approach for Calibration-Free Low-Bit Vector Quantization of KV
// Cache" (gist.science/paper/2505.18231), sections "1. Normalize-Shift-Normalize
// (NSN)", "2. Hadamard Transform" and "3. Vector Quantization and Codebook".
//
// Three launches when the channel mean o is computed:
//   k_stats    per-chunk channel sums of y = x / s1 (fixed-order block reduce)
//   k_mean     o = (sum over chunks) / L, fixed order
//   k_encode4  (g = 4) or k_encode8 (g = 8), per token: NSN with that o,
//              Hadamard, nearest centroid, alpha
// With a reused o (the append path) only the per-token kernel runs.
//
// Randomized Hadamard (the random-sign transform section 2 names for its variance
// guarantee; a codebook option): the per-token kernels rotate by H D, D the
// handle's channel signs, by flipping the shift and the loaded channels before
// the transform (a separate template case, so the plain path is unchanged).
//
// Nearest centroid, g = 4: exact pruned search.  After the rotation every lane
// holds one 4-dim sub-vector.  Its cell in a uniform grid over [-4, 4]^4 names at
// most 12 candidate centroids (the table built in nsn_cells.hip keeps every
// centroid that can be nearest somewhere in the cell), and the lane evaluates
// only those: ||v||^2 + ||c||^2 - 2 <v, c> in fp32 from the fp16 centroid.  A
// token with a sub-vector outside the grid (or in a cell whose list overflows)
// falls back to the exhaustive matrix-core search below for the whole token.
//
// Nearest centroid, exhaustive (g = 8, and the g = 4 fallback): a matrix-core
// distance GEMM.  For a column (one sub-vector w) and a row (one centroid C_k)
// the 32x32x16 fp16 MFMA forms
//   D = ||C_k||^2 - 2 <w, C_k> + ||w||^2
// with w split as w_hi + w_lo (both fp16) and ||.||^2 split likewise, so every
// product is exact in fp32 and only the fp32 accumulation rounds.
//
// Both searches pack (distance with its low 8 bits cleared, centroid index) into
// one int, so that v_min3 retires two candidates and exact ties go to the lowest
// index.
#include "nsn_device.h"

namespace nsn {
namespace {

constexpr float kSqrtD = 11.313708498984761f;      // sqrt(128)
constexpr float kInvSqrtD = 0.08838834764831845f;  // 1 / sqrt(128)

// Sum over the N consecutive lanes that hold one token (N = 16: one DPP row;
// N = 32: a half-wave), every lane of the group gets the total.
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

template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N == 32) {
    return half_wave_sum(v);
  } else {
    static_assert(N == 16, "group of 16 or 32 lanes");
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    v += dpp_f<0x141>(v);
    v += dpp_f<0x140>(v);
    return v;
  }
}

// ---------------------------------------------------------------- pass 1
// Grid (nchunk, BH), 256 threads.  Each lane loads 16 bytes (VPL channels) of a
// token; LPT lanes cover one token, a wave covers TPW tokens per load and keeps
// UNR loads in flight.  Per-channel sums of y = x / s1 are reduced over the
// token slots of the block in a fixed order.
// DQ: also the smallest and largest fp16 pattern of the non-zero s1 of the chunk
// (s1mm[chunk] = {min, max}; {0xFFFF, 0} when the chunk has none).
template <typename T, bool DQ>
__global__ __launch_bounds__(256) void k_stats(const T* __restrict__ x, int L, int TC, int nchunk,
                                               float* __restrict__ part, uint32_t* __restrict__ s1mm) {
  constexpr int VPL = 16 / sizeof(T), LPT = kD / VPL, TPW = 64 / LPT, UNR = 4;
  __shared__ float red[4 * TPW][kD];
  __shared__ uint32_t s_mm[2][256];
  uint32_t pmin = 0xFFFFu, pmax = 0u;
  const int bh = blockIdx.y, chunk = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = lane / LPT, p = lane % LPT;
  const int t0 = chunk * TC, t1 = min(L, t0 + TC);
  const T* xb = x + (size_t)bh * L * kD;
  float acc[VPL];
#pragma unroll
  for (int c = 0; c < VPL; ++c) acc[c] = 0.f;
  for (int base = t0 + wave * TPW * UNR; base < t1; base += 4 * TPW * UNR) {
    float v[UNR][VPL];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int t = base + u * TPW + slot;
      if (t < t1) {
        const uint4 raw = *reinterpret_cast<const uint4*>(xb + (size_t)t * kD + p * VPL);
        const T* e = reinterpret_cast<const T*>(&raw);
#pragma unroll
        for (int c = 0; c < VPL; ++c) v[u][c] = (float)e[c];
      } else {
#pragma unroll
        for (int c = 0; c < VPL; ++c) v[u][c] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < VPL; ++c) ss += v[u][c] * v[u][c];
      ss = group_sum<LPT>(ss);
      const float inv = ss > 0.f ? __builtin_amdgcn_rsqf(ss) * kSqrtD : 0.f;  // 1 / s1
      if constexpr (DQ) {
        if (ss > 0.f) {  // s1 as the encode kernel forms it
          const uint32_t b = f16_bits(ss * __builtin_amdgcn_rsqf(ss) * kInvSqrtD);
          pmin = min(pmin, b);
          pmax = max(pmax, b);
        }
      }
#pragma unroll
      for (int c = 0; c < VPL; ++c) acc[c] += v[u][c] * inv;
    }
  }
#pragma unroll
  for (int c = 0; c < VPL; ++c) red[wave * TPW + slot][p * VPL + c] = acc[c];
  __syncthreads();
  if constexpr (DQ) {
    s_mm[0][threadIdx.x] = pmin;
    s_mm[1][threadIdx.x] = pmax;
  }
  __syncthreads();
  if (threadIdx.x < kD) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4 * TPW; ++i) s += red[i][threadIdx.x];
    part[((size_t)bh * nchunk + chunk) * kD + threadIdx.x] = s;
  }
  if constexpr (DQ) {
    if (threadIdx.x == 0) {
      uint32_t a = 0xFFFFu, b = 0u;
      for (int i = 0; i < 256; ++i) {
        a = min(a, s_mm[0][i]);
        b = max(b, s_mm[1][i]);
      }
      s1mm[((size_t)bh * nchunk + chunk) * 2 + 0] = a;
      s1mm[((size_t)bh * nchunk + chunk) * 2 + 1] = b;
    }
  }
}

// ---------------------------------------------------------------- pass 1b
// o = (sum of the chunk partials) / L.  8 groups of 32 threads take every 8th
// chunk (4 channels per thread), then the groups are added in a fixed order.
__global__ __launch_bounds__(256) void k_mean(const float* __restrict__ part, int nchunk, int L,
                                              float* __restrict__ o) {
  __shared__ float4 red[8][32];
  const int bh = blockIdx.x, gi = threadIdx.x >> 5, c4 = threadIdx.x & 31;
  const float4* pp = reinterpret_cast<const float4*>(part + (size_t)bh * nchunk * kD) + c4;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int i = gi; i < nchunk; i += 8) {
    const float4 v = pp[(size_t)i * (kD / 4)];
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  red[gi][c4] = s;
  __syncthreads();
  if (threadIdx.x < 32) {
    float4 t = red[0][c4];
#pragma unroll
    for (int i = 1; i < 8; ++i) {
      t.x += red[i][c4].x; t.y += red[i][c4].y; t.z += red[i][c4].z; t.w += red[i][c4].w;
    }
    const float inv = 1.f / (float)L;
    reinterpret_cast<float4*>(o + (size_t)bh * kD)[c4] = make_float4(t.x * inv, t.y * inv, t.z * inv, t.w * inv);
  }
}

// ---------------------------------------------------------------- pass 1b (DQ)
// The head record of a double-quantized tensor: o as k_mean forms it, then its
// 4-bit absmax codes (scale = max |o| / 7, code = nearest integer of o / scale,
// ties to even), and the s1 grid from the chunks' pattern ranges
// (stride = max(1, ceil((max - min) / 14)); base 0x3C00, stride 1 without a
// non-zero token).
__global__ __launch_bounds__(256) void k_mean_dq(const float* __restrict__ part, const uint32_t* __restrict__ s1mm,
                                                 int nchunk, int L, nsn_dq_head* __restrict__ heads) {
  __shared__ float4 red[8][32];
  __shared__ float s_o[kD];
  __shared__ float s_abs[kD];
  __shared__ uint32_t s_mm[2][256];
  const int bh = blockIdx.x, gi = threadIdx.x >> 5, c4 = threadIdx.x & 31;
  const float4* pp = reinterpret_cast<const float4*>(part + (size_t)bh * nchunk * kD) + c4;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int i = gi; i < nchunk; i += 8) {
    const float4 v = pp[(size_t)i * (kD / 4)];
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  red[gi][c4] = s;
  uint32_t a = 0xFFFFu, b = 0u;
  for (int i = threadIdx.x; i < nchunk; i += 256) {
    a = min(a, s1mm[((size_t)bh * nchunk + i) * 2 + 0]);
    b = max(b, s1mm[((size_t)bh * nchunk + i) * 2 + 1]);
  }
  s_mm[0][threadIdx.x] = a;
  s_mm[1][threadIdx.x] = b;
  __syncthreads();
  if (threadIdx.x < 32) {
    float4 t = red[0][c4];
#pragma unroll
    for (int i = 1; i < 8; ++i) {
      t.x += red[i][c4].x; t.y += red[i][c4].y; t.z += red[i][c4].z; t.w += red[i][c4].w;
    }
    const float inv = 1.f / (float)L;
    const float o4[4] = {t.x * inv, t.y * inv, t.z * inv, t.w * inv};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      s_o[4 * c4 + c] = o4[c];
      s_abs[4 * c4 + c] = fabsf(o4[c]);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = 0.f;
    for (int c = 0; c < kD; ++c) m = fmaxf(m, s_abs[c]);
    const float scale = m / 7.f;
    s_abs[0] = scale;
    uint32_t lo = 0xFFFFu, hi = 0u;
    for (int i = 0; i < 256; ++i) {
      lo = min(lo, s_mm[0][i]);
      hi = max(hi, s_mm[1][i]);
    }
    nsn_dq_head* hd = heads + bh;
    hd->o_scale = scale;
    if (lo > hi) {
      hd->s1_base = 0x3C00;
      hd->s1_stride = 1;
    } else {
      hd->s1_base = (uint16_t)lo;
      hd->s1_stride = (uint16_t)max(1u, (hi - lo + 13u) / 14u);
    }
    hd->reserved[0] = 0u;
    hd->reserved[1] = 0u;
  }
  __syncthreads();
  if (threadIdx.x < kD / 2) {  // byte j: channels 2j (low nibble) and 2j + 1
    const float scale = s_abs[0];
    int q[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float v = scale > 0.f ? rintf(s_o[2 * threadIdx.x + e] / scale) : 0.f;
      q[e] = (int)fminf(fmaxf(v, -7.f), 7.f) + 8;
    }
    heads[bh].o_codes[threadIdx.x] = (uint8_t)(q[0] | (q[1] << 4));
  }
}

// ---------------------------------------------------------------- DQ pack
// Token words (s1 code | s2' << 16) of one call, relative rows [bh][L], to the
// cache: s2 at positions pos0 .. pos0+L-1 and the codes into bytes of two tokens.
// One thread per byte: a byte shared with a token outside the call keeps that
// token's nibble, so appends at any position never race.
__global__ __launch_bounds__(256) void k_dq_pack(const uint32_t* __restrict__ words, int L, int L_cap, int pos0,
                                                 uint16_t* __restrict__ s2, uint8_t* __restrict__ s1c) {
  const int bh = blockIdx.y;
  const int k = (pos0 >> 1) + blockIdx.x * 256 + threadIdx.x;  // byte: positions 2k, 2k + 1
  const int a0 = 2 * k;
  if (a0 >= pos0 + L) return;
  const int capb = (L_cap + 1) >> 1;
  uint8_t* cb = s1c + (size_t)bh * capb + k;
  const uint32_t* wr = words + (size_t)bh * L;
  uint16_t* s2r = s2 + (size_t)bh * L_cap;
  uint32_t nib[2];
  bool in[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int t = a0 + e - pos0;  // token of this call
    in[e] = t >= 0 && t < L;
    nib[e] = 0u;
    if (in[e]) {
      const uint32_t w = wr[t];
      nib[e] = w & 15u;
      s2r[a0 + e] = (uint16_t)(w >> 16);
    }
  }
  if (!in[0] || !in[1]) {
    const uint32_t old = *cb;
    if (!in[0]) nib[0] = old & 15u;
    if (!in[1]) nib[1] = old >> 4;
  }
  *cb = (uint8_t)(nib[0] | (nib[1] << 4));
}

// ---------------------------------------------------------------- pass 2 helpers
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

// ---------------------------------------------------------------- pass 2, g = 4
// Grid (ceil(L / TPB), BH), kEnc4Threads threads (16 waves; two workgroups of
// 64 KB LDS per CU).  Each wave takes token pairs, one token per half-wave; after
// the rotation lane p of a half owns sub-vector p (channels 4p .. 4p+3) of its
// token.  The centroid records sit in LDS 16 times over, one 256-byte row per
// centroid, and lane i reads copy i % 16: a 16-lane group covers all banks
// whatever the centroids, and the row address k * 256 + 16 (i % 16) is one v_perm
// of the index byte.
constexpr int kEnc4Threads = 1024;

__device__ __forceinline__ uint32_t rec_addr(uint32_t word, uint32_t laneoff, int byte) {
  // bytes: [laneoff, byte `byte` of word, 0, 0] -> index * 256 + laneoff
  return __builtin_amdgcn_perm(word, laneoff, 0x0C0C0000u | ((uint32_t)(4 + byte) << 8));
}

// DQ: o_q and the s1 grid come from the head records, and the 32-bit word per
// token is (s1 code | s2' fp16 << 16) at row sc_cap * bh + sc_pos0 + t.
template <typename T, bool DQ, bool RHT>
__global__ __launch_bounds__(kEnc4Threads) __attribute__((amdgpu_waves_per_eu(8, 8))) void k_encode4(
    const T* __restrict__ x, int L, int L_cap, int pos0, int TPB, const float* __restrict__ o,
    const nsn_dq_head* __restrict__ heads, const uint4* __restrict__ cells, const uint4* __restrict__ rec,
    const uint16_t* __restrict__ encA, uint8_t* __restrict__ idx_out, uint16_t* __restrict__ scales_out,
    int sc_cap, int sc_pos0, uint4 smask) {
  constexpr int kWaves4 = kEnc4Threads / 64;
  __shared__ uint4 s_rec[kK * 16];
  const int bh = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, p = lane & 31;
  const int t0 = blockIdx.x * TPB, t1 = min(L, t0 + TPB);
  // uniform bases of this block's tokens; per-lane offsets stay 32-bit
  const T* xblk = x + ((size_t)bh * L + t0) * kD;
  uint8_t* iblk = idx_out + ((size_t)bh * L_cap + pos0 + t0) * (kD / 4);
  uint32_t* sblk = reinterpret_cast<uint32_t*>(scales_out) + ((size_t)bh * sc_cap + sc_pos0 + t0);
  const char* srec = reinterpret_cast<const char*>(s_rec);
  const uint32_t laneoff = (uint32_t)(lane & 15) << 4;

  // Each token pair's channels are loaded one iteration ahead, issued after the
  // cell lookup so that waiting for the lookup does not wait for them; the first
  // pair is loaded before the barrier, so every path into the loop has the same
  // outstanding loads and the compiler's wait at its top stays partial.
  using R4 = typename raw4<T>::type;
  const int nblk = t1 - t0;
  const int xbytes = nblk * kD * (int)sizeof(T);  // this block's rows; loads past them read 0
  const uint32_t xlane = (uint32_t)(half * kD + 4 * p) * (uint32_t)sizeof(T);
  R4 xr = buffer_raw4(xblk, xbytes, xlane + (uint32_t)(2 * wave * kD * sizeof(T)));

  for (int e = tid; e < kK * 16; e += kEnc4Threads) s_rec[e] = rec[e >> 4];
  float ov[4];
  DqS1 dq;
  if constexpr (DQ) {
    dq_o_load(heads + bh, p, ov);
    dq = dq_s1_load(heads + bh);
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) ov[c] = o[(size_t)bh * kD + 4 * p + c];
  }
  // randomized rotation H D: D z = D x / s1 - D o, so the shift and each token's
  // channels are flipped before the transform
  const Sign4 sg = lane_signs(smask, p);
  if constexpr (RHT) flip4(ov, sg);
  __syncthreads();

  for (int base = t0 + 2 * wave; base < t1; base += 2 * kWaves4) {
    const int t = base + half;
    const bool valid = t < t1;
    float h[4], s1, s2, rz;
    bool degen;
    uint32_t s1code = 0;
    const uint32_t tr = (uint32_t)(t - t0);  // token row inside the block
    {
      float xv[4];
      if constexpr (RHT) unpack4(flip_raw(xr, sg), xv);
      else unpack4(xr, xv);
      nsn_rotate<DQ>(xv, p, ov, h, s1, s2, rz, degen, &dq, &s1code);
    }
    // The lane's sub-vector is v = rz h; the search needs only m2 = -2 v (the
    // power-of-two factor keeps it bit-equal to -2 (rz h)), ||v||^2 = ||m2||^2 / 4
    // and the cell of v.
    float m2[4];
    const float r2 = -2.f * rz;
#pragma unroll
    for (int c = 0; c < 4; ++c) m2[c] = h[c] * r2;

    // ---------------- cell of this lane's sub-vector and its candidate row
    const float gs = rz * kGridInv;
    int ic[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) ic[c] = cvt_flr(fmaf(h[c], gs, kGridOff));
    const uint32_t mx = max(max((uint32_t)ic[0], (uint32_t)ic[1]), max((uint32_t)ic[2], (uint32_t)ic[3]));
    const bool inside = mx < (uint32_t)kGridN;
    const uint32_t cell =
        __umul24(__umul24(__umul24((uint32_t)ic[0], kGridN) + (uint32_t)ic[1], kGridN) + (uint32_t)ic[2], kGridN) +
        (uint32_t)ic[3];
    // a sub-vector outside the grid reads past the table: a zero row (count 0)
    const uint4 lst = buffer_load_u4(cells, kGridCells * 16, inside ? cell << 4 : 0x80000000u);
    const bool defer = valid && (!inside || (lst.w >> 24) != 0u);
    xr = buffer_raw4(xblk, xbytes, xlane + (uint32_t)((base - t0 + 2 * kWaves4) * kD * sizeof(T)));

    // ---------------- candidates: key = (bits of ||v||^2 + ||c||^2 - 2 <v, c>) with byte 0 = index
    const float nv = 0.25f * (m2[0] * m2[0] + m2[1] * m2[1] + m2[2] * m2[2] + m2[3] * m2[3]);
    const uint32_t lw[3] = {lst.x, lst.y, lst.z};
    const uint32_t cnt = lst.w & 0xffu;  // list length; the row is padded with its last entry
    int best = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < kCellList; j += 2) {
      // candidates j, j + 1 only while some lane of the wave still has them
      if (j > 0 && __ballot(cnt > (uint32_t)j) == 0) break;
      int key[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int jj = j + u;
        const uint32_t word = lw[jj >> 2];
        const uint4 r = *reinterpret_cast<const uint4*>(srec + rec_addr(word, laneoff, jj & 3));
        float d = nv + __uint_as_float(r.z);
        d = fmaf(m2[0], f16_lo(r.x), d);
        d = fmaf(m2[1], f16_hi(r.x), d);
        d = fmaf(m2[2], f16_lo(r.y), d);
        d = fmaf(m2[3], f16_hi(r.y), d);
        // bytes 1..3 from the distance, byte 0 = candidate index (byte jj % 4 of the row word)
        key[u] = (int)__builtin_amdgcn_perm(__float_as_uint(d), word, 0x07060500u | (uint32_t)(jj & 3));
      }
      best = min(min(best, key[0]), key[1]);
    }

    // ---------------- rare: exhaustive search for tokens with a deferred sub-vector
    const uint64_t dm = __ballot(defer);
    if (dm != 0) {
      // B pieces of this lane's sub-vector: P = (-2 v) hi | lo, Q = (1, 1, ||v||^2 hi, lo)
      half8 P, Q;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const _Float16 ah = (_Float16)m2[e];
        P[e] = ah;
        P[4 + e] = (_Float16)(m2[e] - (float)ah);
      }
      const _Float16 nh = (_Float16)nv;
      Q[0] = (_Float16)1.f; Q[1] = (_Float16)1.f; Q[2] = nh; Q[3] = (_Float16)(nv - (float)nh);
      Q[4] = (_Float16)0.f; Q[5] = (_Float16)0.f; Q[6] = (_Float16)0.f; Q[7] = (_Float16)0.f;
      // column set of the token of half tau: lanes 0-31 take P, lanes 32-63 take Q,
      // both from the lanes of half tau
      uint4 pw = __builtin_bit_cast(uint4, P), qw = __builtin_bit_cast(uint4, Q);
      uint32_t b0[4], b1[4];
      const uint32_t pa[4] = {pw.x, pw.y, pw.z, pw.w}, qa[4] = {qw.x, qw.y, qw.z, qw.w};
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const auto r = __builtin_amdgcn_permlane32_swap(pa[d], qa[d], false, false);
        b0[d] = r[0];  // {P of half 0, Q of half 0}
        b1[d] = r[1];  // {P of half 1, Q of half 1}
      }
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        if (((dm >> (32 * tau)) & 0xffffffffull) == 0) continue;
        const uint32_t* bb = tau ? b1 : b0;
        const half8 B = __builtin_bit_cast(half8, make_uint4(bb[0], bb[1], bb[2], bb[3]));
        const int col = mfma_argmin_col4(B, encA, lane);
        if (half == tau && defer) best = col;
      }
    }
    const uint32_t k = (uint32_t)best & 0xffu;

    // ---------------- alpha = ||w||^2 / <w, w_hat> = d / <w, w_hat> = -2 d / <m2, w_hat>
    const uint4 rk = *reinterpret_cast<const uint4*>(srec + rec_addr((uint32_t)best, laneoff, 0));
    float dot = m2[0] * f16_lo(rk.x);
    dot = fmaf(m2[1], f16_hi(rk.x), dot);
    dot = fmaf(m2[2], f16_lo(rk.y), dot);
    dot = fmaf(m2[3], f16_hi(rk.y), dot);
    dot = half_sum_swz(dot);  // -2 <w, w_hat>
    // rows of tokens past t1 lie outside both descriptors: those stores are dropped
    buffer_store_u8((uint8_t)k, iblk, nblk * (kD / 4), tr * (kD / 4) + p);
    const float alpha = (!degen && dot < 0.f) ? (-2.f * kD) * __builtin_amdgcn_rcpf(dot) : 1.f;
    const uint32_t sw = (DQ ? s1code : (uint32_t)f16_bits(s1)) | ((uint32_t)f16_bits(s2 * alpha) << 16);
    buffer_store_u32(sw, sblk, nblk * 4, p == 0 ? 4 * tr : 0x80000000u);  // one writer per token
  }
}

// ---------------------------------------------------------------- pass 2, g = 8
// Grid (ceil(L / TPB), BH), 256 threads.  Each wave takes token pairs.
//  phase A (pair layout): NSN + Hadamard, one token per half-wave -> LDS
//  phase B (MFMA layout): column c = lane % 32 is sub-vector c % 16 of token
//           c / 16; the two lane halves hold the hi and lo parts of -2 w and
//           complementary rows of the 32x32 result.
template <typename T, bool DQ, bool RHT>
__global__ __launch_bounds__(256) void k_encode8(const T* __restrict__ x, int L, int L_cap, int pos0,
                                                 int TPB, const float* __restrict__ o,
                                                 const nsn_dq_head* __restrict__ heads,
                                                 const uint16_t* __restrict__ encA,
                                                 const float* __restrict__ c32,
                                                 uint8_t* __restrict__ idx_out,
                                                 uint16_t* __restrict__ scales_out, int sc_cap, int sc_pos0,
                                                 uint4 smask) {
  constexpr int G = 8, M = kD / G;
  __shared__ float s_c[kK * G];
  __shared__ float s_w[4][2][kD];
  const int bh = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, p = lane & 31;
  for (int i = tid; i < kK * G; i += 256) s_c[i] = c32[i];

  // A fragments of the distance GEMM: tile t holds centroids 32t .. 32t+31.
  half8 A[kTiles];
  half8 Ax[kTiles];
#pragma unroll
  for (int t = 0; t < kTiles; ++t) {
    A[t] = *reinterpret_cast<const half8*>(encA + ((size_t)(t * 2 + 0) * 64 + lane) * 8);
    Ax[t] = *reinterpret_cast<const half8*>(encA + ((size_t)(t * 2 + 1) * 64 + lane) * 8);
  }
  float ov[4];
  DqS1 dq;
  if constexpr (DQ) {
    dq_o_load(heads + bh, p, ov);
    dq = dq_s1_load(heads + bh);
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) ov[c] = o[(size_t)bh * kD + 4 * p + c];
  }
  // randomized rotation H D: D z = D x / s1 - D o, so the shift and each token's
  // channels are flipped before the transform
  const Sign4 sg = lane_signs(smask, p);
  if constexpr (RHT) flip4(ov, sg);
  __syncthreads();

  const T* xb = x + (size_t)bh * L * kD;
  const size_t out_row0 = (size_t)bh * L_cap + pos0;
  const size_t sc_row0 = (size_t)bh * sc_cap + sc_pos0;
  const int t0 = blockIdx.x * TPB, t1 = min(L, t0 + TPB);
  float* wv = s_w[wave][0];

  for (int base = t0 + 2 * wave; base < t1; base += 8) {
    // ---------------- phase A: NSN + Hadamard, one token per half-wave
    const int t = base + half;
    float z[4], s1, s2;
    bool degen;
    float xv[4] = {0.f, 0.f, 0.f, 0.f};
    if (t < t1) load4(xb + (size_t)t * kD, p, xv);
    if constexpr (RHT) flip4(xv, sg);
    float rz;
    uint32_t s1code = 0;
    nsn_rotate<DQ>(xv, p, ov, z, s1, s2, rz, degen, &dq, &s1code);
#pragma unroll
    for (int c = 0; c < 4; ++c) z[c] *= rz;  // H_sylvester z / ||z|| = (H / sqrt(d)) u
#pragma unroll
    for (int c = 0; c < 4; ++c) wv[half * kD + 4 * p + c] = z[c];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---------------- phase B: distance GEMM + argmin + alpha
    const int h = half, col = p;
    const int tok = col >> 4, sv = col & 15;
    float w[G];
#pragma unroll
    for (int e = 0; e < G; ++e) w[e] = wv[tok * kD + sv * G + e];
    float wn = 0.f;
#pragma unroll
    for (int e = 0; e < G; ++e) wn += w[e] * w[e];
    const _Float16 wn_hi = (_Float16)wn;
    const _Float16 wn_lo = (_Float16)(wn - (float)wn_hi);
    half8 Bf, Bx;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float a = -2.f * w[e];
      const _Float16 ah = (_Float16)a;
      Bf[e] = h == 0 ? ah : (_Float16)(a - (float)ah);
    }
    if (h == 0) {
      Bx[0] = (_Float16)1.f; Bx[1] = (_Float16)1.f; Bx[2] = wn_hi; Bx[3] = wn_lo;
    } else {
      Bx[0] = (_Float16)0.f; Bx[1] = (_Float16)0.f; Bx[2] = (_Float16)0.f; Bx[3] = (_Float16)0.f;
    }
    Bx[4] = (_Float16)0.f; Bx[5] = (_Float16)0.f; Bx[6] = (_Float16)0.f; Bx[7] = (_Float16)0.f;
    int best = 0x7fffffff;
    // software pipelined: tile tt+1's MFMA is in flight while tile tt's keys reduce
    floatx16 Dn = {};
    Dn = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[0], Bf, Dn, 0, 0, 0);
    Dn = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ax[0], Bx, Dn, 0, 0, 0);
#pragma unroll
    for (int tt = 0; tt < kTiles; ++tt) {
      const floatx16 D = Dn;
      if (tt + 1 < kTiles) {
        floatx16 Z = {};
        Dn = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[tt + 1], Bf, Z, 0, 0, 0);
        Dn = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ax[tt + 1], Bx, Dn, 0, 0, 0);
      }
      // row of register r in this lane half: 8 (r / 4) + 4 h + r % 4 -> centroid 32 tt + row.
      // Keys carry the in-tile row tag 8 (r / 4) + r % 4 (< 32, an inline constant);
      // the tile base 32 tt is added once per tile and the half bit 4 h once at the end.
      int tb = 0x7fffffff;
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float d0 = D[r], d1 = D[r + 1];
        const int key0 = (__float_as_int(d0) & ~0xff) | (8 * (r >> 2) + (r & 3));
        const int key1 = (__float_as_int(d1) & ~0xff) | (8 * ((r + 1) >> 2) + ((r + 1) & 3));
        tb = min(min(tb, key0), key1);  // one v_min3
      }
      best = min(best, tb + 32 * tt);
    }
    best |= h << 2;
    {
      const auto r = __builtin_amdgcn_permlane32_swap((uint32_t)best, (uint32_t)best, false, false);
      best = min((int)r[0], (int)r[1]);
    }
    const int k = best & 0xff;
    // alpha = ||w||^2 / <w, w_hat>; <w, w_hat> summed over the 16 columns of the token
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < G; ++e) dot += w[e] * s_c[k * G + e];
    dot += dpp_f<0xB1>(dot);
    dot += dpp_f<0x4E>(dot);
    dot += dpp_f<0x141>(dot);
    dot += dpp_f<0x140>(dot);  // sum over the 16-lane row = the token's 16 columns
    const int tg = base + tok;  // token of this column
    if (h == 0 && tg < t1) idx_out[(out_row0 + tg) * M + sv] = (uint8_t)k;
    // scale writer: a lane of the half that ran phase A for this token, with that token's dot
    const bool writer = (lane == 0 || lane == 48);
    if (writer && tg < t1) {
      const float alpha = (!degen && dot > 0.f) ? (float)kD * __builtin_amdgcn_rcpf(dot) : 1.f;
      const uint32_t packed = (DQ ? s1code : (uint32_t)f16_bits(s1)) | ((uint32_t)f16_bits(s2 * alpha) << 16);
      *reinterpret_cast<uint32_t*>(scales_out + (sc_row0 + tg) * 2) = packed;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }
}

int pick_tpb(int BH, int L) {
  // aim for >= ~2048 blocks on 256 CUs, 128 .. 512 tokens per block
  long total = (long)BH * L;
  long tpb = total / 2048;
  tpb = (tpb + 7) / 8 * 8;
  if (tpb < 128) tpb = 128;
  if (tpb > 512) tpb = 512;
  return (int)tpb;
}

int pick_tpb4(int BH, int L) {
  // about 1024 workgroups (two rounds of two per CU), a multiple of the 32
  // tokens one pass of the 16 waves covers
  long tpb = ((long)BH * L + 1023) / 1024;
  tpb = (tpb + 31) / 32 * 32;
  if (tpb < 32) tpb = 32;
  return (int)tpb;
}

int stats_tc(int BH, int L) {
  // >= ~2048 blocks when the tensor is long, 1024 .. 8192 tokens per block
  long tc = (long)BH * L / 2048;
  tc = (tc + 255) / 256 * 256;
  if (tc < 1024) tc = 1024;
  if (tc > 8192) tc = 8192;
  return (int)tc;
}

// Per-token kernel of one call: plain (scales = (s1 | s2') at (L_cap, pos0)) or
// DQ (words = (code | s2') at rows [bh][L]).
template <bool DQ, bool RHT>
hipError_t launch_token_kernel_s(const nsn_codebook* cb, const void* x, int x_dtype, int BH, int L, int L_cap,
                                 int pos0, const float* o, const nsn_dq_head* heads, uint8_t* idx,
                                 uint16_t* scales, int sc_cap, int sc_pos0, hipStream_t st) {
  const uint4 sm = make_uint4(cb->sgn[0], cb->sgn[1], cb->sgn[2], cb->sgn[3]);
  if (cb->g == 4) {
    const int tpb = pick_tpb4(BH, L);
    dim3 g2((L + tpb - 1) / tpb, BH);
    if (x_dtype == NSN_F16)
      k_encode4<_Float16, DQ, RHT><<<g2, kEnc4Threads, 0, st>>>(static_cast<const _Float16*>(x), L, L_cap, pos0,
                                                                tpb, o, heads, cb->d_cells, cb->d_rec, cb->d_encA,
                                                                idx, scales, sc_cap, sc_pos0, sm);
    else
      k_encode4<float, DQ, RHT><<<g2, kEnc4Threads, 0, st>>>(static_cast<const float*>(x), L, L_cap, pos0, tpb, o,
                                                             heads, cb->d_cells, cb->d_rec, cb->d_encA, idx, scales,
                                                             sc_cap, sc_pos0, sm);
  } else {
    const int tpb = pick_tpb(BH, L);
    dim3 g2((L + tpb - 1) / tpb, BH);
    if (x_dtype == NSN_F16)
      k_encode8<_Float16, DQ, RHT><<<g2, 256, 0, st>>>(static_cast<const _Float16*>(x), L, L_cap, pos0, tpb, o,
                                                       heads, cb->d_encA, cb->d_c32, idx, scales, sc_cap, sc_pos0,
                                                       sm);
    else
      k_encode8<float, DQ, RHT><<<g2, 256, 0, st>>>(static_cast<const float*>(x), L, L_cap, pos0, tpb, o, heads,
                                                    cb->d_encA, cb->d_c32, idx, scales, sc_cap, sc_pos0, sm);
  }
  return hipGetLastError();
}

template <bool DQ>
hipError_t launch_token_kernel(const nsn_codebook* cb, const void* x, int x_dtype, int BH, int L, int L_cap,
                               int pos0, const float* o, const nsn_dq_head* heads, uint8_t* idx,
                               uint16_t* scales, int sc_cap, int sc_pos0, hipStream_t st) {
  return cb->rht ? launch_token_kernel_s<DQ, true>(cb, x, x_dtype, BH, L, L_cap, pos0, o, heads, idx, scales,
                                                   sc_cap, sc_pos0, st)
                 : launch_token_kernel_s<DQ, false>(cb, x, x_dtype, BH, L, L_cap, pos0, o, heads, idx, scales,
                                                    sc_cap, sc_pos0, st);
}

int stats_chunks(int BH, int L) { return (L + stats_tc(BH, L) - 1) / stats_tc(BH, L); }

}  // namespace

size_t encode_ws_bytes(int BH, int L) {
  return (size_t)BH * stats_chunks(BH, L) * kD * sizeof(float);
}

// DQ workspace: [chunk partials][s1 pattern ranges][token words], 256-byte aligned pieces.
static size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }
size_t encode_dq_ws_bytes(int BH, int L) {
  return align256(encode_ws_bytes(BH, L)) + align256((size_t)BH * stats_chunks(BH, L) * 2 * sizeof(uint32_t)) +
         (size_t)BH * L * sizeof(uint32_t);
}

hipError_t launch_encode(const nsn_codebook* cb, const void* x, int x_dtype, int BH, int L, int L_cap,
                         int pos0, int o_mode, float* o, uint8_t* idx, uint16_t* scales, void* ws,
                         hipStream_t st) {
  if (o_mode == NSN_O_COMPUTE) {
    const int tc = stats_tc(BH, L);
    const int nchunk = (L + tc - 1) / tc;
    float* part = static_cast<float*>(ws);
    dim3 g1(nchunk, BH);
    if (x_dtype == NSN_F16)
      k_stats<_Float16, false><<<g1, 256, 0, st>>>(static_cast<const _Float16*>(x), L, tc, nchunk, part, nullptr);
    else
      k_stats<float, false><<<g1, 256, 0, st>>>(static_cast<const float*>(x), L, tc, nchunk, part, nullptr);
    k_mean<<<BH, 256, 0, st>>>(part, nchunk, L, o);
  }
  hipError_t e = launch_token_kernel<false>(cb, x, x_dtype, BH, L, L_cap, pos0, o, nullptr, idx, scales, L_cap, pos0,
                                            st);
  return e;
}

hipError_t launch_encode_dq(const nsn_codebook* cb, const void* x, int x_dtype, int BH, int L, int L_cap,
                            int pos0, int o_mode, nsn_dq_head* heads, uint8_t* idx, uint16_t* s2, uint8_t* s1c,
                            void* ws, hipStream_t st) {
  char* wsb = static_cast<char*>(ws);
  const int tc = stats_tc(BH, L);
  const int nchunk = stats_chunks(BH, L);
  float* part = reinterpret_cast<float*>(wsb);
  uint32_t* s1mm = reinterpret_cast<uint32_t*>(wsb + align256(encode_ws_bytes(BH, L)));
  uint32_t* words = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(s1mm) +
                                                align256((size_t)BH * nchunk * 2 * sizeof(uint32_t)));
  if (o_mode == NSN_O_COMPUTE) {
    dim3 g1(nchunk, BH);
    if (x_dtype == NSN_F16)
      k_stats<_Float16, true><<<g1, 256, 0, st>>>(static_cast<const _Float16*>(x), L, tc, nchunk, part, s1mm);
    else
      k_stats<float, true><<<g1, 256, 0, st>>>(static_cast<const float*>(x), L, tc, nchunk, part, s1mm);
    k_mean_dq<<<BH, 256, 0, st>>>(part, s1mm, nchunk, L, heads);
  }
  hipError_t e = launch_token_kernel<true>(cb, x, x_dtype, BH, L, L_cap, pos0, nullptr, heads, idx,
                                           reinterpret_cast<uint16_t*>(words), L, 0, st);
  if (e != hipSuccess) return e;
  const int nbytes = ((pos0 + L - 1) >> 1) - (pos0 >> 1) + 1;
  dim3 g3((nbytes + 255) / 256, BH);
  k_dq_pack<<<g3, 256, 0, st>>>(words, L, L_cap, pos0, s2, s1c);
  return hipGetLastError();
}

}  // namespace nsn
