// NSNQuant encode on gfx950: Normalize-Shift-Normalize, Hadamard rotation and
// nearest-centroid vector quantization with the scale adjustment.
//
// Follows the Technical Summary of the explainer "NSNQuant: A Double
// Normalization Approach for Calibration-Free Low-Bit Vector Quantization of KV
// Cache" (gist.science/paper/2505.18231), sections "1. Normalize-Shift-Normalize
// (NSN)", "2. Hadamard Transform" and "3. Vector Quantization and Codebook".
//
// Three launches when the channel mean o is computed:
//   k_stats   per-chunk channel sums of y = x / s1 (fixed-order block reduce)
//   k_mean    o = (sum over chunks) / L, fixed order
//   k_encode  per token: NSN with that o, Hadamard, nearest centroid, alpha
// With a reused o (the append path) only k_encode runs.
//
// Nearest centroid is a matrix-core distance GEMM: for a column (one sub-vector
// w) and a row (one centroid C_k) the 32x32x16 fp16 MFMA forms
//   D = ||C_k||^2 - 2 <w, C_k> + ||w||^2
// with w split as w_hi + w_lo (both fp16) and ||.||^2 split likewise, so every
// product is exact in fp32 and only the fp32 accumulation rounds.  The argmin
// packs (distance with its low 8 bits cleared, centroid index) into one int so
// that one v_min3 retires two candidates; exact ties go to the lowest index.
#include "nsn_device.h"

namespace nsn {
namespace {

// ---------------------------------------------------------------- pass 1
// Grid (nchunk, BH); chunk = TC tokens; 4 waves, each takes token pairs.
template <typename T>
__global__ __launch_bounds__(256) void k_stats(const T* __restrict__ x, int L, int TC, int nchunk,
                                               float* __restrict__ part) {
  __shared__ float red[8][kD];
  const int bh = blockIdx.y, chunk = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, p = lane & 31;
  const int t0 = chunk * TC, t1 = min(L, t0 + TC);
  const T* xb = x + (size_t)bh * L * kD;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int base = t0 + 2 * wave; base < t1; base += 8) {
    const int t = base + half;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (t < t1) load4(xb + (size_t)t * kD, p, v);
    const float ss = half_wave_sum(v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3]);
    const float inv = ss > 0.f ? sqrtf((float)kD / ss) : 0.f;  // 1 / s1
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] += v[c] * inv;
  }
  const int hw = wave * 2 + half;
#pragma unroll
  for (int c = 0; c < 4; ++c) red[hw][4 * p + c] = acc[c];
  __syncthreads();
  if (threadIdx.x < kD) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += red[i][threadIdx.x];
    part[((size_t)bh * nchunk + chunk) * kD + threadIdx.x] = s;
  }
}

// ---------------------------------------------------------------- pass 1b
__global__ __launch_bounds__(128) void k_mean(const float* __restrict__ part, int nchunk, int L,
                                              float* __restrict__ o) {
  const int bh = blockIdx.x, c = threadIdx.x;
  const float* pp = part + (size_t)bh * nchunk * kD + c;
  float s = 0.f;
  for (int i = 0; i < nchunk; ++i) s += pp[(size_t)i * kD];
  o[(size_t)bh * kD + c] = s / (float)L;
}

// ---------------------------------------------------------------- pass 2
// Grid (ceil(L / TPB), BH), 256 threads.  Each wave takes token pairs.
//  phase A (pair layout): s1, z = y - o, s2, u, w = H u     -> LDS
//  phase B (MFMA layout): column c = lane % 32 is one sub-vector; the two lane
//           halves (h = lane / 32) hold complementary K-slots of the operand
//           and complementary rows of the 32x32 result.
// G = 4: one 32-column set per token (m = 32); G = 8: one set per pair (m = 16).
template <int G, typename T>
__global__ __launch_bounds__(256) void k_encode(const T* __restrict__ x, int L, int L_cap, int pos0,
                                                int TPB, const float* __restrict__ o,
                                                const uint16_t* __restrict__ encA,
                                                const float* __restrict__ c32,
                                                uint8_t* __restrict__ idx_out,
                                                uint16_t* __restrict__ scales_out) {
  constexpr int M = kD / G;
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
    if (G == 8) Ax[t] = *reinterpret_cast<const half8*>(encA + ((size_t)(t * 2 + 1) * 64 + lane) * 8);
  }
  float ov[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) ov[c] = o[(size_t)bh * kD + 4 * p + c];
  __syncthreads();

  const T* xb = x + (size_t)bh * L * kD;
  const size_t out_row0 = (size_t)bh * L_cap + pos0;
  const int t0 = blockIdx.x * TPB, t1 = min(L, t0 + TPB);
  float* wv = s_w[wave][0];

  for (int base = t0 + 2 * wave; base < t1; base += 8) {
    // ---------------- phase A: NSN + Hadamard, one token per half-wave
    const int t = base + half;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (t < t1) load4(xb + (size_t)t * kD, p, v);
    const float ss = half_wave_sum(v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3]);
    const float s1 = sqrtf(ss / (float)kD);
    const float inv1 = ss > 0.f ? sqrtf((float)kD / ss) : 0.f;
    float z[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) z[c] = v[c] * inv1 - ov[c];
    const float zz = half_wave_sum(z[0] * z[0] + z[1] * z[1] + z[2] * z[2] + z[3] * z[3]);
    const float rel = sqrtf(zz / (float)kD);  // ||z|| / sqrt(d)
    const bool degen = !(rel > kEpsZ);
    const float s2 = degen ? 0.f : rel;
    const float f = degen ? 0.f : 1.0f / sqrtf(zz);  // u / sqrt(d) = z / (s2 sqrt(d))
#pragma unroll
    for (int c = 0; c < 4; ++c) z[c] *= f;
    fwht128_pair(z, p);  // w = (H / sqrt(d)) u
#pragma unroll
    for (int c = 0; c < 4; ++c) wv[half * kD + 4 * p + c] = z[c];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---------------- phase B: distance GEMM + argmin + alpha
    const int h = half, col = p;
#pragma unroll
    for (int cs = 0; cs < (G == 4 ? 2 : 1); ++cs) {
      const int tok = (G == 4) ? cs : (col >> 4);
      const int sv = (G == 4) ? col : (col & 15);
      float w[G];
#pragma unroll
      for (int e = 0; e < G; ++e) w[e] = wv[tok * kD + sv * G + e];
      float wn = 0.f;
#pragma unroll
      for (int e = 0; e < G; ++e) wn += w[e] * w[e];
      const _Float16 wn_hi = (_Float16)wn;
      const _Float16 wn_lo = (_Float16)(wn - (float)wn_hi);
      half8 Bf, Bx;
      if (G == 4) {
        if (h == 0) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float a = -2.f * w[e];
            const _Float16 ah = (_Float16)a;
            Bf[e] = ah;
            Bf[4 + e] = (_Float16)(a - (float)ah);
          }
        } else {
          Bf[0] = (_Float16)1.f; Bf[1] = (_Float16)1.f; Bf[2] = wn_hi; Bf[3] = wn_lo;
          Bf[4] = (_Float16)0.f; Bf[5] = (_Float16)0.f; Bf[6] = (_Float16)0.f; Bf[7] = (_Float16)0.f;
        }
      } else {
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
      }
      int best = 0x7fffffff;
#pragma unroll
      for (int tt = 0; tt < kTiles; ++tt) {
        floatx16 D = {};
        D = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[tt], Bf, D, 0, 0, 0);
        if (G == 8) D = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ax[tt], Bx, D, 0, 0, 0);
        // row of register r in this lane half: 8 (r / 4) + 4 h + r % 4 -> centroid 32 tt + row
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const int k0 = 32 * tt + 8 * (r >> 2) + (r & 3);
          const int k1 = 32 * tt + 8 * ((r + 1) >> 2) + ((r + 1) & 3);
          // copy the element out first: a bit cast of a vector element
          // expression would read the vector's first element instead
          const float d0 = D[r], d1 = D[r + 1];
          const int key0 = (__float_as_int(d0) & ~0xff) | k0;
          const int key1 = (__float_as_int(d1) & ~0xff) | k1;
          best = min(best, min(key0, key1));
        }
      }
      best |= h << 2;
      best = min(best, __shfl_xor(best, 32));
      const int k = best & 0xff;
      // alpha = ||w||^2 / <w, w_hat>; <w, w_hat> summed over the token's sub-vectors
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < G; ++e) dot += w[e] * s_c[k * G + e];
#pragma unroll
      for (int msk = 1; msk < (G == 4 ? 32 : 16); msk <<= 1) dot += __shfl_xor(dot, msk);
      const int tg = base + tok;  // token of this column
      if (h == 0 && tg < t1) idx_out[(out_row0 + tg) * M + sv] = (uint8_t)k;
      // scale writer: a lane of the half that ran phase A for this token, with that token's dot
      const bool writer = (G == 4) ? (lane == 32 * cs) : (lane == 0 || lane == 48);
      if (writer && tg < t1) {
        const float alpha = (!degen && dot > 0.f) ? (float)kD / dot : 1.f;
        const uint32_t packed = (uint32_t)f16_bits(s1) | ((uint32_t)f16_bits(s2 * alpha) << 16);
        *reinterpret_cast<uint32_t*>(scales_out + (out_row0 + tg) * 2) = packed;
      }
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

constexpr int kStatsTC = 256;

}  // namespace

size_t encode_ws_bytes(int BH, int L) {
  const int nchunk = (L + kStatsTC - 1) / kStatsTC;
  return (size_t)BH * nchunk * kD * sizeof(float);
}

hipError_t launch_encode(const nsn_codebook* cb, const void* x, int x_dtype, int BH, int L, int L_cap,
                         int pos0, int o_mode, float* o, uint8_t* idx, uint16_t* scales, void* ws,
                         hipStream_t st) {
  if (o_mode == NSN_O_COMPUTE) {
    const int nchunk = (L + kStatsTC - 1) / kStatsTC;
    float* part = static_cast<float*>(ws);
    dim3 g1(nchunk, BH);
    if (x_dtype == NSN_F16)
      k_stats<_Float16><<<g1, 256, 0, st>>>(static_cast<const _Float16*>(x), L, kStatsTC, nchunk, part);
    else
      k_stats<float><<<g1, 256, 0, st>>>(static_cast<const float*>(x), L, kStatsTC, nchunk, part);
    k_mean<<<BH, 128, 0, st>>>(part, nchunk, L, o);
  }
  const int tpb = pick_tpb(BH, L);
  dim3 g2((L + tpb - 1) / tpb, BH);
  if (cb->g == 4) {
    if (x_dtype == NSN_F16)
      k_encode<4, _Float16><<<g2, 256, 0, st>>>(static_cast<const _Float16*>(x), L, L_cap, pos0, tpb, o,
                                                cb->d_encA, cb->d_c32, idx, scales);
    else
      k_encode<4, float><<<g2, 256, 0, st>>>(static_cast<const float*>(x), L, L_cap, pos0, tpb, o,
                                             cb->d_encA, cb->d_c32, idx, scales);
  } else {
    if (x_dtype == NSN_F16)
      k_encode<8, _Float16><<<g2, 256, 0, st>>>(static_cast<const _Float16*>(x), L, L_cap, pos0, tpb, o,
                                                cb->d_encA, cb->d_c32, idx, scales);
    else
      k_encode<8, float><<<g2, 256, 0, st>>>(static_cast<const float*>(x), L, L_cap, pos0, tpb, o,
                                             cb->d_encA, cb->d_c32, idx, scales);
  }
  return hipGetLastError();
}

}  // namespace nsn
