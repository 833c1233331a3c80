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
// Grid (nchunk, BH), 256 threads.  Each lane loads 16 bytes (VPL channels) of a
// token; LPT lanes cover one token, a wave covers TPW tokens per load and keeps
// UNR loads in flight.  Per-channel sums of y = x / s1 are reduced over the
// token slots of the block in a fixed order.
template <typename T>
__global__ __launch_bounds__(256) void k_stats(const T* __restrict__ x, int L, int TC, int nchunk,
                                               float* __restrict__ part) {
  constexpr int VPL = 16 / sizeof(T), LPT = kD / VPL, TPW = 64 / LPT, UNR = 4;
  __shared__ float red[4 * TPW][kD];
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
#pragma unroll
      for (int m = 1; m < LPT; m <<= 1) ss += __shfl_xor(ss, m);
      const float inv = ss > 0.f ? sqrtf((float)kD / ss) : 0.f;  // 1 / s1
#pragma unroll
      for (int c = 0; c < VPL; ++c) acc[c] += v[u][c] * inv;
    }
  }
#pragma unroll
  for (int c = 0; c < VPL; ++c) red[wave * TPW + slot][p * VPL + c] = acc[c];
  __syncthreads();
  if (threadIdx.x < kD) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4 * TPW; ++i) s += red[i][threadIdx.x];
    part[((size_t)bh * nchunk + chunk) * kD + threadIdx.x] = s;
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
      // software pipelined: tile tt+1's MFMA is in flight while tile tt's keys reduce
      floatx16 Dn = {};
      Dn = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[0], Bf, Dn, 0, 0, 0);
      if (G == 8) Dn = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ax[0], Bx, Dn, 0, 0, 0);
#pragma unroll
      for (int tt = 0; tt < kTiles; ++tt) {
        const floatx16 D = Dn;
        if (tt + 1 < kTiles) {
          floatx16 Z = {};
          Dn = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[tt + 1], Bf, Z, 0, 0, 0);
          if (G == 8) Dn = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ax[tt + 1], Bx, Dn, 0, 0, 0);
        }
        // row of register r in this lane half: 8 (r / 4) + 4 h + r % 4 -> centroid 32 tt + row.
        // Keys carry the in-tile row tag 8 (r / 4) + r % 4 (< 32, an inline constant);
        // the tile base 32 tt is added once per tile and the half bit 4 h once at the end.
        int tb = 0x7fffffff;
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          // copy the element out first: a bit cast of a vector element
          // expression would read the vector's first element instead
          const float d0 = D[r], d1 = D[r + 1];
          const int key0 = (__float_as_int(d0) & ~0xff) | (8 * (r >> 2) + (r & 3));
          const int key1 = (__float_as_int(d1) & ~0xff) | (8 * ((r + 1) >> 2) + ((r + 1) & 3));
          tb = min(min(tb, key0), key1);  // one v_min3
        }
        best = min(best, tb + 32 * tt);
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

int stats_tc(int BH, int L) {
  // >= ~2048 blocks when the tensor is long, 1024 .. 8192 tokens per block
  long tc = (long)BH * L / 2048;
  tc = (tc + 255) / 256 * 256;
  if (tc < 1024) tc = 1024;
  if (tc > 8192) tc = 8192;
  return (int)tc;
}

}  // namespace

size_t encode_ws_bytes(int BH, int L) {
  const int nchunk = (L + stats_tc(BH, L) - 1) / stats_tc(BH, L);
  return (size_t)BH * nchunk * kD * sizeof(float);
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
      k_stats<_Float16><<<g1, 256, 0, st>>>(static_cast<const _Float16*>(x), L, tc, nchunk, part);
    else
      k_stats<float><<<g1, 256, 0, st>>>(static_cast<const float*>(x), L, tc, nchunk, part);
    k_mean<<<BH, 256, 0, st>>>(part, nchunk, L, o);
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
