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
#include <algorithm>

#include "nsn_pair.h"

namespace nsn {
namespace {

// Sum over the N consecutive lanes that hold one token (N = 16: one DPP row;
// N = 32: a half-wave), every lane of the group gets the total.
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

// 16 bytes at byte offset voff of [base, base + bytes) (zeros past the end),
// streaming (nt sc1: read once, kept out of the L2's way)
__device__ __forceinline__ uint4 buffer_load_x16(const void* base, int bytes, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)voff, 0, 18));
#else
  (void)base; (void)bytes; (void)voff;
  return uint4{};
#endif
}

// ---------------------------------------------------------------- pass 1
// Grid (nchunk, BH), 256 threads, about four workgroups per compute unit, all
// resident at once (a second, partial round of workgroups would run with the
// chip mostly idle).  Each lane loads 16 bytes (VPL channels) of a token; LPT
// lanes cover one token, a wave covers TPW tokens per load and issues UNR = 16
// loads (16 KB) per iteration before it sums the first.  Per-channel sums of
// y = x / s1 are reduced over the token slots of the block in a fixed order.
// DQ: also the smallest and largest fp16 pattern of the non-zero s1 of the chunk
// (s1mm[chunk] = {min, max}; {0xFFFF, 0} when the chunk has none).
template <typename T, bool DQ>
__global__ __launch_bounds__(256) void k_stats(const T* __restrict__ x, int L, int TC, int nchunk,
                                               float* __restrict__ part, uint32_t* __restrict__ s1mm) {
  constexpr int VPL = 16 / sizeof(T), LPT = kD / VPL, TPW = 64 / LPT, UNR = 16;
  constexpr int SPAN = 4 * TPW * UNR;  // tokens of one block iteration
  constexpr uint32_t kUStride = TPW * kD * sizeof(T), kItStride = SPAN * kD * sizeof(T);
  __shared__ float red[4 * TPW][kD];
  __shared__ uint32_t s_mm[2][256];
  uint32_t pmin = 0xFFFFu, pmax = 0u;
  const int bh = blockIdx.y, chunk = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = lane / LPT, p = lane % LPT;
  const int t0 = chunk * TC, t1 = min(L, t0 + TC);
  // the chunk's rows as one buffer: loads past t1 read zeros, and a zero token
  // adds nothing (its 1 / s1 is taken as 0)
  const T* xc = x + ((size_t)bh * L + t0) * kD;
  const int bytes = (t1 - t0) * kD * (int)sizeof(T);
  const uint32_t voff0 = (uint32_t)(((wave * TPW * UNR + slot) * kD + p * VPL) * sizeof(T));
  float acc[VPL];
#pragma unroll
  for (int c = 0; c < VPL; ++c) acc[c] = 0.f;
  for (uint32_t off = voff0; off < (uint32_t)bytes + voff0; off += kItStride) {
    uint4 r[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) r[u] = buffer_load_x16(xc, bytes, off + u * kUStride);
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const T* e = reinterpret_cast<const T*>(&r[u]);
      float v[VPL];
#pragma unroll
      for (int c = 0; c < VPL; ++c) v[c] = (float)e[c];
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < VPL; ++c) ss += v[c] * v[c];
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
      for (int c = 0; c < VPL; ++c) acc[c] += v[c] * inv;
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
    float nv = 0.25f * (m2[0] * m2[0] + m2[1] * m2[1] + m2[2] * m2[2] + m2[3] * m2[3]);
    asm volatile("" : "+v"(nv));  // one rounded nv for every candidate (no per-candidate fusion)
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

// ---------------------------------------------------------------- pass 2, g = 4, fp16 input: matrix-core layout
// Persistent grid: one workgroup of 16 waves per compute unit (4 waves per SIMD),
// each taking a contiguous range of 16-token tiles (tiles of one (b, h) row are
// consecutive); a wave takes every 16th tile of its workgroup's range.
//
// Rotation on the matrix cores.  NSN commutes with the transform up to the shift:
// H_syl z = H_syl x / s1 - H_syl o, so the Sylvester matrix is applied to the raw
// fp16 tokens (exact operands: +-1 and fp16 values, every product exact, fp32
// sums) as 8 row tiles x 4 K-steps of v_mfma_f32_16x16x32_f16, and the shift
// enters afterwards as P = H_syl o (per wave, recomputed when its tiles move to
// another (b, h)).
// Operand layout: B of K-step ks, lane l = 16 gq + n: channels 32 ks + 8 gq .. + 7
// of token n (16 contiguous bytes of its row); result tile mt, lane l = 16 g + n:
// rotated channels 16 mt + 4 g + r, r = 0..3, of token n.  So every lane holds 8
// whole 4-dim sub-vectors (4 mt + g) of one token, and a per-token sum is 32
// in-lane terms plus two cross-lane adds (lanes n, n + 16, n + 32, n + 48).
// A fragments: H_syl[16 mt + i][32 ks + k] = s(mt, ks) F_{mt & 1}[i][k] with
// s(mt, ks) = (-1)^(mt2 ks1 + mt1 ks0) and, in lane l (i = l & 15, k = 8 (l >> 4) + j),
// F_0 = (-1)^(l3 l4 + l2 j2 + l1 j1 + l0 j0), F_1 = F_0 (-1)^(l5): four fragments
// (+-F_0, +-F_1) serve all 32 products.
//
// Candidate rows: the central cube of the grid, bins 6 .. 13 of every coordinate
// ([-1.6, 1.6)^4, about 63% of the sub-vectors of N(0,1) data), sits in LDS; the
// other rows are read from the table in global memory.  (The kernel is bound by
// its vector-memory accesses, and the row lookups are most of them.)
constexpr int kEnc4pWaves = 16;
constexpr int kEnc4pThreads = 64 * kEnc4pWaves;
constexpr int kHotLo = 6;         // first bin of the LDS cube on every coordinate
constexpr int kHotCells = 4096;   // 8^4 rows

// sum over the four lanes n, n + 16, n + 32, n + 48 that hold one token
__device__ __forceinline__ float token_sum4(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---------------------------------------------------------------- matrix-core tile front end
// Shared by the fp16 kernels of both sub-vector sizes (16-token tiles, lane
// l = 16 g + n, see above).

// The transform's sign fragments (+F_0, -F_0, +F_1, -F_1) and, for the randomized
// rotation, the sign bits of each lane's 32 input channels (channel 32 ks + 8 g + j
// -> bit 8 ks + j) as fp16 sign masks; written once per workgroup, by waves 1 and 2.
template <bool RHT>
__device__ __forceinline__ void tile_tables_init(int wave, int lane, uint4 smask, uint4 (*s_frag)[64],
                                                 uint4 (*s_rmask)[64]) {
  const int g = lane >> 4;
  if (wave == 1) {
#pragma unroll
    for (int f = 0; f < 4; ++f) s_frag[f][lane] = __builtin_bit_cast(uint4, hsyl_frag(lane, f >> 1, f & 1));
  }
  if constexpr (RHT) {
    if (wave == 2) {
      const uint32_t mw[4] = {smask.x, smask.y, smask.z, smask.w};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const uint32_t byte = (mw[ks] >> (8 * g)) & 0xffu;  // channels 32 ks + 8 g .. + 7
        uint32_t mk[4];
#pragma unroll
        for (int d = 0; d < 4; ++d)
          mk[d] = (((byte >> (2 * d)) & 1u) << 15) | (((byte >> (2 * d + 1)) & 1u) << 31);
        s_rmask[ks][lane] = make_uint4(mk[0], mk[1], mk[2], mk[3]);
      }
    }
  }
}

// P = H_syl o (randomized rotation: H_syl D o) of row bh into the wave's slot P[32],
// by the pair-layout butterfly; DQ: o_q from the head record, and the row's s1 grid.
template <bool DQ, bool RHT>
__device__ __forceinline__ void tile_row_shift(int bh, int lane, const float* __restrict__ o,
                                               const nsn_dq_head* __restrict__ heads, uint4 smask, float4* P,
                                               DqS1& dq) {
  const int p = lane & 31;
  float ov[4];
  if constexpr (DQ) {
    dq_o_load(heads + bh, p, ov);
    dq = dq_s1_load(heads + bh);
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) ov[c] = o[(size_t)bh * kD + 4 * p + c];
  }
  if constexpr (RHT) flip4(ov, lane_signs(smask, p));
  fwht128_pair(ov, p);
  if (lane < 32) P[p] = make_float4(ov[0], ov[1], ov[2], ov[3]);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// NSN of one tile with H_syl on the matrix cores.  xf: the lane's channels 32 ks +
// 8 g .. + 7 of token n (raw fp16; flipped here for the randomized rotation).  On
// return D[mt] holds Zr = H_syl z = a H_syl x - P (a = 1 / s1; DQ: 1 / s1_q) at
// channels 16 mt + 4 g + r of token n, q[mt] the sum of its four squares, and s1
// (DQ: also its code), s2, and rz = 1 / ||H_syl z|| (0 for a degenerate z).
template <bool DQ, bool RHT>
__device__ __forceinline__ void tile_nsn(uint4 xf[4], const uint4 (*s_frag)[64], const uint4 (*s_rmask)[64],
                                         const float4* P, int lane, const DqS1& dq, floatx4 D[8], float q[8],
                                         float& s1, uint32_t& s1code, bool& degen, float& rz, float& s2) {
  const int g = lane >> 4;
  if constexpr (RHT) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint4 mk = s_rmask[ks][lane];
      xf[ks].x ^= mk.x;
      xf[ks].y ^= mk.y;
      xf[ks].z ^= mk.z;
      xf[ks].w ^= mk.w;
    }
  }
  // ---------------- H_syl x on the matrix cores; ||x||^2 from the fp16 channels
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) D[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float ss = 0.f;
  const half8 F0p = __builtin_bit_cast(half8, s_frag[0][lane]), F0n = __builtin_bit_cast(half8, s_frag[1][lane]);
  const half8 F1p = __builtin_bit_cast(half8, s_frag[2][lane]), F1n = __builtin_bit_cast(half8, s_frag[3][lane]);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const half8 B = __builtin_bit_cast(half8, xf[ks]);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const bool ng = ((((mt >> 2) & 1) & ((ks >> 1) & 1)) ^ (((mt >> 1) & 1) & (ks & 1))) != 0;
      const half8 A = (mt & 1) ? (ng ? F1n : F1p) : (ng ? F0n : F0p);
      D[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B, D[mt], 0, 0, 0);
    }
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const uint32_t wv[4] = {xf[ks].x, xf[ks].y, xf[ks].z, xf[ks].w};
#pragma unroll
    for (int d = 0; d < 4; ++d)
      ss = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, wv[d]), __builtin_bit_cast(h2, wv[d]), ss, false);
  }
  ss = token_sum4(ss);
  const float r1 = ss > 0.f ? __builtin_amdgcn_rsqf(ss) : 0.f;  // 1 / ||x||
  s1 = ss * r1 * kInvSqrtD;
  float a = r1 * kSqrtD;  // 1 / s1 (0 for a zero token)
  s1code = 0;
  if constexpr (DQ) {
    s1code = ss > 0.f ? dq_s1_code(s1, dq) : 0u;
    a = s1code ? __builtin_amdgcn_rcpf(f16_val((uint16_t)dq_s1_pattern(s1code, dq))) : 0.f;
  }
  // ---------------- Zr = H_syl z = a H_syl x - P; per-sub-vector squares
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    const float4 Pm = P[4 * mt + g];
    D[mt][0] = fmaf(D[mt][0], a, -Pm.x);
    D[mt][1] = fmaf(D[mt][1], a, -Pm.y);
    D[mt][2] = fmaf(D[mt][2], a, -Pm.z);
    D[mt][3] = fmaf(D[mt][3], a, -Pm.w);
    float t = D[mt][0] * D[mt][0];
    t = fmaf(D[mt][1], D[mt][1], t);
    t = fmaf(D[mt][2], D[mt][2], t);
    t = fmaf(D[mt][3], D[mt][3], t);
    q[mt] = t;
  }
  float zz = ((q[0] + q[1]) + (q[2] + q[3])) + ((q[4] + q[5]) + (q[6] + q[7]));
  zz = token_sum4(zz);  // ||H_syl z||^2 = d ||z||^2
  degen = !(zz > kEpsZ * kEpsZ * (float)(kD * kD));  // ||z|| <= kEpsZ sqrt(d)
  rz = degen ? 0.f : __builtin_amdgcn_rsqf(zz);
  s2 = zz * rz * (1.f / (float)kD);  // ||z|| / sqrt(d) = sqrt(zz) / d
}

// T tiles of 16 tokens: tile i is tokens 16 (i % ntb) .. of row bh = i / ntb.
template <bool DQ, bool RHT>
__global__ __launch_bounds__(kEnc4pThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void k_encode4p(
    const _Float16* __restrict__ x, int L, int L_cap, int pos0, int ntb, int T, const float* __restrict__ o,
    const nsn_dq_head* __restrict__ heads, const uint4* __restrict__ cells, const uint4* __restrict__ rec,
    const uint16_t* __restrict__ encA, uint8_t* __restrict__ idx_out, uint16_t* __restrict__ scales_out,
    int sc_cap, int sc_pos0, uint4 smask) {
  // One LDS array, carved by hand so that the centroid records start at byte 0:
  // a record's address is then one v_perm (index byte * 256 + lane copy), with no
  // base to add in the candidate loop (ds_read offsets stop at 64 KB).
  constexpr int kRm = RHT ? 4 : 1;
  __shared__ uint4 s_lds[kK * 16 + (kHotCells + 1) + 4 * 64 + kRm * 64 + kEnc4pWaves * kD / 4 +
                         kEnc4pWaves * 16 * 4 / 2];
  uint4* const s_rec = s_lds;                                // 16 lane copies of every record
  uint4* const s_hot = s_rec + kK * 16;                      // the LDS cube + a zero row
  uint4 (*const s_frag)[64] = reinterpret_cast<uint4 (*)[64]>(s_hot + kHotCells + 1);  // +F_0, -F_0, +F_1, -F_1
  uint4 (*const s_rmask)[64] = s_frag + 4;  // randomized rotation: fp16 sign masks of each lane's channels
  float4 (*const s_P)[kD / 4] = reinterpret_cast<float4 (*)[kD / 4]>(s_rmask + kRm);  // each wave's H_syl o
  // index rows of each wave's tile (16 tokens x 32 bytes): each lane drops its 8
  // bytes (stride 4) here and stores 8 contiguous ones, so a tile's indices leave in
  // one store instruction instead of eight byte stores
  uint2 (*const s_irow)[16 * 4] = reinterpret_cast<uint2 (*)[16 * 4]>(s_P + kEnc4pWaves);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int tlo = (int)((long)T * blockIdx.x / gridDim.x), thi = (int)((long)T * (blockIdx.x + 1) / gridDim.x);
  const char* srec = reinterpret_cast<const char*>(s_rec);
  const uint32_t laneoff = (uint32_t)(lane & 15) << 4;
  const uint32_t xlane = (uint32_t)(n * kD * 2 + 16 * g);

  // a tile's rows: base, number of valid rows
  auto tile_rows = [&](int tile, int& bh, int& t0, int& nr) {
    bh = tile / ntb;
    t0 = (tile - bh * ntb) * 16;
    nr = min(16, L - t0);
  };
  auto load_x = [&](int tile, uint4 xf[4]) {
    int bh, t0, nr;
    tile_rows(tile < thi ? tile : thi - 1, bh, t0, nr);
    const _Float16* xb = x + ((size_t)bh * L + t0) * kD;
    const int bytes = tile < thi ? nr * kD * 2 : 0;  // past the range: zeros
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) xf[ks] = buffer_load_x16(xb, bytes, xlane + (uint32_t)(64 * ks));
  };

  // first tile's channels, issued before the prologue
  uint4 xf[4];
  load_x(tlo + wave, xf);

  for (int e = tid; e < kK * 16; e += kEnc4pThreads) s_rec[e] = rec[e >> 4];
  for (int r = tid; r < kHotCells; r += kEnc4pThreads) {
    const int u0 = r >> 9, u1 = (r >> 6) & 7, u2 = (r >> 3) & 7, u3 = r & 7;
    const int cell = (((u0 + kHotLo) * kGridN + u1 + kHotLo) * kGridN + u2 + kHotLo) * kGridN + u3 + kHotLo;
    s_hot[r] = cells[cell];
  }
  if (tid == 0) s_hot[kHotCells] = make_uint4(0u, 0u, 0u, 0u);
  // sign fragments of the transform, kept in LDS (reloaded per tile: registers are
  // the limit of this kernel, LDS reads are not)
  tile_tables_init<RHT>(wave, lane, smask, s_frag, s_rmask);
  __syncthreads();

  int cur_bh = -1;
  DqS1 dq;
  for (int tile = tlo + wave; tile < thi; tile += kEnc4pWaves) {
    // the loop-invariant LDS reads (sign fragments, P) stay inside the loop: held
    // across the search they would take registers this kernel cannot spare
    asm volatile("" ::: "memory");
    int bh, t0, nblk;
    tile_rows(tile, bh, t0, nblk);
    if (bh != cur_bh) {  // the row's shift P = H_syl o
      cur_bh = bh;
      tile_row_shift<DQ, RHT>(bh, lane, o, heads, smask, s_P[wave], dq);
    }
    uint8_t* iblk = idx_out + ((size_t)bh * L_cap + pos0 + t0) * (kD / 4);
    uint32_t* sblk = reinterpret_cast<uint32_t*>(scales_out) + ((size_t)bh * sc_cap + sc_pos0 + t0);
    const uint32_t tr = (uint32_t)n;  // token row inside the tile
    const bool valid = (int)tr < nblk;
    floatx4 D[8];
    float q[8], s1, rz, s2;
    uint32_t s1code;
    bool degen;
    tile_nsn<DQ, RHT>(xf, s_frag, s_rmask, s_P[wave], lane, dq, D, q, s1, s1code, degen, rz, s2);
    // the rotated token w = sqrt(d) rz Zr (||w||^2 = d); the search takes -2 w,
    // ||v||^2 per sub-vector and the grid cell of w
    const float sw = kSqrtD * rz;
    const float m2s = -2.f * sw, gs = kGridInv * sw, sw2 = sw * sw;

    // ---------------- cells of the sub-vectors and their candidate rows, fetched
    // two slots ahead: the LDS cube, else the global table (a sub-vector outside the
    // grid reads past the table: a zero row)
    // The cube test uses the integer bins themselves (a cube row is the global row
    // of the same cell).  The grid test uses the largest |coordinate| in grid units
    // with a margin: a sub-vector within 0.01 bin of the grid's edge takes the
    // exhaustive search (the same argmin), so the bins of an accepted one are always
    // inside the grid.
    const float in_lim = (float)(kGridN / 2) - 0.01f;  // |2.5 w| below: inside the grid
    // Every lane reads both tables, without branches: the LDS cube (a zero row when
    // the sub-vector is outside it) and the global table (an offset past its end,
    // which reads as zeros, when inside the cube or outside the grid); the two rows
    // are ORed where the row is used.  Rows written under divergent branches would
    // share registers, and every LDS read would then wait for all vector-memory
    // loads in flight, the lookahead and the next tile's channels included.
    auto lookup = [&](int mt, uint4& rl, uint4& rg) {
      const float amax = fmaxf(fmaxf(fabsf(D[mt][0]), fabsf(D[mt][1])), fmaxf(fabsf(D[mt][2]), fabsf(D[mt][3]))) * gs;
      int u[4];  // bin - kHotLo on each coordinate
#pragma unroll
      for (int r = 0; r < 4; ++r) u[r] = cvt_flr(fmaf(D[mt][r], gs, kGridOff - (float)kHotLo));
      // in the cube: every u in 0 .. 7 (a negative u sets high bits)
      const bool hot = ((u[0] | u[1] | u[2] | u[3]) & ~7) == 0;
      rl = s_hot[hot ? ((u[0] << 9) | (u[1] << 6) | (u[2] << 3) | u[3]) : kHotCells];
      // cell of bins u + kHotLo = ((u0 N + u1) N + u2) N + u3 + kHotLo (N^3 + N^2 + N + 1), in 24-bit products
      const int cell = __mul24(u[0], kGridN * kGridN * kGridN) + __mul24(u[1], kGridN * kGridN) +
                       __mul24(u[2], kGridN) + u[3] + kHotLo * (kGridN * kGridN * kGridN + kGridN * kGridN + kGridN + 1);
      rg = buffer_load_u4(cells, kGridCells * 16, (!hot && amax < in_lim) ? (uint32_t)cell << 4 : 0x80000000u);
    };
    uint4 lsl[2], lsg[2];
    lookup(0, lsl[0], lsg[0]);
    lookup(1, lsl[1], lsg[1]);

    float dot = 0.f;  // <m2, w_hat> summed over the lane's sub-vectors = -2 <w, w_hat> over them
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      float m2[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) m2[r] = D[mt][r] * m2s;
      float nv = q[mt] * sw2;  // ||v||^2
      // nv is one rounded value for every candidate: left visible, the compiler fuses
      // the product into the first candidates' sums only, and an exact tie between
      // two equal centroids could then go to the higher index
      asm volatile("" : "+v"(nv));
      const uint4 row = make_uint4(lsl[mt & 1].x | lsg[mt & 1].x, lsl[mt & 1].y | lsg[mt & 1].y,
                                   lsl[mt & 1].z | lsg[mt & 1].z, lsl[mt & 1].w | lsg[mt & 1].w);
      if (mt < 6) lookup(mt + 2, lsl[mt & 1], lsg[mt & 1]);
      if (mt == 6) load_x(tile + kEnc4pWaves, xf);  // the next tile's channels (slots 0-5 no longer hold registers)
      // deferred: outside the grid (zero row: count 0) or an overflowing cell
      const bool df = valid && ((row.w & 0xffu) == 0u || (row.w >> 24) != 0u);
      // ---------------- candidates: key = (bits of ||v||^2 + ||c||^2 - 2 <v, c>) with byte 0 = index
      const uint32_t lw[3] = {row.x, row.y, row.z};
      const uint32_t cnt = row.w & 0xffu;  // list length; the row is padded with its last entry
      int best = 0x7fffffff;
#pragma unroll
      for (int j = 0; j < kCellList; j += 2) {
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
          key[u] = (int)__builtin_amdgcn_perm(__float_as_uint(d), word, 0x07060500u | (uint32_t)(jj & 3));
        }
        best = min(min(best, key[0]), key[1]);
      }
      // ---------------- rare: exhaustive search for deferred sub-vectors of this slot
      const uint64_t dm = __ballot(df);
      if (dm != 0) {
        half8 Pf, Qf;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const _Float16 ah = (_Float16)m2[e];
          Pf[e] = ah;
          Pf[4 + e] = (_Float16)(m2[e] - (float)ah);
        }
        const _Float16 nh = (_Float16)nv;
        Qf[0] = (_Float16)1.f; Qf[1] = (_Float16)1.f; Qf[2] = nh; Qf[3] = (_Float16)(nv - (float)nh);
        Qf[4] = (_Float16)0.f; Qf[5] = (_Float16)0.f; Qf[6] = (_Float16)0.f; Qf[7] = (_Float16)0.f;
        const uint4 pw = __builtin_bit_cast(uint4, Pf), qw = __builtin_bit_cast(uint4, Qf);
        uint32_t b0[4], b1[4];
        const uint32_t pa[4] = {pw.x, pw.y, pw.z, pw.w}, qa[4] = {qw.x, qw.y, qw.z, qw.w};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const auto r = __builtin_amdgcn_permlane32_swap(pa[d], qa[d], false, false);
          b0[d] = r[0];  // columns = the sub-vectors of lanes 0-31: P in lanes 0-31, Q in 32-63
          b1[d] = r[1];  // columns = the sub-vectors of lanes 32-63
        }
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
          if (((dm >> (32 * tau)) & 0xffffffffull) == 0) continue;
          const uint32_t* bb = tau ? b1 : b0;
          const half8 Bx = __builtin_bit_cast(half8, make_uint4(bb[0], bb[1], bb[2], bb[3]));
          const int col = mfma_argmin_col4(Bx, encA, lane);
          if ((lane >> 5) == tau && df) best = col;
        }
      }
      // ---------------- this sub-vector's index; its share of <m2, w_hat>
      const uint4 rk = *reinterpret_cast<const uint4*>(srec + rec_addr((uint32_t)best, laneoff, 0));
      dot = fmaf(m2[0], f16_lo(rk.x), dot);
      dot = fmaf(m2[1], f16_hi(rk.x), dot);
      dot = fmaf(m2[2], f16_lo(rk.y), dot);
      dot = fmaf(m2[3], f16_hi(rk.y), dot);
      // index byte of sub-vector 4 mt + g of token n into the tile's LDS rows
      reinterpret_cast<uint8_t*>(s_irow[wave])[n * (kD / 4) + 4 * mt + g] = (uint8_t)((uint32_t)best & 0xffu);
    }
    // bytes 8 g .. 8 g + 7 of token n's row (written by the four lanes of the token:
    // the wave's LDS accesses complete in order, so a wave barrier suffices)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint2 row8 = s_irow[wave][n * 4 + g];
    // rows past the tile's valid rows lie outside the descriptors: those stores are dropped
    buffer_store_u64(row8, iblk, nblk * (kD / 4), tr * (kD / 4) + 8 * g);
    // ---------------- alpha = ||w||^2 / <w, w_hat> = d / <w, w_hat> = -2 d / <m2, w_hat>
    dot = token_sum4(dot);
    const float alpha = (!degen && dot < 0.f) ? (-2.f * kD) * __builtin_amdgcn_rcpf(dot) : 1.f;
    const uint32_t sw32 = (DQ ? s1code : (uint32_t)f16_bits(s1)) | ((uint32_t)f16_bits(s2 * alpha) << 16);
    buffer_store_u32(sw32, sblk, nblk * 4, g == 0 ? 4 * tr : 0x80000000u);  // one writer per token
  }
}

// ---------------------------------------------------------------- pass 2, g = 8, fp16 input: matrix-core layout
// The persistent 16-token tiles and the front end of k_encode4p (H_syl on the
// matrix cores, NSN in the MFMA layout), then an exhaustive search per sub-vector.
// Lane l = 16 g + n holds, for row tile mt, channels 16 mt + 4 g + r of token n:
// half of sub-vector s = 2 mt + (g >> 1).
//
// Distance GEMM (one v_mfma_f32_16x16x32_f16 per 16-centroid tile t and sub-vector
// s; columns = the tile's 16 tokens, rows = the centroids 16 t .. 16 t + 15), with
// K = 32 slots in four groups of eight (lane group q = l >> 4 of each operand):
//   q = 0: A = C_k (fp16),               B = fp16 hi part of -2 w_s
//   q = 1: A = C_k,                      B = fp16 lo part of -2 w_s (the residue)
//   q = 2: A = (||C_k||^2 hi, lo, 1, 1),  B = (1, 1, ||w_s||^2 hi, lo)
//   q = 3: zeros
// so D = ||C_k||^2 - 2 <w_s, C_k> + ||w_s||^2 = ||w_s - C_k||^2 with every product
// exact and fp32 sums, in one instruction.  Lane (n, g) of the result holds rows
// 4 g + r of column n; the keys (distance with its low 8 bits cleared | row tag)
// reduce with v_min3 (two candidates per instruction) and finally over the four
// lanes of the column.  The B operand is assembled through a per-wave LDS stage:
// each lane writes the hi and lo parts of its four channels (and one lane of the
// two that hold a sub-vector its ||w_s||^2 record), then reads its 16-byte slot.
constexpr int kEnc8pWaves = 12;
constexpr int kEnc8pThreads = 64 * kEnc8pWaves;
constexpr int kEnc8pTiles = kK / 16;  // 16-centroid tiles

template <bool DQ, bool RHT>
__global__ __launch_bounds__(kEnc8pThreads) __attribute__((amdgpu_waves_per_eu(3, 3))) void k_encode8p(
    const _Float16* __restrict__ x, int L, int L_cap, int pos0, int ntb, int T, const float* __restrict__ o,
    const nsn_dq_head* __restrict__ heads, const uint16_t* __restrict__ encA16, uint8_t* __restrict__ idx_out,
    uint16_t* __restrict__ scales_out, int sc_cap, int sc_pos0, uint4 smask) {
  constexpr int M = kD / 8;  // index bytes per token
  __shared__ uint4 s_frag[4][64];
  __shared__ uint4 s_rmask[RHT ? 4 : 1][64];
  __shared__ float4 s_P[kEnc8pWaves][kD / 4];
  // per wave: the 16 sub-vectors x 16 tokens x (hi, lo, norm record).  The 48-byte
  // token stride puts the 16 tokens of a write or read on distinct banks; lane group
  // q = 3 reads the hi part, which meets zeros in A.
  __shared__ uint4 s_stage[kEnc8pWaves][16][16][3];
  __shared__ float s_cn2[kK];  // ||C_k||^2 (fp32 of the fp16 hi + lo split in the A fragments)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int tlo = (int)((long)T * blockIdx.x / gridDim.x), thi = (int)((long)T * (blockIdx.x + 1) / gridDim.x);
  const uint32_t xlane = (uint32_t)(n * kD * 2 + 16 * g);

  auto tile_rows = [&](int tile, int& bh, int& t0, int& nr) {
    bh = tile / ntb;
    t0 = (tile - bh * ntb) * 16;
    nr = min(16, L - t0);
  };
  auto load_x = [&](int tile, uint4 xf[4]) {
    int bh, t0, nr;
    tile_rows(tile < thi ? tile : thi - 1, bh, t0, nr);
    const _Float16* xb = x + ((size_t)bh * L + t0) * kD;
    const int bytes = tile < thi ? nr * kD * 2 : 0;  // past the range: zeros
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) xf[ks] = buffer_load_x16(xb, bytes, xlane + (uint32_t)(64 * ks));
  };

  uint4 xf[4];
  load_x(tlo + wave, xf);
  // the distance GEMM's A operands stay in registers for the whole kernel
  half8 A[kEnc8pTiles];
#pragma unroll
  for (int t = 0; t < kEnc8pTiles; ++t) A[t] = *reinterpret_cast<const half8*>(encA16 + ((size_t)t * 64 + lane) * 8);

  for (int e = tid; e < kK; e += kEnc8pThreads) {
    const uint32_t hl = reinterpret_cast<const uint32_t*>(encA16)[((e >> 4) * 64 + 32 + (e & 15)) * 4];
    s_cn2[e] = f16_val((uint16_t)(hl & 0xffffu)) + f16_val((uint16_t)(hl >> 16));
  }
  {  // zeros in the norm records' upper halves (only their lower halves are rewritten)
    uint4* st = &s_stage[0][0][0][0];
    for (int e = tid; e < kEnc8pWaves * 16 * 16 * 3; e += kEnc8pThreads) st[e] = make_uint4(0u, 0u, 0u, 0u);
  }
  tile_tables_init<RHT>(wave, lane, smask, s_frag, s_rmask);
  __syncthreads();

  int cur_bh = -1;
  DqS1 dq;
  for (int tile = tlo + wave; tile < thi; tile += kEnc8pWaves) {
    asm volatile("" ::: "memory");
    int bh, t0, nblk;
    tile_rows(tile, bh, t0, nblk);
    if (bh != cur_bh) {  // the row's shift P = H_syl o
      cur_bh = bh;
      tile_row_shift<DQ, RHT>(bh, lane, o, heads, smask, s_P[wave], dq);
    }
    floatx4 D[8];
    float q[8], s1, rz, s2;
    uint32_t s1code;
    bool degen;
    tile_nsn<DQ, RHT>(xf, s_frag, s_rmask, s_P[wave], lane, dq, D, q, s1, s1code, degen, rz, s2);
    // -2 w = m2s Zr (||w||^2 = d), and ||w_s||^2 = sw2 (sum over the sub-vector's
    // eight Zr squares)
    const float sw = kSqrtD * rz;
    const float m2s = -2.f * sw, sw2 = sw * sw;

    // ---- stage the B operands of all 16 sub-vectors: this lane's four channels of
    // sub-vector 2 mt + (g >> 1) as fp16 hi and lo parts, and (from one of its two
    // lanes) the sub-vector's norm record (1, 1, ||w_s||^2 hi, lo)
    uint4 (*const stg)[16][3] = s_stage[wave];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const float v0 = D[mt][0] * m2s, v1 = D[mt][1] * m2s, v2 = D[mt][2] * m2s, v3 = D[mt][3] * m2s;
      const uint32_t h01 = hi_pair(v0, v1), h23 = hi_pair(v2, v3);
      const uint32_t l01 = lo_pair(h01, v0, v1), l23 = lo_pair(h23, v2, v3);
      const auto rq = __builtin_amdgcn_permlane16_swap(__float_as_uint(q[mt]), __float_as_uint(q[mt]), false, false);
      const float nv = (__uint_as_float(rq[0]) + __uint_as_float(rq[1])) * sw2;  // lanes g and g ^ 1
      const _Float16 nh = (_Float16)nv;
      const _Float16 nl = (_Float16)(nv - (float)nh);
      const uint32_t nvw =
          (uint32_t)__builtin_bit_cast(uint16_t, nh) | ((uint32_t)__builtin_bit_cast(uint16_t, nl) << 16);
      unsigned char* rowb = reinterpret_cast<unsigned char*>(&stg[2 * mt + (g >> 1)][n][0]);
      *reinterpret_cast<uint2*>(rowb + 8 * (g & 1)) = make_uint2(h01, h23);
      *reinterpret_cast<uint2*>(rowb + 16 + 8 * (g & 1)) = make_uint2(l01, l23);
      if ((g & 1) == 0) *reinterpret_cast<uint2*>(rowb + 32) = make_uint2(0x3C003C00u, nvw);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    load_x(tile + kEnc8pWaves, xf);  // the next tile's channels, in flight during the search

    // ---- the search, two sub-vectors at a time (independent chains: one's MFMA
    // runs while the other's keys reduce)
    uint64_t iw01 = 0, iw23 = 0;  // the token's 16 index bytes (every lane of the token)
    const int part = g < 3 ? g : 0;
    // <w, w_hat> from the search itself: per sub-vector 2 <w_s, C_k> = ||w_s||^2 +
    // ||C_k||^2 - ||w_s - C_k||^2, the last being the winning key's distance (its
    // low 8 bits cleared: a relative error below 2^-15), and the ||w_s||^2 sum to
    // ||w||^2 = d.  So sum (||w_s - C_k||^2 - ||C_k||^2) = d - 2 <w, w_hat>.
    float dsum = 0.f;
#pragma unroll 1
    for (int sp = 0; sp < 8; ++sp) {
      const half8 B0 = __builtin_bit_cast(half8, stg[2 * sp][n][part]);
      const half8 B1 = __builtin_bit_cast(half8, stg[2 * sp + 1][n][part]);
      // Row 4 g + r of tile t = 4 tg + j is centroid 64 tg + 16 j + 4 g + r.  The
      // keys carry the tag 16 j + r (an inline constant: one v_and_or_b32 each, where
      // a tag above 64 would take two instructions), each group of four tiles adds
      // its base 64 tg once, and g enters after the loop.
      int best0 = 0x7fffffff, best1 = 0x7fffffff;
#pragma unroll
      for (int tg = 0; tg < kEnc8pTiles / 4; ++tg) {
        int gb0 = 0x7fffffff, gb1 = 0x7fffffff;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const floatx4 z = {0.f, 0.f, 0.f, 0.f};
          const floatx4 d = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[4 * tg + j], B0, z, 0, 0, 0);
          const floatx4 e = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[4 * tg + j], B1, z, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; r += 2) {
            const float d0 = d[r], d1 = d[r + 1], e0 = e[r], e1 = e[r + 1];
            gb0 = min(min(gb0, (__float_as_int(d0) & ~0xff) | (16 * j + r)), (__float_as_int(d1) & ~0xff) | (16 * j + r + 1));
            gb1 = min(min(gb1, (__float_as_int(e0) & ~0xff) | (16 * j + r)), (__float_as_int(e1) & ~0xff) | (16 * j + r + 1));
          }
        }
        best0 = min(best0, gb0 + 64 * tg);
        best1 = min(best1, gb1 + 64 * tg);
      }
      best0 |= g << 2;
      best1 |= g << 2;
      {
        auto r0 = __builtin_amdgcn_permlane16_swap((uint32_t)best0, (uint32_t)best0, false, false);
        auto r1 = __builtin_amdgcn_permlane16_swap((uint32_t)best1, (uint32_t)best1, false, false);
        best0 = min((int)r0[0], (int)r0[1]);
        best1 = min((int)r1[0], (int)r1[1]);
        r0 = __builtin_amdgcn_permlane32_swap((uint32_t)best0, (uint32_t)best0, false, false);
        r1 = __builtin_amdgcn_permlane32_swap((uint32_t)best1, (uint32_t)best1, false, false);
        best0 = min((int)r0[0], (int)r0[1]);
        best1 = min((int)r1[0], (int)r1[1]);
      }
      // sub-vectors 2 sp and 2 sp + 1 are bytes 2 sp and 2 sp + 1 of the row
      const uint32_t k0 = (uint32_t)best0 & 0xffu, k1 = (uint32_t)best1 & 0xffu;
      const uint64_t sh = (uint64_t)(k0 | (k1 << 8)) << (16 * (sp & 3));
      iw01 |= sp < 4 ? sh : 0;
      iw23 |= sp < 4 ? 0 : sh;
      dsum += (__int_as_float(best0 & ~0xff) - s_cn2[k0]) + (__int_as_float(best1 & ~0xff) - s_cn2[k1]);
    }
    // index bytes 4 g .. 4 g + 3 of token n (selects: a lane-indexed array would live in scratch)
    const uint64_t half_w = g < 2 ? iw01 : iw23;
    const uint32_t mine = (g & 1) ? (uint32_t)(half_w >> 32) : (uint32_t)half_w;
    // ---------------- stores; alpha = d / <w, w_hat> = 2 d / (d - dsum)
    uint8_t* iblk = idx_out + ((size_t)bh * L_cap + pos0 + t0) * M;
    uint32_t* sblk = reinterpret_cast<uint32_t*>(scales_out) + ((size_t)bh * sc_cap + sc_pos0 + t0);
    // rows of tokens past the tile's valid rows lie outside the descriptors: those stores are dropped
    buffer_store_u32(mine, iblk, nblk * M, (uint32_t)(n * M + 4 * g));
    const float dot = (float)kD - dsum;  // 2 <w, w_hat>
    const float alpha = (!degen && dot > 0.f) ? (2.f * kD) * __builtin_amdgcn_rcpf(dot) : 1.f;
    const uint32_t sw32 = (DQ ? s1code : (uint32_t)f16_bits(s1)) | ((uint32_t)f16_bits(s2 * alpha) << 16);
    buffer_store_u32(sw32, sblk, nblk * 4, g == 0 ? 4u * (uint32_t)n : 0x80000000u);  // one writer per token
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
  // about 1024 blocks (four per compute unit) when the tensor is long, 256 ..
  // 16384 tokens per block
  long tc = ((long)BH * L + 1023) / 1024;
  tc = (tc + 255) / 256 * 256;
  if (tc < 256) tc = 256;
  if (tc > 16384) tc = 16384;
  return (int)tc;
}

// Per-token kernel of one call: plain (scales = (s1 | s2') at (L_cap, pos0)) or
// DQ (words = (code | s2') at rows [bh][L]).
template <bool DQ, bool RHT>
hipError_t launch_token_kernel_s(const nsn_codebook* cb, const void* x, int x_dtype, int BH, int L, int L_cap,
                                 int pos0, const float* o, const nsn_dq_head* heads, uint8_t* idx,
                                 uint16_t* scales, int sc_cap, int sc_pos0, hipStream_t st) {
  const uint4 sm = make_uint4(cb->sgn[0], cb->sgn[1], cb->sgn[2], cb->sgn[3]);
  if (cb->g == 4 && x_dtype == NSN_F16) {
    // persistent: one workgroup per compute unit, at least one tile per wave
    const int ntb = (L + 15) / 16;
    const int T = BH * ntb;  // fits: BH * L tokens of 256 bytes fit in device memory
    const int grid = std::max(1, std::min(cb->num_cu, (T + kEnc4pWaves - 1) / kEnc4pWaves));
    k_encode4p<DQ, RHT><<<grid, kEnc4pThreads, 0, st>>>(static_cast<const _Float16*>(x), L, L_cap, pos0, ntb, T, o,
                                                        heads, cb->d_cells, cb->d_rec, cb->d_encA, idx, scales, sc_cap,
                                                        sc_pos0, sm);
  } else if (cb->g == 4) {
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
  } else if (x_dtype == NSN_F16) {
    const int ntb = (L + 15) / 16;
    const int T = BH * ntb;
    const int grid = std::max(1, std::min(cb->num_cu, (T + kEnc8pWaves - 1) / kEnc8pWaves));
    k_encode8p<DQ, RHT><<<grid, kEnc8pThreads, 0, st>>>(static_cast<const _Float16*>(x), L, L_cap, pos0, ntb, T, o,
                                                        heads, cb->d_encA16, idx, scales, sc_cap, sc_pos0, sm);
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
