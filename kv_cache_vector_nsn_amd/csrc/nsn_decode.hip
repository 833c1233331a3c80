// Decode attention directly over the NSNQuant-quantized KV cache on gfx950.
//
// Follows "4. Implementation Details" of the Technical Summary of the explainer
// "NSNQuant: A Double Normalization Approach for Calibration-Free Low-Bit Vector
// Quantization of KV Cache" (gist.science/paper/2505.18231): attention scores
// use the NSN byproducts (s1, s2', o) directly, dequantization runs out of
// on-chip memory.  With x_hat = s1 (s2' H w_hat + o) and the orthonormal,
// symmetric Hadamard H:
//   q . k_hat_i = s1_i (s2'_i <H q, w_hat_i> + <q, o_K>)
//   sum_i p_i v_hat_i = H (sum_i p_i s1_i s2'_i w_hat_i) + (sum_i p_i s1_i) o_V
// so the kernel never leaves the rotated domain inside the token loop and
// applies H once per query head at the end.  With the randomized Hadamard option
// (x_hat = s1 (s2' D H w_hat + o), D the handle's channel signs) the query takes
// D before its transform and the output after the final one.
//
// Mapping (one workgroup = one (batch, KV head, token chunk); 8 waves, each
// taking 32-token steps):
//   * the codebook lives in LDS replicated so that each lane reads its own bank
//     group (32 copies of the 8-byte entry for g = 4, 16 copies of the 16-byte
//     entry for g = 8, one 256-byte row per entry); the gather address
//     entry * 256 + lane_offset is a single v_perm of the index byte;
//   * scores: 16x16x32 fp16 MFMA, A = dequantized K sub-vectors (rows = 16
//     tokens, K = 32 channels), B = H q split into fp16 hi/lo parts occupying
//     head slots 0..GQ-1 and GQ..2GQ-1 -- both parts are exact, so the score
//     carries fp32 accuracy; the two slots are summed after the MFMA;
//   * values: 16x16x32 fp16 MFMA, A = softmax weight times the token's value
//     scales, rounded to fp16 (rows = head slots, K = 32 tokens), B = centroid
//     channel t of 8 tokens x 16 sub-vectors (one MFMA per t, repacked from the
//     gathered entries with v_perm);
//   * split-KV: each workgroup writes (max, sum, beta, acc[128]) per query head;
//     k_combine merges the chunks in a fixed order and applies H;
//   * a residual window of fp16 tokens gets one more workgroup per (batch, KV
//     head), launched after the chunk workgroups (residual_block).
#include <algorithm>
#include <cmath>

#include "nsn_pair.h"

namespace nsn {
namespace {

constexpr int kPartStride = 132;  // m, l, beta, pad, acc[128]
constexpr int kWaves = 8;         // waves per workgroup: one ~140 KB workgroup per CU -> 2 waves per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kStepSpan = 32 * kWaves;  // tokens of one block step: one 32-token step per wave
constexpr int kStages = 4;              // LDS ring of block steps; loads run kStages - 1 steps ahead

// One staged block step.  Each wave stages only its own 32 tokens into its region
// of the slot, so the waves need no barrier per step and run out of step with each
// other.  A wave's region holds its K index rows (1 KB), its V index rows at +1 KB
// (g = 8: 512 B each, the other half of the 1 KB written by duplicate lanes), then:
//   plain caches: at +2 KB its K scale words (128 B, then 128 B of duplicates) and
//     V scale words at +2304;
//   double-quantized caches: at +2 KB one 256-byte block that four exec-masked loads
//     share: K s2' (lanes 0-15, 64 B), V s2' (lanes 16-31), K s1 codes (lanes 32-35,
//     16 B: a nibble per token) and V s1 codes (lanes 36-39).
constexpr int kWaveRegion = 2560;
constexpr int kWaveRegionDQ = 2304;
template <int G, bool DQ = false>
constexpr int stage_bytes() { return kWaves * (DQ ? kWaveRegionDQ : kWaveRegion); }
// global -> LDS loads one wave issues per staged step (K idx, V idx, then plain: K
// and V scales; DQ: the four masked scale parts)
template <int G, bool DQ = false>
constexpr int loads_per_stage() { return DQ ? 6 : 4; }

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// byte address inside LDS of a pointer to a __shared__ object (the low 32 bits of
// its generic address: the LDS aperture base has zero low bits)
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }

// LDS-DMA of 64 lanes x SIZE bytes: lane l loads `base + voff` (a buffer of
// `bytes` valid bytes -- reads past it return 0) into LDS at dst + SIZE * l.
// The buffer descriptor type exists only in the device compilation pass.
template <int SIZE>
__device__ __forceinline__ void dma_to_lds(const void* base, int bytes, uint32_t voff, unsigned char* dst) {
#if defined(__HIP_DEVICE_COMPILE__)
  const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
  static_assert(SIZE == 16 || SIZE == 4, "dwordx4 or dword");
  if constexpr (SIZE == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, voff, 0, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 4, voff, 0, 0, 0);
#endif
}

// s_waitcnt vmcnt(N), other counters untouched
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// two floats -> packed fp16 pair, round to nearest even (v_cvt_pk_f16_f32); the
// softmax weights lose no bias this way (truncation would shrink every weight)
__device__ __forceinline__ uint32_t pack_f16_rne(float a, float b) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  typedef float f2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){a, b}, h2));
}

template <int G>
__device__ __forceinline__ uint32_t gather_addr(uint32_t word, uint32_t laneoff, int byte) {
  // bytes: [laneoff, index, 0, 0] -> index * 256 + laneoff
  const uint32_t sel = 0x0C0C0000u | ((uint32_t)(4 + byte) << 8);
  return __builtin_amdgcn_perm(word, laneoff, sel);
}

// +inf in a scalar register the compiler cannot see through (see max2)
__device__ __forceinline__ float opaque_inf() {
  uint32_t v;
  asm("s_mov_b32 %0, 0x7f800000" : "=s"(v));
  return __uint_as_float(v);
}
// max(a, b) as one v_med3_f32 (the median of a, b and +inf).  fmaxf would first
// quiet each operand that comes from another lane (one v_max_f32 x, x, x per
// operand), and a literal +inf lets the compiler turn the median back into fmaxf.
// The scores and weights reduced here are finite or -inf.
__device__ __forceinline__ float max2(float a, float b) { return __builtin_amdgcn_fmed3f(a, b, opaque_inf()); }

// max / sum of the values held by lanes l, l ^ 16, l ^ 32, l ^ 48 (the four
// 16-lane rows): v_permlane16/32_swap exchange rows without going through LDS
__device__ __forceinline__ float rows_max(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = max2(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float rows_sum(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// lanes of the DPP banks in BANKS (4 lanes per bank, 4 banks per 16-lane row)
// take src from lane i - S of their row; the other lanes keep old
template <int S, int BANKS>
__device__ __forceinline__ float shr_into(float old, float src) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src), 0x110 + S, 0xf, BANKS, false));
}
// lanes of the DPP banks in BANKS take src from lane i + S of their row
template <int S, int BANKS>
__device__ __forceinline__ uint32_t shl_into(uint32_t old, uint32_t src) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)src, 0x100 + S, 0xf, BANKS, false);
}
// value of lane (i + S) mod 16 of the row (every lane is written: no old value)
template <int S>
__device__ __forceinline__ float row_ror(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x120 + S, 0xf, 0xf, false));
}

// Lazy rescaling of the online softmax: the reference maximum a wave's weights
// are taken against moves only when a step's score passes it by more than this
// (log2 units), so weights stay below 2^8 and most steps leave the sums alone.
constexpr float kLazyMax = 8.f;

// lane i of each 16-lane row reads lane i + k (DPP row_shl:k; 0 past the row end)
template <int K>
__device__ __forceinline__ float row_shl(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x100 + K, 0xf, 0xf, true));
}

// Head-transposed reduction of GQ per-lane partial scores over a 32-lane half.
// Level k halves the heads a lane carries across lane bit 4 - k: the lane with the
// bit clear keeps the lower half of its heads and receives its partner's, the other
// keeps the upper half.  After log2(GQ) levels lane p carries head p >> (5 - log2 GQ),
// summed over the lanes that differ from it in those top bits.
template <int GQ>
__device__ __forceinline__ float reduce_scatter_heads(float d[GQ], int p) {
  if constexpr (GQ == 1) {
    return d[0];
  } else {
    constexpr int n = GQ / 2;
    static_assert(GQ == 2 || GQ == 4 || GQ == 8, "heads per KV head");
    // first level: bit 4
    const bool up = (p & 16) != 0;
    float e[n];
#pragma unroll
    for (int j = 0; j < n; ++j) {
      const float keep = up ? d[j + n] : d[j];
      const float send = up ? d[j] : d[j + n];
      e[j] = keep + swz_xor<16>(send);
    }
    if constexpr (GQ == 2) {
      return e[0];
    } else {
      const bool up3 = (p & 8) != 0;
      constexpr int n2 = n / 2;
      float f[n2];
#pragma unroll
      for (int j = 0; j < n2; ++j) {
        const float keep = up3 ? e[j + n2] : e[j];
        const float send = up3 ? e[j] : e[j + n2];
        f[j] = keep + swz_xor<8>(send);
      }
      if constexpr (GQ == 4) {
        return f[0];
      } else {
        const bool up2 = (p & 4) != 0;
        const float keep = up2 ? f[1] : f[0];
        const float send = up2 ? f[0] : f[1];
        return keep + swz_xor<4>(send);
      }
    }
  }
}

// Sum over the lanes of the half that differ only in the low B bits (B = 2 .. 5).
template <int B>
__device__ __forceinline__ float sum_low_bits(float v, int p) {
  static_assert(B >= 2 && B <= 5, "low-bit group of 4 .. 32 lanes");
  (void)p;
  v += dpp_f<0xB1>(v);                       // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);                       // quad_perm [2,3,0,1]
  if constexpr (B >= 3) v += dpp_f<0x141>(v);  // row_half_mirror
  if constexpr (B >= 4) v += dpp_f<0x140>(v);  // row_mirror
  if constexpr (B >= 5) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  return v;
}

// out[r] = the value v of the lanes whose head is this lane's head ^ r (their
// lane differs in the top bits: lane p ^ (r << HSH)).
template <int GQ, int HSH>
__device__ __forceinline__ void gather_heads(float v, float out[GQ]) {
  out[0] = v;
  if constexpr (GQ >= 2) out[1] = swz_xor<(1 << HSH)>(v);
  if constexpr (GQ >= 4) {
    out[2] = swz_xor<(2 << HSH)>(v);
    out[3] = swz_xor<(3 << HSH)>(v);
  }
  if constexpr (GQ >= 8) {
    out[4] = swz_xor<(4 << HSH)>(v);
    out[5] = swz_xor<(5 << HSH)>(v);
    out[6] = swz_xor<(6 << HSH)>(v);
    out[7] = swz_xor<(7 << HSH)>(v);
  }
}

// Residual window of one (batch, KV head) inside k_decode: one extra workgroup
// (after all chunk workgroups in launch order) runs the R fp16 window tokens while
// the chunk workgroups run the quantized ones.  Pair layout (one token per half-wave, channels 4p..4p+3
// in lane p), 16 tokens per workgroup pass; the GQ scores are reduced
// head-transposed (each lane then runs the online softmax of its own head, in the
// log2 units of the chunk partials) and the value rows accumulate in the original
// domain.  The 16 half-wave states merge in a fixed order into one partial per
// query head, rpart[b Hq + h] = (m, l, 0, 0, acc[128]), which k_combine adds to the
// chunk partials.  scr: LDS scratch of 16 GQ kD floats, sst: 16 GQ 2 floats.
template <int GQ>
__device__ void residual_block(int hk, int b, const uint16_t* __restrict__ q, int Hq, int Hkv,
                               const uint16_t* __restrict__ k_res, const uint16_t* __restrict__ v_res, int R,
                               int R_cap, float* __restrict__ rpart, float* scr, float* sst) {
  constexpr int LOG = GQ == 1 ? 0 : GQ == 2 ? 1 : GQ == 4 ? 2 : 3;
  constexpr int HSH = 5 - LOG;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, p = lane & 31;
  const int hown = p >> HSH;
  const float cscale = 1.4426950408889634f * 0.08838834764831845f;  // log2(e) / sqrt(d)
  float qv[GQ][4];
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    float v[4];
    load4(reinterpret_cast<const _Float16*>(q + ((size_t)b * Hq + (size_t)hk * GQ + h) * kD), p, v);
#pragma unroll
    for (int c = 0; c < 4; ++c) qv[h][c] = v[c] * cscale;
  }
  const size_t rbase = ((size_t)b * Hkv + hk) * (size_t)R_cap * kD;
  float m_own = -INFINITY, l_own = 0.f, acc[GQ][4];
#pragma unroll
  for (int r = 0; r < GQ; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[r][c] = 0.f;
  for (int t0 = 2 * wave; t0 < R; t0 += 2 * kWaves) {
    const int t = t0 + half;
    const bool valid = t < R;
    const size_t row = rbase + (size_t)(valid ? t : R - 1) * kD;  // rows past R may hold anything
    float kx[4], vx[4];
    load4(reinterpret_cast<const _Float16*>(k_res + row), p, kx);
    load4(reinterpret_cast<const _Float16*>(v_res + row), p, vx);
    float dh[GQ];
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
      dh[h] = qv[h][0] * kx[0];
#pragma unroll
      for (int c = 1; c < 4; ++c) dh[h] = fmaf(qv[h][c], kx[c], dh[h]);
    }
    float d = reduce_scatter_heads<GQ>(dh, p);
    d = sum_low_bits<HSH>(d, p);
    if (!valid) d = -INFINITY;
    float corr = 1.f;
    if (d > m_own) {
      corr = (m_own == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_own - d);
      l_own *= corr;
      m_own = d;
    }
    if (__builtin_amdgcn_ballot_w64(corr != 1.f) != 0) {
      float cr[GQ];
      gather_heads<GQ, HSH>(corr, cr);
#pragma unroll
      for (int r = 0; r < GQ; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] *= cr[r];
    }
    const float pr = valid ? __builtin_amdgcn_exp2f(d - m_own) : 0.f;
    l_own += pr;
    float wr[GQ];
    gather_heads<GQ, HSH>(pr, wr);
#pragma unroll
    for (int c = 0; c < 4; ++c) vx[c] = valid ? vx[c] : 0.f;
#pragma unroll
    for (int r = 0; r < GQ; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[r][c] = fmaf(wr[r], vx[c], acc[r][c]);
  }
  const int slot = 2 * wave + half;
#pragma unroll
  for (int r = 0; r < GQ; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) scr[(slot * GQ + (hown ^ r)) * kD + 4 * p + c] = acc[r][c];
  if ((p & ((1 << HSH) - 1)) == 0) {
    sst[(slot * GQ + hown) * 2 + 0] = m_own;
    sst[(slot * GQ + hown) * 2 + 1] = l_own;
  }
  __syncthreads();
  for (int i = tid; i < GQ * kD; i += kThreads) {
    const int h = i / kD, c = i % kD;
    float Mx = -INFINITY;
    for (int w = 0; w < 2 * kWaves; ++w) Mx = fmaxf(Mx, sst[(w * GQ + h) * 2]);
    float a = 0.f, l = 0.f;
    for (int w = 0; w < 2 * kWaves; ++w) {
      const float mw = sst[(w * GQ + h) * 2];
      const float f = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - Mx);
      a += f * scr[(w * GQ + h) * kD + c];
      l += f * sst[(w * GQ + h) * 2 + 1];
    }
    float* dst = rpart + ((size_t)b * Hq + (size_t)hk * GQ + h) * kPartStride;
    dst[4 + c] = a;
    if (c == 0) {
      dst[0] = Mx;
      dst[1] = l;
      dst[2] = 0.f;
      dst[3] = 0.f;
    }
  }
}

// The decode step's new token ("4. Implementation Details", "Residuals": a new
// token is quantized with the stored shift and appended): the workgroup of each
// (batch, KV head)'s last chunk encodes the fp16 K and V rows of that token, writes
// their records at slot pos of the caches and joins the token to its softmax
// without reading it back.  pos < 0: no token.
struct AppendArgs {
  const _Float16* k_new = nullptr;  // [B * Hkv][128]
  const _Float16* v_new = nullptr;
  const uint16_t* encA = nullptr;   // the codebook's distance-GEMM A fragments
  const float* c32 = nullptr;       // the codebook, fp32 [256][G]
  const float* k_o = nullptr;       // the stored channel means [B * Hkv][128]
  const float* v_o = nullptr;
  uint8_t* k_idx = nullptr;         // the caches (written at slot pos only)
  uint16_t* k_sc = nullptr;
  uint8_t* v_idx = nullptr;
  uint16_t* v_sc = nullptr;
  int pos = 0;                      // the new token's slot (the number of cached tokens)
};

// A cache whose flushed residual blocks each keep their own channel mean ("4.
// Implementation Details", "Residuals": a full window is quantized on its own, NSN
// of "1. Normalize-Shift-Normalize" taking the mean of the tensor it quantizes):
// tokens [0, S0) share the stored o, block j holds tokens [S0 + j Rb, S0 + (j+1) Rb)
// with o_K = k_ob[j][b][h].  Each block is one chunk (its own <q, o_K> and its own
// beta in the partial); the prefix is chunked as usual into the first nchunk0
// chunks.  Rb = 0: no blocks (one o per (batch, KV head)).
struct SegArgs {
  const float* k_ob = nullptr;  // [nblk][B * Hkv][128]
  int S0 = 0;
  int Rb = 0;
  int nchunk0 = 0;
};

// DQ: k_sc / v_sc are the s2' arrays (fp16 per token), k_nib / v_nib the 4-bit s1
// codes and k_hd / v_hd the tensors' head records; each wave expands its 32
// tokens' scales into the (s1 | s2') words of the plain layout in a private LDS
// area before reading them.
template <int G, int GQ, bool DQ, bool APP = false>
__global__ __launch_bounds__(kThreads, 1) void k_decode(const uint16_t* __restrict__ q, int Hq, int Hkv, int S,
                                                   int S_cap, int CH, int nchunk,
                                                   const uint8_t* __restrict__ k_idx,
                                                   const uint16_t* __restrict__ k_sc,
                                                   const float* __restrict__ k_o,
                                                   const uint8_t* __restrict__ v_idx,
                                                   const uint16_t* __restrict__ v_sc,
                                                   const uint8_t* __restrict__ k_nib,
                                                   const uint8_t* __restrict__ v_nib,
                                                   const nsn_dq_head* __restrict__ k_hd,
                                                   const nsn_dq_head* __restrict__ v_hd,
                                                   const uint16_t* __restrict__ c16x2,
                                                   float* __restrict__ part,
                                                   const uint16_t* __restrict__ k_res,
                                                   const uint16_t* __restrict__ v_res, int R, int R_cap,
                                                   float* __restrict__ rpart, int BH, uint4 smask,
                                                   AppendArgs ap, SegArgs sg) {
  constexpr int M = kD / G;            // indices per token
  constexpr int NB = (G == 4) ? 2 : 1; // 16-column value blocks
  constexpr int NT = G;                // channel offsets per sub-vector
  constexpr int SB = stage_bytes<G, DQ>();
  constexpr int LPS = loads_per_stage<G, DQ>();
  __shared__ __attribute__((aligned(256))) unsigned char s_tab[kK * 256];  // replicated codebook
  // the ring slots are separate LDS objects so that the compiler can tell a refill
  // in flight from the slot being read (no forced wait on every outstanding load)
  static_assert(kStages == 4, "four ring slots");
  __shared__ __attribute__((aligned(16))) unsigned char s_st0[SB];
  __shared__ __attribute__((aligned(16))) unsigned char s_st1[SB];
  __shared__ __attribute__((aligned(16))) unsigned char s_st2[SB];
  __shared__ __attribute__((aligned(16))) unsigned char s_st3[SB];
  __shared__ float s_q[8][kD];
  __shared__ float s_qo[8];
  __shared__ __attribute__((aligned(16))) uint32_t s_scw[DQ ? kWaves : 1][64];  // DQ: per wave K words, V words
  // 1-D grid: nchunk BH chunk workgroups (chunk fastest), then BH residual-window ones
  const int lin = (int)blockIdx.x;
  if constexpr (!DQ) {
    if (lin >= nchunk * BH) {  // the residual window's workgroup (the codebook LDS is its scratch)
      const int rbh = lin - nchunk * BH;
      residual_block<GQ>(rbh % Hkv, rbh / Hkv, q, Hq, Hkv, k_res, v_res, R, R_cap, rpart,
                         reinterpret_cast<float*>(s_tab), &s_q[0][0]);
      return;
    }
  }

  const int chunk = lin % nchunk, hk = (lin / nchunk) % Hkv, b = lin / nchunk / Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bh = b * Hkv + hk;
  // the chunk's tokens and channel mean: a prefix chunk, or one flushed block
  const bool blk = sg.Rb > 0 && chunk >= sg.nchunk0;
  const int c0 = blk ? sg.S0 + (chunk - sg.nchunk0) * sg.Rb : chunk * CH;
  const int c1 = blk ? c0 + sg.Rb : min(sg.Rb > 0 ? sg.S0 : S, c0 + CH);
  const float* const ko_src = blk ? sg.k_ob + (size_t)(chunk - sg.nchunk0) * BH * kD : k_o;
  const size_t row0 = (size_t)bh * S_cap;
  const int nsteps = (c1 - c0 + kStepSpan - 1) / kStepSpan;

  // ---- staged loads: block step s (tokens c0 + 256 s ..) goes to ring slot s % kStages
  // straight from global memory into LDS (buffer_load ... lds); each wave loads its own
  // 32 tokens into its region of the slot (see kWaveRegion / kWaveRegionDQ).
  // Each load takes a buffer descriptor based at the step's first row whose record
  // count ends at the (b, h) slab's capacity S_cap: rows past the slab read as 0 and
  // rows in [c1, S_cap) are masked, so no per-lane clamping is needed.  The per-lane
  // offsets are loop invariant: the compiler treats a DMA load's address registers
  // as busy until the load lands, and registers that are never rewritten never make
  // it wait.
  constexpr int MM = kD / G;
  const uint32_t voff_idx = (uint32_t)(32 * wave * MM + (G == 4 ? 16 * lane : 16 * (lane & 31)));
  // plain: scale words; DQ: s2' pairs (lanes 0-31) and code bytes (lanes 32-39)
  const uint32_t voff_sc = !DQ ? (uint32_t)(4 * (32 * wave + (lane & 31)))
                                : (uint32_t)(lane < 32 ? 64 * wave + 4 * (lane & 15) : 16 * wave + 4 * (lane & 3));
  const uint8_t* kslab = k_idx + row0 * MM;
  const uint8_t* vslab = v_idx + row0 * MM;
  const unsigned char* ksslab = reinterpret_cast<const unsigned char*>(k_sc + row0 * (DQ ? 1 : 2));
  const unsigned char* vsslab = reinterpret_cast<const unsigned char*>(v_sc + row0 * (DQ ? 1 : 2));
  const int capb = (S_cap + 1) >> 1;  // DQ: code bytes per (b, h)
  const unsigned char* knslab = DQ ? k_nib + (size_t)bh * capb : nullptr;
  const unsigned char* vnslab = DQ ? v_nib + (size_t)bh * capb : nullptr;
  auto issue_into = [&](unsigned char* dst, int st) {
    const int sb = c0 + st * kStepSpan;
    const int rows_left = max(0, S_cap - sb);
    if constexpr (!DQ) {  // this wave's 32 tokens only (lanes 32-63 repeat rows / words into pads)
      unsigned char* rg = dst + wave * kWaveRegion;
      dma_to_lds<16>(kslab + (size_t)sb * MM, rows_left * MM, voff_idx, rg);
      dma_to_lds<16>(vslab + (size_t)sb * MM, rows_left * MM, voff_idx, rg + 1024);
      dma_to_lds<4>(ksslab + (size_t)sb * 4, rows_left * 4, voff_sc, rg + 2048);
      dma_to_lds<4>(vsslab + (size_t)sb * 4, rows_left * 4, voff_sc, rg + 2304);
      return;
    }
    // DQ: this wave's index rows, then its four scale parts into one 256-byte block;
    // each part is one load whose lanes outside it are masked off (every part has
    // active lanes, so each wave issues exactly loads_per_stage loads per step)
    unsigned char* rg = dst + wave * kWaveRegionDQ;
    dma_to_lds<16>(kslab + (size_t)sb * MM, rows_left * MM, voff_idx, rg);
    dma_to_lds<16>(vslab + (size_t)sb * MM, rows_left * MM, voff_idx, rg + 1024);
    const int nb_left = max(0, capb - sb / 2);
    if (lane < 16) dma_to_lds<4>(ksslab + (size_t)sb * 2, rows_left * 2, voff_sc, rg + 2048);
    if (lane >= 16 && lane < 32) dma_to_lds<4>(vsslab + (size_t)sb * 2, rows_left * 2, voff_sc, rg + 2048);
    if (lane >= 32 && lane < 36) dma_to_lds<4>(knslab + sb / 2, nb_left, voff_sc, rg + 2048);
    if (lane >= 36 && lane < 40) dma_to_lds<4>(vnslab + sb / 2, nb_left, voff_sc, rg + 2048);
  };

  // ---- codebook -> LDS by LDS-DMA: entry k replicated over its 256-byte row (16
  // copies of the 16-byte row of c16x2).  Loading the table the same way as the
  // stages matters for the compiler's wait tracking: an LDS read of an object that
  // no LDS-DMA ever wrote is made to wait for every LDS-DMA load in flight, while a
  // read of a DMA-written object waits only for the loads into that object.
#pragma unroll
  for (int i = 0; i < kK * 256 / 1024 / kWaves; ++i) {
    const int blk = wave * (kK * 256 / 1024 / kWaves) + i;  // 1 KB = rows 4 blk .. 4 blk + 3
    __builtin_amdgcn_global_load_lds(c16x2 + (size_t)(4 * blk + (lane >> 4)) * 8, s_tab + 1024 * blk, 16, 0, 0);
  }
  // ---- q~ = c H q / sqrt(d) with c = log2(e) / sqrt(d) (scores come out in log2
  // units), and c <q, o_K>, for the GQ query heads (pair layout)
  const float cscale = 1.4426950408889634f * 0.08838834764831845f;
  {
    const int p = lane & 31, hf = lane >> 5;
    const int h = wave * 2 + hf;
    if (h < GQ) {
      const uint16_t* qr = q + ((size_t)b * Hq + (size_t)hk * GQ + h) * kD;
      float v[4];
      load4(reinterpret_cast<const _Float16*>(qr), p, v);
      float qo = 0.f;
      float ko[4];
      if constexpr (DQ) {
        const uint32_t b = *reinterpret_cast<const uint16_t*>(k_hd[bh].o_codes + 2 * p);
#pragma unroll
        for (int c = 0; c < 4; ++c) ko[c] = (float)((int)((b >> (4 * c)) & 15u) - 8) * k_hd[bh].o_scale;
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) ko[c] = ko_src[(size_t)bh * kD + 4 * p + c];
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) qo += v[c] * ko[c];
      qo = half_wave_sum(qo);
      flip4(v, lane_signs(smask, p));  // randomized rotation: <q, D H w> = <H D q, w>
      fwht128_pair_valu(v, p);
      const float rs = 0.08838834764831845f * cscale;
#pragma unroll
      for (int c = 0; c < 4; ++c) s_q[h][4 * p + c] = v[c] * rs;
      if (p == 0) s_qo[h] = qo * cscale;
    }
  }
  __syncthreads();  // q in LDS (and the table loads drained) for every wave

  const int n = lane & 15;   // head slot (score B / value A) or token (score A) or column (value B)
  const int grp = lane >> 4; // K-slot group of the operands, row group of the results
  // score B fragments: slot n < GQ -> hi part of head n, GQ <= n < 2GQ -> lo part
  half8 QB[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = 32 * grp + 8 * s + e;
      _Float16 val = (_Float16)0.f;
      if (n < 2 * GQ) {
        const float qv = s_q[n % GQ][c];
        const _Float16 hi = (_Float16)qv;
        val = (n < GQ) ? hi : (_Float16)(qv - (float)hi);
      }
      QB[s][e] = val;
    }
  }
  const float qo = s_qo[n % GQ];
  uint32_t dq_kbase = 0, dq_kstride = 1, dq_vbase = 0, dq_vstride = 1;
  if constexpr (DQ) {
    dq_kbase = k_hd[bh].s1_base;
    dq_kstride = k_hd[bh].s1_stride;
    dq_vbase = v_hd[bh].s1_base;
    dq_vstride = v_hd[bh].s1_stride;
  }
  // lanes whose softmax values are real; the rest feed zero rows of the value MFMA
  const uint32_t live_mask = n < GQ ? 0xffffffffu : 0u;

  const uint32_t laneoff = (G == 4) ? 8u * (lane & 31) : 16u * (lane & 15);
  const unsigned char* tab = s_tab;

  // Exactly kStages - 1 steps are always in flight: refills past the chunk end load
  // row c1 - 1 on every lane (one cache line per instruction), so each step can wait
  // with the same unconditional vmcnt and the compiler sees that wait on every path.
  issue_into(s_st0, 0);
  issue_into(s_st1, 1);
  issue_into(s_st2, 2);


  floatx4 acc[NB][NT];
#pragma unroll
  for (int bl = 0; bl < NB; ++bl)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[bl][t] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f, beta_run = 0.f;
  // The value weights p s1 s2' enter the value MFMA as fp16, where a finite token
  // with s1 s2' near or above the fp16 range would overflow.  The wave keeps its
  // value sums in units of 2^vexp: every step's weights are scaled by 2^-vexp (one
  // v_ldexp each), and vexp grows -- with the sums rescaled by the same exact power
  // of two, inside the rescaling block the online softmax already has -- only when
  // a step's largest live weight would exceed 2^14 in those units.
  int vexp = 0;

  // Words of one 32-token step, read from the LDS stage right before use.
  // With GQ >= 4 the softmax runs on a redistributed layout: lane n = h + GQ k of
  // a row holds RV = GQ/2 consecutive tokens of head h (see compute_step), so it
  // reads only those tokens' scales.
  constexpr bool RED = GQ >= 4;
  constexpr int RV = RED ? GQ / 2 : 8;
  const int kk = n / GQ;                                   // k of this lane (RED layout)
  const int rtok0 = RED ? (16 * ((kk * RV) / 4) + 4 * grp + (kk * RV) % 4) : 0;  // first token of the lane
  struct StepIn {
    uint32_t kx[2][G == 4 ? 2 : 1];
    uint32_t kw[RV], vw[RV], vx[8];
  };
  // This wave's 32 tokens inside a staged block step, read in ONE inline-asm block
  // that ends with its own lgkmcnt(0) wait (so every output is complete when the
  // block ends).  The reads are hidden from the compiler on purpose: its wait
  // tracking cannot tell which LDS-DMA (buffer_load ... lds) a plain LDS read
  // depends on and would otherwise drain every staged load in flight first.  The
  // explicit vmcnt wait and barrier before each step order these reads after the
  // step's loads.  Offsets (immediates): K rows 16 a + n (a = 0, 1) -> + 16 M a;
  // V rows 16 (e / 4) + 4 grp + e % 4 -> + (16 (e / 4) + e % 4) M.
  auto read_in = [&](StepIn& in, const unsigned char* stg) {
    // K rows of the wave's tokens, V rows (plain: in the wave's region)
    const unsigned char* kr0 = stg + wave * (DQ ? kWaveRegionDQ : kWaveRegion);
    const unsigned char* vr0 = kr0 + 1024;
    const uint32_t ka = lds_addr(kr0 + n * M + (G == 4 ? 8 : 4) * grp);
    const uint32_t va = lds_addr(vr0 + 4 * grp * M + (G == 4 ? 2 * n : n));
    if constexpr (DQ) {
      // lane = 32 which + j expands token 32 wave + j of K (which 0) or V (which 1):
      // (s1 pattern of its code | s2' << 16) into this wave's word area
      const int j = lane & 31, which = lane >> 5, tok = 32 * wave + j;
      const unsigned char* sc = kr0 + 2048;  // K s2' | V s2' | K codes | V codes
      const uint32_t a_s2 = lds_addr(sc + 64 * which + 2 * j);
      const uint32_t a_nb = lds_addr(sc + 128 + 16 * which + (j >> 1));
      uint32_t s2b, nb;
      asm volatile("ds_read_u16 %0, %2\n\tds_read_u8 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                   : "=&v"(s2b), "=&v"(nb)
                   : "v"(a_s2), "v"(a_nb)
                   : "memory");
      const uint32_t code = (nb >> (4 * (tok & 1))) & 15u;
      const uint32_t base = which ? dq_vbase : dq_kbase, stride = which ? dq_vstride : dq_kstride;
      const uint32_t pat = code ? min(base + (code - 1u) * stride, 0x7BFFu) : 0u;
      asm volatile("ds_write_b32 %0, %1" ::"v"(lds_addr(&s_scw[DQ ? wave : 0][lane])), "v"(pat | (s2b << 16))
                   : "memory");
    }
    // K words of the wave's tokens, then V words (plain: in the stage; DQ: the expanded area)
    const unsigned char* ksb = DQ ? reinterpret_cast<const unsigned char*>(s_scw[DQ ? wave : 0])
                                  : stg + wave * kWaveRegion + 2048;
    const uint32_t ksa = lds_addr(ksb + 4 * (RED ? rtok0 : 4 * grp));
    const uint32_t vsa = ksa + (DQ ? 128 : 256);
    uint32_t x0, x1, x2, x3, x4, x5, x6, x7;
    if constexpr (G == 4 && RED && RV == 2) {
      u32x2 k0, k1, s0, s1;
      asm volatile(
          "ds_read_b64 %0, %12\n\tds_read_b64 %1, %12 offset:512\n\t"
          "ds_read_b64 %2, %13\n\tds_read_b64 %3, %14\n\t"
          "ds_read_u16 %4, %15\n\tds_read_u16 %5, %15 offset:32\n\t"
          "ds_read_u16 %6, %15 offset:64\n\tds_read_u16 %7, %15 offset:96\n\t"
          "ds_read_u16 %8, %15 offset:512\n\tds_read_u16 %9, %15 offset:544\n\t"
          "ds_read_u16 %10, %15 offset:576\n\tds_read_u16 %11, %15 offset:608\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(k0), "=&v"(k1), "=&v"(s0), "=&v"(s1), "=&v"(x0), "=&v"(x1), "=&v"(x2), "=&v"(x3), "=&v"(x4),
            "=&v"(x5), "=&v"(x6), "=&v"(x7)
          : "v"(ka), "v"(ksa), "v"(vsa), "v"(va)
          : "memory");
      in.kx[0][0] = k0[0]; in.kx[0][1 % (G == 4 ? 2 : 1)] = k0[1];
      in.kx[1][0] = k1[0]; in.kx[1][1 % (G == 4 ? 2 : 1)] = k1[1];
      in.kw[0] = s0[0]; in.kw[1 % RV] = s0[1];
      in.vw[0] = s1[0]; in.vw[1 % RV] = s1[1];
    } else if constexpr (G == 4 && RED) {  // RV == 4
      u32x2 k0, k1;
      u32x4 s0, s1;
      asm volatile(
          "ds_read_b64 %0, %12\n\tds_read_b64 %1, %12 offset:512\n\t"
          "ds_read_b128 %2, %13\n\tds_read_b128 %3, %14\n\t"
          "ds_read_u16 %4, %15\n\tds_read_u16 %5, %15 offset:32\n\t"
          "ds_read_u16 %6, %15 offset:64\n\tds_read_u16 %7, %15 offset:96\n\t"
          "ds_read_u16 %8, %15 offset:512\n\tds_read_u16 %9, %15 offset:544\n\t"
          "ds_read_u16 %10, %15 offset:576\n\tds_read_u16 %11, %15 offset:608\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(k0), "=&v"(k1), "=&v"(s0), "=&v"(s1), "=&v"(x0), "=&v"(x1), "=&v"(x2), "=&v"(x3), "=&v"(x4),
            "=&v"(x5), "=&v"(x6), "=&v"(x7)
          : "v"(ka), "v"(ksa), "v"(vsa), "v"(va)
          : "memory");
      in.kx[0][0] = k0[0]; in.kx[0][1 % (G == 4 ? 2 : 1)] = k0[1];
      in.kx[1][0] = k1[0]; in.kx[1][1 % (G == 4 ? 2 : 1)] = k1[1];
#pragma unroll
      for (int q = 0; q < RV; ++q) { in.kw[q] = s0[q & 3]; in.vw[q] = s1[q & 3]; }
    } else if constexpr (G == 4) {  // 8 scale words per lane: tokens 4 grp .. + 3 and 16 + 4 grp .. + 3
      u32x2 k0, k1;
      u32x4 s0, s1, s2, s3;
      asm volatile(
          "ds_read_b64 %0, %14\n\tds_read_b64 %1, %14 offset:512\n\t"
          "ds_read_b128 %2, %15\n\tds_read_b128 %3, %15 offset:64\n\t"
          "ds_read_b128 %4, %16\n\tds_read_b128 %5, %16 offset:64\n\t"
          "ds_read_u16 %6, %17\n\tds_read_u16 %7, %17 offset:32\n\t"
          "ds_read_u16 %8, %17 offset:64\n\tds_read_u16 %9, %17 offset:96\n\t"
          "ds_read_u16 %10, %17 offset:512\n\tds_read_u16 %11, %17 offset:544\n\t"
          "ds_read_u16 %12, %17 offset:576\n\tds_read_u16 %13, %17 offset:608\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(k0), "=&v"(k1), "=&v"(s0), "=&v"(s1), "=&v"(s2), "=&v"(s3), "=&v"(x0), "=&v"(x1), "=&v"(x2),
            "=&v"(x3), "=&v"(x4), "=&v"(x5), "=&v"(x6), "=&v"(x7)
          : "v"(ka), "v"(ksa), "v"(vsa), "v"(va)
          : "memory");
      in.kx[0][0] = k0[0]; in.kx[0][1 % (G == 4 ? 2 : 1)] = k0[1];
      in.kx[1][0] = k1[0]; in.kx[1][1 % (G == 4 ? 2 : 1)] = k1[1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        in.kw[i % RV] = s0[i]; in.kw[(4 + i) % RV] = s1[i];
        in.vw[i % RV] = s2[i]; in.vw[(4 + i) % RV] = s3[i];
      }
    } else if constexpr (RED && RV == 2) {  // G == 8
      uint32_t k0, k1;
      u32x2 s0, s1;
      asm volatile(
          "ds_read_b32 %0, %12\n\tds_read_b32 %1, %12 offset:256\n\t"
          "ds_read_b64 %2, %13\n\tds_read_b64 %3, %14\n\t"
          "ds_read_u8 %4, %15\n\tds_read_u8 %5, %15 offset:16\n\t"
          "ds_read_u8 %6, %15 offset:32\n\tds_read_u8 %7, %15 offset:48\n\t"
          "ds_read_u8 %8, %15 offset:256\n\tds_read_u8 %9, %15 offset:272\n\t"
          "ds_read_u8 %10, %15 offset:288\n\tds_read_u8 %11, %15 offset:304\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(k0), "=&v"(k1), "=&v"(s0), "=&v"(s1), "=&v"(x0), "=&v"(x1), "=&v"(x2), "=&v"(x3), "=&v"(x4),
            "=&v"(x5), "=&v"(x6), "=&v"(x7)
          : "v"(ka), "v"(ksa), "v"(vsa), "v"(va)
          : "memory");
      in.kx[0][0] = k0;
      in.kx[1][0] = k1;
      in.kw[0] = s0[0]; in.kw[1 % RV] = s0[1];
      in.vw[0] = s1[0]; in.vw[1 % RV] = s1[1];
    } else if constexpr (RED) {  // G == 8, RV == 4
      uint32_t k0, k1;
      u32x4 s0, s1;
      asm volatile(
          "ds_read_b32 %0, %12\n\tds_read_b32 %1, %12 offset:256\n\t"
          "ds_read_b128 %2, %13\n\tds_read_b128 %3, %14\n\t"
          "ds_read_u8 %4, %15\n\tds_read_u8 %5, %15 offset:16\n\t"
          "ds_read_u8 %6, %15 offset:32\n\tds_read_u8 %7, %15 offset:48\n\t"
          "ds_read_u8 %8, %15 offset:256\n\tds_read_u8 %9, %15 offset:272\n\t"
          "ds_read_u8 %10, %15 offset:288\n\tds_read_u8 %11, %15 offset:304\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(k0), "=&v"(k1), "=&v"(s0), "=&v"(s1), "=&v"(x0), "=&v"(x1), "=&v"(x2), "=&v"(x3), "=&v"(x4),
            "=&v"(x5), "=&v"(x6), "=&v"(x7)
          : "v"(ka), "v"(ksa), "v"(vsa), "v"(va)
          : "memory");
      in.kx[0][0] = k0;
      in.kx[1][0] = k1;
#pragma unroll
      for (int q = 0; q < RV; ++q) { in.kw[q] = s0[q & 3]; in.vw[q] = s1[q & 3]; }
    } else {  // G == 8, not redistributed
      uint32_t k0, k1;
      u32x4 s0, s1, s2, s3;
      asm volatile(
          "ds_read_b32 %0, %14\n\tds_read_b32 %1, %14 offset:256\n\t"
          "ds_read_b128 %2, %15\n\tds_read_b128 %3, %15 offset:64\n\t"
          "ds_read_b128 %4, %16\n\tds_read_b128 %5, %16 offset:64\n\t"
          "ds_read_u8 %6, %17\n\tds_read_u8 %7, %17 offset:16\n\t"
          "ds_read_u8 %8, %17 offset:32\n\tds_read_u8 %9, %17 offset:48\n\t"
          "ds_read_u8 %10, %17 offset:256\n\tds_read_u8 %11, %17 offset:272\n\t"
          "ds_read_u8 %12, %17 offset:288\n\tds_read_u8 %13, %17 offset:304\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(k0), "=&v"(k1), "=&v"(s0), "=&v"(s1), "=&v"(s2), "=&v"(s3), "=&v"(x0), "=&v"(x1), "=&v"(x2),
            "=&v"(x3), "=&v"(x4), "=&v"(x5), "=&v"(x6), "=&v"(x7)
          : "v"(ka), "v"(ksa), "v"(vsa), "v"(va)
          : "memory");
      in.kx[0][0] = k0;
      in.kx[1][0] = k1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        in.kw[i % RV] = s0[i]; in.kw[(4 + i) % RV] = s1[i];
        in.vw[i % RV] = s2[i]; in.vw[(4 + i) % RV] = s3[i];
      }
    }
    in.vx[0] = x0; in.vx[1] = x1; in.vx[2] = x2; in.vx[3] = x3;
    in.vx[4] = x4; in.vx[5] = x5; in.vx[6] = x6; in.vx[7] = x7;
  };

  // One step: K gathers + score MFMAs; V gathers (independent of the softmax,
  // issued early); softmax; value MFMAs.  The step's global words were loaded one
  // step earlier into the other buffer.
  auto compute_step = [&]<bool full>(const StepIn& in, int base) {
    // ---------------- scores: two 16-token halves (rows = tokens, cols = head slots)
    floatx4 sc[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      floatx4 d = {0.f, 0.f, 0.f, 0.f};
      if (G == 4) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint32_t wd = in.kx[a][s >> 1];
          const uint2 e0 = *reinterpret_cast<const uint2*>(tab + gather_addr<G>(wd, laneoff, (2 * s) & 3));
          const uint2 e1 = *reinterpret_cast<const uint2*>(tab + gather_addr<G>(wd, laneoff, (2 * s + 1) & 3));
          const uint4 av = make_uint4(e0.x, e0.y, e1.x, e1.y);
          d = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, av), QB[s], d, 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint4 av = *reinterpret_cast<const uint4*>(tab + gather_addr<G>(in.kx[a][0], laneoff, s));
          d = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, av), QB[s], d, 0, 0, 0);
        }
      }
      sc[a] = d;
    }
    // ---------------- value gathers for every 16-column block
    uint32_t E[NB][8][NT / 2];
#pragma unroll
    for (int bl = 0; bl < NB; ++bl)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t ad = gather_addr<G>(in.vx[e], laneoff, (G == 4) ? bl : 0);
        if (G == 4) {
          const uint2 ev = *reinterpret_cast<const uint2*>(tab + ad);
          E[bl][e][0] = ev.x;
          E[bl][e][NT / 2 - 1] = ev.y;
        } else {
          const uint4 ev = *reinterpret_cast<const uint4*>(tab + ad);
          E[bl][e][0] = ev.x;
          E[bl][e][1 % (NT / 2)] = ev.y;
          E[bl][e][2 % (NT / 2)] = ev.z;
          E[bl][e][3 % (NT / 2)] = ev.w;
        }
      }
    // ---------------- online softmax.  Lane (slot n, group grp) holds tokens
    // base + 16a + 4 grp + r; slot n + GQ carries the lo part of head n's dot.
    constexpr int NW = RED ? RV : 8;
    float pw[NW];  // this lane's value weights of the step
    float corr;
    if constexpr (RED) {
      // Redistribute: head h's 8 token dots (flat f = 4a + r, in lane h) go to
      // lane h + GQ (f / RV), register f % RV, so all 16 lanes of a row hold live
      // values (RV = GQ / 2 each).  DPP banks are 4 lanes: the destination lanes
      // of step k are banks [GQ k / 4, GQ (k+1) / 4).
      float v8[8];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float d = sc[a][r];
          v8[4 * a + r] = d + row_shl<GQ>(d);
        }
      float val[RV];
#pragma unroll
      for (int q = 0; q < RV; ++q) val[q] = v8[q];
#pragma unroll
      for (int k = 1; k < 16 / GQ; ++k) {
#pragma unroll
        for (int q = 0; q < RV; ++q) {
          if (GQ == 4) {
            if (k == 1) val[q] = shr_into<4, 0x2>(val[q], v8[1 * RV + q]);
            if (k == 2) val[q] = shr_into<8, 0x4>(val[q], v8[2 * RV + q]);
            if (k == 3) val[q] = shr_into<12, 0x8>(val[q], v8[3 * RV + q]);
          } else {  // GQ == 8
            if (k == 1) val[q] = shr_into<8, 0xc>(val[q], v8[1 * RV + q]);
          }
        }
      }
      float s8[RV];
      float mloc = -INFINITY;
#pragma unroll
      for (int q = 0; q < RV; ++q) {
        const float ks1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(in.kw[q] & 0xffffu));
        const float ks2 = (float)__builtin_bit_cast(_Float16, (uint16_t)(in.kw[q] >> 16));
        float sv = ks1 * (ks2 * val[q] + qo);
        if (!full && base + rtok0 + q >= c1) sv = -INFINITY;
        s8[q] = sv;
        mloc = fmaxf(mloc, sv);
      }
      // max over the lanes of head h: h + GQ k in every row
      if (GQ == 4) {
        mloc = max2(mloc, row_ror<4>(mloc));
        mloc = max2(mloc, row_ror<8>(mloc));
      } else {
        mloc = max2(mloc, row_ror<8>(mloc));
      }
      mloc = rows_max(mloc);
      corr = 1.f;
      if (__any(mloc > m_run + kLazyMax)) {  // the first computed step always moves it
        const float m_new = fmaxf(m_run, mloc);
        corr = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
      }
      float lsum = 0.f, bsum = 0.f;
#pragma unroll
      for (int q = 0; q < RV; ++q) {
        const float vs1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(in.vw[q] & 0xffffu));
        const float vs2 = (float)__builtin_bit_cast(_Float16, (uint16_t)(in.vw[q] >> 16));
        const float pv = __builtin_amdgcn_exp2f(s8[q] - m_run);  // masked tokens: exp2(-inf) = 0
        float p1 = __builtin_fmaf(vs1, pv, 0.f);
        float p2 = __builtin_fmaf(vs2, p1, 0.f);
        if (!full && base + rtok0 + q >= c1) {
          p1 = 0.f;  // a masked token's scales may be any bits (even NaN): select, don't multiply
          p2 = 0.f;
        }
        lsum += pv;
        bsum += p1;
        pw[q] = p2;
      }
      l_run = l_run * corr + lsum;
      beta_run = beta_run * corr + bsum;
    } else {
      float s8[8];
      float mloc = -INFINITY;
#pragma unroll
      for (int a = 0; a < 2; ++a) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 4 * a + r;
          const float d = sc[a][r];
          const float dsum = d + row_shl<GQ>(d);
          // s1 (low half) and s2' (high half) feed v_fma_mix directly
          const float ks1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(in.kw[i % RV] & 0xffffu));
          const float ks2 = (float)__builtin_bit_cast(_Float16, (uint16_t)(in.kw[i % RV] >> 16));
          float sv = ks1 * (ks2 * dsum + qo);
          if (!full && base + 16 * a + 4 * grp + r >= c1) sv = -INFINITY;
          s8[i] = sv;
          mloc = fmaxf(mloc, sv);
        }
      }
      mloc = rows_max(mloc);
      corr = 1.f;
      if (__any(n < GQ && mloc > m_run + kLazyMax)) {  // live head slots decide
        const float m_new = fmaxf(m_run, mloc);
        corr = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
      }
      float lsum = 0.f, bsum = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float vs1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(in.vw[i % RV] & 0xffffu));
        const float vs2 = (float)__builtin_bit_cast(_Float16, (uint16_t)(in.vw[i % RV] >> 16));
        const float pv = __builtin_amdgcn_exp2f(s8[i] - m_run);  // masked tokens: exp2(-inf) = 0
        float p1 = __builtin_fmaf(vs1, pv, 0.f);                 // v_fma_mix: fp16 operand read in place
        float p2 = __builtin_fmaf(vs2, p1, 0.f);
        if (!full && base + 16 * (i >> 2) + 4 * grp + (i & 3) >= c1) {
          p1 = 0.f;  // a masked token's scales may be any bits (even NaN): select, don't multiply
          p2 = 0.f;
        }
        lsum += pv;
        bsum += p1;
        pw[i] = p2;
      }
      l_run = l_run * corr + lsum;
      beta_run = beta_run * corr + bsum;
    }
    // weights in units of 2^vexp; dead lanes (plain layout, n >= GQ) never count
    float wm = 0.f;
#pragma unroll
    for (int q = 0; q < NW; ++q) {
      pw[q] = __builtin_amdgcn_ldexpf(pw[q], -vexp);
      wm = fmaxf(wm, pw[q]);
    }
    if (!RED && n >= GQ) wm = 0.f;
    // rescale accumulators (rows 4 grp + r are head slots) unless no head's max
    // moved and every weight fits
    if (__any(corr != 1.f || wm > 16384.f)) {
      // row 4 grp + r is head slot 4 grp + r; head h's factor sits in lane h.  Live
      // slots are < GQ <= 8, so only grp 0 (and grp 1 for GQ = 8) rows matter: the
      // factors come from v_readlane (no LDS-pipe instruction here, see the stage ring)
      float cr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float lo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(corr), r));
        if constexpr (GQ > 4) {
          const float hi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(corr), 4 + r));
          cr[r] = grp == 0 ? lo : hi;
        } else {
          cr[r] = lo;
        }
      }
      if (__any(wm > 16384.f)) {
        // rare: raise vexp by k so that the wave's largest weight, m in [2^(e-1), 2^e),
        // drops to at most 2^14; sums and this step's weights shift by the same 2^-k
        float m = max2(wm, row_ror<8>(wm));
        m = max2(m, row_ror<4>(m));
        m = max2(m, row_ror<2>(m));
        m = max2(m, row_ror<1>(m));
        m = rows_max(m);
        const int k = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_frexp_expf(m) - 14);
        vexp += k;
#pragma unroll
        for (int r = 0; r < 4; ++r) cr[r] = __builtin_amdgcn_ldexpf(cr[r], -k);
#pragma unroll
        for (int q = 0; q < NW; ++q) pw[q] = __builtin_amdgcn_ldexpf(pw[q], -k);
      }
#pragma unroll
      for (int bl = 0; bl < NB; ++bl)
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[bl][t][r] *= cr[r];
    }
    half8 PA;
    if constexpr (RED) {
      // back to the value-MFMA A layout: row h holds tokens f = 0..7 (half e = f).
      // Lane h + GQ k packs its RV values (f = k RV ..) into RV / 2 dwords; dword
      // j = f / 2 of row h comes from lane h + GQ (2 j / RV).  Dead rows stay 0.
      uint32_t pk[RV / 2];
#pragma unroll
      for (int j = 0; j < RV / 2; ++j)
        pk[j] = pack_f16_rne(pw[2 * j], pw[2 * j + 1]);
      const uint32_t own = n < GQ ? 0xffffffffu : 0u;
      uint32_t pa[4];
      if (GQ == 4) {  // RV = 2: one dword per lane; row h = lanes 0..3 (bank 0)
        pa[0] = pk[0] & own;
        pa[1] = shl_into<4, 0x1>(0u, pk[0]);
        pa[2] = shl_into<8, 0x1>(0u, pk[0]);
        pa[3] = shl_into<12, 0x1>(0u, pk[0]);
      } else {  // GQ == 8, RV = 4: two dwords per lane; rows 0..7 (banks 0, 1)
        pa[0] = pk[0] & own;
        pa[1] = pk[(RV / 2) - 1] & own;
        pa[2] = shl_into<8, 0x3>(0u, pk[0]);
        pa[3] = shl_into<8, 0x3>(0u, pk[(RV / 2) - 1]);
      }
      PA = __builtin_bit_cast(half8, make_uint4(pa[0], pa[1], pa[2], pa[3]));
    } else {
      uint4 pa;
      pa.x = pack_f16_rne(pw[0], pw[1]);
      pa.y = pack_f16_rne(pw[2], pw[3]);
      pa.z = pack_f16_rne(pw[4], pw[5]);
      pa.w = pack_f16_rne(pw[6], pw[7]);
      pa.x &= live_mask; pa.y &= live_mask; pa.z &= live_mask; pa.w &= live_mask;
      PA = __builtin_bit_cast(half8, pa);
    }
    // ---------------- values: B = centroid channel t of the lane's 8 tokens
#pragma unroll
    for (int bl = 0; bl < NB; ++bl) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
        uint4 bv;
        bv.x = __builtin_amdgcn_perm(E[bl][1][t >> 1], E[bl][0][t >> 1], sel);
        bv.y = __builtin_amdgcn_perm(E[bl][3][t >> 1], E[bl][2][t >> 1], sel);
        bv.z = __builtin_amdgcn_perm(E[bl][5][t >> 1], E[bl][4][t >> 1], sel);
        bv.w = __builtin_amdgcn_perm(E[bl][7][t >> 1], E[bl][6][t >> 1], sel);
        acc[bl][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(PA, __builtin_bit_cast(half8, bv), acc[bl][t], 0, 0, 0);
      }
    }
  };

  // ---------------- block steps: wait for the staged step, refill the freed slot,
  // every wave computes its 32 tokens.  Full block steps (all 256 tokens valid) run
  // unrolled over the four ring slots so that each refill and each read names its
  // slot statically; a final partial step (if any) follows with masking.
  // Each wave needs only its own vmcnt wait: it reads and refills nothing but its
  // own region, so the waves drift apart freely (no barrier per step).  The asm
  // clobber keeps the compiler from moving LDS accesses across.
  auto wait_stage = [&]() {
    wait_vm<(kStages - 2) * LPS>();  // this wave's loads of the oldest step in flight are done
    asm volatile("" ::: "memory");
  };
  auto full_step = [&]<int SL>(int st) {
    wait_stage();
    unsigned char* const rd = SL == 0 ? s_st0 : SL == 1 ? s_st1 : SL == 2 ? s_st2 : s_st3;
    unsigned char* const wr = SL == 0 ? s_st3 : SL == 1 ? s_st0 : SL == 2 ? s_st1 : s_st2;
    StepIn in;
    read_in(in, rd);  // before the refill: reads and the new loads stay apart
    issue_into(wr, st + kStages - 1);
    compute_step.template operator()<true>(in, c0 + st * kStepSpan + 32 * wave);
  };
  // unguarded groups of four full steps: no control-flow join inside a group, so the
  // compiler keeps exact track of which slot each load in flight writes
  const int nfull = (c1 - c0) / kStepSpan;
  const int ngrp = nfull / 4;
  for (int g4 = 0; g4 < ngrp; ++g4) {
    const int st = 4 * g4;
    full_step.template operator()<0>(st);
    full_step.template operator()<1>(st + 1);
    full_step.template operator()<2>(st + 2);
    full_step.template operator()<3>(st + 3);
  }
  // remaining full steps and the partial last step: slots named dynamically (the
  // compiler then drains the loads in flight first -- only for these last steps)
  for (int st = 4 * ngrp; st < nsteps; ++st) {
    wait_stage();
    const int sl = st & 3;
    unsigned char* const rd = sl == 0 ? s_st0 : sl == 1 ? s_st1 : sl == 2 ? s_st2 : s_st3;
    unsigned char* const wr = sl == 0 ? s_st3 : sl == 1 ? s_st0 : sl == 2 ? s_st1 : s_st2;
    const int bs = c0 + st * kStepSpan + 32 * wave;
    StepIn in;
    if (bs < c1) read_in(in, rd);
    issue_into(wr, st + kStages - 1);
    if (bs < c1) compute_step.template operator()<false>(in, bs);
  }
  wait_vm<0>();  // the trailing refills (dummy rows) have landed

  // ---------------- per-wave state -> LDS -> block merge -> workspace
  if constexpr (RED) {  // partial sums are spread over lanes h + GQ k of each row
    if (GQ == 4) {
      l_run += row_ror<4>(l_run);
      l_run += row_ror<8>(l_run);
      beta_run += row_ror<4>(beta_run);
      beta_run += row_ror<8>(beta_run);
    } else {
      l_run += row_ror<8>(l_run);
      beta_run += row_ror<8>(beta_run);
    }
  }
  l_run = rows_sum(l_run);
  beta_run = rows_sum(beta_run);
  __syncthreads();  // table no longer needed: reuse it for the partials
  // APP: entry kWaves is the decode step's new token (last chunk only)
  constexpr int NE = kWaves + (APP ? 1 : 0);
  bool app = false;
  if constexpr (APP) app = chunk == nchunk - 1;
  float* s_acc = reinterpret_cast<float*>(s_tab);             // [NE][GQ heads][128]
  float* s_st = s_acc + NE * GQ * kD;                          // [NE][GQ][3]
#pragma unroll
  for (int bl = 0; bl < NB; ++bl)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int slot = 4 * grp + r;
        const int j = (G == 4) ? (2 * n + bl) : n;
        if (slot < GQ)
          s_acc[((size_t)wave * GQ + slot) * kD + G * j + t] = __builtin_amdgcn_ldexpf(acc[bl][t][r], vexp);
      }
  if (grp == 0 && n < GQ) {
    s_st[(wave * GQ + n) * 3 + 0] = m_run;
    s_st[(wave * GQ + n) * 3 + 1] = l_run;
    s_st[(wave * GQ + n) * 3 + 2] = beta_run;
  }
  if constexpr (APP) {
    if (app && wave == kWaves - 1) {
      // encode the pair (half 0: K, half 1: V) with the stored o, write the records
      const int hf = lane >> 5, p = lane & 31;
      const size_t row = (size_t)bh * S_cap + ap.pos;
      float wq[4], s1q, s2q;
      encode_pair<G, true>((hf ? ap.v_new : ap.k_new) + (size_t)bh * kD, (hf ? ap.v_o : ap.k_o) + (size_t)bh * kD,
                           ap.encA, ap.c32, smask, lane, s_acc + 12 * 1024, (hf ? ap.v_idx : ap.k_idx) + row * M,
                           (hf ? ap.v_sc : ap.k_sc) + row * 2, wq, s1q, s2q);
      // the token's partial: its own maximum (its score, log2 units as in the
      // loop), l = 1, beta = s1_V, acc = s1_V s2'_V w_hat_V (rotated domain)
      const float ks1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s1q), 0));
      const float ks2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s2q), 0));
      const float vs1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s1q), 32));
      const float vs2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s2q), 32));
#pragma unroll
      for (int hh = 0; hh < GQ; ++hh) {
        float dk = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) dk = fmaf(s_q[hh][4 * p + c], wq[c], dk);
        dk = half_sum_swz(dk);  // half 0: <q~, w_hat_K>
        const float dkk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dk), 0));
        if (hf == 1) {
#pragma unroll
          for (int c = 0; c < 4; ++c) s_acc[((size_t)kWaves * GQ + hh) * kD + 4 * p + c] = vs1 * vs2 * wq[c];
        }
        if (lane == 0) {
          s_st[(kWaves * GQ + hh) * 3 + 0] = ks1 * (ks2 * dkk + s_qo[hh]);
          s_st[(kWaves * GQ + hh) * 3 + 1] = 1.f;
          s_st[(kWaves * GQ + hh) * 3 + 2] = vs1;
        }
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < GQ * kD; i += kThreads) {
    const int h = i / kD, c = i % kD;
    const int nent = app ? kWaves + 1 : kWaves;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NE; ++w)
      if (w < nent) M = fmaxf(M, s_st[(w * GQ + h) * 3]);
    float a = 0.f, l = 0.f, be = 0.f;
#pragma unroll
    for (int w = 0; w < NE; ++w) {
      if (w >= nent) break;
      const float mw = s_st[(w * GQ + h) * 3];
      const float f = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      a += f * s_acc[((size_t)w * GQ + h) * kD + c];
      l += f * s_st[(w * GQ + h) * 3 + 1];
      be += f * s_st[(w * GQ + h) * 3 + 2];
    }
    float* dst = part + (((size_t)b * Hq + (size_t)hk * GQ + h) * nchunk + chunk) * kPartStride;
    dst[4 + c] = a;
    if (c == 0) {
      dst[0] = M;
      dst[1] = l;
      dst[2] = be;
      dst[3] = 0.f;
    }
  }
}

// max over the 64 lanes of a wave, every lane gets the result
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, swz_xor<1>(v));
  v = fmaxf(v, swz_xor<2>(v));
  v = fmaxf(v, swz_xor<4>(v));
  v = fmaxf(v, swz_xor<8>(v));
  v = fmaxf(v, swz_xor<16>(v));
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Merge the chunk partials of one (batch, query head) and leave the rotated domain.
// The chunk maxima are read first (all at once) and reduced to the block maximum M
// (per wave, then over the four waves); then 8 groups of 32 threads (4 channels
// each) add every 8th chunk's partial scaled by exp2(m_i - M) -- independent
// loads, no serial rescaling chain -- and one half-wave merges the groups in a
// fixed order and applies H in registers (two barriers in all).
//
// RES: the full-precision residual window ([IMPL] "Residuals": the newest tokens
// stay unquantized until the window fills) joins the same softmax.  Its partial
// (m, l, acc[128] already in the original domain, from the window's workgroup of
// k_decode) is added to H(acc) + beta o_V with the usual max rescaling.
// nchunk = 0 (no quantized tokens) leaves only the window.
// SEG: the chunks from nchunk0 on are flushed blocks with their own o_V
// (v_ob[j][b][h]); the beta o_V part is then summed per chunk, in the original
// domain, beside the rotated-domain sums.
template <bool RES, bool DQ, bool SEG = false>
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ part, int nchunk, int Hq, int Hkv,
                                                 const float* __restrict__ v_o, const nsn_dq_head* __restrict__ v_hd,
                                                 const float* __restrict__ rpart, float* __restrict__ out,
                                                 uint4 smask, const float* __restrict__ v_ob = nullptr,
                                                 int nchunk0 = 0, int BH = 0) {
  __shared__ float s_m[4];
  __shared__ float s_l[8], s_be[8];
  __shared__ float4 s_a[8][32];
  __shared__ float4 s_bo[SEG ? 8 : 1][32];
  const int bq = blockIdx.x, tid = threadIdx.x, gi = tid >> 5, c4 = tid & 31;
  const int b = bq / Hq, hq = bq % Hq;
  const int hk = hq / (Hq / Hkv);
  const float* pp = part + (size_t)bq * nchunk * kPartStride;
  // block maximum of the chunk maxima: per wave, then over the four waves
  {
    float m = -INFINITY;
    for (int i = tid; i < nchunk; i += 256) m = fmaxf(m, pp[(size_t)i * kPartStride]);
    m = wave_max(m);
    if ((tid & 63) == 0) s_m[tid >> 6] = m;
  }
  __syncthreads();
  const float M = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
  float l = 0.f, be = 0.f;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  float4 bo = make_float4(0.f, 0.f, 0.f, 0.f);  // SEG: sum of f beta o_V, channels 4 c4 ..
  const int bh = b * Hkv + hk;
#pragma unroll 4
  for (int i = gi; i < nchunk; i += 8) {
    const float* pc = pp + (size_t)i * kPartStride;
    const float mi = pc[0];
    const float f = (mi == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mi - M);
    const float4 v = reinterpret_cast<const float4*>(pc + 4)[c4];
    l += pc[1] * f;
    be += pc[2] * f;
    a.x += v.x * f; a.y += v.y * f; a.z += v.z * f; a.w += v.w * f;
    if constexpr (SEG) {
      const float* vo = i < nchunk0 ? v_o + (size_t)bh * kD : v_ob + ((size_t)(i - nchunk0) * BH + bh) * kD;
      const float4 o4 = reinterpret_cast<const float4*>(vo)[c4];
      const float fb = f * pc[2];
      bo.x += fb * o4.x; bo.y += fb * o4.y; bo.z += fb * o4.z; bo.w += fb * o4.w;
    }
  }
  s_a[gi][c4] = a;
  if constexpr (SEG) s_bo[gi][c4] = bo;
  if (c4 == 0) { s_l[gi] = l; s_be[gi] = be; }
  __syncthreads();
  if (tid >= 64) return;
  // wave 0: lane p of each half holds channels 4p .. 4p+3 (the pair layout), the
  // groups merge in a fixed order and H runs in registers
  const int p = tid & 31;
  float t[4];
  {
    float4 u = s_a[0][p];
#pragma unroll
    for (int g = 1; g < 8; ++g) {
      const float4 v = s_a[g][p];
      u.x += v.x; u.y += v.y; u.z += v.z; u.w += v.w;
    }
    t[0] = u.x; t[1] = u.y; t[2] = u.z; t[3] = u.w;
  }
  float L = 0.f, BE = 0.f;
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    L += s_l[g];
    BE += s_be[g];
  }
  fwht128_pair(t, p);
  flip4(t, lane_signs(smask, p));  // randomized rotation: D H
  if (tid >= 32) return;
  const float rs = 0.08838834764831845f;
  float num[4] = {0.f, 0.f, 0.f, 0.f}, den = 0.f;
  if (nchunk > 0) {
    float vo[4];
    if constexpr (DQ) {
      const nsn_dq_head* hd = v_hd + (size_t)b * Hkv + hk;
      const uint32_t nb = *reinterpret_cast<const uint16_t*>(hd->o_codes + 2 * p);
#pragma unroll
      for (int c = 0; c < 4; ++c) vo[c] = (float)((int)((nb >> (4 * c)) & 15u) - 8) * hd->o_scale;
    } else {
      const float4 v4 = reinterpret_cast<const float4*>(v_o + ((size_t)b * Hkv + hk) * kD)[p];
      vo[0] = v4.x; vo[1] = v4.y; vo[2] = v4.z; vo[3] = v4.w;
    }
    if constexpr (SEG) {
      float4 u = s_bo[0][p];
#pragma unroll
      for (int g = 1; g < 8; ++g) {
        const float4 v = s_bo[g][p];
        u.x += v.x; u.y += v.y; u.z += v.z; u.w += v.w;
      }
      const float ub[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int c = 0; c < 4; ++c) num[c] = fmaf(t[c], rs, ub[c]);
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) num[c] = fmaf(t[c], rs, BE * vo[c]);
    }
    den = L;
  }
  if constexpr (RES) {
    const float* rp = rpart + (size_t)bq * kPartStride;
    const float Mr = rp[0], lr = rp[1];
    const float4 a4 = reinterpret_cast<const float4*>(rp + 4)[p];
    const float ar[4] = {a4.x, a4.y, a4.z, a4.w};
    const float Mt = fmaxf(M, Mr);
    const float fc = (nchunk > 0) ? __builtin_amdgcn_exp2f(M - Mt) : 0.f;
    const float fr = (Mr == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(Mr - Mt);
#pragma unroll
    for (int c = 0; c < 4; ++c) num[c] = fc * num[c] + fr * ar[c];
    den = fc * den + fr * lr;
  }
  reinterpret_cast<float4*>(out + (size_t)bq * kD)[p] = make_float4(num[0] / den, num[1] / den, num[2] / den,
                                                                    num[3] / den);
}

// ---------------------------------------------------------------- keys before RoPE
// "4. Implementation Details": NSN runs on the keys before the rotary position
// embedding, so the cache holds pre-RoPE keys and the score rotates each
// dequantized key by its position: score_i = q . R(i) k_hat_i / sqrt(d), q the
// query already rotated to its own position, R the rotate-half embedding (channel
// j pairs with j + 64, angle i theta_j, theta_j = base^(-j/64)).  A rotation that
// changes with the token does not commute with H, so this path dequantizes every
// key in the original domain (FWHT of the gathered centroids) instead of scoring
// in the rotated domain; the values keep the rotated-domain accumulation, and the
// partials (m, l, beta, acc) have the same layout as k_decode's, so k_combine
// finishes both.
//
// cos / sin of i theta_j = angle sum of (256 (i >> 8)) theta_j and (i & 255) theta_j,
// from two tables built in fp64: ta[a][j] (a < na) and, right after it, tb[b][j]
// (b < 256), both as (cos, sin) in fp32.  They depend only on the RoPE base and the
// number of positions, so one pair serves every codebook and every call up to that
// length; the sign the randomized rotation gives a frequency's sine is applied in the
// decode kernel.
__global__ __launch_bounds__(256) void k_rope_tables(double ln_base, int na, float2* __restrict__ ta) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int j = i & 63, r = i >> 6;
  const double theta = exp(-(double)j / 64.0 * ln_base);
  if (r < na) {
    const double a = 256.0 * (double)r * theta;
    ta[i] = make_float2((float)cos(a), (float)sin(a));
  }
  if (r < 256) {
    const double b = (double)r * theta;
    ta[(size_t)na * 64 + i] = make_float2((float)cos(b), (float)sin(b));
  }
}

// Grid (nchunk, Hkv, B), 256 threads (4 waves).  A wave takes 16 consecutive tokens
// per step (wave w, step k: tokens c0 + 64 k + 16 w + n for lane n % 16):
//  * the key's w_hat is gathered from the bank-replicated LDS codebook straight into
//    the B operand of H_sylvester (16x16x32 fp16 MFMA with the encode's +-1
//    fragments): lane (g = lane / 16, n) then holds channels 16 mt + 4 g + r of
//    token n's H w_hat, mt = 0..7, r = 0..3 -- both channels of every rotary pair
//    (c, c + 64) in one lane;
//  * x = s2' H w_hat / sqrt(d) + D o is rotated by the token's position with the
//    (cos, sin) each lane carries for its 16 frequencies (advanced by e^(64 i theta)
//    per step, taken from the fp64-built tables every 32 steps) and split into fp16
//    hi + lo parts.  In the D-signed domain the sine of frequency f changes sign
//    where channels f and f + 64 carry different signs;
//  * scores on the matrix cores: A = the rotated keys (rows = tokens), B = the query
//    in the same channel order (hi parts in head slots 0..GQ-1, lo parts in
//    GQ..2GQ-1), fp32 sums: k_decode's score layout, so its online softmax and value
//    products (here 16x16x16 MFMA over the 16 tokens, rotated domain) follow;
//  * a step's index rows and scale words are staged per wave in LDS; a token past the
//    chunk's end gets zero value scales there, so its weights vanish without a
//    per-step select, and its score is set to -inf on the rare partial step only.
// The partials (m, l, beta, acc[128]) have k_decode's layout, so k_combine finishes.
template <int G, int GQ>
__global__ __launch_bounds__(256, 1) void k_decode_rope(const uint16_t* __restrict__ q, int Hq, int Hkv, int S,
                                                        int S_cap, int CH, int nchunk,
                                                        const uint8_t* __restrict__ k_idx,
                                                        const uint16_t* __restrict__ k_sc,
                                                        const float* __restrict__ k_o,
                                                        const uint8_t* __restrict__ v_idx,
                                                        const uint16_t* __restrict__ v_sc,
                                                        const uint16_t* __restrict__ c16x2,
                                                        const float2* __restrict__ ta, const float2* __restrict__ tb,
                                                        float* __restrict__ part, uint4 smask) {
  constexpr int M = kD / G;                 // indices per token
  constexpr int NB = (G == 4) ? 2 : 1;      // 16-column value blocks
  constexpr int NT = G;                     // channel offsets per sub-vector
  constexpr int RB = 32 * M;                // a step's K rows (16 tokens), then its V rows
  constexpr int WB = RB + 128;              // + the K and V scale words of the 16 tokens
  __shared__ __attribute__((aligned(256))) unsigned char s_tab[kK * 256];  // replicated codebook
  __shared__ __attribute__((aligned(16))) unsigned char s_stage[4][WB];
  __shared__ __attribute__((aligned(16))) float s_ko[kD];     // D o_K
  __shared__ __attribute__((aligned(16))) float2 s_step[64];  // e^(64 i theta_j), D-domain sine sign
  const int chunk = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, grp = lane >> 4;
  const int bh = b * Hkv + hk;
  const int c0 = chunk * CH, c1 = min(S, c0 + CH);
  const size_t row0 = (size_t)bh * S_cap;

  // ---- the codebook (16 copies of each 16-byte entry per 256-byte row) by LDS-DMA
#pragma unroll
  for (int i = 0; i < kK * 256 / 1024 / 4; ++i) {
    const int blk = wave * (kK * 256 / 1024 / 4) + i;
    __builtin_amdgcn_global_load_lds(c16x2 + (size_t)(4 * blk + (lane >> 4)) * 8, s_tab + 1024 * blk, 16, 0, 0);
  }
  const uint32_t smw[4] = {smask.x, smask.y, smask.z, smask.w};
  if (tid < kD) {
    const float sg = ((smw[tid >> 5] >> (tid & 31)) & 1u) ? -1.f : 1.f;
    s_ko[tid] = sg * k_o[(size_t)bh * kD + tid];
  } else if (tid < kD + 64) {
    const int j = tid - kD;
    const float2 w = tb[(size_t)64 * 64 + j];
    const bool flip = ((smw[j >> 5] ^ smw[2 + (j >> 5)]) >> (j & 31)) & 1u;  // channels j, j + 64 differ
    s_step[j] = make_float2(w.x, flip ? -w.y : w.y);
  }
  // ---- score B operand: q~ = c D q (c = log2(e) / sqrt(d): scores in log2 units) in
  // the rotated key's channel order: step s, slot 8 grp + e <-> channel 16 (2 s + e / 4)
  // + 4 grp + e % 4
  const float cscale = 1.4426950408889634f * 0.08838834764831845f;
  half8 QB[4];
  {
    // every lane loads (slots past 2 GQ read head 0 and are zeroed): 8 four-channel loads
    const _Float16* qr = reinterpret_cast<const _Float16*>(q) + ((size_t)b * Hq + (size_t)hk * GQ + (n % GQ)) * kD;
    half4 qh[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) qh[u] = *reinterpret_cast<const half4*>(qr + 16 * u + 4 * grp);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int u = 2 * s + (e >> 2), c = 16 * u + 4 * grp + (e & 3);
        const float sg = ((smw[c >> 5] >> (c & 31)) & 1u) ? -1.f : 1.f;
        const float qv = sg * cscale * (float)qh[u][e & 3];
        const _Float16 hi = (_Float16)qv;
        const _Float16 val = (n < GQ) ? hi : (_Float16)(qv - (float)hi);
        QB[s][e] = n < 2 * GQ ? val : (_Float16)0.f;
      }
    }
  }
  // H_sylvester fragments of this lane
  const half8 F0p = hsyl_frag(lane, 0, 0), F0n = hsyl_frag(lane, 0, 1);
  const half8 F1p = hsyl_frag(lane, 1, 0), F1n = hsyl_frag(lane, 1, 1);
  const uint32_t live_mask = n < GQ ? 0xffffffffu : 0u;
  const uint32_t laneoff = (G == 4) ? 8u * (lane & 31) : 16u * (lane & 15);
  wait_vm<0>();      // this wave's codebook DMA has landed
  __syncthreads();  // table, D o_K and the step rotation in LDS

  // ---- rotation state of this lane's token: frequencies j = 16 mt + 4 grp + r (mt, r < 4)
  float zc[16], zs[16];
  const int na = (S + 255) / 256;  // rows of the coarse table read here
  auto anchor = [&](int pos) {
    // bit 4 mt + r: the sine sign of frequency 16 mt + 4 grp + r flips in the D domain
    // (rebuilt here, every 32 steps, rather than held in a register)
    uint32_t swl = 0;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      swl |= (((smw[mt >> 1] ^ smw[2 + (mt >> 1)]) >> (16 * (mt & 1) + 4 * grp)) & 0xfu) << (4 * mt);
    asm volatile("" : "+v"(swl));  // opaque: the 16 sign masks are not hoisted out of the loop
    const int pa = min(pos >> 8, na - 1);
    const float2* ra = ta + (size_t)pa * 64 + 4 * grp;
    const float2* rb = tb + (size_t)(pos & 255) * 64 + 4 * grp;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float4 a4 = *reinterpret_cast<const float4*>(ra + 16 * mt + 2 * h);
        const float4 b4 = *reinterpret_cast<const float4*>(rb + 16 * mt + 2 * h);
        const int f = 4 * mt + 2 * h;
        zc[f] = a4.x * b4.x - a4.y * b4.y;
        zs[f] = __uint_as_float(__float_as_uint(a4.y * b4.x + a4.x * b4.y) ^ (((swl >> f) & 1u) << 31));
        zc[f + 1] = a4.z * b4.z - a4.w * b4.w;
        zs[f + 1] = __uint_as_float(__float_as_uint(a4.w * b4.z + a4.z * b4.w) ^ (((swl >> (f + 1)) & 1u) << 31));
      }
    }
  };

  // ---- a step's loads: the 16 tokens' K and V index rows and scale words; rows past
  // the slab's last row are clamped to it (their tokens are masked)
  unsigned char* const stg = s_stage[wave];
  auto load_step = [&](int k, uint4& rw, uint32_t& sw) {
    const int t0 = c0 + 64 * k + 16 * wave;
    if constexpr (G == 4) {  // lanes 0-31: K rows (16 bytes each), 32-63: V rows; lanes 0-15 / 16-31: K / V words
      const int tt = min(t0 + ((lane & 31) >> 1), S_cap - 1);
      rw = *reinterpret_cast<const uint4*>((lane < 32 ? k_idx : v_idx) + (row0 + tt) * M + 16 * (lane & 1));
      const int tw = min(t0 + n, S_cap - 1);
      sw = *reinterpret_cast<const uint32_t*>(((lane & 16) ? v_sc : k_sc) + (row0 + tw) * 2);
    } else {  // lanes 0-15 / 16-31: K / V rows; lanes 32-47 / 48-63: K / V words
      const int tt = min(t0 + n, S_cap - 1);
      rw = *reinterpret_cast<const uint4*>(((lane & 16) ? v_idx : k_idx) + (row0 + tt) * M);
      sw = *reinterpret_cast<const uint32_t*>(((lane & 16) ? v_sc : k_sc) + (row0 + tt) * 2);
    }
  };
  auto stage_step = [&](const uint4& rw, uint32_t sw, int t0) {
    if ((lane & 16) && t0 + n >= c1) sw = 0u;  // the value words of tokens past the chunk
    if constexpr (G == 4) {
      *reinterpret_cast<uint4*>(stg + 16 * lane) = rw;
      if (lane < 32) *reinterpret_cast<uint32_t*>(stg + RB + 4 * lane) = sw;
    } else {
      if (lane < 32) *reinterpret_cast<uint4*>(stg + 16 * lane) = rw;
      else *reinterpret_cast<uint32_t*>(stg + RB + 4 * (lane - 32)) = sw;
    }
  };

  floatx4 acc[NB][NT];
#pragma unroll
  for (int bl = 0; bl < NB; ++bl)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[bl][t] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f, beta_run = 0.f;
  int vexp = 0;  // value sums in units of 2^vexp (fp16 weights, as in k_decode)

  const int nsteps = max(0, (c1 - c0 - 16 * wave + 63) / 64);
  // two steps' loads in flight: the loop runs two steps per iteration, each with its
  // own registers for the staged rows and words (named statically)
  auto step_body = [&](int k, uint4& rw, uint32_t& sw) {
    const int t0 = c0 + 64 * k + 16 * wave;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();  // the previous step's reads of the stage are done
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    stage_step(rw, sw, t0);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (k + 2 < nsteps) load_step(k + 2, rw, sw);  // two steps in flight
    // ---- K w_hat into the B operand of H_sylvester: step s, slots 8 grp + j <->
    // channels 32 s + 8 grp + j of token n
    half8 Bk[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if constexpr (G == 4) {
        const uint32_t w2 = *reinterpret_cast<const uint16_t*>(stg + 32 * n + 8 * s + 2 * grp);
        const uint2 e0 = *reinterpret_cast<const uint2*>(s_tab + gather_addr<4>(w2, laneoff, 0));
        const uint2 e1 = *reinterpret_cast<const uint2*>(s_tab + gather_addr<4>(w2, laneoff, 1));
        Bk[s] = __builtin_bit_cast(half8, make_uint4(e0.x, e0.y, e1.x, e1.y));
      } else {
        const uint32_t w1 = stg[16 * n + 4 * s + grp];
        Bk[s] = __builtin_bit_cast(half8, *reinterpret_cast<const uint4*>(s_tab + gather_addr<8>(w1, laneoff, 0)));
      }
    }
    floatx4 X[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) X[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const bool ng = hsyl_neg(mt, s);
        const half8 A = (mt & 1) ? (ng ? F1n : F1p) : (ng ? F0n : F0p);
        X[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bk[s], X[mt], 0, 0, 0);
      }
    // ---- x = s2' H w_hat / sqrt(d) + D o, rotated by the token's position
    const uint32_t kwn = *reinterpret_cast<const uint32_t*>(stg + RB + 4 * n);
    const float ka = (float)__builtin_bit_cast(_Float16, (uint16_t)(kwn >> 16)) * 0.08838834764831845f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const float4 oa = *reinterpret_cast<const float4*>(s_ko + 16 * mt + 4 * grp);
      const float4 ob = *reinterpret_cast<const float4*>(s_ko + 64 + 16 * mt + 4 * grp);
      const float oav[4] = {oa.x, oa.y, oa.z, oa.w}, obv[4] = {ob.x, ob.y, ob.z, ob.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int f = 4 * mt + r;
        const float xc = fmaf(ka, X[mt][r], oav[r]);
        const float xp = fmaf(ka, X[mt + 4][r], obv[r]);
        X[mt][r] = xc * zc[f] - xp * zs[f];
        X[mt + 4][r] = xp * zc[f] + xc * zs[f];
      }
    }
    // advance the lane's rotation by 64 positions (exact restart every 32 steps)
    if (((k + 1) & 31) == 0) {
      anchor(t0 + 64 + n);
    } else {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float4 w4 = *reinterpret_cast<const float4*>(s_step + 16 * mt + 4 * grp + 2 * h);
          const int f = 4 * mt + 2 * h;
          const float c0v = zc[f], s0v = zs[f], c1v = zc[f + 1], s1v = zs[f + 1];
          zc[f] = c0v * w4.x - s0v * w4.y;
          zs[f] = s0v * w4.x + c0v * w4.y;
          zc[f + 1] = c1v * w4.z - s1v * w4.w;
          zs[f + 1] = s1v * w4.z + c1v * w4.w;
        }
      }
    }
    // ---- scores: A = the rotated keys as fp16 hi + lo (slot 8 grp + e of step s is
    // channel 16 (2 s + e / 4) + 4 grp + e % 4: X[2 s + e / 4][e % 4])
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    typedef float f2 __attribute__((ext_vector_type(2)));
    floatx4 sc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v0 = X[2 * s + (e >> 1)][2 * (e & 1)], v1 = X[2 * s + (e >> 1)][2 * (e & 1) + 1];
        const h2 hh = __builtin_convertvector((f2){v0, v1}, h2);
        hw[e] = __builtin_bit_cast(uint32_t, hh);
        lw[e] = lo_pair(hw[e], v0, v1);
      }
      sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, make_uint4(hw[0], hw[1], hw[2], hw[3])),
                                                  QB[s], sc, 0, 0, 0);
      sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, make_uint4(lw[0], lw[1], lw[2], lw[3])),
                                                  QB[s], sc, 0, 0, 0);
    }
    // ---- online softmax.  Lane (slot n, group grp) holds tokens t0 + 4 grp + r;
    // slot n + GQ carries the lo part of head n's dot
    const uint4 kw4 = *reinterpret_cast<const uint4*>(stg + RB + 16 * grp);
    const uint4 vw4 = *reinterpret_cast<const uint4*>(stg + RB + 64 + 16 * grp);
    const uint32_t kwv[4] = {kw4.x, kw4.y, kw4.z, kw4.w}, vwv[4] = {vw4.x, vw4.y, vw4.z, vw4.w};
    float s4[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float d = sc[r];
      const float dsum = d + row_shl<GQ>(d);
      const float ks1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(kwv[r] & 0xffffu));
      s4[r] = ks1 * dsum;
    }
    if (__builtin_expect(t0 + 16 > c1, 0)) {  // the chunk's last, partial step (wave-uniform)
      asm volatile("");                        // kept as a branch: no selects on full steps
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (t0 + 4 * grp + r >= c1) s4[r] = -INFINITY;
    }
    float mloc = fmaxf(fmaxf(s4[0], s4[1]), fmaxf(s4[2], s4[3]));
    mloc = rows_max(mloc);
    float corr = 1.f;
    if (__any(n < GQ && mloc > m_run + kLazyMax)) {  // live head slots decide
      const float m_new = fmaxf(m_run, mloc);
      corr = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
    }
    float lsum = 0.f, bsum = 0.f, pw[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float vs1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(vwv[r] & 0xffffu));
      const float vs2 = (float)__builtin_bit_cast(_Float16, (uint16_t)(vwv[r] >> 16));
      // masked tokens: exp2(-inf) = 0 and staged value scales of zero, so p1 = p2 = 0
      const float pv = __builtin_amdgcn_exp2f(s4[r] - m_run);
      const float p1 = vs1 * pv;
      const float p2 = vs2 * p1;
      lsum += pv;
      bsum += p1;
      pw[r] = p2;
    }
    l_run = l_run * corr + lsum;
    beta_run = beta_run * corr + bsum;
    float wm = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pw[r] = __builtin_amdgcn_ldexpf(pw[r], -vexp);
      wm = fmaxf(wm, pw[r]);
    }
    if (n >= GQ) wm = 0.f;
    if (__any(corr != 1.f || wm > 16384.f)) {
      float cr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float lo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(corr), r));
        if constexpr (GQ > 4) {
          const float hi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(corr), 4 + r));
          cr[r] = grp == 0 ? lo : hi;
        } else {
          cr[r] = lo;
        }
      }
      if (__any(wm > 16384.f)) {
        float mm = max2(wm, row_ror<8>(wm));
        mm = max2(mm, row_ror<4>(mm));
        mm = max2(mm, row_ror<2>(mm));
        mm = max2(mm, row_ror<1>(mm));
        mm = rows_max(mm);
        const int ke = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_frexp_expf(mm) - 14);
        vexp += ke;
#pragma unroll
        for (int r = 0; r < 4; ++r) cr[r] = __builtin_amdgcn_ldexpf(cr[r], -ke);
#pragma unroll
        for (int r = 0; r < 4; ++r) pw[r] = __builtin_amdgcn_ldexpf(pw[r], -ke);
      }
#pragma unroll
      for (int bl = 0; bl < NB; ++bl)
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[bl][t][r] *= cr[r];
    }
    const half4 PA = __builtin_bit_cast(half4, make_uint2(pack_f16_rne(pw[0], pw[1]) & live_mask,
                                                          pack_f16_rne(pw[2], pw[3]) & live_mask));
    // ---- values: B = channel t of the lane's value sub-vector(s) for tokens 4 grp + j
#pragma unroll
    for (int bl = 0; bl < NB; ++bl) {
      uint32_t Ev[4][NT / 2];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (G == 4) {
          const uint32_t w2 = *reinterpret_cast<const uint16_t*>(stg + 16 * M + 32 * (4 * grp + j) + 2 * n);
          const uint2 ev = *reinterpret_cast<const uint2*>(s_tab + gather_addr<4>(w2, laneoff, bl));
          Ev[j][0] = ev.x;
          Ev[j][NT / 2 - 1] = ev.y;
        } else {
          const uint32_t w1 = stg[16 * M + 16 * (4 * grp + j) + n];
          const uint4 ev = *reinterpret_cast<const uint4*>(s_tab + gather_addr<8>(w1, laneoff, 0));
          Ev[j][0] = ev.x;
          Ev[j][1 % (NT / 2)] = ev.y;
          Ev[j][2 % (NT / 2)] = ev.z;
          Ev[j][3 % (NT / 2)] = ev.w;
        }
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
        const uint2 bv = make_uint2(__builtin_amdgcn_perm(Ev[1][t >> 1], Ev[0][t >> 1], sel),
                                    __builtin_amdgcn_perm(Ev[3][t >> 1], Ev[2][t >> 1], sel));
        acc[bl][t] = __builtin_amdgcn_mfma_f32_16x16x16f16(PA, __builtin_bit_cast(half4, bv), acc[bl][t], 0, 0, 0);
      }
    }
  };
  uint4 rwA, rwB;
  uint32_t swA, swB;
  if (nsteps > 0) {
    load_step(0, rwA, swA);
    anchor(c0 + 16 * wave + n);
  }
  if (nsteps > 1) load_step(1, rwB, swB);
  for (int k = 0; k < nsteps; k += 2) {
    step_body(k, rwA, swA);
    if (k + 1 < nsteps) step_body(k + 1, rwB, swB);
  }

  // ---------------- per-wave state -> LDS -> block merge -> workspace
  l_run = rows_sum(l_run);
  beta_run = rows_sum(beta_run);
  __syncthreads();  // table no longer needed: reuse it for the partials
  float* s_acc = reinterpret_cast<float*>(s_tab);  // [4 waves][GQ heads][128]
  float* s_st = s_acc + 4 * GQ * kD;               // [4][GQ][3]
#pragma unroll
  for (int bl = 0; bl < NB; ++bl)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int slot = 4 * grp + r;
        const int j = (G == 4) ? (2 * n + bl) : n;
        if (slot < GQ)
          s_acc[((size_t)wave * GQ + slot) * kD + G * j + t] = __builtin_amdgcn_ldexpf(acc[bl][t][r], vexp);
      }
  if (grp == 0 && n < GQ) {
    s_st[(wave * GQ + n) * 3 + 0] = m_run;
    s_st[(wave * GQ + n) * 3 + 1] = l_run;
    s_st[(wave * GQ + n) * 3 + 2] = beta_run;
  }
  __syncthreads();
  for (int i = tid; i < GQ * kD; i += 256) {
    const int h = i / kD, c = i % kD;
    float Mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) Mx = fmaxf(Mx, s_st[(w * GQ + h) * 3]);
    float a = 0.f, l = 0.f, be = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = s_st[(w * GQ + h) * 3];
      const float f = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - Mx);
      a += f * s_acc[((size_t)w * GQ + h) * kD + c];
      l += f * s_st[(w * GQ + h) * 3 + 1];
      be += f * s_st[(w * GQ + h) * 3 + 2];
    }
    float* dst = part + (((size_t)b * Hq + (size_t)hk * GQ + h) * nchunk + chunk) * kPartStride;
    dst[4 + c] = a;
    if (c == 0) {
      dst[0] = Mx;
      dst[1] = l;
      dst[2] = be;
      dst[3] = 0.f;
    }
  }
}

void pick_chunks(int B, int Hkv, int S, int& CH, int& nchunk, bool res = false) {
  // about one workgroup per CU (each holds ~140 KB of LDS), chunks a multiple of
  // the kStepSpan tokens of one block step.  With a residual window and few (b, KV
  // head) pairs, one CU per pair is left to the window's workgroup so that it runs
  // beside the chunks; with many pairs the windows' short workgroups run last.
  long bh = (long)B * Hkv;
  long want = (256 + bh - 1) / bh;
  if (res && bh <= 32) want = (256 - bh) / bh;
  long maxc = (S + kStepSpan - 1) / kStepSpan;
  if (want > maxc) want = maxc;
  if (want < 1) want = 1;
  long ch = (S + want - 1) / want;
  ch = (ch + kStepSpan - 1) / kStepSpan * kStepSpan;
  CH = (int)ch;
  nchunk = (int)((S + ch - 1) / ch);
}

template <int G, bool DQ, bool APP = false>
hipError_t launch_g(int GQ, dim3 grid, hipStream_t st, const uint16_t* q, int Hq, int Hkv, int S, int S_cap,
                    int CH, int nchunk, const uint8_t* k_idx, const uint16_t* k_sc, const float* k_o,
                    const uint8_t* v_idx, const uint16_t* v_sc, const uint8_t* k_nib, const uint8_t* v_nib,
                    const nsn_dq_head* k_hd, const nsn_dq_head* v_hd, const uint16_t* c16, float* part,
                    const uint16_t* k_res, const uint16_t* v_res, int R, int R_cap, float* rpart, int BH,
                    uint4 sm, const AppendArgs& ap = AppendArgs{}, const SegArgs& sg = SegArgs{}) {
#define NSN_DECODE_ARGS \
  q, Hq, Hkv, S, S_cap, CH, nchunk, k_idx, k_sc, k_o, v_idx, v_sc, k_nib, v_nib, k_hd, v_hd, c16, part, k_res, v_res, R, \
      R_cap, rpart, BH, sm, ap, sg
  switch (GQ) {
    case 1: k_decode<G, 1, DQ, APP><<<grid, kThreads, 0, st>>>(NSN_DECODE_ARGS); break;
    case 2: k_decode<G, 2, DQ, APP><<<grid, kThreads, 0, st>>>(NSN_DECODE_ARGS); break;
    case 4: k_decode<G, 4, DQ, APP><<<grid, kThreads, 0, st>>>(NSN_DECODE_ARGS); break;
    default: k_decode<G, 8, DQ, APP><<<grid, kThreads, 0, st>>>(NSN_DECODE_ARGS); break;
  }
#undef NSN_DECODE_ARGS
  return hipGetLastError();
}

template <int G>
hipError_t launch_rope_g(int GQ, dim3 grid, hipStream_t st, const uint16_t* q, int Hq, int Hkv, int S, int S_cap,
                         int CH, int nchunk, const uint8_t* k_idx, const uint16_t* k_sc, const float* k_o,
                         const uint8_t* v_idx, const uint16_t* v_sc, const uint16_t* c16x2, const float2* ta,
                         const float2* tb, float* part, uint4 sm) {
#define NSN_ROPE_ARGS q, Hq, Hkv, S, S_cap, CH, nchunk, k_idx, k_sc, k_o, v_idx, v_sc, c16x2, ta, tb, part, sm
  switch (GQ) {
    case 1: k_decode_rope<G, 1><<<grid, 256, 0, st>>>(NSN_ROPE_ARGS); break;
    case 2: k_decode_rope<G, 2><<<grid, 256, 0, st>>>(NSN_ROPE_ARGS); break;
    case 4: k_decode_rope<G, 4><<<grid, 256, 0, st>>>(NSN_ROPE_ARGS); break;
    default: k_decode_rope<G, 8><<<grid, 256, 0, st>>>(NSN_ROPE_ARGS); break;
  }
#undef NSN_ROPE_ARGS
  return hipGetLastError();
}


// Two 4-wave workgroups per CU (each holds ~70 KB of LDS): about 512 workgroups,
// chunks a multiple of the 64 tokens one step of the four waves covers.
void pick_chunks_rope(int B, int Hkv, int S, int& CH, int& nchunk) {
  long bh = (long)B * Hkv;
  long want = (512 + bh - 1) / bh;
  long maxc = (S + 63) / 64;
  if (want > maxc) want = maxc;
  if (want < 1) want = 1;
  long ch = (S + want - 1) / want;
  ch = (ch + 63) / 64 * 64;
  CH = (int)ch;
  nchunk = (int)((S + ch - 1) / ch);
}

}  // namespace

// the coarse table (one row per 256 positions), then the fine one (256 rows)
size_t rope_table_bytes(int S) { return (size_t)((S + 255) / 256 + 256) * 64 * sizeof(float2); }

static size_t rope_part_bytes(int B, int Hq, int Hkv, int S) {
  int CH, nchunk;
  pick_chunks_rope(B, Hkv, S, CH, nchunk);
  return ((size_t)B * Hq * nchunk * kPartStride * sizeof(float) + 255) & ~(size_t)255;
}

size_t decode_rope_ws_bytes(int B, int Hq, int Hkv, int S) {
  return rope_part_bytes(B, Hq, Hkv, S) + rope_table_bytes(S);
}

size_t decode_rope_tables_ws_bytes(int B, int Hq, int Hkv, int S) { return rope_part_bytes(B, Hq, Hkv, S); }

hipError_t launch_rope_tables(double rope_base, int S, void* tables, hipStream_t st) {
  const int na = (S + 255) / 256;
  const int rows = max(na, 256);
  k_rope_tables<<<(rows * 64 + 255) / 256, 256, 0, st>>>(std::log(rope_base), na, static_cast<float2*>(tables));
  return hipGetLastError();
}

// tables: the coarse rows for positions below S_tab (S <= S_tab), then the fine rows
hipError_t launch_decode_rope_tables(const nsn_codebook* cb, const uint16_t* q, int B, int Hq, int Hkv, int S,
                                     int S_cap, const void* tables, int S_tab, const uint8_t* k_idx,
                                     const uint16_t* k_scales, const float* k_o, const uint8_t* v_idx,
                                     const uint16_t* v_scales, const float* v_o, float* out, void* ws,
                                     hipStream_t st) {
  int CH, nchunk;
  pick_chunks_rope(B, Hkv, S, CH, nchunk);
  float* part = static_cast<float*>(ws);
  const float2* ta = static_cast<const float2*>(tables);
  const float2* tb = ta + (size_t)((S_tab + 255) / 256) * 64;
  dim3 grid(nchunk, Hkv, B);
  const int GQ = Hq / Hkv;
  const uint4 sm = make_uint4(cb->sgn[0], cb->sgn[1], cb->sgn[2], cb->sgn[3]);
  hipError_t e = (cb->g == 4) ? launch_rope_g<4>(GQ, grid, st, q, Hq, Hkv, S, S_cap, CH, nchunk, k_idx, k_scales, k_o,
                                                 v_idx, v_scales, cb->d_c16x2, ta, tb, part, sm)
                              : launch_rope_g<8>(GQ, grid, st, q, Hq, Hkv, S, S_cap, CH, nchunk, k_idx, k_scales, k_o,
                                                 v_idx, v_scales, cb->d_c16x2, ta, tb, part, sm);
  if (e != hipSuccess) return e;
  k_combine<false, false><<<B * Hq, 256, 0, st>>>(part, nchunk, Hq, Hkv, v_o, nullptr, nullptr, out, sm);
  return hipGetLastError();
}

// self-contained: the tables for S positions are built in the workspace, after the partials
hipError_t launch_decode_rope(const nsn_codebook* cb, const uint16_t* q, int B, int Hq, int Hkv, int S, int S_cap,
                              double rope_base, const uint8_t* k_idx, const uint16_t* k_scales, const float* k_o,
                              const uint8_t* v_idx, const uint16_t* v_scales, const float* v_o, float* out, void* ws,
                              hipStream_t st) {
  void* tables = static_cast<char*>(ws) + rope_part_bytes(B, Hq, Hkv, S);
  hipError_t e = launch_rope_tables(rope_base, S, tables, st);
  if (e != hipSuccess) return e;
  return launch_decode_rope_tables(cb, q, B, Hq, Hkv, S, S_cap, tables, S, k_idx, k_scales, k_o, v_idx, v_scales, v_o,
                                   out, ws, st);
}

// chunk partials [B][Hq][nchunk], then the residual window's partials [B][Hq]
size_t decode_ws_bytes(int B, int Hq, int Hkv, int S) {
  int CH = 0, nchunk = 0;
  if (S > 0) pick_chunks(B, Hkv, S, CH, nchunk);
  return (size_t)B * Hq * (nchunk + 1) * kPartStride * sizeof(float);
}

hipError_t launch_decode(const nsn_codebook* cb, const uint16_t* q, int B, int Hq, int Hkv, int S, int S_cap,
                         const uint8_t* k_idx, const uint16_t* k_scales, const float* k_o, const uint8_t* v_idx,
                         const uint16_t* v_scales, const float* v_o, const uint16_t* k_res, const uint16_t* v_res,
                         int R, int R_cap, float* out, void* ws, hipStream_t st, const uint8_t* k_nib,
                         const uint8_t* v_nib, const nsn_dq_head* k_hd, const nsn_dq_head* v_hd) {
  const bool dq = k_hd != nullptr;
  const bool res = !dq && R > 0;
  int CH = 0, nchunk = 0;
  if (S > 0) pick_chunks(B, Hkv, S, CH, nchunk, res);  // never more chunks than the workspace holds
  const uint4 sm = make_uint4(cb->sgn[0], cb->sgn[1], cb->sgn[2], cb->sgn[3]);
  float* part = static_cast<float*>(ws);
  float* rpart = part + (size_t)B * Hq * nchunk * kPartStride;
  if ((nchunk > 0 || res) && ws == nullptr) return hipErrorInvalidValue;  // callers check the workspace first
  if (nchunk > 0 || res) {
    const int BH = B * Hkv;
    const dim3 grid((unsigned)((nchunk + (res ? 1 : 0)) * BH));  // chunk workgroups, then the windows'
    const int GQ = Hq / Hkv;
    hipError_t e;
    if (cb->g == 4)
      e = dq ? launch_g<4, true>(GQ, grid, st, q, Hq, Hkv, S, S_cap, CH, nchunk, k_idx, k_scales, k_o, v_idx,
                                 v_scales, k_nib, v_nib, k_hd, v_hd, cb->d_c16x2, part, nullptr, nullptr, 0, 0,
                                 nullptr, BH, sm)
             : launch_g<4, false>(GQ, grid, st, q, Hq, Hkv, S, S_cap, CH, nchunk, k_idx, k_scales, k_o, v_idx,
                                  v_scales, nullptr, nullptr, nullptr, nullptr, cb->d_c16x2, part, k_res, v_res, R,
                                  R_cap, rpart, BH, sm);
    else
      e = dq ? launch_g<8, true>(GQ, grid, st, q, Hq, Hkv, S, S_cap, CH, nchunk, k_idx, k_scales, k_o, v_idx,
                                 v_scales, k_nib, v_nib, k_hd, v_hd, cb->d_c16x2, part, nullptr, nullptr, 0, 0,
                                 nullptr, BH, sm)
             : launch_g<8, false>(GQ, grid, st, q, Hq, Hkv, S, S_cap, CH, nchunk, k_idx, k_scales, k_o, v_idx,
                                  v_scales, nullptr, nullptr, nullptr, nullptr, cb->d_c16x2, part, k_res, v_res, R,
                                  R_cap, rpart, BH, sm);
    if (e != hipSuccess) return e;
  }
  if (dq)
    k_combine<false, true><<<B * Hq, 256, 0, st>>>(part, nchunk, Hq, Hkv, nullptr, v_hd, nullptr, out, sm);
  else if (res)
    k_combine<true, false><<<B * Hq, 256, 0, st>>>(part, nchunk, Hq, Hkv, v_o, nullptr, rpart, out, sm);
  else
    k_combine<false, false><<<B * Hq, 256, 0, st>>>(part, nchunk, Hq, Hkv, v_o, nullptr, nullptr, out, sm);
  return hipGetLastError();
}

// Chunk partials [B][Hq][nchunk0 + nblk], then the residual window's [B][Hq].
size_t decode_blocks_ws_bytes(int B, int Hq, int Hkv, int S0, int nblk) {
  int CH = 0, nchunk0 = 0;
  if (S0 > 0) pick_chunks(B, Hkv, S0, CH, nchunk0, true);
  int CH1 = 0, nchunk1 = 0;  // (the chunking without a window never has more chunks)
  if (S0 > 0) pick_chunks(B, Hkv, S0, CH1, nchunk1, false);
  return (size_t)B * Hq * (std::max(nchunk0, nchunk1) + nblk + 1) * kPartStride * sizeof(float);
}

// Decode over a prefix with one o per (batch, KV head) and nblk flushed blocks of Rb
// tokens with their own o, plus an optional fp16 window: one chunk workgroup per block
// after the prefix chunks, the window's workgroups last, then k_combine<SEG>.
hipError_t launch_decode_blocks(const nsn_codebook* cb, const uint16_t* q, int B, int Hq, int Hkv, int S0, int nblk,
                                int Rb, int S_cap, const uint8_t* k_idx, const uint16_t* k_scales, const float* k_o,
                                const float* k_ob, const uint8_t* v_idx, const uint16_t* v_scales, const float* v_o,
                                const float* v_ob, const uint16_t* k_res, const uint16_t* v_res, int R, int R_cap,
                                float* out, void* ws, hipStream_t st) {
  const bool res = R > 0;
  int CH = kStepSpan, nchunk0 = 0;
  if (S0 > 0) pick_chunks(B, Hkv, S0, CH, nchunk0, res);
  const int nchunk = nchunk0 + nblk;
  if (ws == nullptr) return hipErrorInvalidValue;  // callers check the workspace first
  const uint4 sm = make_uint4(cb->sgn[0], cb->sgn[1], cb->sgn[2], cb->sgn[3]);
  float* part = static_cast<float*>(ws);
  float* rpart = part + (size_t)B * Hq * nchunk * kPartStride;
  const int BH = B * Hkv;
  if (nchunk > 0 || res) {
    SegArgs sg;
    sg.k_ob = k_ob;
    sg.S0 = S0;
    sg.Rb = nblk > 0 ? Rb : 0;
    sg.nchunk0 = nchunk0;
    const int S = S0 + nblk * Rb;
    const dim3 grid((unsigned)((nchunk + (res ? 1 : 0)) * BH));
    const int GQ = Hq / Hkv;
    const hipError_t e =
        (cb->g == 4) ? launch_g<4, false>(GQ, grid, st, q, Hq, Hkv, S, S_cap, CH, nchunk, k_idx, k_scales, k_o, v_idx,
                                          v_scales, nullptr, nullptr, nullptr, nullptr, cb->d_c16x2, part, k_res, v_res,
                                          R, R_cap, rpart, BH, sm, AppendArgs{}, sg)
                     : launch_g<8, false>(GQ, grid, st, q, Hq, Hkv, S, S_cap, CH, nchunk, k_idx, k_scales, k_o, v_idx,
                                          v_scales, nullptr, nullptr, nullptr, nullptr, cb->d_c16x2, part, k_res, v_res,
                                          R, R_cap, rpart, BH, sm, AppendArgs{}, sg);
    if (e != hipSuccess) return e;
  }
  if (res)
    k_combine<true, false, true><<<B * Hq, 256, 0, st>>>(part, nchunk, Hq, Hkv, v_o, nullptr, rpart, out, sm, v_ob,
                                                         nchunk0, BH);
  else
    k_combine<false, false, true><<<B * Hq, 256, 0, st>>>(part, nchunk, Hq, Hkv, v_o, nullptr, nullptr, out, sm,
                                                          v_ob, nchunk0, BH);
  return hipGetLastError();
}

// The decode step in two launches: k_decode over the S cached tokens, whose last
// chunk's workgroups also encode and append the new K and V tokens at slot S and
// join them to the softmax, then k_combine.  An empty cache (S = 0) still runs one
// (empty) chunk per (batch, KV head) for the new token.
hipError_t launch_decode_step(const nsn_codebook* cb, const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                              int B, int Hq, int Hkv, int S, int S_cap, uint8_t* k_idx, uint16_t* k_scales,
                              const float* k_o, uint8_t* v_idx, uint16_t* v_scales, const float* v_o, float* out,
                              void* ws, hipStream_t st) {
  int CH = kStepSpan, nchunk = 1;
  if (S > 0) pick_chunks(B, Hkv, S, CH, nchunk);
  if (ws == nullptr) return hipErrorInvalidValue;  // callers check the workspace first
  const uint4 sm = make_uint4(cb->sgn[0], cb->sgn[1], cb->sgn[2], cb->sgn[3]);
  float* part = static_cast<float*>(ws);
  const int BH = B * Hkv;
  const int GQ = Hq / Hkv;
  AppendArgs ap;
  ap.k_new = reinterpret_cast<const _Float16*>(k_new);
  ap.v_new = reinterpret_cast<const _Float16*>(v_new);
  ap.encA = cb->d_encA;
  ap.c32 = cb->d_c32;
  ap.k_o = k_o;
  ap.v_o = v_o;
  ap.k_idx = k_idx;
  ap.k_sc = k_scales;
  ap.v_idx = v_idx;
  ap.v_sc = v_scales;
  ap.pos = S;
  const dim3 grid((unsigned)(nchunk * BH));
  hipError_t e = (cb->g == 4)
                     ? launch_g<4, false, true>(GQ, grid, st, q, Hq, Hkv, S, S_cap, CH, nchunk, k_idx, k_scales, k_o,
                                                v_idx, v_scales, nullptr, nullptr, nullptr, nullptr, cb->d_c16x2, part,
                                                nullptr, nullptr, 0, 0, nullptr, BH, sm, ap)
                     : launch_g<8, false, true>(GQ, grid, st, q, Hq, Hkv, S, S_cap, CH, nchunk, k_idx, k_scales, k_o,
                                                v_idx, v_scales, nullptr, nullptr, nullptr, nullptr, cb->d_c16x2, part,
                                                nullptr, nullptr, 0, 0, nullptr, BH, sm, ap);
  if (e != hipSuccess) return e;
  k_combine<false, false><<<B * Hq, 256, 0, st>>>(part, nchunk, Hq, Hkv, v_o, nullptr, nullptr, out, sm);
  return hipGetLastError();
}

}  // namespace nsn
