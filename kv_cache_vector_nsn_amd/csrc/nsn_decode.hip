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
// applies H once per query head at the end.
//
// Mapping (one workgroup = one (batch, KV head, token chunk); 4 waves, each
// taking 32-token steps):
//   * the codebook lives in LDS replicated so that each lane reads its own bank
//     group (32 copies of the 8-byte entry for g = 4, 16 copies of the 16-byte
//     entry for g = 8, one 256-byte row per entry); the gather address
//     entry * 256 + lane_offset is a single v_perm of the index byte;
//   * scores: 16x16x32 fp16 MFMA, A = dequantized K sub-vectors (rows = 16
//     tokens, K = 32 channels), B = H q split into fp16 hi/lo parts occupying
//     head slots 0..GQ-1 and GQ..2GQ-1 -- both parts are exact, so the score
//     carries fp32 accuracy; the two slots are summed after the MFMA;
//   * values: 16x16x32 fp16 MFMA, A = softmax weights (head slots hi/lo, K = 32
//     tokens), B = centroid channel t of 8 tokens x 16 sub-vectors (one MFMA per
//     t, repacked from the gathered entries with v_perm);
//   * split-KV: each workgroup writes (max, sum, beta, acc[128]) per query head;
//     k_combine merges the chunks in a fixed order and applies H.
#include "nsn_device.h"

namespace nsn {
namespace {

constexpr int kPartStride = 132;  // m, l, beta, pad, acc[128]
constexpr int kWaves = 4;         // waves per workgroup: two 68 KB workgroups per CU -> 2 waves per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kStepSpan = 32 * kWaves;  // tokens covered by one step of every wave

template <int G>
__device__ __forceinline__ uint32_t gather_addr(uint32_t word, uint32_t laneoff, int byte) {
  // bytes: [laneoff, index, 0, 0] -> index * 256 + laneoff
  const uint32_t sel = 0x0C0C0000u | ((uint32_t)(4 + byte) << 8);
  return __builtin_amdgcn_perm(word, laneoff, sel);
}

// max / sum of the values held by lanes l, l ^ 16, l ^ 32, l ^ 48 (the four
// 16-lane rows): v_permlane16/32_swap exchange rows without going through LDS
__device__ __forceinline__ float rows_max(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
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
// value of lane (i + S) mod 16 of the row
template <int S>
__device__ __forceinline__ float row_ror(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x120 + S, 0xf, 0xf, false));
}

// lane i of each 16-lane row reads lane i + k (DPP row_shl:k; 0 past the row end)
template <int K>
__device__ __forceinline__ float row_shl(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x100 + K, 0xf, 0xf, true));
}

template <int G, int GQ, bool SCV>
__global__ __launch_bounds__(kThreads, 2) void k_decode(const uint16_t* __restrict__ q, int Hq, int Hkv, int S,
                                                   int S_cap, int CH, int nchunk,
                                                   const uint8_t* __restrict__ k_idx,
                                                   const uint16_t* __restrict__ k_sc,
                                                   const float* __restrict__ k_o,
                                                   const uint8_t* __restrict__ v_idx,
                                                   const uint16_t* __restrict__ v_sc,
                                                   const uint16_t* __restrict__ c16,
                                                   float* __restrict__ part) {
  constexpr int M = kD / G;            // indices per token
  constexpr int NB = (G == 4) ? 2 : 1; // 16-column value blocks
  constexpr int NT = G;                // channel offsets per sub-vector
  __shared__ __attribute__((aligned(256))) unsigned char s_tab[kK * 256];  // replicated codebook
  __shared__ float s_q[8][kD];
  __shared__ float s_qo[8];

  const int chunk = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bh = b * Hkv + hk;

  // ---- codebook -> LDS: entry k replicated across its 256-byte row.  Lane l
  // writes 16-byte column (i + l) % 16 at step i so the lanes of one write
  // cover distinct banks.
  if (tid < kK) {
    const int k = tid;  // threads 0..255 write one row each
    uint4 e;
    if (G == 4) {
      const uint2 v = *reinterpret_cast<const uint2*>(c16 + (size_t)k * 4);
      e = make_uint4(v.x, v.y, v.x, v.y);
    } else {
      e = *reinterpret_cast<const uint4*>(c16 + (size_t)k * 8);
    }
    uint4* row = reinterpret_cast<uint4*>(s_tab + (size_t)k * 256);
#pragma unroll
    for (int i = 0; i < 16; ++i) row[(i + lane) & 15] = e;
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
#pragma unroll
      for (int c = 0; c < 4; ++c) qo += v[c] * k_o[(size_t)bh * kD + 4 * p + c];
      qo = half_wave_sum(qo);
      fwht128_pair(v, p);
      const float rs = 0.08838834764831845f * cscale;
#pragma unroll
      for (int c = 0; c < 4; ++c) s_q[h][4 * p + c] = v[c] * rs;
      if (p == 0) s_qo[h] = qo * cscale;
    }
  }
  __syncthreads();

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
  // lanes whose softmax values are real; the rest feed zero rows of the value MFMA
  const uint32_t live_mask = n < GQ ? 0xffffffffu : 0u;

  const uint32_t laneoff = (G == 4) ? 8u * (lane & 31) : 16u * (lane & 15);
  const unsigned char* tab = s_tab;

  const int c0 = chunk * CH, c1 = min(S, c0 + CH);
  const size_t row0 = (size_t)bh * S_cap;
  // per-lane byte offsets inside one 32-token step (constant across steps)
  const uint32_t koff0 = (uint32_t)(n * M + (G == 4 ? 8 : 4) * grp);     // K index words, half a adds 16 M
  const uint32_t soff0 = (uint32_t)(4 * grp * 4);                          // scales of tokens 4 grp .. +3
  const uint32_t voff0 = (uint32_t)(4 * grp * M + (G == 4 ? 2 * n : n));   // V index of token 4 grp

  floatx4 acc[NB][NT];
#pragma unroll
  for (int bl = 0; bl < NB; ++bl)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[bl][t] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f, beta_run = 0.f;

  // Global words of one 32-token step, loaded one step ahead of their use.
  // With GQ >= 4 the softmax runs on a redistributed layout: lane n = h + GQ k of
  // a row holds RV = GQ/2 consecutive tokens of head h (see compute_step), so it
  // loads only those tokens' scales.
  constexpr bool RED = GQ >= 4;
  constexpr int RV = RED ? GQ / 2 : 8;
  const int kk = n / GQ;                                   // k of this lane (RED layout)
  const int rtok0 = RED ? (16 * ((kk * RV) / 4) + 4 * grp + (kk * RV) % 4) : 0;  // first token of the lane
  struct StepIn {
    uint32_t kx[2][G == 4 ? 2 : 1];
    uint32_t kw[RV], vw[RV], vx[8];
  };
  // full: every token of the step is below c1, so no guard is needed.  The last
  // step of a chunk may be partial: its out-of-range tokens read an in-range row
  // (token c1-1, or any row for a whole 4-token scale group at or past S_cap --
  // with S_cap % 4 == 0 a group never straddles S_cap) and are masked out of the
  // softmax.
  // K index words of the score rows (tokens base + 16a + n)
  auto load_k = [&]<bool full>(StepIn& in, int base) {
    const int bu = __builtin_amdgcn_readfirstlane(base);
    const int rem = c1 - bu;  // >= 1 valid tokens in this step
    const uint8_t* kb = k_idx + (row0 + bu) * M;
    auto tok = [&](int t) { return full ? t : min(t, rem - 1); };
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const uint32_t ko = (uint32_t)(tok(16 * a + n) * M + (G == 4 ? 8 : 4) * grp);
      if (G == 4) {
        const uint2 v = *reinterpret_cast<const uint2*>(kb + ko);
        in.kx[a][0] = v.x;
        in.kx[a][G == 4 ? 1 : 0] = v.y;
      } else {
        in.kx[a][0] = *reinterpret_cast<const uint32_t*>(kb + ko);
      }
    }
  };
  // K/V scale words of the softmax layout and V index words of the value layout
  auto load_rest = [&]<bool full>(StepIn& in, int base) {
    const int bu = __builtin_amdgcn_readfirstlane(base);
    const int rem = c1 - bu;
    const unsigned char* ksb = reinterpret_cast<const unsigned char*>(k_sc + (row0 + bu) * 2);
    const unsigned char* vsb = reinterpret_cast<const unsigned char*>(v_sc + (row0 + bu) * 2);
    const uint8_t* vb = v_idx + (row0 + bu) * M;
    auto tok = [&](int t) { return full ? t : min(t, rem - 1); };
    if (!RED) {
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        if (SCV) {  // 4 consecutive tokens: one 16-byte load each for K and V
          int g4 = 16 * a + 4 * grp;
          if (!full && bu + g4 >= S_cap) g4 = S_cap - 4 - bu;
          const uint4 k4 = *reinterpret_cast<const uint4*>(ksb + 4u * (uint32_t)g4);
          const uint4 v4 = *reinterpret_cast<const uint4*>(vsb + 4u * (uint32_t)g4);
          in.kw[(4 * a + 0) % RV] = k4.x; in.kw[(4 * a + 1) % RV] = k4.y;
          in.kw[(4 * a + 2) % RV] = k4.z; in.kw[(4 * a + 3) % RV] = k4.w;
          in.vw[(4 * a + 0) % RV] = v4.x; in.vw[(4 * a + 1) % RV] = v4.y;
          in.vw[(4 * a + 2) % RV] = v4.z; in.vw[(4 * a + 3) % RV] = v4.w;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t so = (uint32_t)tok(16 * a + 4 * grp + r) * 4u;
            in.kw[(4 * a + r) % RV] = *reinterpret_cast<const uint32_t*>(ksb + so);
            in.vw[(4 * a + r) % RV] = *reinterpret_cast<const uint32_t*>(vsb + so);
          }
        }
      }
    } else {  // RV consecutive tokens from rtok0 (never straddle S_cap when S_cap % 4 == 0)
      if (SCV) {
        int t0 = rtok0;
        if (!full && bu + t0 >= S_cap) t0 = S_cap - RV - bu;
        if (RV == 2) {
          const uint2 k2 = *reinterpret_cast<const uint2*>(ksb + 4u * (uint32_t)t0);
          const uint2 v2 = *reinterpret_cast<const uint2*>(vsb + 4u * (uint32_t)t0);
          in.kw[0] = k2.x; in.kw[1 % RV] = k2.y;
          in.vw[0] = v2.x; in.vw[1 % RV] = v2.y;
        } else {
          const uint4 k4 = *reinterpret_cast<const uint4*>(ksb + 4u * (uint32_t)t0);
          const uint4 v4 = *reinterpret_cast<const uint4*>(vsb + 4u * (uint32_t)t0);
          in.kw[0] = k4.x; in.kw[1 % RV] = k4.y; in.kw[2 % RV] = k4.z; in.kw[3 % RV] = k4.w;
          in.vw[0] = v4.x; in.vw[1 % RV] = v4.y; in.vw[2 % RV] = v4.z; in.vw[3 % RV] = v4.w;
        }
      } else {
#pragma unroll
        for (int q = 0; q < RV; ++q) {
          const uint32_t so = (uint32_t)tok(rtok0 + q) * 4u;
          in.kw[q] = *reinterpret_cast<const uint32_t*>(ksb + so);
          in.vw[q] = *reinterpret_cast<const uint32_t*>(vsb + so);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t vo = (uint32_t)(tok(16 * (e >> 2) + 4 * grp + (e & 3)) * M + (G == 4 ? 2 * n : n));
      if (G == 4)
        in.vx[e] = *reinterpret_cast<const uint16_t*>(vb + vo);
      else
        in.vx[e] = vb[vo];
    }
  };
  auto load_k_any = [&](StepIn& in, int bs) {
    if (bs + 32 <= c1) load_k.template operator()<true>(in, bs);
    else load_k.template operator()<false>(in, bs);
  };
  auto load_rest_any = [&](StepIn& in, int bs) {
    if (bs + 32 <= c1) load_rest.template operator()<true>(in, bs);
    else load_rest.template operator()<false>(in, bs);
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
    half8 PA;
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
        mloc = fmaxf(mloc, row_ror<4>(mloc));
        mloc = fmaxf(mloc, row_ror<8>(mloc));
      } else {
        mloc = fmaxf(mloc, row_ror<8>(mloc));
      }
      mloc = rows_max(mloc);
      const float m_new = fmaxf(m_run, mloc);
      corr = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      float lsum = 0.f, bsum = 0.f;
      float pw[RV];
#pragma unroll
      for (int q = 0; q < RV; ++q) {
        const float vs1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(in.vw[q] & 0xffffu));
        const float vs2 = (float)__builtin_bit_cast(_Float16, (uint16_t)(in.vw[q] >> 16));
        const float pv = __builtin_amdgcn_exp2f(s8[q] - m_new);  // masked tokens: exp2(-inf) = 0
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
      // back to the value-MFMA A layout: row h holds tokens f = 0..7 (half e = f).
      // Lane h + GQ k packs its RV values (f = k RV ..) into RV / 2 dwords; dword
      // j = f / 2 of row h comes from lane h + GQ (2 j / RV).  Dead rows stay 0.
      uint32_t pk[RV / 2];
#pragma unroll
      for (int j = 0; j < RV / 2; ++j)
        pk[j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(pw[2 * j], pw[2 * j + 1]));
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
      const float m_new = fmaxf(m_run, mloc);
      corr = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      float lsum = 0.f, bsum = 0.f;
      float pw[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float vs1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(in.vw[i % RV] & 0xffffu));
        const float vs2 = (float)__builtin_bit_cast(_Float16, (uint16_t)(in.vw[i % RV] >> 16));
        const float pv = __builtin_amdgcn_exp2f(s8[i] - m_new);  // masked tokens: exp2(-inf) = 0
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
      uint4 pa;
      pa.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(pw[0], pw[1]));
      pa.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(pw[2], pw[3]));
      pa.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(pw[4], pw[5]));
      pa.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(pw[6], pw[7]));
      pa.x &= live_mask; pa.y &= live_mask; pa.z &= live_mask; pa.w &= live_mask;
      PA = __builtin_bit_cast(half8, pa);
    }
    // rescale accumulators (rows 4 grp + r are head slots) unless no head's max moved
    if (__any(corr != 1.f)) {
      float cr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        cr[r] = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * (4 * grp + r), __float_as_int(corr)));
#pragma unroll
      for (int bl = 0; bl < NB; ++bl)
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[bl][t][r] *= cr[r];
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

  // two step buffers, each filled one step before it is consumed
  StepIn bufA, bufB;
  auto load = [&](StepIn& in, int bs) {
    load_k_any(in, bs);
    load_rest_any(in, bs);
  };
  auto compute = [&](const StepIn& in, int bs) {
    if (bs + 32 <= c1) compute_step.template operator()<true>(in, bs);
    else compute_step.template operator()<false>(in, bs);
  };
  int base = c0 + 32 * wave;
  if (base < c1) load(bufA, base);
  while (base < c1) {
    if (base + kStepSpan < c1) load(bufB, base + kStepSpan);
    compute(bufA, base);
    base += kStepSpan;
    if (base >= c1) break;
    if (base + kStepSpan < c1) load(bufA, base + kStepSpan);
    compute(bufB, base);
    base += kStepSpan;
  }

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
  float* s_acc = reinterpret_cast<float*>(s_tab);             // [kWaves][GQ heads][128]
  float* s_st = s_acc + kWaves * GQ * kD;                      // [kWaves][GQ][3]
#pragma unroll
  for (int bl = 0; bl < NB; ++bl)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int slot = 4 * grp + r;
        const int j = (G == 4) ? (2 * n + bl) : n;
        if (slot < GQ) s_acc[((size_t)wave * GQ + slot) * kD + G * j + t] = acc[bl][t][r];
      }
  if (grp == 0 && n < GQ) {
    s_st[(wave * GQ + n) * 3 + 0] = m_run;
    s_st[(wave * GQ + n) * 3 + 1] = l_run;
    s_st[(wave * GQ + n) * 3 + 2] = beta_run;
  }
  __syncthreads();
  for (int i = tid; i < GQ * kD; i += kThreads) {
    const int h = i / kD, c = i % kD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_st[(w * GQ + h) * 3]);
    float a = 0.f, l = 0.f, be = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = s_st[(w * GQ + h) * 3];
      const float f = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
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

// Merge the chunk partials of one (batch, query head) and leave the rotated domain.
// 8 groups of 32 threads (4 channels each) merge every 8th chunk online, then the
// groups are merged in a fixed order and H is applied to the 128-vector.
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ part, int nchunk, int Hq, int Hkv,
                                                 const float* __restrict__ v_o, float* __restrict__ out) {
  __shared__ float s_st[8][3];
  __shared__ float4 s_a[8][32];
  __shared__ float s[kD];
  const int bq = blockIdx.x, tid = threadIdx.x, gi = tid >> 5, c4 = tid & 31;
  const int b = bq / Hq, hq = bq % Hq;
  const int hk = hq / (Hq / Hkv);
  const float* pp = part + (size_t)bq * nchunk * kPartStride;
  float M = -INFINITY, l = 0.f, be = 0.f;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int i = gi; i < nchunk; i += 8) {
    const float* q = pp + (size_t)i * kPartStride;
    const float mi = q[0];
    if (mi == -INFINITY) continue;
    const float Mn = fmaxf(M, mi);
    const float fo = exp2f(M - Mn), fn = exp2f(mi - Mn);
    const float4 v = reinterpret_cast<const float4*>(q + 4)[c4];
    l = l * fo + q[1] * fn;
    be = be * fo + q[2] * fn;
    a.x = a.x * fo + v.x * fn; a.y = a.y * fo + v.y * fn; a.z = a.z * fo + v.z * fn; a.w = a.w * fo + v.w * fn;
    M = Mn;
  }
  s_a[gi][c4] = a;
  if (c4 == 0) { s_st[gi][0] = M; s_st[gi][1] = l; s_st[gi][2] = be; }
  __syncthreads();
  float MM = -INFINITY;
#pragma unroll
  for (int g = 0; g < 8; ++g) MM = fmaxf(MM, s_st[g][0]);
  if (tid < 32) {
    float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const float f = s_st[g][0] == -INFINITY ? 0.f : exp2f(s_st[g][0] - MM);
      const float4 v = s_a[g][tid];
      t.x += v.x * f; t.y += v.y * f; t.z += v.z * f; t.w += v.w * f;
    }
    s[4 * tid + 0] = t.x; s[4 * tid + 1] = t.y; s[4 * tid + 2] = t.z; s[4 * tid + 3] = t.w;
  }
  float L = 0.f, BE = 0.f;
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    const float f = s_st[g][0] == -INFINITY ? 0.f : exp2f(s_st[g][0] - MM);
    L += s_st[g][1] * f;
    BE += s_st[g][2] * f;
  }
  __syncthreads();
  const int c = tid;
#pragma unroll
  for (int hsz = 1; hsz < kD; hsz <<= 1) {
    float v = 0.f;
    if (c < kD) {
      const int pr = c ^ hsz;
      v = (c & hsz) ? (s[pr] - s[c]) : (s[c] + s[pr]);
    }
    __syncthreads();
    if (c < kD) s[c] = v;
    __syncthreads();
  }
  if (c < kD) {
    const float rs = 0.08838834764831845f;
    out[(size_t)bq * kD + c] = (s[c] * rs + BE * v_o[((size_t)b * Hkv + hk) * kD + c]) / L;
  }
}

void pick_chunks(int B, int Hkv, int S, int& CH, int& nchunk) {
  // about 512 workgroups (two are resident per CU with 68 KB of LDS each), chunks a
  // multiple of kStepSpan tokens (kWaves waves x 32-token steps)
  long bh = (long)B * Hkv;
  long want = (512 + bh - 1) / bh;
  long maxc = (S + kStepSpan - 1) / kStepSpan;
  if (want > maxc) want = maxc;
  if (want < 1) want = 1;
  long ch = (S + want - 1) / want;
  ch = (ch + kStepSpan - 1) / kStepSpan * kStepSpan;
  CH = (int)ch;
  nchunk = (int)((S + ch - 1) / ch);
}

template <int G, bool SCV>
hipError_t launch_gs(int GQ, dim3 grid, hipStream_t st, const uint16_t* q, int Hq, int Hkv, int S, int S_cap,
                     int CH, int nchunk, const uint8_t* k_idx, const uint16_t* k_sc, const float* k_o,
                     const uint8_t* v_idx, const uint16_t* v_sc, const uint16_t* c16, float* part) {
  switch (GQ) {
    case 1: k_decode<G, 1, SCV><<<grid, kThreads, 0, st>>>(q, Hq, Hkv, S, S_cap, CH, nchunk, k_idx, k_sc, k_o, v_idx, v_sc, c16, part); break;
    case 2: k_decode<G, 2, SCV><<<grid, kThreads, 0, st>>>(q, Hq, Hkv, S, S_cap, CH, nchunk, k_idx, k_sc, k_o, v_idx, v_sc, c16, part); break;
    case 4: k_decode<G, 4, SCV><<<grid, kThreads, 0, st>>>(q, Hq, Hkv, S, S_cap, CH, nchunk, k_idx, k_sc, k_o, v_idx, v_sc, c16, part); break;
    default: k_decode<G, 8, SCV><<<grid, kThreads, 0, st>>>(q, Hq, Hkv, S, S_cap, CH, nchunk, k_idx, k_sc, k_o, v_idx, v_sc, c16, part); break;
  }
  return hipGetLastError();
}

template <int G>
hipError_t launch_g(int GQ, dim3 grid, hipStream_t st, const uint16_t* q, int Hq, int Hkv, int S, int S_cap,
                    int CH, int nchunk, const uint8_t* k_idx, const uint16_t* k_sc, const float* k_o,
                    const uint8_t* v_idx, const uint16_t* v_sc, const uint16_t* c16, float* part) {
  // scale rows are 4 bytes per token: 16-byte loads of 4 tokens need S_cap % 4 == 0
  if (S_cap % 4 == 0)
    return launch_gs<G, true>(GQ, grid, st, q, Hq, Hkv, S, S_cap, CH, nchunk, k_idx, k_sc, k_o, v_idx, v_sc, c16, part);
  return launch_gs<G, false>(GQ, grid, st, q, Hq, Hkv, S, S_cap, CH, nchunk, k_idx, k_sc, k_o, v_idx, v_sc, c16, part);
}

}  // namespace

size_t decode_ws_bytes(int B, int Hq, int Hkv, int S) {
  int CH, nchunk;
  pick_chunks(B, Hkv, S, CH, nchunk);
  return (size_t)B * Hq * nchunk * kPartStride * sizeof(float);
}

hipError_t launch_decode(const nsn_codebook* cb, const uint16_t* q, int B, int Hq, int Hkv, int S, int S_cap,
                         const uint8_t* k_idx, const uint16_t* k_scales, const float* k_o, const uint8_t* v_idx,
                         const uint16_t* v_scales, const float* v_o, float* out, void* ws, hipStream_t st) {
  int CH, nchunk;
  pick_chunks(B, Hkv, S, CH, nchunk);
  float* part = static_cast<float*>(ws);
  dim3 grid(nchunk, Hkv, B);
  const int GQ = Hq / Hkv;
  hipError_t e = (cb->g == 4)
                     ? launch_g<4>(GQ, grid, st, q, Hq, Hkv, S, S_cap, CH, nchunk, k_idx, k_scales, k_o, v_idx, v_scales, cb->d_c16, part)
                     : launch_g<8>(GQ, grid, st, q, Hq, Hkv, S, S_cap, CH, nchunk, k_idx, k_scales, k_o, v_idx, v_scales, cb->d_c16, part);
  if (e != hipSuccess) return e;
  k_combine<<<B * Hq, 256, 0, st>>>(part, nchunk, Hq, Hkv, v_o, out);
  return hipGetLastError();
}

}  // namespace nsn
