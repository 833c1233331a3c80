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

template <int G>
__device__ __forceinline__ uint32_t gather_addr(uint32_t word, uint32_t laneoff, int byte) {
  // bytes: [laneoff, index, 0, 0] -> index * 256 + laneoff
  const uint32_t sel = 0x0C0C0000u | ((uint32_t)(4 + byte) << 8);
  return __builtin_amdgcn_perm(word, laneoff, sel);
}

template <int G, int GQ>
__global__ __launch_bounds__(256) void k_decode(const uint16_t* __restrict__ q, int Hq, int Hkv, int S,
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
  __shared__ __attribute__((aligned(16))) unsigned char s_tab[kK * 256];  // replicated codebook
  __shared__ float s_q[8][kD];
  __shared__ float s_qo[8];

  const int chunk = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bh = b * Hkv + hk;

  // ---- codebook -> LDS, entry k replicated across its 256-byte row
  {
    const int k = tid;  // 256 threads, one row each
    uint4 e;
    if (G == 4) {
      const uint2 v = *reinterpret_cast<const uint2*>(c16 + (size_t)k * 4);
      e = make_uint4(v.x, v.y, v.x, v.y);
    } else {
      e = *reinterpret_cast<const uint4*>(c16 + (size_t)k * 8);
    }
    uint4* row = reinterpret_cast<uint4*>(s_tab + (size_t)k * 256);
#pragma unroll
    for (int i = 0; i < 16; ++i) row[i] = e;
  }
  // ---- q~ = H q / sqrt(d) and <q, o_K> for the GQ query heads (pair layout)
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
      const float rs = 0.08838834764831845f;  // 1/sqrt(128)
#pragma unroll
      for (int c = 0; c < 4; ++c) s_q[h][4 * p + c] = v[c] * rs;
      if (p == 0) s_qo[h] = qo;
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
  const int hh = (n < 2 * GQ) ? (n % GQ) : 0;  // head this lane's softmax column belongs to
  const float qo = s_qo[hh];
  const float cscale = 1.4426950408889634f * 0.08838834764831845f;  // log2(e) / sqrt(d)

  const uint32_t laneoff = (G == 4) ? 8u * (lane & 31) : 16u * (lane & 15);
  const unsigned char* tab = s_tab;

  const int c0 = chunk * CH, c1 = min(S, c0 + CH);
  const size_t row0 = (size_t)bh * S_cap;

  floatx4 acc[NB][NT];
#pragma unroll
  for (int bl = 0; bl < NB; ++bl)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[bl][t] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f, beta_run = 0.f;

  for (int base = c0 + 32 * wave; base < c1; base += 128) {
    // ---------------- scores: two 16-token halves
    floatx4 sc[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int tk = base + 16 * a + n;
      floatx4 d = {0.f, 0.f, 0.f, 0.f};
      if (G == 4) {
        uint2 kx = make_uint2(0u, 0u);
        if (tk < c1) kx = *reinterpret_cast<const uint2*>(k_idx + (row0 + tk) * M + 8 * grp);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint32_t wd = (s < 2) ? kx.x : kx.y;
          const uint2 e0 = *reinterpret_cast<const uint2*>(tab + gather_addr<G>(wd, laneoff, (2 * s) & 3));
          const uint2 e1 = *reinterpret_cast<const uint2*>(tab + gather_addr<G>(wd, laneoff, (2 * s + 1) & 3));
          const uint4 av = make_uint4(e0.x, e0.y, e1.x, e1.y);
          d = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, av), QB[s], d, 0, 0, 0);
        }
      } else {
        uint32_t kx = 0u;
        if (tk < c1) kx = *reinterpret_cast<const uint32_t*>(k_idx + (row0 + tk) * M + 4 * grp);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint4 av = *reinterpret_cast<const uint4*>(tab + gather_addr<G>(kx, laneoff, s));
          d = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, av), QB[s], d, 0, 0, 0);
        }
      }
      sc[a] = d;
    }
    // result lane (slot n, group grp) holds tokens base + 16a + 4 grp + r; add the hi/lo slots
    float ks1[8], ks2[8], vs1[8], vs2[8];
    bool valid[8];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int t4 = base + 16 * a + 4 * grp;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tt = t4 + r;
        valid[4 * a + r] = tt < c1;
        uint32_t kw = 0u, vw = 0u;
        if (tt < c1) {
          kw = *reinterpret_cast<const uint32_t*>(k_sc + (row0 + tt) * 2);
          vw = *reinterpret_cast<const uint32_t*>(v_sc + (row0 + tt) * 2);
        }
        ks1[4 * a + r] = f16_val((uint16_t)(kw & 0xffffu));
        ks2[4 * a + r] = f16_val((uint16_t)(kw >> 16));
        vs1[4 * a + r] = f16_val((uint16_t)(vw & 0xffffu));
        vs2[4 * a + r] = f16_val((uint16_t)(vw >> 16));
      }
    }
    float s8[8];
    float mloc = -INFINITY;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float dsum = sc[a][r] + __shfl_xor(sc[a][r], GQ);
        const int i = 4 * a + r;
        const float sv = valid[i] ? ks1[i] * (ks2[i] * dsum + qo) * cscale : -INFINITY;
        s8[i] = sv;
        mloc = fmaxf(mloc, sv);
      }
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float m_new = fmaxf(m_run, mloc);
    const float corr = exp2f(m_run - m_new);
    m_run = m_new;
    float lsum = 0.f, bsum = 0.f;
    half8 PA;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float pv = exp2f(s8[i] - m_new);
      const float pw = valid[i] ? pv * vs1[i] * vs2[i] : 0.f;
      lsum += pv;
      bsum += valid[i] ? pv * vs1[i] : 0.f;
      const _Float16 hi = (_Float16)pw;
      PA[i] = (n < GQ) ? hi : ((n < 2 * GQ) ? (_Float16)(pw - (float)hi) : (_Float16)0.f);
    }
    l_run = l_run * corr + lsum;
    beta_run = beta_run * corr + bsum;
    // rescale accumulators: rows 4 grp + r are head slots
    float cr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) cr[r] = __shfl(corr, 4 * grp + r);
#pragma unroll
    for (int bl = 0; bl < NB; ++bl)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[bl][t][r] *= cr[r];

    // ---------------- values: lane (column n, group grp) gathers 8 tokens
#pragma unroll
    for (int bl = 0; bl < NB; ++bl) {
      const int j = (G == 4) ? (2 * n + bl) : n;
      uint32_t E[8][NT / 2];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tt = base + 16 * (e >> 2) + 4 * grp + (e & 3);
        uint32_t word = 0u;
        if (tt < c1) {
          if (G == 4)
            word = *reinterpret_cast<const uint16_t*>(v_idx + (row0 + tt) * M + 2 * n);
          else
            word = v_idx[(row0 + tt) * M + j];
        }
        const uint32_t ad = gather_addr<G>(word, laneoff, (G == 4) ? bl : 0);
        if (G == 4) {
          const uint2 ev = *reinterpret_cast<const uint2*>(tab + ad);
          E[e][0] = ev.x;
          E[e][1] = ev.y;
        } else {
          const uint4 ev = *reinterpret_cast<const uint4*>(tab + ad);
          E[e][0] = ev.x;
          E[e][1] = ev.y;
          E[e][2] = ev.z;
          E[e][3] = ev.w;
        }
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
        uint4 bv;
        bv.x = __builtin_amdgcn_perm(E[1][t >> 1], E[0][t >> 1], sel);
        bv.y = __builtin_amdgcn_perm(E[3][t >> 1], E[2][t >> 1], sel);
        bv.z = __builtin_amdgcn_perm(E[5][t >> 1], E[4][t >> 1], sel);
        bv.w = __builtin_amdgcn_perm(E[7][t >> 1], E[6][t >> 1], sel);
        acc[bl][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(PA, __builtin_bit_cast(half8, bv), acc[bl][t], 0, 0, 0);
      }
    }
  }

  // ---------------- per-wave state -> LDS -> block merge -> workspace
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  beta_run += __shfl_xor(beta_run, 16);
  beta_run += __shfl_xor(beta_run, 32);
  __syncthreads();  // table no longer needed: reuse it for the partials
  float* s_acc = reinterpret_cast<float*>(s_tab);             // [4 waves][2GQ slots][128]
  float* s_st = s_acc + 4 * 2 * GQ * kD;                       // [4 waves][GQ][3]
#pragma unroll
  for (int bl = 0; bl < NB; ++bl)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int slot = 4 * grp + r;
        const int j = (G == 4) ? (2 * n + bl) : n;
        if (slot < 2 * GQ) s_acc[((size_t)wave * 2 * GQ + slot) * kD + G * j + t] = acc[bl][t][r];
      }
  if (grp == 0 && n < GQ) {
    s_st[(wave * GQ + n) * 3 + 0] = m_run;
    s_st[(wave * GQ + n) * 3 + 1] = l_run;
    s_st[(wave * GQ + n) * 3 + 2] = beta_run;
  }
  __syncthreads();
  for (int i = tid; i < GQ * kD; i += 256) {
    const int h = i / kD, c = i % kD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, s_st[(w * GQ + h) * 3]);
    float a = 0.f, l = 0.f, be = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = s_st[(w * GQ + h) * 3];
      const float f = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
      a += f * (s_acc[((size_t)w * 2 * GQ + h) * kD + c] + s_acc[((size_t)w * 2 * GQ + GQ + h) * kD + c]);
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
__global__ __launch_bounds__(128) void k_combine(const float* __restrict__ part, int nchunk, int Hq, int Hkv,
                                                 const float* __restrict__ v_o, float* __restrict__ out) {
  __shared__ float s[kD];
  const int bq = blockIdx.x, c = threadIdx.x;
  const int b = bq / Hq, hq = bq % Hq;
  const int hk = hq / (Hq / Hkv);
  const float* pp = part + (size_t)bq * nchunk * kPartStride;
  float M = -INFINITY;
  for (int i = 0; i < nchunk; ++i) M = fmaxf(M, pp[(size_t)i * kPartStride]);
  float a = 0.f, l = 0.f, be = 0.f;
  for (int i = 0; i < nchunk; ++i) {
    const float* q = pp + (size_t)i * kPartStride;
    const float f = (q[0] == -INFINITY) ? 0.f : exp2f(q[0] - M);
    a += f * q[4 + c];
    l += f * q[1];
    be += f * q[2];
  }
  s[c] = a;
  __syncthreads();
#pragma unroll
  for (int hsz = 1; hsz < kD; hsz <<= 1) {
    float v = 0.f;
    const int pr = c ^ hsz;
    v = (c & hsz) ? (s[pr] - s[c]) : (s[c] + s[pr]);
    __syncthreads();
    s[c] = v;
    __syncthreads();
  }
  const float rs = 0.08838834764831845f;
  out[(size_t)bq * kD + c] = (s[c] * rs + be * v_o[((size_t)b * Hkv + hk) * kD + c]) / l;
}

void pick_chunks(int B, int Hkv, int S, int& CH, int& nchunk) {
  long bh = (long)B * Hkv;
  long want = (2048 + bh - 1) / bh;
  long maxc = (S + 127) / 128;
  if (want > maxc) want = maxc;
  if (want < 1) want = 1;
  long ch = (S + want - 1) / want;
  ch = (ch + 31) / 32 * 32;
  CH = (int)ch;
  nchunk = (int)((S + ch - 1) / ch);
}

template <int G>
hipError_t launch_g(int GQ, dim3 grid, hipStream_t st, const uint16_t* q, int Hq, int Hkv, int S, int S_cap,
                    int CH, int nchunk, const uint8_t* k_idx, const uint16_t* k_sc, const float* k_o,
                    const uint8_t* v_idx, const uint16_t* v_sc, const uint16_t* c16, float* part) {
  switch (GQ) {
    case 1: k_decode<G, 1><<<grid, 256, 0, st>>>(q, Hq, Hkv, S, S_cap, CH, nchunk, k_idx, k_sc, k_o, v_idx, v_sc, c16, part); break;
    case 2: k_decode<G, 2><<<grid, 256, 0, st>>>(q, Hq, Hkv, S, S_cap, CH, nchunk, k_idx, k_sc, k_o, v_idx, v_sc, c16, part); break;
    case 4: k_decode<G, 4><<<grid, 256, 0, st>>>(q, Hq, Hkv, S, S_cap, CH, nchunk, k_idx, k_sc, k_o, v_idx, v_sc, c16, part); break;
    default: k_decode<G, 8><<<grid, 256, 0, st>>>(q, Hq, Hkv, S, S_cap, CH, nchunk, k_idx, k_sc, k_o, v_idx, v_sc, c16, part); break;
  }
  return hipGetLastError();
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
  k_combine<<<B * Hq, 128, 0, st>>>(part, nchunk, Hq, Hkv, v_o, out);
  return hipGetLastError();
}

}  // namespace nsn
