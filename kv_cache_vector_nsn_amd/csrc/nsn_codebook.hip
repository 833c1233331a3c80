// Global N(0,1) codebook by k-means on the GPU (fp64).
//
// "3. Vector Quantization and Codebook" of the Technical Summary of the
// explainer "NSNQuant: A Double Normalization Approach for Calibration-Free
// Low-Bit Vector Quantization of KV Cache" (gist.science/paper/2505.18231): the
// single codebook is initialised by k-means on synthetic standard-normal data
// and reused for every tensor.
//
// Samples come from a counter-based stream so that any range can be drawn
// independently: SplitMix64 (Steele, Lea, Flood 2014) output i of seed s is
// mix(s + (i + 1) * 0x9E3779B97F4A7C15); normal pair p takes outputs 2p, 2p+1,
// u1 = (top 53 bits + 1) 2^-53, u2 = top 53 bits 2^-53, and Box-Muller (1958)
// gives sqrt(-2 ln u1) (cos, sin)(2 pi u2).  Sample i is normals i*g .. i*g+g-1.
//
// Lloyd iterations (initial centroids = the first K samples): assign every
// sample to its nearest centroid (squared L2, lowest index on ties), stop if no
// assignment changed, else move each centroid to its cell mean; empty cells
// take, in increasing index, the samples farthest from their assigned centroid
// (lower sample index first).  Cell sums run per block in sample order and
// over blocks in block order, so the result is deterministic.
//
// Cosine fine-tune (same page and section: after k-means the codebook is tuned
// to minimise the cosine distance between original and quantized vectors, with
// no model involved).  Training vectors are d = 128 normals of the same stream
// (vector i = normals 128 i .. 128 i + 127, i.e. g-samples m i .. m i + m - 1,
// m = 128 / g).  Each iteration assigns every g-block to its nearest centroid,
// forms per vector c = <w, w_hat> / (|w| |w_hat|) and the derivative
// dc/dw_hat = w / (|w| |w_hat|) - c w_hat / |w_hat|^2, sums minus that derivative
// over the blocks of each centroid (divided by the number of vectors) in the
// same fixed order as the k-means cell sums, and steps C <- C - lr * gradient.
#include <cmath>
#include <cstring>
#include <numeric>
#include <vector>
#include <algorithm>

#include "nsn_internal.h"

namespace nsn {
namespace {

constexpr int kAssignBlock = 256;
constexpr int kSumSamples = 1024;  // samples per partial-sum block

__device__ __forceinline__ uint64_t splitmix64_at(uint64_t seed, uint64_t i) {
  uint64_t z = seed + (i + 1ull) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__global__ void k_gen(uint64_t seed, int64_t npairs, double* __restrict__ X) {
  const int64_t pidx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (pidx >= npairs) return;
  const uint64_t a = splitmix64_at(seed, 2 * (uint64_t)pidx) >> 11;
  const uint64_t b = splitmix64_at(seed, 2 * (uint64_t)pidx + 1) >> 11;
  const double u1 = ((double)a + 1.0) * 0x1.0p-53;
  const double u2 = (double)b * 0x1.0p-53;
  const double r = sqrt(-2.0 * log(u1));
  const double t = 2.0 * M_PI * u2;
  X[2 * pidx] = r * cos(t);
  X[2 * pidx + 1] = r * sin(t);
}

template <int G>
__global__ __launch_bounds__(kAssignBlock) void k_assign(const double* __restrict__ X, int64_t n,
                                                         const double* __restrict__ C, int K,
                                                         int* __restrict__ assign, double* __restrict__ dist,
                                                         int* __restrict__ changed) {
  __shared__ double s_c[256 * G];
  for (int i = threadIdx.x; i < K * G; i += blockDim.x) s_c[i] = C[i];
  __syncthreads();
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= n) return;
  double x[G];
#pragma unroll
  for (int e = 0; e < G; ++e) x[e] = X[i * G + e];
  double best = INFINITY;
  int bi = 0;
  for (int k = 0; k < K; ++k) {
    double dk = 0.0;
#pragma unroll
    for (int e = 0; e < G; ++e) {
      const double df = x[e] - s_c[k * G + e];
      dk = __dadd_rn(dk, __dmul_rn(df, df));
    }
    if (dk < best) {
      best = dk;
      bi = k;
    }
  }
  if (changed != nullptr && assign[i] != bi) atomicOr(changed, 1);
  assign[i] = bi;
  dist[i] = best;
}

// One block per kSumSamples samples; thread k accumulates cell k in sample order.
template <int G>
__global__ __launch_bounds__(256) void k_cellsum(const double* __restrict__ X, int64_t n,
                                                 const int* __restrict__ assign, double* __restrict__ psum,
                                                 int* __restrict__ pcnt) {
  __shared__ double s_x[kSumSamples * G];
  __shared__ int s_a[kSumSamples];
  const int64_t s0 = (int64_t)blockIdx.x * kSumSamples;
  const int cnt = (int)min((int64_t)kSumSamples, n - s0);
  for (int i = threadIdx.x; i < cnt * G; i += 256) s_x[i] = X[s0 * G + i];
  for (int i = threadIdx.x; i < cnt; i += 256) s_a[i] = assign[s0 + i];
  __syncthreads();
  const int k = threadIdx.x;
  double acc[G];
#pragma unroll
  for (int e = 0; e < G; ++e) acc[e] = 0.0;
  int c = 0;
  for (int i = 0; i < cnt; ++i) {
    if (s_a[i] == k) {
      ++c;
#pragma unroll
      for (int e = 0; e < G; ++e) acc[e] += s_x[i * G + e];
    }
  }
#pragma unroll
  for (int e = 0; e < G; ++e) psum[((size_t)blockIdx.x * 256 + k) * G + e] = acc[e];
  pcnt[(size_t)blockIdx.x * 256 + k] = c;
}

template <int G>
__global__ __launch_bounds__(256) void k_update(const double* __restrict__ psum, const int* __restrict__ pcnt,
                                                int nblk, double* __restrict__ C, int* __restrict__ counts) {
  const int k = threadIdx.x;
  double acc[G];
#pragma unroll
  for (int e = 0; e < G; ++e) acc[e] = 0.0;
  long c = 0;
  for (int b = 0; b < nblk; ++b) {
#pragma unroll
    for (int e = 0; e < G; ++e) acc[e] += psum[((size_t)b * 256 + k) * G + e];
    c += pcnt[(size_t)b * 256 + k];
  }
  counts[k] = (int)c;
  if (c > 0) {
#pragma unroll
    for (int e = 0; e < G; ++e) C[k * G + e] = acc[e] / (double)c;
  }
}

// One thread per training vector: coefficients of dc/dw_hat and 1 - c.
template <int G>
__global__ __launch_bounds__(256) void k_cos(const double* __restrict__ X, int64_t nvec,
                                             const double* __restrict__ C, const int* __restrict__ assign,
                                             double* __restrict__ coef_a, double* __restrict__ coef_b,
                                             double* __restrict__ dist) {
  constexpr int M = kD / G;
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= nvec) return;
  double ww = 0.0, wh = 0.0, hh = 0.0;
  for (int b = 0; b < M; ++b) {
    const int k = assign[i * M + b];
#pragma unroll
    for (int e = 0; e < G; ++e) {
      const double x = X[(i * M + b) * G + e], c = C[k * G + e];
      ww = fma(x, x, ww);
      wh = fma(x, c, wh);
      hh = fma(c, c, hh);
    }
  }
  double a = 0.0, bb = 0.0, t = 1.0;
  if (ww > 0.0 && hh > 0.0) {
    const double nw = sqrt(ww), nh = sqrt(hh);
    const double c = wh / (nw * nh);
    a = 1.0 / (nw * nh);
    bb = c / hh;
    t = 1.0 - c;
  }
  coef_a[i] = a;
  coef_b[i] = bb;
  dist[i] = t;
}

// Per-centroid partial sums of -(a_i x_j - b_i C_{k_j}) / nvec over the blocks j of
// kSumSamples consecutive g-samples (thread k sums centroid k in sample order).
template <int G>
__global__ __launch_bounds__(256) void k_gradsum(const double* __restrict__ X, int64_t n,
                                                 const int* __restrict__ assign, const double* __restrict__ C,
                                                 const double* __restrict__ coef_a,
                                                 const double* __restrict__ coef_b, double inv_nvec,
                                                 double* __restrict__ psum) {
  constexpr int M = kD / G;
  __shared__ double s_x[kSumSamples * G];
  __shared__ int s_a[kSumSamples];
  const int64_t s0 = (int64_t)blockIdx.x * kSumSamples;
  const int cnt = (int)min((int64_t)kSumSamples, n - s0);
  for (int i = threadIdx.x; i < cnt; i += 256) s_a[i] = assign[s0 + i];
  __syncthreads();
  for (int i = threadIdx.x; i < cnt * G; i += 256) {
    const int64_t j = s0 + i / G;
    const int e = i % G;
    const int64_t v = j / M;
    s_x[i] = -(coef_a[v] * X[j * G + e] - coef_b[v] * C[s_a[i / G] * G + e]) * inv_nvec;
  }
  __syncthreads();
  const int k = threadIdx.x;
  double acc[G];
#pragma unroll
  for (int e = 0; e < G; ++e) acc[e] = 0.0;
  for (int i = 0; i < cnt; ++i) {
    if (s_a[i] == k) {
#pragma unroll
      for (int e = 0; e < G; ++e) acc[e] += s_x[i * G + e];
    }
  }
#pragma unroll
  for (int e = 0; e < G; ++e) psum[((size_t)blockIdx.x * 256 + k) * G + e] = acc[e];
}

template <int G>
__global__ __launch_bounds__(256) void k_gradstep(const double* __restrict__ psum, int nblk, double lr,
                                                  double* __restrict__ C) {
  const int k = threadIdx.x;
  double acc[G];
#pragma unroll
  for (int e = 0; e < G; ++e) acc[e] = 0.0;
  for (int b = 0; b < nblk; ++b) {
#pragma unroll
    for (int e = 0; e < G; ++e) acc[e] += psum[((size_t)b * 256 + k) * G + e];
  }
#pragma unroll
  for (int e = 0; e < G; ++e) C[k * G + e] -= lr * acc[e];
}

struct DevBuf {
  void* p = nullptr;
  ~DevBuf() {
    if (p) (void)hipFree(p);
  }
};

template <int G>
int run(uint64_t seed, int K, int64_t n, int max_iters, float* centroids, double* distortion, int* iterations) {
  DevBuf dX, dC, dA, dD, dS, dP, dCnt, dF;
  const int nblk = (int)((n + kSumSamples - 1) / kSumSamples);
  hipError_t e;
  if ((e = hipMalloc(&dX.p, sizeof(double) * n * G)) != hipSuccess) return hip_fail(e, "hipMalloc(samples)");
  if ((e = hipMalloc(&dC.p, sizeof(double) * K * G)) != hipSuccess) return hip_fail(e, "hipMalloc(centroids)");
  if ((e = hipMalloc(&dA.p, sizeof(int) * n)) != hipSuccess) return hip_fail(e, "hipMalloc(assign)");
  if ((e = hipMalloc(&dD.p, sizeof(double) * n)) != hipSuccess) return hip_fail(e, "hipMalloc(dist)");
  if ((e = hipMalloc(&dS.p, sizeof(double) * nblk * 256 * G)) != hipSuccess) return hip_fail(e, "hipMalloc(psum)");
  if ((e = hipMalloc(&dP.p, sizeof(int) * nblk * 256)) != hipSuccess) return hip_fail(e, "hipMalloc(pcnt)");
  if ((e = hipMalloc(&dCnt.p, sizeof(int) * 256)) != hipSuccess) return hip_fail(e, "hipMalloc(counts)");
  if ((e = hipMalloc(&dF.p, sizeof(int))) != hipSuccess) return hip_fail(e, "hipMalloc(flag)");
  double* X = (double*)dX.p;
  double* C = (double*)dC.p;
  int* A = (int*)dA.p;
  double* D = (double*)dD.p;
  const int64_t npairs = n * G / 2;
  k_gen<<<(unsigned)((npairs + 255) / 256), 256>>>(seed, npairs, X);
  if ((e = hipMemcpy(C, X, sizeof(double) * K * G, hipMemcpyDeviceToDevice)) != hipSuccess)
    return hip_fail(e, "init centroids");
  const unsigned ablk = (unsigned)((n + kAssignBlock - 1) / kAssignBlock);
  std::vector<int> counts(256);
  std::vector<double> hd, hC(K * G);
  int it = 0;
  bool first = true;
  while (it < max_iters) {
    int zero = 0;
    if ((e = hipMemcpy(dF.p, &zero, sizeof(int), hipMemcpyHostToDevice)) != hipSuccess) return hip_fail(e, "flag");
    k_assign<G><<<ablk, kAssignBlock>>>(X, n, C, K, A, D, first ? nullptr : (int*)dF.p);
    ++it;
    int changed = 0;
    if ((e = hipMemcpy(&changed, dF.p, sizeof(int), hipMemcpyDeviceToHost)) != hipSuccess) return hip_fail(e, "assign");
    if (!first && !changed) break;
    first = false;
    k_cellsum<G><<<nblk, 256>>>(X, n, A, (double*)dS.p, (int*)dP.p);
    k_update<G><<<1, 256>>>((const double*)dS.p, (const int*)dP.p, nblk, C, (int*)dCnt.p);
    if ((e = hipMemcpy(counts.data(), dCnt.p, sizeof(int) * 256, hipMemcpyDeviceToHost)) != hipSuccess)
      return hip_fail(e, "update");
    std::vector<int> empty;
    for (int k = 0; k < K; ++k)
      if (counts[k] == 0) empty.push_back(k);
    if (!empty.empty()) {  // rare: re-seed from the farthest samples
      hd.resize(n);
      if ((e = hipMemcpy(hd.data(), D, sizeof(double) * n, hipMemcpyDeviceToHost)) != hipSuccess) return hip_fail(e, "dist");
      std::vector<int64_t> order(n);
      std::iota(order.begin(), order.end(), 0);
      std::stable_sort(order.begin(), order.end(), [&](int64_t a, int64_t b) { return hd[a] > hd[b]; });
      for (size_t j = 0; j < empty.size(); ++j) {
        if ((e = hipMemcpy(C + empty[j] * G, X + order[j] * G, sizeof(double) * G, hipMemcpyDeviceToDevice)) != hipSuccess)
          return hip_fail(e, "reseed");
      }
    }
  }
  if ((e = hipMemcpy(hC.data(), C, sizeof(double) * K * G, hipMemcpyDeviceToHost)) != hipSuccess) return hip_fail(e, "result");
  for (int i = 0; i < K * G; ++i) {
    const _Float16 h = (_Float16)hC[i];  // round to nearest even
    hC[i] = (double)h;
    centroids[i] = (float)h;
  }
  if (iterations) *iterations = it;
  if (distortion) {
    if ((e = hipMemcpy(C, hC.data(), sizeof(double) * K * G, hipMemcpyHostToDevice)) != hipSuccess) return hip_fail(e, "rounded");
    k_assign<G><<<ablk, kAssignBlock>>>(X, n, C, K, A, D, nullptr);
    hd.resize(n);
    if ((e = hipMemcpy(hd.data(), D, sizeof(double) * n, hipMemcpyDeviceToHost)) != hipSuccess) return hip_fail(e, "distortion");
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i) s += hd[i];
    *distortion = s / (double)n / (double)G;
  }
  if ((e = hipDeviceSynchronize()) != hipSuccess) return hip_fail(e, "build_codebook");
  return NSN_OK;
}

template <int G>
int run_finetune(const float* cin, int K, uint64_t seed, int64_t nvec, int iters, double lr, float* cout,
                 double* raw, double* cos_dist) {
  constexpr int M = kD / G;
  const int64_t n = nvec * M;  // g-samples
  const int nblk = (int)((n + kSumSamples - 1) / kSumSamples);
  DevBuf dX, dC, dA, dD, dS, dCa, dCb, dT;
  hipError_t e;
  if ((e = hipMalloc(&dX.p, sizeof(double) * n * G)) != hipSuccess) return hip_fail(e, "hipMalloc(vectors)");
  if ((e = hipMalloc(&dC.p, sizeof(double) * K * G)) != hipSuccess) return hip_fail(e, "hipMalloc(centroids)");
  if ((e = hipMalloc(&dA.p, sizeof(int) * n)) != hipSuccess) return hip_fail(e, "hipMalloc(assign)");
  if ((e = hipMalloc(&dD.p, sizeof(double) * n)) != hipSuccess) return hip_fail(e, "hipMalloc(dist)");
  if ((e = hipMalloc(&dS.p, sizeof(double) * nblk * 256 * G)) != hipSuccess) return hip_fail(e, "hipMalloc(psum)");
  if ((e = hipMalloc(&dCa.p, sizeof(double) * nvec)) != hipSuccess) return hip_fail(e, "hipMalloc(coef)");
  if ((e = hipMalloc(&dCb.p, sizeof(double) * nvec)) != hipSuccess) return hip_fail(e, "hipMalloc(coef)");
  if ((e = hipMalloc(&dT.p, sizeof(double) * nvec)) != hipSuccess) return hip_fail(e, "hipMalloc(cos)");
  double* X = (double*)dX.p;
  double* C = (double*)dC.p;
  int* A = (int*)dA.p;
  std::vector<double> hC(K * G), ht(nvec);
  for (int i = 0; i < K * G; ++i) hC[i] = (double)cin[i];
  if ((e = hipMemcpy(C, hC.data(), sizeof(double) * K * G, hipMemcpyHostToDevice)) != hipSuccess)
    return hip_fail(e, "upload centroids");
  const int64_t npairs = n * G / 2;
  k_gen<<<(unsigned)((npairs + 255) / 256), 256>>>(seed, npairs, X);
  const unsigned ablk = (unsigned)((n + kAssignBlock - 1) / kAssignBlock);
  const unsigned vblk = (unsigned)((nvec + 255) / 256);
  auto mean_dist = [&](int slot) -> int {
    k_assign<G><<<ablk, kAssignBlock>>>(X, n, C, K, A, (double*)dD.p, nullptr);
    k_cos<G><<<vblk, 256>>>(X, nvec, C, A, (double*)dCa.p, (double*)dCb.p, (double*)dT.p);
    if (cos_dist != nullptr) {
      hipError_t e2 = hipMemcpy(ht.data(), dT.p, sizeof(double) * nvec, hipMemcpyDeviceToHost);
      if (e2 != hipSuccess) return hip_fail(e2, "cosine distances");
      double sum = 0.0;
      for (int64_t i = 0; i < nvec; ++i) sum += ht[i];
      cos_dist[slot] = sum / (double)nvec;
    }
    return NSN_OK;
  };
  for (int it = 0; it < iters; ++it) {
    int r = mean_dist(it);
    if (r != NSN_OK) return r;
    k_gradsum<G><<<nblk, 256>>>(X, n, A, C, (const double*)dCa.p, (const double*)dCb.p, 1.0 / (double)nvec,
                                (double*)dS.p);
    k_gradstep<G><<<1, 256>>>((const double*)dS.p, nblk, lr, C);
  }
  if ((e = hipMemcpy(hC.data(), C, sizeof(double) * K * G, hipMemcpyDeviceToHost)) != hipSuccess)
    return hip_fail(e, "result");
  for (int i = 0; i < K * G; ++i) {
    if (raw != nullptr) raw[i] = hC[i];
    const _Float16 h = (_Float16)hC[i];  // round to nearest even
    hC[i] = (double)h;
    cout[i] = (float)h;
  }
  if (cos_dist != nullptr) {  // the rounded codebook
    if ((e = hipMemcpy(C, hC.data(), sizeof(double) * K * G, hipMemcpyHostToDevice)) != hipSuccess)
      return hip_fail(e, "rounded");
    int r = mean_dist(iters);
    if (r != NSN_OK) return r;
  }
  if ((e = hipDeviceSynchronize()) != hipSuccess) return hip_fail(e, "finetune_codebook");
  return NSN_OK;
}

}  // namespace

int finetune_codebook_device(const float* cin, int g, int K, uint64_t seed, int64_t nvec, int iters, double lr,
                             float* cout, double* raw, double* cos_dist) {
  return g == 4 ? run_finetune<4>(cin, K, seed, nvec, iters, lr, cout, raw, cos_dist)
                : run_finetune<8>(cin, K, seed, nvec, iters, lr, cout, raw, cos_dist);
}

int build_codebook_device(uint64_t seed, int g, int K, int64_t n, int max_iters, float* centroids, double* distortion,
                          int* iterations) {
  return g == 4 ? run<4>(seed, K, n, max_iters, centroids, distortion, iterations)
                : run<8>(seed, K, n, max_iters, centroids, distortion, iterations);
}

}  // namespace nsn
