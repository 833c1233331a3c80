// Candidate table of the exact pruned nearest-centroid search (g = 4).
//
// The assignment itself is the exhaustive one of "3. Vector Quantization and
// Codebook" in the Technical Summary of the explainer "NSNQuant: A Double
// Normalization Approach for Calibration-Free Low-Bit Vector Quantization of KV
// Cache" (gist.science/paper/2505.18231): the nearest of the K centroids in
// squared L2.  The encode kernel reaches the same argmin through this table:
// R^4 is cut into a uniform grid and each cell keeps only the centroids that can
// be nearest to some point of the cell.
//
// Exclusion rule (exact and conservative): centroid c leaves the list of cell B
// when another centroid c' is strictly closer than c at every point of B,
//   max over x in B of ( ||x - c'||^2 - ||x - c||^2 ) < 0.
// The difference is affine in x, 2 <x, c - c'> + ||c'||^2 - ||c||^2, so its
// maximum over the box is sum_d max(a_d lo_d, a_d hi_d) + ||c'||^2 - ||c||^2
// with a = 2 (c - c').  A centroid removed this way is never the nearest one of
// a point of B, so the exhaustive argmin over all K is always in the list.
// Centroids whose smallest distance to the box exceeds
// U = min_c' max over x in B of ||x - c'||^2 are skipped before the pairwise
// test: the minimiser of U is closer than them everywhere in B.
//
// Second rule (also exact and conservative): a survivor c can still be beaten
// everywhere on B by different centroids at different points.  With
// f_j(x) = ||x - c||^2 - ||x - c_j||^2 (affine in x) over the other survivors c_j,
// any weights lambda >= 0 summing to 1 with
//   min over x in B of sum_j lambda_j f_j(x) > 0
// prove that at every x some f_j(x) > 0, i.e. some c_j is closer than c, so c is
// never the nearest centroid on B (LP duality: such weights exist exactly when
// the Voronoi cell of c misses B).  The weights are searched by exponentiated-
// gradient ascent on that minimum; only the final fp64 evaluation of the minimum
// decides, so a poor search keeps a centroid but never drops a needed one.
// All decisions are fp64; the box is enlarged by kGridMargin on every side so
// that a point whose fp32 cell index is off by rounding is still covered.
#include "nsn_internal.h"

namespace nsn {
namespace {

__device__ __forceinline__ void put_byte(uint32_t& w0, uint32_t& w1, uint32_t& w2, int j, int c) {
  const uint32_t b = (uint32_t)c << (8 * (j & 3));
  if (j < 4) w0 |= b;
  else if (j < 8) w1 |= b;
  else w2 |= b;
}

constexpr int kPairMax = 32;       // survivors of the pairwise rule the certificate search examines
constexpr int kCertIters = 200;    // exponentiated-gradient steps per candidate
constexpr float kCertStep = 5.0f;  // step of the weight update

// True when candidate `self` of the n survivors `mem` is proved never nearest on
// the box [lo, hi] (the second rule above).
__device__ bool certified_out(int self, const uint8_t* mem, int n, const double (*sc)[4], const double* sn,
                              const double lo[4], const double hi[4]) {
  double a[kPairMax][4], b[kPairMax];  // f_j(x) = <a_j, x> + b_j
  float lam[kPairMax];
  int m = 0;
  const int c = mem[self];
  for (int j = 0; j < n; ++j) {
    if (j == self) continue;
    const int cj = mem[j];
#pragma unroll
    for (int d = 0; d < 4; ++d) a[m][d] = 2.0 * (sc[cj][d] - sc[c][d]);
    b[m] = sn[c] - sn[cj];
    lam[m] = 1.f / (float)(n - 1);
    ++m;
  }
  for (int it = 0; it < kCertIters; ++it) {
    // the combination, its minimiser over the box (a corner) and its minimum, in fp64
    double coef[4] = {0.0, 0.0, 0.0, 0.0}, cst = 0.0, x[4];
    for (int j = 0; j < m; ++j) {
#pragma unroll
      for (int d = 0; d < 4; ++d) coef[d] += (double)lam[j] * a[j][d];
      cst += (double)lam[j] * b[j];
    }
    double val = cst;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      x[d] = coef[d] > 0.0 ? lo[d] : hi[d];
      val += coef[d] * x[d];
    }
    if (val > 1e-9) return true;
    // more weight on the differences that are largest at that corner
    float fx[kPairMax], fmx = -INFINITY;
    for (int j = 0; j < m; ++j) {
      double f = b[j];
#pragma unroll
      for (int d = 0; d < 4; ++d) f += a[j][d] * x[d];
      fx[j] = (float)f;
      fmx = fmaxf(fmx, fx[j]);
    }
    float tot = 0.f;
    for (int j = 0; j < m; ++j) {
      lam[j] *= __expf(kCertStep * (fx[j] - fmx));
      tot += lam[j];
    }
    for (int j = 0; j < m; ++j) lam[j] /= tot;
  }
  return false;
}

// One thread per cell; cell id = ((i0 * N + i1) * N + i2) * N + i3 with i_d the
// bin of coordinate d, bin i covering [(i - kGridOff) / kGridInv, (i + 1 - kGridOff) / kGridInv).
__global__ __launch_bounds__(256) void k_cells(const float* __restrict__ c32, uint4* __restrict__ cells,
                                               int* __restrict__ stats) {
  __shared__ double sc[kK][4];
  __shared__ double sn[kK];
  for (int i = threadIdx.x; i < kK; i += blockDim.x) {
    double n = 0.0;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const double v = (double)c32[i * 4 + d];
      sc[i][d] = v;
      n += v * v;
    }
    sn[i] = n;
  }
  __syncthreads();
  const int cell = blockIdx.x * blockDim.x + threadIdx.x;
  if (cell >= kGridCells) return;
  double lo[4], hi[4];
  int t = cell;
  for (int d = 3; d >= 0; --d) {
    const int i = t % kGridN;
    t /= kGridN;
    lo[d] = ((double)i - (double)kGridOff) / (double)kGridInv - kGridMargin;
    hi[d] = ((double)i + 1.0 - (double)kGridOff) / (double)kGridInv + kGridMargin;
  }
  double U = INFINITY;
  for (int c = 0; c < kK; ++c) {
    double m = 0.0;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const double a = lo[d] - sc[c][d], b = hi[d] - sc[c][d];
      m += fmax(a * a, b * b);
    }
    U = fmin(U, m);
  }
  uint8_t mem[kPairMax];  // pairwise survivors, ascending
  int npair = 0;
  for (int c = 0; c < kK; ++c) {
    double lb = 0.0;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const double q = fmax(fmax(lo[d] - sc[c][d], sc[c][d] - hi[d]), 0.0);
      lb += q * q;
    }
    if (lb > U + 1e-9) continue;
    bool dropped = false;
    for (int c2 = 0; c2 < kK && !dropped; ++c2) {
      if (c2 == c) continue;
      double m = sn[c2] - sn[c];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const double a = 2.0 * (sc[c][d] - sc[c2][d]);
        m += fmax(a * lo[d], a * hi[d]);
      }
      dropped = m < -1e-9;
    }
    if (dropped) continue;
    if (npair < kPairMax) mem[npair] = (uint8_t)c;
    ++npair;
  }
  uint32_t w0 = 0, w1 = 0, w2 = 0;
  int cnt = 0, last = 0;
  if (npair > kPairMax) {
    cnt = npair;  // overflows the row either way
  } else {
    for (int i = 0; i < npair; ++i) {
      if (npair > 1 && certified_out(i, mem, npair, sc, sn, lo, hi)) continue;
      if (cnt < kCellList) put_byte(w0, w1, w2, cnt, mem[i]);
      last = mem[i];
      ++cnt;
    }
  }
  for (int j = cnt; j < kCellList; ++j) put_byte(w0, w1, w2, j, last);
  const bool overflow = cnt > kCellList || cnt == 0;
  const uint32_t w3 = (uint32_t)min(cnt, 255) | ((overflow ? 1u : 0u) << 24);
  cells[cell] = make_uint4(w0, w1, w2, w3);
  atomicMax(&stats[0], cnt);
  if (overflow) atomicAdd(&stats[1], 1);
}

}  // namespace

hipError_t build_cells(nsn_codebook* cb) {
  hipError_t e = hipMalloc(&cb->d_cells, sizeof(uint4) * (size_t)kGridCells);
  if (e != hipSuccess) return e;
  int* d_stats = nullptr;
  if ((e = hipMalloc(&d_stats, 2 * sizeof(int))) != hipSuccess) return e;
  int st[2] = {0, 0};
  if ((e = hipMemcpy(d_stats, st, sizeof(st), hipMemcpyHostToDevice)) == hipSuccess) {
    k_cells<<<(kGridCells + 255) / 256, 256>>>(cb->d_c32, cb->d_cells, d_stats);
    e = hipGetLastError();
    if (e == hipSuccess) e = hipMemcpy(st, d_stats, sizeof(st), hipMemcpyDeviceToHost);
  }
  (void)hipFree(d_stats);
  cb->cell_max = st[0];
  cb->cell_overflow = st[1];
  return e;
}

}  // namespace nsn
