// C ABI of the NSNQuant library: argument validation (pure host code, runs
// before any HIP call), the codebook handle, workspace queries and status text.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "nsn_internal.h"

namespace nsn {

static thread_local std::string g_last_error;

int set_error(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return set_error(e == hipErrorOutOfMemory ? NSN_ENOMEM : NSN_EHIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

static int ok() {
  g_last_error.clear();
  return NSN_OK;
}

static bool f16_exact(float v) {
  const _Float16 h = (_Float16)v;
  return (float)h == v;
}

// Encode-side argument checks (shared by encode and dequantize).
static int check_common(const nsn_codebook* cb, int B, int H, int L, int L_cap, int d) {
  if (cb == nullptr) return set_error(NSN_EINVAL, "codebook handle is NULL");
  if (B <= 0 || H <= 0 || L <= 0 || L_cap <= 0) return set_error(NSN_EINVAL, "sizes must be positive (B=%d H=%d L=%d L_cap=%d)", B, H, L, L_cap);
  if (d != kD) return set_error(NSN_EUNSUPPORTED, "head dimension %d unsupported (only %d)", d, kD);
  if ((long)B * H * L_cap > (long)INT32_MAX) return set_error(NSN_EUNSUPPORTED, "B*H*L_cap exceeds 2^31-1");
  // the per-token kernels run a grid row per (batch, head)
  if ((long)B * H > 65535) return set_error(NSN_EUNSUPPORTED, "B*H = %ld exceeds 65535", (long)B * H);
  return NSN_OK;
}

// The handle's tables live on the device it was created on; a call made with
// another device current would hand those pointers to kernels running elsewhere.
static int check_device(const nsn_codebook* cb) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != cb->device)
    return set_error(NSN_EINVAL, "codebook was created on device %d, the current device is %d", cb->device, dev);
  return NSN_OK;
}

}  // namespace nsn

using namespace nsn;

extern "C" {

int nsn_version(void) { return 10000; }

const char* nsn_last_error(void) { return g_last_error.c_str(); }

int nsn_codebook_g(const nsn_codebook* cb) { return cb ? cb->g : 0; }

int nsn_codebook_search_stats(const nsn_codebook* cb, int* max_list, int* overflow_cells) {
  if (cb == nullptr) return set_error(NSN_EINVAL, "NULL codebook");
  if (max_list) *max_list = cb->cell_max;
  if (overflow_cells) *overflow_cells = cb->cell_overflow;
  return ok();
}

int nsn_search_grid_edges(float* edges, int cap) {
  if (edges == nullptr) return set_error(NSN_EINVAL, "NULL edges");
  if (cap < kGridN + 1) return set_error(NSN_EINVAL, "cap %d < %d edges", cap, kGridN + 1);
  for (int j = 0; j <= kGridN; ++j) edges[j] = ((float)j - kGridOff) / kGridInv;
  ok();
  return kGridN + 1;
}

int nsn_build_codebook(uint64_t seed, int g, int K, int64_t n_samples, int max_iters, float* centroids,
                       double* distortion, int* iterations) {
  if (centroids == nullptr) return set_error(NSN_EINVAL, "centroids is NULL");
  if (g != 4 && g != 8) return set_error(NSN_EUNSUPPORTED, "g=%d unsupported (4 or 8)", g);
  if (K != kK) return set_error(NSN_EUNSUPPORTED, "K=%d unsupported (256)", K);
  if (n_samples < K) return set_error(NSN_EINVAL, "n_samples=%lld < K", (long long)n_samples);
  if (n_samples > ((int64_t)1 << 28)) return set_error(NSN_EUNSUPPORTED, "n_samples above 2^28");
  if (max_iters < 1) return set_error(NSN_EINVAL, "max_iters must be >= 1");
  const int r = build_codebook_device(seed, g, K, n_samples, max_iters, centroids, distortion, iterations);
  return r == NSN_OK ? ok() : r;
}

int nsn_finetune_codebook(const float* centroids_in, int g, int K, uint64_t seed, int64_t n_vectors, int iters,
                          double lr, float* centroids_out, double* centroids_raw, double* cos_dist) {
  if (centroids_in == nullptr || centroids_out == nullptr) return set_error(NSN_EINVAL, "NULL centroid array");
  if (g != 4 && g != 8) return set_error(NSN_EUNSUPPORTED, "g=%d unsupported (4 or 8)", g);
  if (K != kK) return set_error(NSN_EUNSUPPORTED, "K=%d unsupported (256)", K);
  if (n_vectors < 1) return set_error(NSN_EINVAL, "n_vectors=%lld must be positive", (long long)n_vectors);
  if (n_vectors > ((int64_t)1 << 22)) return set_error(NSN_EUNSUPPORTED, "n_vectors above 2^22");
  if (iters < 0) return set_error(NSN_EINVAL, "iters must be >= 0");
  if (!std::isfinite(lr) || lr < 0.0) return set_error(NSN_EINVAL, "lr must be finite and >= 0");
  for (int i = 0; i < K * g; ++i)
    if (!std::isfinite(centroids_in[i])) return set_error(NSN_EINVAL, "centroid entry %d is not finite", i);
  const int r = finetune_codebook_device(centroids_in, g, K, seed, n_vectors, iters, lr, centroids_out, centroids_raw,
                                         cos_dist);
  return r == NSN_OK ? ok() : r;
}

int nsn_codebook_create(const float* centroids, int g, int K, nsn_codebook** out) {
  if (centroids == nullptr || out == nullptr) return set_error(NSN_EINVAL, "NULL argument");
  if (g != 4 && g != 8) return set_error(NSN_EUNSUPPORTED, "g=%d unsupported (4 or 8)", g);
  if (K != kK) return set_error(NSN_EUNSUPPORTED, "K=%d unsupported (256)", K);
  for (int i = 0; i < K * g; ++i) {
    if (!std::isfinite(centroids[i]) || !f16_exact(centroids[i]))
      return set_error(NSN_EINVAL, "centroid entry %d (%g) is not an exact fp16 value", i, (double)centroids[i]);
  }
  nsn_codebook* cb = new (std::nothrow) nsn_codebook();
  if (cb == nullptr) return set_error(NSN_ENOMEM, "host allocation failed");
  cb->g = g;
  cb->K = K;
  std::memcpy(cb->host, centroids, sizeof(float) * K * g);
  // fp16 copy and encode MFMA A fragments: [tile][kind][lane][8]
  uint16_t c16[kK * 8];
  for (int i = 0; i < K * g; ++i) {
    const _Float16 h = (_Float16)centroids[i];
    std::memcpy(&c16[i], &h, 2);
  }
  static_assert(sizeof(_Float16) == 2, "fp16");
  uint16_t encA[kTiles * 2 * 64 * 8];
  auto put = [&](int t, int kind, int lane, int e, float v) {
    const _Float16 h = (_Float16)v;
    std::memcpy(&encA[(((t * 2 + kind) * 64) + lane) * 8 + e], &h, 2);
  };
  for (int t = 0; t < kTiles; ++t) {
    for (int lane = 0; lane < 64; ++lane) {
      const int k = 32 * t + (lane & 31), hsel = lane >> 5;
      double n2 = 0.0;
      for (int e = 0; e < g; ++e) n2 += (double)centroids[k * g + e] * centroids[k * g + e];
      const _Float16 nh = (_Float16)n2;
      const _Float16 nl = (_Float16)(n2 - (double)nh);
      for (int e = 0; e < 8; ++e) {
        float v0 = 0.f, v1 = 0.f;
        if (g == 4) {
          if (hsel == 0) v0 = centroids[k * 4 + (e & 3)];
          else v0 = (e == 0) ? (float)nh : (e == 1) ? (float)nl : (e == 2 || e == 3) ? 1.f : 0.f;
        } else {
          v0 = centroids[k * 8 + e];
          if (hsel == 0) v1 = (e == 0) ? (float)nh : (e == 1) ? (float)nl : (e == 2 || e == 3) ? 1.f : 0.f;
        }
        put(t, 0, lane, e, v0);
        put(t, 1, lane, e, v1);
      }
    }
  }
  hipError_t e;
  if ((e = hipGetDevice(&cb->device)) != hipSuccess) { delete cb; return hip_fail(e, "hipGetDevice"); }
  if ((e = hipDeviceGetAttribute(&cb->num_cu, hipDeviceAttributeMultiprocessorCount, cb->device)) != hipSuccess) {
    delete cb;
    return hip_fail(e, "hipDeviceGetAttribute");
  }
  if (cb->num_cu < 1) cb->num_cu = 1;
  if ((e = hipMalloc(&cb->d_c32, sizeof(float) * K * g)) != hipSuccess ||
      (e = hipMalloc(&cb->d_c16, sizeof(uint16_t) * K * g)) != hipSuccess ||
      (e = hipMalloc(&cb->d_encA, sizeof(encA))) != hipSuccess) {
    nsn_codebook_destroy(cb);
    return hip_fail(e, "hipMalloc(codebook)");
  }
  if ((e = hipMemcpy(cb->d_c32, centroids, sizeof(float) * K * g, hipMemcpyHostToDevice)) != hipSuccess ||
      (e = hipMemcpy(cb->d_c16, c16, sizeof(uint16_t) * K * g, hipMemcpyHostToDevice)) != hipSuccess ||
      (e = hipMemcpy(cb->d_encA, encA, sizeof(encA), hipMemcpyHostToDevice)) != hipSuccess) {
    nsn_codebook_destroy(cb);
    return hip_fail(e, "hipMemcpy(codebook)");
  }
  if (g == 8) {
    // 16x16x32 distance-GEMM A fragments: tile t, lane l (row i = l % 16, slot group
    // q = l / 16): q = 0, 1: centroid 16 t + i; q = 2: (||C||^2 hi, lo, 1, 1); q = 3: 0
    uint16_t a16[16 * 64 * 8];
    for (int t = 0; t < 16; ++t)
      for (int lane = 0; lane < 64; ++lane) {
        const int k = 16 * t + (lane & 15), qg = lane >> 4;
        double n2 = 0.0;
        for (int e = 0; e < 8; ++e) n2 += (double)centroids[k * 8 + e] * centroids[k * 8 + e];
        const _Float16 nh = (_Float16)n2;
        const _Float16 nl = (_Float16)(n2 - (double)nh);
        for (int e = 0; e < 8; ++e) {
          const float v = qg < 2 ? centroids[k * 8 + e]
                                 : qg == 2 ? (e == 0 ? (float)nh : e == 1 ? (float)nl : e < 4 ? 1.f : 0.f) : 0.f;
          const _Float16 h = (_Float16)v;
          std::memcpy(&a16[((t * 64) + lane) * 8 + e], &h, 2);
        }
      }
    if ((e = hipMalloc(&cb->d_encA16, sizeof(a16))) != hipSuccess ||
        (e = hipMemcpy(cb->d_encA16, a16, sizeof(a16), hipMemcpyHostToDevice)) != hipSuccess) {
      nsn_codebook_destroy(cb);
      return hip_fail(e, "encode fragments");
    }
  }
  {
    // decode table rows: 16 bytes per centroid (g = 4: the 8-byte entry twice)
    uint16_t rows[kK * 8];
    for (int k = 0; k < K; ++k)
      for (int j = 0; j < 8; ++j) rows[k * 8 + j] = c16[k * g + (j % g)];
    if ((e = hipMalloc(&cb->d_c16x2, sizeof(rows))) != hipSuccess ||
        (e = hipMemcpy(cb->d_c16x2, rows, sizeof(rows), hipMemcpyHostToDevice)) != hipSuccess) {
      nsn_codebook_destroy(cb);
      return hip_fail(e, "decode table rows");
    }
  }
  if (g == 4) {
    // pruned-search tables: per-centroid records and the candidate grid
    uint32_t rec[kK * 4];
    for (int k = 0; k < K; ++k) {
      double n2 = 0.0;
      for (int d = 0; d < 4; ++d) n2 += (double)centroids[k * 4 + d] * centroids[k * 4 + d];
      const float n2f = (float)n2;
      uint32_t nb;
      std::memcpy(&nb, &n2f, 4);
      rec[k * 4 + 0] = (uint32_t)c16[k * 4 + 0] | ((uint32_t)c16[k * 4 + 1] << 16);
      rec[k * 4 + 1] = (uint32_t)c16[k * 4 + 2] | ((uint32_t)c16[k * 4 + 3] << 16);
      rec[k * 4 + 2] = nb;
      rec[k * 4 + 3] = 0u;
    }
    if ((e = hipMalloc(&cb->d_rec, sizeof(rec))) != hipSuccess ||
        (e = hipMemcpy(cb->d_rec, rec, sizeof(rec), hipMemcpyHostToDevice)) != hipSuccess ||
        (e = build_cells(cb)) != hipSuccess) {
      nsn_codebook_destroy(cb);
      return hip_fail(e, "codebook search tables");
    }
  }
  *out = cb;
  return ok();
}

int nsn_codebook_create_rht(const float* centroids, int g, int K, const uint8_t* sign_mask, nsn_codebook** out) {
  if (sign_mask == nullptr || out == nullptr) return set_error(NSN_EINVAL, "NULL argument");
  nsn_codebook* cb = nullptr;
  const int r = nsn_codebook_create(centroids, g, K, &cb);
  if (r != NSN_OK) return r;
  for (int w = 0; w < 4; ++w) {
    cb->sgn[w] = (uint32_t)sign_mask[4 * w] | ((uint32_t)sign_mask[4 * w + 1] << 8) |
                 ((uint32_t)sign_mask[4 * w + 2] << 16) | ((uint32_t)sign_mask[4 * w + 3] << 24);
    cb->rht = cb->rht || cb->sgn[w] != 0u;
  }
  *out = cb;
  return ok();
}

int nsn_codebook_sign_mask(const nsn_codebook* cb, uint8_t* sign_mask) {
  if (cb == nullptr || sign_mask == nullptr) return set_error(NSN_EINVAL, "NULL argument");
  for (int c = 0; c < 16; ++c) sign_mask[c] = (uint8_t)(cb->sgn[c / 4] >> (8 * (c % 4)));
  return ok();
}

void nsn_codebook_destroy(nsn_codebook* cb) {
  if (cb == nullptr) return;
  if (cb->d_c32) (void)hipFree(cb->d_c32);
  if (cb->d_c16) (void)hipFree(cb->d_c16);
  if (cb->d_encA) (void)hipFree(cb->d_encA);
  if (cb->d_encA16) (void)hipFree(cb->d_encA16);
  if (cb->d_rec) (void)hipFree(cb->d_rec);
  if (cb->d_c16x2) (void)hipFree(cb->d_c16x2);
  if (cb->d_cells) (void)hipFree(cb->d_cells);
  delete cb;
}

size_t nsn_encode_workspace_size(int B, int H, int L, int d) {
  if (B <= 0 || H <= 0 || L <= 0 || d != kD) return 0;
  return encode_ws_bytes(B * H, L);
}

int nsn_encode(const nsn_codebook* cb, const void* x, int x_dtype, int B, int H, int L, int L_cap, int pos0, int d,
               int o_mode, float* o, uint8_t* idx, uint16_t* scales, void* ws, size_t ws_bytes, void* stream) {
  int r = check_common(cb, B, H, L, L_cap, d);
  if (r != NSN_OK) return r;
  if (x == nullptr || o == nullptr || idx == nullptr || scales == nullptr) return set_error(NSN_EINVAL, "NULL tensor pointer");
  if (x_dtype != NSN_F16 && x_dtype != NSN_F32) return set_error(NSN_EINVAL, "x_dtype %d invalid", x_dtype);
  if (o_mode != NSN_O_COMPUTE && o_mode != NSN_O_REUSE) return set_error(NSN_EINVAL, "o_mode %d invalid", o_mode);
  if (pos0 < 0 || (long)pos0 + L > (long)L_cap) return set_error(NSN_EINVAL, "pos0 %d + L %d exceeds L_cap %d", pos0, L, L_cap);
  if (o_mode == NSN_O_COMPUTE) {  // o = the mean of these L tokens (at any pos0: a flushed block's own o)
    const size_t need = encode_ws_bytes(B * H, L);
    if (ws == nullptr || ws_bytes < need) return set_error(NSN_EWORKSPACE, "workspace %zu bytes < %zu", ws_bytes, need);
  }
  if ((r = check_device(cb)) != NSN_OK) return r;
  hipError_t e = launch_encode(cb, x, x_dtype, B * H, L, L_cap, pos0, o_mode, o, idx, scales, ws, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "nsn_encode launch");
  return ok();
}

int nsn_codebook_dq4(const float* centroids, int K, int g, uint8_t* codes, float* step, float* centroids_q) {
  if (centroids == nullptr || centroids_q == nullptr) return set_error(NSN_EINVAL, "NULL centroid array");
  if (K <= 0 || g <= 0 || (long)K * g > (1L << 24)) return set_error(NSN_EINVAL, "sizes K=%d g=%d invalid", K, g);
  double m = 0.0;
  for (long i = 0; i < (long)K * g; ++i) {
    if (!std::isfinite(centroids[i])) return set_error(NSN_EINVAL, "centroid entry %ld is not finite", i);
    m = std::max(m, std::fabs((double)centroids[i]));
  }
  const float D = (float)(m / 7.5);
  if (step != nullptr) *step = D;
  for (long i = 0; i < (long)K * g; ++i) {
    int k = 8;
    if (D > 0.f) k = (int)std::min(15.0, std::max(0.0, std::floor((double)centroids[i] / (double)D + 8.0)));
    if (codes != nullptr) codes[i] = (uint8_t)k;
    centroids_q[i] = D > 0.f ? (float)(_Float16)(((double)k - 7.5) * (double)D) : 0.f;  // nearest even
  }
  return ok();
}

size_t nsn_encode_dq_workspace_size(int B, int H, int L, int d) {
  if (B <= 0 || H <= 0 || L <= 0 || d != kD) return 0;
  return encode_dq_ws_bytes(B * H, L);
}

int nsn_encode_dq(const nsn_codebook* cb, const void* x, int x_dtype, int B, int H, int L, int L_cap, int pos0, int d,
                  int o_mode, nsn_dq_head* head, uint8_t* idx, uint16_t* s2, uint8_t* s1c, void* ws, size_t ws_bytes,
                  void* stream) {
  int r = check_common(cb, B, H, L, L_cap, d);
  if (r != NSN_OK) return r;
  if (x == nullptr || head == nullptr || idx == nullptr || s2 == nullptr || s1c == nullptr)
    return set_error(NSN_EINVAL, "NULL tensor pointer");
  if (x_dtype != NSN_F16 && x_dtype != NSN_F32) return set_error(NSN_EINVAL, "x_dtype %d invalid", x_dtype);
  if (o_mode != NSN_O_COMPUTE && o_mode != NSN_O_REUSE) return set_error(NSN_EINVAL, "o_mode %d invalid", o_mode);
  if (pos0 < 0 || (long)pos0 + L > (long)L_cap) return set_error(NSN_EINVAL, "pos0 %d + L %d exceeds L_cap %d", pos0, L, L_cap);
  if (o_mode == NSN_O_COMPUTE && pos0 != 0) return set_error(NSN_EINVAL, "o_mode COMPUTE needs pos0 == 0 (all tokens share o)");
  if ((long)B * H * L > (long)INT32_MAX / 4) return set_error(NSN_EUNSUPPORTED, "B*H*L exceeds 2^29");
  const size_t need = encode_dq_ws_bytes(B * H, L);
  if (ws == nullptr || ws_bytes < need) return set_error(NSN_EWORKSPACE, "workspace %zu bytes < %zu", ws_bytes, need);
  if ((r = check_device(cb)) != NSN_OK) return r;
  hipError_t e = launch_encode_dq(cb, x, x_dtype, B * H, L, L_cap, pos0, o_mode, head, idx, s2, s1c, ws,
                                  (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "nsn_encode_dq launch");
  return ok();
}

size_t nsn_decode_workspace_size(int B, int Hq, int Hkv, int S, int d) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || S < 0 || d != kD || Hq % Hkv) return 0;
  return decode_ws_bytes(B, Hq, Hkv, S);
}

// ws_kind: whose workspace size applies (the plain decode's, the pre-RoPE-key decode's
// with its tables, or that decode's partials alone when the tables come prepared).
enum WsKind { kWsDecode, kWsRope, kWsRopeTables };
static int check_decode(const nsn_codebook* cb, const void* q, int B, int Hq, int Hkv, int S, int S_cap, int d,
                        const void* k_idx, const void* k_scales, const void* k_o, const void* v_idx,
                        const void* v_scales, const void* v_o, const void* out, const void* ws, size_t ws_bytes,
                        WsKind ws_kind = kWsDecode, bool static_ws = false) {
  if (cb == nullptr) return set_error(NSN_EINVAL, "codebook handle is NULL");
  if (q == nullptr || k_idx == nullptr || k_scales == nullptr || k_o == nullptr || v_idx == nullptr ||
      v_scales == nullptr || v_o == nullptr || out == nullptr)
    return set_error(NSN_EINVAL, "NULL tensor pointer");
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || S <= 0 || S_cap <= 0)
    return set_error(NSN_EINVAL, "sizes must be positive (B=%d Hq=%d Hkv=%d S=%d S_cap=%d)", B, Hq, Hkv, S, S_cap);
  if (S > S_cap) return set_error(NSN_EINVAL, "S %d exceeds S_cap %d", S, S_cap);
  if (Hq % Hkv) return set_error(NSN_EINVAL, "Hq %d is not a multiple of Hkv %d", Hq, Hkv);
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return set_error(NSN_EUNSUPPORTED, "Hq/Hkv = %d unsupported (1,2,4,8)", G);
  if (d != kD) return set_error(NSN_EUNSUPPORTED, "head dimension %d unsupported (only %d)", d, kD);
  if ((long)B * Hkv * S_cap > (long)INT32_MAX) return set_error(NSN_EUNSUPPORTED, "B*Hkv*S_cap exceeds 2^31-1");
  if (B > 65535 || Hkv > 65535) return set_error(NSN_EUNSUPPORTED, "B or Hkv above 65535");
  const size_t need = ws_kind == kWsRope         ? decode_rope_ws_bytes(B, Hq, Hkv, S)
                      : ws_kind == kWsRopeTables ? decode_rope_tables_ws_bytes(B, Hq, Hkv, S)
                                                 : decode_ws_bytes(B, Hq, Hkv, S);
  if ((ws == nullptr && !static_ws) || ws_bytes < need)
    return set_error(NSN_EWORKSPACE, "workspace %zu bytes < %zu", ws_bytes, need);
  // the handle is read only after every check above has passed
  if (cb->g != 4 && cb->g != 8) return set_error(NSN_EUNSUPPORTED, "g=%d unsupported (4 or 8)", cb->g);
  // one (batch, KV head) slab of index rows is addressed with 32-bit byte offsets
  if ((long)S_cap * (kD / cb->g) > (long)INT32_MAX)
    return set_error(NSN_EUNSUPPORTED, "S_cap %d: index slab of %ld bytes exceeds 2^31-1", S_cap,
                     (long)S_cap * (kD / cb->g));
  return NSN_OK;
}

// Workspace of nsn_decode_attention_noalloc: a fixed array in device memory, one
// copy per device, held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it only stands in for the symbol); it
// takes the device address that hipGetSymbolAddress returns, looked up once per
// device with that device current.  The split-KV partials are written in full
// before they are read, so nothing in it needs clearing between calls.
constexpr size_t kNoAllocScratchBytes = size_t(4) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

static int scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return set_error(NSN_EUNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return NSN_OK;
}

int nsn_decode_attention_noalloc(const nsn_codebook* cb, const uint16_t* q, int B, int Hq, int Hkv, int S, int S_cap,
                                 int d, const uint8_t* k_idx, const uint16_t* k_scales, const float* k_o,
                                 const uint8_t* v_idx, const uint16_t* v_scales, const float* v_o, float* out,
                                 void* stream) {
  // every check of nsn_decode_attention, with the static array's size as the workspace
  // (its address is looked up only once the device is known to be the right one)
  int r = check_decode(cb, q, B, Hq, Hkv, S, S_cap, d, k_idx, k_scales, k_o, v_idx, v_scales, v_o, out, nullptr,
                       kNoAllocScratchBytes, kWsDecode, true);
  if (r == NSN_EWORKSPACE)
    return set_error(NSN_EWORKSPACE, "decode needs %zu bytes of workspace, more than the %zu of the static scratch "
                     "array (use nsn_decode_attention with a caller workspace)",
                     decode_ws_bytes(B, Hq, Hkv, S), kNoAllocScratchBytes);
  if (r != NSN_OK) return r;
  if ((r = check_device(cb)) != NSN_OK) return r;
  void* ws = nullptr;
  if ((r = scratch_address(cb->device, &ws)) != NSN_OK) return r;
  hipError_t e = launch_decode(cb, q, B, Hq, Hkv, S, S_cap, k_idx, k_scales, k_o, v_idx, v_scales, v_o, nullptr,
                               nullptr, 0, 0, out, ws, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "nsn_decode_attention_noalloc launch");
  return ok();
}

int nsn_decode_attention(const nsn_codebook* cb, const uint16_t* q, int B, int Hq, int Hkv, int S, int S_cap, int d,
                         const uint8_t* k_idx, const uint16_t* k_scales, const float* k_o, const uint8_t* v_idx,
                         const uint16_t* v_scales, const float* v_o, float* out, void* ws, size_t ws_bytes,
                         void* stream) {
  int r = check_decode(cb, q, B, Hq, Hkv, S, S_cap, d, k_idx, k_scales, k_o, v_idx, v_scales, v_o, out, ws, ws_bytes);
  if (r != NSN_OK) return r;
  if ((r = check_device(cb)) != NSN_OK) return r;
  hipError_t e = launch_decode(cb, q, B, Hq, Hkv, S, S_cap, k_idx, k_scales, k_o, v_idx, v_scales, v_o, nullptr,
                               nullptr, 0, 0, out, ws, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "nsn_decode_attention launch");
  return ok();
}

/* Checks of nsn_decode_attention_residual: the quantized part as in
 * nsn_decode_attention when S > 0 (nothing of it is read when S = 0), plus the
 * residual window. */
static int check_residual(const nsn_codebook* cb, const void* q, int B, int Hq, int Hkv, int S, int S_cap, int d,
                          const void* k_idx, const void* k_scales, const void* k_o, const void* v_idx,
                          const void* v_scales, const void* v_o, const void* k_res, const void* v_res, int R,
                          int R_cap, const void* out, const void* ws, size_t ws_bytes) {
  if (cb == nullptr) return set_error(NSN_EINVAL, "codebook handle is NULL");
  if (S < 0 || R < 0) return set_error(NSN_EINVAL, "S %d and R %d must not be negative", S, R);
  if (S + (long)R < 1) return set_error(NSN_EINVAL, "no token to attend to (S = R = 0)");
  if (R_cap <= 0 || R > R_cap) return set_error(NSN_EINVAL, "R %d outside residual capacity R_cap %d", R, R_cap);
  if (R > 0 && (k_res == nullptr || v_res == nullptr)) return set_error(NSN_EINVAL, "NULL residual pointer");
  if (S > 0)
    return check_decode(cb, q, B, Hq, Hkv, S, S_cap, d, k_idx, k_scales, k_o, v_idx, v_scales, v_o, out, ws, ws_bytes);
  if (q == nullptr || out == nullptr) return set_error(NSN_EINVAL, "NULL tensor pointer");
  if (B <= 0 || Hq <= 0 || Hkv <= 0) return set_error(NSN_EINVAL, "sizes must be positive (B=%d Hq=%d Hkv=%d)", B, Hq, Hkv);
  if (Hq % Hkv) return set_error(NSN_EINVAL, "Hq %d is not a multiple of Hkv %d", Hq, Hkv);
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return set_error(NSN_EUNSUPPORTED, "Hq/Hkv = %d unsupported (1,2,4,8)", G);
  if (d != kD) return set_error(NSN_EUNSUPPORTED, "head dimension %d unsupported (only %d)", d, kD);
  if ((long)B * Hq > (long)INT32_MAX) return set_error(NSN_EUNSUPPORTED, "B*Hq exceeds 2^31-1");
  const size_t need = decode_ws_bytes(B, Hq, Hkv, 0);  // the window's partials
  if (R > 0 && (ws == nullptr || ws_bytes < need))
    return set_error(NSN_EWORKSPACE, "workspace %zu bytes < %zu", ws_bytes, need);
  return NSN_OK;
}

int nsn_decode_attention_residual(const nsn_codebook* cb, const uint16_t* q, int B, int Hq, int Hkv, int S, int S_cap,
                                  int d, const uint8_t* k_idx, const uint16_t* k_scales, const float* k_o,
                                  const uint8_t* v_idx, const uint16_t* v_scales, const float* v_o,
                                  const uint16_t* k_res, const uint16_t* v_res, int R, int R_cap, float* out, void* ws,
                                  size_t ws_bytes, void* stream) {
  int r = check_residual(cb, q, B, Hq, Hkv, S, S_cap, d, k_idx, k_scales, k_o, v_idx, v_scales, v_o, k_res, v_res, R,
                         R_cap, out, ws, ws_bytes);
  if (r != NSN_OK) return r;
  if ((r = check_device(cb)) != NSN_OK) return r;
  hipError_t e = launch_decode(cb, q, B, Hq, Hkv, S, S_cap, k_idx, k_scales, k_o, v_idx, v_scales, v_o, k_res, v_res,
                               R, R_cap, out, ws, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "nsn_decode_attention_residual launch");
  return ok();
}

size_t nsn_decode_blocks_workspace_size(int B, int Hq, int Hkv, int S0, int nblk, int d) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || S0 < 0 || nblk < 0 || d != kD || Hq % Hkv) return 0;
  return decode_blocks_ws_bytes(B, Hq, Hkv, S0, nblk);
}

/* Checks of nsn_decode_attention_blocks (host only, the handle is read last). */
static int check_blocks(const nsn_codebook* cb, const void* q, int B, int Hq, int Hkv, int S0, int nblk, int Rb,
                        int nblk_cap, int S_cap, int d, const void* k_idx, const void* k_scales, const void* k_o,
                        const void* k_ob, const void* v_idx, const void* v_scales, const void* v_o, const void* v_ob,
                        const void* k_res, const void* v_res, int R, int R_cap, const void* out, const void* ws,
                        size_t ws_bytes) {
  if (cb == nullptr) return set_error(NSN_EINVAL, "codebook handle is NULL");
  if (S0 < 0 || nblk < 0 || R < 0) return set_error(NSN_EINVAL, "S0 %d, nblk %d and R %d must not be negative", S0, nblk, R);
  if (nblk > 0 && (Rb < 1 || nblk > nblk_cap))
    return set_error(NSN_EINVAL, "nblk %d blocks of Rb %d tokens need Rb >= 1 and nblk <= nblk_cap %d", nblk, Rb,
                     nblk_cap);
  const long S = (long)S0 + (long)nblk * (nblk > 0 ? Rb : 0);
  if (S + R < 1) return set_error(NSN_EINVAL, "no token to attend to");
  if (S > S_cap) return set_error(NSN_EINVAL, "S0 + nblk * Rb = %ld exceeds S_cap %d", S, S_cap);
  if (R > 0 && (k_res == nullptr || v_res == nullptr || R > R_cap))
    return set_error(NSN_EINVAL, "residual window: NULL rows or R %d above R_cap %d", R, R_cap);
  if (q == nullptr || out == nullptr) return set_error(NSN_EINVAL, "NULL tensor pointer");
  if (S > 0 && (k_idx == nullptr || k_scales == nullptr || v_idx == nullptr || v_scales == nullptr))
    return set_error(NSN_EINVAL, "NULL cache pointer");
  if (S0 > 0 && (k_o == nullptr || v_o == nullptr)) return set_error(NSN_EINVAL, "NULL o of the prefix");
  if (nblk > 0 && (k_ob == nullptr || v_ob == nullptr)) return set_error(NSN_EINVAL, "NULL block o table");
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || (S > 0 && S_cap <= 0))
    return set_error(NSN_EINVAL, "sizes must be positive (B=%d Hq=%d Hkv=%d S_cap=%d)", B, Hq, Hkv, S_cap);
  if (Hq % Hkv) return set_error(NSN_EINVAL, "Hq %d is not a multiple of Hkv %d", Hq, Hkv);
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return set_error(NSN_EUNSUPPORTED, "Hq/Hkv = %d unsupported (1,2,4,8)", G);
  if (d != kD) return set_error(NSN_EUNSUPPORTED, "head dimension %d unsupported (only %d)", d, kD);
  if ((long)B * Hkv * (long)std::max(S_cap, 1) > (long)INT32_MAX || (long)B * Hq > (long)INT32_MAX)
    return set_error(NSN_EUNSUPPORTED, "B*Hkv*S_cap exceeds 2^31-1");
  if ((long)nblk_cap * B * Hkv * kD > (long)INT32_MAX * 4L) return set_error(NSN_EUNSUPPORTED, "block o table too large");
  if (B > 65535 || Hkv > 65535) return set_error(NSN_EUNSUPPORTED, "B or Hkv above 65535");
  const size_t need = decode_blocks_ws_bytes(B, Hq, Hkv, S0, nblk);
  if (ws == nullptr || ws_bytes < need) return set_error(NSN_EWORKSPACE, "workspace %zu bytes < %zu", ws_bytes, need);
  if (cb->g != 4 && cb->g != 8) return set_error(NSN_EUNSUPPORTED, "g=%d unsupported (4 or 8)", cb->g);
  if ((long)S_cap * (kD / cb->g) > (long)INT32_MAX)
    return set_error(NSN_EUNSUPPORTED, "S_cap %d: index slab exceeds 2^31-1 bytes", S_cap);
  return NSN_OK;
}

int nsn_decode_attention_blocks(const nsn_codebook* cb, const uint16_t* q, int B, int Hq, int Hkv, int S0, int nblk,
                                int Rb, int nblk_cap, int S_cap, int d, const uint8_t* k_idx, const uint16_t* k_scales,
                                const float* k_o, const float* k_ob, const uint8_t* v_idx, const uint16_t* v_scales,
                                const float* v_o, const float* v_ob, const uint16_t* k_res, const uint16_t* v_res,
                                int R, int R_cap, float* out, void* ws, size_t ws_bytes, void* stream) {
  int r = check_blocks(cb, q, B, Hq, Hkv, S0, nblk, Rb, nblk_cap, S_cap, d, k_idx, k_scales, k_o, k_ob, v_idx, v_scales,
                       v_o, v_ob, k_res, v_res, R, R_cap, out, ws, ws_bytes);
  if (r != NSN_OK) return r;
  if ((r = check_device(cb)) != NSN_OK) return r;
  hipError_t e = launch_decode_blocks(cb, q, B, Hq, Hkv, S0, nblk, Rb, S_cap, k_idx, k_scales, k_o, k_ob, v_idx,
                                      v_scales, v_o, v_ob, k_res, v_res, R, R_cap, out, ws, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "nsn_decode_attention_blocks launch");
  return ok();
}

/* Host-only argument check of nsn_decode_attention_blocks. */
int nsn_check_decode_blocks_args(int g, const void* q, int B, int Hq, int Hkv, int S0, int nblk, int Rb, int nblk_cap,
                                 int S_cap, int d, const void* k_idx, const void* k_scales, const void* k_o,
                                 const void* k_ob, const void* v_idx, const void* v_scales, const void* v_o,
                                 const void* v_ob, const void* k_res, const void* v_res, int R, int R_cap,
                                 const void* out, const void* ws, size_t ws_bytes) {
  nsn_codebook fake;
  fake.g = g;
  fake.K = kK;
  const int r = check_blocks(&fake, q, B, Hq, Hkv, S0, nblk, Rb, nblk_cap, S_cap, d, k_idx, k_scales, k_o, k_ob, v_idx,
                             v_scales, v_o, v_ob, k_res, v_res, R, R_cap, out, ws, ws_bytes);
  return r == NSN_OK ? ok() : r;
}

int nsn_decode_attention_dq(const nsn_codebook* cb, const uint16_t* q, int B, int Hq, int Hkv, int S, int S_cap,
                            int d, const uint8_t* k_idx, const uint16_t* k_s2, const uint8_t* k_s1c,
                            const nsn_dq_head* k_head, const uint8_t* v_idx, const uint16_t* v_s2,
                            const uint8_t* v_s1c, const nsn_dq_head* v_head, float* out, void* ws, size_t ws_bytes,
                            void* stream) {
  if (k_s1c == nullptr || v_s1c == nullptr) return set_error(NSN_EINVAL, "NULL s1 code array");
  int r = check_decode(cb, q, B, Hq, Hkv, S, S_cap, d, k_idx, k_s2, k_head, v_idx, v_s2, v_head, out, ws, ws_bytes);
  if (r != NSN_OK) return r;
  if ((r = check_device(cb)) != NSN_OK) return r;
  hipError_t e = launch_decode(cb, q, B, Hq, Hkv, S, S_cap, k_idx, k_s2, nullptr, v_idx, v_s2, nullptr, nullptr,
                               nullptr, 0, 0, out, ws, (hipStream_t)stream, k_s1c, v_s1c, k_head, v_head);
  if (e != hipSuccess) return hip_fail(e, "nsn_decode_attention_dq launch");
  return ok();
}

size_t nsn_decode_rope_workspace_size(int B, int Hq, int Hkv, int S, int d) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || S <= 0 || d != kD || Hq % Hkv) return 0;
  return decode_rope_ws_bytes(B, Hq, Hkv, S);
}

int nsn_decode_attention_rope(const nsn_codebook* cb, const uint16_t* q, int B, int Hq, int Hkv, int S, int S_cap,
                              int d, double rope_base, const uint8_t* k_idx, const uint16_t* k_scales,
                              const float* k_o, const uint8_t* v_idx, const uint16_t* v_scales, const float* v_o,
                              float* out, void* ws, size_t ws_bytes, void* stream) {
  if (!std::isfinite(rope_base) || rope_base <= 1.0) return set_error(NSN_EINVAL, "rope_base %g must exceed 1", rope_base);
  int r = check_decode(cb, q, B, Hq, Hkv, S, S_cap, d, k_idx, k_scales, k_o, v_idx, v_scales, v_o, out, ws, ws_bytes,
                       kWsRope);
  if (r != NSN_OK) return r;
  if ((r = check_device(cb)) != NSN_OK) return r;
  hipError_t e = launch_decode_rope(cb, q, B, Hq, Hkv, S, S_cap, rope_base, k_idx, k_scales, k_o, v_idx, v_scales, v_o,
                                    out, ws, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "nsn_decode_attention_rope launch");
  return ok();
}

size_t nsn_rope_tables_size(int S_tab) { return S_tab <= 0 ? 0 : rope_table_bytes(S_tab); }

int nsn_rope_tables(double rope_base, int S_tab, void* tables, size_t bytes, void* stream) {
  if (!std::isfinite(rope_base) || rope_base <= 1.0) return set_error(NSN_EINVAL, "rope_base %g must exceed 1", rope_base);
  if (S_tab <= 0) return set_error(NSN_EINVAL, "S_tab %d must be positive", S_tab);
  if (tables == nullptr) return set_error(NSN_EINVAL, "tables pointer is NULL");
  if (reinterpret_cast<uintptr_t>(tables) & 15) return set_error(NSN_EINVAL, "tables not 16-byte aligned");
  const size_t need = rope_table_bytes(S_tab);
  if (bytes < need) return set_error(NSN_EINVAL, "tables buffer %zu bytes < %zu", bytes, need);
  const hipError_t e = launch_rope_tables(rope_base, S_tab, tables, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "nsn_rope_tables launch");
  return ok();
}

size_t nsn_decode_rope_tables_workspace_size(int B, int Hq, int Hkv, int S, int d) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || S <= 0 || d != kD || Hq % Hkv) return 0;
  return decode_rope_tables_ws_bytes(B, Hq, Hkv, S);
}

int nsn_decode_attention_rope_tables(const nsn_codebook* cb, const uint16_t* q, int B, int Hq, int Hkv, int S,
                                     int S_cap, int d, const void* tables, int S_tab, const uint8_t* k_idx,
                                     const uint16_t* k_scales, const float* k_o, const uint8_t* v_idx,
                                     const uint16_t* v_scales, const float* v_o, float* out, void* ws,
                                     size_t ws_bytes, void* stream) {
  if (tables == nullptr) return set_error(NSN_EINVAL, "tables pointer is NULL");
  if (reinterpret_cast<uintptr_t>(tables) & 15) return set_error(NSN_EINVAL, "tables not 16-byte aligned");
  if (S_tab <= 0) return set_error(NSN_EINVAL, "S_tab %d must be positive", S_tab);
  if (S > S_tab) return set_error(NSN_EINVAL, "S %d exceeds the %d positions of the tables", S, S_tab);
  int r = check_decode(cb, q, B, Hq, Hkv, S, S_cap, d, k_idx, k_scales, k_o, v_idx, v_scales, v_o, out, ws, ws_bytes,
                       kWsRopeTables);
  if (r != NSN_OK) return r;
  if ((r = check_device(cb)) != NSN_OK) return r;
  const hipError_t e = launch_decode_rope_tables(cb, q, B, Hq, Hkv, S, S_cap, tables, S_tab, k_idx, k_scales, k_o,
                                                 v_idx, v_scales, v_o, out, ws, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "nsn_decode_attention_rope_tables launch");
  return ok();
}

int nsn_decode_step(const nsn_codebook* cb, const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new, int B,
                    int Hq, int Hkv, int S, int S_cap, int d, uint8_t* k_idx, uint16_t* k_scales, const float* k_o,
                    uint8_t* v_idx, uint16_t* v_scales, const float* v_o, float* out, void* ws, size_t ws_bytes,
                    void* stream) {
  if (k_new == nullptr || v_new == nullptr) return set_error(NSN_EINVAL, "NULL new-token pointer");
  if (S < 0) return set_error(NSN_EINVAL, "S %d negative", S);
  int r = check_decode(cb, q, B, Hq, Hkv, S + 1, S_cap, d, k_idx, k_scales, k_o, v_idx, v_scales, v_o, out, ws, ws_bytes);
  if (r != NSN_OK) return r;
  hipStream_t st = (hipStream_t)stream;
  if ((r = check_device(cb)) != NSN_OK) return r;
  const hipError_t e = launch_decode_step(cb, q, k_new, v_new, B, Hq, Hkv, S, S_cap, k_idx, k_scales, k_o, v_idx,
                                          v_scales, v_o, out, ws, st);
  if (e != hipSuccess) return hip_fail(e, "nsn_decode_step");
  return ok();
}

int nsn_dequantize(const nsn_codebook* cb, const uint8_t* idx, const uint16_t* scales, const float* o, int B, int H,
                   int L, int L_cap, int d, float* x_hat, void* stream) {
  int r = check_common(cb, B, H, L, L_cap, d);
  if (r != NSN_OK) return r;
  if (idx == nullptr || scales == nullptr || o == nullptr || x_hat == nullptr) return set_error(NSN_EINVAL, "NULL tensor pointer");
  if (L > L_cap) return set_error(NSN_EINVAL, "L %d exceeds L_cap %d", L, L_cap);
  if ((r = check_device(cb)) != NSN_OK) return r;
  hipError_t e = launch_dequantize(cb, idx, scales, o, B * H, L, L_cap, x_hat, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "nsn_dequantize launch");
  return ok();
}

/* Host-only argument check of nsn_encode with a codebook of sub-vector length g
 * (no handle needed): lets the validation be exercised without a device. */
int nsn_check_encode_args(int g, const void* x, int x_dtype, int B, int H, int L, int L_cap, int pos0, int d,
                          int o_mode, const void* o, const void* idx, const void* scales, const void* ws,
                          size_t ws_bytes) {
  nsn_codebook fake;
  fake.g = g;
  fake.K = kK;
  if (g != 4 && g != 8) return set_error(NSN_EUNSUPPORTED, "g=%d unsupported (4 or 8)", g);
  int r = check_common(&fake, B, H, L, L_cap, d);
  if (r != NSN_OK) return r;
  if (x == nullptr || o == nullptr || idx == nullptr || scales == nullptr) return set_error(NSN_EINVAL, "NULL tensor pointer");
  if (x_dtype != NSN_F16 && x_dtype != NSN_F32) return set_error(NSN_EINVAL, "x_dtype %d invalid", x_dtype);
  if (o_mode != NSN_O_COMPUTE && o_mode != NSN_O_REUSE) return set_error(NSN_EINVAL, "o_mode %d invalid", o_mode);
  if (pos0 < 0 || (long)pos0 + L > (long)L_cap) return set_error(NSN_EINVAL, "pos0 %d + L %d exceeds L_cap %d", pos0, L, L_cap);
  if (o_mode == NSN_O_COMPUTE) {
    const size_t need = encode_ws_bytes(B * H, L);
    if (ws == nullptr || ws_bytes < need) return set_error(NSN_EWORKSPACE, "workspace %zu bytes < %zu", ws_bytes, need);
  }
  return ok();
}

/* Host-only argument check of nsn_decode_attention (see nsn_check_encode_args). */
int nsn_check_decode_args(int g, const void* q, int B, int Hq, int Hkv, int S, int S_cap, int d, const void* k_idx,
                          const void* k_scales, const void* k_o, const void* v_idx, const void* v_scales,
                          const void* v_o, const void* out, const void* ws, size_t ws_bytes) {
  nsn_codebook fake;
  fake.g = g;
  fake.K = kK;
  const int r = check_decode(&fake, q, B, Hq, Hkv, S, S_cap, d, k_idx, k_scales, k_o, v_idx, v_scales, v_o, out, ws,
                             ws_bytes);
  return r == NSN_OK ? ok() : r;
}

/* Host-only argument check of nsn_decode_attention_residual. */
int nsn_check_decode_residual_args(int g, const void* q, int B, int Hq, int Hkv, int S, int S_cap, int d,
                                   const void* k_idx, const void* k_scales, const void* k_o, const void* v_idx,
                                   const void* v_scales, const void* v_o, const void* k_res, const void* v_res, int R,
                                   int R_cap, const void* out, const void* ws, size_t ws_bytes) {
  nsn_codebook fake;
  fake.g = g;
  fake.K = kK;
  const int r = check_residual(&fake, q, B, Hq, Hkv, S, S_cap, d, k_idx, k_scales, k_o, v_idx, v_scales, v_o, k_res,
                               v_res, R, R_cap, out, ws, ws_bytes);
  return r == NSN_OK ? ok() : r;
}

}  // extern "C"
