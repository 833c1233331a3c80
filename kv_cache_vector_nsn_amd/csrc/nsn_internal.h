// Internal declarations of the NSNQuant gfx950 library (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "../../include/nsn.h"

namespace nsn {

constexpr int kD = 128;        // head dimension
constexpr int kK = 256;        // codebook entries
constexpr int kTiles = 8;      // 32-centroid MFMA tiles in the encode distance GEMM
constexpr float kEpsZ = 1e-4f; // ||z|| <= kEpsZ*sqrt(d): the shifted token counts as zero

// Candidate grid of the exact pruned search for 4-dim sub-vectors: kGridN^4 cells
// of side kGridStep tile [-kGridR, kGridR]^4.  A cell keeps every centroid that is
// nearest to some point of the cell (enlarged by kGridMargin): a centroid is
// dropped only when one other centroid is strictly closer on the whole cell.
constexpr int kGridN = 20;
constexpr float kGridStep = 0.4f;
constexpr float kGridR = 4.0f;                 // kGridN * kGridStep / 2
constexpr float kGridInv = 2.5f;               // 1 / kGridStep (exact)
constexpr float kGridOff = 10.0f;              // kGridR / kGridStep
constexpr double kGridMargin = 1e-4;           // cell enlargement, absorbs the fp32 cell-index rounding
constexpr int kGridCells = kGridN * kGridN * kGridN * kGridN;
constexpr int kCellList = 12;                  // candidates stored per cell (bytes 0..11 of a 16-byte row)

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// Status helpers (nsn_api.cpp).  Each returns `code`.
int set_error(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int hip_fail(hipError_t e, const char* what);

}  // namespace nsn

// Codebook handle.  Immutable after nsn_codebook_create.
struct nsn_codebook {
  int g = 0;
  int K = 0;
  int device = 0;
  int num_cu = 256;              // compute units of that device (persistent encode grid)
  float host[nsn::kK * 8];       // centroids, fp16-exact fp32, [K][g]
  float* d_c32 = nullptr;        // device copy, fp32 [K][g]
  uint16_t* d_c16 = nullptr;     // device copy, fp16 bits [K][g]
  uint16_t* d_encA = nullptr;    // encode MFMA A fragments [tile][2][64 lanes][8] fp16 bits
  uint16_t* d_encA16 = nullptr;  // g = 8 only: 16x16x32 A fragments [16 tiles][64 lanes][8] fp16 bits
  uint16_t* d_c16x2 = nullptr;   // [K] 16-byte rows: the fp16 entry (g = 4: twice) -- decode table source
  uint32_t sgn[4] = {0, 0, 0, 0};  // randomized Hadamard: channel c negated <=> bit c % 32 of sgn[c / 32]
  bool rht = false;                // some channel is negated
  // g = 4 only: pruned-search tables
  uint4* d_rec = nullptr;        // [K] {c0|c1, c2|c3 fp16 bits, ||c||^2 fp32 bits, 0}
  uint4* d_cells = nullptr;      // [kGridCells] candidate rows: bytes 0..11 centroid indices
                                 // (ascending, padded with the last), byte 12 count, byte 15 overflow flag
  int cell_max = 0;              // longest candidate list over all cells
  int cell_overflow = 0;         // cells whose list exceeds kCellList (searched exhaustively)
};

namespace nsn {

// Launchers (device code files).  All validate nothing: callers checked sizes.
hipError_t launch_encode(const nsn_codebook* cb, const void* x, int x_dtype, int BH, int L, int L_cap,
                         int pos0, int o_mode, float* o, uint8_t* idx, uint16_t* scales, void* ws,
                         hipStream_t st);
size_t encode_ws_bytes(int BH, int L);
hipError_t launch_encode_dq(const nsn_codebook* cb, const void* x, int x_dtype, int BH, int L, int L_cap,
                            int pos0, int o_mode, nsn_dq_head* heads, uint8_t* idx, uint16_t* s2, uint8_t* s1c,
                            void* ws, hipStream_t st);
size_t encode_dq_ws_bytes(int BH, int L);
static_assert(sizeof(nsn_dq_head) == 80, "nsn_dq_head is 80 bytes");

hipError_t launch_decode(const nsn_codebook* cb, const uint16_t* q, int B, int Hq, int Hkv, int S,
                         int S_cap, const uint8_t* k_idx, const uint16_t* k_scales, const float* k_o,
                         const uint8_t* v_idx, const uint16_t* v_scales, const float* v_o,
                         const uint16_t* k_res, const uint16_t* v_res, int R, int R_cap, float* out,
                         void* ws, hipStream_t st, const uint8_t* k_nib = nullptr,
                         const uint8_t* v_nib = nullptr, const nsn_dq_head* k_hd = nullptr,
                         const nsn_dq_head* v_hd = nullptr);
size_t decode_ws_bytes(int B, int Hq, int Hkv, int S);
hipError_t launch_decode_blocks(const nsn_codebook* cb, const uint16_t* q, int B, int Hq, int Hkv, int S0, int nblk,
                                int Rb, int S_cap, const uint8_t* k_idx, const uint16_t* k_scales, const float* k_o,
                                const float* k_ob, const uint8_t* v_idx, const uint16_t* v_scales, const float* v_o,
                                const float* v_ob, const uint16_t* k_res, const uint16_t* v_res, int R, int R_cap,
                                float* out, void* ws, hipStream_t st);
size_t decode_blocks_ws_bytes(int B, int Hq, int Hkv, int S0, int nblk);
hipError_t launch_decode_rope(const nsn_codebook* cb, const uint16_t* q, int B, int Hq, int Hkv, int S, int S_cap,
                              double rope_base, const uint8_t* k_idx, const uint16_t* k_scales, const float* k_o,
                              const uint8_t* v_idx, const uint16_t* v_scales, const float* v_o, float* out, void* ws,
                              hipStream_t st);
size_t decode_rope_ws_bytes(int B, int Hq, int Hkv, int S);
size_t rope_table_bytes(int S);
hipError_t launch_rope_tables(double rope_base, int S, void* tables, hipStream_t st);
hipError_t launch_decode_rope_tables(const nsn_codebook* cb, const uint16_t* q, int B, int Hq, int Hkv, int S,
                                     int S_cap, const void* tables, int S_tab, const uint8_t* k_idx,
                                     const uint16_t* k_scales, const float* k_o, const uint8_t* v_idx,
                                     const uint16_t* v_scales, const float* v_o, float* out, void* ws,
                                     hipStream_t st);
size_t decode_rope_tables_ws_bytes(int B, int Hq, int Hkv, int S);

hipError_t launch_dequantize(const nsn_codebook* cb, const uint8_t* idx, const uint16_t* scales,
                             const float* o, int BH, int L, int L_cap, float* x_hat, hipStream_t st);

// nsn_decode_step: the new token's K and V are encoded (with the stored o) and
// appended at slot S by the decode kernel itself, which attends over S + 1 tokens.
hipError_t launch_decode_step(const nsn_codebook* cb, const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                              int B, int Hq, int Hkv, int S, int S_cap, uint8_t* k_idx, uint16_t* k_scales,
                              const float* k_o, uint8_t* v_idx, uint16_t* v_scales, const float* v_o, float* out,
                              void* ws, hipStream_t st);

// Candidate rows of the pruned g = 4 search (fp64, on the device); fills
// cb->d_cells, cb->cell_max and cb->cell_overflow.  Synchronous.
hipError_t build_cells(nsn_codebook* cb);

int finetune_codebook_device(const float* cin, int g, int K, uint64_t seed, int64_t nvec, int iters, double lr,
                             float* cout, double* raw, double* cos_dist);
int build_codebook_device(uint64_t seed, int g, int K, int64_t n, int max_iters, float* centroids,
                          double* distortion, int* iterations);

}  // namespace nsn
