/*
 * nsn.h -- C ABI of the NSNQuant KV-cache quantizer for AMD Instinct MI355X (gfx950).
 *
 * The operations follow the Technical Summary of the explainer "NSNQuant: A
 * Double Normalization Approach for Calibration-Free Low-Bit Vector
 * Quantization of KV Cache" (gist.science/paper/2505.18231):
 *   [NSN]  section "1. Normalize-Shift-Normalize (NSN)"
 *   [HAD]  section "2. Hadamard Transform"
 *   [VQ]   section "3. Vector Quantization and Codebook"
 *   [IMPL] section "4. Implementation Details"
 *
 * Conventions shared by every call
 *   - Every call returns an int status (enum nsn_status); no exception or
 *     signal crosses the ABI.  After a non-OK return, nsn_last_error() gives a
 *     thread-local description.
 *   - Arguments are validated on the host before any HIP call, so a
 *     validation failure never touches the device.
 *   - Device pointers are caller-owned device memory (e.g. torch tensors);
 *     the library never allocates or frees caller memory.  Host pointers are
 *     marked "host".  The only calls that allocate device memory themselves are
 *     nsn_codebook_create / nsn_codebook_create_rht (released by
 *     nsn_codebook_destroy) and nsn_build_codebook (releases before
 *     returning).
 *   - A codebook handle belongs to the device that was current when it was
 *     created; every call that launches work with it returns NSN_EINVAL when
 *     another device is current.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls that take a stream only enqueue work on it and return without
 *     synchronizing; device-side faults surface at the caller's next sync.
 *   - Head dimension d is 128.  Sub-vector length g is 4 (2 bits per element)
 *     or 8 (1 bit per element) with a K = 256 entry codebook, so every
 *     sub-vector index is one byte.  m = d / g indices per token.
 *   - Results are bitwise reproducible for identical inputs and shapes (all
 *     reductions run in a fixed order; no floating-point atomics).
 *   - Non-finite inputs give unspecified (but in-bounds) results.
 *   - Size limits (NSN_EUNSUPPORTED beyond them): B*H*L_cap and B*Hkv*S_cap at
 *     most 2^31-1; B*H at most 65535 for the encode and dequantize calls; B and
 *     Hkv at most 65535 and S_cap*m at most 2^31-1 bytes (S_cap <= 2^26 at
 *     g = 4, 2^27 at g = 8) for the decode calls.
 *
 * Cache layout (per K or V tensor), all row-major and contiguous:
 *   idx    uint8  [B][H][L_cap][m]   sub-vector codebook indices
 *   scales fp16   [B][H][L_cap][2]   (s1, s2') per token: x_hat = s1 (s2' H w_hat + o)
 *   o      fp32   [B][H][d]          channel mean of the token-normalized tensor
 */
#ifndef NSN_H_
#define NSN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum nsn_status {
  NSN_OK = 0,
  NSN_EINVAL = -1,        /* a null pointer, a non-positive or inconsistent size */
  NSN_EUNSUPPORTED = -2,  /* a valid request outside what is built (d != 128, g, K) */
  NSN_EWORKSPACE = -3,    /* workspace missing or smaller than the queried size */
  NSN_EHIP = -4,          /* a HIP runtime call failed (text in nsn_last_error) */
  NSN_ENOMEM = -5         /* a device or host allocation failed */
};

enum nsn_dtype { NSN_F16 = 0, NSN_F32 = 1 };
enum nsn_o_mode { NSN_O_COMPUTE = 0, NSN_O_REUSE = 1 };

typedef struct nsn_codebook nsn_codebook; /* opaque, immutable once created */

/* Library ABI version (major * 10000 + minor * 100 + patch). */
int nsn_version(void);

/* Text of the last non-OK status returned on this thread ("" if none). */
const char* nsn_last_error(void);

/*
 * [VQ] "Codebook Construction": one global codebook fitted by k-means to
 * synthetic N(0,1) data, built on the GPU (device 0 of the calling thread).
 *   seed          SplitMix64 seed of the sample stream; sample i is the g
 *                 standard normals i*g .. i*g+g-1 of a Box-Muller stream whose
 *                 pair p uses SplitMix64 outputs 2p and 2p+1.
 *   g, K          sub-vector length (4 or 8) and codebook size (256).
 *   n_samples     number of g-dim samples (>= K).
 *   max_iters     Lloyd iteration cap (>= 1).  Initial centroids are the first
 *                 K samples; an iteration assigns every sample to its nearest
 *                 centroid (lowest index on ties) and stops when no assignment
 *                 changed; otherwise centroids move to their cell means, and
 *                 empty cells take, in increasing index, the samples farthest
 *                 from their centroid.  Arithmetic is fp64.
 *   centroids     host [K][g] fp32, written with the fp16-rounded centroids.
 *   distortion    host, optional: mean over samples of min_k ||x - C_k||^2 / g
 *                 for the rounded codebook.
 *   iterations    host, optional: Lloyd iterations run.
 * Synchronous; allocates and frees its own device buffers (about
 * n_samples * g * 8 bytes plus small per-block partials).
 * Errors: NSN_EINVAL, NSN_EUNSUPPORTED, NSN_ENOMEM, NSN_EHIP.
 */
int nsn_build_codebook(uint64_t seed, int g, int K, int64_t n_samples, int max_iters,
                       float* centroids, double* distortion, int* iterations);

/*
 * [VQ] "Codebook Construction", second step: fine-tune a codebook to minimise
 * the mean cosine distance between d = 128 N(0,1) vectors and their
 * quantization (each contiguous g-block replaced by its nearest centroid), on
 * the GPU in fp64.  Vector i is the normals 128 i .. 128 i + 127 of the stream of
 * nsn_build_codebook with `seed`.  Each of `iters` iterations assigns every
 * block to its nearest centroid (lowest index on ties), then takes one
 * full-batch gradient step C <- C - lr * dL/dC of L = mean (1 - cos(w, w_hat))
 * with that assignment held fixed.
 *   centroids_in   host [K][g] fp32 (typically from nsn_build_codebook).
 *   n_vectors      1 .. 2^22 training vectors; iters >= 0; lr >= 0.
 *   centroids_out  host [K][g] fp32, the result rounded to fp16 (nearest even).
 *   centroids_raw  host [K][g] fp64 or NULL: the result before rounding.
 *   cos_dist       host double[iters + 1] or NULL: L before each step, then L of
 *                  the rounded result.
 * Synchronous; allocates and frees its own device buffers (about
 * n_vectors * 1.1 KiB).  Errors: NSN_EINVAL, NSN_EUNSUPPORTED, NSN_ENOMEM, NSN_EHIP.
 */
int nsn_finetune_codebook(const float* centroids_in, int g, int K, uint64_t seed, int64_t n_vectors,
                          int iters, double lr, float* centroids_out, double* centroids_raw,
                          double* cos_dist);

/*
 * Upload a codebook ([VQ] "single global codebook").
 *   centroids  host [K][g] fp32; every entry must be exactly representable in
 *              fp16 (the matrix-core kernels use it as an exact fp16 operand),
 *              else NSN_EINVAL.
 *   out        host, receives the handle.  The handle owns device memory on the
 *              current device (a few KiB; for g = 4 also the 2.5 MiB candidate
 *              grid of the pruned nearest-centroid search, built here in fp64
 *              on the device); destroy it with nsn_codebook_destroy.
 * Synchronous.  Errors: NSN_EINVAL, NSN_EUNSUPPORTED (g not 4/8, K != 256),
 * NSN_ENOMEM, NSN_EHIP.
 */
int nsn_codebook_create(const float* centroids, int g, int K, nsn_codebook** out);

/*
 * Upload a codebook for the randomized Hadamard transform ([HAD]: the random-
 * sign transform named there for its guarantee that the rotated channels have
 * variance close to 1; the plain transform above is the one the method uses).
 * Every call that takes this handle rotates by H D instead of H, with
 * D = diag(+-1): the encode quantizes w = H D u, and dequantization and decode
 * attention rebuild x_hat = s1 (s2' D H w_hat + o).  The shift o, the scales and
 * the index layout are unchanged; a cache encoded with one handle is read
 * correctly only through a handle with the same signs.
 *   centroids  as for nsn_codebook_create.
 *   sign_mask  host uint8[16]: channel c is negated when bit c % 8 of byte c / 8
 *              is set.  The random draw is the caller's; an all-zero mask gives
 *              the plain transform exactly.
 *   out        host, receives the handle (destroy with nsn_codebook_destroy).
 * Synchronous.  Errors: those of nsn_codebook_create; NSN_EINVAL for a NULL
 * sign_mask.
 */
int nsn_codebook_create_rht(const float* centroids, int g, int K, const uint8_t* sign_mask,
                            nsn_codebook** out);

/*
 * The handle's 16-byte channel sign mask (all zero for nsn_codebook_create).
 *   sign_mask  host uint8[16], written.
 * Errors: NSN_EINVAL (NULL argument).
 */
int nsn_codebook_sign_mask(const nsn_codebook* cb, uint8_t* sign_mask);
void nsn_codebook_destroy(nsn_codebook* cb);
int nsn_codebook_g(const nsn_codebook* cb);

/*
 * Statistics of the g = 4 candidate grid (a search aid; it changes no result):
 * the grid cuts [-4, 4]^4 into 20^4 cubes (the bin edges of
 * nsn_search_grid_edges on every coordinate) and each cell lists the centroids
 * that can be nearest to a point of it.
 *   max_list        host, optional: longest list over all cells.
 *   overflow_cells  host, optional: cells with more than 12 candidates; their
 *                   sub-vectors (like those outside the grid) take the
 *                   exhaustive search.
 * For g = 8 both are 0.  Errors: NSN_EINVAL (NULL handle).
 */
int nsn_codebook_search_stats(const nsn_codebook* cb, int* max_list, int* overflow_cells);

/*
 * Bin edges of the g = 4 candidate grid, the same on each of the four
 * coordinates of a rotated sub-vector: ascending, edges[0] = -4 and the last
 * = 4, a step of 0.4 (a search aid; it changes no result).
 *   edges  host, written: the edges (bins + 1 values).
 *   cap    capacity of edges in values.
 * Returns the number of edges (21), or NSN_EINVAL when edges is NULL or cap is
 * smaller.  Host only; makes no HIP call.
 */
int nsn_search_grid_edges(float* edges, int cap);

/*
 * Device workspace (bytes) that nsn_encode needs for B*H tensors of L tokens.
 * 0 is never returned for valid sizes; returns 0 for invalid sizes.
 */
size_t nsn_encode_workspace_size(int B, int H, int L, int d);

/*
 * Encode L tokens of B*H K or V tensors ([NSN], [HAD], [VQ]):
 *   s1 = ||x||/sqrt(d), y = x/s1; o = mean over the L tokens of y (o_mode
 *   COMPUTE) or the given o (REUSE); z = y - o, s2 = ||z||/sqrt(d), u = z/s2
 *   (a token with ||z|| <= 1e-4*sqrt(d) gets s2 = 0, u = 0); w = H u with the
 *   Sylvester Hadamard H/sqrt(d); each contiguous g-block of w is replaced by
 *   the index of its nearest codebook entry (squared L2, lowest index on ties);
 *   alpha = ||w||^2 / <w, w_hat> (1 if that is <= 0 or s2 = 0); s2' = s2*alpha.
 *
 *   x        device, [B][H][L][d], fp16 (x_dtype NSN_F16) or fp32 (NSN_F32).
 *   L_cap    token capacity of the cache arrays; tokens are written at
 *            positions pos0 .. pos0+L-1 (pos0 + L <= L_cap).
 *   o_mode   NSN_O_COMPUTE: o is written (fp32 [B][H][d]), the mean of these L
 *            tokens, at any pos0: a tensor encoded on its own (a whole prompt at
 *            pos0 = 0, or a flushed residual block placed after the earlier ones,
 *            whose o then goes to that block's slot of the table that
 *            nsn_decode_attention_blocks reads).
 *            NSN_O_REUSE: o is read (the append path for new tokens).
 *   idx      device, [B][H][L_cap][d/g] uint8, written at the token positions.
 *   scales   device, [B][H][L_cap][2] fp16 (s1, s2'), written likewise.
 *   ws       device workspace of at least nsn_encode_workspace_size bytes
 *            (unused with NSN_O_REUSE; may then be NULL).
 * Asynchronous on `stream`.  Errors: NSN_EINVAL, NSN_EUNSUPPORTED,
 * NSN_EWORKSPACE, NSN_EHIP.
 */
int nsn_encode(const nsn_codebook* cb, const void* x, int x_dtype, int B, int H, int L, int L_cap,
               int pos0, int d, int o_mode, float* o, uint8_t* idx, uint16_t* scales, void* ws,
               size_t ws_bytes, void* stream);

/*
 * Device workspace (bytes) that nsn_decode_attention / nsn_decode_step /
 * nsn_decode_attention_residual need: the per-chunk partials of the S cached
 * tokens plus one partial per query head for a residual window.  S may be 0
 * (a residual-window-only decode).  Returns 0 for invalid sizes.
 */
size_t nsn_decode_workspace_size(int B, int Hq, int Hkv, int S, int d);

/*
 * Decode attention of one query per head over S cached tokens ([IMPL]:
 * attention computed directly on the quantized cache with the NSN byproducts):
 *   out[b][h] = sum_i softmax_i(q . k_hat_i / sqrt(d)) v_hat_i, over the S tokens of
 *   KV head h / (Hq/Hkv), with k_hat / v_hat the dequantized cache entries
 *   x_hat = s1 (s2' H w_hat + o).  No mask, no positional rotation.
 *
 *   q        device, [B][Hq][d] fp16.   Hq % Hkv == 0, Hq/Hkv in {1,2,4,8}.
 *   k_*,v_*  device, the cache arrays above with L_cap = S_cap, S <= S_cap.
 *   out      device, [B][Hq][d] fp32.
 *   ws       device workspace of at least nsn_decode_workspace_size bytes.
 * Asynchronous on `stream`.  Errors: NSN_EINVAL, NSN_EUNSUPPORTED,
 * NSN_EWORKSPACE, NSN_EHIP.
 */
int nsn_decode_attention(const nsn_codebook* cb, const uint16_t* q, int B, int Hq, int Hkv, int S,
                         int S_cap, int d, const uint8_t* k_idx, const uint16_t* k_scales,
                         const float* k_o, const uint8_t* v_idx, const uint16_t* v_scales,
                         const float* v_o, float* out, void* ws, size_t ws_bytes, void* stream);

/*
 * nsn_decode_attention for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation, kernels and results, with the workspace taken from a static
 * array of 4 MiB per device (held until the process ends) instead of a caller
 * buffer.  Sizes whose nsn_decode_workspace_size exceeds 4 MiB are refused with
 * NSN_EWORKSPACE; the call allocates nothing.  All calls on one device share that
 * array: calls that overlap on one device (other streams, other host threads)
 * race and must be serialised by the caller.  Arguments and other errors as
 * nsn_decode_attention.
 */
int nsn_decode_attention_noalloc(const nsn_codebook* cb, const uint16_t* q, int B, int Hq, int Hkv, int S,
                                 int S_cap, int d, const uint8_t* k_idx, const uint16_t* k_scales,
                                 const float* k_o, const uint8_t* v_idx, const uint16_t* v_scales,
                                 const float* v_o, float* out, void* stream);

/*
 * Decode attention over a coded cache plus a window of the newest tokens kept
 * as raw fp16 rows ([IMPL] "Residuals": once the window is full its tokens are
 * coded and added to the end of the cache).  One softmax
 * runs over the S quantized tokens followed by the R residual tokens:
 *   out[b][h] = sum_i softmax_i(q . k_i / sqrt(d)) v_i, i over the S dequantized
 *   entries k_hat/v_hat (as in nsn_decode_attention) and the R residual rows.
 *
 *   q, k_*, v_*, S, S_cap, out   as in nsn_decode_attention, except that S may be
 *            0: the quantized arrays are then not read (may be NULL).
 *   k_res, v_res  device, [B][Hkv][R_cap][d] fp16, the residual tokens in
 *            positions 0 .. R-1 of each (b, KV head); 0 <= R <= R_cap, S + R >= 1.
 *   ws       device, nsn_decode_workspace_size(B, Hq, Hkv, S, d) bytes (also for
 *            S = 0 when R > 0: the window's per-head partial lives there).
 * Flushing a full window with a single o per (b, KV head) is nsn_encode of k_res
 * (then v_res) with L = R_cap, L_cap = S_cap, pos0 = S and NSN_O_REUSE on the
 * stored o (NSN_O_COMPUTE when S = 0, which sets o from the flushed block); with
 * one o per flushed block, see nsn_decode_attention_blocks.
 * Asynchronous on `stream`.  Errors: NSN_EINVAL, NSN_EUNSUPPORTED,
 * NSN_EWORKSPACE, NSN_EHIP.
 */
int nsn_decode_attention_residual(const nsn_codebook* cb, const uint16_t* q, int B, int Hq, int Hkv,
                                  int S, int S_cap, int d, const uint8_t* k_idx,
                                  const uint16_t* k_scales, const float* k_o, const uint8_t* v_idx,
                                  const uint16_t* v_scales, const float* v_o, const uint16_t* k_res,
                                  const uint16_t* v_res, int R, int R_cap, float* out, void* ws,
                                  size_t ws_bytes, void* stream);

/*
 * Decode attention over a cache whose flushed residual blocks each keep their own
 * channel mean ([IMPL] "Residuals": a full window is quantized and appended;
 * [NSN]: the shift is the channel mean of the tensor being quantized, here the
 * block).  The quantized tokens are a prefix [0, S0) with the stored o (k_o, v_o,
 * [B][Hkv][d]) followed by nblk blocks of Rb tokens: block j holds tokens
 * S0 + j Rb .. S0 + (j+1) Rb - 1 and its o in k_ob[j], v_ob[j]; then the R fp16
 * residual rows as in nsn_decode_attention_residual.  One softmax over all:
 *   out[b][h] = sum_i softmax_i(q . k_i / sqrt(d)) v_i, with k_hat_i = s1_i
 *   (s2'_i H w_hat_i + o_seg(i)) (likewise v_hat_i), seg(i) the prefix or i's block.
 *
 *   S0, nblk, Rb   S0 >= 0, nblk >= 0, Rb >= 1 when nblk > 0; S0 + nblk Rb <= S_cap.
 *   k_ob, v_ob     device, [nblk_cap][B][Hkv][d] fp32 (nblk <= nblk_cap): block j's o
 *                  is the slab k_ob + j B Hkv d, as nsn_encode writes it with
 *                  NSN_O_COMPUTE for that block (pos0 = S0 + j Rb, L = Rb).
 *   k_o, v_o       the prefix's o (may be NULL when S0 = 0).
 *   k_res, v_res, R, R_cap   the fp16 window (R = 0: none; may be NULL).
 *   ws             device, nsn_decode_blocks_workspace_size(B, Hq, Hkv, S0, nblk, d)
 *                  bytes.
 * Each block is decoded by its own workgroups (its <q, o_K> and its sum of p s1);
 * the merge adds each chunk's beta o_V.  Asynchronous on `stream`.  Errors:
 * NSN_EINVAL, NSN_EUNSUPPORTED, NSN_EWORKSPACE, NSN_EHIP.
 */
size_t nsn_decode_blocks_workspace_size(int B, int Hq, int Hkv, int S0, int nblk, int d);
int nsn_decode_attention_blocks(const nsn_codebook* cb, const uint16_t* q, int B, int Hq, int Hkv, int S0,
                                int nblk, int Rb, int nblk_cap, int S_cap, int d, const uint8_t* k_idx,
                                const uint16_t* k_scales, const float* k_o, const float* k_ob,
                                const uint8_t* v_idx, const uint16_t* v_scales, const float* v_o,
                                const float* v_ob, const uint16_t* k_res, const uint16_t* v_res, int R,
                                int R_cap, float* out, void* ws, size_t ws_bytes, void* stream);

/*
 * One decode step ([IMPL] "Residuals": a new token is quantized and appended):
 * k_new, v_new ([B][Hkv][d] fp16) are encoded with the stored o (as with
 * NSN_O_REUSE: NSN, rotation, nearest centroid, alpha) and written at position S
 * of the caches, and the output is decode attention over the S + 1 tokens.  Two
 * launches: the decode kernel encodes the new pair inside the workgroup of each
 * (batch, KV head)'s last chunk and joins it to that chunk's softmax without
 * reading it back, then the chunk merge.  Only row S of the caches is written.
 * Requires S + 1 <= S_cap (S = 0: an empty cache).  Same workspace as
 * nsn_decode_attention for S + 1.  Asynchronous on `stream`.  Errors as
 * nsn_decode_attention.
 */
int nsn_decode_step(const nsn_codebook* cb, const uint16_t* q, const uint16_t* k_new,
                    const uint16_t* v_new, int B, int Hq, int Hkv, int S, int S_cap, int d,
                    uint8_t* k_idx, uint16_t* k_scales, const float* k_o, uint8_t* v_idx,
                    uint16_t* v_scales, const float* v_o, float* out, void* ws, size_t ws_bytes,
                    void* stream);

/*
 * Decode attention over a cache whose keys were quantized before the rotary
 * position embedding ([IMPL] "Attention Computation": NSN is applied to keys
 * before RoPE).  Cached token i sits at position i; its key is rotated by that
 * position inside the score:
 *   out[b][h] = sum_i softmax_i(q . R(i) k_hat_i / sqrt(d)) v_hat_i,
 *   R(i): rotate-half embedding, channel j < d/2 paired with j + d/2, angle
 *   i * rope_base^(-2j/d); q is the query already rotated to its own position.
 * Values are not rotated.  Arguments as nsn_decode_attention, plus
 *   rope_base  > 1 (10000 for LLaMA / Mistral-7B-v0.1);
 *   ws         nsn_decode_rope_workspace_size(B, Hq, Hkv, S, d) bytes (chunk
 *              partials and the fp32 cos / sin tables, built per call; see
 *              nsn_rope_tables below to build them once).
 * Asynchronous on `stream`.  Errors: NSN_EINVAL, NSN_EUNSUPPORTED,
 * NSN_EWORKSPACE, NSN_EHIP.
 */
size_t nsn_decode_rope_workspace_size(int B, int Hq, int Hkv, int S, int d);
int nsn_decode_attention_rope(const nsn_codebook* cb, const uint16_t* q, int B, int Hq, int Hkv,
                              int S, int S_cap, int d, double rope_base, const uint8_t* k_idx,
                              const uint16_t* k_scales, const float* k_o, const uint8_t* v_idx,
                              const uint16_t* v_scales, const float* v_o, float* out, void* ws,
                              size_t ws_bytes, void* stream);

/*
 * The cos / sin tables of nsn_decode_attention_rope built once, for callers that
 * decode many times over caches of up to S_tab tokens (the same pre-RoPE keys of
 * [IMPL] "Attention Computation").  The tables hold the angles i * rope_base^(-2j/d)
 * of every position i < S_tab as fp32 (cos, sin) pairs evaluated in fp64: a coarse
 * table (one row of 64 frequencies per 256 positions) followed by a fine one (256
 * rows).  They depend on rope_base and S_tab only, not on a codebook.
 *   nsn_rope_tables_size(S_tab)  bytes of the tables (0 if S_tab <= 0);
 *   nsn_rope_tables              builds them into `tables`: device memory the caller
 *                                owns, 16-byte aligned, at least that many bytes;
 *                                asynchronous on `stream`;
 *   nsn_decode_attention_rope_tables
 *                                nsn_decode_attention_rope with the tables passed
 *                                in: `tables` built by nsn_rope_tables for S_tab
 *                                positions and the RoPE base wanted, S <= S_tab;
 *                                the workspace holds only the chunk partials,
 *                                nsn_decode_rope_tables_workspace_size(B, Hq, Hkv,
 *                                S, d) bytes.  The output equals bit for bit that
 *                                of nsn_decode_attention_rope with the same base.
 * The tables are only read by the decode; concurrent decodes may share them.
 * Errors: NSN_EINVAL (NULL or misaligned tables, S_tab <= 0, S > S_tab, rope_base
 * not above 1, tables buffer too small, and the checks of nsn_decode_attention),
 * NSN_EUNSUPPORTED, NSN_EWORKSPACE, NSN_EHIP.
 */
size_t nsn_rope_tables_size(int S_tab);
int nsn_rope_tables(double rope_base, int S_tab, void* tables, size_t bytes, void* stream);
size_t nsn_decode_rope_tables_workspace_size(int B, int Hq, int Hkv, int S, int d);
int nsn_decode_attention_rope_tables(const nsn_codebook* cb, const uint16_t* q, int B, int Hq,
                                     int Hkv, int S, int S_cap, int d, const void* tables,
                                     int S_tab, const uint8_t* k_idx, const uint16_t* k_scales,
                                     const float* k_o, const uint8_t* v_idx,
                                     const uint16_t* v_scales, const float* v_o, float* out,
                                     void* ws, size_t ws_bytes, void* stream);

/*
 * ---- Double quantization ([VQ] "Double Quantization (DQ)": the NSN parameters
 * o and s1 and the codebook entries are themselves quantized to 4 bits).
 *
 * A double-quantized K or V cache of B*H tensors with token capacity L_cap is:
 *   idx   [B][H][L_cap][d/g] uint8     as in the plain cache;
 *   s2    [B][H][L_cap] fp16           s2' (the adjusted second scale);
 *   s1c   [B][H][(L_cap+1)/2] uint8    4-bit s1 codes, token t in byte t/2,
 *                                      low nibble for even t;
 *   head  [B][H] nsn_dq_head           the tensor's 4-bit o and s1 grid.
 * s1 codes: 0 marks a zero token (s1 = 0); code c >= 1 stands for the fp16
 * value whose bit pattern is s1_base + (c - 1) * s1_stride (capped at 0x7BFF),
 * a uniform grid over the fp16 pattern, i.e. piecewise logarithmic in s1.
 * o codes: channel c in byte c/2 (low nibble for even c) holds code + 8,
 * code in -7 .. 7; o_q[c] = code * o_scale (fp32).
 * The encoding uses the quantized values themselves (y = x / s1_q,
 * z = y - o_q), so x_hat = s1_q (s2' H w_hat + o_q) is exact up to the
 * vector quantization.
 */
typedef struct nsn_dq_head {
  uint8_t o_codes[64];
  float o_scale;        /* max |o| / 7 (fp32); 0 for o = 0 */
  uint16_t s1_base;     /* fp16 pattern of the smallest non-zero s1 of the tensor */
  uint16_t s1_stride;   /* >= 1: ceil((largest pattern - s1_base) / 14) */
  uint32_t reserved[2]; /* written as 0 */
} nsn_dq_head;          /* 80 bytes */

/*
 * 4-bit codebook entries: one step D = max |C| / 7.5 (fp32) for the whole
 * codebook, mid-rise levels (k - 7.5) D, k = 0 .. 15, each entry to the
 * nearest level (k = clamp(floor(C / D + 8), 0, 15), in fp64), the level
 * value rounded to fp16 (nearest even) so that nsn_codebook_create accepts it.
 *   centroids  host [K][g] fp32;  codes host [K][g] uint8 (or NULL);
 *   step       host (or NULL): D;  centroids_q host [K][g] fp32, fp16-exact.
 * Host only.  Errors: NSN_EINVAL.
 */
int nsn_codebook_dq4(const float* centroids, int K, int g, uint8_t* codes, float* step,
                     float* centroids_q);

/*
 * Device workspace (bytes) that nsn_encode_dq needs (both o modes).
 */
size_t nsn_encode_dq_workspace_size(int B, int H, int L, int d);

/*
 * Encode L tokens of B*H tensors into a double-quantized cache (see above);
 * arguments as in nsn_encode, with head in place of o:
 *   o_mode NSN_O_COMPUTE (pos0 = 0): head is written: o = mean over the L
 *          tokens of x / s1 (unquantized s1), quantized to 4 bits; the s1 grid
 *          spans the fp16 patterns of the tokens' non-zero s1.
 *   o_mode NSN_O_REUSE: head is read (appends; any pos0, odd ones included:
 *          the nibble shared with token pos0 - 1 or pos0 + L is preserved).
 *   s2, s1c written at the token positions; ws of at least
 *   nsn_encode_dq_workspace_size bytes (both modes).
 * Asynchronous on `stream`.  Errors: NSN_EINVAL, NSN_EUNSUPPORTED,
 * NSN_EWORKSPACE, NSN_EHIP.
 */
int nsn_encode_dq(const nsn_codebook* cb, const void* x, int x_dtype, int B, int H, int L, int L_cap,
                  int pos0, int d, int o_mode, nsn_dq_head* head, uint8_t* idx, uint16_t* s2,
                  uint8_t* s1c, void* ws, size_t ws_bytes, void* stream);

/*
 * Decode attention over double-quantized K and V caches: the same attention
 * as nsn_decode_attention on the dequantized entries
 * x_hat = s1_q (s2' H w_hat + o_q).  Arguments as there, with (idx, s2, s1c,
 * head) per cache; workspace nsn_decode_workspace_size(B, Hq, Hkv, S, d).
 * Asynchronous on `stream`.  Errors: NSN_EINVAL, NSN_EUNSUPPORTED,
 * NSN_EWORKSPACE, NSN_EHIP.
 */
int nsn_decode_attention_dq(const nsn_codebook* cb, const uint16_t* q, int B, int Hq, int Hkv, int S,
                            int S_cap, int d, const uint8_t* k_idx, const uint16_t* k_s2,
                            const uint8_t* k_s1c, const nsn_dq_head* k_head, const uint8_t* v_idx,
                            const uint16_t* v_s2, const uint8_t* v_s1c, const nsn_dq_head* v_head,
                            float* out, void* ws, size_t ws_bytes, void* stream);

/*
 * Dequantize L tokens ([NSN]: the byproducts reconstruct the tensor):
 *   x_hat[b][h][i] = s1 (s2' H w_hat + o), w_hat the concatenated centroids.
 *   idx/scales have token capacity L_cap (L <= L_cap); o fp32 [B][H][d];
 *   x_hat device fp32 [B][H][L][d].  Asynchronous on `stream`.
 * Errors: NSN_EINVAL, NSN_EUNSUPPORTED, NSN_EHIP.
 */
int nsn_dequantize(const nsn_codebook* cb, const uint8_t* idx, const uint16_t* scales,
                   const float* o, int B, int H, int L, int L_cap, int d, float* x_hat,
                   void* stream);

/*
 * Host-only argument checks, identical to the validation nsn_encode and
 * nsn_decode_attention run before any HIP call, for a codebook of sub-vector
 * length g.  They touch no device and need no handle, so the validation can be
 * exercised on a machine without a GPU.  Same status codes as the real calls.
 */
int nsn_check_encode_args(int g, const void* x, int x_dtype, int B, int H, int L, int L_cap, int pos0,
                          int d, int o_mode, const void* o, const void* idx, const void* scales,
                          const void* ws, size_t ws_bytes);
int nsn_check_decode_args(int g, const void* q, int B, int Hq, int Hkv, int S, int S_cap, int d,
                          const void* k_idx, const void* k_scales, const void* k_o, const void* v_idx,
                          const void* v_scales, const void* v_o, const void* out, const void* ws,
                          size_t ws_bytes);

int nsn_check_decode_residual_args(int g, const void* q, int B, int Hq, int Hkv, int S, int S_cap,
                                   int d, const void* k_idx, const void* k_scales, const void* k_o,
                                   const void* v_idx, const void* v_scales, const void* v_o,
                                   const void* k_res, const void* v_res, int R, int R_cap,
                                   const void* out, const void* ws, size_t ws_bytes);

int nsn_check_decode_blocks_args(int g, const void* q, int B, int Hq, int Hkv, int S0, int nblk, int Rb,
                                 int nblk_cap, int S_cap, int d, const void* k_idx, const void* k_scales,
                                 const void* k_o, const void* k_ob, const void* v_idx, const void* v_scales,
                                 const void* v_o, const void* v_ob, const void* k_res, const void* v_res, int R,
                                 int R_cap, const void* out, const void* ws, size_t ws_bytes);

#ifdef __cplusplus
}
#endif

#endif /* NSN_H_ */
