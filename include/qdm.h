/*
 * qdm.h -- C ABI of the MI355X (gfx950) one-row quantized decode MLP library.
 *
 * What the library computes is defined on the meTile documentation pages:
 *   - "Compute-Graph Fusion", section "Automatic Gated Epilogues": two
 *     projections share the activation input, the SwiGLU epilogue
 *     silu(gate) * up is applied on chip, and for one-row decode the
 *     transformer residual is added inside the down projection.
 *   - "MLX-LM Backend", section "Dispatch Policy": affine weights keep
 *     per-group scales and biases (groups of 32, 64, 128 along the input
 *     dim), 4-bit weights keep their nibbles, dense BF16 weights get an
 *     interleaved gate/up view; gate and up share each activation load and
 *     the SwiGLU epilogue precedes the only write of h; the down projection's
 *     typed store adds the residual; RMSNorm accumulates in FP32.
 *   - "Compute-Graph Fusion", opening GraphBuilder example: residual add
 *     followed by RMSNorm keeps the sum as a second output (one
 *     multi-output kernel).
 *
 * Conventions for every entry point:
 *   - Return 0 (QDM_OK) or a negative qdm_status.  Nothing is printed and no
 *     exception crosses the ABI.  Every argument is checked before anything
 *     is launched or written: on error no output byte is touched.
 *   - Pointers named "device" are device (HBM) addresses owned by the
 *     caller; "host" pointers are ordinary host memory owned by the caller.
 *     The library allocates, frees and synchronizes nothing: every buffer a
 *     kernel writes, scratch included, is an argument (a workspace sized by
 *     the matching *_workspace_bytes query), so any call may be captured
 *     into a HIP graph.  The only state it keeps is a per-device cache of
 *     occupancy queries.  Calls on different streams are independent when
 *     their workspaces and outputs are distinct.
 *   - GPU work is enqueued on `stream` (a hipStream_t; NULL = the legacy
 *     default stream) and the call returns without waiting.  A failed
 *     launch returns QDM_ERR_HIP.
 *   - Row-major storage throughout.  bf16 / f16 values are IEEE binary16
 *     formats stored as 16-bit words.
 *
 * Weight formats (the `bits` field of qdm_weight):
 *   8  : affine uint8 codes, one per byte, row-major [n][k];
 *   4  : affine 4-bit codes, two per byte, row-major [n][k/2]; byte i of a row
 *        holds code 2i in its low nibble and code 2i+1 in its high nibble;
 *   16 : dense bf16 weights [n][k] (no scale/bias; group = 0);
 *   QDM_U8_SB16, QDM_U4_SB16 : the affine 8 / 4-bit formats with the
 *        (scale, bias) pairs stored as bf16 (two uint16 per group,
 *        [n][k/group][2], 4-byte aligned), the dtype MLX keeps them in for
 *        bf16 models;
 *   QDM_MXFP8, QDM_MXFP4 : block-scaled weights ("MLX-LM Backend" page,
 *        section "Block-Scaled MLX Primitive": E8M0 block scales with E4M3 or
 *        E2M1 elements; read as the OCP Microscaling formats): blocks of 32
 *        along k (group = 32), element codes row-major [n][k] one per byte
 *        (E4M3) or [n][k/2] two per byte low nibble first (E2M1), and one
 *        E8M0 byte per block in block_scales [n][k/32].
 * Affine value of code q in group j of row i:  w = scale[i][j]*q + bias[i][j]
 * with fp32 (scale, bias) stored as adjacent pairs, [n][k/group][2].
 * MX value of element code c in block j of row i:
 *   w = 2^(block_scales[i][j] - 127) * value(c), value from the element format
 *   (E2M1: sign, 2 exponent bits with bias 1, 1 mantissa bit, largest 6;
 *    E4M3: sign, 4 exponent bits with bias 7, 3 mantissa bits, largest 448).
 * Gate/up pairs are interleaved by rows: packed row 2f is gate row f and
 * packed row 2f+1 is up row f, for the codes ([ffn][2][...]) and for the
 * scale/bias pairs ([ffn][2][d/group][2]) or block scales ([ffn][2][d/32]).
 */
#ifndef QDM_H
#define QDM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qdm_status {
    QDM_OK = 0,
    QDM_ERR_INVALID_ARG = -1,   /* NULL pointer, non-positive or inconsistent size, non-finite weight */
    QDM_ERR_UNSUPPORTED = -2,   /* valid but not provided: bits/group/dtype/row-count combination */
    QDM_ERR_ALIGNMENT = -3,     /* a pointer is not aligned as the entry point requires */
    QDM_ERR_WORKSPACE = -4,     /* workspace NULL or smaller than its *_workspace_bytes() query */
    QDM_ERR_HIP = -5,           /* the HIP runtime refused a launch */
    QDM_ERR_TOO_LARGE = -6      /* qdm_mlp_decode_noalloc: the call needs more than its fixed scratch */
} qdm_status;

typedef enum qdm_dtype { QDM_F32 = 0, QDM_F16 = 1, QDM_BF16 = 2 } qdm_dtype;

/* Values of qdm_weight.bits besides 4, 8 and 16 (the low byte is the code width). */
enum { QDM_MXFP4 = 0x104, QDM_MXFP8 = 0x108, QDM_U4_SB16 = 0x204, QDM_U8_SB16 = 0x208 };

/* A packed weight matrix in device memory, described once per weight set and
 * reused for every call (the pages bind prepared weights once into a warmed
 * executor: "MLX-LM Backend", "Dispatch Policy").
 *   n, k        logical shape [n][k]; the contraction runs over k.  For a
 *               gate/up pair descriptor n = ffn (the number of pairs) and
 *               k = d.
 *   bits        8, 4, 16, QDM_MXFP8 or QDM_MXFP4 (see above).
 *   group       32, 64 or 128 for bits 8/4 (k % group == 0); 0 for bits 16;
 *               32 for the MX formats.
 *   q           device, 16-byte aligned: packed codes or bf16 words.
 *   scale_bias  device, 8-byte aligned: fp32 pairs (bf16 pairs, 4-byte aligned, for
 *               the _SB16 formats); NULL for bits 16 and MX.
 *   block_scales device: E8M0 bytes [n][k/32] for MX; NULL otherwise.
 * MX and _SB16 weights are taken by the one-row calls (m = 1) whose projections run on
 * the weight-streaming kernel, and by the MLP calls with 2..16 rows and a
 * 16-bit act dtype whose projections run on the matrix-core streaming
 * kernels; anything else (qdm_gemv_linear with m > 1 among it) returns
 * QDM_ERR_UNSUPPORTED. */
typedef struct qdm_weight {
    int32_t n;
    int32_t k;
    int32_t bits;
    int32_t group;
    const void* q;
    const float* scale_bias;
    const uint8_t* block_scales;
} qdm_weight;

/* ----------------------------------------------------------------- sizes */

/* Bytes of one packed [n][k] code matrix (bits 4/8) or bf16 matrix (bits 16);
 * 0 if the arguments are invalid. */
size_t qdm_packed_q_bytes(int32_t n, int32_t k, int32_t bits);

/* Number of fp32 values of the scale/bias pairs of an [n][k] matrix: 2*n*k/group;
 * 0 if invalid. */
size_t qdm_scale_bias_floats(int32_t n, int32_t k, int32_t group);

/* Bytes of the E8M0 block scales of an MX [n][k] matrix: n*k/32; 0 if invalid. */
size_t qdm_mx_scale_bytes(int32_t n, int32_t k);

/* Workspace sizes.  A projection whose kernel splits the contraction across
 * thread blocks (2..16 rows of the down projection on the matrix cores; more
 * than 16 rows on the tiled kernels when their output tiles alone would not
 * fill the chip) writes fp32 partial sums to the caller's workspace; these
 * queries give the bytes a call with the same arguments needs, computed from
 * the shapes and formats only (no device is touched; the tiled kernels' split
 * is sized for the full 256-CU chip, which bounds any device).  They return 0
 * for invalid arguments, which the call itself then rejects. */

/* qdm_gemv_gate_up_swiglu: partials only (0 when that call splits nothing). */
size_t qdm_gemv_gate_up_workspace_bytes(int32_t m, qdm_dtype act, const qdm_weight* gate_up);

/* qdm_gemv_down_residual: partials only (0 when that call splits nothing). */
size_t qdm_gemv_down_workspace_bytes(int32_t m, qdm_dtype act, const qdm_weight* down);

/* qdm_mlp_decode: the fp32 hidden rows h[m][ffn] (rounded up to 256 bytes),
 * then the larger of the two projections' partials (rounded up to 256). */
size_t qdm_mlp_workspace_bytes(int32_t m, qdm_dtype act, const qdm_weight* gate_up, const qdm_weight* down);

/* ----------------------------------------------------------------- host: quantize / pack
 * Ahead-of-time preparation, once per weight set, on host buffers.  The pages
 * prepare packed views ahead of time and keep the originals ("MLX-LM Backend",
 * intro and "Dispatch Policy"); inputs are never modified.  These run on host
 * threads and are bit-exact: the same inputs always give the same bytes.
 *
 * Quantizer (the pages name an affine format with per-group scale and bias but
 * print no formula; this is the plain reading): for each row and group,
 *   mn, mx = min, max of the group's fp32 weights (a zero minimum is stored as +0)
 *   scale  = (float)(((double)mx - (double)mn) / (2^bits - 1))   nearest-even
 *   bias   = mn
 *   q      = clamp(nearbyint(((double)w - (double)mn) / (double)scale), 0, 2^bits - 1)
 *   and q = 0 for the whole group when scale == 0.                          */

/* w host fp32 [n][k] -> codes host uint8 [n][k], scale/bias host fp32 [n][k/group].
 * INVALID_ARG for NULLs, non-positive sizes, k % group != 0, or a non-finite
 * weight; UNSUPPORTED for bits not in {4, 8} or group not in {32, 64, 128}. */
int qdm_quantize_affine(const float* w, int32_t n, int32_t k, int32_t bits, int32_t group,
                        uint8_t* codes, float* scale, float* bias);

/* Logical codes/scale/bias -> packed codes q_out (host, qdm_packed_q_bytes bytes)
 * and scale_bias_out (host, qdm_scale_bias_floats floats).  This is the repack
 * that keeps codes, scales and biases unchanged (no requantization).
 * INVALID_ARG also for a code >= 2^bits. */
int qdm_pack_rows(const uint8_t* codes, const float* scale, const float* bias,
                  int32_t n, int32_t k, int32_t bits, int32_t group,
                  void* q_out, float* scale_bias_out);

/* Quantize and pack in one pass: w host fp32 [n][k] -> q_out, scale_bias_out. */
int qdm_quantize_pack_rows(const float* w, int32_t n, int32_t k, int32_t bits, int32_t group,
                           void* q_out, float* scale_bias_out);

/* Gate and up matrices (each host fp32 [ffn][d]) -> interleaved packed codes
 * q_out [ffn][2][d*bits/8] and scale_bias_out [ffn][2][d/group][2]. */
int qdm_quantize_pack_gate_up(const float* w_gate, const float* w_up, int32_t ffn, int32_t d,
                              int32_t bits, int32_t group, void* q_out, float* scale_bias_out);

/* Same from logical codes/scales/biases (repack without requantizing). */
int qdm_pack_gate_up(const uint8_t* gate_codes, const float* gate_scale, const float* gate_bias,
                     const uint8_t* up_codes, const float* up_scale, const float* up_bias,
                     int32_t ffn, int32_t d, int32_t bits, int32_t group,
                     void* q_out, float* scale_bias_out);

/* Affine quantize + pack with bf16 (scale, bias) pairs (the pages do not
 * print the pairs' storage type; MLX keeps them in the model's dtype).  The
 * pair is computed as for qdm_quantize_affine, each value rounded once to bf16
 * (nearest-even), then every code chosen against the rounded pair:
 *   q = clamp(nearbyint(((double)w - bias_bf16) / scale_bf16), 0, 2^bits - 1)
 * (all 0 when the rounded scale is 0).  bits 4 or 8 (storage as for the fp32
 * pairs); scale_bias_out host uint16 [n][k/group][2].  Bit-exact. */
int qdm_quantize_pack_rows_sb16(const float* w, int32_t n, int32_t k, int32_t bits, int32_t group, void* q_out,
                                uint16_t* scale_bias_out);

/* The same for a gate/up pair: interleaved codes and bf16 pairs [ffn][2][d/group][2]. */
int qdm_quantize_pack_gate_up_sb16(const float* w_gate, const float* w_up, int32_t ffn, int32_t d, int32_t bits,
                                   int32_t group, void* q_out, uint16_t* scale_bias_out);

/* MX quantizer (the pages name the formats, not a quantizer; this is the OCP
 * Microscaling conversion, the plain reading): per block of 32,
 *   shared = clamp(floor(log2(max |w|)) - emax, -127, 127)   (emax 2 for E2M1,
 *            8 for E4M3; an all-zero block takes shared = -127)
 *   scale code = shared + 127
 *   element = the element value nearest |w| / 2^shared (ties to the even
 *            mantissa), saturated at the largest; the sign bit set for w < 0.
 * w host fp32 [n][k] (k % 32 == 0) -> q_out (qdm_packed_q_bytes(n, k, format)
 * bytes) and scales_out (qdm_mx_scale_bytes(n, k) bytes).  Bit-exact.
 * INVALID_ARG for NULLs, bad sizes or a non-finite weight; UNSUPPORTED for a
 * format other than QDM_MXFP4 / QDM_MXFP8. */
int qdm_quantize_mx(const float* w, int32_t n, int32_t k, int32_t format, void* q_out, uint8_t* scales_out);

/* Gate and up (each host fp32 [ffn][d]) -> interleaved MX codes [ffn][2][...]
 * and block scales [ffn][2][d/32]. */
int qdm_quantize_mx_gate_up(const float* w_gate, const float* w_up, int32_t ffn, int32_t d, int32_t format,
                            void* q_out, uint8_t* scales_out);

/* Dense bf16 gate and up [ffn][d] (host uint16 words) -> interleaved
 * out [ffn][2][d] (the interleaved gate/up view of "Dispatch Policy"). */
int qdm_pack_dense_gate_up(const uint16_t* gate_bf16, const uint16_t* up_bf16,
                           int32_t ffn, int32_t d, uint16_t* out);

/* ----------------------------------------------------------------- device: the hot path
 * Supported combinations (anything else returns QDM_ERR_UNSUPPORTED):
 *   act     QDM_F32, QDM_BF16 or QDM_F16: the dtype of x, r and out.
 *   weights bits 8 or 4 with group 32/64/128, or bits 16 (dense bf16).
 *   m       1..4096 rows.  Up to 16 rows run in one pass of the kernels.
 *           More rows run on tiled dual-GEMM kernels (64 rows per weight
 *           read; meTile docs, "MLX-LM Backend", section "Dispatch Policy":
 *           multi-row calls take a fused dual-GEMM gate/up with SwiGLU in
 *           registers) for 8/4-bit affine (either pair storage) and MX
 *           weights with a 16-bit act dtype, n a multiple of 16 and k a
 *           multiple of 128 (4-bit codes, or any codes in groups of 32) or 64
 *           (8-bit codes in wider groups); otherwise,
 *           and for qdm_gemv_linear, as passes of 16 rows (each pass
 *           streams the weights again).
 *   k       a multiple of 16 (bits 8), 32 (bits 4) or 8 (bits 16).
 * Device pointers x, r, out, h, s_out, n_out, a, b, w must be 16-byte aligned. */

/* h[m][ffn] = silu(G) * U with G = x W_gate^T, U = x W_up^T, fp32 accumulation,
 * one write of h (fp32) per element.  Defined by "Compute-Graph Fusion",
 * section "Automatic Gated Epilogues" (two projections over one activation,
 * silu(gate) * up applied on chip) and "MLX-LM Backend", section "Dispatch
 * Policy" (gate and up share each activation load; the SwiGLU epilogue
 * precedes the only write of the hidden tile).
 *   x          device, act dtype, [m][d]
 *   gate_up    interleaved pair descriptor (n = ffn, k = d)
 *   workspace  device, >= qdm_gemv_gate_up_workspace_bytes(m, act, gate_up)
 *              bytes, 16-byte aligned; may be NULL when that is 0
 *   h_out      device fp32 [m][ffn]
 * x, h_out and the workspace must not overlap (INVALID_ARG).               */
int qdm_gemv_gate_up_swiglu(const void* x, int32_t m, qdm_dtype act, const qdm_weight* gate_up,
                            void* workspace, size_t workspace_bytes, float* h_out, void* stream);

/* out[m][d] = r + h W_down^T, fp32 accumulation, the residual added in fp32 and
 * the sum rounded once (nearest-even) to the act dtype.  Defined by
 * "Compute-Graph Fusion", section "Automatic Gated Epilogues" (for one-row
 * decode the transformer residual is added inside the down projection) and
 * "MLX-LM Backend", section "Dispatch Policy" (the typed store adds the
 * residual without materializing the projection's own result).
 *   h          device fp32 [m][ffn];  r, out: device, act dtype, [m][d]
 *   down       descriptor with n = d, k = ffn
 *   workspace  device, >= qdm_gemv_down_workspace_bytes(m, act, down) bytes,
 *              16-byte aligned; may be NULL when that is 0
 * out may alias r; out must not overlap h, and the workspace none of h, r,
 * out (INVALID_ARG). */
int qdm_gemv_down_residual(const float* h, const void* r, int32_t m, qdm_dtype act, const qdm_weight* down,
                           void* workspace, size_t workspace_bytes, void* out, void* stream);

/* out[m][n] = x W^T + bias, fp32 accumulation, bias added in fp32, the sum
 * rounded once (nearest-even) to the act dtype.  The one-row decode
 * projections other than the MLP ("MLX-LM Backend" page, the passages on
 * vocabulary compression -- an untied lm_head, or a tied embedding table used
 * as the linear map -- and on attention-projection compression -- q/k/v/o
 * with their biases kept): the down projection's GEMV with the bias where the
 * residual was.
 *   x     device, act dtype, [m][k]
 *   w     descriptor [n][k]: bits 8/4 with group 32/64/128, or 16 (dense
 *         bf16); a tied embedding is the [vocab][d] table itself (n = vocab).
 *   bias  device, act dtype, [n], shared by the m rows; NULL for none.
 *   out   device, act dtype, [m][n]; may overlap neither x nor bias.
 * One row runs on the weight-streaming kernel; 2..16 rows on the vector
 * kernel four rows a pass. */
int qdm_gemv_linear(const void* x, int32_t m, qdm_dtype act, const qdm_weight* w, const void* bias, void* out,
                    void* stream);

/* The whole MLP, out = r + W_down (silu(W_gate x) * (W_up x)): the two
 * projections above on one stream ("Compute-Graph Fusion", "Automatic Gated
 * Epilogues": the gated pair, then the down projection with the residual).
 *   x, r, out  device, act dtype, [m][d]; out may alias x or r
 *   workspace  device, >= qdm_mlp_workspace_bytes(m, act, gate_up, down)
 *              bytes, 16-byte aligned, overlapping none of x, r, out
 *              (INVALID_ARG): h, then the projections' partial sums
 * gate_up->k must equal down->n (= d) and gate_up->n must equal down->k (= ffn);
 * both descriptors must use the same bits. */
int qdm_mlp_decode(const void* x, const void* r, int32_t m, qdm_dtype act,
                   const qdm_weight* gate_up, const qdm_weight* down,
                   void* workspace, size_t workspace_bytes, void* out, void* stream);

/* qdm_mlp_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and kernels, with the workspace (h and the split-K
 * partials) in a fixed array of QDM_NOALLOC_SCRATCH_BYTES that the library
 * holds on every GPU it runs on until the process ends, instead of a caller's
 * buffer.  Arguments as for qdm_mlp_decode without the workspace.
 * QDM_ERR_TOO_LARGE when qdm_mlp_workspace_bytes(m, act, gate_up, down)
 * exceeds the array (16 MiB: h and partials of up to 16 rows at Llama-3-8B
 * and Qwen3-8B shapes; more rows need the ordinary entry point); nothing is
 * launched then.  The array keeps the last call's contents; the kernels write
 * every byte they read, so nothing is cleared between calls.  All calls on one
 * GPU share its array: calls that can overlap in time on that GPU (different
 * streams, or threads without ordering) race and must be ordered by the
 * caller.  Allocates nothing: the array's device address is looked up once
 * per device, on the first call made with that device current. */
#define QDM_NOALLOC_SCRATCH_BYTES (16u << 20)
int qdm_mlp_decode_noalloc(const void* x, const void* r, int32_t m, qdm_dtype act,
                           const qdm_weight* gate_up, const qdm_weight* down, void* out, void* stream);

/* Residual add + RMSNorm with both outputs, per row ("Compute-Graph Fusion",
 * the opening GraphBuilder example: the add feeds RMSNorm and the sum stays a
 * second output of one kernel; "MLX-LM Backend", "Dispatch Policy": RMSNorm
 * accumulates in FP32):
 *   s = a + b rounded once to `dtype`;  n = s * w / sqrt(mean(s^2) + eps)
 * with fp32 accumulation of the mean square; n rounded once to `dtype`.
 *   a, b, s_out, n_out: device, dtype, [rows][n];  w: device, dtype, [n]
 *   eps >= 0 and finite.  s_out may alias a or b. */
int qdm_add_rmsnorm(const void* a, const void* b, const void* w, int32_t rows, int32_t n,
                    float eps, qdm_dtype dtype, void* s_out, void* n_out, void* stream);

/* Workspace bytes qdm_mlp_decode_rmsnorm needs: h[m][ffn] fp32, two [m][d]
 * rows of the act dtype, then the projections' partial sums, each part
 * rounded up to 256 bytes; 0 if invalid. */
size_t qdm_mlp_rmsnorm_workspace_bytes(int32_t m, qdm_dtype act, const qdm_weight* gate_up, const qdm_weight* down);

/* The decode chain across the layer boundary: the residual add + RMSNorm
 * above feeding the MLP, with the sum as the MLP's residual ("Compute-Graph
 * Fusion": the GraphBuilder example's add + RMSNorm with the sum kept, and
 * the gated MLP with the residual added in the down projection):
 *   s = a + b (rounded once),  n = s * w / sqrt(mean(s^2) + eps) (rounded once),
 *   out = s + W_down (silu(W_gate n) * (W_up n)).
 * Results are bitwise those of qdm_add_rmsnorm followed by qdm_mlp_decode
 * with x = n and r = s.  With one row and shapes the one-row streaming
 * kernels take, two launches: every gate/up block recomputes s, the mean
 * square and n from a, b and w, and the down launch adds s as its residual
 * (n and s never go to HBM).  With 2..16 rows on the matrix-core kernels
 * every gate/up block rebuilds n likewise and s goes through the workspace
 * to the down projection.  Otherwise the three launches run in order
 * through the workspace.
 *   a, b     device, act dtype, [m][d]; out may alias either.
 *   norm_w   device, act dtype, [d];  eps >= 0 and finite.
 *   s_out    device, act dtype, [m][d], or NULL (s not written); may alias
 *            a or b, not out.
 *   workspace device, >= qdm_mlp_rmsnorm_workspace_bytes(m, act, gate_up,
 *            down) bytes, 16-byte aligned, overlapping none of a, b, norm_w,
 *            s_out, out (INVALID_ARG).
 *   Weights as for qdm_mlp_decode (gate_up->k = down->n = d, same bits). */
int qdm_mlp_decode_rmsnorm(const void* a, const void* b, const void* norm_w, float eps, int32_t m, qdm_dtype act,
                           const qdm_weight* gate_up, const qdm_weight* down,
                           void* workspace, size_t workspace_bytes, void* s_out, void* out, void* stream);

/* ----------------------------------------------------------------- misc */

/* A static string naming a status code. */
const char* qdm_status_string(int status);

/* Library ABI version (major * 100 + minor). */
int qdm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QDM_H */
