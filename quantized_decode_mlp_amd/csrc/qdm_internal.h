// Internal interface between the C-ABI layer (qdm_api.cpp, host C++) and the
// HIP launchers (qdm_*.hip).  Arguments are already validated when these run.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "qdm.h"

namespace qdm {

// Each returns 0 on success or the hipError_t of the failed launch.
int launch_gate_up_swiglu(const void* x, int m, int act, const qdm_weight& gu, float* h,
                          void* stream);
// part: fp32 split-K partials, at least down_mma_stream_partials_bytes(dn, m)
// when mma_stream_down_supported(dn, m, act) (unused otherwise).
int launch_down_residual(const float* h, const void* r, int m, int act, const qdm_weight& dn,
                         void* out, float* part, void* stream);
// True when one row of x (xb bytes per element) times w runs on the
// weight-streaming kernel (the only kernel that takes MX weights).
bool stream_supported(const qdm_weight& w, int xb);
// A projection out[m][n] = x W^T (+ bias[n] when bias is not null), act dtype in and out.
int launch_linear(const void* x, int m, int act, const qdm_weight& w, const void* bias, void* out, void* stream);
// Few-row (2..16) projections on the matrix cores (qdm_mfma.hip).
bool mma_rows_supported(const qdm_weight& w, int m);
int launch_gate_up_mma(const void* x_bf16, int m, const qdm_weight& gu, float* h, void* stream);
int launch_down_mma(const float* h, const void* r, int m, int act, const qdm_weight& dn, void* out, void* stream);
// 2..16 rows, 8/4-bit affine weights, 16-bit activations: persistent blocks
// streaming the weights once (qdm_mma_stream.hip).
bool mma_stream_gate_up_supported(const qdm_weight& w, int m, int act);
int launch_gate_up_mma_stream(const void* x, int m, int act, const qdm_weight& gu, float* h, void* stream);
// The same with the decode chain's rows: x = rmsnorm(a + b) * w per row, recomputed
// in every block; block 0 stores s = a + b to s_buf (act dtype, [m][k]).
int launch_gate_up_mma_stream_norm(const void* a, const void* b, const void* w, float eps, int m, int act,
                                   const qdm_weight& gu, float* h, void* s_buf, void* stream);
// 2..16 rows, 8/4-bit affine weights, 16-bit output: K split across blocks
// with the fp32 partials in part, a caller-owned buffer of at least
// down_mma_stream_partials_bytes(dn, m) bytes (qdm_mma_down.hip).
bool mma_stream_down_supported(const qdm_weight& w, int m, int act);
size_t down_mma_stream_partials_bytes(const qdm_weight& w, int m);
// r_copy: when not null, also receives r (the decode chain's s).
int launch_down_mma_stream(const float* h, const void* r, int m, int act, const qdm_weight& dn, void* out,
                           float* part, void* stream, void* r_copy = nullptr);
// One row, both projections on the streaming kernels: the decode chain with
// add + RMSNorm folded into the MLP's two launches (qdm_chain.hip).
bool chain_stream_supported(const qdm_weight& gu, const qdm_weight& dn, int act);
int launch_mlp_chain_stream(const void* a, const void* b, const void* w, float eps, int act, const qdm_weight& gu,
                            const qdm_weight& dn, float* h, void* s_out, void* out, void* stream);
// More than 16 rows, 8/4-bit affine (either pair storage) or MX weights, 16-bit
// activations: tiled dual GEMM, 64 rows x 64 outputs per block (qdm_prefill.hip).
// A launch whose output tiles do not fill the chip splits K and writes fp32
// partials to part, a caller-owned buffer of at least prefill_partials_bytes
// (0: no split, part unused).
bool prefill_supported(const qdm_weight& w, int m, int act);
size_t prefill_partials_bytes(const qdm_weight& w, int m, bool gate_up);
int launch_gate_up_prefill(const void* x, int m, int act, const qdm_weight& gu, float* h, float* part, void* stream);
int launch_down_prefill(const float* h, const void* r, int m, int act, const qdm_weight& dn, void* out, float* part,
                        void* stream);
// qdm_mlp_decode after validation: h and the partials in `workspace`, laid
// out for qdm_mlp_workspace_bytes(m, act, &gu, &dn) bytes (qdm_api.cpp).
int mlp_decode_in(const void* x, const void* r, int32_t m, int act, const qdm_weight& gu, const qdm_weight& dn,
                  void* workspace, void* out, void* stream);
int launch_add_rmsnorm(const void* a, const void* b, const void* w, int rows, int n, float eps,
                       int dtype, void* s_out, void* n_out, void* stream);

}  // namespace qdm
