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
int launch_down_residual(const float* h, const void* r, int m, int act, const qdm_weight& dn,
                         void* out, void* stream);
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
// with the partials in a device scratch the library allocates on first use
// (qdm_mma_down.hip).
bool mma_stream_down_supported(const qdm_weight& w, int m, int act);
// r_copy: when not null, also receives r (the decode chain's s).
int launch_down_mma_stream(const float* h, const void* r, int m, int act, const qdm_weight& dn, void* out,
                           void* stream, void* r_copy = nullptr);
// One row, both projections on the streaming kernels: the decode chain with
// add + RMSNorm folded into the MLP's two launches (qdm_chain.hip).
bool chain_stream_supported(const qdm_weight& gu, const qdm_weight& dn, int act);
int launch_mlp_chain_stream(const void* a, const void* b, const void* w, float eps, int act, const qdm_weight& gu,
                            const qdm_weight& dn, float* h, void* s_out, void* out, void* stream);
// The device's fp32 partials buffer (at least bytes), shared by the split-K
// kernels; grows outside graph capture only.  Null with err set on failure.
float* partials_scratch(size_t bytes, void* stream, int& err);
// More than 16 rows, 8/4-bit affine (either pair storage) or MX weights, 16-bit
// activations: tiled dual GEMM, 64 rows x 64 outputs per block (qdm_prefill.hip).
bool prefill_supported(const qdm_weight& w, int m, int act);
int launch_gate_up_prefill(const void* x, int m, int act, const qdm_weight& gu, float* h, void* stream);
int launch_down_prefill(const float* h, const void* r, int m, int act, const qdm_weight& dn, void* out, void* stream);
int launch_add_rmsnorm(const void* a, const void* b, const void* w, int rows, int n, float eps,
                       int dtype, void* s_out, void* n_out, void* stream);

}  // namespace qdm
