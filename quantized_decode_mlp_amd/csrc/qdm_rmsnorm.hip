// Residual add + RMSNorm with two outputs (s and n), one block per row.
//
// Pages: meTile docs, "Compute-Graph Fusion", opening GraphBuilder example
// (summed = values + residual; normalized = rms_norm(summed, weight, 1e-5);
// summed stays an output, so the lowering is one multi-output kernel);
// "MLX-LM Backend", "Dispatch Policy" (BF16/FP16/FP32 values and weights,
// FP32 accumulation).
//
// Each thread adds its elements in fp32 (exact for f16/bf16 inputs, correctly
// rounded for f32), rounds the sum once to the storage dtype and writes s;
// the mean square of the rounded s is accumulated in fp32 and reduced across
// the block in a fixed order; the second pass recomputes the same s and
// writes n = s * w / sqrt(mean + eps), rounded once.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qdm_device.h"
#include "qdm_internal.h"

namespace qdm {
namespace {

constexpr int kThreads = 256;

template <int DT>
__global__ void __launch_bounds__(kThreads)
add_rmsnorm_kernel(const void* a, const void* b, const void* __restrict__ w,
                   int n, float eps, void* s_out, void* __restrict__ n_out) {
    const int64_t base = static_cast<int64_t>(blockIdx.x) * n;
    float ss = 0.f;
    for (int i = threadIdx.x; i < n; i += kThreads) {
        const float s = round_trip<DT>(load_elem<DT>(a, base + i) + load_elem<DT>(b, base + i));
        ss = fmaf(s, s, ss);
    }
    __shared__ float red[kThreads / 64];
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < kThreads / 64; ++i) tot += red[i];
    const float inv = 1.0f / sqrtf(tot / static_cast<float>(n) + eps);
    for (int i = threadIdx.x; i < n; i += kThreads) {
        const float s = round_trip<DT>(load_elem<DT>(a, base + i) + load_elem<DT>(b, base + i));
        store_elem<DT>(s_out, base + i, s);
        store_elem<DT>(n_out, base + i, s * inv * load_elem<DT>(w, i));
    }
}

}  // namespace

int launch_add_rmsnorm(const void* a, const void* b, const void* w, int rows, int n, float eps, int dtype,
                       void* s_out, void* n_out, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    dim3 grid(rows), block(kThreads);
    switch (dtype) {
        case DT_F32: return launch(add_rmsnorm_kernel<DT_F32>, grid, block, 0, s, a, b, w, n, eps, s_out, n_out);
        case DT_F16: return launch(add_rmsnorm_kernel<DT_F16>, grid, block, 0, s, a, b, w, n, eps, s_out, n_out);
        default: return launch(add_rmsnorm_kernel<DT_BF16>, grid, block, 0, s, a, b, w, n, eps, s_out, n_out);
    }
}

}  // namespace qdm
