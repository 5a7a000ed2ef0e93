// Residual add + RMSNorm with two outputs (s and n), one block per row.
//
// Pages: meTile docs, "Compute-Graph Fusion", opening GraphBuilder example
// (summed = values + residual; normalized = rms_norm(summed, weight, 1e-5);
// summed stays an output, so the lowering is one multi-output kernel);
// "MLX-LM Backend", "Dispatch Policy" (BF16/FP16/FP32 values and weights,
// FP32 accumulation).
//
// Each thread adds its elements in fp32 (exact for f16/bf16 inputs, correctly
// rounded for f32) and rounds the sum once to the storage dtype; the mean
// square of the rounded s is accumulated in fp32 in the fixed order that
// norm_chunk / kNormThreads define (the one-row and few-row decode chains'
// gate/up prologues repeat it, so their n is bitwise this kernel's).  Rows of
// up to kNormThreads * kHeld chunks take one pass: each thread's H chunks of
// a, b and w are loaded at once (16 bytes per load when the row length
// allows; H = the row's chunks / kNormThreads rounded up, a template
// argument, and every load issued unconditionally at a clamped chunk index,
// since a load inside a branch ends the branch with a wait for it), s stays in
// registers, and n = s * w / sqrt(mean + eps), rounded once, is stored with
// s.  Longer rows recompute s in a second pass.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qdm_device.h"
#include "qdm_internal.h"

namespace qdm {
namespace {

constexpr int kThreads = kNormThreads;
constexpr int kHeld = 4;   // chunks per thread held in registers by the one-pass form

__device__ __forceinline__ float block_sum(float ss) {
    __shared__ float red[kThreads / 64];
    ss = wave_total(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < kThreads / 64; ++i) tot += red[i];
    return tot;
}

// The CE = norm_chunk<DT> elements of chunk c of a row starting at element
// base, as fp32 (elements past n read as 0).  VEC: one 16-byte load (the row
// length is a multiple of CE, so chunks are aligned).
template <int DT, bool VEC>
__device__ __forceinline__ void load_chunk(const void* p, int64_t base, int c, int n, float (&v)[norm_chunk<DT>()]) {
    constexpr int CE = norm_chunk<DT>();
    if constexpr (VEC) {
        load_vec<DT, CE>(p, base + static_cast<int64_t>(c) * CE, v);
    } else {
#pragma unroll
        for (int e = 0; e < CE; ++e) {
            const int i = c * CE + e;
            v[e] = i < n ? load_elem<DT>(p, base + i) : 0.f;
        }
    }
}

template <int DT, bool VEC>
__device__ __forceinline__ void store_chunk(void* p, int64_t base, int c, int n, const float (&v)[norm_chunk<DT>()]) {
    constexpr int CE = norm_chunk<DT>();
    if constexpr (VEC && DT == DT_F32) {
        *reinterpret_cast<float4*>(static_cast<float*>(p) + base + static_cast<int64_t>(c) * CE) =
            float4{v[0], v[1], v[2], v[3]};
    } else if constexpr (VEC) {
        uint4 o;
        uint32_t wd[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t lo = DT == DT_BF16 ? f32_to_bf16(v[2 * j]) : f32_to_f16(v[2 * j]);
            const uint32_t hi = DT == DT_BF16 ? f32_to_bf16(v[2 * j + 1]) : f32_to_f16(v[2 * j + 1]);
            wd[j] = lo | (hi << 16);
        }
        o.x = wd[0]; o.y = wd[1]; o.z = wd[2]; o.w = wd[3];
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p) + base + static_cast<int64_t>(c) * CE) = o;
    } else {
#pragma unroll
        for (int e = 0; e < CE; ++e) {
            const int i = c * CE + e;
            if (i < n) store_elem<DT>(p, base + i, v[e]);
        }
    }
}

// H: chunks per thread held in registers (one pass), or 0 (two passes).
template <int DT, bool VEC, int H>
__global__ void __launch_bounds__(kThreads)
add_rmsnorm_kernel(const void* a, const void* b, const void* __restrict__ w,
                   int n, float eps, void* s_out, void* __restrict__ n_out) {
    constexpr int CE = norm_chunk<DT>();
    const int64_t base = static_cast<int64_t>(blockIdx.x) * n;
    const int t = static_cast<int>(threadIdx.x);
    const int nch = (n + CE - 1) / CE;
    // s of chunk c, rounded once, squares accumulated in element order; a chunk
    // that is not live (past the row, loaded at a clamped index) adds nothing.
    // Selects, not branches: a branch around the use lets the compiler sink
    // the chunk's loads into it and wait for each on its own.
    auto sum_chunk = [&](const float (&av)[CE], const float (&bv)[CE], float (&sv)[CE], int c, bool live, float& ss) {
#pragma unroll
        for (int e = 0; e < CE; ++e) {
            sv[e] = round_trip<DT>(av[e] + bv[e]);
            const float sq = fmaf(sv[e], sv[e], ss);
            ss = live && c * CE + e < n ? sq : ss;
        }
    };
    float ss = 0.f;
    if constexpr (H > 0) {
        float sv[H][CE], wv[H][CE];
        {
            float av[H][CE], bv[H][CE];
#pragma unroll
            for (int j = 0; j < H; ++j) {   // every load in flight together
                const int c = min(t + j * kThreads, nch - 1);
                load_chunk<DT, VEC>(a, base, c, n, av[j]);
                load_chunk<DT, VEC>(b, base, c, n, bv[j]);
                load_chunk<DT, VEC>(w, 0, c, n, wv[j]);
            }
#pragma unroll
            for (int j = 0; j < H; ++j) sum_chunk(av[j], bv[j], sv[j], t + j * kThreads, t + j * kThreads < nch, ss);
        }
        const float inv = 1.0f / sqrtf(block_sum(ss) / static_cast<float>(n) + eps);
#pragma unroll
        for (int j = 0; j < H; ++j) {
            const int c = t + j * kThreads;
            if (c < nch) {
                float nv[CE];
#pragma unroll
                for (int e = 0; e < CE; ++e) nv[e] = sv[j][e] * inv * wv[j][e];
                store_chunk<DT, VEC>(s_out, base, c, n, sv[j]);
                store_chunk<DT, VEC>(n_out, base, c, n, nv);
            }
        }
    } else {
        for (int c = t; c < nch; c += kThreads) {
            float av[CE], bv[CE], sv[CE];
            load_chunk<DT, VEC>(a, base, c, n, av);
            load_chunk<DT, VEC>(b, base, c, n, bv);
            sum_chunk(av, bv, sv, c, true, ss);
        }
        const float inv = 1.0f / sqrtf(block_sum(ss) / static_cast<float>(n) + eps);
        for (int c = t; c < nch; c += kThreads) {
            float av[CE], bv[CE], wv[CE], sv[CE], nv[CE];
            load_chunk<DT, VEC>(a, base, c, n, av);
            load_chunk<DT, VEC>(b, base, c, n, bv);
            load_chunk<DT, VEC>(w, 0, c, n, wv);
            float dummy = 0.f;
            sum_chunk(av, bv, sv, c, true, dummy);
#pragma unroll
            for (int e = 0; e < CE; ++e) nv[e] = sv[e] * inv * wv[e];
            store_chunk<DT, VEC>(s_out, base, c, n, sv);
            store_chunk<DT, VEC>(n_out, base, c, n, nv);
        }
    }
}

template <int DT, bool VEC>
int run_v(const void* a, const void* b, const void* w, int rows, int n, float eps, void* s_out, void* n_out,
          hipStream_t s) {
    const dim3 grid(rows), block(kThreads);
    static_assert(kHeld == 4, "one-pass instances for 1..4 chunks per thread");
    const int nch = (n + norm_chunk<DT>() - 1) / norm_chunk<DT>();
    switch ((nch + kThreads - 1) / kThreads) {
        case 0:
        case 1: return launch(add_rmsnorm_kernel<DT, VEC, 1>, grid, block, 0, s, a, b, w, n, eps, s_out, n_out);
        case 2: return launch(add_rmsnorm_kernel<DT, VEC, 2>, grid, block, 0, s, a, b, w, n, eps, s_out, n_out);
        case 3: return launch(add_rmsnorm_kernel<DT, VEC, 3>, grid, block, 0, s, a, b, w, n, eps, s_out, n_out);
        case 4: return launch(add_rmsnorm_kernel<DT, VEC, 4>, grid, block, 0, s, a, b, w, n, eps, s_out, n_out);
        default: return launch(add_rmsnorm_kernel<DT, VEC, 0>, grid, block, 0, s, a, b, w, n, eps, s_out, n_out);
    }
}

template <int DT>
int run(const void* a, const void* b, const void* w, int rows, int n, float eps, void* s_out, void* n_out,
        hipStream_t s) {
    if (n % norm_chunk<DT>() == 0) return run_v<DT, true>(a, b, w, rows, n, eps, s_out, n_out, s);
    return run_v<DT, false>(a, b, w, rows, n, eps, s_out, n_out, s);
}

}  // namespace

int launch_add_rmsnorm(const void* a, const void* b, const void* w, int rows, int n, float eps, int dtype,
                       void* s_out, void* n_out, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (dtype) {
        case DT_F32: return run<DT_F32>(a, b, w, rows, n, eps, s_out, n_out, s);
        case DT_F16: return run<DT_F16>(a, b, w, rows, n, eps, s_out, n_out, s);
        default: return run<DT_BF16>(a, b, w, rows, n, eps, s_out, n_out, s);
    }
}

}  // namespace qdm
