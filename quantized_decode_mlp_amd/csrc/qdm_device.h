// Device-side helpers shared by the gfx950 kernels: dtype loads/stores,
// wave64 reductions, and a launch wrapper that reports hipError_t.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <utility>

namespace qdm {

enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

template <int DT> struct DType;
template <> struct DType<DT_F32> { using T = float; };
template <> struct DType<DT_F16> { using T = uint16_t; };
template <> struct DType<DT_BF16> { using T = uint16_t; };

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
    _Float16 h = __builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16));
    return static_cast<float>(h);
}

// Nearest-even fp32 -> bf16: gfx950's v_cvt_pk_bf16_f32 under the default
// round mode (a NaN stays a NaN).  One instruction; the integer form (add
// 0x7fff plus the kept lsb, with a NaN test) compiled to a dozen scalar and
// vector instructions with exec-mask branching per element.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Nearest-even fp32 -> f16 (the hardware conversion rounds to nearest-even).
__device__ __forceinline__ uint16_t f32_to_f16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

template <int DT>
__device__ __forceinline__ float load_elem(const void* p, int64_t i) {
    if constexpr (DT == DT_F32) return static_cast<const float*>(p)[i];
    else if constexpr (DT == DT_BF16) return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
    else return f16_to_f32(static_cast<const uint16_t*>(p)[i]);
}

template <int DT>
__device__ __forceinline__ void store_elem(void* p, int64_t i, float v) {
    if constexpr (DT == DT_F32) static_cast<float*>(p)[i] = v;
    else if constexpr (DT == DT_BF16) static_cast<uint16_t*>(p)[i] = f32_to_bf16(v);
    else static_cast<uint16_t*>(p)[i] = f32_to_f16(v);
}

// v rounded once (nearest-even) to DT and back to fp32.
template <int DT>
__device__ __forceinline__ float round_trip(float v) {
    if constexpr (DT == DT_F32) return v;
    else if constexpr (DT == DT_BF16) return bf16_to_f32(f32_to_bf16(v));
    else return f16_to_f32(f32_to_f16(v));
}

// Element-wise f over the activation-type values packed in two dwords (one
// fp32 value, or two 16-bit values low half first); the results are rounded
// once to the type and packed the same way.
template <int DT, typename F>
__device__ __forceinline__ uint32_t dword_map(uint32_t xa, uint32_t xb, F f) {
    if constexpr (DT == DT_F32) {
        return __float_as_uint(f(__uint_as_float(xa), __uint_as_float(xb)));
    } else {
        auto val = [](uint32_t h) { return DT == DT_BF16 ? bf16_to_f32(h) : f16_to_f32(h); };
        auto bits = [](float v) -> uint32_t { return DT == DT_BF16 ? f32_to_bf16(v) : f32_to_f16(v); };
        const uint32_t lo = bits(f(val(xa & 0xffffu), val(xb & 0xffffu)));
        const uint32_t hi = bits(f(val(xa >> 16), val(xb >> 16)));
        return lo | (hi << 16);
    }
}

// The sum-of-squares order of add + RMSNorm, shared by the standalone kernel
// and the decode chain's gate/up prologues (which must reproduce its n bit for
// bit): thread t of kNormThreads takes the 16-byte chunks t, t + kNormThreads,
// ... of the row (norm_chunk<DT> elements each) and accumulates the squares of
// their elements in index order with fmaf; the lanes of each wave are then
// summed by wave_total and the kNormThreads / 64 wave sums in wave order.
constexpr int kNormThreads = 256;
template <int DT>
__host__ __device__ constexpr int norm_chunk() { return DT == DT_F32 ? 4 : 8; }

// Loads N consecutive elements (N * sizeof(elem) in {4, 8, 16, 32} bytes, aligned
// to min(16, that size)) as fp32.
template <int DT, int N>
__device__ __forceinline__ void load_vec(const void* base, int64_t i, float (&out)[N]) {
    if constexpr (DT == DT_F32) {
        const float* p = static_cast<const float*>(base) + i;
        if constexpr (N % 4 == 0) {
#pragma unroll
            for (int j = 0; j < N; j += 4) {
                float4 v = *reinterpret_cast<const float4*>(p + j);
                out[j] = v.x; out[j + 1] = v.y; out[j + 2] = v.z; out[j + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int j = 0; j < N; j += 2) {
                float2 v = *reinterpret_cast<const float2*>(p + j);
                out[j] = v.x; out[j + 1] = v.y;
            }
        }
    } else {
        const uint16_t* p = static_cast<const uint16_t*>(base) + i;
        uint32_t w[N / 2];
        if constexpr (N % 8 == 0) {
#pragma unroll
            for (int j = 0; j < N; j += 8) {
                uint4 v = *reinterpret_cast<const uint4*>(p + j);
                w[j / 2] = v.x; w[j / 2 + 1] = v.y; w[j / 2 + 2] = v.z; w[j / 2 + 3] = v.w;
            }
        } else if constexpr (N % 4 == 0) {
#pragma unroll
            for (int j = 0; j < N; j += 4) {
                uint2 v = *reinterpret_cast<const uint2*>(p + j);
                w[j / 2] = v.x; w[j / 2 + 1] = v.y;
            }
        } else {
#pragma unroll
            for (int j = 0; j < N; j += 2) w[j / 2] = *reinterpret_cast<const uint32_t*>(p + j);
        }
#pragma unroll
        for (int j = 0; j < N / 2; ++j) {
            if constexpr (DT == DT_BF16) {
                out[2 * j] = __uint_as_float(w[j] << 16);
                out[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
            } else {
                out[2 * j] = f16_to_f32(w[j] & 0xffffu);
                out[2 * j + 1] = f16_to_f32(w[j] >> 16);
            }
        }
    }
}

// Sum over the 64 lanes of a wave with DPP row steps (xor 1, xor 2, half-row
// mirror, row mirror) and the four row sums read back from lanes 0/16/32/48;
// the result is wave-uniform.  Fixed order, so bitwise reproducible.
__device__ __forceinline__ float dpp_add(float v, int ctrl_sel) {
    int x = __builtin_bit_cast(int, v);
    int y;
    switch (ctrl_sel) {
        case 0: y = __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false); break;   // quad_perm 1,0,3,2
        case 1: y = __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false); break;   // quad_perm 2,3,0,1
        case 2: y = __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false); break;  // row_half_mirror
        default: y = __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false); break; // row_mirror
    }
    return v + __builtin_bit_cast(float, y);
}

__device__ __forceinline__ float wave_total(float v) {
    v = dpp_add(v, 0);
    v = dpp_add(v, 1);
    v = dpp_add(v, 2);
    v = dpp_add(v, 3);
    const int x = __builtin_bit_cast(int, v);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(x, 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(x, 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(x, 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(x, 48));
    return (r0 + r1) + (r2 + r3);
}

// Sum over the 64 lanes of a wave; every lane gets the total.  Fixed order.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// hipLaunchKernel with the kernel's own parameter types; returns its hipError_t.
template <typename... KArgs, typename... Args, size_t... I>
hipError_t launch_impl(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shmem,
                       hipStream_t stream, std::index_sequence<I...>, Args&&... args) {
    std::tuple<KArgs...> held(std::forward<Args>(args)...);
    void* argv[] = {static_cast<void*>(&std::get<I>(held))..., nullptr};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, shmem, stream);
}

template <typename... KArgs, typename... Args>
hipError_t launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shmem, hipStream_t stream,
                  Args&&... args) {
    static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
    return launch_impl(kernel, grid, block, shmem, stream, std::index_sequence_for<KArgs...>{},
                       std::forward<Args>(args)...);
}

}  // namespace qdm
