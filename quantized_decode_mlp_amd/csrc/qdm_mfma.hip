// Few-row (2..16 rows) decode MLP projections on gfx950 matrix cores.
//
// Pages: meTile docs, "MLX-LM Backend", section "Dispatch Policy": for one
// token a 16-row matrix tile wastes most of its rows, so the one-row path
// stays on vector units; multi-row calls run a fused dual GEMM (gate and up
// reuse each activation fragment, SwiGLU on the accumulators, only the final
// hidden tile is stored) with row-masked loads and stores for ragged tiles.
//
// v_mfma_f32_16x16x32_bf16 computes D[16 m][16 n] += A[16 m][32 k] * B[32 k][16 n];
// lane l holds A row l%16 / B column l%16 at k = (l/16)*8 + 0..7 and D rows
// (l/16)*4 + 0..3 of column l%16.  Here A is the activation rows (rows past
// the caller's m are zero) and B the weight rows, so a wave computes a 16 x 16
// output tile.
//
// Exactness: the codes enter the MMA as exact bf16 integers (0..255 fit in
// bf16), converted with v_cvt_f32_ubyte and a byte permute (no
// dequantization before the MMA).  Each quantization group's 16 x 16 partial
// P = X Q^T is folded in fp32 as scale * P + bias * sum_k X, the per-row sums
// coming from one more MMA against a block of ones.  Activations in bf16 are
// exact operands; the fp32 hidden row of the down projection is split into a
// bf16 high part and a bf16 low part (h = hi + lo to about 16 significant
// bits) and both go through the MMA.
//
// Work split: a block is S waves holding the same NT output tiles, each wave a
// contiguous 1/S of the quantization groups along K, with the next kStages
// groups' loads in flight (a rolling register pipeline).  The S partial tiles
// meet in LDS and are summed in wave order; wave 0 applies the epilogue.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qdm_device.h"
#include "qdm_internal.h"
#include "qdm_launch.h"

namespace qdm {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kMmaStages = 4;   // k-blocks in flight per wave

// Byte i of w as fp32 (selects v_cvt_f32_ubyte<i>).
template <int I>
__device__ __forceinline__ float ubyte_f32(uint32_t w) { return static_cast<float>((w >> (8 * I)) & 0xffu); }

// Packs the high halves of two fp32 values (exact bf16 values) into one dword:
// element 0 (low half) = a, element 1 = b.
__device__ __forceinline__ uint32_t pack_hi16(float a, float b) {
    return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}

// 8 codes (one packed k-slot of a lane) -> bf16x8 operand, element i = code of k + i.
template <int BITS>
struct Codes;

template <>
struct Codes<4> {
    using raw = uint32_t;   // 8 nibbles, low nibble first
    __device__ __forceinline__ static bf16x8 to_bf16(raw w) {
        const uint32_t lo = w & 0x0F0F0F0Fu;          // codes 0, 2, 4, 6
        const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;   // codes 1, 3, 5, 7
        u32x4 r;
        r[0] = pack_hi16(ubyte_f32<0>(lo), ubyte_f32<0>(hi));
        r[1] = pack_hi16(ubyte_f32<1>(lo), ubyte_f32<1>(hi));
        r[2] = pack_hi16(ubyte_f32<2>(lo), ubyte_f32<2>(hi));
        r[3] = pack_hi16(ubyte_f32<3>(lo), ubyte_f32<3>(hi));
        return __builtin_bit_cast(bf16x8, r);
    }
};

template <>
struct Codes<8> {
    using raw = u32x2;      // 8 bytes
    __device__ __forceinline__ static bf16x8 to_bf16(raw w) {
        u32x4 r;
        r[0] = pack_hi16(ubyte_f32<0>(w[0]), ubyte_f32<1>(w[0]));
        r[1] = pack_hi16(ubyte_f32<2>(w[0]), ubyte_f32<3>(w[0]));
        r[2] = pack_hi16(ubyte_f32<0>(w[1]), ubyte_f32<1>(w[1]));
        r[3] = pack_hi16(ubyte_f32<2>(w[1]), ubyte_f32<3>(w[1]));
        return __builtin_bit_cast(bf16x8, r);
    }
};

template <>
struct Codes<16> {
    using raw = u32x4;      // 8 bf16 weights
    __device__ __forceinline__ static bf16x8 to_bf16(raw w) { return __builtin_bit_cast(bf16x8, w); }
};

__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Activation fragment of one k-step (32 k) for the lane: bf16 rows of x, or
// the hi/lo split of fp32 h.
template <bool SPLIT>
struct Frag;

template <>
struct Frag<false> {
    u32x4 v;   // 8 bf16
    __device__ __forceinline__ void load(const void* base, int64_t off, bool live) {
        v = live ? *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + off) : u32x4{0, 0, 0, 0};
    }
    __device__ __forceinline__ bf16x8 hi() const { return __builtin_bit_cast(bf16x8, v); }
};

template <>
struct Frag<true> {
    f32x4 a, b;   // 8 fp32
    __device__ __forceinline__ void load(const void* base, int64_t off, bool live) {
        const float* p = static_cast<const float*>(base) + off;
        a = live ? *reinterpret_cast<const f32x4*>(p) : f32x4{0.f, 0.f, 0.f, 0.f};
        b = live ? *reinterpret_cast<const f32x4*>(p + 4) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // high part: the top 16 bits of each value (truncation)
    __device__ __forceinline__ bf16x8 hi() const {
        u32x4 r;
        r[0] = pack_hi16(a[0], a[1]); r[1] = pack_hi16(a[2], a[3]);
        r[2] = pack_hi16(b[0], b[1]); r[3] = pack_hi16(b[2], b[3]);
        return __builtin_bit_cast(bf16x8, r);
    }
    // low part: the exact remainder h - hi, truncated to bf16
    __device__ __forceinline__ bf16x8 lo() const {
        auto rem = [](float v) { return v - __uint_as_float(__float_as_uint(v) & 0xffff0000u); };
        u32x4 r;
        r[0] = pack_hi16(rem(a[0]), rem(a[1])); r[1] = pack_hi16(rem(a[2]), rem(a[3]));
        r[2] = pack_hi16(rem(b[0]), rem(b[1])); r[3] = pack_hi16(rem(b[2]), rem(b[3]));
        return __builtin_bit_cast(bf16x8, r);
    }
};

// Codes per 16-byte lane chunk, and MMA steps (8 codes per lane each) in it.
template <int BITS>
struct Chunk {
    static constexpr int LU = 128 / BITS;    // codes per lane chunk: 32, 16 or 8
    static constexpr int STEPS = LU / 8;     // MMA steps per chunk: 4, 2, 1
    static constexpr int KB = 4 * LU;        // k per block (the four k sub-slots of a wave)
};

// 8 codes of MMA step t from a lane's 16-byte chunk.
template <int BITS>
__device__ __forceinline__ bf16x8 chunk_codes(const u32x4& c, int t) {
    if constexpr (BITS == 4) return Codes<4>::to_bf16(c[t]);
    else if constexpr (BITS == 8) return Codes<8>::to_bf16(u32x2{c[2 * t], c[2 * t + 1]});
    else return Codes<16>::to_bf16(c);
}

// Keeps the fragment only on lanes whose k sub-slot belongs to quantization
// sub-group j of the block (sub-groups of width g inside a KB-wide block).
__device__ __forceinline__ bf16x8 lane_mask(bf16x8 v, bool keep) {
    const u32x4 u = __builtin_bit_cast(u32x4, v);
    return __builtin_bit_cast(bf16x8, keep ? u : u32x4{0u, 0u, 0u, 0u});
}

// GU: rows are gate/up pairs (packed rows 2n, 2n+1), x bf16, output h fp32 [m][N] = silu(g) * u.
// !GU: rows are down rows, input h fp32 (split hi/lo), output [m][N] = r + acc in ODT.
// G: quantization group (0 for dense).  A k-block is KB consecutive k of every
// row: lane (n, kg) loads its 16-byte chunk kg of the block (one instruction
// reads 16 rows x 64 contiguous bytes), and MMA step t takes codes
// kg*LU + 8t + 0..7 of the block from each lane; the activation fragment
// follows the same k assignment.  When a block spans NGB = KB/G groups, each
// group gets its own MMA with the activation masked to that group's lanes.
template <int BITS, int ODT, bool GU, int G, int S, int NT>
__global__ void __launch_bounds__(64 * S)
qmm_kernel(const uint8_t* __restrict__ q, const float* __restrict__ sb, const void* __restrict__ xin,
           const void* __restrict__ resid, void* __restrict__ out, int N, int K, int m_rows) {
    constexpr bool AFFINE = BITS != 16;
    constexpr bool SPLIT = !GU;
    constexpr int NV = GU ? 2 : 1;
    constexpr int LU = Chunk<BITS>::LU, STEPS = Chunk<BITS>::STEPS, KB = Chunk<BITS>::KB;
    constexpr int NGB = (AFFINE && G < KB) ? KB / G : 1;   // groups inside one k-block
    // large stages (the fp32 hidden row split in two, or four groups per block)
    // keep two k-blocks in flight so the registers do not spill
    constexpr int U = (SPLIT && STEPS > 1) || NGB > 2 ? 2 : kMmaStages;

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int li = lane & 15;         // A row m / B column n of this lane
    const int kg = lane >> 4;         // k sub-slot of the lane inside a block
    const int nblocks = K / KB;
    const int bpw = nblocks / S;      // k-blocks per wave (host guarantees divisibility)
    const int b_begin = w * bpw;
    const uint32_t rb = static_cast<uint32_t>(K) * BITS / 8;   // bytes per packed row
    const int ngroups = AFFINE ? K / G : 1;
    const int n_tile0 = blockIdx.x * NT * 16;
    const int my_sub = AFFINE && NGB > 1 ? (kg * LU) / G : 0;  // this lane's group inside a block

    const bool live = li < m_rows;    // activation rows past m_rows are zero
    const int64_t xrow = static_cast<int64_t>(live ? li : 0) * K;

    struct Stage {
        Frag<SPLIT> x[STEPS];
        u32x4 c[NT][NV];
        f32x2 p[NT][NV][NGB];
    };
    Stage st[U];

    auto issue = [&](Stage& s, int blk) {
#pragma unroll
        for (int t = 0; t < STEPS; ++t)
            s.x[t].load(xin, xrow + static_cast<int64_t>(blk) * KB + kg * LU + 8 * t, live);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int n = n_tile0 + nt * 16 + li;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const uint32_t row = GU ? 2u * static_cast<uint32_t>(n) + v : static_cast<uint32_t>(n);
                const uint8_t* qrow = q + static_cast<size_t>(row) * rb;
                s.c[nt][v] = *reinterpret_cast<const u32x4*>(qrow + static_cast<uint32_t>(blk) * (KB * BITS / 8) + kg * 16u);
                if constexpr (AFFINE) {
#pragma unroll
                    for (int j = 0; j < NGB; ++j) {
                        const int grp = (blk * KB) / G + j;
                        s.p[nt][v][j] = *reinterpret_cast<const f32x2*>(sb + 2 * (static_cast<size_t>(row) * ngroups + grp));
                    }
                }
            }
        }
    };

    f32x4 acc[NT][NV];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int v = 0; v < NV; ++v) acc[nt][v] = f32x4{0.f, 0.f, 0.f, 0.f};

    const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});

    auto compute = [&](const Stage& s) {
        // activation operands per step; per-group lane masks are applied on the fly
        bf16x8 xh[STEPS], xl[STEPS];
#pragma unroll
        for (int t = 0; t < STEPS; ++t) {
            xh[t] = s.x[t].hi();
            if constexpr (SPLIT) xl[t] = s.x[t].lo();
        }
        bf16x8 b[NT][NV][STEPS];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int v = 0; v < NV; ++v)
#pragma unroll
                for (int t = 0; t < STEPS; ++t) b[nt][v][t] = chunk_codes<BITS>(s.c[nt][v], t);
        if constexpr (!AFFINE) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int v = 0; v < NV; ++v)
#pragma unroll
                    for (int t = 0; t < STEPS; ++t) {
                        acc[nt][v] = mma(xh[t], b[nt][v][t], acc[nt][v]);
                        if constexpr (SPLIT) acc[nt][v] = mma(xl[t], b[nt][v][t], acc[nt][v]);
                    }
        } else {
#pragma unroll
            for (int j = 0; j < NGB; ++j) {
                const bool keep = NGB == 1 || my_sub == j;
                f32x4 xs = {0.f, 0.f, 0.f, 0.f};
                f32x4 part[NT][NV];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int v = 0; v < NV; ++v) part[nt][v] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int t = 0; t < STEPS; ++t) {
                    const bf16x8 ah = NGB > 1 ? lane_mask(xh[t], keep) : xh[t];
                    xs = mma(ah, ones, xs);
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                        for (int v = 0; v < NV; ++v) part[nt][v] = mma(ah, b[nt][v][t], part[nt][v]);
                    if constexpr (SPLIT) {
                        const bf16x8 al = NGB > 1 ? lane_mask(xl[t], keep) : xl[t];
                        xs = mma(al, ones, xs);
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                            for (int v = 0; v < NV; ++v) part[nt][v] = mma(al, b[nt][v][t], part[nt][v]);
                    }
                }
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int v = 0; v < NV; ++v) {
                        const float sc = s.p[nt][v][j].x, bi = s.p[nt][v][j].y;
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            acc[nt][v][i] = fmaf(sc, part[nt][v][i], fmaf(bi, xs[i], acc[nt][v][i]));
                    }
            }
        }
    };

    // rolling pipeline over this wave's k-blocks
#pragma unroll
    for (int u = 0; u < U; ++u)
        if (u < bpw) issue(st[u], b_begin + u);
    for (int base = 0; base < bpw; base += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = base + u;
            if (i < bpw) {
                compute(st[u]);
                if (i + U < bpw) issue(st[u], b_begin + i + U);
            }
        }
    }

    // combine the S partial tiles in wave order, then the epilogue
    __shared__ f32x4 part[S > 1 ? S - 1 : 1][NT][NV][64];
    if constexpr (S > 1) {
        if (w > 0) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int v = 0; v < NV; ++v) part[w - 1][nt][v][lane] = acc[nt][v];
        }
        __syncthreads();
        if (w != 0) return;
#pragma unroll
        for (int s = 0; s < S - 1; ++s)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    const f32x4 o = part[s][nt][v][lane];
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[nt][v][i] += o[i];
                }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int n = n_tile0 + nt * 16 + li;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = kg * 4 + i;
            if (m < m_rows) {
                const int64_t o = static_cast<int64_t>(m) * N + n;
                if constexpr (GU) {
                    const float g = acc[nt][0][i];
                    static_cast<float*>(out)[o] = g / (1.0f + expf(-g)) * acc[nt][NV - 1][i];
                } else {
                    store_elem<ODT>(out, o, load_elem<ODT>(resid, o) + acc[nt][0][i]);
                }
            }
        }
    }
}

// Waves per block along K: the largest of 8, 4, 2, 1 that divides the k-block
// count and leaves each wave at least two k-blocks.
int pick_split(int nblocks) {
    for (int s = 8; s > 1; s >>= 1)
        if (nblocks % s == 0 && nblocks / s >= 2) return s;
    return 1;
}

template <int BITS, int ODT, bool GU, int G, int S>
int run_s(const qdm_weight& w, const void* x, const void* r, void* out, int N, int K, int m, hipStream_t s) {
    constexpr int NT = 1;
    dim3 grid(N / (16 * NT)), block(64 * S);
    return static_cast<int>(launch(qmm_kernel<BITS, ODT, GU, G, S, NT>, grid, block, 0, s,
                                   static_cast<const uint8_t*>(w.q), w.scale_bias, x, r, out, N, K, m));
}

template <int BITS, int ODT, bool GU, int G>
int run_g(const qdm_weight& w, const void* x, const void* r, void* out, int N, int K, int m, hipStream_t s) {
    switch (pick_split(K / Chunk<BITS>::KB)) {
        case 8: return run_s<BITS, ODT, GU, G, 8>(w, x, r, out, N, K, m, s);
        case 4: return run_s<BITS, ODT, GU, G, 4>(w, x, r, out, N, K, m, s);
        case 2: return run_s<BITS, ODT, GU, G, 2>(w, x, r, out, N, K, m, s);
        default: return run_s<BITS, ODT, GU, G, 1>(w, x, r, out, N, K, m, s);
    }
}

template <int BITS, int ODT, bool GU>
int run_bits(const qdm_weight& w, const void* x, const void* r, void* out, int N, int K, int m, hipStream_t s) {
    if constexpr (BITS == 16) {
        return run_g<16, ODT, GU, 0>(w, x, r, out, N, K, m, s);
    } else {
        switch (w.group) {
            case 32: return run_g<BITS, ODT, GU, 32>(w, x, r, out, N, K, m, s);
            case 64: return run_g<BITS, ODT, GU, 64>(w, x, r, out, N, K, m, s);
            default: return run_g<BITS, ODT, GU, 128>(w, x, r, out, N, K, m, s);
        }
    }
}

template <int ODT, bool GU>
int run_fmt(const qdm_weight& w, const void* x, const void* r, void* out, int N, int K, int m, hipStream_t s) {
    switch (w.bits) {
        case 8: return run_bits<8, ODT, GU>(w, x, r, out, N, K, m, s);
        case 4: return run_bits<4, ODT, GU>(w, x, r, out, N, K, m, s);
        default: return run_bits<16, ODT, GU>(w, x, r, out, N, K, m, s);
    }
}

}  // namespace

bool mma_rows_supported(const qdm_weight& w, int m) {
    // 2..16 rows, output width a whole number of 16-wide tiles, K a whole number of k-blocks
    const int kb = w.bits == 4 ? Chunk<4>::KB : w.bits == 8 ? Chunk<8>::KB : Chunk<16>::KB;
    return m >= 2 && m <= 16 && w.n % 16 == 0 && w.k % kb == 0;
}

int launch_gate_up_mma(const void* x, int m, const qdm_weight& gu, float* h, void* stream) {
    return run_fmt<DT_F32, true>(gu, x, nullptr, h, gu.n, gu.k, m, static_cast<hipStream_t>(stream));
}

int launch_down_mma(const float* h, const void* r, int m, int act, const qdm_weight& dn, void* out, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (act) {
        case DT_F32: return run_fmt<DT_F32, false>(dn, h, r, out, dn.n, dn.k, m, s);
        case DT_F16: return run_fmt<DT_F16, false>(dn, h, r, out, dn.n, dn.k, m, s);
        default: return run_fmt<DT_BF16, false>(dn, h, r, out, dn.n, dn.k, m, s);
    }
}

}  // namespace qdm
