// Few-row (2..16 rows) gate/up projection with 8/4-bit affine weights on the
// gfx950 matrix cores, weights streamed once by persistent blocks.
//
// Pages: meTile docs, "MLX-LM Backend", section "Dispatch Policy": calls with
// several activation rows run a fused dual GEMM in which gate and up reuse
// every activation fragment, SwiGLU is applied to the accumulators and only
// the final hidden tile is stored; ragged row counts are masked inside the
// 16-row matrix tile.  Quantization: MLX-LM affine groups, w = scale * q + bias
// per group of G consecutive k of a row.
//
// Matrix-core form: v_mfma_f32_16x16x32_f16 computes D[16 m][16 n] +=
// A[16 m][32 k] * B[32 k][16 n].  Lane l supplies A row m = l % 16 and B column
// n = l % 16 for the eight k of slot kq = l / 16, and holds D rows
// 4 kq + 0..3 of column l % 16.  A is the activation rows (rows at or past the
// caller's m are zero), B a tile of 16 weight rows.
//
// Exact operands.  A code enters B as an exact f16 value by placing its bits
// in the mantissa under a fixed exponent: an 8-bit code c gives 1024 + c (one
// byte permute per two codes), a 4-bit code c gives 1 + c/16 (a shift and an
// and-or per two codes; the small offset keeps the fp32 accumulation far from
// cancellation).  The activations are staged once per block in LDS as f16
// after a per-row power-of-two scale that puts the row's largest magnitude in
// [2^14, 2^15): bf16 and f16 values convert exactly unless they lie more than
// 2^28 below that maximum.  For each fold chunk of k (one quantization group,
// or 64 k when the group is wider) the partial tile P = sum (off + mul c) x'
// is folded in fp32 as
//     acc += (scale / mul) * (P - off * X') + bias * X',
// X' the chunk's sum of the staged activations (kept in LDS), so no weight is
// dequantized before the MMA.  The row scale comes off in the epilogue.
//
// Lane k assignment inside a 64-wide k-block: with groups of 64 or more, lane
// kq holds k 16 kq + 8 t + e for k-steps t = 0, 1 (one 8- or 16-byte load per
// row); with 32-wide groups it holds k 32 t + 8 kq + e (one load per step), so
// that every k-step lies in one group.
//
// Work split: a block is S x P waves.  Wave (ks, p) takes 16-row tiles
// b*P + p + i*G*P (G = grid size) and, of each tile, the 64-wide k-blocks
// ks, ks + S, ks + 2S, ...; the next U k-blocks (crossing into the next tile)
// are always in flight.  The S partial tiles meet in LDS and are summed in
// wave order.  In the packed gate/up layout rows 2n and 2n + 1 are gate and up
// of output n, so one tile reads 32 packed rows.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qdm_device.h"
#include "qdm_internal.h"
#include "qdm_launch.h"

namespace qdm {
namespace {

typedef _Float16 h16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kRows = 16;     // rows of the matrix tile
constexpr int kPad = 8;       // f16 padding per staged row: 16 bytes, four LDS banks per row
constexpr int kLdsCap = 160 * 1024;

__device__ __forceinline__ f32x4 mma_f16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h16x8, a), __builtin_bit_cast(h16x8, b), c, 0,
                                                  0, 0);
}

// The eight codes of one lane and k-step as f16 operand values off + mul * c.
template <int BITS>
struct StepCodes;

template <>
struct StepCodes<8> {
    using raw = u32x2;     // codes k + 0..7, one byte each
    using words = u32x4;   // two k-steps
    __device__ __forceinline__ static raw step(const words& w, int t) { return u32x2{w[2 * t], w[2 * t + 1]}; }
    __device__ __forceinline__ static void set_step(words& w, int t, raw r) {
        w[2 * t] = r[0];
        w[2 * t + 1] = r[1];
    }
    static constexpr float kOff = 1024.f;
    static constexpr float kInvMul = 1.f;
    // element e of the operand holds the code of k + e
    __device__ __forceinline__ static u32x4 operand(raw w) {
        return u32x4{__builtin_amdgcn_perm(0x64646464u, w[0], 0x04010400u),
                     __builtin_amdgcn_perm(0x64646464u, w[0], 0x04030402u),
                     __builtin_amdgcn_perm(0x64646464u, w[1], 0x04010400u),
                     __builtin_amdgcn_perm(0x64646464u, w[1], 0x04030402u)};
    }
};

template <>
struct StepCodes<4> {
    using raw = uint32_t;   // codes k + 0..7, low nibble first
    using words = u32x2;    // two k-steps
    __device__ __forceinline__ static raw step(const words& w, int t) { return w[t]; }
    __device__ __forceinline__ static void set_step(words& w, int t, raw r) { w[t] = r; }
    static constexpr float kOff = 1.f;
    static constexpr float kInvMul = 16.f;
    // nibbles e and e + 4 into mantissa bits 9..6 of the two halves of 1.0:
    // operand elements 2e and 2e + 1 hold the codes of k + e and k + e + 4
    __device__ __forceinline__ static u32x4 operand(raw w) {
        return u32x4{((w << 6) & 0x03c003c0u) | 0x3c003c00u, ((w << 2) & 0x03c003c0u) | 0x3c003c00u,
                     ((w >> 2) & 0x03c003c0u) | 0x3c003c00u, ((w >> 6) & 0x03c003c0u) | 0x3c003c00u};
    }
};

// Position, inside an aligned group of eight staged activations, of the
// activation of k offset e: the order the codes take in the operand.
template <int BITS>
__device__ __forceinline__ int slot_of(int e) {
    return BITS == 4 ? ((e & 3) << 1) | (e >> 2) : e;
}

__host__ __device__ constexpr size_t round16(size_t v) { return (v + 15) & ~static_cast<size_t>(15); }

template <int G>
constexpr int fold_width() { return G < 64 ? G : 64; }

// Dynamic LDS of the gate/up kernel: staged rows, then the fold-chunk sums.
template <int G>
size_t gate_up_lds_bytes(int m, int k) {
    return round16(static_cast<size_t>(m) * (k + kPad) * 2) + static_cast<size_t>(k / fold_width<G>()) * kRows * 4;
}

template <int BITS, int XDT, int G, int S, int P, int U, int XPT, int NPL>
__global__ void __launch_bounds__(64 * S * P)
qmm_gate_up_stream_kernel(const uint8_t* __restrict__ q, const float* __restrict__ sb, const void* __restrict__ xin,
                          float* __restrict__ hout, int N, int K, int m_rows) {
    using SC = StepCodes<BITS>;
    constexpr int NT = 64 * S * P;
    constexpr int FG = fold_width<G>();   // fold chunk (k)
    constexpr int FPB = 64 / FG;          // fold chunks per k-block: 1 or 2
    constexpr int SPF = FG / 32;          // k-steps per fold chunk: 1 or 2

    extern __shared__ __align__(16) uint8_t lds[];
    __shared__ float rowmax[kRows];
    __shared__ float unscale[kRows];
    __shared__ f32x4 part[S > 1 ? S - 1 : 1][P][2][64];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ks = w % S, p = w / S;
    const int li = lane & 15, kq = lane >> 4;
    const int ldx = K + kPad;
    uint16_t* xs = reinterpret_cast<uint16_t*>(lds);
    float* xsum = reinterpret_cast<float*>(lds + round16(static_cast<size_t>(m_rows) * ldx * 2));

    const int ntiles = N / kRows;
    const int nkw = K / 64 / S;              // this wave's k-blocks per tile: kb = ks * nkw + j
    const int gw = nkw * 64 / G;             // and their groups: gbase + 0 .. gw - 1
    const int gbase = ks * gw;
    const int GP = static_cast<int>(gridDim.x) * P;
    const int t0 = static_cast<int>(blockIdx.x) * P + p;
    const int rounds = (ntiles - static_cast<int>(blockIdx.x) * P + GP - 1) / GP;   // same for the block
    if (rounds <= 0) return;   // uniform per block, before any barrier
    const uint32_t rb = static_cast<uint32_t>(K) * BITS / 8;
    const int ngroups = K / G;

    // activation pieces (16 bytes, 8 values) ahead of the first weights
    const int ppr = K / 8;
    const int npieces = m_rows * ppr;
    const u32x4* xg = static_cast<const u32x4*>(xin);
    u32x4 xt[XPT];
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
        const int u = static_cast<int>(threadIdx.x) + j * NT;
        if (u < npieces) xt[j] = xg[u];
    }

    // the lane's 16 codes of a k-block (two k-steps): one load when a k-block
    // lies inside one group (lane kq holds k 16 kq + 8 t + e), else one load
    // per k-step (lane kq holds k 32 t + 8 kq + e) so that each step stays in
    // its own 32-wide group
    constexpr bool WIDE = G >= 64;
    using Words = typename SC::words;
    struct Stage {
        Words c[2];   // [gate, up]
    };
    Stage st[U];
    const int nflat = rounds * nkw;

    // Scale/bias pairs of the wave's groups for one tile, 16 bytes a lane:
    // register r of lane (row li, slot kq) holds groups gbase + 8r + 2kq, +1;
    // a k-block takes its pair from lane li + 16 * slot with a shuffle.
    f32x4 pw[2][NPL];
    auto load_pairs = [&](int i) {
        const int tile = t0 + i * GP;
        if (tile >= ntiles) return;   // wave-uniform
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            const size_t row = 2u * static_cast<uint32_t>(tile * kRows + li) + v;
#pragma unroll
            for (int r = 0; r < NPL; ++r) {
                const int g = 8 * r + 2 * kq;
                if (g < gw) pw[v][r] = *reinterpret_cast<const f32x4*>(sb + 2 * (row * ngroups + gbase + g));
            }
        }
    };
    auto pair_of = [&](int v, int gl) -> f32x2 {
        const int r = gl >> 3, src = li + 16 * ((gl & 7) >> 1);
        f32x4 q4 = pw[v][0];
#pragma unroll
        for (int rr = 1; rr < NPL; ++rr)
            if (r == rr) q4 = pw[v][rr];
        const float x = (gl & 1) ? q4[2] : q4[0], y = (gl & 1) ? q4[3] : q4[1];
        return f32x2{__shfl(x, src, 64), __shfl(y, src, 64)};
    };

    // loads of flat step f (round f / nkw, k-block f % nkw)
    auto issue = [&](Stage& s, int f) {
        const int i = f / nkw, j = f - i * nkw;
        const int tile = t0 + i * GP;
        if (tile >= ntiles) return;   // wave-uniform
        const int kb = ks * nkw + j;
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            const uint32_t row = 2u * static_cast<uint32_t>(tile * kRows + li) + v;
            const uint8_t* qrow = q + static_cast<size_t>(row) * rb;
            if constexpr (WIDE) {
                const uint32_t k0 = static_cast<uint32_t>(kb * 64 + 16 * kq);
                s.c[v] = *reinterpret_cast<const Words*>(qrow + k0 * BITS / 8);
            } else {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const uint32_t k0 = static_cast<uint32_t>(kb * 64 + 32 * t + 8 * kq);
                    SC::set_step(s.c[v], t, *reinterpret_cast<const typename SC::raw*>(qrow + k0 * BITS / 8));
                }
            }
        }
    };

    load_pairs(0);
#pragma unroll
    for (int u = 0; u < U; ++u)
        if (u < nflat) issue(st[u], u);

    // stage the rows: raw 16-bit values into the padded rows
    for (int j = 0; j < XPT; ++j) {
        const int u = static_cast<int>(threadIdx.x) + j * NT;
        if (u < npieces) {
            const int m = u / ppr, c = u - m * ppr;
            *reinterpret_cast<u32x4*>(xs + m * ldx + c * 8) = xt[j];
        }
    }
    for (int u = static_cast<int>(threadIdx.x) + XPT * NT; u < npieces; u += NT) {
        const int m = u / ppr, c = u - m * ppr;
        *reinterpret_cast<u32x4*>(xs + m * ldx + c * 8) = xg[u];
    }
    __syncthreads();

    auto to_f32 = [](uint32_t bits16) -> float {
        if constexpr (XDT == DT_BF16) return __uint_as_float(bits16 << 16);
        else return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
    };
    // per-row largest magnitude: wave w takes rows w, w + S*P, ...
    for (int m = w; m < m_rows; m += S * P) {
        float mx = 0.f;
        for (int c = lane; c < ppr; c += 64) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(xs + m * ldx + c * 8);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                mx = fmaxf(mx, fmaxf(fabsf(to_f32(v[e] & 0xffffu)), fabsf(to_f32(v[e] >> 16))));
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
        if (lane == 0) rowmax[m] = mx;
    }
    __syncthreads();

    // scaled f16 in place (operand order), and the fold-chunk sums X' (zero for rows past m)
    const int nchunks = K / FG;
    for (int u = static_cast<int>(threadIdx.x); u < nchunks * kRows; u += NT) {
        const int m = u % kRows, ch = u / kRows;
        float sum = 0.f;
        if (m < m_rows) {
            const int sg = 15 - __builtin_amdgcn_frexp_expf(rowmax[m]);
#pragma unroll
            for (int c8 = 0; c8 < FG / 8; ++c8) {
                uint16_t* piece = xs + m * ldx + ch * FG + c8 * 8;
                const u32x4 v = *reinterpret_cast<const u32x4*>(piece);
                uint16_t o[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t b16 = (e & 1) ? (v[e >> 1] >> 16) : (v[e >> 1] & 0xffffu);
                    const _Float16 hv = static_cast<_Float16>(__builtin_amdgcn_ldexpf(to_f32(b16), sg));
                    o[slot_of<BITS>(e)] = __builtin_bit_cast(uint16_t, hv);
                }
                // the words are built in a plain array: assigning the lanes of a
                // vector one by one and feeding each to v_dot2 as it is built
                // compiled to dot products that all read the first word
                uint32_t rw[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    rw[i] = static_cast<uint32_t>(o[2 * i]) | (static_cast<uint32_t>(o[2 * i + 1]) << 16);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sum = __builtin_amdgcn_fdot2(__builtin_bit_cast(h16x2, rw[i]), __builtin_bit_cast(h16x2, 0x3c003c00u),
                                                 sum, false);
                *reinterpret_cast<u32x4*>(piece) = u32x4{rw[0], rw[1], rw[2], rw[3]};
            }
        }
        xsum[ch * kRows + m] = sum;
    }
    if (threadIdx.x < kRows) {
        const int m = static_cast<int>(threadIdx.x);
        unscale[m] = m < m_rows ? __builtin_amdgcn_ldexpf(1.f, __builtin_amdgcn_frexp_expf(rowmax[m]) - 15) : 0.f;
    }
    __syncthreads();

    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    const bool arow = li < m_rows;   // this lane's A row is live

    auto compute = [&](const Stage& s, int f) {
        const int i = f / nkw, j = f - i * nkw;
        if (t0 + i * GP >= ntiles) return;   // wave-uniform
        if (j == 0 && i > 0) load_pairs(i);
        const int kb = ks * nkw + j;
#pragma unroll
        for (int fi = 0; fi < FPB; ++fi) {
            f32x4 pt[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int ts = 0; ts < SPF; ++ts) {
                const int t = fi * SPF + ts;
                u32x4 a = u32x4{0u, 0u, 0u, 0u};
                const int ka = WIDE ? kb * 64 + 16 * kq + 8 * t : kb * 64 + 32 * t + 8 * kq;
                if (arow) a = *reinterpret_cast<const u32x4*>(xs + li * ldx + ka);
                pt[0] = mma_f16(a, SC::operand(SC::step(s.c[0], t)), pt[0]);
                pt[1] = mma_f16(a, SC::operand(SC::step(s.c[1], t)), pt[1]);
            }
            const f32x4 xc = *reinterpret_cast<const f32x4*>(xsum + ((kb * 64) / FG + fi) * kRows + 4 * kq);
#pragma unroll
            for (int v = 0; v < 2; ++v) {
                const f32x2 pv = pair_of(v, (j * 64 + fi * FG) / G);
                const float se = pv.x * SC::kInvMul, bi = pv.y;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc[v][e] = fmaf(se, fmaf(-SC::kOff, xc[e], pt[v][e]), fmaf(bi, xc[e], acc[v][e]));
            }
        }
    };

    auto combine = [&](int i) {
        if constexpr (S > 1) {
            if (ks > 0) {
                part[ks - 1][p][0][lane] = acc[0];
                part[ks - 1][p][1][lane] = acc[1];
            }
            __syncthreads();
        }
        const int tile = t0 + i * GP;
        if (ks == 0 && tile < ntiles) {
#pragma unroll
            for (int s2 = 0; s2 < S - 1; ++s2) {
                const f32x4 g2 = part[s2][p][0][lane], u2 = part[s2][p][1][lane];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc[0][e] += g2[e];
                    acc[1][e] += u2[e];
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = 4 * kq + e;
                if (m < m_rows) {
                    const float g = acc[0][e] * unscale[m], uu = acc[1][e] * unscale[m];
                    hout[static_cast<int64_t>(m) * N + tile * kRows + li] = g / (1.0f + expf(-g)) * uu;
                }
            }
        }
        if constexpr (S > 1) __syncthreads();
        acc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
    };

    // flat pipeline over (round, k-block): U in flight, the tile's partials
    // combined after its last k-block
    for (int f0 = 0; f0 < nflat; f0 += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int f = f0 + u;
            if (f < nflat) {
                compute(st[u], f);
                if (f + U < nflat) issue(st[u], f + U);
                if ((f + 1) % nkw == 0) combine(f / nkw);
            }
        }
    }
}

// Block shape: S waves along K per tile, P tiles per block, U k-blocks in flight.
constexpr int kS = 4, kP = 4, kU = 4;
// pair registers per row set (8 groups each): the groups of one wave and tile
// for K up to 8192 at 64- and 128-wide groups, 4096 at 32-wide ones
template <int G>
constexpr int pair_regs() { return G == 32 ? 4 : 2; }

template <int BITS, int XDT, int G>
int run_gate_up(const qdm_weight& w, const void* x, float* h, int m, hipStream_t s) {
    constexpr int NT = 64 * kS * kP;
    constexpr int XPT = 8;
    auto kern = qmm_gate_up_stream_kernel<BITS, XDT, G, kS, kP, kU, XPT, pair_regs<G>()>;
    const size_t lds = gate_up_lds_bytes<G>(m, w.k);
    const int res = resident_blocks(kern, NT, lds);
    if (res <= 0) return static_cast<int>(hipErrorInvalidValue);
    const int ntiles = w.n / kRows;
    const int need = (ntiles + kP - 1) / kP;
    const int blocks = need < res ? need : res;
    return static_cast<int>(launch(kern, dim3(blocks), dim3(NT), lds, s, static_cast<const uint8_t*>(w.q),
                                   w.scale_bias, x, h, w.n, w.k, m));
}

template <int BITS, int XDT>
int run_gate_up_g(const qdm_weight& w, const void* x, float* h, int m, hipStream_t s) {
    switch (w.group) {
        case 32: return run_gate_up<BITS, XDT, 32>(w, x, h, m, s);
        case 64: return run_gate_up<BITS, XDT, 64>(w, x, h, m, s);
        default: return run_gate_up<BITS, XDT, 128>(w, x, h, m, s);
    }
}

template <int XDT>
int run_gate_up_x(const qdm_weight& w, const void* x, float* h, int m, hipStream_t s) {
    return w.bits == 8 ? run_gate_up_g<8, XDT>(w, x, h, m, s) : run_gate_up_g<4, XDT>(w, x, h, m, s);
}

}  // namespace

bool mma_stream_gate_up_supported(const qdm_weight& w, int m, int act) {
    if (m < 2 || m > kRows) return false;
    if (w.bits != 8 && w.bits != 4) return false;
    if (w.group != 32 && w.group != 64 && w.group != 128) return false;
    if (act != DT_BF16 && act != DT_F16) return false;
    if (w.n % kRows != 0 || w.k % (64 * kS) != 0) return false;
    // each wave's groups: a whole, even number, at most 8 per pair register
    const int gw = w.k / kS / w.group;
    const int npl = w.group == 32 ? pair_regs<32>() : pair_regs<64>();
    if (gw * w.group * kS != w.k || gw % 2 != 0 || gw > 8 * npl) return false;
    // staged rows, chunk sums and the combine buffer within one CU's LDS
    const size_t lds = (w.group == 32 ? gate_up_lds_bytes<32>(m, w.k) : gate_up_lds_bytes<64>(m, w.k)) +
                       static_cast<size_t>(kS - 1) * kP * 2 * 64 * 16 + 2 * kRows * 4;
    return lds <= kLdsCap;
}

int launch_gate_up_mma_stream(const void* x, int m, int act, const qdm_weight& gu, float* h, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    return act == DT_F16 ? run_gate_up_x<DT_F16>(gu, x, h, m, s) : run_gate_up_x<DT_BF16>(gu, x, h, m, s);
}

}  // namespace qdm
