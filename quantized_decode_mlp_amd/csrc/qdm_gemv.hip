// One-row (and few-row) quantized GEMV kernels for gfx950: gate/up with the
// SwiGLU epilogue, and down with the residual epilogue.
//
// Pages: meTile docs, "Compute-Graph Fusion", section "Automatic Gated
// Epilogues" (two projections sharing the activation, silu(gate) * up on chip,
// residual added inside the one-row down projection); "MLX-LM Backend",
// section "Dispatch Policy" (gate and up share each activation load, SwiGLU
// before the only write of h, typed residual store; tunables: outputs per
// SIMD-group, SIMD-groups per threadgroup, K unroll).
//
// CDNA4 mapping.  A block is S wave64s that own the same R output rows (R
// gate/up pairs, or R down rows).  A row's packed bytes are cut into 16-byte
// chunks; one K-tile is 64 consecutive chunks (1 KiB per row), so a wave's
// dwordx4 load of one row is fully coalesced.  The S waves of a block take
// the K-tiles round robin, each keeping fp32 partial sums for every
// (row, activation row) in registers.  For affine weights a 16-byte chunk
// always lies inside one group (16/32 codes vs groups of >= 32), so its dot
// product is folded as scale * sum(q*x) + bias * sum(x): one fp32 FMA per
// weight plus two per chunk.  Partials are reduced across the wave with
// shuffles, then across the S waves through LDS, in a fixed order (results
// are bitwise reproducible); one lane per output applies the epilogue.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qdm_device.h"
#include "qdm_internal.h"
#include "qdm_launch.h"

namespace qdm {
namespace {

constexpr int kWaves = 4;   // S: waves per block, splitting K
constexpr int kRows = 4;    // R: outputs (pairs for gate/up) per block

// Adds the contribution of one packed dword (EPD codes) for every activation row.
// xv[m][e] are the EPD activations matching the dword's codes.
template <int BITS, int M, int EPD>
__device__ __forceinline__ void dot_dword(uint32_t w, const float (&xv)[M][EPD], float (&dot)[M]) {
#pragma unroll
    for (int e = 0; e < EPD; ++e) {
        float c;
        if constexpr (BITS == 8) c = static_cast<float>((w >> (8 * e)) & 0xffu);
        else if constexpr (BITS == 4) c = static_cast<float>((w >> (4 * e)) & 0xfu);
        else c = (e == 0) ? __uint_as_float(w << 16) : __uint_as_float(w & 0xffff0000u);
#pragma unroll
        for (int m = 0; m < M; ++m) dot[m] = fmaf(c, xv[m][e], dot[m]);
    }
}

// GU: gate/up pairs (q rows interleaved [n][2][k]), epilogue h = silu(g) * u (fp32 out).
// !GU: single rows, epilogue out = r + acc rounded to ODT.
template <int BITS, int XDT, int ODT, int M, bool GU>
__global__ void __launch_bounds__(64 * kWaves)
qgemv_kernel(const uint8_t* __restrict__ q, const float* __restrict__ sb,
             const void* __restrict__ xin, const void* __restrict__ resid, void* __restrict__ out,
             int n_out, int k, int gshift, int m_rows) {
    constexpr int E = 128 / BITS;   // codes per 16-byte chunk
    constexpr int EPD = E / 4;      // codes per dword
    constexpr int NV = GU ? 2 : 1;
    constexpr int R = kRows;
    constexpr bool AFFINE = BITS != 16;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int row0 = blockIdx.x * R;
    const int nrows = min(R, n_out - row0);
    const int64_t rb = static_cast<int64_t>(k) * BITS / 8;   // bytes per packed row
    const int C = static_cast<int>(rb >> 4);                  // chunks per row
    const int T = (C + 63) >> 6;                              // K-tiles
    const int ng = AFFINE ? (k >> gshift) : 0;

    float acc[NV][R][M];
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < M; ++m) acc[v][r][m] = 0.f;

    for (int t = wave; t < T; t += kWaves) {
        const int c = (t << 6) + lane;
        if (c < C) {
            const int k0 = c * E;
            // issue every weight load of this tile first
            uint4 wq[R][NV];
            float2 p[R][NV];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                if (r < nrows) {
#pragma unroll
                    for (int v = 0; v < NV; ++v) {
                        const int64_t prow = GU ? 2 * static_cast<int64_t>(row0 + r) + v
                                                : static_cast<int64_t>(row0 + r);
                        wq[r][v] = *reinterpret_cast<const uint4*>(q + prow * rb + static_cast<int64_t>(c) * 16);
                        if constexpr (AFFINE)
                            p[r][v] = *reinterpret_cast<const float2*>(sb + 2 * (prow * ng + (k0 >> gshift)));
                    }
                }
            }
            float dot[R][NV][M];
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int v = 0; v < NV; ++v)
#pragma unroll
                    for (int m = 0; m < M; ++m) dot[r][v][m] = 0.f;
            float xs[M];
#pragma unroll
            for (int m = 0; m < M; ++m) xs[m] = 0.f;

#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float xv[M][EPD];
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    if (m < m_rows) {
                        load_vec<XDT, EPD>(xin, static_cast<int64_t>(m) * k + k0 + i * EPD, xv[m]);
                    } else {
#pragma unroll
                        for (int e = 0; e < EPD; ++e) xv[m][e] = 0.f;
                    }
                    if constexpr (AFFINE) {
#pragma unroll
                        for (int e = 0; e < EPD; ++e) xs[m] += xv[m][e];
                    }
                }
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    if (r < nrows) {
#pragma unroll
                        for (int v = 0; v < NV; ++v) {
                            const uint32_t w = i == 0 ? wq[r][v].x : i == 1 ? wq[r][v].y
                                             : i == 2 ? wq[r][v].z : wq[r][v].w;
                            dot_dword<BITS, M, EPD>(w, xv, dot[r][v]);
                        }
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int v = 0; v < NV; ++v)
#pragma unroll
                    for (int m = 0; m < M; ++m) {
                        if constexpr (AFFINE)
                            acc[v][r][m] += fmaf(p[r][v].x, dot[r][v][m], p[r][v].y * xs[m]);
                        else
                            acc[v][r][m] += dot[r][v][m];
                    }
        }
    }

    __shared__ float part[kWaves][NV][R][M];
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const float s = wave_sum(acc[v][r][m]);
                if (lane == 0) part[wave][v][r][m] = s;
            }
    __syncthreads();

    const int tid = threadIdx.x;
    if (tid < R * M) {
        const int r = tid / M, m = tid % M;
        if (r < nrows && m < m_rows) {
            float a0 = 0.f, a1 = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                a0 += part[w][0][r][m];
                if constexpr (GU) a1 += part[w][NV - 1][r][m];
            }
            const int64_t o = static_cast<int64_t>(m) * n_out + row0 + r;
            if constexpr (GU) {
                // silu(g) * u with silu(g) = g / (1 + e^-g); the tails give g and -0.
                const float sg = a0 / (1.0f + expf(-a0));
                static_cast<float*>(out)[o] = sg * a1;
            } else {
                store_elem<ODT>(out, o, load_elem<ODT>(resid, o) + a0);
            }
        }
    }
}


// ---------------------------------------------------------------------------
// One-row streaming kernel.  Persistent blocks (as many as fit on the chip)
// walk the outputs (a gate/up pair, or one down row) in rounds.  A block is P
// independent row streams of S wave64s each; the S waves of a stream split
// K: wave ks owns TW consecutive K-tiles, i.e. chunk c = (ks*TW + j)*64 +
// lane for j < TW, and holds the matching fp32 activations (TW*E of them, at
// most 64) and their sums in registers for the whole launch.
//
// The activation row is copied once per block into LDS (each thread moves a
// few 16-byte pieces, issued before the first weight loads) and every wave
// reads its slice from there: one copy per block instead of one per wave
// through the vector-memory path, which a CU shares between all of its
// waves (fp32 h is 4 bytes per 8-bit down code).
//
// Each round a wave loads its TW weight chunks of the round's row(s) and the
// scale/bias pair of each chunk's group (non-temporal: weights are read
// exactly once), reduces them, and only then issues the next round: one
// round in flight per wave.  Deeper per-wave pipelines (two to six rounds,
// with the CU's register file spent on them instead of on more waves)
// measured slower on this part; so did loading a wave's pairs once and
// spreading them with ds_bpermute (an LDS round trip on every round).  Loads
// are unconditional: a lane past the end of a row or a stream past its last
// row reads a clamped, valid address and its contribution is zeroed through
// the activations (0 for such lanes) or not stored.  Row bases are wave-uniform
// (scalar registers) and lane offsets 32-bit.  Wave totals come from DPP row
// reductions; the split-K partials of up to kBatch rounds are parked in LDS
// and combined in wave order after one barrier per batch, so results are
// bitwise reproducible.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 b16x2 __attribute__((ext_vector_type(2)));

template <int BITS>
struct StreamShape {
    static constexpr int E = 128 / BITS;                              // codes per 16-byte chunk
    static constexpr int TW_MAX = 64 / E;                             // K-tiles per wave at most
};

constexpr int kBatch = 16;            // rounds whose split-K partials share one LDS combine
constexpr int kStreamLds = 65536;     // largest activation row staged in LDS (bytes)

template <int XDT>
constexpr int x_bytes() { return XDT == DT_F32 ? 4 : 2; }

// Stream (block b, p) takes groups b*P + p + i*G*P for rounds i = 0, 1, ...
// (G = gridDim); every wave walks the same number of rounds, so the block's
// barriers line up even when a stream has run out of groups.
template <int BITS, int XDT, int ODT, bool GU, int S, int TW, int P>
__global__ void __launch_bounds__(64 * S * P)
qgemv_stream_kernel(const uint8_t* __restrict__ q, const float* __restrict__ sb,
                    const void* __restrict__ xin, const void* __restrict__ resid, void* __restrict__ out,
                    int n_out, int k, int gshift) {
    constexpr int E = StreamShape<BITS>::E;
    constexpr int EPD = E / 4;
    constexpr int NV = GU ? 2 : 1;
    constexpr bool AFFINE = BITS != 16;
    constexpr int NT = 64 * S * P;
    constexpr int XU = 4;   // 16-byte activation pieces per thread loaded ahead of the first weights

    extern __shared__ __align__(16) uint8_t xlds[];   // the activation row, k * x_bytes bytes
    __shared__ float part[(S > 1) ? kBatch : 1][P][S][NV];

    const int lane = threadIdx.x & 63;
    // wave-uniform by construction; readfirstlane lets the compiler keep it scalar
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ks = wv % S, p = wv / S;
    const uint32_t rb = static_cast<uint32_t>(k) * BITS / 8;   // bytes per packed row
    const int C = static_cast<int>(rb >> 4);
    const int ng = AFFINE ? (k >> gshift) : 0;
    const int GP = static_cast<int>(gridDim.x) * P;
    const int g0 = static_cast<int>(blockIdx.x) * P + p;
    const int rounds = (n_out - static_cast<int>(blockIdx.x) * P + GP - 1) / GP;   // same for every wave
    if (rounds <= 0) return;   // uniform per block, before any barrier

    // first pieces of the activation row (issued before the weights: the
    // in-order load counter then lets them land without waiting for weights)
    const int nunits = (k * x_bytes<XDT>()) >> 4;
    const u32x4* xg = static_cast<const u32x4*>(xin);
    u32x4* xl = reinterpret_cast<u32x4*>(xlds);
    u32x4 xt[XU];
#pragma unroll
    for (int u = 0; u < XU; ++u) {
        const int idx = static_cast<int>(threadIdx.x) + u * NT;
        if (idx < nunits) xt[u] = xg[idx];
    }

    // lane offsets (bytes) of this wave's chunks and of their scale/bias pairs,
    // clamped into the row
    uint32_t qoff[TW], soff[TW];
    bool vj[TW];
#pragma unroll
    for (int j = 0; j < TW; ++j) {
        const int c = (ks * TW + j) * 64 + lane;
        vj[j] = c < C;
        const uint32_t cc = static_cast<uint32_t>(vj[j] ? c : C - 1);
        qoff[j] = cc * 16u;
        soff[j] = AFFINE ? ((cc * E) >> gshift) * 8u : 0u;
    }

    u32x4 wbuf[NV][TW];
    f32x2 pbuf[NV][TW];

    // loads of group grp (rows clamped; a stream past its last group reloads row n_out - 1)
    auto issue = [&](u32x4 (&wq)[NV][TW], f32x2 (&pp)[NV][TW], int grp) {
        const uint32_t row = static_cast<uint32_t>(min(grp, n_out - 1));
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const uint32_t prow = GU ? 2u * row + v : row;
            const uint8_t* qrow = q + static_cast<size_t>(prow) * rb;
            const uint8_t* srow = reinterpret_cast<const uint8_t*>(sb) + static_cast<size_t>(prow) * ng * 8u;
#pragma unroll
            for (int j = 0; j < TW; ++j) {
                wq[v][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(qrow + qoff[j]));
                if constexpr (AFFINE)
                    pp[v][j] = __builtin_nontemporal_load(reinterpret_cast<const f32x2*>(srow + soff[j]));
            }
        }
    };

    // the first round goes in flight before the activations are set up
    if (g0 < n_out) issue(wbuf, pbuf, g0);

    // rest of the activation copy, then this wave's slice
#pragma unroll
    for (int u = 0; u < XU; ++u) {
        const int idx = static_cast<int>(threadIdx.x) + u * NT;
        if (idx < nunits) xl[idx] = xt[u];
    }
    for (int idx = static_cast<int>(threadIdx.x) + XU * NT; idx < nunits; idx += NT) xl[idx] = xg[idx];
    __syncthreads();

    // Dot-product form.  DM 0: fp32 activations, one FMA per code.  DM 1
    // (8/4-bit codes, 16-bit activations): v_dot2_f32_f16 on two codes at a
    // time.  A code becomes an exact f16 value by placing its bits in the
    // mantissa under a fixed exponent: an 8-bit code c under the exponent
    // byte 0x64 gives 1024 + c (one byte permute per two codes); a 4-bit
    // code n in the top mantissa bits of 1.0 gives 1 + n/16 (a shift and an
    // and-or per two codes), which keeps the offset small against the code.
    // The activations are held as f16 after a per-lane power-of-two scale
    // 2^sg that puts the lane's largest magnitude in [2^14, 2^15) (a bf16 or
    // f16 value converts exactly unless it lies more than 2^28 below it); the
    // offset's share (1024 or 1 times the chunk's scaled activation sum) is
    // taken off per chunk before the group scale applies, and the powers of
    // two come off once per row.  DM 2 (bf16 weights, bf16 activations):
    // v_dot2_f32_bf16 straight on the packed words.
    constexpr int DM = (AFFINE && XDT != DT_F32) ? 1 : (BITS == 16 && XDT == DT_BF16) ? 2 : 0;
    float xv[TW][E];
    float xs[TW];
#pragma unroll
    for (int j = 0; j < TW; ++j) {
        xs[j] = 0.f;
        const int c = (ks * TW + j) * 64 + lane;
        if (vj[j]) {
            load_vec<XDT, E>(xlds, static_cast<int64_t>(c) * E, xv[j]);
            if constexpr (DM != 1) {   // DM 1 takes the sum from the f16 pairs below
#pragma unroll
                for (int e = 0; e < E; ++e) xs[j] += xv[j][e];
            }
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) xv[j][e] = 0.f;
        }
    }
    uint32_t xp[TW][DM == 0 ? 1 : E / 2];   // packed 16-bit activation pairs (DM 1, 2)
    float xoff[TW];                         // DM 1: the offset's share of a chunk's dot product
    int nsg = 0;                            // DM 1: -sg (+4 for 4-bit codes, which enter as n/16)
    if constexpr (DM == 1) {
        float m = 0.f;
#pragma unroll
        for (int j = 0; j < TW; ++j)
#pragma unroll
            for (int e = 0; e < E; ++e) m = fmaxf(m, fabsf(xv[j][e]));
        const int sg = 15 - __builtin_amdgcn_frexp_expf(m);
        nsg = BITS == 8 ? -sg : 4 - sg;
#pragma unroll
        for (int j = 0; j < TW; ++j) {
            _Float16 hv[E];
#pragma unroll
            for (int e = 0; e < E; ++e) hv[e] = static_cast<_Float16>(__builtin_amdgcn_ldexpf(xv[j][e], sg));
            // pair order matches the code pairs built in finish(): 8-bit (4i+2h, 4i+2h+1),
            // 4-bit (8i+e, 8i+e+4)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int h = 0; h < E / 8; ++h) {
                    const int a = BITS == 8 ? 4 * i + 2 * h : 8 * i + h;
                    const int b = BITS == 8 ? a + 1 : a + 4;
                    xp[j][i * (E / 8) + h] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hv[a])) |
                                             (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hv[b])) << 16);
                }
            }
            // the chunk's scaled sum (pairs against 1.0), and the unscaled sum for the
            // bias term: exact scalings of one another
            float t = 0.f;
#pragma unroll
            for (int i = 0; i < E / 2; ++i)
                t = __builtin_amdgcn_fdot2(__builtin_bit_cast(h16x2, xp[j][i]), __builtin_bit_cast(h16x2, 0x3c003c00u), t,
                                           false);
            xoff[j] = (BITS == 8 ? 1024.f : 1.f) * t;
            xs[j] = __builtin_amdgcn_ldexpf(t, -sg);
        }
    } else if constexpr (DM == 2) {
#pragma unroll
        for (int j = 0; j < TW; ++j)
#pragma unroll
            for (int i = 0; i < E / 2; ++i)   // the activations are bf16 values: their fp32 high halves
                xp[j][i] = (__float_as_uint(xv[j][2 * i]) >> 16) | (__float_as_uint(xv[j][2 * i + 1]) & 0xffff0000u);
    }

    auto epilogue = [&](int grp, const float (&t)[NV]) {
        if constexpr (GU) {
            const float gs = t[0];
            static_cast<float*>(out)[grp] = gs / (1.0f + expf(-gs)) * t[NV - 1];
        } else {
            store_elem<ODT>(out, grp, load_elem<ODT>(resid, grp) + t[0]);
        }
    };

    // combines the parked partials of rounds first .. first+cnt-1 for every stream
    auto combine = [&](int first, int cnt) {
        __syncthreads();
        const int t = threadIdx.x;
        if (t < cnt * P) {
            const int slot = t / P, sp = t % P;
            const int grp = static_cast<int>(blockIdx.x) * P + sp + (first + slot) * GP;
            if (grp < n_out) {
                float tot[NV];
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    float a = 0.f;
#pragma unroll
                    for (int s2 = 0; s2 < S; ++s2) a += part[slot][sp][s2][v];
                    tot[v] = a;
                }
                epilogue(grp, tot);
            }
        }
        __syncthreads();
    };

    auto finish = [&](const u32x4 (&wq)[NV][TW], const f32x2 (&pp)[NV][TW], int grp, int slot) {
        if (grp >= n_out) return;   // this stream is past its last group (wave-uniform)
        float tot[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            float acc = 0.f, acc2 = 0.f;
#pragma unroll
            for (int j = 0; j < TW; ++j) {
                float dot = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t word = wq[v][j][i];
                    if constexpr (DM == 1 && BITS == 8) {
                        const uint32_t c01 = __builtin_amdgcn_perm(0x64646464u, word, 0x04010400u);
                        const uint32_t c23 = __builtin_amdgcn_perm(0x64646464u, word, 0x04030402u);
                        dot = __builtin_amdgcn_fdot2(__builtin_bit_cast(h16x2, c01), __builtin_bit_cast(h16x2, xp[j][2 * i]),
                                                     dot, false);
                        dot = __builtin_amdgcn_fdot2(__builtin_bit_cast(h16x2, c23),
                                                     __builtin_bit_cast(h16x2, xp[j][2 * i + 1]), dot, false);
                    } else if constexpr (DM == 1) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            // nibbles e and e + 4 into mantissa bits 9..6 of the two halves
                            const uint32_t sh = e < 2 ? word << (6 - 4 * e) : word >> (4 * e - 6);
                            const uint32_t ce = (sh & 0x03c003c0u) | 0x3c003c00u;
                            dot = __builtin_amdgcn_fdot2(__builtin_bit_cast(h16x2, ce),
                                                         __builtin_bit_cast(h16x2, xp[j][4 * i + e]), dot, false);
                        }
                    } else if constexpr (DM == 2) {
                        dot = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b16x2, word),
                                                              __builtin_bit_cast(b16x2, xp[j][i]), dot, false);
                    } else {
#pragma unroll
                        for (int e = 0; e < EPD; ++e) {
                            float c;
                            if constexpr (BITS == 8) c = static_cast<float>((word >> (8 * e)) & 0xffu);
                            else if constexpr (BITS == 4) c = static_cast<float>((word >> (4 * e)) & 0xfu);
                            else c = (e == 0) ? __uint_as_float(word << 16) : __uint_as_float(word & 0xffff0000u);
                            dot = fmaf(c, xv[j][i * EPD + e], dot);
                        }
                    }
                }
                if constexpr (AFFINE) {
                    const float sc = pp[v][j].x, bi = pp[v][j].y;
                    if constexpr (DM == 1) {
                        acc = fmaf(sc, dot - xoff[j], acc);
                        acc2 = fmaf(bi, xs[j], acc2);
                    } else {
                        acc += fmaf(sc, dot, bi * xs[j]);
                    }
                } else {
                    acc += dot;
                }
            }
            if constexpr (DM == 1) acc = __builtin_amdgcn_ldexpf(acc, nsg) + acc2;
            tot[v] = wave_total(acc);
        }
        if constexpr (S == 1) {
            if (lane == 0) epilogue(grp, tot);
        } else {
            if (lane == 0) {
#pragma unroll
                for (int v = 0; v < NV; ++v) part[slot][p][ks][v] = tot[v];
            }
        }
    };

    // one round in flight per wave: reduce round i, then issue round i + 1
    int slot = 0, first = 0;
    for (int i = 0; i < rounds; ++i) {   // uniform per block
        finish(wbuf, pbuf, g0 + i * GP, slot);
        const int gn = g0 + (i + 1) * GP;
        if (gn < n_out) issue(wbuf, pbuf, gn);
        if constexpr (S > 1) {
            if (++slot == kBatch || i + 1 == rounds) { combine(first, slot); slot = 0; first = i + 1; }
        }
    }
}

// K split of the streaming kernel for rows of k codes (t 1-KiB K-tiles),
// from measured sweeps over the Qwen3-8B, Llama-3.2-1B, Llama-3-8B 4-bit and
// Qwen2.5-1.5B bf16 shapes: one tile per wave for t <= 3 and odd t <= 8, two
// for other t <= 16, beyond that ceil(t/8) tiles on ceil(t/TW) waves.
// Returns false when a wave would need more activations than registers
// allow, or when the activation row (xb bytes per element) does not fit in
// the LDS stage.
struct StreamSplit { int s, tw; };

bool stream_split(int bits, int k, int xb, StreamSplit& out) {
    if (static_cast<int64_t>(k) * xb > kStreamLds) return false;
    const int64_t rb = static_cast<int64_t>(k) * bits / 8;
    const int t = static_cast<int>(((rb >> 4) + 63) >> 6);
    const int tw_max = bits == 8 ? 4 : bits == 4 ? 2 : 8;
    if (t <= 3 || (t % 2 == 1 && t <= 8)) { out = {t, 1}; return true; }
    if (t <= 16) { out = {(t + 1) / 2, 2}; return true; }
    const int tw = (t + 7) / 8;
    if (tw > tw_max) return false;
    out = {(t + tw - 1) / tw, tw};
    return true;
}

// Row streams per block (measured): up to 12 waves per block, and at most 4
// streams when each wave holds a single tile.  At most 12 waves keeps at
// least 170 VGPRs per wave (three waves per SIMD), more than any split here
// needs.
constexpr int stream_rows_per_block(int s, int tw) {
    const int p = s < 12 ? 12 / s : 1;
    return tw == 1 && p > 4 ? 4 : p;
}

template <int BITS, int XDT, int ODT, bool GU, int S, int TW>
int run_stream_st(const qdm_weight& w, const void* x, const void* r, void* out, int n_out, int k, hipStream_t s) {
    if constexpr (TW > StreamShape<BITS>::TW_MAX) {
        return static_cast<int>(hipErrorInvalidValue);
    } else {
        constexpr int P = stream_rows_per_block(S, TW);
        auto kern = qgemv_stream_kernel<BITS, XDT, ODT, GU, S, TW, P>;
        const size_t lds = static_cast<size_t>(k) * x_bytes<XDT>();
        const int res = resident_blocks(kern, 64 * S * P, lds);
        if (res <= 0) return static_cast<int>(hipErrorInvalidValue);
        const int need = (n_out + P - 1) / P;
        const int blocks = need < res ? need : res;
        return static_cast<int>(launch(kern, dim3(blocks), dim3(64 * S * P), lds, s,
                                       static_cast<const uint8_t*>(w.q), w.scale_bias, x, r, out, n_out, k,
                                       gshift_of(w.group)));
    }
}

template <int BITS, int XDT, int ODT, bool GU, int S>
int run_stream_s(const qdm_weight& w, const void* x, const void* r, void* out, int n_out, int k, int tw,
                 hipStream_t s) {
    switch (tw) {
        case 1: return run_stream_st<BITS, XDT, ODT, GU, S, 1>(w, x, r, out, n_out, k, s);
        case 2: return run_stream_st<BITS, XDT, ODT, GU, S, 2>(w, x, r, out, n_out, k, s);
        case 3: return run_stream_st<BITS, XDT, ODT, GU, S, 3>(w, x, r, out, n_out, k, s);
        case 4: return run_stream_st<BITS, XDT, ODT, GU, S, 4>(w, x, r, out, n_out, k, s);
        case 5: return run_stream_st<BITS, XDT, ODT, GU, S, 5>(w, x, r, out, n_out, k, s);
        case 6: return run_stream_st<BITS, XDT, ODT, GU, S, 6>(w, x, r, out, n_out, k, s);
        case 7: return run_stream_st<BITS, XDT, ODT, GU, S, 7>(w, x, r, out, n_out, k, s);
        default: return run_stream_st<BITS, XDT, ODT, GU, S, 8>(w, x, r, out, n_out, k, s);
    }
}

template <int BITS, int XDT, int ODT, bool GU, int S>
int run_stream_s12(const qdm_weight& w, const void* x, const void* r, void* out, int n_out, int k, int tw,
                   hipStream_t s) {
    return tw == 1 ? run_stream_st<BITS, XDT, ODT, GU, S, 1>(w, x, r, out, n_out, k, s)
                   : run_stream_st<BITS, XDT, ODT, GU, S, 2>(w, x, r, out, n_out, k, s);
}

template <int BITS, int XDT, int ODT, bool GU>
int run_stream(const qdm_weight& w, const void* x, const void* r, void* out, int n_out, int k, const StreamSplit& sp,
               hipStream_t s) {
    switch (sp.s) {
        case 1: return run_stream_s12<BITS, XDT, ODT, GU, 1>(w, x, r, out, n_out, k, sp.tw, s);
        case 2: return run_stream_s12<BITS, XDT, ODT, GU, 2>(w, x, r, out, n_out, k, sp.tw, s);
        case 3: return run_stream_s12<BITS, XDT, ODT, GU, 3>(w, x, r, out, n_out, k, sp.tw, s);
        case 4: return run_stream_s12<BITS, XDT, ODT, GU, 4>(w, x, r, out, n_out, k, sp.tw, s);
        case 5: return run_stream_s12<BITS, XDT, ODT, GU, 5>(w, x, r, out, n_out, k, sp.tw, s);
        case 6: return run_stream_s<BITS, XDT, ODT, GU, 6>(w, x, r, out, n_out, k, sp.tw, s);
        case 7: return run_stream_s<BITS, XDT, ODT, GU, 7>(w, x, r, out, n_out, k, sp.tw, s);
        default: return run_stream_s<BITS, XDT, ODT, GU, 8>(w, x, r, out, n_out, k, sp.tw, s);
    }
}

template <int BITS, int XDT, int ODT, int M, bool GU>
int run(const qdm_weight& w, const void* x, const void* r, void* out, int n_out, int k, int m_rows,
        hipStream_t s) {
    dim3 grid((n_out + kRows - 1) / kRows), block(64 * kWaves);
    return static_cast<int>(launch(qgemv_kernel<BITS, XDT, ODT, M, GU>, grid, block, 0, s,
                                   static_cast<const uint8_t*>(w.q), w.scale_bias, x, r, out, n_out, k,
                                   gshift_of(w.group), m_rows));
}

template <int XDT, int ODT, int M, bool GU>
int run_bits(const qdm_weight& w, const void* x, const void* r, void* out, int n_out, int k,
             int m_rows, hipStream_t s) {
    switch (w.bits) {
        case 8: return run<8, XDT, ODT, M, GU>(w, x, r, out, n_out, k, m_rows, s);
        case 4: return run<4, XDT, ODT, M, GU>(w, x, r, out, n_out, k, m_rows, s);
        default: return run<16, XDT, ODT, M, GU>(w, x, r, out, n_out, k, m_rows, s);
    }
}

template <int XDT, int ODT, bool GU>
int run_rows(const qdm_weight& w, const void* x, int64_t x_row, const void* r, void* out,
             int64_t o_row, int n_out, int k, int m, hipStream_t s) {
    // one row: the streaming kernel while K fits 8 waves of 64 activations; otherwise (and for
    // several rows) the block-per-row-group kernel, rows in blocks of up to 4
    if (m == 1) {
        StreamSplit sp;
        if (stream_split(w.bits, k, x_bytes<XDT>(), sp)) {
            switch (w.bits) {
                case 8: return run_stream<8, XDT, ODT, GU>(w, x, r, out, n_out, k, sp, s);
                case 4: return run_stream<4, XDT, ODT, GU>(w, x, r, out, n_out, k, sp, s);
                default: return run_stream<16, XDT, ODT, GU>(w, x, r, out, n_out, k, sp, s);
            }
        }
        return run_bits<XDT, ODT, 1, GU>(w, x, r, out, n_out, k, 1, s);
    }
    // 2..16 rows on the matrix cores.  Gate/up with 8/4-bit weights and 16-bit
    // activations, down with 8/4-bit weights and a 16-bit output: the
    // weight-streaming kernels (down split along K).  Otherwise the tile-per-block
    // kernel: gate/up with bf16 activations (exact MMA operands), down with any
    // 16-bit output (h enters as a bf16 hi/lo split, ~16 significant bits, so
    // fp32 outputs stay on the vector path)
    if constexpr (GU) {
        if (mma_stream_gate_up_supported(w, m, XDT))
            return launch_gate_up_mma_stream(x, m, XDT, w, static_cast<float*>(out), s);
    } else {
        if (mma_stream_down_supported(w, m, ODT))
            return launch_down_mma_stream(static_cast<const float*>(x), r, m, ODT, w, out, s);
    }
    if (mma_rows_supported(w, m)) {
        if constexpr (GU) {
            if (XDT == DT_BF16) return launch_gate_up_mma(x, m, w, static_cast<float*>(out), s);
        } else {
            if (ODT != DT_F32) return launch_down_mma(static_cast<const float*>(x), r, m, ODT, w, out, s);
        }
    }
    const size_t xe = XDT == DT_F32 ? 4 : 2;
    const size_t oe = GU ? 4 : (ODT == DT_F32 ? 4 : 2);
    for (int m0 = 0; m0 < m; m0 += 4) {
        const int mr = m - m0 < 4 ? m - m0 : 4;
        const void* xp = static_cast<const char*>(x) + static_cast<size_t>(m0) * x_row * xe;
        const void* rp = r ? static_cast<const char*>(r) + static_cast<size_t>(m0) * o_row * oe : nullptr;
        void* op = static_cast<char*>(out) + static_cast<size_t>(m0) * o_row * oe;
        const int e = run_bits<XDT, ODT, 4, GU>(w, xp, rp, op, n_out, k, mr, s);
        if (e) return e;
    }
    return 0;
}

}  // namespace

int launch_gate_up_swiglu(const void* x, int m, int act, const qdm_weight& gu, float* h, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int ffn = gu.n, d = gu.k;
    switch (act) {
        case DT_F32: return run_rows<DT_F32, DT_F32, true>(gu, x, d, nullptr, h, ffn, ffn, d, m, s);
        case DT_F16: return run_rows<DT_F16, DT_F32, true>(gu, x, d, nullptr, h, ffn, ffn, d, m, s);
        default: return run_rows<DT_BF16, DT_F32, true>(gu, x, d, nullptr, h, ffn, ffn, d, m, s);
    }
}

int launch_down_residual(const float* h, const void* r, int m, int act, const qdm_weight& dn, void* out,
                         void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int d = dn.n, ffn = dn.k;
    switch (act) {
        case DT_F32: return run_rows<DT_F32, DT_F32, false>(dn, h, ffn, r, out, d, d, ffn, m, s);
        case DT_F16: return run_rows<DT_F32, DT_F16, false>(dn, h, ffn, r, out, d, d, ffn, m, s);
        default: return run_rows<DT_F32, DT_BF16, false>(dn, h, ffn, r, out, d, d, ffn, m, s);
    }
}

}  // namespace qdm
