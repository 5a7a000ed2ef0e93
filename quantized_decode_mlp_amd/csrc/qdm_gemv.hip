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
#include "qdm_stream.h"

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
// !GU: single rows, epilogue out = r + acc rounded to ODT, r's rows r_row
// elements apart (0: one row shared by all, e.g. a projection's bias); no r
// when resid is null.
template <int BITS, int XDT, int ODT, int M, bool GU>
__global__ void __launch_bounds__(64 * kWaves)
qgemv_kernel(const uint8_t* __restrict__ q, const float* __restrict__ sb,
             const void* __restrict__ xin, const void* __restrict__ resid, void* __restrict__ out,
             int n_out, int k, int gshift, int m_rows, int r_row) {
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
                const int64_t ro = static_cast<int64_t>(m) * r_row + row0 + r;
                store_elem<ODT>(out, o, resid ? load_elem<ODT>(resid, ro) + a0 : a0);
            }
        }
    }
}


template <int BITS, int XDT, int ODT, int M, bool GU>
int run(const qdm_weight& w, const void* x, const void* r, void* out, int n_out, int k, int m_rows,
        hipStream_t s, int r_row) {
    dim3 grid((n_out + kRows - 1) / kRows), block(64 * kWaves);
    return static_cast<int>(launch(qgemv_kernel<BITS, XDT, ODT, M, GU>, grid, block, 0, s,
                                   static_cast<const uint8_t*>(w.q), w.scale_bias, x, r, out, n_out, k,
                                   gshift_of(w.group), m_rows, r_row));
}

// r_row: elements between r's rows (the output's row length for a residual)
template <int XDT, int ODT, int M, bool GU>
int run_bits(const qdm_weight& w, const void* x, const void* r, void* out, int n_out, int k,
             int m_rows, hipStream_t s, int r_row) {
    switch (w.bits) {
        case 8: return run<8, XDT, ODT, M, GU>(w, x, r, out, n_out, k, m_rows, s, r_row);
        case 4: return run<4, XDT, ODT, M, GU>(w, x, r, out, n_out, k, m_rows, s, r_row);
        default: return run<16, XDT, ODT, M, GU>(w, x, r, out, n_out, k, m_rows, s, r_row);
    }
}

template <int XDT, int ODT, bool GU>
int run_rows(const qdm_weight& w, const void* x, int64_t x_row, const void* r, void* out,
             int64_t o_row, int n_out, int k, int m, float* part, hipStream_t s) {
    // one row: the streaming kernel while K fits 8 waves of 64 activations; otherwise (and for
    // several rows) the block-per-row-group kernel, rows in blocks of up to 4
    if (m == 1) {
        StreamSplit sp;
        if (stream_split(w.bits, k, x_bytes<XDT>(), sp)) {
            sp.nr = stream_rows_per_group(sp, GU);
            if (!GU && XDT == DT_F32) stream_split_down(w.bits, k, sp);
            if (GU) stream_split_gate_up(w.bits, sp);
            switch (w.bits) {
                case 8: return run_stream<8, XDT, ODT, GU, kEpiPlain>(w, x, r, out, n_out, k, sp, s, ChainArgs{});
                case 4: return run_stream<4, XDT, ODT, GU, kEpiPlain>(w, x, r, out, n_out, k, sp, s, ChainArgs{});
                case QDM_U8_SB16:
                    return run_stream<QDM_U8_SB16, XDT, ODT, GU, kEpiPlain>(w, x, r, out, n_out, k, sp, s, ChainArgs{});
                case QDM_U4_SB16:
                    return run_stream<QDM_U4_SB16, XDT, ODT, GU, kEpiPlain>(w, x, r, out, n_out, k, sp, s, ChainArgs{});
                case QDM_MXFP8:
                    return run_stream<QDM_MXFP8, XDT, ODT, GU, kEpiPlain>(w, x, r, out, n_out, k, sp, s, ChainArgs{});
                case QDM_MXFP4:
                    return run_stream<QDM_MXFP4, XDT, ODT, GU, kEpiPlain>(w, x, r, out, n_out, k, sp, s, ChainArgs{});
                default: return run_stream<16, XDT, ODT, GU, kEpiPlain>(w, x, r, out, n_out, k, sp, s, ChainArgs{});
            }
        }
        if (is_mx(w.bits) || is_sb16(w.bits)) return static_cast<int>(hipErrorInvalidValue);   // streaming kernel only
        return run_bits<XDT, ODT, 1, GU>(w, x, r, out, n_out, k, 1, s, n_out);
    }
    // 2..16 rows on the matrix cores.  Gate/up with 8/4-bit or MX weights and
    // 16-bit activations, down with such weights and a 16-bit output: the
    // weight-streaming kernels (down split along K).  Otherwise the tile-per-block
    // kernel: gate/up with bf16 activations (exact MMA operands), down with any
    // 16-bit output (h enters as a bf16 hi/lo split, ~16 significant bits, so
    // fp32 outputs stay on the vector path); MX weights take only the former.
    if constexpr (GU) {
        if (mma_stream_gate_up_supported(w, m, XDT))
            return launch_gate_up_mma_stream(x, m, XDT, w, static_cast<float*>(out), s);
    } else {
        if (mma_stream_down_supported(w, m, ODT))
            return launch_down_mma_stream(static_cast<const float*>(x), r, m, ODT, w, out, part, s);
    }
    if (is_mx(w.bits) || is_sb16(w.bits)) return static_cast<int>(hipErrorInvalidValue);
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
        const int e = run_bits<XDT, ODT, 4, GU>(w, xp, rp, op, n_out, k, mr, s, static_cast<int>(o_row));
        if (e) return e;
    }
    return 0;
}

// A projection out[m][n] = x W^T (+ bias): one row on the streaming kernel,
// several on the vector kernel four rows a pass, the bias shared by the rows.
template <int XDT>
int run_linear(const qdm_weight& w, const void* x, int m, const void* bias, void* out, hipStream_t s) {
    const int n = w.n, k = w.k;
    StreamSplit sp;
    if (m == 1 && stream_split(w.bits, k, x_bytes<XDT>(), sp)) {
        sp.nr = stream_rows_per_group(sp, false);
        switch (w.bits) {
            case 8: return run_stream<8, XDT, XDT, false, kEpiLinear>(w, x, bias, out, n, k, sp, s, ChainArgs{});
            case 4: return run_stream<4, XDT, XDT, false, kEpiLinear>(w, x, bias, out, n, k, sp, s, ChainArgs{});
            case QDM_U8_SB16:
                return run_stream<QDM_U8_SB16, XDT, XDT, false, kEpiLinear>(w, x, bias, out, n, k, sp, s, ChainArgs{});
            case QDM_U4_SB16:
                return run_stream<QDM_U4_SB16, XDT, XDT, false, kEpiLinear>(w, x, bias, out, n, k, sp, s, ChainArgs{});
            case QDM_MXFP8:
                return run_stream<QDM_MXFP8, XDT, XDT, false, kEpiLinear>(w, x, bias, out, n, k, sp, s, ChainArgs{});
            case QDM_MXFP4:
                return run_stream<QDM_MXFP4, XDT, XDT, false, kEpiLinear>(w, x, bias, out, n, k, sp, s, ChainArgs{});
            default: return run_stream<16, XDT, XDT, false, kEpiLinear>(w, x, bias, out, n, k, sp, s, ChainArgs{});
        }
    }
    if (is_mx(w.bits) || is_sb16(w.bits)) return static_cast<int>(hipErrorInvalidValue);
    const size_t xe = XDT == DT_F32 ? 4 : 2;
    for (int m0 = 0; m0 < m; m0 += 4) {
        const int mr = m - m0 < 4 ? m - m0 : 4;
        const void* xp = static_cast<const char*>(x) + static_cast<size_t>(m0) * k * xe;
        void* op = static_cast<char*>(out) + static_cast<size_t>(m0) * n * xe;
        const int e = mr == 1 ? run_bits<XDT, XDT, 1, false>(w, xp, bias, op, n, k, 1, s, 0)
                              : run_bits<XDT, XDT, 4, false>(w, xp, bias, op, n, k, mr, s, 0);
        if (e) return e;
    }
    return 0;
}

}  // namespace

bool stream_supported(const qdm_weight& w, int xb) {
    StreamSplit sp;
    return stream_split(w.bits, w.k, xb, sp);
}

int launch_linear(const void* x, int m, int act, const qdm_weight& w, const void* bias, void* out, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (act) {
        case DT_F32: return run_linear<DT_F32>(w, x, m, bias, out, s);
        case DT_F16: return run_linear<DT_F16>(w, x, m, bias, out, s);
        default: return run_linear<DT_BF16>(w, x, m, bias, out, s);
    }
}

int launch_gate_up_swiglu(const void* x, int m, int act, const qdm_weight& gu, float* h, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int ffn = gu.n, d = gu.k;
    switch (act) {
        case DT_F32: return run_rows<DT_F32, DT_F32, true>(gu, x, d, nullptr, h, ffn, ffn, d, m, nullptr, s);
        case DT_F16: return run_rows<DT_F16, DT_F32, true>(gu, x, d, nullptr, h, ffn, ffn, d, m, nullptr, s);
        default: return run_rows<DT_BF16, DT_F32, true>(gu, x, d, nullptr, h, ffn, ffn, d, m, nullptr, s);
    }
}

int launch_down_residual(const float* h, const void* r, int m, int act, const qdm_weight& dn, void* out,
                         float* part, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int d = dn.n, ffn = dn.k;
    switch (act) {
        case DT_F32: return run_rows<DT_F32, DT_F32, false>(dn, h, ffn, r, out, d, d, ffn, m, part, s);
        case DT_F16: return run_rows<DT_F32, DT_F16, false>(dn, h, ffn, r, out, d, d, ffn, m, part, s);
        default: return run_rows<DT_F32, DT_BF16, false>(dn, h, ffn, r, out, d, d, ffn, m, part, s);
    }
}

}  // namespace qdm
