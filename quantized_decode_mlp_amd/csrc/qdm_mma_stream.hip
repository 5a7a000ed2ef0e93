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
// Matrix-core form: v_mfma_f32_16x16x32_{bf16,f16} computes D[16 m][16 n] +=
// A[16 m][32 k] * B[32 k][16 n].  Lane l supplies A row m = l % 16 and B column
// n = l % 16 for the eight k of slot kq = l / 16, and holds D rows
// 4 kq + 0..3 of column l % 16.  A is the activation rows (rows at or past the
// caller's m are zero), B a tile of 16 weight rows.
//
// Exact operands.  The MMA runs in the activations' own 16-bit type, so the
// activations are staged once per block in LDS as they are, with the fp32 sum
// X of every fold chunk (one quantization group, or the k-block when the
// group is wider).  A code enters B as an exact value off + c/inv (see
// StepCodes), and the chunk's partial tile P = sum (off + c/inv) x is folded
// in fp32 as
//     acc += scale * inv * P + (bias - scale * inv * off) * X,
// which is scale * sum c x + bias * X: no weight is dequantized before the MMA.
//
// Lane k assignment: see BlockLayout (16-byte code loads per lane and row
// whenever the quantization group allows it).
//
// Work split: a block is S x P waves.  Wave (ks, p) takes 16-row tiles
// b*P + p + i*G*P (G = grid size) and, of each tile, 1/S of its k-blocks
// (every S-th one from ks when a k-block holds two or more groups, else the
// ks-th contiguous 1/S), with the next U k-blocks in flight and the tile's
// scale/bias pairs for those k-blocks loaded once.  The S partial tiles meet
// in LDS and are summed in wave order.  In the packed gate/up layout rows 2n
// and 2n + 1 are gate and up of output n, so one tile reads 32 packed rows.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qdm_device.h"
#include "qdm_internal.h"
#include "qdm_launch.h"
#include "qdm_mma_common.h"

namespace qdm {
namespace {

// Dynamic LDS of the gate/up kernel: staged rows, then the fold-chunk sums
// (MX weights have no bias term and keep none).
template <int BITS, int G>
size_t gate_up_lds_bytes(int m, int k) {
    return round16(static_cast<size_t>(m) * (k + kPad) * 2) +
           (mx_bits(BITS) ? 0 : static_cast<size_t>(k / BlockLayout<BITS, G>::FG) * kRows * 4);
}

// Inputs of the decode-chain form (NORM): the staged rows are
// n = rmsnorm(a + b) * w with a = xin, and block 0 stores s = a + b to s_buf.
struct NormArgs {
    const void* b;
    const void* w;
    void* s_buf;
    float eps;
};

template <int BITS, int XDT, int G, int S, int P, int U, int XPT, int NPL, bool NORM>
__global__ void __launch_bounds__(64 * S * P)
qmm_gate_up_stream_kernel(const uint8_t* __restrict__ q, const float* __restrict__ sb, const void* __restrict__ xin,
                          float* __restrict__ hout, int N, int K, int m_rows, NormArgs na) {
    using SC = StepCodes<BITS, XDT>;
    using L = BlockLayout<BITS, G>;
    constexpr int NT = 64 * S * P;
    constexpr int KBK = L::KBK, STEPS = L::STEPS, NF = L::NF, FG = L::FG;
    constexpr bool WIDE = L::WIDE;
    constexpr int CPF = FG / 8;   // 16-byte activation pieces per fold chunk
    static_assert(!NORM || NT % kNormThreads == 0, "the norm prologue takes rows in 256-thread groups");

    extern __shared__ __align__(16) uint8_t lds[];
    __shared__ f32x4 part[S > 1 ? S - 1 : 1][P][2][64];
    __shared__ float nred[NORM ? kRows : 1][kNormThreads / 64];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ks = w % S, p = w / S;
    const int li = lane & 15, kq = lane >> 4;
    const int ldx = K + kPad;
    uint16_t* xs = reinterpret_cast<uint16_t*>(lds);
    float* xsum = reinterpret_cast<float*>(lds + round16(static_cast<size_t>(m_rows) * ldx * 2));

    const int ntiles = N / kRows;
    const int nkw = K / KBK / S;             // this wave's k-blocks per tile
    const int gw = nkw * KBK / G;            // and their groups
    // Which k-blocks: with two or more groups per k-block the S waves of a tile
    // interleave, wave ks taking k-blocks j * S + ks, so that at any time they
    // read neighbouring k-blocks of each row (the tile's rows then stream as
    // 256-byte runs instead of four runs 1/4 of a row apart: Llama-3-8B 4-bit
    // g64, 4 rows 41.3 -> 40.0 us per layer, 16 rows 45.0 -> 44.5); otherwise
    // wave ks takes the contiguous quarter ks * nkw + j.  A wave's local group
    // g (its k-blocks' groups in order) is global group gidx(g); the two groups
    // of one pair register stay neighbours either way.
    constexpr int GPK = KBK / G >= 1 ? KBK / G : 1;   // groups per k-block
    constexpr bool ILV = KBK / G >= 2;
    auto kblock = [&](int j) { return ILV ? j * S + ks : ks * nkw + j; };
    auto gidx = [&](int g) { return ILV ? ((g / GPK) * S + ks) * GPK + g % GPK : ks * gw + g; };
    const int GP = static_cast<int>(gridDim.x) * P;
    const int t0 = static_cast<int>(blockIdx.x) * P + p;
    const int rounds = (ntiles - static_cast<int>(blockIdx.x) * P + GP - 1) / GP;   // same for the block
    if (rounds <= 0) return;   // uniform per block, before any barrier
    const uint32_t rb = static_cast<uint32_t>(K) * L::CB / 8;
    const int ngroups = K / G;

    // activation pieces (16 bytes, 8 values) ahead of the first weights
    const int ppr = K / 8;
    const int npieces = m_rows * ppr;
    const u32x4* xg = static_cast<const u32x4*>(xin);
    const u32x4* bg = static_cast<const u32x4*>(na.b);
    u32x4 xt[XPT], bt[XPT];
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
        const int u = static_cast<int>(threadIdx.x) + j * NT;
        if (u < npieces) {
            xt[j] = xg[u];
            if constexpr (NORM) bt[j] = bg[u];
        }
    }

    using Words = typename L::Words;
    struct Stage {
        Words c[2];   // [gate, up]: the lane's codes of one k-block
    };
    Stage st[U];

    // Scale/bias pairs of the wave's groups for one tile, 16 bytes a lane:
    // register r of lane (row li, slot kq) holds local groups 8r + 2kq, +1;
    // a fold chunk takes its pair from lane li + 16 * slot with a shuffle.
    // Loads are issued on every path (tile, k-block and group clamped to the
    // range; what a clamped load brings is never used): the compiler can then
    // count them and wait only for the oldest, where a load on some paths only
    // turns every wait into a full drain.
    f32x4 pw[2][NPL];
    auto load_pairs = [&](int i) {
        const int tile = min(t0 + i * GP, ntiles - 1);
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            const size_t row = 2u * static_cast<uint32_t>(tile * kRows + li) + v;
#pragma unroll
            for (int r = 0; r < NPL; ++r) {
                const int g = 8 * r + 2 * kq < gw ? 8 * r + 2 * kq : 0;
                {
                    if constexpr (mx_bits(BITS)) {
                        // MX: the two blocks' E8M0 bytes as (scale, 0) pairs
                        const uint8_t* e = reinterpret_cast<const uint8_t*>(sb) + row * ngroups + gidx(g);
                        const uint32_t e0 = e[0], e1 = e[1];
                        pw[v][r] = f32x4{e8m0_value(e0), 0.f, e8m0_value(e1), 0.f};
                    } else if constexpr (sb16_bits(BITS)) {
                        // bf16 pairs: the two groups' (scale, bias) in 8 bytes
                        const u32x2 p2 = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint8_t*>(sb) +
                                                                        (row * ngroups + gidx(g)) * 4);
                        const uint32_t p0 = p2[0], p1 = p2[1];
                        pw[v][r] = f32x4{bf16_to_f32(p0 & 0xffffu), bf16_to_f32(p0 >> 16), bf16_to_f32(p1 & 0xffffu),
                                         bf16_to_f32(p1 >> 16)};
                    } else {
                        pw[v][r] = *reinterpret_cast<const f32x4*>(sb + 2 * (row * ngroups + gidx(g)));
                    }
                }
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

    // loads of k-block j of round i's tile
    auto issue = [&](Stage& s, int i, int j) {
        const int tile = min(t0 + i * GP, ntiles - 1);
        const int kb = kblock(min(j, nkw - 1));
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            const uint32_t row = 2u * static_cast<uint32_t>(tile * kRows + li) + v;
            const uint8_t* qrow = q + static_cast<size_t>(row) * rb;
            if constexpr (WIDE) {
                const uint32_t k0 = static_cast<uint32_t>(kb * KBK + L::LK * kq);
                s.c[v] = *reinterpret_cast<const Words*>(qrow + k0 * L::CB / 8);
            } else if constexpr (L::GROUPED) {
                // the lane's group kq of the block, whole; exchanged at use
                const uint32_t k0 = static_cast<uint32_t>(kb * KBK + 32 * kq);
                s.c[v] = *reinterpret_cast<const Words*>(qrow + k0 * L::CB / 8);
            } else {
#pragma unroll
                for (int t = 0; t < STEPS; ++t) {
                    const uint32_t k0 = static_cast<uint32_t>(kb * KBK + 32 * t + 8 * kq);
                    SC::set_step(s.c[v], t, *reinterpret_cast<const typename SC::raw*>(qrow + k0 * L::CB / 8));
                }
            }
        }
    };

    // Every wave has issued its activation pieces before any weight load goes
    // out (an execution barrier only: nothing is waited for).  A CU returns
    // load data in issue order, so pieces issued behind another wave's weight
    // misses would hold the staging barrier until those drain (Llama-3-8B
    // 4-bit, 16 rows: 47.8 -> 45.8 us per layer with the down kernel's
    // matching order).
    __builtin_amdgcn_s_barrier();
    load_pairs(0);
#pragma unroll
    for (int u = 0; u < U; ++u) issue(st[u], 0, u);

    // Stage the rows in LDS as they are (operand order for 4-bit codes) with
    // the fp32 sum of each fold chunk: a piece's sum, then the sum over the
    // chunk's CPF consecutive lanes.  Sums of rows past m are zero.
    auto stage_piece = [&](int u, const u32x4& v) {
        float sum = 0.f;
        int m = 0, c = 0;
        if (u < npieces) {
            m = u / ppr;
            c = u - m * ppr;
            u32x4 o = v;
            if constexpr (nibble_pairs(BITS)) {
                // elements (0, 4), (1, 5), (2, 6), (3, 7) of the piece per word
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    o[i] = __builtin_amdgcn_perm(v[2 + (i >> 1)], v[i >> 1], (i & 1) ? 0x07060302u : 0x05040100u);
            }
            *reinterpret_cast<u32x4*>(xs + m * ldx + c * 8) = o;
            if constexpr (!mx_bits(BITS)) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    // the word goes through a scalar: __builtin_bit_cast of a vector
                    // element expression reinterprets the vector's first element
                    const uint32_t word = v[i];
                    if constexpr (XDT == DT_BF16)
                        sum += __uint_as_float(word << 16) + __uint_as_float(word & 0xffff0000u);
                    else
                        sum = __builtin_amdgcn_fdot2(__builtin_bit_cast(h16x2, word),
                                                     __builtin_bit_cast(h16x2, 0x3c003c00u), sum, false);
                }
            }
        }
        if constexpr (!mx_bits(BITS)) {
#pragma unroll
            for (int o2 = 1; o2 < CPF; o2 <<= 1) sum += __shfl_xor(sum, o2, 64);
            if (u < npieces && c % CPF == 0) xsum[(c / CPF) * kRows + m] = sum;
        }
    };
    if constexpr (NORM) {
        // The decode chain's RMSNorm per row, recomputed by every block: s =
        // a + b rounded once, staged as is (block 0 also stores it for the
        // down projection's residual); each row's mean square summed exactly
        // as the standalone add + RMSNorm kernel sums it (norm_chunk /
        // kNormThreads order; rows in 256-thread groups); then n = s * inv * w
        // rounded once goes through stage_piece in place.  n is the value that
        // kernel would store.
        const int tid = static_cast<int>(threadIdx.x);
        u32x4* sg = static_cast<u32x4*>(na.s_buf);
        auto sum_piece = [&](int u, const u32x4 av, const u32x4 bv) {
            const int m = u / ppr, c = u - m * ppr;
            u32x4 sv;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t aw = av[i], bw = bv[i];
                sv[i] = dword_map<XDT>(aw, bw, [](float x, float y) { return x + y; });
            }
            *reinterpret_cast<u32x4*>(xs + m * ldx + c * 8) = sv;
            if (blockIdx.x == 0) sg[u] = sv;
        };
#pragma unroll
        for (int j = 0; j < XPT; ++j)
            if (tid + j * NT < npieces) sum_piece(tid + j * NT, xt[j], bt[j]);
        for (int u = XPT * NT + tid; u < npieces; u += NT) sum_piece(u, xg[u], bg[u]);
        __syncthreads();
        const int t = tid & (kNormThreads - 1);
        constexpr int CE = norm_chunk<XDT>();
        for (int m = tid / kNormThreads; m < m_rows; m += NT / kNormThreads) {
            float ss = 0.f;
            for (int c = t; c * CE < K; c += kNormThreads) {   // the standalone kernel's order
#pragma unroll
                for (int e = 0; e < CE; ++e) {
                    const uint32_t h = xs[m * ldx + c * CE + e];
                    const float v = XDT == DT_BF16 ? bf16_to_f32(h) : f16_to_f32(h);
                    ss = fmaf(v, v, ss);
                }
            }
            ss = wave_total(ss);
            if ((t & 63) == 0) nred[m][t >> 6] = ss;
        }
        __syncthreads();
        const u32x4* wg = static_cast<const u32x4*>(na.w);
        for (int u0 = 0; u0 < npieces; u0 += NT) {   // uniform: stage_piece shuffles across lanes
            const int u = u0 + tid;
            u32x4 nv = u32x4{0u, 0u, 0u, 0u};
            if (u < npieces) {
                const int m = u / ppr, c = u - m * ppr;
                float tot = 0.f;
#pragma unroll
                for (int i = 0; i < kNormThreads / 64; ++i) tot += nred[m][i];
                const float inv = 1.0f / sqrtf(tot / static_cast<float>(K) + na.eps);
                const u32x4 sv = *reinterpret_cast<const u32x4*>(xs + m * ldx + c * 8);
                const u32x4 wv = wg[c];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t sw = sv[i], ww = wv[i];
                    nv[i] = dword_map<XDT>(sw, ww, [inv](float x, float y) { return x * inv * y; });
                }
            }
            stage_piece(u, nv);
        }
    } else {
        const int tid = static_cast<int>(threadIdx.x);
#pragma unroll
        for (int j = 0; j < XPT; ++j) stage_piece(tid + j * NT, xt[j]);
        // longer rows: XPT more pieces per thread at a time, all loaded (at
        // clamped indices) before any is staged, so a batch costs one wait
        for (int u0 = XPT * NT; u0 < npieces; u0 += XPT * NT) {   // uniform
#pragma unroll
            for (int j = 0; j < XPT; ++j) xt[j] = xg[min(u0 + j * NT + tid, npieces - 1)];
#pragma unroll
            for (int j = 0; j < XPT; ++j) stage_piece(u0 + j * NT + tid, xt[j]);
        }
    }
    if constexpr (!mx_bits(BITS)) {
        for (int u = static_cast<int>(threadIdx.x); u < (K / FG) * (kRows - m_rows); u += NT) {
            const int ch = u / (kRows - m_rows), m = m_rows + (u - ch * (kRows - m_rows));
            xsum[ch * kRows + m] = 0.f;
        }
    }
    __syncthreads();

    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    const bool arow = li < m_rows;   // this lane's A row is live

    auto compute = [&](const Stage& s, int j) {
        const int kb = kblock(j);
        // one partial tile per fold chunk; a wide k-block spanning NF groups runs
        // every step once per chunk with the activation kept only on the lanes
        // whose k lie in that chunk, a narrow one gives step t to chunk t
        f32x4 pt[NF][2];
#pragma unroll
        for (int fc = 0; fc < NF; ++fc) pt[fc][0] = pt[fc][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        Words cg = s.c[0], cu = s.c[1];
        if constexpr (L::GROUPED) {
            cg = transpose_slots(cg);
            cu = transpose_slots(cu);
        }
#pragma unroll
        for (int t = 0; t < STEPS; ++t) {
            const int ka = WIDE ? kb * KBK + L::LK * kq + 8 * t : kb * KBK + 32 * t + 8 * kq;
            const u32x4 a = arow ? *reinterpret_cast<const u32x4*>(xs + li * ldx + ka) : u32x4{0u, 0u, 0u, 0u};
            const u32x4 bg = SC::operand(SC::step(cg, t)), bu = SC::operand(SC::step(cu, t));
#pragma unroll
            for (int fc = 0; fc < NF; ++fc) {
                if constexpr (!WIDE) {
                    if (t != fc) continue;
                }
                u32x4 at = a;
                if constexpr (WIDE && NF > 1) {
                    if ((kq * L::LK) / FG != fc) at = u32x4{0u, 0u, 0u, 0u};
                }
                pt[fc][0] = mma<XDT>(at, bg, pt[fc][0]);
                pt[fc][1] = mma<XDT>(at, bu, pt[fc][1]);
            }
        }
#pragma unroll
        for (int fc = 0; fc < NF; ++fc) {
            if constexpr (mx_bits(BITS)) {
                // MX: the block scale times the partial tile (no bias, no offset)
#pragma unroll
                for (int v = 0; v < 2; ++v) {
                    const float se = pair_of(v, (j * KBK + fc * FG) / G).x;
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[v][e] = fmaf(se, pt[fc][v][e], acc[v][e]);
                }
            } else {
                const f32x4 xc = *reinterpret_cast<const f32x4*>(xsum + ((kb * KBK) / FG + fc) * kRows + 4 * kq);
#pragma unroll
                for (int v = 0; v < 2; ++v) {
                    const f32x2 pv = pair_of(v, (j * KBK + fc * FG) / G);
                    // scale * sum c x + bias * X with sum c x = inv * (P - off * X)
                    const float se = pv.x * SC::kInvMul, be = fmaf(-SC::kOff, se, pv.y);
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[v][e] = fmaf(se, pt[fc][v][e], fmaf(be, xc[e], acc[v][e]));
                }
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
                    const float g = acc[0][e], uu = acc[1][e];
                    hout[static_cast<int64_t>(m) * N + tile * kRows + li] = g / (1.0f + expf(-g)) * uu;
                }
            }
        }
        if constexpr (S > 1) __syncthreads();
        acc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
    };

    // per round (one tile): its pairs and first U k-blocks (round 0's went out
    // before the staging), then its k-blocks with U in flight, then the
    // combine; compute runs only inside the range, the loads on every path
    for (int i = 0; i < rounds; ++i) {   // uniform per block
        const bool live = t0 + i * GP < ntiles;   // wave-uniform
        if (i > 0) {
            load_pairs(i);
#pragma unroll
            for (int u = 0; u < U; ++u) issue(st[u], i, u);
        }
        for (int j0 = 0; j0 < nkw; j0 += U) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (live && j0 + u < nkw) compute(st[u], j0 + u);
                issue(st[u], i, j0 + u + U);
            }
        }
        combine(i);
    }
}

// Block shape: S waves along K per tile, P tiles per block, U k-blocks in flight.
constexpr int kS = 4, kP = 4, kU = 4;
// 32-wide groups keep the most registers live (pairs of 32 groups per wave
// and fragment, whole-group code words) and, affine, the most chunk sums in
// LDS: two tiles per block, so that a wave may hold 256 registers instead of
// 128 and 16 staged rows of d = 4096 still fit beside the sums and the
// combine buffer.  MXFP4 (byte scales, 16-byte code words) fits four.
template <int BITS, int G>
constexpr int gate_up_tiles() { return G == 32 && BITS != QDM_MXFP4 ? 2 : kP; }

template <int BITS, int XDT, int G, bool NORM>
int run_gate_up(const qdm_weight& w, const void* x, float* h, int m, hipStream_t s, const NormArgs& na) {
    constexpr int P = gate_up_tiles<BITS, G>();
    constexpr int NT = 64 * kS * P;
    constexpr int XPT = 4;
    // the same bytes in flight per wave: four 64-wide or two 128-wide k-blocks
    constexpr int U = BlockLayout<BITS, G>::KBK == 128 ? kU / 2 : kU;
    auto kern = qmm_gate_up_stream_kernel<BITS, XDT, G, kS, P, U, XPT, pair_regs<G>(), NORM>;
    const size_t lds = gate_up_lds_bytes<BITS, G>(m, w.k);
    const int res = resident_blocks(kern, NT, lds);
    if (res <= 0) return static_cast<int>(hipErrorInvalidValue);
    const int ntiles = w.n / kRows;
    const int need = (ntiles + P - 1) / P;
    const int blocks = need < res ? need : res;
    // MX: the block scales take the scale/bias argument (the kernel reads bytes)
    const float* sbp = mx_bits(BITS) ? reinterpret_cast<const float*>(w.block_scales) : w.scale_bias;
    if (!sbp) return static_cast<int>(hipErrorInvalidValue);
    return static_cast<int>(launch(kern, dim3(blocks), dim3(NT), lds, s, static_cast<const uint8_t*>(w.q), sbp, x, h,
                                   w.n, w.k, m, na));
}

template <int BITS, int XDT, bool NORM>
int run_gate_up_g(const qdm_weight& w, const void* x, float* h, int m, hipStream_t s, const NormArgs& na) {
    switch (w.group) {
        case 32: return run_gate_up<BITS, XDT, 32, NORM>(w, x, h, m, s, na);
        case 64: return run_gate_up<BITS, XDT, 64, NORM>(w, x, h, m, s, na);
        default: return run_gate_up<BITS, XDT, 128, NORM>(w, x, h, m, s, na);
    }
}

template <int XDT, bool NORM>
int run_gate_up_x(const qdm_weight& w, const void* x, float* h, int m, hipStream_t s, const NormArgs& na) {
    switch (w.bits) {
        case 8: return run_gate_up_g<8, XDT, NORM>(w, x, h, m, s, na);
        case QDM_U8_SB16: return run_gate_up_g<QDM_U8_SB16, XDT, NORM>(w, x, h, m, s, na);
        case QDM_U4_SB16: return run_gate_up_g<QDM_U4_SB16, XDT, NORM>(w, x, h, m, s, na);
        case QDM_MXFP8: return run_gate_up<QDM_MXFP8, XDT, 32, NORM>(w, x, h, m, s, na);
        case QDM_MXFP4: return run_gate_up<QDM_MXFP4, XDT, 32, NORM>(w, x, h, m, s, na);
        default: return run_gate_up_g<4, XDT, NORM>(w, x, h, m, s, na);
    }
}

}  // namespace

bool mma_stream_gate_up_supported(const qdm_weight& w, int m, int act) {
    if (m < 2 || m > kRows) return false;
    if (w.bits != 8 && w.bits != 4 && !mx_bits(w.bits) && !sb16_bits(w.bits)) return false;
    if (w.group != 32 && w.group != 64 && w.group != 128) return false;
    if (mx_bits(w.bits) && w.group != 32) return false;
    if (act != DT_BF16 && act != DT_F16) return false;
    const int cw = code_width(w.bits);
    const int kbk = (cw == 4 || w.group == 32) ? 128 : 64;
    if (w.n % kRows != 0 || w.k % (kbk * kS) != 0) return false;
    // each wave's groups: a whole, even number, at most 8 per pair register
    const int gw = w.k / kS / w.group;
    const int npl = w.group == 32 ? pair_regs<32>() : pair_regs<64>();
    if (gw * w.group * kS != w.k || gw % 2 != 0 || gw > 8 * npl) return false;
    // staged rows, chunk sums and the combine buffer within one CU's LDS
    const size_t dyn = mx_bits(w.bits) ? gate_up_lds_bytes<QDM_MXFP8, 32>(m, w.k)
                     : cw == 4 ? (w.group == 32 ? gate_up_lds_bytes<4, 32>(m, w.k)
                                      : w.group == 64 ? gate_up_lds_bytes<4, 64>(m, w.k)
                                                      : gate_up_lds_bytes<4, 128>(m, w.k))
                                   : (w.group == 32 ? gate_up_lds_bytes<8, 32>(m, w.k)
                                                    : gate_up_lds_bytes<8, 64>(m, w.k));
    const int tiles = w.group == 32 && w.bits != QDM_MXFP4 ? gate_up_tiles<8, 32>() : kP;
    const size_t lds = dyn + static_cast<size_t>(kS - 1) * tiles * 2 * 64 * 16 + 2 * kRows * 4 + kRows * 4 * 4;
    return lds <= kLdsCap;
}

int launch_gate_up_mma_stream(const void* x, int m, int act, const qdm_weight& gu, float* h, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    const NormArgs na{nullptr, nullptr, nullptr, 0.f};
    return act == DT_F16 ? run_gate_up_x<DT_F16, false>(gu, x, h, m, s, na)
                         : run_gate_up_x<DT_BF16, false>(gu, x, h, m, s, na);
}

int launch_gate_up_mma_stream_norm(const void* a, const void* b, const void* w, float eps, int m, int act,
                                   const qdm_weight& gu, float* h, void* s_buf, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    const NormArgs na{b, w, s_buf, eps};
    return act == DT_F16 ? run_gate_up_x<DT_F16, true>(gu, a, h, m, s, na)
                         : run_gate_up_x<DT_BF16, true>(gu, a, h, m, s, na);
}

}  // namespace qdm
