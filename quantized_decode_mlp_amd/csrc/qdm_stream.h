// One-row streaming GEMV kernel for gfx950 (gate/up with the SwiGLU epilogue,
// down with the residual epilogue) and its host launchers, optionally with
// the decode chain's residual add + RMSNorm folded in, or as a plain
// projection with an optional bias (the epilogue mode EPI).  Included by
// qdm_gemv.hip (the MLP's projections and the plain projection) and
// qdm_chain.hip (the chained forms); each translation unit instantiates what
// it launches.
//
// Pages: meTile docs, "Compute-Graph Fusion", section "Automatic Gated
// Epilogues" (two projections sharing the activation, silu(gate) * up on chip,
// residual added inside the one-row down projection) and the opening
// GraphBuilder example (residual add feeding RMSNorm, the sum kept as an
// output); "MLX-LM Backend", section "Dispatch Policy" (gate and up share each
// activation load, SwiGLU before the only write of h, typed residual store,
// RMSNorm accumulating in FP32).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "qdm_device.h"
#include "qdm_internal.h"
#include "qdm_launch.h"

namespace qdm {

// Epilogue modes of the streaming kernel.  Plain: SwiGLU (gate/up) or the
// residual add (down).  Chain: the decode chain's forms.  Linear (down only):
// a projection, out = acc (+ bias[row] when the residual pointer is not null).
constexpr int kEpiPlain = 0;
constexpr int kEpiChain = 1;
constexpr int kEpiLinear = 2;

// Inputs of the chained forms (unused otherwise).  Gate/up: the block's
// activation row is n = rmsnorm(a + b) * w, recomputed in every block.  Down:
// the residual is s = a + b (rounded once), optionally stored to s_out.
struct ChainArgs {
    const void* a;
    const void* b;
    const void* w;
    void* s_out;
    float eps;
};

namespace {

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

// Half h (0: bits 0-15, 1: bits 16-31) of w as an f16 value widened to fp32;
// as an FMA operand the widening folds into v_fma_mix_f32.  A 16-bit field
// below 0x400 is the subnormal field * 2^-24 (the kernels keep f16
// subnormals: the default denormal mode).
__device__ __forceinline__ float f16_half(uint32_t w, int h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h ? w >> 16 : w)));
}

// BITS is the weight format: 4 / 8 (affine), 16 (dense bf16), QDM_U4_SB16 /
// QDM_U8_SB16 (affine, bf16 pairs), QDM_MXFP4 / QDM_MXFP8 (block-scaled);
// the low byte is the code width.
constexpr bool is_mx(int bits) { return bits == QDM_MXFP4 || bits == QDM_MXFP8; }
constexpr bool is_sb16(int bits) { return bits == QDM_U4_SB16 || bits == QDM_U8_SB16; }
constexpr int code_bits(int bits) { return bits & 0xff; }

template <int BITS>
struct StreamShape {
    static constexpr int E = 128 / code_bits(BITS);                   // codes per 16-byte chunk
    static constexpr int TW_MAX = 64 / E;                             // K-tiles per wave at most
};

constexpr int kBatch = 16;            // rounds whose split-K partials share one LDS combine
constexpr bool kDownStageFirst = true;   // stage the fp32 hidden row before the first weight loads
constexpr bool kGateUpStageFirst = false;   // the same for gate/up's activation row
constexpr int kStreamLds = 65536;     // largest activation row staged in LDS (bytes)

template <int XDT>
constexpr int x_bytes() { return XDT == DT_F32 ? 4 : 2; }

// Stream (block b, p) takes groups b*P + p + i*G*P for rounds i = 0, 1, ...
// (G = gridDim); every wave walks the same number of rounds, so the block's
// barriers line up even when a stream has run out of groups.  A group is NR
// consecutive outputs: gate/up pairs (GU), or rows of the other projections.
// With NR = 2 a wave keeps two outputs' loads in flight per round against the
// one activation slice it holds: twice the bytes in flight for the same
// activation registers, for splits whose waves hold a single K-tile.
template <int BITS, int XDT, int ODT, bool GU, int S, int TW, int P, int EPI, int NR>
__global__ void __launch_bounds__(64 * S * P) __attribute__((amdgpu_waves_per_eu(NR == 2 ? S * P / 2 : 1)))
qgemv_stream_kernel(const uint8_t* __restrict__ q, const float* __restrict__ sb,
                    const void* __restrict__ xin, const void* __restrict__ resid, void* __restrict__ out,
                    int n_out, int k, int gshift, ChainArgs ch) {
    constexpr int E = StreamShape<BITS>::E;
    constexpr int EPD = E / 4;
    constexpr int NV = GU ? 2 * NR : NR;   // packed rows loaded per group
    static_assert(NR == 1 || NR == 2, "one or two outputs per group");
    constexpr bool MX = is_mx(BITS);
    constexpr int CB = code_bits(BITS);
    constexpr bool SB16 = is_sb16(BITS);                 // affine with bf16 (scale, bias) pairs
    constexpr bool AFFINE = (CB == 4 || CB == 8) && !MX;
    constexpr int NT = 64 * S * P;
    constexpr int XU = 4;   // 16-byte activation pieces per thread loaded ahead of the first weights
    constexpr bool NORM = EPI == kEpiChain && GU;   // the activation row is rmsnorm(a + b) * w
    static_assert(!NORM || NT >= kNormThreads, "the norm prologue needs four waves");

    extern __shared__ __align__(16) uint8_t xlds[];   // the activation row, k * x_bytes bytes
    __shared__ float part[(S > 1) ? kBatch : 1][P][S][NV];
    __shared__ float nred[NORM ? kNormThreads / 64 : 1];

    const int lane = threadIdx.x & 63;
    // wave-uniform by construction; readfirstlane lets the compiler keep it scalar
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ks = wv % S, p = wv / S;
    const uint32_t rb = static_cast<uint32_t>(k) * CB / 8;   // bytes per packed row
    const int C = static_cast<int>(rb >> 4);
    const int ng = AFFINE ? (k >> gshift) : 0;
    const int nbk = MX ? (k >> 5) : 0;                            // MX: scale bytes per row
    const int GP = static_cast<int>(gridDim.x) * P;
    const int g0 = static_cast<int>(blockIdx.x) * P + p;
    const int n_grp = (n_out + NR - 1) / NR;   // groups of NR outputs (pairs for gate/up)
    const int rounds = (n_grp - static_cast<int>(blockIdx.x) * P + GP - 1) / GP;   // same for every wave
    if (rounds <= 0) return;   // uniform per block, before any barrier

    // first pieces of the activation row (issued before the weights: the
    // in-order load counter then lets them land without waiting for weights)
    const int nunits = (k * x_bytes<XDT>()) >> 4;
    const int tid = static_cast<int>(threadIdx.x);
    const u32x4* xg = static_cast<const u32x4*>(NORM ? ch.a : xin);
    u32x4* xl = reinterpret_cast<u32x4*>(xlds);
    u32x4 xt[XU], bt, wt;
    if constexpr (NORM) {
        // unconditional at a clamped index, with unconditional uses below: a
        // load under a branch, or one whose only use is, ends up waited for
        // together with the first round's weights
        const int idx = min(tid, nunits - 1);
        xt[0] = xg[idx];
        bt = static_cast<const u32x4*>(ch.b)[idx];
        wt = static_cast<const u32x4*>(ch.w)[idx];
    } else {
#pragma unroll
        for (int u = 0; u < XU; ++u) {
            const int idx = tid + u * NT;
            if (idx < nunits) xt[u] = xg[idx];
        }
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
        soff[j] = AFFINE ? ((cc * E) >> gshift) * (SB16 ? 4u : 8u) : MX ? (cc * E) >> 5 : 0u;
    }

    // per chunk: the affine (scale, bias) pair (fp32, or two bf16 in a dword),
    // or the MX block's E8M0 code; decoded where used, so no load is waited on early
    using ChunkScale = typename std::conditional<MX || SB16, uint32_t, f32x2>::type;
    u32x4 wbuf[NV][TW];
    ChunkScale pbuf[NV][TW];

    // loads of group grp (rows clamped; a stream past its last group reloads the last row)
    auto issue = [&](u32x4 (&wq)[NV][TW], ChunkScale (&pp)[NV][TW], int grp) {
        const uint32_t row = static_cast<uint32_t>(min(grp, n_grp - 1));
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const uint32_t prow =
                GU ? 2u * static_cast<uint32_t>(min(NR * static_cast<int>(row) + v / 2, n_out - 1)) + (v & 1)
                   : static_cast<uint32_t>(min(NR * static_cast<int>(row) + v, n_out - 1));
            const uint8_t* qrow = q + static_cast<size_t>(prow) * rb;
            const uint8_t* srow =
                reinterpret_cast<const uint8_t*>(sb) + static_cast<size_t>(prow) * (MX ? nbk : ng * (SB16 ? 4 : 8));
#pragma unroll
            for (int j = 0; j < TW; ++j) {
                wq[v][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(qrow + qoff[j]));
                if constexpr (SB16)
                    pp[v][j] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(srow + soff[j]));
                else if constexpr (AFFINE)
                    pp[v][j] = __builtin_nontemporal_load(reinterpret_cast<const f32x2*>(srow + soff[j]));
                else if constexpr (MX)
                    pp[v][j] = __builtin_nontemporal_load(srow + soff[j]);
            }
        }
    };

    // Down (fp32 hidden row): the row is staged completely before the first
    // weight loads.  A CU returns load data in issue order, so hidden-row
    // pieces queued behind other waves' weight misses would arrive only as
    // the HBM queue drains (measured: the staging barrier at 4 us into an
    // 11 us launch); loaded first they come back from the caches at once.
    constexpr bool HFIRST = !NORM && (GU ? kGateUpStageFirst : kDownStageFirst && XDT == DT_F32);
    if constexpr (HFIRST) {
#pragma unroll
        for (int u = 0; u < XU; ++u) {
            const int idx = tid + u * NT;
            if (idx < nunits) xl[idx] = xt[u];
        }
        for (int idx = tid + XU * NT; idx < nunits; idx += NT) xl[idx] = xg[idx];
    }

    // the first round goes in flight before the activations are set up (the
    // chained form issues it on every path, rows clamped, so that the waits
    // of its prologue count exactly)
    if (NORM || g0 < n_grp) issue(wbuf, pbuf, g0);

    if constexpr (NORM) {
        // The decode chain's RMSNorm, recomputed by every block from a, b and w
        // (L2-resident after the first blocks): s = a + b rounded once, staged
        // in LDS; the mean square of s summed exactly as the standalone add +
        // RMSNorm kernel does (norm_chunk / kNormThreads order); then
        // n = s * inv * w rounded once, in place.  n is therefore the value
        // that kernel would store.
        const u32x4* bg = static_cast<const u32x4*>(ch.b);
        const u32x4* wg = static_cast<const u32x4*>(ch.w);
        auto add_piece = [&](int idx, const u32x4 av, const u32x4 bv) {
            u32x4 sv;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t aw = av[i], bw = bv[i];
                sv[i] = dword_map<XDT>(aw, bw, [](float x, float y) { return x + y; });
            }
            xl[idx] = sv;
        };
        add_piece(min(tid, nunits - 1), xt[0], bt);   // threads past the row rewrite the last piece, same bytes
        for (int idx = tid + NT; idx < nunits; idx += NT) add_piece(idx, xg[idx], bg[idx]);
        __syncthreads();
        if (tid < kNormThreads) {
            // the standalone kernel's order: chunks tid, tid + kNormThreads, ...
            constexpr int CE = norm_chunk<XDT>();
            float ss = 0.f;
            for (int c = tid; c * CE < k; c += kNormThreads) {
                float v[CE];   // one 16-byte LDS read per chunk, squares in element order
                load_vec<XDT, CE>(xlds, static_cast<int64_t>(c) * CE, v);
#pragma unroll
                for (int e = 0; e < CE; ++e) {
                    const float sq = fmaf(v[e], v[e], ss);
                    ss = c * CE + e < k ? sq : ss;
                }
            }
            ss = wave_total(ss);
            if ((tid & 63) == 0) nred[tid >> 6] = ss;
        }
        __syncthreads();
        float tot = 0.f;
#pragma unroll
        for (int i = 0; i < kNormThreads / 64; ++i) tot += nred[i];
        const float inv = 1.0f / sqrtf(tot / static_cast<float>(k) + ch.eps);
        auto norm_piece = [&](int idx, const u32x4 wv) {
            const u32x4 sv = xl[idx];
            u32x4 nv;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t sw = sv[i], ww = wv[i];
                nv[i] = dword_map<XDT>(sw, ww, [inv](float x, float y) { return x * inv * y; });
            }
            xl[idx] = nv;
        };
        if (tid < nunits) norm_piece(tid, wt);
        for (int idx = tid + NT; idx < nunits; idx += NT) norm_piece(idx, wg[idx]);
    } else if constexpr (!HFIRST) {
        // rest of the activation copy, then this wave's slice
#pragma unroll
        for (int u = 0; u < XU; ++u) {
            const int idx = tid + u * NT;
            if (idx < nunits) xl[idx] = xt[u];
        }
        for (int idx = tid + XU * NT; idx < nunits; idx += NT) xl[idx] = xg[idx];
    }
    __syncthreads();

    // Dot-product form.  DM 0: fp32 activations, one FMA per code (4-bit codes
    // enter the mixed-precision FMA as f16 halves; see finish()).  DM 1
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
    // v_dot2_f32_bf16 straight on the packed words.  MX weights: the hardware
    // converts element pairs exactly (E4M3 bytes 0,1 / 2,3 of a dword, or an
    // E2M1 byte's low and high nibble) -- DM 3 to f16 pairs for v_dot2 against
    // the activations scaled to f16 as in DM 1 (no offset), DM 4 to fp32 for
    // FMAs with fp32 activations; the block's E8M0 scale multiplies each
    // chunk's dot product.
    constexpr int DM = MX ? (XDT == DT_F32 ? 4 : 3)
                          : (AFFINE && XDT != DT_F32) ? 1 : (BITS == 16 && XDT == DT_BF16) ? 2 : 0;
    float xv[TW][E];
    float xs[TW];
#pragma unroll
    for (int j = 0; j < TW; ++j) {
        xs[j] = 0.f;
        const int c = (ks * TW + j) * 64 + lane;
        if (vj[j]) {
            load_vec<XDT, E>(xlds, static_cast<int64_t>(c) * E, xv[j]);
            if constexpr (DM == 0 || DM == 2) {   // DM 1 takes the sum from the f16 pairs below
#pragma unroll
                for (int e = 0; e < E; ++e) xs[j] += xv[j][e];
            }
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) xv[j][e] = 0.f;
        }
    }
    uint32_t xp[TW][DM == 0 || DM == 4 ? 1 : E / 2];   // packed 16-bit activation pairs (DM 1, 2, 3)
    float xoff[TW];                         // DM 1: the offset's share of a chunk's dot product
    int nsg = 0;                            // DM 1: -sg (+4 for 4-bit codes, which enter as n/16)
    if constexpr (DM == 1) {
        float m = 0.f;
#pragma unroll
        for (int j = 0; j < TW; ++j)
#pragma unroll
            for (int e = 0; e < E; ++e) m = fmaxf(m, fabsf(xv[j][e]));
        const int sg = 15 - __builtin_amdgcn_frexp_expf(m);
        nsg = CB == 8 ? -sg : 4 - sg;
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
                    const int a = CB == 8 ? 4 * i + 2 * h : 8 * i + h;
                    const int b = CB == 8 ? a + 1 : a + 4;
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
            xoff[j] = (CB == 8 ? 1024.f : 1.f) * t;
            xs[j] = __builtin_amdgcn_ldexpf(t, -sg);
        }
    } else if constexpr (DM == 3) {
        float m = 0.f;
#pragma unroll
        for (int j = 0; j < TW; ++j)
#pragma unroll
            for (int e = 0; e < E; ++e) m = fmaxf(m, fabsf(xv[j][e]));
        const int sg = 15 - __builtin_amdgcn_frexp_expf(m);
        nsg = -sg;
#pragma unroll
        for (int j = 0; j < TW; ++j) {
            _Float16 hv[E];
#pragma unroll
            for (int e = 0; e < E; ++e) hv[e] = static_cast<_Float16>(__builtin_amdgcn_ldexpf(xv[j][e], sg));
            // pairs in the conversions' order: E4M3 (4i+2h, 4i+2h+1), E2M1 (8i+2h, 8i+2h+1)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int h = 0; h < E / 8; ++h) {
                    const int a = CB == 8 ? 4 * i + 2 * h : 8 * i + 2 * h;
                    xp[j][i * (E / 8) + h] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hv[a])) |
                                             (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hv[a + 1])) << 16);
                }
            }
        }
    } else if constexpr (DM == 2) {
#pragma unroll
        for (int j = 0; j < TW; ++j)
#pragma unroll
            for (int i = 0; i < E / 2; ++i)   // the activations are bf16 values: their fp32 high halves
                xp[j][i] = (__float_as_uint(xv[j][2 * i]) >> 16) | (__float_as_uint(xv[j][2 * i + 1]) & 0xffff0000u);
    }

    // output row o of a single-row projection gets the dot product t
    auto store_row = [&](int o, float t) {
        if constexpr (EPI == kEpiChain) {
            // the residual is the chain's sum s = a + b, rounded once as stored
            const float sv = round_trip<ODT>(load_elem<ODT>(ch.a, o) + load_elem<ODT>(ch.b, o));
            if (ch.s_out) store_elem<ODT>(ch.s_out, o, sv);
            store_elem<ODT>(out, o, sv + t);
        } else if constexpr (EPI == kEpiLinear) {
            // a projection: the optional bias takes the residual's place
            store_elem<ODT>(out, o, resid ? load_elem<ODT>(resid, o) + t : t);
        } else {
            store_elem<ODT>(out, o, load_elem<ODT>(resid, o) + t);
        }
    };
    auto epilogue = [&](int grp, const float (&t)[NV]) {
        if constexpr (GU) {
#pragma unroll
            for (int j = 0; j < NR; ++j) {
                const float gs = t[2 * j];
                if (NR * grp + j < n_out) static_cast<float*>(out)[NR * grp + j] = gs / (1.0f + expf(-gs)) * t[2 * j + 1];
            }
        } else {
#pragma unroll
            for (int v = 0; v < NV; ++v)
                if (NR * grp + v < n_out) store_row(NR * grp + v, t[v]);
        }
    };

    // combines the parked partials of rounds first .. first+cnt-1 for every stream
    auto combine = [&](int first, int cnt) {
        __syncthreads();
        const int t = threadIdx.x;
        if (t < cnt * P) {
            const int slot = t / P, sp = t % P;
            const int grp = static_cast<int>(blockIdx.x) * P + sp + (first + slot) * GP;
            if (grp < n_grp) {
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

    // DM 1, 4-bit: the nibble mask lives in a register, so that each pair of
    // codes takes one v_and_or_b32 after its shift (with both constants as
    // literals the compiler splits it into an and and an or)
    uint32_t nmask = 0x03c003c0u;
    if constexpr (DM == 1 && CB == 4) asm volatile("" : "+v"(nmask));

    auto finish = [&](const u32x4 (&wq)[NV][TW], const ChunkScale (&pp)[NV][TW], int grp, int slot) {
        if (grp >= n_grp) return;   // this stream is past its last group (wave-uniform)
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
                    if constexpr (DM == 1 && CB == 8) {
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
                            const uint32_t ce = (sh & nmask) | 0x3c003c00u;
                            dot = __builtin_amdgcn_fdot2(__builtin_bit_cast(h16x2, ce),
                                                         __builtin_bit_cast(h16x2, xp[j][4 * i + e]), dot, false);
                        }
                    } else if constexpr (DM == 2) {
                        dot = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b16x2, word),
                                                              __builtin_bit_cast(b16x2, xp[j][i]), dot, false);
                    } else if constexpr (DM == 3 && CB == 8) {
                        const auto c01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, false);
                        const auto c23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, true);
                        dot = __builtin_amdgcn_fdot2(__builtin_bit_cast(h16x2, c01), __builtin_bit_cast(h16x2, xp[j][2 * i]),
                                                     dot, false);
                        dot = __builtin_amdgcn_fdot2(__builtin_bit_cast(h16x2, c23),
                                                     __builtin_bit_cast(h16x2, xp[j][2 * i + 1]), dot, false);
                    } else if constexpr (DM == 3) {
                        const auto c0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 0);
                        const auto c1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 1);
                        const auto c2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 2);
                        const auto c3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 3);
                        dot = __builtin_amdgcn_fdot2(__builtin_bit_cast(h16x2, c0), __builtin_bit_cast(h16x2, xp[j][4 * i]),
                                                     dot, false);
                        dot = __builtin_amdgcn_fdot2(__builtin_bit_cast(h16x2, c1),
                                                     __builtin_bit_cast(h16x2, xp[j][4 * i + 1]), dot, false);
                        dot = __builtin_amdgcn_fdot2(__builtin_bit_cast(h16x2, c2),
                                                     __builtin_bit_cast(h16x2, xp[j][4 * i + 2]), dot, false);
                        dot = __builtin_amdgcn_fdot2(__builtin_bit_cast(h16x2, c3),
                                                     __builtin_bit_cast(h16x2, xp[j][4 * i + 3]), dot, false);
                    } else if constexpr (DM == 4 && CB == 8) {
                        const f32x2 f01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(word, 1.0f, false);
                        const f32x2 f23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(word, 1.0f, true);
                        dot = fmaf(f01.x, xv[j][4 * i], dot);
                        dot = fmaf(f01.y, xv[j][4 * i + 1], dot);
                        dot = fmaf(f23.x, xv[j][4 * i + 2], dot);
                        dot = fmaf(f23.y, xv[j][4 * i + 3], dot);
                    } else if constexpr (DM == 4) {
                        const f32x2 f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 0);
                        const f32x2 f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 1);
                        const f32x2 f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 2);
                        const f32x2 f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 3);
                        dot = fmaf(f0.x, xv[j][8 * i], dot);
                        dot = fmaf(f0.y, xv[j][8 * i + 1], dot);
                        dot = fmaf(f1.x, xv[j][8 * i + 2], dot);
                        dot = fmaf(f1.y, xv[j][8 * i + 3], dot);
                        dot = fmaf(f2.x, xv[j][8 * i + 4], dot);
                        dot = fmaf(f2.y, xv[j][8 * i + 5], dot);
                        dot = fmaf(f3.x, xv[j][8 * i + 6], dot);
                        dot = fmaf(f3.y, xv[j][8 * i + 7], dot);
                    } else if constexpr (CB == 4) {
                        // DM 0, 4-bit: nibbles e and e + 4 become the f16 subnormals
                        // n * 2^-24 of one word's halves (a shift and an and per two
                        // codes); the mixed-precision FMA multiplies an f16 half with
                        // an fp32 activation exactly, and 2^24 goes into the scale
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const uint32_t pr = (word >> (4 * e)) & 0x000f000fu;
                            dot = fmaf(xv[j][i * 8 + e], f16_half(pr, 0), dot);
                            dot = fmaf(xv[j][i * 8 + e + 4], f16_half(pr, 1), dot);
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < EPD; ++e) {
                            float c;
                            if constexpr (CB == 8) c = static_cast<float>((word >> (8 * e)) & 0xffu);
                            else c = (e == 0) ? __uint_as_float(word << 16) : __uint_as_float(word & 0xffff0000u);
                            dot = fmaf(c, xv[j][i * EPD + e], dot);
                        }
                    }
                }
                if constexpr (MX) {
                    // E8M0 code e is 2^(e - 127): e in the fp32 exponent field, e = 0 the subnormal 2^-127
                    const uint32_t e8 = pp[v][j];
                    acc = fmaf(__uint_as_float(e8 ? e8 << 23 : 0x00400000u), dot, acc);
                } else if constexpr (AFFINE) {
                    float sc, bi;
                    if constexpr (SB16) {
                        const uint32_t pr = pp[v][j];
                        sc = bf16_to_f32(pr & 0xffffu);
                        bi = bf16_to_f32(pr >> 16);
                    } else {
                        sc = pp[v][j].x;
                        bi = pp[v][j].y;
                    }
                    if constexpr (DM == 1) {
                        acc = fmaf(sc, dot - xoff[j], acc);
                        acc2 = fmaf(bi, xs[j], acc2);
                    } else {
                        acc += fmaf(CB == 4 ? sc * 16777216.f : sc, dot, bi * xs[j]);
                    }
                } else {
                    acc += dot;
                }
            }
            if constexpr (DM == 1) acc = __builtin_amdgcn_ldexpf(acc, nsg) + acc2;
            if constexpr (DM == 3) acc = __builtin_amdgcn_ldexpf(acc, nsg);
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

    int slot = 0, first = 0;
    auto bookkeep = [&](int i) {
        if constexpr (S > 1) {
            if (++slot == kBatch || i + 1 == rounds) { combine(first, slot); slot = 0; first = i + 1; }
        }
    };
    // one round in flight per wave: reduce round i, then issue round i + 1
    for (int i = 0; i < rounds; ++i) {   // uniform per block
        finish(wbuf, pbuf, g0 + i * GP, slot);
        const int gn = g0 + (i + 1) * GP;
        if (gn < n_grp) issue(wbuf, pbuf, gn);
        bookkeep(i);
    }
}

// K split of the streaming kernel for rows of k codes (t 1-KiB K-tiles),
// from measured sweeps over the Qwen3-8B, Llama-3.2-1B, Llama-3-8B 4-bit and
// Qwen2.5-1.5B bf16 shapes: one tile per wave for t <= 3 and odd t <= 8, two
// for other t <= 16, beyond that ceil(t/8) tiles on ceil(t/TW) waves.
// Returns false when a wave would need more activations than registers
// allow, or when the activation row (xb bytes per element) does not fit in
// the LDS stage.
struct StreamSplit { int s, tw, nr = 1, p = 0; };   // p: row streams per block (0: the default rule)

bool stream_split(int bits, int k, int xb, StreamSplit& out) {
    if (static_cast<int64_t>(k) * xb > kStreamLds) return false;
    const int cb = code_bits(bits);
    const int64_t rb = static_cast<int64_t>(k) * cb / 8;
    const int t = static_cast<int>(((rb >> 4) + 63) >> 6);
    const int tw_max = cb == 8 ? 4 : cb == 4 ? 2 : 8;
    if (t <= 3 || (t % 2 == 1 && t <= 8)) { out = {t, 1}; return true; }
    if (t <= 16) { out = {(t + 1) / 2, 2}; return true; }
    const int tw = (t + 7) / 8;
    if (tw > tw_max) return false;
    out = {(t + tw - 1) / tw, tw};
    return true;
}

// Outputs per group of a one-row projection's streams (measured on the four
// MLP shapes and the Qwen3-8B lm_head): two rows for a down projection or a
// plain projection whose waves hold one K-tile (Llama-3-8B 4-bit down: 12.85
// against 13.45 us), one otherwise (two rows with two tiles per wave: Qwen3-8B
// down 12.15 against 11.38 us; two pairs per group for gate/up: 3-6 % slower
// on every shape).
// The down projection (fp32 hidden row, staged whole in every block's LDS):
// four waves per row and four rows per block, i.e. 16-wave blocks and one
// block per CU, when the row has at least five K-tiles and four waves can
// hold them.  One staged copy of the hidden row per CU instead of two, and
// no second block trailing the first (measured, down / layer: Qwen3-8B
// 11.12 -> 10.89 / 29.17 -> 28.47 us, Llama-3.2-1B 6.50 -> 5.69 / 14.49 ->
// 14.16, Llama-3-8B 4-bit 11.90 -> 11.92 / 28.25 -> 26.88, Qwen2.5-1.5B
// dense 7.62 -> 6.86 / 17.16 -> 16.88; other shapes of 16-wave blocks --
// 3 x 4 tiles, 8 x 1 tile with two rows, two rounds in flight -- were slower).
inline void stream_split_down(int bits, int k, StreamSplit& sp) {
    const int cb = code_bits(bits);
    const int64_t rb = static_cast<int64_t>(k) * cb / 8;
    const int t = static_cast<int>(((rb >> 4) + 63) >> 6);
    const int tw_max = cb == 8 ? 4 : cb == 4 ? 2 : 8;
    const int tw = (t + 3) / 4;
    if (t >= 5 && tw <= tw_max) sp = StreamSplit{4, tw, 1, 4};
}

// Gate/up with 8-bit codes whose rows split into two waves of one K-tile
// (Llama-3.2-1B-shaped, d = 2048): eight pairs per block, 16-wave blocks
// (measured 8.29 -> 7.93 us; the same for 4-bit codes, or for wider splits
// such as the Qwen3-8B shape, was 3-9 % slower).
inline void stream_split_gate_up(int bits, StreamSplit& sp) {
    if (code_bits(bits) == 8 && sp.s == 2 && sp.tw == 1 && sp.nr == 1) sp.p = 8;
}

inline int stream_rows_per_group(const StreamSplit& sp, bool gate_up) {
    return !gate_up && sp.tw == 1 && sp.s >= 2 ? 2 : 1;
}

// Row streams per block (measured): up to 12 waves per block, and at most 4
// streams when each wave holds a single tile.  At most 12 waves keeps at
// least 170 VGPRs per wave (three waves per SIMD), more than any split here
// needs.
constexpr int stream_rows_per_block(int s, int tw) {
    const int p = s < 12 ? 12 / s : 1;
    return tw == 1 && p > 4 ? 4 : p;
}

template <int BITS, int XDT, int ODT, bool GU, int EPI, int NR, int S, int TW>
int run_stream_st(const qdm_weight& w, const void* x, const void* r, void* out, int n_out, int k, hipStream_t s,
                  const ChainArgs& ch);

// The launch with P row streams per block (S * P waves).
template <int BITS, int XDT, int ODT, bool GU, int EPI, int NR, int S, int TW, int P>
int run_stream_p(const qdm_weight& w, const void* x, const void* r, void* out, int n_out, int k, hipStream_t s,
                 const ChainArgs& ch) {
    if constexpr (TW > StreamShape<BITS>::TW_MAX) {
        return static_cast<int>(hipErrorInvalidValue);
    } else {
        auto kern = qgemv_stream_kernel<BITS, XDT, ODT, GU, S, TW, P, EPI, NR>;
        const size_t lds = static_cast<size_t>(k) * x_bytes<XDT>();
        const int res = resident_blocks(kern, 64 * S * P, lds);
        if (res <= 0) return static_cast<int>(hipErrorInvalidValue);
        const int groups = (n_out + NR - 1) / NR;
        const int need = (groups + P - 1) / P;
        const int blocks = need < res ? need : res;
        // MX: the block scales ride in the scale/bias argument (the kernel reads bytes)
        const float* sbp = is_mx(BITS) ? reinterpret_cast<const float*>(w.block_scales) : w.scale_bias;
        return static_cast<int>(launch(kern, dim3(blocks), dim3(64 * S * P), lds, s,
                                       static_cast<const uint8_t*>(w.q), sbp, x, r, out, n_out, k,
                                       gshift_of(w.group), ch));
    }
}

template <int BITS, int XDT, int ODT, bool GU, int EPI, int NR, int S, int TW>
int run_stream_st(const qdm_weight& w, const void* x, const void* r, void* out, int n_out, int k, hipStream_t s,
                  const ChainArgs& ch) {
    return run_stream_p<BITS, XDT, ODT, GU, EPI, NR, S, TW, stream_rows_per_block(S, TW)>(w, x, r, out, n_out,
                                                                                                 k, s, ch);
}

template <int BITS, int XDT, int ODT, bool GU, int EPI, int NR, int S>
int run_stream_s(const qdm_weight& w, const void* x, const void* r, void* out, int n_out, int k, int tw,
                 hipStream_t s, const ChainArgs& ch) {
    switch (tw) {
        case 1: return run_stream_st<BITS, XDT, ODT, GU, EPI, NR, S, 1>(w, x, r, out, n_out, k, s, ch);
        case 2: return run_stream_st<BITS, XDT, ODT, GU, EPI, NR, S, 2>(w, x, r, out, n_out, k, s, ch);
        case 3: return run_stream_st<BITS, XDT, ODT, GU, EPI, NR, S, 3>(w, x, r, out, n_out, k, s, ch);
        case 4: return run_stream_st<BITS, XDT, ODT, GU, EPI, NR, S, 4>(w, x, r, out, n_out, k, s, ch);
        case 5: return run_stream_st<BITS, XDT, ODT, GU, EPI, NR, S, 5>(w, x, r, out, n_out, k, s, ch);
        case 6: return run_stream_st<BITS, XDT, ODT, GU, EPI, NR, S, 6>(w, x, r, out, n_out, k, s, ch);
        case 7: return run_stream_st<BITS, XDT, ODT, GU, EPI, NR, S, 7>(w, x, r, out, n_out, k, s, ch);
        default: return run_stream_st<BITS, XDT, ODT, GU, EPI, NR, S, 8>(w, x, r, out, n_out, k, s, ch);
    }
}

template <int BITS, int XDT, int ODT, bool GU, int EPI, int NR, int S>
int run_stream_s12(const qdm_weight& w, const void* x, const void* r, void* out, int n_out, int k, int tw,
                   hipStream_t s, const ChainArgs& ch) {
    // splits with up to 5 waves per row use 1 or 2 tiles per wave; anything else
    // is not instantiated and is refused rather than run short
    if (tw == 1) return run_stream_st<BITS, XDT, ODT, GU, EPI, NR, S, 1>(w, x, r, out, n_out, k, s, ch);
    if (tw == 2) return run_stream_st<BITS, XDT, ODT, GU, EPI, NR, S, 2>(w, x, r, out, n_out, k, s, ch);
    return static_cast<int>(hipErrorInvalidValue);
}

template <int BITS, int XDT, int ODT, bool GU, int EPI, int NR>
int run_stream_nr(const qdm_weight& w, const void* x, const void* r, void* out, int n_out, int k,
                  const StreamSplit& sp, hipStream_t s, const ChainArgs& ch) {
    switch (sp.s) {
        case 1: return run_stream_s12<BITS, XDT, ODT, GU, EPI, NR, 1>(w, x, r, out, n_out, k, sp.tw, s, ch);
        case 2: return run_stream_s12<BITS, XDT, ODT, GU, EPI, NR, 2>(w, x, r, out, n_out, k, sp.tw, s, ch);
        case 3: return run_stream_s12<BITS, XDT, ODT, GU, EPI, NR, 3>(w, x, r, out, n_out, k, sp.tw, s, ch);
        case 4: return run_stream_s12<BITS, XDT, ODT, GU, EPI, NR, 4>(w, x, r, out, n_out, k, sp.tw, s, ch);
        case 5: return run_stream_s12<BITS, XDT, ODT, GU, EPI, NR, 5>(w, x, r, out, n_out, k, sp.tw, s, ch);
        case 6: return run_stream_s<BITS, XDT, ODT, GU, EPI, NR, 6>(w, x, r, out, n_out, k, sp.tw, s, ch);
        case 7: return run_stream_s<BITS, XDT, ODT, GU, EPI, NR, 7>(w, x, r, out, n_out, k, sp.tw, s, ch);
        default: return run_stream_s<BITS, XDT, ODT, GU, EPI, NR, 8>(w, x, r, out, n_out, k, sp.tw, s, ch);
    }
}

template <int BITS, int XDT, int ODT, bool GU, int EPI>
int run_stream(const qdm_weight& w, const void* x, const void* r, void* out, int n_out, int k, const StreamSplit& sp,
               hipStream_t s, const ChainArgs& ch) {
    if constexpr (GU && code_bits(BITS) == 8) {
        if (sp.p == 8 && sp.s == 2 && sp.tw == 1)
            return run_stream_p<BITS, XDT, ODT, GU, EPI, 1, 2, 1, 8>(w, x, r, out, n_out, k, s, ch);
    }
    if constexpr (!GU) {   // two pairs per group measured slower for gate/up: not instantiated
        if constexpr (XDT == DT_F32) {   // the down projection's 16-wave blocks
            if (sp.p == 4 && sp.s == 4) {
                switch (sp.tw) {
                    case 2: return run_stream_p<BITS, XDT, ODT, GU, EPI, 1, 4, 2, 4>(w, x, r, out, n_out, k, s, ch);
                    case 3: return run_stream_p<BITS, XDT, ODT, GU, EPI, 1, 4, 3, 4>(w, x, r, out, n_out, k, s, ch);
                    case 4: return run_stream_p<BITS, XDT, ODT, GU, EPI, 1, 4, 4, 4>(w, x, r, out, n_out, k, s, ch);
                    case 5: return run_stream_p<BITS, XDT, ODT, GU, EPI, 1, 4, 5, 4>(w, x, r, out, n_out, k, s, ch);
                    case 6: return run_stream_p<BITS, XDT, ODT, GU, EPI, 1, 4, 6, 4>(w, x, r, out, n_out, k, s, ch);
                    case 7: return run_stream_p<BITS, XDT, ODT, GU, EPI, 1, 4, 7, 4>(w, x, r, out, n_out, k, s, ch);
                    case 8: return run_stream_p<BITS, XDT, ODT, GU, EPI, 1, 4, 8, 4>(w, x, r, out, n_out, k, s, ch);
                    default: return static_cast<int>(hipErrorInvalidValue);
                }
            }
        }
        if (sp.nr == 2) return run_stream_nr<BITS, XDT, ODT, GU, EPI, 2>(w, x, r, out, n_out, k, sp, s, ch);
    }
    return run_stream_nr<BITS, XDT, ODT, GU, EPI, 1>(w, x, r, out, n_out, k, sp, s, ch);
}

}  // namespace
}  // namespace qdm
