// Few-row (2..16 rows) down projection with the residual, 8/4-bit affine
// weights, on the gfx950 matrix cores: y = r + W_down h for fp32 h [m][K].
//
// Pages: meTile docs, "MLX-LM Backend", section "Dispatch Policy" (several
// activation rows go to 16-row matrix tiles, ragged row counts masked in the
// tile); "Compute-Graph Fusion" for the residual fused into the projection.
// Quantization: MLX-LM affine groups, w = scale * q + bias.
//
// The hidden row is long (K = ffn) and fp32, so no block can stage all of it:
// K is split into NS slices.  Kernel 1: block (slice s, tile group) stages
// h[:, slice] in LDS as a bf16 high part and the bf16 remainder
// (h = hi + lo to about 16 significant bits) with the fp32 sum X of every
// fold chunk, then streams 16-row weight tiles of that slice through
// v_mfma_f32_16x16x32_bf16 (two MMAs per k-step, hi and lo) with the codes as
// exact operands and each chunk's partial folded as in the gate/up kernel;
// the partial tile goes to part[s][m][n] (in the caller's workspace).  Kernel 2 adds the NS partials in
// slice order and the residual and rounds to the output type.  Work split,
// lane layout and scale/bias handling match the gate/up kernel: S waves take
// contiguous quarters of a tile's k-range in the slice, P tiles per block,
// tiles t0 + i * GP over rounds i.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "qdm_device.h"
#include "qdm_internal.h"
#include "qdm_launch.h"
#include "qdm_mma_common.h"

namespace qdm {
namespace {

// One wave per tile over the block's whole slice (no cross-wave combine), 16
// tiles per block, k-blocks in flight as in gate/up.
constexpr int kDS = 1, kDP = 16, kDU = 4;

// Dynamic LDS of the down kernel: hi rows, lo rows, fold-chunk sums.
template <int BITS, int G>
size_t down_lds_bytes(int m, int kr) {
    return 2 * round16(static_cast<size_t>(m) * (kr + kPad) * 2) +
           static_cast<size_t>(kr / BlockLayout<BITS, G>::FG) * kRows * 4;
}

template <int BITS, int G, int S, int P, int U, int NPL>
__global__ void __launch_bounds__(64 * S * P)
qmm_down_part_kernel(const uint8_t* __restrict__ q, const float* __restrict__ sb, const float* __restrict__ h,
                     float* __restrict__ part, int N, int K, int KR, int TB, int m_rows) {
    using SC = StepCodes<BITS, DT_BF16>;
    using L = BlockLayout<BITS, G>;
    constexpr int KBK = L::KBK, STEPS = L::STEPS, NF = L::NF, FG = L::FG;
    constexpr bool WIDE = L::WIDE;
    constexpr int CPF = FG / 8;   // 8-value pieces per fold chunk

    extern __shared__ __align__(16) uint8_t lds[];
    __shared__ f32x4 comb[S > 1 ? S - 1 : 1][P][64];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ks = w % S, p = w / S;
    const int li = lane & 15, kq = lane >> 4;
    const int NS = K / KR;
    const int ksl = static_cast<int>(blockIdx.x) % NS, tb = static_cast<int>(blockIdx.x) / NS;
    const int ldx = KR + kPad;
    const size_t rows_bytes = round16(static_cast<size_t>(m_rows) * ldx * 2);
    uint16_t* xh = reinterpret_cast<uint16_t*>(lds);
    uint16_t* xl = reinterpret_cast<uint16_t*>(lds + rows_bytes);
    float* xsum = reinterpret_cast<float*>(lds + 2 * rows_bytes);

    const int ntiles = N / kRows;
    const int kw = KR / S;                   // this wave's k-range of the slice
    const int nkw = kw / KBK;
    const int k0w = ksl * KR + ks * kw;      // its first k in the row
    const int gw = kw / G;
    const int gbase = k0w / G;
    const int GP = TB * P;
    const int t0 = tb * P + p;
    const int rounds = (ntiles - tb * P + GP - 1) / GP;   // same for the block
    if (rounds <= 0) return;   // uniform per block, before any barrier
    const uint32_t rb = static_cast<uint32_t>(K) * L::CB / 8;
    const int ngroups = K / G;

    using Words = typename L::Words;
    Words st[U];

    f32x4 pw[NPL];
    auto load_pairs = [&](int i) {
        const int tile = t0 + i * GP;
        if (tile >= ntiles) return;   // wave-uniform
        const size_t row = static_cast<uint32_t>(tile * kRows + li);
#pragma unroll
        for (int r = 0; r < NPL; ++r) {
            const int g = 8 * r + 2 * kq;
            if (g < gw) {
                if constexpr (mx_bits(BITS)) {
                    // MX: the two blocks' E8M0 bytes as (scale, 0) pairs
                    const uint8_t* e = reinterpret_cast<const uint8_t*>(sb) + row * ngroups + gbase + g;
                    const uint32_t e0 = e[0], e1 = e[1];
                    pw[r] = f32x4{e8m0_value(e0), 0.f, e8m0_value(e1), 0.f};
                } else if constexpr (sb16_bits(BITS)) {
                    // bf16 pairs: the two groups' (scale, bias) in 8 bytes
                    const u32x2 p2 = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint8_t*>(sb) +
                                                                    (row * ngroups + gbase + g) * 4);
                    const uint32_t p0 = p2[0], p1 = p2[1];
                    pw[r] = f32x4{bf16_to_f32(p0 & 0xffffu), bf16_to_f32(p0 >> 16), bf16_to_f32(p1 & 0xffffu),
                                  bf16_to_f32(p1 >> 16)};
                } else {
                    pw[r] = *reinterpret_cast<const f32x4*>(sb + 2 * (row * ngroups + gbase + g));
                }
            }
        }
    };
    auto pair_of = [&](int gl) -> f32x2 {
        const int r = gl >> 3, src = li + 16 * ((gl & 7) >> 1);
        f32x4 q4 = pw[0];
#pragma unroll
        for (int rr = 1; rr < NPL; ++rr)
            if (r == rr) q4 = pw[rr];
        const float x = (gl & 1) ? q4[2] : q4[0], y = (gl & 1) ? q4[3] : q4[1];
        return f32x2{__shfl(x, src, 64), __shfl(y, src, 64)};
    };
    // code loads of k-block j (clamped to the range) of the wave's tile of round
    // i (clamped to the last tile): issued on every path, so the compiler can
    // count them and wait only for the oldest
    auto issue = [&](Words& c, int i, int j) {
        const int tile = min(t0 + i * GP, ntiles - 1);
        const uint8_t* qrow = q + static_cast<size_t>(tile * kRows + li) * rb;
        const int kb0 = k0w + min(j, nkw - 1) * KBK;
        if constexpr (WIDE) {
            c = *reinterpret_cast<const Words*>(qrow + static_cast<uint32_t>(kb0 + L::LK * kq) * L::CB / 8);
        } else if constexpr (L::GROUPED) {
            // the lane's group kq of the block, whole; exchanged at use
            c = *reinterpret_cast<const Words*>(qrow + static_cast<uint32_t>(kb0 + 32 * kq) * L::CB / 8);
        } else {
#pragma unroll
            for (int t = 0; t < STEPS; ++t)
                SC::set_step(c, t,
                             *reinterpret_cast<const typename SC::raw*>(
                                 qrow + static_cast<uint32_t>(kb0 + 32 * t + 8 * kq) * L::CB / 8));
        }
    };


    // stage h[:, slice] as bf16 hi + lo (operand order for 4-bit codes) and the
    // fold-chunk sums of hi + lo; sums of rows past m are zero
    const int ppr = KR / 8;
    const int npieces = m_rows * ppr;
    auto pack2 = [](uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); };
    // two pieces per thread at a time, both loaded (at clamped indices) before
    // either is staged: one wait per pair of pieces
    constexpr int HB = 2;
    constexpr int NT = 64 * S * P;
    f32x4 ld[HB][2];
    auto load_batch = [&](int u0) {
#pragma unroll
        for (int j = 0; j < HB; ++j) {
            const int u = min(u0 + j * NT + static_cast<int>(threadIdx.x), npieces - 1);
            const int m = u / ppr, c = u - m * ppr;
            const f32x4* src = reinterpret_cast<const f32x4*>(h + static_cast<size_t>(m) * K + ksl * KR + c * 8);
            ld[j][0] = src[0];
            ld[j][1] = src[1];
        }
    };
    auto stage_batch = [&](int u0) {
#pragma unroll
        for (int j = 0; j < HB; ++j) {
            const int u = u0 + j * NT + static_cast<int>(threadIdx.x);
            float sum = 0.f;
            int m = 0, c = 0;
            if (u < npieces) {
                m = u / ppr;
                c = u - m * ppr;
                const f32x4 a0 = ld[j][0], a1 = ld[j][1];
                uint32_t hi[8], lo[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float v = e < 4 ? a0[e] : a1[e - 4];
                    hi[e] = __float_as_uint(v) & 0xffff0000u;   // truncation: the exact top half
                    const float rem = v - __uint_as_float(hi[e]);
                    lo[e] = __float_as_uint(rem) & 0xffff0000u;
                    sum += __uint_as_float(hi[e]) + __uint_as_float(lo[e]);
                }
                u32x4 oh, ol;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    // element pairs (2i, 2i+1), or (i, i+4) for 4-bit codes
                    const int ea = nibble_pairs(BITS) ? i : 2 * i, eb = nibble_pairs(BITS) ? i + 4 : 2 * i + 1;
                    oh[i] = pack2(hi[ea], hi[eb]);
                    ol[i] = pack2(lo[ea], lo[eb]);
                }
                *reinterpret_cast<u32x4*>(xh + m * ldx + c * 8) = oh;
                *reinterpret_cast<u32x4*>(xl + m * ldx + c * 8) = ol;
            }
#pragma unroll
            for (int o2 = 1; o2 < CPF; o2 <<= 1) sum += __shfl_xor(sum, o2, 64);
            if (u < npieces && c % CPF == 0) xsum[(c / CPF) * kRows + m] = sum;
        }
    };
    load_batch(0);
    // The first round's pairs and code loads go out behind the first h loads
    // of every wave (an execution barrier only: nothing is waited for), so
    // the weight stream starts while the slice is staged, and no wave's h
    // pieces queue behind another wave's weight misses (a CU returns load data
    // in issue order).
    __builtin_amdgcn_s_barrier();
    if (t0 < ntiles) load_pairs(0);
#pragma unroll
    for (int u = 0; u < U; ++u) issue(st[u], 0, u);
    stage_batch(0);
    for (int u0 = HB * NT; u0 < npieces; u0 += HB * NT) {   // uniform
        load_batch(u0);
        stage_batch(u0);
    }
    for (int u = static_cast<int>(threadIdx.x); u < (KR / FG) * (kRows - m_rows); u += 64 * S * P) {
        const int ch = u / (kRows - m_rows), m = m_rows + (u - ch * (kRows - m_rows));
        xsum[ch * kRows + m] = 0.f;
    }
    __syncthreads();

    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    const bool arow = li < m_rows;

    auto compute = [&](const Words& cw, int j) {
        const int kl = ks * kw + j * KBK;    // k-block start inside the staged slice
        f32x4 pt[NF];
#pragma unroll
        for (int fc = 0; fc < NF; ++fc) pt[fc] = f32x4{0.f, 0.f, 0.f, 0.f};
        Words cwx = cw;
        if constexpr (L::GROUPED) cwx = transpose_slots(cwx);
#pragma unroll
        for (int t = 0; t < STEPS; ++t) {
            const int ka = WIDE ? kl + L::LK * kq + 8 * t : kl + 32 * t + 8 * kq;
            const u32x4 z = u32x4{0u, 0u, 0u, 0u};
            const u32x4 ah = arow ? *reinterpret_cast<const u32x4*>(xh + li * ldx + ka) : z;
            const u32x4 al = arow ? *reinterpret_cast<const u32x4*>(xl + li * ldx + ka) : z;
            const u32x4 b = SC::operand(SC::step(cwx, t));
#pragma unroll
            for (int fc = 0; fc < NF; ++fc) {
                if constexpr (!WIDE) {
                    if (t != fc) continue;
                }
                u32x4 th = ah, tl = al;
                if constexpr (WIDE && NF > 1) {
                    if ((kq * L::LK) / FG != fc) th = tl = z;
                }
                pt[fc] = mma<DT_BF16>(th, b, pt[fc]);
                pt[fc] = mma<DT_BF16>(tl, b, pt[fc]);
            }
        }
#pragma unroll
        for (int fc = 0; fc < NF; ++fc) {
            const f32x4 xc = *reinterpret_cast<const f32x4*>(xsum + (kl / FG + fc) * kRows + 4 * kq);
            const f32x2 pv = pair_of((j * KBK + fc * FG) / G);
            const float se = pv.x * SC::kInvMul, be = fmaf(-SC::kOff, se, pv.y);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = fmaf(se, pt[fc][e], fmaf(be, xc[e], acc[e]));
        }
    };

    auto combine = [&](int i) {
        if constexpr (S > 1) {
            if (ks > 0) comb[ks - 1][p][lane] = acc;
            __syncthreads();
        }
        const int tile = t0 + i * GP;
        if (ks == 0 && tile < ntiles) {
#pragma unroll
            for (int s2 = 0; s2 < S - 1; ++s2) {
                const f32x4 o = comb[s2][p][lane];
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] += o[e];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = 4 * kq + e;
                if (m < m_rows) part[(static_cast<size_t>(ksl) * m_rows + m) * N + tile * kRows + li] = acc[e];
            }
        }
        if constexpr (S > 1) __syncthreads();
        acc = f32x4{0.f, 0.f, 0.f, 0.f};
    };

    // per round (one tile): its pairs, then its k-blocks with U code loads in
    // flight; compute runs only inside the range, the loads on every path
    for (int i = 0; i < rounds; ++i) {   // uniform per block
        const bool live = t0 + i * GP < ntiles;   // wave-uniform
        if (i > 0) {   // round 0's loads went out before the staging
            if (live) load_pairs(i);
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

// y[m][n] = r[m][n] + sum over slices s (in order) of part[s][m][n]
template <int ODT>
__global__ void __launch_bounds__(256)
qmm_down_reduce_kernel(const float* __restrict__ part, const void* __restrict__ r, void* __restrict__ out, int N,
                       int m_rows, int NS, void* __restrict__ r_copy) {
    const int idx = static_cast<int>(blockIdx.x) * 256 + static_cast<int>(threadIdx.x);
    if (idx >= m_rows * N) return;
    const size_t stride = static_cast<size_t>(m_rows) * N;
    const float rv = load_elem<ODT>(r, idx);
    // sixteen slices' loads in flight at a time (one round trip for up to 16
    // slices), summed in slice order
    float acc = 0.f;
    for (int s0 = 0; s0 < NS; s0 += 16) {
        float v[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) v[j] = part[min(s0 + j, NS - 1) * stride + idx];
#pragma unroll
        for (int j = 0; j < 16; ++j) acc += s0 + j < NS ? v[j] : 0.f;
    }
    store_elem<ODT>(out, idx, rv + acc);
    if (r_copy) store_elem<ODT>(r_copy, idx, rv);   // the residual's copy, when asked (the decode chain's s)
}

// Slice length KR and tile groups per slice TB.  A wave's range (KR / S) is
// a multiple of the k-block and of two groups and fits the pair registers, and
// the staged slice fits LDS: the longest such slice (fewest partials, longest
// k-run per tile).  Each slice gets the fewest tile groups that still give one
// block per CU (all of them if the CUs cannot be covered).
struct DownSplit { int kr, tb; };

template <int BITS, int G>
bool pick_down_split(int m, int n, int k, int cus, DownSplit& out) {
    const int kbk = BlockLayout<BITS, G>::KBK;
    const int unit = kbk > 2 * G ? kbk : 2 * G;   // both are powers of two
    const int pw_max = 8 * pair_regs<G>() * G;
    const size_t cap = kLdsCap - static_cast<size_t>(kDS > 1 ? kDS - 1 : 1) * kDP * 64 * 16;
    const int groups = (n / kRows + kDP - 1) / kDP;
    bool found = false;
    for (int pw = unit; pw <= pw_max; pw += unit) {
        const int kr = kDS * pw;
        if (k % kr != 0 || down_lds_bytes<BITS, G>(m, kr) > cap) continue;
        const int ns = k / kr;
        out = {kr, std::min(groups, (cus + ns - 1) / ns)};
        found = true;
    }
    return found;
}

}  // namespace

namespace {

template <int BITS, int G, int ODT>
int run_down(const qdm_weight& w, const float* h, const void* r, void* out, int m, hipStream_t s, float* part,
             void* r_copy) {
    constexpr int NT = 64 * kDS * kDP;
    constexpr int U = kDU;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return static_cast<int>(hipErrorInvalidDevice);
    DownSplit sp;
    if (!pick_down_split<BITS, G>(m, w.n, w.k, cus, sp)) return static_cast<int>(hipErrorInvalidValue);
    const int ns = w.k / sp.kr;
    if (!part) return static_cast<int>(hipErrorInvalidValue);
    auto kern = qmm_down_part_kernel<BITS, G, kDS, kDP, U, pair_regs<G>()>;
    const size_t lds = down_lds_bytes<BITS, G>(m, sp.kr);
    if (lds > 65536 && hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds)) != hipSuccess)
        return static_cast<int>(hipErrorInvalidValue);
    // MX: the block scales take the scale/bias argument (the kernel reads bytes)
    const float* sbp = mx_bits(BITS) ? reinterpret_cast<const float*>(w.block_scales) : w.scale_bias;
    if (!sbp) return static_cast<int>(hipErrorInvalidValue);
    hipError_t e = launch(kern, dim3(ns * sp.tb), dim3(NT), lds, s, static_cast<const uint8_t*>(w.q), sbp, h,
                          part, w.n, w.k, sp.kr, sp.tb, m);
    if (e != hipSuccess) return static_cast<int>(e);
    const int outs = m * w.n;
    e = launch(qmm_down_reduce_kernel<ODT>, dim3((outs + 255) / 256), dim3(256), 0, s,
               static_cast<const float*>(part), r, out, w.n, m, ns, r_copy);
    return static_cast<int>(e);
}

template <int BITS, int ODT>
int run_down_g(const qdm_weight& w, const float* h, const void* r, void* out, int m, hipStream_t s, float* part,
               void* rc) {
    switch (w.group) {
        case 32: return run_down<BITS, 32, ODT>(w, h, r, out, m, s, part, rc);
        case 64: return run_down<BITS, 64, ODT>(w, h, r, out, m, s, part, rc);
        default: return run_down<BITS, 128, ODT>(w, h, r, out, m, s, part, rc);
    }
}

template <int ODT>
int run_down_b(const qdm_weight& w, const float* h, const void* r, void* out, int m, hipStream_t s, float* part,
               void* rc) {
    switch (w.bits) {
        case 8: return run_down_g<8, ODT>(w, h, r, out, m, s, part, rc);
        case QDM_U8_SB16: return run_down_g<QDM_U8_SB16, ODT>(w, h, r, out, m, s, part, rc);
        case QDM_U4_SB16: return run_down_g<QDM_U4_SB16, ODT>(w, h, r, out, m, s, part, rc);
        case QDM_MXFP8: return run_down<QDM_MXFP8, 32, ODT>(w, h, r, out, m, s, part, rc);
        case QDM_MXFP4: return run_down<QDM_MXFP4, 32, ODT>(w, h, r, out, m, s, part, rc);
        default: return run_down_g<4, ODT>(w, h, r, out, m, s, part, rc);
    }
}

// Slices of the split (0 when no split fits); the slice count does not depend
// on the device, only the tile groups per slice do.
template <int BITS, int G>
int split_slices(int m, int n, int k) {
    DownSplit sp;
    return pick_down_split<BITS, G>(m, n, k, 1, sp) ? k / sp.kr : 0;
}

int down_slices(const qdm_weight& w, int m) {
    if (w.bits == QDM_MXFP8) return w.group == 32 ? split_slices<QDM_MXFP8, 32>(m, w.n, w.k) : 0;
    if (w.bits == QDM_MXFP4) return w.group == 32 ? split_slices<QDM_MXFP4, 32>(m, w.n, w.k) : 0;
    if (code_width(w.bits) == 4)
        return w.group == 32 ? split_slices<4, 32>(m, w.n, w.k)
             : w.group == 64 ? split_slices<4, 64>(m, w.n, w.k) : split_slices<4, 128>(m, w.n, w.k);
    return w.group == 32 ? split_slices<8, 32>(m, w.n, w.k)
         : w.group == 64 ? split_slices<8, 64>(m, w.n, w.k) : split_slices<8, 128>(m, w.n, w.k);
}

}  // namespace

bool mma_stream_down_supported(const qdm_weight& w, int m, int act) {
    if (m < 2 || m > kRows) return false;
    if (w.bits != 8 && w.bits != 4 && !mx_bits(w.bits) && !sb16_bits(w.bits)) return false;
    if (w.group != 32 && w.group != 64 && w.group != 128) return false;
    if (act != DT_BF16 && act != DT_F16) return false;   // h enters at ~16 bits: 16-bit outputs only
    if (w.n % kRows != 0) return false;
    return down_slices(w, m) > 0;
}

size_t down_mma_stream_partials_bytes(const qdm_weight& w, int m) {
    return static_cast<size_t>(down_slices(w, m)) * static_cast<size_t>(m) * static_cast<size_t>(w.n) *
           sizeof(float);
}

int launch_down_mma_stream(const float* h, const void* r, int m, int act, const qdm_weight& dn, void* out,
                           float* part, void* stream, void* r_copy) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    return act == DT_F16 ? run_down_b<DT_F16>(dn, h, r, out, m, s, part, r_copy)
                         : run_down_b<DT_BF16>(dn, h, r, out, m, s, part, r_copy);
}

}  // namespace qdm
