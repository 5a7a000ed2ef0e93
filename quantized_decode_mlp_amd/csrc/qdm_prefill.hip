// Multi-row prefill (more than 16 rows): tiled dual GEMM on the gfx950 matrix
// cores, the weights read once per 64 activation rows instead of once per 16.
//
// Pages: meTile docs, "MLX-LM Backend", section "Dispatch Policy": multi-row
// calls run a fused dual-GEMM gate/up kernel with register-resident SwiGLU
// that reuses activation fragments for both GEMMs and stores only the final
// hidden tile, with row-masked loads and stores for ragged tiles.
// Quantization: MLX-LM affine groups, w = scale * q + bias; MX block scales.
//
// Tile.  A block is four waves over 64 activation rows (four 16-row MMA
// tiles); wave w owns NO 16-output fragments, outputs n0 + 16 j + 0..15 with
// n0 = block base + 16 NO w (for gate/up each output has a gate and an up
// fragment, so a wave holds 2 NO weight fragments).  Every activation
// fragment read from LDS feeds all of the wave's weight fragments.
//
// Chunked k layout.  The K loop runs over k-blocks of KBK k (16 code bytes per
// lane and weight fragment, 32 for 8-bit codes in 32-wide groups); a k-block
// is NF fold chunks of FG = min(G, KBK) k and every 32-k MMA step lies inside
// one chunk: in chunk c, lane slot kq (lane / 16) holds the FG/4 consecutive
// k from c FG + kq FG/4, step s of the chunk takes eight of them.  So each
// code load is one contiguous piece per lane and chunk (with 32-wide groups,
// one load of the slot's whole group and an exchange of words between the
// slots), and no MMA runs on masked lanes.  The codes enter the MMA as
// exact operands (StepCodes) and each chunk's partial tile P is folded in fp32
// as scale * P + (bias - scale * off) * X, X the chunk's activation sum,
// which one more MMA per row tile and step computes against an all-ones
// operand (it lands in the accumulator layout of the fold, and the matrix
// cores have room where the vector units have none).
//
// Pipeline.  The activation k-block is staged in one of two LDS buffers
// while the other is computed on, one barrier per k-block;
// activation loads run one k-block ahead in registers, weight loads two.
//
// Split K.  When the output tiles alone do not fill the chip, the k-blocks
// are split over S slices; a slice's tile goes to fp32 partials
// part[s][m][n'] in the caller's workspace and a second kernel adds the
// slices in order (so results do not depend on timing) and applies SwiGLU
// (gate/up) or the residual and the output rounding (down).
//
// Gate/up takes the activations in their own 16-bit type; down takes the fp32
// hidden rows as a bf16 high part and the bf16 remainder (two MMAs per
// fragment and step, about 16 significant bits).
#include <algorithm>

#include "qdm_internal.h"
#include "qdm_launch.h"
#include "qdm_mma_common.h"

namespace qdm {
namespace {

constexpr int kPA = 4;            // 16-row activation tiles per block
constexpr int kPW = 4;            // waves per block
constexpr int kPBM = 16 * kPA;    // activation rows per block
constexpr int kPT = 64 * kPW;     // threads per block

template <int BITS, int G>
struct TileLayout {
    static constexpr int CB = code_width(BITS);
    static constexpr int KBK = (CB == 4 || G == 32) ? 128 : 64;
    static constexpr int FG = G < KBK ? G : KBK;   // fold chunk
    static constexpr int NF = KBK / FG;
    static constexpr int SPC = FG / 32;            // MMA steps per chunk
    static constexpr int LB = FG / 4 * CB / 8;     // code bytes per lane and chunk: 4, 8 or 16
    static_assert(LB == 4 || LB == 8 || LB == 16, "chunk piece size");
    // 32-wide groups: lane slot kq loads the whole group kq (16 bytes of 4-bit
    // codes, 32 of 8-bit ones) and the slots exchange words before the MMAs
    // (transpose_slots), which gives each slot its chunk pieces of every group
    static constexpr bool GROUPED = FG == 32;
    using Words = typename std::conditional<GROUPED && CB == 8, u32x8, u32x4>::type;
};

// Dynamic LDS: two buffers of NH staged parts [64][KBK + pad] (16-bit).
template <int BITS, int G, bool GU>
constexpr size_t prefill_lds_bytes() {
    using L = TileLayout<BITS, G>;
    return 2 * (GU ? 1 : 2) * static_cast<size_t>(kPBM) * (L::KBK + kPad) * 2;
}

// Gate/up holds one output fragment pair per wave, down two fragments; both
// run two waves per SIMD.
template <int BITS, int G, int XDT, bool GU, int ODT, int NO>
__global__ void __launch_bounds__(kPT) __attribute__((amdgpu_waves_per_eu(2)))
qmm_prefill_kernel(const uint8_t* __restrict__ q, const float* __restrict__ sb, const void* __restrict__ xin,
                   const void* __restrict__ resid, void* __restrict__ out, float* __restrict__ part, int N, int K,
                   int M, int S) {
    using L = TileLayout<BITS, G>;
    constexpr int MDT = GU ? XDT : DT_BF16;   // the MMA's operand type
    using SC = StepCodes<BITS, MDT>;
    constexpr int KBK = L::KBK, NF = L::NF, FG = L::FG, SPC = L::SPC, LB = L::LB;
    constexpr bool MX = mx_bits(BITS), SB16 = sb16_bits(BITS);
    constexpr int NV = GU ? 2 * NO : NO;      // weight fragments per wave
    constexpr int NH = GU ? 1 : 2;            // staged parts: the activations, or h's hi and lo
    constexpr int PPR = KBK / 8;              // 8-element pieces of a staged row
    constexpr int PT = kPBM * PPR / kPT;      // pieces per thread and k-block
    constexpr int LDA = KBK + kPad;
    constexpr int XBUF = NH * kPBM * LDA;     // uint16 per staging buffer
    static_assert(PT * kPT == kPBM * PPR, "pieces split evenly");
    using PairRaw = typename std::conditional<MX || SB16, uint32_t, f32x2>::type;

    extern __shared__ __align__(16) uint8_t lds[];
    uint16_t* xs = reinterpret_cast<uint16_t*>(lds);

    const int tid = static_cast<int>(threadIdx.x);
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 15, kq = lane >> 4;
    const int slice = static_cast<int>(blockIdx.x) % S;
    const int nblk = static_cast<int>(blockIdx.x) / S;
    const int m0 = static_cast<int>(blockIdx.y) * kPBM;
    const int n0 = (nblk * kPW + w) * 16 * NO;   // this wave's first output
    const bool wlive = n0 < N;                    // wave-uniform (N % 16 == 0)
    const int nkb = K / KBK;
    const int kb0 = static_cast<int>((static_cast<int64_t>(nkb) * slice) / S);
    const int nk = static_cast<int>((static_cast<int64_t>(nkb) * (slice + 1)) / S) - kb0;   // >= 1
    const uint32_t rb = static_cast<uint32_t>(K) * L::CB / 8;
    const int ngroups = K / G;

    // weight rows of the wave's fragments (fragments past N read row N - 1 and store nothing)
    uint32_t wrow[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int j = GU ? v >> 1 : v;
        const int n = min(n0 + 16 * j + li, N - 1);
        wrow[v] = GU ? 2u * static_cast<uint32_t>(n) + (v & 1) : static_cast<uint32_t>(n);
    }

    // ---- activation pieces: piece u = tid + j * kPT of the 64 x KBK tile, row u / PPR, piece u % PPR
    u32x4 ax[GU ? PT : 1];
    f32x4 ah[GU ? 1 : PT][2];
    auto load_a = [&](int kb) {
#pragma unroll
        for (int j = 0; j < PT; ++j) {
            const int u = tid + j * kPT, row = u / PPR, c = u - row * PPR;
            // rows past M read row 0; stage_a zeroes them (a select here would wait for the load)
            const size_t off = static_cast<size_t>(m0 + row < M ? m0 + row : 0) * K + kb * KBK + c * 8;
            if constexpr (GU) {
                ax[j] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(xin) + off);
            } else {
                const f32x4* src = reinterpret_cast<const f32x4*>(static_cast<const float*>(xin) + off);
                ah[j][0] = src[0];
                ah[j][1] = src[1];
            }
        }
    };
    // staged in MMA operand order (pairs (e, e + 4) for 4-bit affine codes)
    auto stage_a = [&](int buf) {
        uint16_t* xb = xs + buf * XBUF;
#pragma unroll
        for (int j = 0; j < PT; ++j) {
            const int u = tid + j * kPT, row = u / PPR, c = u - row * PPR;
            const bool live = m0 + row < M;
            if constexpr (GU) {
                const u32x4 v = live ? ax[j] : u32x4{0u, 0u, 0u, 0u};
                u32x4 o = v;
                if constexpr (nibble_pairs(BITS)) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        o[i] = __builtin_amdgcn_perm(v[2 + (i >> 1)], v[i >> 1], (i & 1) ? 0x07060302u : 0x05040100u);
                }
                *reinterpret_cast<u32x4*>(xb + row * LDA + c * 8) = o;
            } else {
                uint32_t hi[8], lo[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float v = live ? (e < 4 ? ah[j][0][e] : ah[j][1][e - 4]) : 0.f;
                    hi[e] = __float_as_uint(v) & 0xffff0000u;   // truncation: the exact top half
                    lo[e] = __float_as_uint(v - __uint_as_float(hi[e])) & 0xffff0000u;
                }
                u32x4 oh, ol;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int ea = nibble_pairs(BITS) ? i : 2 * i, eb = nibble_pairs(BITS) ? i + 4 : 2 * i + 1;
                    oh[i] = (hi[ea] >> 16) | (hi[eb] & 0xffff0000u);
                    ol[i] = (lo[ea] >> 16) | (lo[eb] & 0xffff0000u);
                }
                *reinterpret_cast<u32x4*>(xb + row * LDA + c * 8) = oh;
                *reinterpret_cast<u32x4*>(xb + (kPBM + row) * LDA + c * 8) = ol;
            }
        }
    };

    // ---- weights: per fragment, the lane's code piece of every chunk and the chunk's pair
    using Words = typename L::Words;
    auto load_b = [&](Words (&cw)[NV], PairRaw (&pr)[NV][NF], int kb) {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const uint8_t* qrow = q + static_cast<size_t>(wrow[v]) * rb;
            if constexpr (L::GROUPED)
                cw[v] = *reinterpret_cast<const Words*>(qrow + static_cast<uint32_t>(kb * KBK + 32 * kq) * L::CB / 8);
#pragma unroll
            for (int c = 0; c < NF; ++c) {
                const uint8_t* src = qrow + static_cast<uint32_t>(kb * KBK + c * FG + kq * (FG / 4)) * L::CB / 8;
                if constexpr (L::GROUPED) {
                    // codes loaded whole above
                } else if constexpr (LB == 16) {
                    cw[v] = *reinterpret_cast<const u32x4*>(src);
                } else if constexpr (LB == 8) {
                    const u32x2 p = *reinterpret_cast<const u32x2*>(src);
                    cw[v][2 * c] = p[0];
                    cw[v][2 * c + 1] = p[1];
                } else {
                    cw[v][c] = *reinterpret_cast<const uint32_t*>(src);
                }
                const size_t gi = static_cast<size_t>(wrow[v]) * ngroups + (kb * KBK + c * FG) / G;
                if constexpr (MX)
                    pr[v][c] = reinterpret_cast<const uint8_t*>(sb)[gi];
                else if constexpr (SB16)
                    pr[v][c] = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(sb) + gi * 4);
                else
                    pr[v][c] = *reinterpret_cast<const f32x2*>(sb + 2 * gi);
            }
        }
    };

    f32x4 acc[kPA][NV];
#pragma unroll
    for (int a = 0; a < kPA; ++a)
#pragma unroll
        for (int v = 0; v < NV; ++v) acc[a][v] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int buf, const Words (&cwl)[NV], const PairRaw (&pr)[NV][NF]) {
        if (!wlive) return;   // wave-uniform
        Words cw[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) cw[v] = L::GROUPED ? transpose_slots(cwl[v]) : cwl[v];
        const uint16_t* xb = xs + buf * XBUF;
        // 1.0 in every element of the operand's 16-bit type: an MMA against it
        // gives each row's chunk sum X in the accumulator layout the fold uses
        constexpr uint32_t kOne = MDT == DT_BF16 ? 0x3f803f80u : 0x3c003c00u;
        const u32x4 ones = {kOne, kOne, kOne, kOne};
#pragma unroll
        for (int c = 0; c < NF; ++c) {
            f32x4 pt[kPA][NV], xc[kPA];
#pragma unroll
            for (int a = 0; a < kPA; ++a) {
                xc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int v = 0; v < NV; ++v) pt[a][v] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int s = 0; s < SPC; ++s) {
                const int t = c * SPC + s;
                const int ka = c * FG + kq * (FG / 4) + 8 * s;
                u32x4 bv[NV];
#pragma unroll
                for (int v = 0; v < NV; ++v) bv[v] = SC::operand(SC::step(cw[v], t));
#pragma unroll
                for (int a = 0; a < kPA; ++a) {
#pragma unroll
                    for (int hp = 0; hp < NH; ++hp) {
                        const u32x4 av = *reinterpret_cast<const u32x4*>(xb + (hp * kPBM + 16 * a + li) * LDA + ka);
#pragma unroll
                        for (int v = 0; v < NV; ++v) pt[a][v] = mma<MDT>(av, bv[v], pt[a][v]);
                        if constexpr (!MX) xc[a] = mma<MDT>(av, ones, xc[a]);
                    }
                }
            }
            // fold: scale * P + (bias - scale * off) * X
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                float se, be;
                if constexpr (MX) {
                    se = e8m0_value(pr[v][c]);
                    be = 0.f;
                } else if constexpr (SB16) {
                    const uint32_t p2 = pr[v][c];
                    se = bf16_to_f32(p2 & 0xffffu) * SC::kInvMul;
                    be = fmaf(-SC::kOff, se, bf16_to_f32(p2 >> 16));
                } else {
                    se = pr[v][c].x * SC::kInvMul;
                    be = fmaf(-SC::kOff, se, pr[v][c].y);
                }
#pragma unroll
                for (int a = 0; a < kPA; ++a) {
                    if constexpr (MX) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[a][v][e] = fmaf(se, pt[a][v][e], acc[a][v][e]);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            acc[a][v][e] = fmaf(se, pt[a][v][e], fmaf(be, xc[a][e], acc[a][v][e]));
                    }
                }
            }
        }
    };

    // Pipeline, iteration i (compute buffer and weight set i % 2): stage the
    // activations of k-block i + 1 into the other buffer, issue the weights of
    // i + 1 into the other set and the activations of i + 2, compute i, barrier.
    // The next stage waits for the activations, the last loads issued, so every
    // load has one compute to arrive, and that holds on the first iteration as
    // on the others (the compiler's wait counts at the loop head take the worse
    // of the paths into it).  Loads past the slice's end repeat its last
    // k-block, and idle waves read row N - 1: a load issued on some paths only
    // would leave the counts unknown and turn every wait into a full drain.  A
    // block staged past the slice lands in the buffer nobody reads again.  The
    // loop body is unrolled by two so that every buffer and set index is a
    // constant.
    Words cw0[NV], cw1[NV];
    PairRaw pr0[NV][NF], pr1[NV][NF];
    load_b(cw0, pr0, kb0);
    load_a(kb0);
    stage_a(0);
    load_a(kb0 + min(1, nk - 1));
    __syncthreads();
    auto iter = [&](int i, int buf, const Words (&cw)[NV], const PairRaw (&pr)[NV][NF], Words (&cwn)[NV],
                    PairRaw (&prn)[NV][NF]) {
        stage_a(buf ^ 1);
        load_b(cwn, prn, kb0 + min(i + 1, nk - 1));
        load_a(kb0 + min(i + 2, nk - 1));
        if (i < nk) compute(buf, cw, pr);
        __syncthreads();
    };
    for (int i = 0; i < nk; i += 2) {   // uniform per block
        iter(i, 0, cw0, pr0, cw1, pr1);
        iter(i + 1, 1, cw1, pr1, cw0, pr0);
    }

    // epilogue: rows 16a + 4kq + e, output n0 + 16j + li
    if (!wlive) return;
    // the residuals first, all loads in flight together (rows and outputs clamped)
    float rv[GU ? 1 : NO][GU ? 1 : kPA][4];
    if constexpr (!GU) {
        if (!part) {
#pragma unroll
            for (int j = 0; j < NO; ++j)
#pragma unroll
                for (int a = 0; a < kPA; ++a)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int m = min(m0 + 16 * a + 4 * kq + e, M - 1), n = min(n0 + 16 * j + li, N - 1);
                        rv[j][a][e] = load_elem<ODT>(resid, static_cast<int64_t>(m) * N + n);
                    }
        }
    }
#pragma unroll
    for (int j = 0; j < NO; ++j) {
        const int n = n0 + 16 * j + li;
        if (n >= N) continue;
#pragma unroll
        for (int a = 0; a < kPA; ++a) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = m0 + 16 * a + 4 * kq + e;
                if (m >= M) continue;
                if (part) {
                    float* prow = part + (static_cast<size_t>(slice) * M + m) * (GU ? 2 * N : N);
                    if constexpr (GU) {
                        prow[n] = acc[a][2 * j][e];
                        prow[N + n] = acc[a][2 * j + 1][e];
                    } else {
                        prow[n] = acc[a][j][e];
                    }
                } else {
                    const int64_t o = static_cast<int64_t>(m) * N + n;
                    if constexpr (GU) {
                        const float g = acc[a][2 * j][e], u = acc[a][2 * j + 1][e];
                        static_cast<float*>(out)[o] = g / (1.0f + expf(-g)) * u;
                    } else {
                        store_elem<ODT>(out, o, rv[j][a][e] + acc[a][j][e]);
                    }
                }
            }
        }
    }
}

// The S slices' partials summed in slice order, then SwiGLU (gate/up: part
// rows hold gate at n and up at N + n) or the residual and the output rounding.
template <bool GU, int ODT>
__global__ void __launch_bounds__(256)
qmm_prefill_reduce_kernel(const float* __restrict__ part, const void* __restrict__ resid, void* __restrict__ out,
                          int N, int M, int S) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= static_cast<int64_t>(M) * N) return;
    const int m = static_cast<int>(i / N), n = static_cast<int>(i - static_cast<int64_t>(m) * N);
    const int64_t W = GU ? 2 * static_cast<int64_t>(N) : N;
    float g = 0.f, u = 0.f;
    for (int s = 0; s < S; ++s) {
        const float* p = part + (static_cast<int64_t>(s) * M + m) * W;
        g += p[n];
        if constexpr (GU) u += p[N + n];
    }
    if constexpr (GU)
        static_cast<float*>(out)[i] = g / (1.0f + expf(-g)) * u;
    else
        store_elem<ODT>(out, i, load_elem<ODT>(resid, i) + g);
}

constexpr int kNoGateUp = 1;   // output fragments per wave (gate/up)
constexpr int kNoDown = 2;     // output fragments per wave (down)

// Slices: doubled until there are two blocks per compute unit, each slice
// keeping at least two k-blocks.  The CU count is capped at the full gfx950
// chip's 256, so the partials' size for the full chip (what the workspace
// queries report) bounds every device this runs on.
constexpr int kMaxCus = 256;

int pick_slices(int tiles, int nkb, int cus) {
    cus = std::min(cus, kMaxCus);
    int s = 1;
    while (tiles * s < 2 * cus && 4 * s <= nkb && s < 16) s *= 2;
    return s;
}

// Output tiles of a projection and its k-blocks, as the launcher lays them out.
template <int BITS, int G, bool GU>
void prefill_grid(const qdm_weight& w, int m, int& nb, int& mb, int& nkb) {
    constexpr int NO = GU ? kNoGateUp : kNoDown;
    const int bn = 16 * NO * kPW;
    nb = (w.n + bn - 1) / bn;
    mb = (m + kPBM - 1) / kPBM;
    nkb = w.k / TileLayout<BITS, G>::KBK;
}

template <int BITS, int G, int XDT, bool GU, int ODT>
int run_prefill(const qdm_weight& w, const void* x, const void* r, void* out, int m, float* part, hipStream_t s) {
    constexpr int NO = GU ? kNoGateUp : kNoDown;
    auto kern = qmm_prefill_kernel<BITS, G, XDT, GU, ODT, NO>;
    const float* sbp = mx_bits(BITS) ? reinterpret_cast<const float*>(w.block_scales) : w.scale_bias;
    if (!sbp) return static_cast<int>(hipErrorInvalidValue);
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return static_cast<int>(hipErrorInvalidDevice);
    int nb = 0, mb = 0, nkb = 0;
    prefill_grid<BITS, G, GU>(w, m, nb, mb, nkb);
    const int S = pick_slices(nb * mb, nkb, cus);
    constexpr size_t lds = prefill_lds_bytes<BITS, G, GU>();
    if (lds > 65536 && hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds)) != hipSuccess)
        return static_cast<int>(hipErrorInvalidValue);
    if (S > 1 && !part) return static_cast<int>(hipErrorInvalidValue);
    // the kernel writes partials exactly when it is given a buffer for them:
    // an unsplit launch gets none, whatever the caller's workspace holds
    float* kpart = S > 1 ? part : nullptr;
    hipError_t e = launch(kern, dim3(nb * S, mb), dim3(kPT), lds, s, static_cast<const uint8_t*>(w.q), sbp, x, r,
                          out, kpart, w.n, w.k, m, S);
    if (e != hipSuccess || S == 1) return static_cast<int>(e);
    const int64_t outs = static_cast<int64_t>(m) * w.n;
    e = launch(qmm_prefill_reduce_kernel<GU, ODT>, dim3(static_cast<unsigned>((outs + 255) / 256)), dim3(256), 0, s,
               static_cast<const float*>(part), r, out, w.n, m, S);
    return static_cast<int>(e);
}

template <int XDT, bool GU, int ODT, int G>
int run_prefill_b(const qdm_weight& w, const void* x, const void* r, void* out, int m, float* part, hipStream_t s) {
    switch (w.bits) {
        case 8: return run_prefill<8, G, XDT, GU, ODT>(w, x, r, out, m, part, s);
        case 4: return run_prefill<4, G, XDT, GU, ODT>(w, x, r, out, m, part, s);
        case QDM_U8_SB16: return run_prefill<QDM_U8_SB16, G, XDT, GU, ODT>(w, x, r, out, m, part, s);
        default: return run_prefill<QDM_U4_SB16, G, XDT, GU, ODT>(w, x, r, out, m, part, s);
    }
}

template <int XDT, bool GU, int ODT>
int run_prefill_g(const qdm_weight& w, const void* x, const void* r, void* out, int m, float* part, hipStream_t s) {
    if (w.bits == QDM_MXFP8) return run_prefill<QDM_MXFP8, 32, XDT, GU, ODT>(w, x, r, out, m, part, s);
    if (w.bits == QDM_MXFP4) return run_prefill<QDM_MXFP4, 32, XDT, GU, ODT>(w, x, r, out, m, part, s);
    switch (w.group) {
        case 32: return run_prefill_b<XDT, GU, ODT, 32>(w, x, r, out, m, part, s);
        case 64: return run_prefill_b<XDT, GU, ODT, 64>(w, x, r, out, m, part, s);
        default: return run_prefill_b<XDT, GU, ODT, 128>(w, x, r, out, m, part, s);
    }
}

// Bytes of fp32 partials a split launch writes with the full chip's CU count
// (0 when the projection runs unsplit).
template <int BITS, int G, bool GU>
size_t partials_for(const qdm_weight& w, int m) {
    int nb = 0, mb = 0, nkb = 0;
    prefill_grid<BITS, G, GU>(w, m, nb, mb, nkb);
    const int S = pick_slices(nb * mb, nkb, kMaxCus);
    if (S == 1) return 0;
    return static_cast<size_t>(S) * static_cast<size_t>(m) * static_cast<size_t>(w.n) * (GU ? 2 : 1) * sizeof(float);
}

template <bool GU, int G>
size_t partials_b(const qdm_weight& w, int m) {
    switch (w.bits) {
        case 8: return partials_for<8, G, GU>(w, m);
        case 4: return partials_for<4, G, GU>(w, m);
        case QDM_U8_SB16: return partials_for<QDM_U8_SB16, G, GU>(w, m);
        default: return partials_for<QDM_U4_SB16, G, GU>(w, m);
    }
}

template <bool GU>
size_t partials_g(const qdm_weight& w, int m) {
    if (w.bits == QDM_MXFP8) return partials_for<QDM_MXFP8, 32, GU>(w, m);
    if (w.bits == QDM_MXFP4) return partials_for<QDM_MXFP4, 32, GU>(w, m);
    switch (w.group) {
        case 32: return partials_b<GU, 32>(w, m);
        case 64: return partials_b<GU, 64>(w, m);
        default: return partials_b<GU, 128>(w, m);
    }
}

}  // namespace

bool prefill_supported(const qdm_weight& w, int m, int act) {
    if (m <= kRows) return false;
    const bool affine = w.bits == 8 || w.bits == 4 || sb16_bits(w.bits);
    if (!affine && !mx_bits(w.bits)) return false;
    if (w.group != 32 && w.group != 64 && w.group != 128) return false;
    if (mx_bits(w.bits) && w.group != 32) return false;
    if (act != DT_BF16 && act != DT_F16) return false;
    const int kbk = (code_width(w.bits) == 4 || w.group == 32) ? 128 : 64;
    return w.n % 16 == 0 && w.k % kbk == 0;
}

size_t prefill_partials_bytes(const qdm_weight& w, int m, bool gate_up) {
    return gate_up ? partials_g<true>(w, m) : partials_g<false>(w, m);
}

int launch_gate_up_prefill(const void* x, int m, int act, const qdm_weight& gu, float* h, float* part, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    return act == DT_F16 ? run_prefill_g<DT_F16, true, DT_F32>(gu, x, nullptr, h, m, part, s)
                         : run_prefill_g<DT_BF16, true, DT_F32>(gu, x, nullptr, h, m, part, s);
}

int launch_down_prefill(const float* h, const void* r, int m, int act, const qdm_weight& dn, void* out, float* part,
                        void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    return act == DT_F16 ? run_prefill_g<DT_F32, false, DT_F16>(dn, h, r, out, m, part, s)
                         : run_prefill_g<DT_F32, false, DT_BF16>(dn, h, r, out, m, part, s);
}

}  // namespace qdm
