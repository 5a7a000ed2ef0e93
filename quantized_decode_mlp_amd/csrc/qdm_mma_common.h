// Pieces shared by the few-row matrix-core kernels (gate/up and down): the
// MMA in the activations' 16-bit type, codes as exact MMA operands, and the
// layout of a k-block across a wave's lanes.
//
// Pages: meTile docs, "MLX-LM Backend", section "Dispatch Policy" (several
// activation rows go to matrix tiles); MLX-LM affine groups w = scale*q + bias.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "qdm.h"
#include "qdm_device.h"

namespace qdm {
namespace {

typedef _Float16 h16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));

constexpr int kRows = 16;     // rows of the matrix tile
constexpr int kPad = 8;       // f16 padding per staged row: 16 bytes, four LDS banks per row
constexpr int kLdsCap = 160 * 1024;

// 16x16x32 MMA in the activations' 16-bit type (bf16 or f16 operands)
template <int XDT>
__device__ __forceinline__ f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
    if constexpr (XDT == DT_BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                       0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h16x8, a), __builtin_bit_cast(h16x8, b), c, 0,
                                                      0, 0);
}

// The eight codes of one lane and k-step as exact operand values off + c / inv
// in the MMA's 16-bit type.  8-bit codes: f16 1024 + c (the byte under the
// exponent byte 0x64, one permute per two codes) or the bf16 integer c (an
// exact byte conversion and a permute of the high halves; no offset).  4-bit
// codes: 1 + c/16 in either type (the nibble in the top mantissa bits of 1.0,
// a shift and an and-or per two codes); element pairs (e, e + 4), so the
// staged activations take that order too.
template <int BITS, int XDT>
struct StepCodes;

template <int BITS>
struct StepWords;

template <>
struct StepWords<8> {
    using raw = u32x2;   // codes k + 0..7, one byte each
    template <class W>
    __device__ __forceinline__ static raw step(const W& w, int t) { return u32x2{w[2 * t], w[2 * t + 1]}; }
    template <class W>
    __device__ __forceinline__ static void set_step(W& w, int t, raw r) {
        w[2 * t] = r[0];
        w[2 * t + 1] = r[1];
    }
};

template <>
struct StepWords<4> {
    using raw = uint32_t;   // codes k + 0..7, low nibble first
    template <class W>
    __device__ __forceinline__ static raw step(const W& w, int t) { return w[t]; }
    template <class W>
    __device__ __forceinline__ static void set_step(W& w, int t, raw r) { w[t] = r; }
};

template <>
struct StepCodes<8, DT_F16> : StepWords<8> {
    static constexpr float kOff = 1024.f, kInvMul = 1.f;
    __device__ __forceinline__ static u32x4 operand(raw w) {
        return u32x4{__builtin_amdgcn_perm(0x64646464u, w[0], 0x04010400u),
                     __builtin_amdgcn_perm(0x64646464u, w[0], 0x04030402u),
                     __builtin_amdgcn_perm(0x64646464u, w[1], 0x04010400u),
                     __builtin_amdgcn_perm(0x64646464u, w[1], 0x04030402u)};
    }
};

template <>
struct StepCodes<8, DT_BF16> : StepWords<8> {
    static constexpr float kOff = 0.f, kInvMul = 1.f;
    // element 0 (low half) = a, element 1 = b, both exact bf16 values
    __device__ __forceinline__ static uint32_t pack_hi(float a, float b) {
        return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
    }
    __device__ __forceinline__ static u32x4 operand(raw w) {
        auto byte = [](uint32_t v, int i) { return static_cast<float>((v >> (8 * i)) & 0xffu); };
        return u32x4{pack_hi(byte(w[0], 0), byte(w[0], 1)), pack_hi(byte(w[0], 2), byte(w[0], 3)),
                     pack_hi(byte(w[1], 0), byte(w[1], 1)), pack_hi(byte(w[1], 2), byte(w[1], 3))};
    }
};

template <>
struct StepCodes<4, DT_F16> : StepWords<4> {
    static constexpr float kOff = 1.f, kInvMul = 16.f;
    // mantissa bits 9..6 of f16 1.0
    __device__ __forceinline__ static u32x4 operand(raw w) {
        return u32x4{((w << 6) & 0x03c003c0u) | 0x3c003c00u, ((w << 2) & 0x03c003c0u) | 0x3c003c00u,
                     ((w >> 2) & 0x03c003c0u) | 0x3c003c00u, ((w >> 6) & 0x03c003c0u) | 0x3c003c00u};
    }
};

template <>
struct StepCodes<4, DT_BF16> : StepWords<4> {
    static constexpr float kOff = 1.f, kInvMul = 16.f;
    // mantissa bits 6..3 of bf16 1.0
    __device__ __forceinline__ static u32x4 operand(raw w) {
        return u32x4{((w << 3) & 0x00780078u) | 0x3f803f80u, ((w >> 1) & 0x00780078u) | 0x3f803f80u,
                     ((w >> 5) & 0x00780078u) | 0x3f803f80u, ((w >> 9) & 0x00780078u) | 0x3f803f80u};
    }
};

// MX block-scaled elements (E4M3 bytes, E2M1 nibbles low first) as exact
// operands in the MMA's type: the hardware converts a pair per instruction
// (E4M3 bytes 0,1 / 2,3 of a dword; E2M1 nibbles of one byte), keeping k
// order, so the staged activations stay in natural order.  No offset; the
// block scale arrives through the (scale, bias) pair as (2^(e - 127), 0).
template <int XDT>
__device__ __forceinline__ uint32_t mx8_pair(uint32_t w, bool hi) {
    if constexpr (XDT == DT_BF16) {
        return hi ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true))
                  : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
    } else {
        return hi ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true))
                  : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
    }
}

template <int XDT, int B>
__device__ __forceinline__ uint32_t mx4_pair(uint32_t w) {
    if constexpr (XDT == DT_BF16)
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, B));
    else
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, B));
}

template <int XDT>
struct StepCodes<QDM_MXFP8, XDT> : StepWords<8> {
    static constexpr float kOff = 0.f, kInvMul = 1.f;
    __device__ __forceinline__ static u32x4 operand(raw w) {
        return u32x4{mx8_pair<XDT>(w[0], false), mx8_pair<XDT>(w[0], true), mx8_pair<XDT>(w[1], false),
                     mx8_pair<XDT>(w[1], true)};
    }
};

template <int XDT>
struct StepCodes<QDM_MXFP4, XDT> : StepWords<4> {
    static constexpr float kOff = 0.f, kInvMul = 1.f;
    __device__ __forceinline__ static u32x4 operand(raw w) {
        return u32x4{mx4_pair<XDT, 0>(w), mx4_pair<XDT, 1>(w), mx4_pair<XDT, 2>(w), mx4_pair<XDT, 3>(w)};
    }
};

// The affine formats with bf16 (scale, bias) pairs take the plain affine codes.
template <int XDT>
struct StepCodes<QDM_U8_SB16, XDT> : StepCodes<8, XDT> {};
template <int XDT>
struct StepCodes<QDM_U4_SB16, XDT> : StepCodes<4, XDT> {};

constexpr bool mx_bits(int bits) { return bits == QDM_MXFP4 || bits == QDM_MXFP8; }
constexpr bool sb16_bits(int bits) { return bits == QDM_U4_SB16 || bits == QDM_U8_SB16; }
// affine 4-bit codes (either pair storage): element pairs (e, e + 4), so the staged rows are permuted
constexpr bool nibble_pairs(int bits) { return bits == 4 || bits == QDM_U4_SB16; }
constexpr int code_width(int bits) { return bits & 0xff; }

// An E8M0 code as its fp32 power of two (code 0: the subnormal 2^-127).
__device__ __forceinline__ float e8m0_value(uint32_t e) { return __uint_as_float(e ? e << 23 : 0x00400000u); }

// k-block layout.  WIDE (groups of 64 or more): a k-block is KBK k, lane kq
// holds the LK = KBK/4 consecutive k from LK*kq (one 16-byte load per row),
// k-step t takes its codes 8t .. 8t+7; a block spanning NF > 1 groups runs
// each step once per group with the activation kept only on that group's
// lanes.  Otherwise (32-wide groups, GROUPED) a k-block is 128 k, lane kq
// holds k 32t + 8kq .. +7 of step t and each step is one group: lane kq
// loads the whole group kq (16 bytes of 4-bit codes, 32 of 8-bit ones) and
// the four lane slots exchange words before use (transpose_slots), so that
// slot kq ends up with its eight codes of every group of the block.
template <int BITS, int G>
struct BlockLayout {
    static constexpr int CB = code_width(BITS);   // bits per code
    static constexpr bool WIDE = G >= 64;
    static constexpr bool GROUPED = !WIDE;
    static constexpr int KBK = (CB == 4 || GROUPED) ? 128 : 64;
    static constexpr int STEPS = KBK / 32;
    static constexpr int LK = KBK / 4;
    static constexpr int FG = WIDE ? (G < KBK ? G : KBK) : 32;   // fold chunk (k)
    static constexpr int NF = KBK / FG;                           // fold chunks per k-block
    using Words = typename std::conditional<GROUPED && CB == 8, u32x8, u32x4>::type;
};

// The four lane slots' words transposed (slots are the wave's 16-lane rows):
// word t of slot kq becomes word kq of slot t, by one exchange of row pairs
// (0,1)<->(2,3) and one of rows 0<->1, 2<->3.
__device__ __forceinline__ u32x4 transpose_slots(const u32x4& w) {
    const uint32_t w0 = w[0], w1 = w[1], w2 = w[2], w3 = w[3];
    const auto a = __builtin_amdgcn_permlane32_swap(w0, w2, false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(w1, w3, false, false);
    const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
    const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
    return u32x4{c[0], c[1], d[0], d[1]};
}

// 8-bit codes: a step's eight codes are the word pair (2t, 2t + 1), so the
// even and the odd words are exchanged separately.
__device__ __forceinline__ u32x8 transpose_slots(const u32x8& w) {
    const u32x4 e = transpose_slots(u32x4{w[0], w[2], w[4], w[6]});
    const u32x4 o = transpose_slots(u32x4{w[1], w[3], w[5], w[7]});
    return u32x8{e[0], o[0], e[1], o[1], e[2], o[2], e[3], o[3]};
}

__host__ __device__ constexpr size_t round16(size_t v) { return (v + 15) & ~static_cast<size_t>(15); }

// Pair registers per row set (8 groups each) for the groups of one wave's
// k-range: up to 16 groups at 64- and 128-wide groups, 32 at 32-wide ones.
template <int G>
constexpr int pair_regs() { return G == 32 ? 4 : 2; }

}  // namespace
}  // namespace qdm
