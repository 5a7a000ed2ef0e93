// Host-side affine and MX block-scaled quantization and packing (ahead of
// time, once per weight set).
//
// Pages: meTile docs, "MLX-LM Backend" -- affine formats keep a scale and a bias
// per group of 32/64/128 along the input dim; the 4-bit repack keeps nibbles,
// scales and biases and does not requantize; dense models get an interleaved
// gate/up view.  The quantizer formula is the plain reading stated in qdm.h.
//
// Built with g++ -ffp-contract=off and without fast-math: each fp64 operation
// below is one IEEE operation, rounded to nearest-even, in a fixed order, so
// the output is unique.
#include <algorithm>
#include <cfenv>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

#include "qdm.h"

namespace {

bool valid_bits_group(int32_t bits, int32_t group) {
    return (bits == 4 || bits == 8) && (group == 32 || group == 64 || group == 128);
}

// Runs fn(row_begin, row_end) over [0, n) on a few host threads.
template <class F>
void parallel_rows(int64_t n, int64_t row_cost, F fn) {
    unsigned hw = std::thread::hardware_concurrency();
    int64_t want = std::max<int64_t>(1, (n * row_cost) / (1 << 20));   // ~1M elements per thread
    int64_t nt = std::min<int64_t>({static_cast<int64_t>(hw ? hw : 1), want, n, 64});
    if (nt <= 1) {
        fn(int64_t{0}, n);
        return;
    }
    std::vector<std::thread> th;
    th.reserve(static_cast<size_t>(nt));
    for (int64_t t = 0; t < nt; ++t) {
        int64_t b = n * t / nt, e = n * (t + 1) / nt;
        th.emplace_back([=] { fn(b, e); });
    }
    for (auto& t : th) t.join();
}

bool all_finite(const float* w, int64_t count) {
    // checked up front so that a rejected call writes nothing
    bool good = true;
    for (int64_t i = 0; i < count; ++i) {
        if (!std::isfinite(w[i])) { good = false; break; }
    }
    return good;
}

// Quantizes one group of g weights: writes g codes (one per byte) and returns (scale, bias).
inline void quantize_group(const float* w, int32_t g, int32_t qmax, uint8_t* codes,
                           float* scale_out, float* bias_out) {
    float mn = w[0], mx = w[0];
    for (int32_t i = 1; i < g; ++i) {
        mn = w[i] < mn ? w[i] : mn;
        mx = w[i] > mx ? w[i] : mx;
    }
    if (mn == 0.0f) mn = 0.0f;                    // store a zero minimum as +0
    const double span = static_cast<double>(mx) - static_cast<double>(mn);
    const float scale = static_cast<float>(span / static_cast<double>(qmax));
    *scale_out = scale;
    *bias_out = mn;
    if (scale == 0.0f) {
        std::memset(codes, 0, static_cast<size_t>(g));
        return;
    }
    const double s = static_cast<double>(scale), b = static_cast<double>(mn);
    for (int32_t i = 0; i < g; ++i) {
        double t = (static_cast<double>(w[i]) - b) / s;
        double q = std::nearbyint(t);             // ties to even in the default mode
        q = q < 0.0 ? 0.0 : (q > qmax ? static_cast<double>(qmax) : q);
        codes[i] = static_cast<uint8_t>(q);
    }
}

// Packs one row of k codes (one per byte) into its storage bytes.
inline void pack_row_codes(const uint8_t* codes, int32_t k, int32_t bits, uint8_t* out) {
    if (bits == 8) {
        std::memcpy(out, codes, static_cast<size_t>(k));
    } else {
        for (int32_t i = 0; i < k / 2; ++i)
            out[i] = static_cast<uint8_t>(codes[2 * i] | (codes[2 * i + 1] << 4));
    }
}

// Quantizes and packs one row: q_row gets k*bits/8 bytes, sb_row 2*(k/group) floats.
void quantize_pack_row(const float* w, int32_t k, int32_t bits, int32_t group,
                       uint8_t* q_row, float* sb_row, uint8_t* scratch) {
    const int32_t qmax = (1 << bits) - 1;
    for (int32_t j = 0; j < k / group; ++j)
        quantize_group(w + static_cast<int64_t>(j) * group, group, qmax,
                       scratch + static_cast<int64_t>(j) * group, sb_row + 2 * j, sb_row + 2 * j + 1);
    pack_row_codes(scratch, k, bits, q_row);
}

bool codes_in_range(const uint8_t* codes, int64_t count, int32_t bits) {
    const int32_t lim = 1 << bits;
    for (int64_t i = 0; i < count; ++i)
        if (codes[i] >= lim) return false;
    return true;
}

// bf16 nearest-even of a finite fp32 value, as its 16 bits.
inline uint16_t bf16_bits(float f) {
    uint32_t u = 0;
    std::memcpy(&u, &f, 4);
    return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

inline double bf16_value(uint16_t b) {
    const uint32_t u = static_cast<uint32_t>(b) << 16;
    float f = 0.0f;
    std::memcpy(&f, &u, 4);
    return static_cast<double>(f);
}

// Quantizes and packs one row with bf16 (scale, bias) pairs: the group's fp32
// pair as in quantize_group, each rounded once to bf16, then the codes chosen
// against the rounded pair.
void quantize_pack_row_sb16(const float* w, int32_t k, int32_t bits, int32_t group, uint8_t* q_row,
                            uint16_t* sb_row, uint8_t* scratch) {
    const int32_t qmax = (1 << bits) - 1;
    for (int32_t j = 0; j < k / group; ++j) {
        const float* g = w + static_cast<int64_t>(j) * group;
        uint8_t* c = scratch + static_cast<int64_t>(j) * group;
        float sc = 0.0f, bi = 0.0f;
        quantize_group(g, group, qmax, c, &sc, &bi);
        const uint16_t sb = bf16_bits(sc), bb = bf16_bits(bi);
        sb_row[2 * j] = sb;
        sb_row[2 * j + 1] = bb;
        const double s = bf16_value(sb), b = bf16_value(bb);
        for (int32_t i = 0; i < group; ++i) {
            if (s == 0.0) {
                c[i] = 0;
                continue;
            }
            double q = std::nearbyint((static_cast<double>(g[i]) - b) / s);
            q = q < 0.0 ? 0.0 : (q > qmax ? static_cast<double>(qmax) : q);
            c[i] = static_cast<uint8_t>(q);
        }
    }
    pack_row_codes(scratch, k, bits, q_row);
}

// MX block-scaled formats: blocks of 32 along k, an E8M0 scale per block,
// E2M1 (MXFP4) or E4M3 (MXFP8) elements -- the OCP Microscaling formats the
// pages' MXFP4 / MXFP8 name ("MLX-LM Backend", "Block-Scaled MLX Primitive").
constexpr int32_t kMxBlock = 32;

struct MxFormat {
    int eb, mb, bias, emax;   // exponent bits, mantissa bits, exponent bias, largest normal exponent
    double vmax;              // largest element magnitude
};

inline bool is_mx(int32_t bits) { return bits == QDM_MXFP4 || bits == QDM_MXFP8; }

inline MxFormat mx_format(int32_t bits) {
    return bits == QDM_MXFP4 ? MxFormat{2, 1, 1, 2, 6.0} : MxFormat{4, 3, 7, 8, 448.0};
}

// |t| rounded to the element grid (ties to even mantissa), saturated at vmax.
inline double mx_round(double t, const MxFormat& f) {
    if (t == 0.0) return 0.0;
    int ex = 0;
    std::frexp(t, &ex);                            // t = m * 2^ex, 0.5 <= m < 1
    const int e = std::max(ex - 1, 1 - f.bias);    // subnormals share the smallest normal exponent
    const double quantum = std::ldexp(1.0, e - f.mb);
    const double r = std::nearbyint(t / quantum) * quantum;
    return r > f.vmax ? f.vmax : r;
}

// A grid magnitude -> its sign-less element code.
inline uint32_t mx_encode(double mag, const MxFormat& f) {
    if (mag == 0.0) return 0;
    int ex = 0;
    std::frexp(mag, &ex);
    const int e = ex - 1, emin = 1 - f.bias;
    if (e < emin) return static_cast<uint32_t>(std::nearbyint(mag / std::ldexp(1.0, emin - f.mb)));
    const uint32_t m = static_cast<uint32_t>(std::nearbyint((mag / std::ldexp(1.0, e) - 1.0) * (1 << f.mb)));
    return (static_cast<uint32_t>(e + f.bias) << f.mb) | m;
}

// Quantizes and stores one row: q_row gets k (MXFP8) or k/2 (MXFP4) bytes, e_row k/32 scale codes.
void quantize_mx_row(const float* w, int32_t k, int32_t bits, uint8_t* q_row, uint8_t* e_row, uint8_t* scratch) {
    const MxFormat f = mx_format(bits);
    const uint32_t sign = 1u << (f.eb + f.mb);
    for (int32_t b = 0; b < k / kMxBlock; ++b) {
        const float* v = w + static_cast<int64_t>(b) * kMxBlock;
        float amax = 0.0f;
        for (int32_t i = 0; i < kMxBlock; ++i) amax = std::max(amax, std::fabs(v[i]));
        int shared = -127;
        if (amax > 0.0f) {
            int ex = 0;
            std::frexp(static_cast<double>(amax), &ex);
            shared = std::min(127, std::max(-127, ex - 1 - f.emax));
        }
        e_row[b] = static_cast<uint8_t>(shared + 127);
        for (int32_t i = 0; i < kMxBlock; ++i) {
            const double t = std::ldexp(std::fabs(static_cast<double>(v[i])), -shared);
            const uint32_t c = mx_encode(mx_round(t, f), f) | (v[i] < 0.0f ? sign : 0u);
            scratch[static_cast<int64_t>(b) * kMxBlock + i] = static_cast<uint8_t>(c);
        }
    }
    pack_row_codes(scratch, k, bits == QDM_MXFP4 ? 4 : 8, q_row);
}

}  // namespace

extern "C" {

int qdm_quantize_pack_rows_sb16(const float* w, int32_t n, int32_t k, int32_t bits, int32_t group, void* q_out,
                                uint16_t* scale_bias_out) {
    if (!w || !q_out || !scale_bias_out || n <= 0 || k <= 0 || group <= 0) return QDM_ERR_INVALID_ARG;
    if (!valid_bits_group(bits, group)) return QDM_ERR_UNSUPPORTED;
    if (k % group) return QDM_ERR_INVALID_ARG;
    if (!all_finite(w, static_cast<int64_t>(n) * k)) return QDM_ERR_INVALID_ARG;
    const int32_t ng = k / group;
    const int64_t rb = static_cast<int64_t>(k) * bits / 8;
    auto* q = static_cast<uint8_t*>(q_out);
    parallel_rows(n, k, [&](int64_t b, int64_t e) {
        std::vector<uint8_t> scratch(static_cast<size_t>(k));
        for (int64_t i = b; i < e; ++i)
            quantize_pack_row_sb16(w + i * k, k, bits, group, q + i * rb, scale_bias_out + 2 * i * ng, scratch.data());
    });
    return QDM_OK;
}

int qdm_quantize_pack_gate_up_sb16(const float* w_gate, const float* w_up, int32_t ffn, int32_t d, int32_t bits,
                                   int32_t group, void* q_out, uint16_t* scale_bias_out) {
    if (!w_gate || !w_up || !q_out || !scale_bias_out || ffn <= 0 || d <= 0 || group <= 0)
        return QDM_ERR_INVALID_ARG;
    if (!valid_bits_group(bits, group)) return QDM_ERR_UNSUPPORTED;
    if (d % group) return QDM_ERR_INVALID_ARG;
    const int64_t nd = static_cast<int64_t>(ffn) * d;
    if (!all_finite(w_gate, nd) || !all_finite(w_up, nd)) return QDM_ERR_INVALID_ARG;
    const int32_t ng = d / group;
    const int64_t rb = static_cast<int64_t>(d) * bits / 8;
    auto* q = static_cast<uint8_t*>(q_out);
    parallel_rows(ffn, 2 * static_cast<int64_t>(d), [&](int64_t b, int64_t e) {
        std::vector<uint8_t> scratch(static_cast<size_t>(d));
        for (int64_t f = b; f < e; ++f) {
            quantize_pack_row_sb16(w_gate + f * d, d, bits, group, q + (2 * f) * rb, scale_bias_out + (2 * f) * 2 * ng,
                                   scratch.data());
            quantize_pack_row_sb16(w_up + f * d, d, bits, group, q + (2 * f + 1) * rb,
                                   scale_bias_out + (2 * f + 1) * 2 * ng, scratch.data());
        }
    });
    return QDM_OK;
}

size_t qdm_mx_scale_bytes(int32_t n, int32_t k) {
    if (n <= 0 || k <= 0 || k % kMxBlock) return 0;
    return static_cast<size_t>(n) * static_cast<size_t>(k / kMxBlock);
}

int qdm_quantize_mx(const float* w, int32_t n, int32_t k, int32_t format, void* q_out, uint8_t* scales_out) {
    if (!w || !q_out || !scales_out || n <= 0 || k <= 0) return QDM_ERR_INVALID_ARG;
    if (!is_mx(format)) return QDM_ERR_UNSUPPORTED;
    if (k % kMxBlock) return QDM_ERR_INVALID_ARG;
    if (!all_finite(w, static_cast<int64_t>(n) * k)) return QDM_ERR_INVALID_ARG;
    const int64_t rb = format == QDM_MXFP4 ? k / 2 : k;
    const int32_t nb = k / kMxBlock;
    auto* q = static_cast<uint8_t*>(q_out);
    parallel_rows(n, k, [&](int64_t b, int64_t e) {
        std::vector<uint8_t> scratch(static_cast<size_t>(k));
        for (int64_t i = b; i < e; ++i) quantize_mx_row(w + i * k, k, format, q + i * rb, scales_out + i * nb, scratch.data());
    });
    return QDM_OK;
}

int qdm_quantize_mx_gate_up(const float* w_gate, const float* w_up, int32_t ffn, int32_t d, int32_t format,
                            void* q_out, uint8_t* scales_out) {
    if (!w_gate || !w_up || !q_out || !scales_out || ffn <= 0 || d <= 0) return QDM_ERR_INVALID_ARG;
    if (!is_mx(format)) return QDM_ERR_UNSUPPORTED;
    if (d % kMxBlock) return QDM_ERR_INVALID_ARG;
    const int64_t nd = static_cast<int64_t>(ffn) * d;
    if (!all_finite(w_gate, nd) || !all_finite(w_up, nd)) return QDM_ERR_INVALID_ARG;
    const int64_t rb = format == QDM_MXFP4 ? d / 2 : d;
    const int32_t nb = d / kMxBlock;
    auto* q = static_cast<uint8_t*>(q_out);
    parallel_rows(ffn, 2 * static_cast<int64_t>(d), [&](int64_t b, int64_t e) {
        std::vector<uint8_t> scratch(static_cast<size_t>(d));
        for (int64_t r = b; r < e; ++r) {
            quantize_mx_row(w_gate + r * d, d, format, q + (2 * r) * rb, scales_out + (2 * r) * nb, scratch.data());
            quantize_mx_row(w_up + r * d, d, format, q + (2 * r + 1) * rb, scales_out + (2 * r + 1) * nb,
                            scratch.data());
        }
    });
    return QDM_OK;
}

size_t qdm_packed_q_bytes(int32_t n, int32_t k, int32_t bits) {
    if (n <= 0 || k <= 0) return 0;
    const size_t nk = static_cast<size_t>(n) * static_cast<size_t>(k);
    if (bits == 8) return nk;
    if (bits == 4) return (k % 2) ? 0 : nk / 2;
    if (bits == 16) return nk * 2;
    if (bits == QDM_U8_SB16) return nk;
    if (bits == QDM_U4_SB16) return (k % 2) ? 0 : nk / 2;
    if (bits == QDM_MXFP8) return nk;
    if (bits == QDM_MXFP4) return (k % 2) ? 0 : nk / 2;
    return 0;
}

size_t qdm_scale_bias_floats(int32_t n, int32_t k, int32_t group) {
    if (n <= 0 || k <= 0 || group <= 0 || k % group) return 0;
    return 2 * static_cast<size_t>(n) * static_cast<size_t>(k / group);
}

int qdm_quantize_affine(const float* w, int32_t n, int32_t k, int32_t bits, int32_t group,
                        uint8_t* codes, float* scale, float* bias) {
    if (!w || !codes || !scale || !bias || n <= 0 || k <= 0 || group <= 0) return QDM_ERR_INVALID_ARG;
    if (!valid_bits_group(bits, group)) return QDM_ERR_UNSUPPORTED;
    if (k % group) return QDM_ERR_INVALID_ARG;
    const int64_t nk = static_cast<int64_t>(n) * k;
    if (!all_finite(w, nk)) return QDM_ERR_INVALID_ARG;
    const int32_t qmax = (1 << bits) - 1, ng = k / group;
    parallel_rows(n, k, [&](int64_t b, int64_t e) {
        for (int64_t i = b; i < e; ++i)
            for (int32_t j = 0; j < ng; ++j)
                quantize_group(w + i * k + static_cast<int64_t>(j) * group, group, qmax,
                               codes + i * k + static_cast<int64_t>(j) * group,
                               scale + i * ng + j, bias + i * ng + j);
    });
    return QDM_OK;
}

int qdm_pack_rows(const uint8_t* codes, const float* scale, const float* bias,
                  int32_t n, int32_t k, int32_t bits, int32_t group,
                  void* q_out, float* scale_bias_out) {
    if (!codes || !scale || !bias || !q_out || !scale_bias_out || n <= 0 || k <= 0 || group <= 0)
        return QDM_ERR_INVALID_ARG;
    if (!valid_bits_group(bits, group)) return QDM_ERR_UNSUPPORTED;
    if (k % group) return QDM_ERR_INVALID_ARG;
    if (!codes_in_range(codes, static_cast<int64_t>(n) * k, bits)) return QDM_ERR_INVALID_ARG;
    const int32_t ng = k / group;
    const int64_t rb = static_cast<int64_t>(k) * bits / 8;
    auto* q = static_cast<uint8_t*>(q_out);
    parallel_rows(n, k, [&](int64_t b, int64_t e) {
        for (int64_t i = b; i < e; ++i) {
            pack_row_codes(codes + i * k, k, bits, q + i * rb);
            for (int32_t j = 0; j < ng; ++j) {
                scale_bias_out[2 * (i * ng + j)] = scale[i * ng + j];
                scale_bias_out[2 * (i * ng + j) + 1] = bias[i * ng + j];
            }
        }
    });
    return QDM_OK;
}

int qdm_quantize_pack_rows(const float* w, int32_t n, int32_t k, int32_t bits, int32_t group,
                           void* q_out, float* scale_bias_out) {
    if (!w || !q_out || !scale_bias_out || n <= 0 || k <= 0 || group <= 0) return QDM_ERR_INVALID_ARG;
    if (!valid_bits_group(bits, group)) return QDM_ERR_UNSUPPORTED;
    if (k % group) return QDM_ERR_INVALID_ARG;
    if (!all_finite(w, static_cast<int64_t>(n) * k)) return QDM_ERR_INVALID_ARG;
    const int32_t ng = k / group;
    const int64_t rb = static_cast<int64_t>(k) * bits / 8;
    auto* q = static_cast<uint8_t*>(q_out);
    parallel_rows(n, k, [&](int64_t b, int64_t e) {
        std::vector<uint8_t> scratch(static_cast<size_t>(k));
        for (int64_t i = b; i < e; ++i)
            quantize_pack_row(w + i * k, k, bits, group, q + i * rb, scale_bias_out + 2 * i * ng,
                              scratch.data());
    });
    return QDM_OK;
}

int qdm_quantize_pack_gate_up(const float* w_gate, const float* w_up, int32_t ffn, int32_t d,
                              int32_t bits, int32_t group, void* q_out, float* scale_bias_out) {
    if (!w_gate || !w_up || !q_out || !scale_bias_out || ffn <= 0 || d <= 0 || group <= 0)
        return QDM_ERR_INVALID_ARG;
    if (!valid_bits_group(bits, group)) return QDM_ERR_UNSUPPORTED;
    if (d % group) return QDM_ERR_INVALID_ARG;
    const int64_t nd = static_cast<int64_t>(ffn) * d;
    if (!all_finite(w_gate, nd) || !all_finite(w_up, nd)) return QDM_ERR_INVALID_ARG;
    const int32_t ng = d / group;
    const int64_t rb = static_cast<int64_t>(d) * bits / 8;
    auto* q = static_cast<uint8_t*>(q_out);
    parallel_rows(ffn, 2 * static_cast<int64_t>(d), [&](int64_t b, int64_t e) {
        std::vector<uint8_t> scratch(static_cast<size_t>(d));
        for (int64_t f = b; f < e; ++f) {
            quantize_pack_row(w_gate + f * d, d, bits, group, q + (2 * f) * rb,
                              scale_bias_out + (2 * f) * 2 * ng, scratch.data());
            quantize_pack_row(w_up + f * d, d, bits, group, q + (2 * f + 1) * rb,
                              scale_bias_out + (2 * f + 1) * 2 * ng, scratch.data());
        }
    });
    return QDM_OK;
}

int qdm_pack_gate_up(const uint8_t* gate_codes, const float* gate_scale, const float* gate_bias,
                     const uint8_t* up_codes, const float* up_scale, const float* up_bias,
                     int32_t ffn, int32_t d, int32_t bits, int32_t group,
                     void* q_out, float* scale_bias_out) {
    if (!gate_codes || !gate_scale || !gate_bias || !up_codes || !up_scale || !up_bias || !q_out ||
        !scale_bias_out || ffn <= 0 || d <= 0 || group <= 0)
        return QDM_ERR_INVALID_ARG;
    if (!valid_bits_group(bits, group)) return QDM_ERR_UNSUPPORTED;
    if (d % group) return QDM_ERR_INVALID_ARG;
    const int64_t nd = static_cast<int64_t>(ffn) * d;
    if (!codes_in_range(gate_codes, nd, bits) || !codes_in_range(up_codes, nd, bits))
        return QDM_ERR_INVALID_ARG;
    const int32_t ng = d / group;
    const int64_t rb = static_cast<int64_t>(d) * bits / 8;
    auto* q = static_cast<uint8_t*>(q_out);
    parallel_rows(ffn, 2 * static_cast<int64_t>(d), [&](int64_t b, int64_t e) {
        for (int64_t f = b; f < e; ++f) {
            for (int v = 0; v < 2; ++v) {
                const uint8_t* c = (v ? up_codes : gate_codes) + f * d;
                const float* s = (v ? up_scale : gate_scale) + f * ng;
                const float* bb = (v ? up_bias : gate_bias) + f * ng;
                const int64_t row = 2 * f + v;
                pack_row_codes(c, d, bits, q + row * rb);
                for (int32_t j = 0; j < ng; ++j) {
                    scale_bias_out[2 * (row * ng + j)] = s[j];
                    scale_bias_out[2 * (row * ng + j) + 1] = bb[j];
                }
            }
        }
    });
    return QDM_OK;
}

int qdm_pack_dense_gate_up(const uint16_t* gate_bf16, const uint16_t* up_bf16,
                           int32_t ffn, int32_t d, uint16_t* out) {
    if (!gate_bf16 || !up_bf16 || !out || ffn <= 0 || d <= 0) return QDM_ERR_INVALID_ARG;
    parallel_rows(ffn, 2 * static_cast<int64_t>(d), [&](int64_t b, int64_t e) {
        for (int64_t f = b; f < e; ++f) {
            std::memcpy(out + (2 * f) * d, gate_bf16 + f * d, sizeof(uint16_t) * d);
            std::memcpy(out + (2 * f + 1) * d, up_bf16 + f * d, sizeof(uint16_t) * d);
        }
    });
    return QDM_OK;
}

}  // extern "C"
