// Host-side affine quantization and packing (ahead of time, once per weight set).
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

}  // namespace

extern "C" {

size_t qdm_packed_q_bytes(int32_t n, int32_t k, int32_t bits) {
    if (n <= 0 || k <= 0) return 0;
    const size_t nk = static_cast<size_t>(n) * static_cast<size_t>(k);
    if (bits == 8) return nk;
    if (bits == 4) return (k % 2) ? 0 : nk / 2;
    if (bits == 16) return nk * 2;
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
