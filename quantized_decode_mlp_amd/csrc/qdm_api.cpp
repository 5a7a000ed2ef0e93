// C-ABI entry points of the device path: argument validation, then dispatch to
// the HIP launchers.  Every check runs before anything is launched, so a
// rejected call writes nothing.  Host C++ only (no HIP headers needed here).
#include <algorithm>
#include <cmath>
#include <cstdint>

#include "qdm.h"
#include "qdm_internal.h"

namespace {

constexpr int kMaxRows = 4096;   // rows per call
constexpr int kPassRows = 16;    // rows per kernel pass (the few-row kernels' matrix tile)

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool valid_dtype(int dt) { return dt == QDM_F32 || dt == QDM_F16 || dt == QDM_BF16; }

// Checks a weight descriptor; n_expect / k_expect < 0 means "any".
int check_weight(const qdm_weight* w) {
    if (!w || !w->q || w->n <= 0 || w->k <= 0) return QDM_ERR_INVALID_ARG;
    if (w->bits == 16) {
        if (w->group != 0) return QDM_ERR_INVALID_ARG;
        if (w->k % 8) return QDM_ERR_UNSUPPORTED;
    } else if (w->bits == QDM_MXFP4 || w->bits == QDM_MXFP8) {
        if (w->group != 32) return QDM_ERR_UNSUPPORTED;
        if (w->k % 32) return QDM_ERR_INVALID_ARG;
        if (!w->block_scales) return QDM_ERR_INVALID_ARG;
    } else if (w->bits == 8 || w->bits == 4 || w->bits == QDM_U8_SB16 || w->bits == QDM_U4_SB16) {
        if (!(w->group == 32 || w->group == 64 || w->group == 128)) return QDM_ERR_UNSUPPORTED;
        if (w->k % w->group) return QDM_ERR_INVALID_ARG;
        if (!w->scale_bias) return QDM_ERR_INVALID_ARG;
        if (!aligned(w->scale_bias, 8)) return QDM_ERR_ALIGNMENT;
    } else {
        return QDM_ERR_UNSUPPORTED;
    }
    if (!aligned(w->q, 16)) return QDM_ERR_ALIGNMENT;
    return QDM_OK;
}

int check_rows(int32_t m) { return (m >= 1 && m <= kMaxRows) ? QDM_OK : (m < 1 ? QDM_ERR_INVALID_ARG : QDM_ERR_UNSUPPORTED); }

int hip_status(int e) { return e == 0 ? QDM_OK : QDM_ERR_HIP; }

bool is_mx(int32_t bits) { return bits == QDM_MXFP4 || bits == QDM_MXFP8; }

// formats that only the weight-streaming kernels (one row) and the few-row
// matrix-core streaming kernels take: MX and the bf16-pair affine formats
bool stream_only(int32_t bits) { return is_mx(bits) || bits == QDM_U4_SB16 || bits == QDM_U8_SB16; }

size_t round256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

size_t act_bytes(int dt) { return dt == QDM_F32 ? 4 : 2; }

// MX weights: one row on the weight-streaming kernel (x of xb bytes); 2..16
// rows of a gate/up (kind 0) or down (kind 1) projection on the matrix-core
// streaming kernels (16-bit activations / outputs); nothing else.
int check_mx_pass(const qdm_weight* w, int32_t m, int xb, int act, int kind) {
    if (m == 1) return qdm::stream_supported(*w, xb) ? QDM_OK : QDM_ERR_UNSUPPORTED;
    if (kind == 0) return qdm::mma_stream_gate_up_supported(*w, m, act) ? QDM_OK : QDM_ERR_UNSUPPORTED;
    if (kind == 1) return qdm::mma_stream_down_supported(*w, m, act) ? QDM_OK : QDM_ERR_UNSUPPORTED;
    return QDM_ERR_UNSUPPORTED;
}

// (rows run in passes of at most kPassRows: the full passes and the remainder are checked)
int check_mx_rows(const qdm_weight* w, int32_t m, int xb, int act, int kind) {
    if (!stream_only(w->bits)) return QDM_OK;
    if (kind != 2 && qdm::prefill_supported(*w, m, act)) return QDM_OK;
    if (m > kPassRows)
        if (int e = check_mx_pass(w, kPassRows, xb, act, kind)) return e;
    const int32_t rem = m % kPassRows;
    return check_mx_pass(w, m <= kPassRows ? m : (rem ? rem : kPassRows), xb, act, kind);
}

// The device calls: one tiled launch for more than kPassRows rows where the
// prefill kernels take the weight, otherwise row passes of at most kPassRows
// rows (each pass streams the weights).
int gate_up_passes(const void* x, int32_t m, int act, const qdm_weight& gu, float* h, void* stream) {
    if (qdm::prefill_supported(gu, m, act)) return qdm::launch_gate_up_prefill(x, m, act, gu, h, stream);
    const size_t xe = act_bytes(act);
    for (int32_t m0 = 0; m0 < m; m0 += kPassRows) {
        const int32_t mr = std::min(kPassRows, m - m0);
        if (int e = qdm::launch_gate_up_swiglu(static_cast<const char*>(x) + static_cast<size_t>(m0) * gu.k * xe, mr,
                                               act, gu, h + static_cast<size_t>(m0) * gu.n, stream))
            return e;
    }
    return 0;
}

int down_passes(const float* h, const void* r, int32_t m, int act, const qdm_weight& dn, void* out, void* stream) {
    if (qdm::prefill_supported(dn, m, act)) return qdm::launch_down_prefill(h, r, m, act, dn, out, stream);
    const size_t oe = act_bytes(act);
    for (int32_t m0 = 0; m0 < m; m0 += kPassRows) {
        const int32_t mr = std::min(kPassRows, m - m0);
        const size_t ro = static_cast<size_t>(m0) * dn.n * oe;
        if (int e = qdm::launch_down_residual(h + static_cast<size_t>(m0) * dn.k, static_cast<const char*>(r) + ro, mr,
                                              act, dn, static_cast<char*>(out) + ro, stream))
            return e;
    }
    return 0;
}

int linear_passes(const void* x, int32_t m, int act, const qdm_weight& w, const void* bias, void* out, void* stream) {
    const size_t xe = act_bytes(act);
    for (int32_t m0 = 0; m0 < m; m0 += kPassRows) {
        const int32_t mr = std::min(kPassRows, m - m0);
        if (int e = qdm::launch_linear(static_cast<const char*>(x) + static_cast<size_t>(m0) * w.k * xe, mr, act, w,
                                       bias, static_cast<char*>(out) + static_cast<size_t>(m0) * w.n * xe, stream))
            return e;
    }
    return 0;
}

}  // namespace

extern "C" {

size_t qdm_mlp_workspace_bytes(int32_t m, int32_t ffn) {
    if (m <= 0 || ffn <= 0) return 0;
    const size_t b = static_cast<size_t>(m) * static_cast<size_t>(ffn) * sizeof(float);
    return (b + 255) & ~static_cast<size_t>(255);
}

int qdm_gemv_gate_up_swiglu(const void* x, int32_t m, qdm_dtype act, const qdm_weight* gate_up,
                            float* h_out, void* stream) {
    if (!x || !h_out) return QDM_ERR_INVALID_ARG;
    if (!valid_dtype(act)) return QDM_ERR_INVALID_ARG;
    if (int e = check_rows(m)) return e;
    if (int e = check_weight(gate_up)) return e;
    if (int e = check_mx_rows(gate_up, m, act == QDM_F32 ? 4 : 2, act, 0)) return e;
    if (!aligned(x, 16) || !aligned(h_out, 16)) return QDM_ERR_ALIGNMENT;
    return hip_status(gate_up_passes(x, m, act, *gate_up, h_out, stream));
}

int qdm_gemv_down_residual(const float* h, const void* r, int32_t m, qdm_dtype act,
                           const qdm_weight* down, void* out, void* stream) {
    if (!h || !r || !out) return QDM_ERR_INVALID_ARG;
    if (static_cast<const void*>(h) == out) return QDM_ERR_INVALID_ARG;
    if (!valid_dtype(act)) return QDM_ERR_INVALID_ARG;
    if (int e = check_rows(m)) return e;
    if (int e = check_weight(down)) return e;
    if (int e = check_mx_rows(down, m, 4, act, 1)) return e;
    if (!aligned(h, 16) || !aligned(r, 16) || !aligned(out, 16)) return QDM_ERR_ALIGNMENT;
    return hip_status(down_passes(h, r, m, act, *down, out, stream));
}

int qdm_gemv_linear(const void* x, int32_t m, qdm_dtype act, const qdm_weight* w, const void* bias, void* out,
                    void* stream) {
    if (!x || !out) return QDM_ERR_INVALID_ARG;
    if (x == out || (bias && bias == out)) return QDM_ERR_INVALID_ARG;
    if (!valid_dtype(act)) return QDM_ERR_INVALID_ARG;
    if (int e = check_rows(m)) return e;
    if (int e = check_weight(w)) return e;
    if (int e = check_mx_rows(w, m, act == QDM_F32 ? 4 : 2, act, 2)) return e;
    if (!aligned(x, 16) || !aligned(out, 16) || !aligned(bias, 16)) return QDM_ERR_ALIGNMENT;
    return hip_status(linear_passes(x, m, act, *w, bias, out, stream));
}

int qdm_mlp_decode(const void* x, const void* r, int32_t m, qdm_dtype act,
                   const qdm_weight* gate_up, const qdm_weight* down,
                   void* workspace, size_t workspace_bytes, void* out, void* stream) {
    if (!x || !r || !out) return QDM_ERR_INVALID_ARG;
    if (!valid_dtype(act)) return QDM_ERR_INVALID_ARG;
    if (int e = check_rows(m)) return e;
    if (int e = check_weight(gate_up)) return e;
    if (int e = check_weight(down)) return e;
    if (gate_up->k != down->n || gate_up->n != down->k) return QDM_ERR_INVALID_ARG;
    if (gate_up->bits != down->bits) return QDM_ERR_UNSUPPORTED;
    if (int e = check_mx_rows(gate_up, m, act == QDM_F32 ? 4 : 2, act, 0)) return e;
    if (int e = check_mx_rows(down, m, 4, act, 1)) return e;
    if (!workspace || workspace_bytes < qdm_mlp_workspace_bytes(m, gate_up->n)) return QDM_ERR_WORKSPACE;
    if (workspace == out) return QDM_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(r, 16) || !aligned(out, 16) || !aligned(workspace, 16))
        return QDM_ERR_ALIGNMENT;
    float* h = static_cast<float*>(workspace);
    if (int e = gate_up_passes(x, m, act, *gate_up, h, stream)) return hip_status(e);
    return hip_status(down_passes(h, r, m, act, *down, out, stream));
}

size_t qdm_mlp_rmsnorm_workspace_bytes(int32_t m, int32_t d, int32_t ffn, qdm_dtype act) {
    if (m <= 0 || d <= 0 || ffn <= 0 || !valid_dtype(act)) return 0;
    return round256(static_cast<size_t>(m) * static_cast<size_t>(ffn) * sizeof(float)) +
           2 * round256(static_cast<size_t>(m) * static_cast<size_t>(d) * act_bytes(act));
}

int qdm_mlp_decode_rmsnorm(const void* a, const void* b, const void* norm_w, float eps, int32_t m, qdm_dtype act,
                           const qdm_weight* gate_up, const qdm_weight* down,
                           void* workspace, size_t workspace_bytes, void* s_out, void* out, void* stream) {
    if (!a || !b || !norm_w || !out) return QDM_ERR_INVALID_ARG;
    if (!valid_dtype(act)) return QDM_ERR_INVALID_ARG;
    if (!std::isfinite(eps) || eps < 0.0f) return QDM_ERR_INVALID_ARG;
    if (int e = check_rows(m)) return e;
    if (int e = check_weight(gate_up)) return e;
    if (int e = check_weight(down)) return e;
    if (gate_up->k != down->n || gate_up->n != down->k) return QDM_ERR_INVALID_ARG;
    if (gate_up->bits != down->bits) return QDM_ERR_UNSUPPORTED;
    if (int e = check_mx_rows(gate_up, m, act == QDM_F32 ? 4 : 2, act, 0)) return e;
    if (int e = check_mx_rows(down, m, 4, act, 1)) return e;
    const int32_t d = gate_up->k, ffn = gate_up->n;
    if (!workspace || workspace_bytes < qdm_mlp_rmsnorm_workspace_bytes(m, d, ffn, act)) return QDM_ERR_WORKSPACE;
    if (s_out == out) return QDM_ERR_INVALID_ARG;
    if (workspace == out || workspace == s_out || workspace == a || workspace == b) return QDM_ERR_INVALID_ARG;
    if (!aligned(a, 16) || !aligned(b, 16) || !aligned(norm_w, 16) || !aligned(out, 16) ||
        !aligned(s_out, 16) || !aligned(workspace, 16))
        return QDM_ERR_ALIGNMENT;
    float* h = static_cast<float*>(workspace);
    if (m == 1 && qdm::chain_stream_supported(*gate_up, *down, act))
        return hip_status(qdm::launch_mlp_chain_stream(a, b, norm_w, eps, act, *gate_up, *down, h, s_out, out,
                                                       stream));
    char* base = static_cast<char*>(workspace);
    const size_t hb = round256(static_cast<size_t>(m) * static_cast<size_t>(ffn) * sizeof(float));
    const size_t vb = round256(static_cast<size_t>(m) * static_cast<size_t>(d) * act_bytes(act));
    // 2..16 rows on the matrix-core kernels: the norm rebuilt in every gate/up
    // block, s through the workspace to the down projection's residual (and to
    // s_out by its last kernel)
    if (m > 1 && qdm::mma_stream_gate_up_supported(*gate_up, m, act) &&
        qdm::mma_stream_down_supported(*down, m, act)) {
        void* s_ws = base + hb + vb;
        if (int e = qdm::launch_gate_up_mma_stream_norm(a, b, norm_w, eps, m, act, *gate_up, h, s_ws, stream))
            return hip_status(e);
        return hip_status(qdm::launch_down_mma_stream(h, s_ws, m, act, *down, out, stream, s_out));
    }
    // otherwise the three launches: add + RMSNorm into the workspace (s into
    // s_out when given), then the MLP on n with s as the residual
    void* n_buf = base + hb;
    void* s_buf = s_out ? s_out : static_cast<void*>(base + hb + vb);
    if (int e = qdm::launch_add_rmsnorm(a, b, norm_w, m, d, eps, act, s_buf, n_buf, stream)) return hip_status(e);
    if (int e = gate_up_passes(n_buf, m, act, *gate_up, h, stream)) return hip_status(e);
    return hip_status(down_passes(h, s_buf, m, act, *down, out, stream));
}

int qdm_add_rmsnorm(const void* a, const void* b, const void* w, int32_t rows, int32_t n,
                    float eps, qdm_dtype dtype, void* s_out, void* n_out, void* stream) {
    if (!a || !b || !w || !s_out || !n_out) return QDM_ERR_INVALID_ARG;
    if (rows <= 0 || n <= 0 || !valid_dtype(dtype)) return QDM_ERR_INVALID_ARG;
    if (!std::isfinite(eps) || eps < 0.0f) return QDM_ERR_INVALID_ARG;
    if (s_out == n_out || n_out == a || n_out == b) return QDM_ERR_INVALID_ARG;
    if (!aligned(a, 16) || !aligned(b, 16) || !aligned(w, 16) || !aligned(s_out, 16) || !aligned(n_out, 16))
        return QDM_ERR_ALIGNMENT;
    return hip_status(qdm::launch_add_rmsnorm(a, b, w, rows, n, eps, dtype, s_out, n_out, stream));
}

const char* qdm_status_string(int status) {
    switch (status) {
        case QDM_OK: return "ok";
        case QDM_ERR_INVALID_ARG: return "invalid argument";
        case QDM_ERR_UNSUPPORTED: return "unsupported combination";
        case QDM_ERR_ALIGNMENT: return "misaligned pointer";
        case QDM_ERR_WORKSPACE: return "workspace missing or too small";
        case QDM_ERR_HIP: return "HIP launch failed";
        default: return "unknown status";
    }
}

int qdm_version(void) { return 100; }

}  // extern "C"
