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

// Does [a, a + an) intersect [b, b + bn)?  (Empty or null ranges never do.)
bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
    if (!a || !b || an == 0 || bn == 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + bn && y < x + an;
}

// Bytes of fp32 split-K partials each projection writes (0: none).  Gate/up
// splits K only on the tiled kernels (more than kPassRows rows); down also on
// the few-row matrix-core kernel, so row passes need the largest pass's share.
size_t gate_up_part_bytes(const qdm_weight& gu, int32_t m, int act) {
    return qdm::prefill_supported(gu, m, act) ? qdm::prefill_partials_bytes(gu, m, true) : 0;
}

size_t down_part_bytes(const qdm_weight& dn, int32_t m, int act) {
    if (qdm::prefill_supported(dn, m, act)) return qdm::prefill_partials_bytes(dn, m, false);
    const int32_t full = std::min(m, kPassRows), rem = m > kPassRows ? m % kPassRows : 0;
    size_t b = 0;
    for (const int32_t mr : {full, rem})
        if (mr >= 2 && qdm::mma_stream_down_supported(dn, mr, act))
            b = std::max(b, qdm::down_mma_stream_partials_bytes(dn, mr));
    return b;
}

// Checks shared by the MLP entry points: rows, dtype, both descriptors and
// their agreement, and the formats' row-count limits.
int check_mlp(int32_t m, int act, const qdm_weight* gate_up, const qdm_weight* down) {
    if (!valid_dtype(act)) return QDM_ERR_INVALID_ARG;
    if (int e = check_rows(m)) return e;
    if (int e = check_weight(gate_up)) return e;
    if (int e = check_weight(down)) return e;
    if (gate_up->k != down->n || gate_up->n != down->k) return QDM_ERR_INVALID_ARG;
    if (gate_up->bits != down->bits) return QDM_ERR_UNSUPPORTED;
    if (int e = check_mx_rows(gate_up, m, act == QDM_F32 ? 4 : 2, act, 0)) return e;
    return check_mx_rows(down, m, 4, act, 1);
}

// The MLP's workspace: h [m][ffn] fp32, then (decode chain only) the
// normalized rows and the sums, then the partials of whichever projection is
// running (the two run one after the other on one stream and share them).
struct MlpLayout {
    size_t h, vec, part, total;
};

MlpLayout mlp_layout(int32_t m, int act, const qdm_weight& gu, const qdm_weight& dn, bool chain) {
    MlpLayout l;
    l.h = round256(static_cast<size_t>(m) * static_cast<size_t>(gu.n) * sizeof(float));
    l.vec = chain ? round256(static_cast<size_t>(m) * static_cast<size_t>(gu.k) * act_bytes(act)) : 0;
    l.part = round256(std::max(gate_up_part_bytes(gu, m, act), down_part_bytes(dn, m, act)));
    l.total = l.h + 2 * l.vec + l.part;
    return l;
}

// The device calls: one tiled launch for more than kPassRows rows where the
// prefill kernels take the weight, otherwise row passes of at most kPassRows
// rows (each pass streams the weights).
int gate_up_passes(const void* x, int32_t m, int act, const qdm_weight& gu, float* h, float* part, void* stream) {
    if (qdm::prefill_supported(gu, m, act)) return qdm::launch_gate_up_prefill(x, m, act, gu, h, part, stream);
    const size_t xe = act_bytes(act);
    for (int32_t m0 = 0; m0 < m; m0 += kPassRows) {
        const int32_t mr = std::min(kPassRows, m - m0);
        if (int e = qdm::launch_gate_up_swiglu(static_cast<const char*>(x) + static_cast<size_t>(m0) * gu.k * xe, mr,
                                               act, gu, h + static_cast<size_t>(m0) * gu.n, stream))
            return e;
    }
    return 0;
}

int down_passes(const float* h, const void* r, int32_t m, int act, const qdm_weight& dn, void* out, float* part,
                void* stream) {
    if (qdm::prefill_supported(dn, m, act)) return qdm::launch_down_prefill(h, r, m, act, dn, out, part, stream);
    const size_t oe = act_bytes(act);
    for (int32_t m0 = 0; m0 < m; m0 += kPassRows) {
        const int32_t mr = std::min(kPassRows, m - m0);
        const size_t ro = static_cast<size_t>(m0) * dn.n * oe;
        if (int e = qdm::launch_down_residual(h + static_cast<size_t>(m0) * dn.k, static_cast<const char*>(r) + ro, mr,
                                              act, dn, static_cast<char*>(out) + ro, part, stream))
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

namespace qdm {

// The MLP's two projections through a workspace laid out by mlp_layout
// (arguments already checked).
int mlp_decode_in(const void* x, const void* r, int32_t m, int act, const qdm_weight& gu, const qdm_weight& dn,
                  void* workspace, void* out, void* stream) {
    const MlpLayout l = mlp_layout(m, act, gu, dn, false);
    float* h = static_cast<float*>(workspace);
    float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + l.h);
    if (int e = gate_up_passes(x, m, act, gu, h, part, stream)) return e;
    return down_passes(h, r, m, act, dn, out, part, stream);
}

}  // namespace qdm

extern "C" {

size_t qdm_gemv_gate_up_workspace_bytes(int32_t m, qdm_dtype act, const qdm_weight* gate_up) {
    if (!valid_dtype(act) || check_rows(m) || check_weight(gate_up)) return 0;
    return round256(gate_up_part_bytes(*gate_up, m, act));
}

size_t qdm_gemv_down_workspace_bytes(int32_t m, qdm_dtype act, const qdm_weight* down) {
    if (!valid_dtype(act) || check_rows(m) || check_weight(down)) return 0;
    return round256(down_part_bytes(*down, m, act));
}

size_t qdm_mlp_workspace_bytes(int32_t m, qdm_dtype act, const qdm_weight* gate_up, const qdm_weight* down) {
    if (check_mlp(m, act, gate_up, down)) return 0;
    return mlp_layout(m, act, *gate_up, *down, false).total;
}

size_t qdm_mlp_rmsnorm_workspace_bytes(int32_t m, qdm_dtype act, const qdm_weight* gate_up, const qdm_weight* down) {
    if (check_mlp(m, act, gate_up, down)) return 0;
    return mlp_layout(m, act, *gate_up, *down, true).total;
}

int qdm_gemv_gate_up_swiglu(const void* x, int32_t m, qdm_dtype act, const qdm_weight* gate_up,
                            void* workspace, size_t workspace_bytes, float* h_out, void* stream) {
    if (!x || !h_out) return QDM_ERR_INVALID_ARG;
    if (!valid_dtype(act)) return QDM_ERR_INVALID_ARG;
    if (int e = check_rows(m)) return e;
    if (int e = check_weight(gate_up)) return e;
    if (int e = check_mx_rows(gate_up, m, act == QDM_F32 ? 4 : 2, act, 0)) return e;
    const size_t xb = static_cast<size_t>(m) * gate_up->k * act_bytes(act);
    const size_t hb = static_cast<size_t>(m) * gate_up->n * sizeof(float);
    const size_t need = gate_up_part_bytes(*gate_up, m, act);
    if (need && (!workspace || workspace_bytes < need)) return QDM_ERR_WORKSPACE;
    if (overlaps(x, xb, h_out, hb)) return QDM_ERR_INVALID_ARG;
    if (need && (overlaps(workspace, workspace_bytes, x, xb) || overlaps(workspace, workspace_bytes, h_out, hb)))
        return QDM_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(h_out, 16) || !aligned(workspace, 16)) return QDM_ERR_ALIGNMENT;
    return hip_status(gate_up_passes(x, m, act, *gate_up, h_out, static_cast<float*>(workspace), stream));
}

int qdm_gemv_down_residual(const float* h, const void* r, int32_t m, qdm_dtype act, const qdm_weight* down,
                           void* workspace, size_t workspace_bytes, void* out, void* stream) {
    if (!h || !r || !out) return QDM_ERR_INVALID_ARG;
    if (!valid_dtype(act)) return QDM_ERR_INVALID_ARG;
    if (int e = check_rows(m)) return e;
    if (int e = check_weight(down)) return e;
    if (int e = check_mx_rows(down, m, 4, act, 1)) return e;
    const size_t hb = static_cast<size_t>(m) * down->k * sizeof(float);
    const size_t ob = static_cast<size_t>(m) * down->n * act_bytes(act);
    const size_t need = down_part_bytes(*down, m, act);
    if (need && (!workspace || workspace_bytes < need)) return QDM_ERR_WORKSPACE;
    if (overlaps(h, hb, out, ob)) return QDM_ERR_INVALID_ARG;
    if (need && (overlaps(workspace, workspace_bytes, h, hb) || overlaps(workspace, workspace_bytes, r, ob) ||
                 overlaps(workspace, workspace_bytes, out, ob)))
        return QDM_ERR_INVALID_ARG;
    if (!aligned(h, 16) || !aligned(r, 16) || !aligned(out, 16) || !aligned(workspace, 16)) return QDM_ERR_ALIGNMENT;
    return hip_status(down_passes(h, r, m, act, *down, out, static_cast<float*>(workspace), stream));
}

int qdm_gemv_linear(const void* x, int32_t m, qdm_dtype act, const qdm_weight* w, const void* bias, void* out,
                    void* stream) {
    if (!x || !out) return QDM_ERR_INVALID_ARG;
    if (!valid_dtype(act)) return QDM_ERR_INVALID_ARG;
    if (int e = check_rows(m)) return e;
    if (int e = check_weight(w)) return e;
    if (int e = check_mx_rows(w, m, act == QDM_F32 ? 4 : 2, act, 2)) return e;
    const size_t ob = static_cast<size_t>(m) * w->n * act_bytes(act);
    if (overlaps(x, static_cast<size_t>(m) * w->k * act_bytes(act), out, ob) ||
        overlaps(bias, static_cast<size_t>(w->n) * act_bytes(act), out, ob))
        return QDM_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(out, 16) || !aligned(bias, 16)) return QDM_ERR_ALIGNMENT;
    return hip_status(linear_passes(x, m, act, *w, bias, out, stream));
}

int qdm_mlp_decode(const void* x, const void* r, int32_t m, qdm_dtype act,
                   const qdm_weight* gate_up, const qdm_weight* down,
                   void* workspace, size_t workspace_bytes, void* out, void* stream) {
    if (!x || !r || !out) return QDM_ERR_INVALID_ARG;
    if (int e = check_mlp(m, act, gate_up, down)) return e;
    const MlpLayout l = mlp_layout(m, act, *gate_up, *down, false);
    if (!workspace || workspace_bytes < l.total) return QDM_ERR_WORKSPACE;
    const size_t vb = static_cast<size_t>(m) * gate_up->k * act_bytes(act);
    if (overlaps(workspace, workspace_bytes, x, vb) || overlaps(workspace, workspace_bytes, r, vb) ||
        overlaps(workspace, workspace_bytes, out, vb))
        return QDM_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(r, 16) || !aligned(out, 16) || !aligned(workspace, 16))
        return QDM_ERR_ALIGNMENT;
    return hip_status(qdm::mlp_decode_in(x, r, m, act, *gate_up, *down, workspace, out, stream));
}

int qdm_mlp_decode_rmsnorm(const void* a, const void* b, const void* norm_w, float eps, int32_t m, qdm_dtype act,
                           const qdm_weight* gate_up, const qdm_weight* down,
                           void* workspace, size_t workspace_bytes, void* s_out, void* out, void* stream) {
    if (!a || !b || !norm_w || !out) return QDM_ERR_INVALID_ARG;
    if (!std::isfinite(eps) || eps < 0.0f) return QDM_ERR_INVALID_ARG;
    if (int e = check_mlp(m, act, gate_up, down)) return e;
    const int32_t d = gate_up->k;
    const MlpLayout l = mlp_layout(m, act, *gate_up, *down, true);
    if (!workspace || workspace_bytes < l.total) return QDM_ERR_WORKSPACE;
    const size_t vb = static_cast<size_t>(m) * d * act_bytes(act);
    if (overlaps(s_out, vb, out, vb)) return QDM_ERR_INVALID_ARG;
    for (const void* p : {a, b, static_cast<const void*>(out), static_cast<const void*>(s_out)})
        if (overlaps(workspace, workspace_bytes, p, vb)) return QDM_ERR_INVALID_ARG;
    if (overlaps(workspace, workspace_bytes, norm_w, static_cast<size_t>(d) * act_bytes(act)))
        return QDM_ERR_INVALID_ARG;
    if (!aligned(a, 16) || !aligned(b, 16) || !aligned(norm_w, 16) || !aligned(out, 16) ||
        !aligned(s_out, 16) || !aligned(workspace, 16))
        return QDM_ERR_ALIGNMENT;
    char* base = static_cast<char*>(workspace);
    float* h = static_cast<float*>(workspace);
    float* part = reinterpret_cast<float*>(base + l.h + 2 * l.vec);
    if (m == 1 && qdm::chain_stream_supported(*gate_up, *down, act))
        return hip_status(qdm::launch_mlp_chain_stream(a, b, norm_w, eps, act, *gate_up, *down, h, s_out, out,
                                                       stream));
    // 2..16 rows on the matrix-core kernels: the norm rebuilt in every gate/up
    // block, s through the workspace to the down projection's residual (and to
    // s_out by its last kernel)
    if (m > 1 && qdm::mma_stream_gate_up_supported(*gate_up, m, act) &&
        qdm::mma_stream_down_supported(*down, m, act)) {
        void* s_ws = base + l.h + l.vec;
        if (int e = qdm::launch_gate_up_mma_stream_norm(a, b, norm_w, eps, m, act, *gate_up, h, s_ws, stream))
            return hip_status(e);
        return hip_status(qdm::launch_down_mma_stream(h, s_ws, m, act, *down, out, part, stream, s_out));
    }
    // otherwise the three launches: add + RMSNorm into the workspace (s into
    // s_out when given), then the MLP on n with s as the residual
    void* n_buf = base + l.h;
    void* s_buf = s_out ? s_out : static_cast<void*>(base + l.h + l.vec);
    if (int e = qdm::launch_add_rmsnorm(a, b, norm_w, m, d, eps, act, s_buf, n_buf, stream)) return hip_status(e);
    if (int e = gate_up_passes(n_buf, m, act, *gate_up, h, part, stream)) return hip_status(e);
    return hip_status(down_passes(h, s_buf, m, act, *down, out, part, stream));
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
        case QDM_ERR_TOO_LARGE: return "call exceeds the fixed scratch of the allocation-free entry point";
        default: return "unknown status";
    }
}

int qdm_version(void) { return 100; }

}  // extern "C"
