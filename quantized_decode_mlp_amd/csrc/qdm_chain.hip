// The decode chain across the layer boundary for one row: the residual add +
// RMSNorm that feeds the MLP is folded into the MLP's two launches.
//
// Pages: meTile docs, "Compute-Graph Fusion", opening GraphBuilder example
// (summed = values + residual, normalized = rms_norm(summed, weight, eps),
// both kept) and section "Automatic Gated Epilogues" (the gated MLP on the
// normalized row, the residual added inside the one-row down projection);
// "MLX-LM Backend", section "Dispatch Policy" (RMSNorm accumulating in FP32).
//
// The gate/up launch's every block rebuilds n = rmsnorm(a + b) * w in LDS
// from a, b and w (3 x d elements, L2-resident after the first blocks) in
// place of copying x; the down launch takes s = a + b as its residual and
// stores it.  Rounding and summation order match the standalone add + RMSNorm
// kernel, so the results are bitwise those of that kernel followed by the
// MLP, with one launch and the n/s round trip through HBM saved.
#include "qdm_stream.h"

namespace qdm {
namespace {

template <int XDT>
int run_chain(const ChainArgs& ch, const qdm_weight& gu, const qdm_weight& dn, float* h, void* out, hipStream_t s) {
    const int d = gu.k, ffn = gu.n;
    StreamSplit sg, sd;
    if (!stream_split(gu.bits, d, x_bytes<XDT>(), sg) || !stream_split(dn.bits, ffn, 4, sd))
        return static_cast<int>(hipErrorInvalidValue);
    sg.nr = stream_rows_per_group(sg, true);
    stream_split_gate_up(gu.bits, sg);
    sd.nr = stream_rows_per_group(sd, false);
    stream_split_down(dn.bits, ffn, sd);
    int e;
    switch (gu.bits) {
        case 8: e = run_stream<8, XDT, DT_F32, true, kEpiChain>(gu, nullptr, nullptr, h, ffn, d, sg, s, ch); break;
        case 4: e = run_stream<4, XDT, DT_F32, true, kEpiChain>(gu, nullptr, nullptr, h, ffn, d, sg, s, ch); break;
        case QDM_U8_SB16: e = run_stream<QDM_U8_SB16, XDT, DT_F32, true, kEpiChain>(gu, nullptr, nullptr, h, ffn, d, sg, s, ch); break;
        case QDM_U4_SB16: e = run_stream<QDM_U4_SB16, XDT, DT_F32, true, kEpiChain>(gu, nullptr, nullptr, h, ffn, d, sg, s, ch); break;
        case QDM_MXFP8: e = run_stream<QDM_MXFP8, XDT, DT_F32, true, kEpiChain>(gu, nullptr, nullptr, h, ffn, d, sg, s, ch); break;
        case QDM_MXFP4: e = run_stream<QDM_MXFP4, XDT, DT_F32, true, kEpiChain>(gu, nullptr, nullptr, h, ffn, d, sg, s, ch); break;
        default: e = run_stream<16, XDT, DT_F32, true, kEpiChain>(gu, nullptr, nullptr, h, ffn, d, sg, s, ch); break;
    }
    if (e) return e;
    switch (dn.bits) {
        case 8: return run_stream<8, DT_F32, XDT, false, kEpiChain>(dn, h, nullptr, out, d, ffn, sd, s, ch);
        case 4: return run_stream<4, DT_F32, XDT, false, kEpiChain>(dn, h, nullptr, out, d, ffn, sd, s, ch);
        case QDM_U8_SB16: return run_stream<QDM_U8_SB16, DT_F32, XDT, false, kEpiChain>(dn, h, nullptr, out, d, ffn, sd, s, ch);
        case QDM_U4_SB16: return run_stream<QDM_U4_SB16, DT_F32, XDT, false, kEpiChain>(dn, h, nullptr, out, d, ffn, sd, s, ch);
        case QDM_MXFP8: return run_stream<QDM_MXFP8, DT_F32, XDT, false, kEpiChain>(dn, h, nullptr, out, d, ffn, sd, s, ch);
        case QDM_MXFP4: return run_stream<QDM_MXFP4, DT_F32, XDT, false, kEpiChain>(dn, h, nullptr, out, d, ffn, sd, s, ch);
        default: return run_stream<16, DT_F32, XDT, false, kEpiChain>(dn, h, nullptr, out, d, ffn, sd, s, ch);
    }
}

}  // namespace

bool chain_stream_supported(const qdm_weight& gu, const qdm_weight& dn, int act) {
    StreamSplit sp;
    return stream_split(gu.bits, gu.k, act == DT_F32 ? 4 : 2, sp) && stream_split(dn.bits, dn.k, 4, sp);
}

int launch_mlp_chain_stream(const void* a, const void* b, const void* w, float eps, int act, const qdm_weight& gu,
                            const qdm_weight& dn, float* h, void* s_out, void* out, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    const ChainArgs ch{a, b, w, s_out, eps};
    switch (act) {
        case DT_F32: return run_chain<DT_F32>(ch, gu, dn, h, out, s);
        case DT_F16: return run_chain<DT_F16>(ch, gu, dn, h, out, s);
        default: return run_chain<DT_BF16>(ch, gu, dn, h, out, s);
    }
}

}  // namespace qdm
