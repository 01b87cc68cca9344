// The C entry points of the streamed decode step (tp_decode.h): the choice
// between the vector-ALU stream on pair strips (tp_packed.hip) and the
// matrix-core stream on MFMA tiles (tp_mfma_stream.hip), argument checks,
// and the dispatch to either.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tp_internal.h"

namespace {
bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }
}  // namespace

// The plan's packed layout and stream: the knob "stream_kind", else the
// one measured faster where both fit.
int tp_packed_kind(const tp_plan_s* p) {
    StreamGeom sg;
    MfmaGeom mg;
    const bool valu = tp_stream_geometry(p, &sg);
    const bool mfma = tp_mfma_geometry(p, &mg);
    if (p->stream_kind == 1) return valu ? 1 : 0;
    if (p->stream_kind == 2) return mfma ? 2 : 0;
    // Measured on MI355X: the matrix-core stream is the faster one from b = 5
    // on, and from b = 2 (or b = 1 with short FFN slices, K_r < 2048) when
    // every 16-column strip stays within one workgroup (H/16 <= its
    // workgroups); where strips are cut between workgroups (H = 5120 on 256
    // CUs) the vector-ALU stream is faster up to b = 4.
    const bool whole = mfma && p->hidden / 16 <= mg.grid;
    const bool short_k = p->inter / p->n_ranks < 2048;
    if (valu && p->batch <= 4 && !(whole && (p->batch >= 2 || short_k))) return 1;
    if (mfma) return 2;
    return valu ? 1 : 0;
}

extern "C" {

tp_status tp_pack_weights(tp_plan_t p, int32_t point, int32_t n_layers, const void* w,
                          void* w_packed, void* stream) {
    if (!p || !w || !w_packed || n_layers < 0) return TP_ERR_INVALID_ARG;
    if (point != TP_POINT_ATTN_OUT && point != TP_POINT_FFN_DOWN) return TP_ERR_INVALID_ARG;
    if (!aligned16(w) || !aligned16(w_packed)) return TP_ERR_ALIGNMENT;
    if (w == w_packed) return TP_ERR_INVALID_ARG;
    const int kind = tp_packed_kind(p);
    if (kind == 0) return TP_ERR_UNSUPPORTED;
    if (kind == 2) return tp_pack_tiles(p, point, n_layers, w, w_packed, stream);
    return tp_pack_pairs(p, point, n_layers, w, w_packed, stream);
}

tp_status tp_pack_activations(tp_plan_t p, int32_t n_layers, const void* x_attn, const void* x_ffn,
                              void* xa_packed, void* xf_packed, void* stream) {
    if (!p || !x_attn || !x_ffn || !xa_packed || !xf_packed || n_layers < 0) return TP_ERR_INVALID_ARG;
    if (!aligned16(x_attn) || !aligned16(x_ffn) || !aligned16(xa_packed) || !aligned16(xf_packed))
        return TP_ERR_ALIGNMENT;
    if (x_attn == xa_packed || x_ffn == xf_packed || xa_packed == xf_packed) return TP_ERR_INVALID_ARG;
    const int kind = tp_packed_kind(p);
    if (kind == 0) return TP_ERR_UNSUPPORTED;
    if (kind == 2) return tp_pack_acts(p, n_layers, x_attn, x_ffn, xa_packed, xf_packed, stream);
    // the vector-ALU stream reads row-major activations: the same bytes
    const int64_t per = (int64_t)n_layers * p->batch * 2;
    if (hipMemcpyAsync(xa_packed, x_attn, per * (p->k_attn / p->n_ranks), hipMemcpyDeviceToDevice,
                       (hipStream_t)stream) != hipSuccess ||
        hipMemcpyAsync(xf_packed, x_ffn, per * (p->inter / p->n_ranks), hipMemcpyDeviceToDevice,
                       (hipStream_t)stream) != hipSuccess)
        return TP_ERR_DEVICE;
    return TP_OK;
}

tp_status tp_decode_layers_packed(tp_plan_t p, int32_t n_layers, int32_t rank, const void* x_attn,
                                  const void* w_o_packed, const void* x_ffn,
                                  const void* w_down_packed, float* slots, float* hidden,
                                  void* ws, void* stream) {
    if (!p || !x_attn || !w_o_packed || !x_ffn || !w_down_packed || !slots || !hidden || !ws)
        return TP_ERR_INVALID_ARG;
    if (n_layers < 0 || rank < 0 || rank >= p->n_ranks) return TP_ERR_INVALID_ARG;
    if (!aligned16(x_attn) || !aligned16(w_o_packed) || !aligned16(x_ffn) ||
        !aligned16(w_down_packed) || !aligned16(slots) || !aligned16(hidden) || !aligned16(ws))
        return TP_ERR_ALIGNMENT;
    const int kind = tp_packed_kind(p);
    if (kind == 0) return TP_ERR_UNSUPPORTED;
    if (kind == 2) {
        if (p->serial_points) return TP_ERR_UNSUPPORTED;  // the serial order: vector-ALU stream only
        return tp_decode_mfma_stream(p, n_layers, rank, x_attn, w_o_packed, x_ffn, w_down_packed,
                                     slots, hidden, ws, stream);
    }
    return tp_decode_stream(p, n_layers, rank, x_attn, w_o_packed, x_ffn, w_down_packed, slots,
                            hidden, nullptr, ws, stream);
}

tp_status tp_rowparallel_partials_packed(tp_plan_t p, int32_t n_layers, const void* x_attn,
                                         const void* w_o_packed, const void* x_ffn,
                                         const void* w_down_packed, float* out, void* ws,
                                         void* stream) {
    if (!p || n_layers < 0) return TP_ERR_INVALID_ARG;
    if (n_layers == 0) return TP_OK;  // nothing is read or written
    if (!x_attn || !w_o_packed || !x_ffn || !w_down_packed || !out || !ws) return TP_ERR_INVALID_ARG;
    if (!aligned16(x_attn) || !aligned16(w_o_packed) || !aligned16(x_ffn) ||
        !aligned16(w_down_packed) || !aligned16(out) || !aligned16(ws))
        return TP_ERR_ALIGNMENT;
    if (tp_packed_kind(p) != 1) return TP_ERR_UNSUPPORTED;
    return tp_decode_stream(p, n_layers, 0, x_attn, w_o_packed, x_ffn, w_down_packed, nullptr,
                            nullptr, out, ws, stream);
}

}  // extern "C"
