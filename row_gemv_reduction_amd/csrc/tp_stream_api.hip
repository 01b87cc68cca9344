// The C entry points of the streamed decode step (tp_decode.h): the choice
// between the vector-ALU stream on pair strips (tp_packed.hip) and the
// matrix-core stream on MFMA tiles (tp_mfma_stream.hip), argument checks,
// and the dispatch to either.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "tp_internal.h"

namespace {
bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Scratch of tp_decode_layers_packed_noalloc, one copy per device, held
// until the process ends: the workspace's fixed region (completion words of
// the serial point order, the matrix-core stream's exchange words and exit
// counter, the error word), then the matrix-core stream's exchange buffers.
constexpr int64_t kScratchFixedBytes = kCounterBytes;       // 256 KiB
constexpr int64_t kScratchXchgBytes = (int64_t)8 << 20;     // 8 MiB
constexpr int64_t kScratchBytes = kScratchFixedBytes + kScratchXchgBytes;
static __device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

// Host code never passes `scratch` itself (its host-side name is not a
// device address): each device's copy is looked up once, with that device
// current, and its address kept here.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
unsigned char* g_scratch[kMaxDevices];

// The current device's scratch, set up on first use: its address, and its
// fixed region cleared by a kernel on `stream` (ahead of the caller's
// launch on the same stream). Null on failure.
unsigned char* device_scratch(void* stream, tp_status* st) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *st = TP_ERR_DEVICE;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            *st = TP_ERR_DEVICE;
            return nullptr;
        }
        *st = tp_fill_u32(static_cast<uint32_t*>(ptr), kScratchFixedBytes / 4, 0u, stream);
        if (*st != TP_OK) return nullptr;
        g_scratch[dev] = static_cast<unsigned char*>(ptr);
    }
    *st = TP_OK;
    return g_scratch[dev];
}
}  // namespace

tp_status tp_scratch_status(int32_t* flags) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TP_ERR_DEVICE;
    unsigned char* base;
    {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        base = g_scratch[dev];
    }
    uint32_t v = 0;
    if (base && hipMemcpy(&v, base + kSyncOffset + 4 * kSyncErr, 4, hipMemcpyDeviceToHost) != hipSuccess)
        return TP_ERR_DEVICE;
    *flags = (int32_t)v;
    return TP_OK;
}

// The plan's packed layout and stream: the knob "stream_kind", else the
// one measured faster where both fit.
int tp_packed_kind(const tp_plan_s* p) {
    StreamGeom sg;
    MfmaGeom mg;
    const bool valu = tp_stream_geometry(p, &sg);
    const bool mfma = tp_mfma_geometry(p, &mg);
    if (p->weight_format != TP_WEIGHTS_BF16) {
        // MX weights, measured on MI355X: where strips stay whole the
        // matrix-core stream is as fast or faster (H4096 MXFP8 b=1: N=4
        // 0.188 against 0.197 ms) except for MXFP4 at one token (N=4 0.172
        // against 0.156) unless a layer's tiles per compute wave fit the
        // stream's 2 SL slots (N=8: 0.118 against 0.132 ms); where strips are
        // cut the vector-ALU stream is faster; beyond 4 tokens the vector-ALU
        // stream's widened vectors spill (N=8 b=8: 0.151 against 0.392 ms).
        if (p->stream_kind == 1) return valu ? 1 : 0;
        if (p->stream_kind == 2) return mfma ? 2 : 0;
        const bool whole = mfma && p->hidden / 16 <= mg.grid;
        const bool small = mfma && (mg.nkb0 + mg.wps - 1) / mg.wps + (mg.nkb1 + mg.wps - 1) / mg.wps <= 2 * mg.sl;
        const bool fp4_one = p->weight_format == TP_WEIGHTS_MXFP4 && p->batch == 1 && !small;
        if (valu && p->batch <= 4 && (!whole || fp4_one)) return 1;
        if (mfma) return 2;
        return valu ? 1 : 0;
    }
    if (p->stream_kind == 1) return valu ? 1 : 0;
    if (p->stream_kind == 2) return mfma ? 2 : 0;
    // Measured on MI355X: the matrix-core stream is the faster one from b = 5
    // on, and at every batch when every 16-column strip stays within one
    // workgroup (H/16 <= its workgroups: H = 4096, b = 1: 0.240 against
    // 0.249 ms at N = 4); where strips are cut between workgroups (H = 5120
    // on 256 CUs) the vector-ALU stream is faster up to b = 4.
    const bool whole = mfma && p->hidden / 16 <= mg.grid;
    if (valu && p->batch <= 4 && !whole) return 1;
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
    if (kind == 0 || p->weight_format != TP_WEIGHTS_BF16) return TP_ERR_UNSUPPORTED;
    if (kind == 2) return tp_pack_tiles(p, point, n_layers, w, w_packed, stream);
    return tp_pack_pairs(p, point, n_layers, w, w_packed, stream);
}

tp_status tp_quantize_mx(tp_plan_t p, int32_t point, int32_t n_layers, const void* w, void* codes,
                         void* scales, void* stream) {
    if (!p || !w || !codes || !scales || n_layers < 0) return TP_ERR_INVALID_ARG;
    if (point != TP_POINT_ATTN_OUT && point != TP_POINT_FFN_DOWN) return TP_ERR_INVALID_ARG;
    if (!aligned16(w) || !aligned16(codes) || !aligned16(scales)) return TP_ERR_ALIGNMENT;
    if (p->weight_format == TP_WEIGHTS_BF16) return TP_ERR_UNSUPPORTED;
    return tp_mx_quantize(p, point, n_layers, w, codes, scales, stream);
}

tp_status tp_pack_weights_mx(tp_plan_t p, int32_t point, int32_t n_layers, const void* codes,
                             const void* scales, void* w_packed, void* stream) {
    if (!p || !codes || !scales || !w_packed || n_layers < 0) return TP_ERR_INVALID_ARG;
    if (point != TP_POINT_ATTN_OUT && point != TP_POINT_FFN_DOWN) return TP_ERR_INVALID_ARG;
    if (!aligned16(codes) || !aligned16(scales) || !aligned16(w_packed)) return TP_ERR_ALIGNMENT;
    if (p->weight_format == TP_WEIGHTS_BF16) return TP_ERR_UNSUPPORTED;
    const int kind = tp_packed_kind(p);
    if (kind == 2) return tp_mx_pack_tiles(p, point, n_layers, codes, scales, w_packed, stream);
    if (kind != 1) return TP_ERR_UNSUPPORTED;
    return tp_mx_pack(p, point, n_layers, codes, scales, w_packed, stream);
}

tp_status tp_pack_activations(tp_plan_t p, int32_t n_layers, const void* x_attn, const void* x_ffn,
                              void* xa_packed, void* xf_packed, void* stream) {
    if (!p || !x_attn || !x_ffn || !xa_packed || !xf_packed || n_layers < 0) return TP_ERR_INVALID_ARG;
    if (!aligned16(x_attn) || !aligned16(x_ffn) || !aligned16(xa_packed) || !aligned16(xf_packed))
        return TP_ERR_ALIGNMENT;
    if (x_attn == xa_packed || x_ffn == xf_packed || xa_packed == xf_packed) return TP_ERR_INVALID_ARG;
    const int kind = tp_packed_kind(p);
    if (kind == 0) return TP_ERR_UNSUPPORTED;
    MfmaGeom mg;
    if (kind == 2 && tp_mfma_geometry(p, &mg) && !mg.acts_rm)
        return tp_pack_acts(p, n_layers, x_attn, x_ffn, xa_packed, xf_packed, stream);
    // the vector-ALU stream, and the matrix-core stream for a few tokens,
    // read row-major activations: the same bytes
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

tp_status tp_decode_layers_packed_noalloc(tp_plan_t p, int32_t n_layers, int32_t rank,
                                          const void* x_attn, const void* w_o_packed,
                                          const void* x_ffn, const void* w_down_packed,
                                          float* slots, float* hidden, void* stream) {
    if (!p || !x_attn || !w_o_packed || !x_ffn || !w_down_packed || !slots || !hidden)
        return TP_ERR_INVALID_ARG;
    if (n_layers < 0 || rank < 0 || rank >= p->n_ranks) return TP_ERR_INVALID_ARG;
    if (!aligned16(x_attn) || !aligned16(w_o_packed) || !aligned16(x_ffn) ||
        !aligned16(w_down_packed) || !aligned16(slots) || !aligned16(hidden))
        return TP_ERR_ALIGNMENT;
    const int kind = tp_packed_kind(p);
    if (kind == 0) return TP_ERR_UNSUPPORTED;
    if (kind == 2 && (p->serial_points || tp_xchg_bytes(p) > kScratchXchgBytes)) return TP_ERR_UNSUPPORTED;
    tp_status st;
    unsigned char* base = device_scratch(stream, &st);
    if (!base) return st;
    if (n_layers == 0) return TP_OK;
    // the error word reports this call: clear it first (a kernel, in stream order)
    st = tp_fill_u32(reinterpret_cast<uint32_t*>(base + kSyncOffset) + kSyncErr, 1, 0u, stream);
    if (st != TP_OK) return st;
    if (kind == 2)
        return tp_decode_mfma_stream_at(p, n_layers, rank, x_attn, w_o_packed, x_ffn, w_down_packed,
                                        slots, hidden, base,
                                        reinterpret_cast<float*>(base + kScratchFixedBytes), stream);
    return tp_decode_stream(p, n_layers, rank, x_attn, w_o_packed, x_ffn, w_down_packed, slots,
                            hidden, nullptr, base, stream);
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
