// Host-side plan: sizes, validation, kernel geometry and workspace layout.
// Touches no device, so it runs (and is tested) without a GPU.
#include <new>
#include <string.h>

#include "tp_internal.h"

namespace {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

int default_valu_cols(int32_t batch) {
    // Narrower column tiles keep the split-K partial traffic small; 256
    // columns = 32 lanes x 16 bytes, two full 256-byte row segments per
    // wave instruction.
    (void)batch;
    return 256;
}

}  // namespace

PointGeom tp_geom_for(const tp_plan_s* p, int64_t k_r, int32_t batch, int32_t splits_user) {
    PointGeom g{};
    g.k_r = k_r;
    g.path = batch >= kMfmaMinBatch ? TP_PATH_MFMA : TP_PATH_VALU;
    int64_t gran, max_rows;
    if (g.path == TP_PATH_VALU) {
        g.cols = p->valu_cols ? p->valu_cols : default_valu_cols(batch);
        int lanes_per_row = g.cols / 8;
        gran = (int64_t)kValuWaves * (64 / lanes_per_row);
        max_rows = valu_rows_max(batch, g.cols);
    } else {
        g.cols = kMfmaCols;
        gran = kMfmaKStep;
        max_rows = kMfmaMaxRows;
    }
    g.col_tiles = (int32_t)ceil_div(p->hidden, g.cols);
    // Vector-ALU tiles: two workgroups per CU. Matrix-core tiles: one per CU
    // (measured, 16-64 tokens at H = 4096: 10 % faster than two, and the
    // whole grid stays resident, which the spread split-K fix-up needs).
    int64_t target = p->target_wgs ? p->target_wgs : (g.path == TP_PATH_MFMA ? kTargetCUs : 2 * kTargetCUs);
    int64_t s = splits_user > 0 ? splits_user
                                : (target + g.col_tiles / 2) / g.col_tiles;
    // On the matrix-core path every split writes and re-reads a b x cols fp32
    // partial; keep at least 256 rows per split so that this traffic stays a
    // fraction of the weights' (b <= 64: at most half).
    if (g.path == TP_PATH_MFMA && splits_user <= 0 && s > ceil_div(k_r, 256)) s = ceil_div(k_r, 256);
    if (s < 1) s = 1;
    int64_t s_max = ceil_div(k_r, gran);
    if (s > s_max) s = s_max;
    int64_t rows = round_up(ceil_div(k_r, s), gran);
    if (rows > max_rows) rows = max_rows;
    s = ceil_div(k_r, rows);
    if (s > kMaxCounters) s = kMaxCounters;  // unreachable for supported sizes
    g.rows = (int32_t)rows;
    g.splits = (int32_t)s;
    g.grid = g.col_tiles * g.splits;
    return g;
}

PointGeom tp_point_geom(const tp_plan_s* p, int point) {
    int64_t k = point == TP_POINT_ATTN_OUT ? p->k_attn : p->inter;
    return tp_geom_for(p, k / p->n_ranks, p->batch, p->splits_user[point]);
}

int64_t tp_ws_partials_offset() { return kCounterBytes; }

int64_t tp_ws_partial_buffer_bytes(const tp_plan_s* p) {
    int64_t m = 0;
    for (int pt = 0; pt < 2; ++pt) {
        PointGeom g = tp_point_geom(p, pt);
        int64_t b = g.splits > 1 ? (int64_t)g.splits * p->batch * p->hidden * 4 : 0;
        if (b > m) m = b;
    }
    return round_up(m, 256);
}

// Persistent decode step: 512- or 256-column tiles (1 KB or 512-byte row
// segments) over long row ranges, as few splits as the LDS copy of the
// tile's x slice (kStepXsWords words of bf16 pairs) and the tile length cap
// allow, so most points need no split exchange at all. With splits_user
// the rows follow the same rule as the per-point launches (equal tiles
// give equal bits).
// The persistent step's kind. Measured on row-major weights (H = 5120 and
// 4096, b = 1..8): below 16 tokens the matrix-core step's 128-column tiles
// win where the points are small (an FFN slice of at most 2048 rows, as at
// H = 4096, N = 8) or at b >= 8 with H < 5120; the vector-ALU step's wide
// tiles win elsewhere.
bool tp_step_mfma(const tp_plan_s* p) {
    if (p->batch >= kMfmaMinBatch || p->step_kind == 2) return true;
    if (p->step_kind == 1) return false;
    const int64_t ki_r = p->inter / p->n_ranks;
    return ki_r <= 2048 || (p->batch >= 8 && p->hidden < 5120);
}

PointGeom tp_step_geom(const tp_plan_s* p, int point) {
    PointGeom g{};
    g.k_r = (point == TP_POINT_ATTN_OUT ? p->k_attn : p->inter) / p->n_ranks;
    if (tp_step_mfma(p)) {
        // matrix-core step: 128 columns, 32-row steps, up to 2048 rows
        g.path = TP_PATH_MFMA;
        g.cols = kMfmaCols;
        g.col_tiles = (int32_t)ceil_div(p->hidden, g.cols);
        int64_t max_rows = p->step_rows > 0 ? p->step_rows : 2048;
        max_rows -= max_rows % kMfmaKStep;
        if (max_rows < kMfmaKStep) max_rows = kMfmaKStep;
        const int32_t su = p->splits_user[point];
        int64_t s = su > 0 ? su : ceil_div(g.k_r, max_rows);
        if (s > ceil_div(g.k_r, kMfmaKStep)) s = ceil_div(g.k_r, kMfmaKStep);
        if (s < 1) s = 1;
        int64_t rows = round_up(ceil_div(g.k_r, s), kMfmaKStep);
        if (rows > max_rows) rows = max_rows;
        g.rows = (int32_t)rows;
        g.splits = (int32_t)ceil_div(g.k_r, rows);
        g.grid = g.col_tiles * g.splits;
        return g;
    }
    g.path = TP_PATH_VALU;
    const bool wide = p->hidden / 512 >= kStepWideTiles;
    g.cols = p->valu_cols ? p->valu_cols : (wide ? 512 : 256);
    g.col_tiles = (int32_t)ceil_div(p->hidden, g.cols);
    const int64_t gran = (int64_t)kValuWaves * (64 / (g.cols / 8));
    const int b = p->batch > 0 ? p->batch : 1;
    // x is staged as bf16 pairs: (rows/2 + 16) * b of the kStepXsWords words
    int64_t max_rows = 2 * (kStepXsWords / b - 16);
    const int64_t cap = p->step_rows > 0 ? p->step_rows : (g.cols >= 512 ? 2048 : 1024);
    if (max_rows > cap) max_rows = cap;
    max_rows -= max_rows % gran;
    if (max_rows < gran) max_rows = gran;
    const int32_t su = p->splits_user[point];
    int64_t s = su > 0 ? su : ceil_div(g.k_r, max_rows);
    int64_t s_max = ceil_div(g.k_r, gran);
    if (s > s_max) s = s_max;
    if (s < 1) s = 1;
    int64_t rows = round_up(ceil_div(g.k_r, s), gran);
    if (rows > max_rows) rows = max_rows;
    g.rows = (int32_t)rows;
    g.splits = (int32_t)ceil_div(g.k_r, rows);
    g.grid = g.col_tiles * g.splits;
    return g;
}

int64_t tp_step_partial_buffer_bytes(const tp_plan_s* p) {
    int64_t m = 0;
    for (int pt = 0; pt < 2; ++pt) {
        PointGeom g = tp_step_geom(p, pt);
        int64_t b = g.splits > 1 ? (int64_t)g.splits * p->batch * p->hidden * 4 : 0;
        if (b > m) m = b;
    }
    return round_up(m, 256);
}

static int64_t partial_bytes(const tp_plan_s* p) {
    int64_t m = tp_ws_partial_buffer_bytes(p);
    if (p->batch <= kMfmaMaxBatch) {
        int64_t s = kStepBufs * tp_step_partial_buffer_bytes(p);
        if (s > m) m = s;
    }
    return m;
}

// The column-parallel up projection (tp_gate_up_swiglu) as a persistent
// partials step: both "points" read x [b][H]; point 0 is the gate, point 1
// the up matrix, each [H][I/N]; the output width is I/N; one rank.
// A column-parallel projection from the full hidden state to `cols`
// columns of this rank, as a persistent partials step of its own: K = H,
// output width cols, one rank.
tp_plan_s tp_colproj_plan(const tp_plan_s* p, int64_t cols) {
    tp_plan_s q = *p;
    q.hidden = cols;
    q.k_attn = p->hidden;
    q.inter = p->hidden;
    q.n_ranks = 1;
    q.splits_user[0] = q.splits_user[1] = 0;
    q.decode_mode = 2;
    q.serial_points = 0;
    q.n_experts = q.top_k = q.ep = 0;
    q.moe_inter = 0;
    // The up projection's points are independent (no residual chain), so
    // the matrix-core step takes a column tile's whole K as one tile: no
    // split partials, and no tile waits for a free split set. Kept within
    // the step's 32-bit buffer offsets.
    const int64_t k_all = round_up(q.k_attn, kMfmaKStep);
    if (p->step_rows <= 0 && tp_step_mfma(&q) && (k_all + 1024) * q.hidden * 2 < (int64_t(1) << 31))
        q.step_rows = (int32_t)k_all;
    return q;
}

tp_plan_s tp_swiglu_plan(const tp_plan_s* p) { return tp_colproj_plan(p, p->inter / p->n_ranks); }

bool tp_qkv_ok(const tp_plan_s* p) {
    return p->qkv_cols > 0 && p->qkv_cols % 8 == 0 && p->batch >= 1 && p->batch <= kMfmaMaxBatch;
}

int64_t tp_ws_qkv_offset(const tp_plan_s* p) {
    tp_plan_s q = tp_colproj_plan(p, p->qkv_cols);
    return kCounterBytes + partial_bytes(&q);
}

// Layers per launch of tp_qkv_proj: an even number (two layers are the
// step's two points) whose fp32 sums [layers][b][cols] fit kSwigluSumsBytes,
// at least two, at most "swiglu_layers" when that is set.
int32_t tp_qkv_layers_per_launch(const tp_plan_s* p) {
    const int64_t per_layer = (int64_t)p->batch * p->qkv_cols * 4;
    int64_t n = per_layer > 0 ? kSwigluSumsBytes / per_layer : 2;
    if (p->swiglu_layers > 0 && n > p->swiglu_layers) n = p->swiglu_layers;
    if (n > 4096) n = 4096;
    n -= n % 2;
    return (int32_t)(n < 2 ? 2 : n);
}

bool tp_swiglu_ok(const tp_plan_s* p) {
    return p->inter % p->n_ranks == 0 && (p->inter / p->n_ranks) % 8 == 0 &&
           p->batch >= 1 && p->batch <= kMfmaMaxBatch;
}

int64_t tp_ws_swiglu_offset(const tp_plan_s* p) {
    tp_plan_s q = tp_swiglu_plan(p);
    return kCounterBytes + partial_bytes(&q);
}

// Layers per launch of tp_gate_up_swiglu: as many as keep the fp32 gate and
// up sums ([layers][2][b][I/N]) within kSwigluSumsBytes (at least one).
int32_t tp_swiglu_layers_per_launch(const tp_plan_s* p) {
    const int64_t per_layer = 2 * (int64_t)p->batch * (p->inter / p->n_ranks) * 4;
    int64_t n = per_layer > 0 ? kSwigluSumsBytes / per_layer : 1;
    if (p->swiglu_layers > 0 && n > p->swiglu_layers) n = p->swiglu_layers;
    return (int32_t)(n < 1 ? 1 : n > 4096 ? 4096 : n);
}

int64_t tp_ws_xchg_offset(const tp_plan_s* p) {
    return tp_ws_partials_offset() + partial_bytes(p);
}

int64_t tp_ws_moe_offset(const tp_plan_s* p) {
    return tp_ws_xchg_offset(p) + round_up(tp_xchg_bytes(p), 256);
}

int64_t tp_workspace_bytes(const tp_plan_s* p) {
    int64_t m = tp_ws_moe_offset(p) + round_up(tp_moe_workspace_bytes(p), 256);
    if (tp_swiglu_ok(p)) {
        // the gate and up sums, fp32 [2][b][I/N], after the derived step's buffers
        const int64_t s = tp_ws_swiglu_offset(p) +
                          round_up((int64_t)tp_swiglu_layers_per_launch(p) * 2 * p->batch *
                                       (p->inter / p->n_ranks) * 4,
                                   256);
        if (s > m) m = s;
    }
    if (tp_qkv_ok(p)) {
        const int64_t s = tp_ws_qkv_offset(p) +
                          round_up((int64_t)tp_qkv_layers_per_launch(p) * p->batch * p->qkv_cols * 4, 256);
        if (s > m) m = s;
    }
    return m;
}

int tp_decode_mode(const tp_plan_s* p) {
    if (p->decode_mode) return p->decode_mode;
    return 2;  // the persistent step (vector ALU below 16 tokens, matrix cores from 16)
}

extern "C" {

tp_status tp_plan(int64_t hidden, int64_t inter, int32_t n_ranks, int32_t batch,
                  tp_plan_t* out) {
    if (!out) return TP_ERR_INVALID_ARG;
    *out = nullptr;
    if (hidden < 1 || inter < 1 || n_ranks < 1 || batch < 1) return TP_ERR_INVALID_ARG;
    if (inter % n_ranks || hidden % n_ranks) return TP_ERR_INVALID_ARG;
    if (((int64_t)batch * hidden) % n_ranks) return TP_ERR_INVALID_ARG;
    if (hidden % 8) return TP_ERR_UNSUPPORTED;
    if (batch > kMfmaMaxBatch) return TP_ERR_UNSUPPORTED;
    if (hidden > (int64_t)1 << 24 || inter > (int64_t)1 << 24) return TP_ERR_UNSUPPORTED;
    tp_plan_s* p = new (std::nothrow) tp_plan_s();
    if (!p) return TP_ERR_OOM;
    p->hidden = hidden;
    p->inter = inter;
    p->k_attn = hidden;
    p->n_ranks = n_ranks;
    p->batch = batch;
    *out = p;
    return TP_OK;
}

tp_status tp_plan_set_attn_dim(tp_plan_t p, int64_t k_attn) {
    if (!p || k_attn < 1 || k_attn % p->n_ranks) return TP_ERR_INVALID_ARG;
    if (k_attn > (int64_t)1 << 24) return TP_ERR_UNSUPPORTED;
    p->k_attn = k_attn;
    return TP_OK;
}

tp_status tp_plan_set_qkv_dim(tp_plan_t p, int64_t cols) {
    if (!p || cols < 8 || cols % 8) return TP_ERR_INVALID_ARG;
    if (cols > (int64_t)1 << 24) return TP_ERR_UNSUPPORTED;
    p->qkv_cols = cols;
    return TP_OK;
}

tp_status tp_plan_set_weight_format(tp_plan_t p, int32_t fmt) {
    if (!p || fmt < TP_WEIGHTS_BF16 || fmt > TP_WEIGHTS_MXFP4) return TP_ERR_INVALID_ARG;
    p->weight_format = fmt;
    return TP_OK;
}

tp_status tp_plan_set_moe(tp_plan_t p, int32_t n_experts, int32_t top_k, int32_t ep,
                          int64_t moe_inter, int32_t max_tokens) {
    if (!p || n_experts < 1 || top_k < 1 || ep < 1 || moe_inter < 1 || max_tokens < 1)
        return TP_ERR_INVALID_ARG;
    if (top_k > n_experts || n_experts % ep) return TP_ERR_INVALID_ARG;
    if (top_k > kMoeMaxTopK || max_tokens > kMoeMaxTokens) return TP_ERR_UNSUPPORTED;
    if (moe_inter > (int64_t)1 << 20 || n_experts > 1 << 16) return TP_ERR_UNSUPPORTED;
    p->n_experts = n_experts;
    p->top_k = top_k;
    p->ep = ep;
    p->moe_inter = moe_inter;
    p->max_tokens = max_tokens;
    return TP_OK;
}

tp_status tp_plan_tune(tp_plan_t p, const char* key, int64_t value) {
    if (!p || !key) return TP_ERR_INVALID_ARG;
    if (!strcmp(key, "splits_attn") || !strcmp(key, "splits_ffn")) {
        if (value < 0 || value > 4096) return TP_ERR_INVALID_ARG;
        p->splits_user[key[7] == 'a' ? 0 : 1] = (int32_t)value;
    } else if (!strcmp(key, "valu_cols")) {
        if (value != 0 && value != 128 && value != 256 && value != 512) return TP_ERR_INVALID_ARG;
        p->valu_cols = (int32_t)value;
    } else if (!strcmp(key, "decode_mode")) {
        if (value < 0 || value > 2) return TP_ERR_INVALID_ARG;
        p->decode_mode = (int32_t)value;
    } else if (!strcmp(key, "segment_loads")) {
        if (value != 0 && value != 4 && value != 8) return TP_ERR_INVALID_ARG;
        p->segment_loads = (int32_t)value;
    } else if (!strcmp(key, "moe_variant")) {
        if (value < 0 || value > 7) return TP_ERR_INVALID_ARG;
        p->moe_variant = (int32_t)value;
    } else if (!strcmp(key, "stream_kind")) {
        if (value < 0 || value > 2) return TP_ERR_INVALID_ARG;
        p->stream_kind = (int32_t)value;
    } else if (!strcmp(key, "stream_flat")) {
        if (value < -1 || value > 1) return TP_ERR_INVALID_ARG;
        p->stream_flat = (int32_t)value;
    } else if (!strcmp(key, "stream_wgs")) {
        if (value < 0 || value > kTargetCUs) return TP_ERR_INVALID_ARG;
        p->stream_wgs = (int32_t)value;
    } else if (!strcmp(key, "mfma_acts")) {
        if (value < 0 || value > 2) return TP_ERR_INVALID_ARG;
        p->mfma_acts = (int32_t)value;
    } else if (!strcmp(key, "mfma_sl")) {
        if (value != 0 && value != 2 && value != 3) return TP_ERR_INVALID_ARG;
        p->mfma_sl = (int32_t)value;
    } else if (!strcmp(key, "mfma_oth")) {
        if (value != 0 && value != 2 && value != 4 && value != 8) return TP_ERR_INVALID_ARG;
        p->mfma_oth = (int32_t)value;
    } else if (!strcmp(key, "mfma_flat")) {
        if (value < -1 || value > 1) return TP_ERR_INVALID_ARG;
        p->mfma_flat = (int32_t)value;
    } else if (!strcmp(key, "mfma_wps")) {
        if (value != 0 && value != 8 && value != 12) return TP_ERR_INVALID_ARG;
        p->mfma_wps = (int32_t)value;
    } else if (!strcmp(key, "serial_points")) {
        if (value != 0 && value != 1) return TP_ERR_INVALID_ARG;
        p->serial_points = (int32_t)value;
    } else if (!strcmp(key, "swiglu_layers")) {
        if (value < 0 || value > 4096) return TP_ERR_INVALID_ARG;
        p->swiglu_layers = (int32_t)value;
    } else if (!strcmp(key, "step_kind")) {
        if (value < 0 || value > 2) return TP_ERR_INVALID_ARG;
        p->step_kind = (int32_t)value;
    } else if (!strcmp(key, "xcd_walk")) {
        if (value < -1 || value > 1) return TP_ERR_INVALID_ARG;
        p->xcd_walk = (int32_t)value;
    } else if (!strcmp(key, "step_rows")) {
        if (value < 0 || value > 65536) return TP_ERR_INVALID_ARG;
        p->step_rows = (int32_t)value;
    } else if (!strcmp(key, "target_wgs")) {
        if (value < 0 || value > 65536) return TP_ERR_INVALID_ARG;
        p->target_wgs = (int32_t)value;
    } else {
        return TP_ERR_INVALID_ARG;
    }
    return TP_OK;
}

tp_status tp_plan_info(tp_plan_t p, struct tp_plan_info* o) {
    if (!p || !o) return TP_ERR_INVALID_ARG;
    memset(o, 0, sizeof *o);
    o->hidden = p->hidden;
    o->inter = p->inter;
    o->k_attn = p->k_attn;
    o->n_ranks = p->n_ranks;
    o->batch = p->batch;
    for (int pt = 0; pt < 2; ++pt) {
        PointGeom g = tp_point_geom(p, pt);
        o->k_rank[pt] = g.k_r;
        o->path[pt] = g.path;
        o->splits[pt] = g.splits;
    }
    o->chunk_elems = (int64_t)p->batch * p->hidden / p->n_ranks;
    o->wire_bytes_bf16 = 2 * (int64_t)(p->n_ranks - 1) * o->chunk_elems * 2;
    o->wire_bytes_fp32 = 2 * (int64_t)(p->n_ranks - 1) * o->chunk_elems * 4;
    o->workspace_bytes = tp_workspace_bytes(p);
    o->n_experts = p->n_experts;
    o->top_k = p->top_k;
    o->ep = p->ep;
    o->local_experts = p->ep ? p->n_experts / p->ep : 0;
    o->moe_inter = p->moe_inter;
    o->max_tokens = p->max_tokens;
    o->packed_kind = tp_packed_kind(p);
    MfmaGeom mg;
    const bool mfma = o->packed_kind == 2 && tp_mfma_geometry(p, &mg);
    o->stream_wgs = mfma ? mg.grid : 0;
    o->acts_layout = mfma && !mg.acts_rm ? 1 : 0;
    o->weight_format = p->weight_format;
    for (int pt = 0; pt < 2; ++pt)
        o->packed_layer_bytes[pt] = o->packed_kind == 1   ? tp_stream_packed_bytes(p, pt, 1)
                                    : o->packed_kind == 2 ? tp_mfma_packed_bytes(p, pt, 1)
                                                          : 0;
    return TP_OK;
}

tp_status tp_plan_info_get(tp_plan_t p, struct tp_plan_info* o) { return tp_plan_info(p, o); }

void tp_plan_destroy(tp_plan_t p) { delete p; }

const char* tp_status_str(tp_status s) {
    switch (s) {
        case TP_OK: return "ok";
        case TP_ERR_INVALID_ARG: return "invalid argument";
        case TP_ERR_UNSUPPORTED: return "unsupported configuration";
        case TP_ERR_ALIGNMENT: return "device pointer not 16-byte aligned";
        case TP_ERR_DEVICE: return "HIP device error";
        case TP_ERR_OOM: return "out of host memory";
    }
    return "unknown status";
}

}  // extern "C"
