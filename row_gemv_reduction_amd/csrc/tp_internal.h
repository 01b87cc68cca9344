// Internal plan representation shared by the host plan code and the HIP
// launchers. Not part of the public interface.
#pragma once

#include <stdint.h>

#include "../../include/tp_decode.h"

// Target device: MI355X, 256 compute units in 8 XCDs of 32.
constexpr int kTargetCUs = 256;
constexpr int kXCDs = 8;

// Workspace layout: [column-tile counters | step sync words | split stream counters]
//                   [split-K partials][split stream slice partials][MoE scratch]
constexpr int64_t kCounterBytes = 256 * 1024;
constexpr int kCounterStride = 16;            // one counter per 64-byte line
constexpr int kMaxCounters = 1024;            // column-tile arrival counters (64 KiB)
constexpr int64_t kSyncOffset = 64 * 1024;    // step sync words: done, exit, error
constexpr int kSyncDone = 0, kSyncExit = 16, kSyncErr = 32;
constexpr int kSyncMoeRoute = 48;  // MoE layer share: routing workgroups done
// Persistent row-major decode step (decode_step): points completed per
// column tile (stride kCounterStride), the x slice of a tile staged in LDS,
// the split buffer / arrival counter sets (points in flight), and the
// default tiles: 512 columns by up to 2048 rows where that still gives at
// least kStepWideTiles column tiles, else 256 by up to 1024 (measured at
// H = 5120 and 4096, b = 1 and 8).
constexpr int64_t kFixedOffset = 192 * 1024;
constexpr int kStepXsWords = 8192;
constexpr int kStepBufs = 8;
constexpr int kStepWideTiles = 10;
// matrix-core decode step (b >= 16): waves per workgroup
constexpr int kStepMfmaWaves = 8;
// VALU GEMV geometry limits
constexpr int kValuWaves = 4;        // waves per workgroup
constexpr int kValuMaxRows = 512;    // rows of x staged in LDS per workgroup
constexpr int kValuXsFloats = 4096;  // LDS floats for the staged x slice
constexpr int kValuMaxBatch = 15;
constexpr int kValuLoadsPerLane = 24;  // a tile's weights are loaded into registers at once

// Rows of one VALU split: every lane holds all of its rows' 16-byte weight
// vectors in registers (kValuLoadsPerLane), and x[rows][B] fits the LDS
// staging buffer.
constexpr int valu_rows_max(int batch, int cols) {
    int r = kValuLoadsPerLane * kValuWaves * (64 / (cols / 8));
    int x = kValuXsFloats / batch;
    r = r > x ? x : r;
    r = r > kValuMaxRows ? kValuMaxRows : r;
    return r - r % 16;
}
constexpr int kMfmaMinBatch = 16;
constexpr int kMfmaMaxBatch = 64;
// The matrix-core stream reads row-major activations up to this batch (automatic choice).
constexpr int kMfmaRowMajorActsMax = 4;
constexpr int kMfmaCols = 128;       // columns per MFMA workgroup
constexpr int kMfmaWaves = 4;
constexpr int kMfmaKStep = 32;       // k rows per MFMA step
constexpr int kMfmaMaxRows = 1024;   // rows per MFMA split (multiple of 128)

// Streamed decode step on pair-strip packed weights
constexpr int kStripMaxBatch = 8;
constexpr int kStreamMaxLdsBytes = 150 * 1024;  // x buffers (dynamic LDS)
// completion words of the serial point order (byte offset in the workspace)
constexpr int64_t kStreamFlagOffset = kSyncOffset + 16 * 1024;

// MFMA stream: strips cut between two workgroups hand a partial over through
// device memory: kXchgRing buffers per kind of point and strip, and per kind
// and strip a "published" and an "acknowledged" word, then the exit counter
constexpr int kXchgRing = 4;
constexpr int kXchgMaxStrips = 512;
constexpr int64_t kXchgFlagOffset = 128 * 1024;
constexpr int64_t kXchgExitOffset = kXchgFlagOffset + 4 * kXchgMaxStrips * 4;

// MoE
constexpr int kMoeMaxTopK = 32;
constexpr int kMoeMaxTokens = 4096;

struct tp_plan_s {
    int64_t hidden = 0, inter = 0, k_attn = 0;
    int32_t n_ranks = 0, batch = 0;
    // tuning (0 = automatic)
    int32_t splits_user[2] = {0, 0};
    int32_t valu_cols = 0;
    int32_t decode_mode = 0;
    int32_t target_wgs = 0;
    int32_t segment_loads = 0;  // 16-byte loads per lane per bank of the streamed step (0 = 4)
    int32_t serial_points = 0;  // decode step: point j+1 waits for all of point j
    int32_t stream_kind = 0;    // 0 = automatic, 1 = pair strips (VALU), 2 = MFMA tiles
    int32_t stream_flat = -1;   // pair-strip stream, dataflow order: banks across points (1) or a point per bank (0); -1 = automatic
    int32_t moe_variant = 0;    // expert kernel variant (0 = default)
    int32_t stream_wgs = 0;     // MFMA stream: workgroups (0 = one per CU, at most H/16)
    int32_t mfma_acts = 0;      // MFMA stream: activations 0 = automatic, 1 = row-major, 2 = A-operand order
    int32_t mfma_sl = 0;        // MFMA stream, up to 32 tokens: tiles per register bank (0 = automatic)
    int32_t mfma_wps = 0;       // MFMA stream, up to 32 tokens: compute waves (0 = automatic)
    int32_t mfma_oth = 0;       // MFMA stream: other ranks' values staged in 2, 4 or 8 buffers (0 = automatic)
    int32_t mfma_flat = -1;     // MFMA stream, up to 32 tokens: register slots across segments (1) or banks per segment (0); -1 = automatic
    int32_t step_rows = 0;      // persistent step: most rows per tile (0 = automatic)
    int32_t step_kind = 0;      // persistent step: 0 = automatic, 1 = vector ALU (b < 16), 2 = matrix cores
    int32_t swiglu_layers = 0;  // tp_gate_up_swiglu: most layers per launch (0 = automatic)
    int32_t xcd_walk = -1;      // persistent step: 1 = XCD-contiguous tile walk, 0 = off, -1 = automatic
    int64_t qkv_cols = 0;       // tp_qkv_proj: the rank's Q, K and V columns (0 = not set)
    int32_t weight_format = 0;  // packed step's weights: TP_WEIGHTS_BF16, _MXFP8 or _MXFP4
    // MoE
    int32_t n_experts = 0, top_k = 0, ep = 0;
    int64_t moe_inter = 0;
    int32_t max_tokens = 0;
};

// Geometry of one point's projection launch, derived from the plan.
struct PointGeom {
    int64_t k_r;        // rows of the rank's slice
    int32_t path;       // tp_path
    int32_t cols;       // columns per workgroup tile
    int32_t col_tiles;  // ceil(H / cols)
    int32_t splits;     // split-K factor S
    int32_t rows;       // rows per split (last split may be shorter)
    int32_t grid;       // col_tiles * splits
};

PointGeom tp_point_geom(const tp_plan_s* p, int point);
PointGeom tp_geom_for(const tp_plan_s* p, int64_t k_r, int32_t batch, int32_t splits_user);
int64_t tp_workspace_bytes(const tp_plan_s* p);
int64_t tp_ws_partials_offset();
// Bytes of one split-K partial buffer of the per-point launches.
int64_t tp_ws_partial_buffer_bytes(const tp_plan_s* p);
// Geometry of the persistent decode step's tiles (long row ranges, streamed)
// and the bytes of one of its kStepBufs split buffers (the workspace holds
// all of them when the step can run, batch < 16).
PointGeom tp_step_geom(const tp_plan_s* p, int point);
bool tp_step_mfma(const tp_plan_s* p);  // the persistent step runs on the matrix cores
int64_t tp_step_partial_buffer_bytes(const tp_plan_s* p);
int64_t tp_ws_moe_offset(const tp_plan_s* p);
int tp_decode_mode(const tp_plan_s* p);

// Microscaled weights: 32 rows of a column share one 8-bit scale.
constexpr int kMxBlock = 32;
// Rows of one column in a 16-byte vector of the vector-ALU stream's
// layout: 2 bf16 pairs, 4 FP8 codes, 8 FP4 codes.
constexpr int stream_rows_per_vec(int weight_format) {
    return weight_format == TP_WEIGHTS_MXFP8 ? 4 : weight_format == TP_WEIGHTS_MXFP4 ? 8 : 2;
}

// Geometry of the streamed decode step (tp_packed.hip).
struct StreamGeom {
    int32_t grid, block;  // workgroups (strip owners) and threads per workgroup
    int32_t ns, wps, sl;  // strips per workgroup, waves per strip, loads per bank
    int32_t kh0, kh1;     // row pairs per point kind (x is staged as bf16 pairs)
    int32_t kv0, kv1;     // 16-byte weight vectors per strip per point kind
    int32_t bpw0, bpw1;   // 1 KB row blocks per compute wave per point kind
    int32_t xoff1, xdwords, lds_bytes;
};
// Bytes of one point's packed weight stack on the vector-ALU stream
// (codes, then for MX weights the scales).
int64_t tp_stream_packed_bytes(const tp_plan_s* p, int point, int64_t n_layers);
bool tp_stream_geometry(const tp_plan_s* p, StreamGeom* g);
tp_status tp_pack_pairs(const tp_plan_s* p, int point, int n_layers, const void* w, void* w_packed,
                        void* stream);
// MX weights: bf16 [L][K][H] -> interchange codes and scales; interchange ->
// the stream's packed layout.
tp_status tp_mx_quantize(const tp_plan_s* p, int point, int n_layers, const void* w, void* codes,
                         void* scales, void* stream);
tp_status tp_mx_pack(const tp_plan_s* p, int point, int n_layers, const void* codes, const void* scales,
                     void* w_packed, void* stream);
// (partials != nullptr: the partials only, into partials [L][2][b][H]; slots
// and hidden unused)
tp_status tp_decode_stream(const tp_plan_s* p, int32_t n_layers, int32_t rank, const void* x_attn,
                           const void* w_o_packed, const void* x_ffn, const void* w_down_packed,
                           float* slots, float* hidden, float* partials, void* ws, void* stream);

// Geometry of the MFMA streamed decode step (tp_mfma_stream.hip).
struct MfmaGeom {
    int32_t grid, block, wps, bt;
    int32_t sl;                    // tiles per register bank
    int32_t acts_rm;               // activations read row-major [L][b][K_r] (else A-operand order)
    int32_t flat;                  // compute waves' register slots run across segments
    int32_t wf;                    // weight format (tp_weight_format)
    int32_t tile_bytes;            // bytes of one packed tile (64 rows x 16 columns)
    int32_t nkb0, nkb1;
    int32_t oth_strip, own_max;    // other ranks' values per owned strip (floats); owned strips
    int32_t oth_lg;                // points staged ahead: 1 << oth_lg buffers
    int32_t lds_bytes;             // dynamic LDS
};
bool tp_mfma_geometry(const tp_plan_s* p, MfmaGeom* g);
int64_t tp_xchg_bytes(const tp_plan_s* p);  // exchange buffers of the MFMA stream
// MX tiles of the matrix-core stream (tp_pack_weights_mx at packed_kind 2)
// and the bytes of a point's packed stack (any weight format).
tp_status tp_mx_pack_tiles(const tp_plan_s* p, int point, int n_layers, const void* codes,
                           const void* scales, void* w_packed, void* stream);
int64_t tp_mfma_packed_bytes(const tp_plan_s* p, int point, int64_t n_layers);
// The column-parallel up projection: its derived plan (a persistent
// partials step with the gate and up matrices as the two points), whether
// the plan supports it, and where its fp32 sums sit in the workspace.
tp_plan_s tp_colproj_plan(const tp_plan_s* p, int64_t cols);
tp_plan_s tp_swiglu_plan(const tp_plan_s* p);
bool tp_swiglu_ok(const tp_plan_s* p);
int64_t tp_ws_swiglu_offset(const tp_plan_s* p);
constexpr int64_t kSwigluSumsBytes = 32 << 20;  // fp32 gate and up sums per launch
int32_t tp_swiglu_layers_per_launch(const tp_plan_s* p);
// The column-parallel QKV projection: the same derived step with two
// consecutive layers as its two points, and its fp32 sums.
bool tp_qkv_ok(const tp_plan_s* p);
int64_t tp_ws_qkv_offset(const tp_plan_s* p);
int32_t tp_qkv_layers_per_launch(const tp_plan_s* p);
int64_t tp_ws_xchg_offset(const tp_plan_s* p);
tp_status tp_pack_tiles(const tp_plan_s* p, int point, int n_layers, const void* w, void* w_packed,
                        void* stream);
// The MFMA tile layout of n_mats row-major bf16 matrices [K][H] (H a
// multiple of 16): T[m][s][kb][h][l][i] = W[m][64kb + 16(l/16) + 8h + i][16s + l%16],
// rows past K zero; 2 KB per tile.
tp_status tp_pack_tile_stack(int64_t n_mats, int64_t K, int64_t H, const void* w, void* w_packed,
                             void* stream);
tp_status tp_pack_acts(const tp_plan_s* p, int n_layers, const void* x_attn, const void* x_ffn,
                       void* xa_packed, void* xf_packed, void* stream);
tp_status tp_decode_mfma_stream(const tp_plan_s* p, int32_t n_layers, int32_t rank,
                                const void* x_attn, const void* w_o_tiles, const void* x_ffn,
                                const void* w_down_tiles, float* slots, float* hidden, void* ws,
                                void* stream);
// The same with the exchange buffers (tp_xchg_bytes(p) bytes) at `xpart`
// instead of at the workspace's exchange offset; `ws` still holds the
// fixed region (exchange words, exit counter, error word).
tp_status tp_decode_mfma_stream_at(const tp_plan_s* p, int32_t n_layers, int32_t rank,
                                   const void* x_attn, const void* w_o_tiles, const void* x_ffn,
                                   const void* w_down_tiles, float* slots, float* hidden, void* ws,
                                   float* xpart, void* stream);
// Fill n words at p with v (a kernel: capturable into a HIP graph).
tp_status tp_fill_u32(uint32_t* p, int64_t n, uint32_t v, void* stream);
// The error word of the no-alloc entry point's scratch on the current
// device (0 if that scratch was never used there).
tp_status tp_scratch_status(int32_t* flags);
// Packed layout (and streamed kernel) the plan uses: 0 none, 1 pair strips, 2 MFMA tiles.
int tp_packed_kind(const tp_plan_s* p);
int64_t tp_moe_workspace_bytes(const tp_plan_s* p);  // pair table and expert projections

// After a kernel launch: TP_ERR_DEVICE if the launch failed; with the debug
// mode on (tp_set_debug_sync), also waits for the stream (unless it is being
// captured) and reports an error the kernels raised.
tp_status tp_launch_status(void* stream);
