/*
 * tp_decode.h — one tensor-parallel rank's share of an LLM decode step on
 * AMD Instinct MI355X (gfx950).
 *
 * Under tensor parallelism every weight matrix W[K, H] of a row-parallel
 * projection is split by rows over N ranks; rank r holds rows K_r and
 * computes a partial p_r = x[:, K_r] . W[K_r, :], and the N partials are
 * summed (an all-reduce) before the residual stream continues. Each layer
 * has two such reconciliation points: after the sequence mixer's output
 * projection and after the FFN down projection ("Interconnects e clusters",
 * llmdeepdive.com lesson 9.9, section 01 · Conceito). The all-reduce is a
 * ring: reduce-scatter then all-gather, 2(N-1)/N of the payload on each
 * rank's wire (same section).
 *
 * On one GPU the N ranks are emulated as N fp32 partial buffers in device
 * memory; the reduction sums them in the fixed order a ring would, so the
 * result is bit-for-bit what a ring all-reduce with the same chunk
 * convention produces.
 *
 * Conventions for every entry point:
 *  - Pointers named x, w, u, partials, residual, out, slots, hidden,
 *    workspace are DEVICE pointers owned by the caller. The library keeps
 *    none of them after the call returns and allocates no device memory.
 *  - bf16 arrays are passed as `const void*` (IEEE bfloat16, 2 bytes each).
 *  - Every device pointer must be 16-byte aligned (TP_ERR_ALIGNMENT).
 *  - `stream` is a hipStream_t (NULL means the default stream). All device
 *    work is enqueued on it asynchronously; results are valid once the
 *    stream has been synchronised.
 *  - Arguments are validated before anything is enqueued; on any error
 *    nothing is enqueued. A failed launch returns TP_ERR_DEVICE.
 *  - No C++ exception crosses this interface.
 *  - A plan is a host object. After its setters have run it is read-only
 *    and may be shared by threads and streams. Calls that share one
 *    workspace must not overlap in time (they would race on it).
 */
#ifndef TP_DECODE_H
#define TP_DECODE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TP_OK = 0,
    TP_ERR_INVALID_ARG = 1, /* null pointer, bad size, N not dividing K or b*H */
    TP_ERR_UNSUPPORTED = 2, /* valid but outside what the kernels handle */
    TP_ERR_ALIGNMENT = 3,   /* a device pointer is not 16-byte aligned */
    TP_ERR_DEVICE = 4,      /* a HIP launch or runtime call failed */
    TP_ERR_OOM = 5          /* host allocation of the plan failed */
} tp_status;

/* The two reconciliation points of a layer (lesson 9.9, Conceito). */
typedef enum {
    TP_POINT_ATTN_OUT = 0, /* sequence-mixer output projection, K = k_attn */
    TP_POINT_FFN_DOWN = 1  /* FFN down projection, K = inter */
} tp_point;

/* Kernel family a point runs on. */
typedef enum {
    TP_PATH_VALU = 0, /* batch < 16: vector-ALU GEMV, 128-bit weight streaming */
    TP_PATH_MFMA = 1  /* batch >= 16: bf16 matrix-core skinny GEMM */
} tp_path;

/* Element formats of the packed step's weights (tp_plan_set_weight_format). */
typedef enum {
    TP_WEIGHTS_BF16 = 0,  /* bf16 */
    TP_WEIGHTS_MXFP8 = 1, /* microscaled FP8 E4M3, 32-row blocks, E8M0 scales */
    TP_WEIGHTS_MXFP4 = 2  /* microscaled FP4 E2M1, 32-row blocks, E8M0 scales */
} tp_weight_format;

typedef struct tp_plan_s* tp_plan_t;

/* What a plan resolved to (tp_plan_info). The struct is named by its tag,
 * `struct tp_plan_info`, or by the typedef tp_plan_info_t: in C a typedef
 * and a function share one namespace, and the function carries the name. */
typedef struct tp_plan_info {
    int64_t hidden;          /* H */
    int64_t inter;           /* FFN intermediate size I */
    int64_t k_attn;          /* K of the mixer output projection (default H) */
    int32_t n_ranks;         /* N */
    int32_t batch;           /* b, decode tokens per step */
    int64_t k_rank[2];       /* K_r = K / N per point (index: tp_point) */
    int32_t path[2];         /* tp_path per point */
    int32_t splits[2];       /* split-K factor the projection kernels use */
    int64_t chunk_elems;     /* C = b*H / N: ring chunk length */
    int64_t wire_bytes_bf16; /* per rank per reduction, bf16 payload: 2(N-1)*C*2 */
    int64_t wire_bytes_fp32; /* the same with the fp32 payload emulated here */
    int64_t workspace_bytes; /* device workspace every entry point may use */
    /* MoE share (zero unless tp_plan_set_moe was called) */
    int32_t n_experts, top_k, ep, local_experts;
    int64_t moe_inter;
    int32_t max_tokens;
    int32_t packed_kind;     /* layout of tp_pack_weights / kernel of tp_decode_layers_packed:
                                0 = the plan is not supported, 1 = pair strips (vector ALU),
                                2 = MFMA tiles (matrix cores) */
    int32_t stream_wgs;      /* packed_kind 2: workgroups of the matrix-core step (0 otherwise) */
    int32_t weight_format;   /* tp_weight_format of the packed step (tp_plan_set_weight_format) */
    int32_t acts_layout;     /* activations of tp_decode_layers_packed (tp_pack_activations):
                                0 = row-major [L][b][K_r] as given, 1 = the matrix-core
                                stream's A-operand order (packed_kind 2 from 5 tokens on) */
    int64_t packed_layer_bytes[2]; /* packed_kind 1: bytes of one layer's packed weights per point */
} tp_plan_info_t;

/*
 * Create a plan for hidden size H, FFN intermediate size I, N ranks and a
 * decode batch of b tokens. Host-only: touches no device.
 * Errors: TP_ERR_INVALID_ARG if any size < 1, N does not divide I or H
 * (the default k_attn), or N does not divide b*H (the ring needs N equal
 * chunks; a model is never split along a boundary its dimensions do not
 * divide, lesson 9.9, Conceito); TP_ERR_UNSUPPORTED if H is not a multiple
 * of 8 (rows are streamed in 16-byte vectors) or b > 64;
 * TP_ERR_OOM if the host allocation fails.
 */
tp_status tp_plan(int64_t hidden, int64_t inter, int32_t n_ranks, int32_t batch,
                  tp_plan_t* out);

/* Override K of the mixer output projection (e.g. 8192 -> 4096). Must be
 * called before the plan is first used. TP_ERR_INVALID_ARG if k_attn < 1
 * or N does not divide it. */
tp_status tp_plan_set_attn_dim(tp_plan_t plan, int64_t k_attn);

/*
 * Give the plan the width of the rank's mixer input projection: `cols` =
 * the Q, K and V columns this rank holds (its heads' columns, with K and V
 * replicated where there are fewer key-value heads than ranks: "Hosting
 * Qwen on Blackwell", Prefillers). Needed by tp_qkv_proj; widens
 * info.workspace_bytes to cover it. TP_ERR_INVALID_ARG unless cols >= 8
 * and cols is a multiple of 8; TP_ERR_UNSUPPORTED above 2^24.
 */
tp_status tp_plan_set_qkv_dim(tp_plan_t plan, int64_t cols);

/* Enable the expert-parallel MoE share: n_experts experts of intermediate
 * size moe_inter, top_k per token, spread over ep ranks (rank r owns the
 * contiguous experts [r*E/ep, (r+1)*E/ep)), for up to max_tokens tokens
 * ("Hosting Qwen on Blackwell", sections Prefillers, MoE Dispatch-Combine
 * and Expert Parallel). Must be called before first use.
 * TP_ERR_INVALID_ARG on sizes < 1, top_k > n_experts or ep not dividing
 * n_experts; TP_ERR_UNSUPPORTED if top_k > 32 or max_tokens > 4096. */
tp_status tp_plan_set_moe(tp_plan_t plan, int32_t n_experts, int32_t top_k, int32_t ep,
                          int64_t moe_inter, int32_t max_tokens);

/*
 * Choose the element format of the packed step's weights ("Hosting Qwen on
 * Blackwell", Quantization: the weights are converted statically to MXFP8;
 * MXFP4 is weighed too). TP_WEIGHTS_BF16 (the default), or microscaled
 * TP_WEIGHTS_MXFP8 / TP_WEIGHTS_MXFP4: blocks of 32 consecutive rows (along
 * K) of a column share one E8M0 scale 2^(E-127), elements FP8 E4M3 or FP4
 * E2M1. With an MX format the packed step (tp_decode_layers_packed and its
 * no-alloc and partials-only forms) runs the vector-ALU stream (packed_kind
 * 1) or the matrix-core stream (packed_kind 2: up to 16 tokens, no
 * partials-only form; chosen where 16-column strips stay whole, except
 * MXFP4 at one token, and beyond 4 tokens; knob stream_kind), on weights packed by
 * tp_pack_weights_mx, and needs K_r of both points to be multiples of 32
 * (packed_kind is 0 otherwise). Must be called before the
 * plan is first used. TP_ERR_INVALID_ARG for another value.
 */
tp_status tp_plan_set_weight_format(tp_plan_t plan, int32_t weight_format);

/* Tuning knobs (advanced; the defaults are tuned for MI355X). A knob that
 * changes the tiles ("splits_*", "valu_cols", "step_rows", "stream_wgs",
 * "target_wgs") can change info.workspace_bytes: size the workspace after
 * tuning ("serial_points" changes no tile). Known keys:
 * "splits_attn", "splits_ffn" (split-K factor, 0 = automatic),
 * "valu_cols" (columns per VALU workgroup: 128, 256 or 512),
 * "decode_mode" (0 = automatic, 1 = one launch per point,
 *                2 = one persistent launch per step),
 * "segment_loads" (16-byte loads per lane in each of the two register
 *                banks of tp_decode_layers_packed: 4 or 8; 0 = automatic,
 *                8 for batch <= 4, else 4; 8 only takes effect for
 *                batch <= 4),
 * "stream_flat" (vector-ALU stream, dataflow order: -1 = automatic: 1
 *                where a layer's blocks fit one register bank, and with
 *                bf16 weights from 4 tokens; 0 = a point per bank, 1 = the
 *                banks run across points with no per-point barrier),
 * "stream_kind" (tp_decode_layers_packed: 0 = automatic, 1 = vector-ALU
 *                stream on pair strips, 2 = matrix-core stream on MFMA tiles),
 * "stream_wgs" (matrix-core stream: workgroups sharing the tiles, 0 = one
 *                per compute unit; at most 256 and H/16, at least H/32),
 * "mfma_acts" (matrix-core stream: the activations' layout, 0 = automatic:
 *                row-major up to 4 tokens, else A-operand order;
 *                1 = row-major (up to 16 tokens), 2 = A-operand order;
 *                see info.acts_layout),
 * "mfma_sl", "mfma_wps" (matrix-core stream, up to 32 tokens: tiles per
 *                register bank and compute waves, the pairs (2, 12) and
 *                (3, 8); 0 = automatic: (3, 8) up to 16 tokens, else (2, 12)),
 * "mfma_oth" (matrix-core stream: the other ranks' values are staged up
 *                to this many points ahead, 2, 4 or 8; 0 = automatic: 2),
 * "mfma_flat" (matrix-core stream, up to 32 tokens: -1 = automatic (1 from
 *                8 to 16 tokens, and with bf16 weights below 8 tokens where
 *                a layer's tiles per compute wave fit the ring of slots,
 *                e.g. H4096 N=8), 0 = a register bank per segment of a point,
 *                1 = a ring of 2 mfma_sl tile slots running across
 *                segments and points),
 * "moe_variant" (tp_moe_partial's expert kernel: 0 = default, 1..7),
 * "serial_points" (tp_decode_layers and tp_decode_layers_packed: 0 = each
 *                hidden-state element follows its own chain, 1 = point j+1
 *                also waits for all of point j, see there),
 * "target_wgs" (per-point launches: workgroups a point's split-K grid
 *                aims at, 0 = automatic: one per CU for the matrix cores,
 *                two for the vector ALU),
 * "step_kind" (tp_decode_layers, tp_rowparallel_partials, batch < 16: the
 *                persistent step's kind, 0 = automatic, 1 = vector ALU,
 *                2 = matrix cores; from 16 tokens always matrix cores),
 * "swiglu_layers" (tp_gate_up_swiglu, tp_qkv_proj: most layers per
 *                launch, 0 = automatic: as many as 32 MiB of fp32 sums hold;
 *                tp_qkv_proj rounds it down to an even number, at least 2),
 * "xcd_walk" (the persistent step: 1 = each XCD's workgroups take
 *                contiguous tiles of every round, so that a point's column
 *                tiles share an L2; the same bits; 0 = off; -1 = automatic,
 *                the default: on for tp_qkv_proj from 16 tokens with at most
 *                2048 columns, where narrow points read a wide x, off
 *                elsewhere),
 * "step_rows" (tp_decode_layers, tp_rowparallel_partials,
 *                tp_gate_up_swiglu: most rows per tile of the persistent
 *                step, 0 = automatic: 2048 for 512-column and matrix-core
 *                tiles, 1024 for narrower vector-ALU ones; the whole K for
 *                matrix-core tiles of tp_gate_up_swiglu).
 * TP_ERR_INVALID_ARG for an unknown key or an out-of-range value. */
tp_status tp_plan_tune(tp_plan_t plan, const char* key, int64_t value);

/*
 * The plan's resolved sizes: K_r per point, the ring chunk length C = b*H/N,
 * the wire bytes per rank per reduction, 2(N-1)*C*e for the pages' bf16
 * payload (e = 2) and for the fp32 payload emulated here (e = 4) (lesson
 * 9.9, Conceito: 2(N-1)/N of the payload on each rank's wire), the
 * workspace bytes the entry points need, and the kernel family of each
 * point. Host-only. TP_ERR_INVALID_ARG for a null argument.
 */
tp_status tp_plan_info(tp_plan_t plan, struct tp_plan_info* out);
/* The same as tp_plan_info (the name this library first exported). */
tp_status tp_plan_info_get(tp_plan_t plan, struct tp_plan_info* out);
void tp_plan_destroy(tp_plan_t plan);
const char* tp_status_str(tp_status status);

/*
 * Prepare a workspace of at least info.workspace_bytes device bytes for use
 * with this plan (clears the completion counters the kernels use). Call it
 * once after allocating the workspace; every later call leaves it ready for
 * the next. The fill is a kernel, not a memset, so it may be captured into
 * a HIP graph.
 */
tp_status tp_workspace_init(tp_plan_t plan, void* workspace, void* stream);

/*
 * Read the workspace's error word (synchronous: waits for the device).
 * workspace = NULL reads the error word of tp_decode_layers_packed_noalloc's
 * scratch on the current device instead (0 if it was never used there).
 * *flags = 0 after successful calls. Bit 0 is set if a bounded wait between
 * workgroups timed out: a decode step's wait for the previous
 * reconciliation point, a matrix-core stream's wait for a cut strip's other
 * piece, or a matrix-core projection's wait for its column tile's other
 * split-K partials (bit 1: a wait between the waves of one workgroup). The
 * launch then drains without completing and its outputs are not valid.
 * Those waits assume that all of the launch's workgroups are resident at
 * once, which the library checks against the device's occupancy before it
 * launches; other work holding compute units for longer than a wait's
 * bound (about a million polls of the flag, well over 0.1 s) can still make
 * it time out. tp_workspace_init clears the word.
 */
tp_status tp_workspace_status(tp_plan_t plan, const void* workspace, int32_t* flags);

/*
 * Row-parallel partial projection for one point (lesson 9.9, Conceito):
 *     p[b, n] = sum_{k < K_r} x[b, k] * w[k, n]
 * bf16 products accumulated in fp32 (split-K, fixed summation order, so
 * repeated calls give identical bits).
 *   x  bf16 [batch][K_r] row-major — the rank's slice of the activation
 *   w  bf16 [K_r][hidden] row-major — the rank's rows of W
 *   p  fp32 [batch][hidden] (output)
 *   workspace: info.workspace_bytes, prepared by tp_workspace_init.
 * Errors: TP_ERR_INVALID_ARG (null pointer, point not 0/1),
 * TP_ERR_ALIGNMENT, TP_ERR_DEVICE.
 */
tp_status tp_rowparallel_partial(tp_plan_t plan, int32_t point, const void* x, const void* w,
                                 float* p, void* workspace, void* stream);

/*
 * The partial projections of a whole layer stack, in layer order, in one
 * call (lesson 9.9, Conceito: the rank's partial at each of a layer's two
 * reconciliation points; no reduction, no residual):
 *     p[l][0] = x_attn[l] . w_o[l],   p[l][1] = x_ffn[l] . w_down[l]
 *   x_attn bf16 [L][batch][k_attn/N]   w_o    bf16 [L][k_attn/N][hidden]
 *   x_ffn  bf16 [L][batch][inter/N]    w_down bf16 [L][inter/N][hidden]
 *   p      fp32 [L][2][batch][hidden] (output)
 * One cooperative launch with the tiles of the persistent decode step
 * (tp_decode_layers): p[l][point] equals the slot that tp_decode_layers
 * writes for this rank with the same plan, bit for bit. With "decode_mode"
 * = 1, one launch per point, equal to tp_rowparallel_partial's. n_layers = 0 does nothing (the pointers may
 * then be null). Errors as tp_rowparallel_partial, and TP_ERR_INVALID_ARG
 * for n_layers < 0, TP_ERR_ALIGNMENT if batch * K_r is not a multiple of 8
 * for either point (the stacked slices must stay 16-byte aligned).
 */
tp_status tp_rowparallel_partials(tp_plan_t plan, int32_t n_layers, const void* x_attn,
                                  const void* w_o, const void* x_ffn, const void* w_down,
                                  float* p, void* workspace, void* stream);

/*
 * Column-parallel FFN up projection with its activation, for a layer stack
 * (lesson 9.9, Conceito: the FFN's up projection is split over the ranks
 * the other way from its down projection, so each rank computes its own
 * columns, and with them its slice of the down projection's input, with no
 * reduction). The pages name no activation; this is SwiGLU, with a gate and
 * an up matrix split by the same columns:
 *     a[l] = bf16( silu(x[l] . w_gate[l]) * (x[l] . w_up[l]) ),
 *     silu(z) = z / (1 + e^-z)
 *   x       bf16 [L][batch][hidden] (the full hidden state of each layer)
 *   w_gate, w_up  bf16 [L][hidden][inter/N] row-major (the rank's columns)
 *   out     bf16 [L][batch][inter/N] (output: the down projection's x slice)
 * The two projections accumulate in fp32 (the persistent step's tiles, the
 * gate and up matrices as the two points of each layer, as many layers per
 * launch as "swiglu_layers" allows, spread evenly over the launches; with
 * matrix-core tiles and "step_rows" unset, one tile spans the whole K of
 * a column tile, so no split partials are written), then silu and the product in fp32,
 * rounded to bf16 nearest-even (a second launch). n_layers = 0 does nothing (the pointers may then be null).
 * TP_ERR_UNSUPPORTED if inter/N is not a multiple of 8; TP_ERR_ALIGNMENT
 * for pointers not 16-byte aligned or batch*inter/N not a multiple of 8;
 * TP_ERR_INVALID_ARG for a null pointer or n_layers < 0.
 */
tp_status tp_gate_up_swiglu(tp_plan_t plan, int32_t n_layers, const void* x, const void* w_gate,
                            const void* w_up, void* out, void* workspace, void* stream);

/*
 * Column-parallel mixer input projection for a layer stack (lesson 9.9,
 * Conceito: the attention heads are split over the ranks by columns, so a
 * rank computes its heads' Q, K and V columns from the full hidden state,
 * with no reduction):
 *     a[l] = bf16( x[l] . w_qkv[l] )
 *   x      bf16 [L][batch][hidden] (the full hidden state of each layer)
 *   w_qkv  bf16 [L][hidden][cols] row-major, cols = tp_plan_set_qkv_dim's
 *   out    bf16 [L][batch][cols] (output)
 * fp32 accumulation on the persistent step's tiles (two consecutive layers
 * as its two points, an odd last layer in a launch of its own; matrix-core
 * tiles span the whole K unless "step_rows" is set), rounded to bf16
 * nearest-even by a second launch. n_layers = 0 does nothing (the pointers
 * may then be null). TP_ERR_UNSUPPORTED if tp_plan_set_qkv_dim was not
 * called; TP_ERR_ALIGNMENT for pointers not 16-byte aligned;
 * TP_ERR_INVALID_ARG for a null pointer or n_layers < 0.
 */
tp_status tp_qkv_proj(tp_plan_t plan, int32_t n_layers, const void* x, const void* w_qkv, void* out,
                      void* workspace, void* stream);

/*
 * Ring-ordered all-reduce sum of the N partials plus the residual
 * (lesson 9.9, Conceito; "Hosting Qwen on Blackwell", All-Reduce). The
 * payload is the flattened [batch x hidden] vector cut into N chunks of
 * C = b*H/N elements; chunk c is summed in rank order c, c+1, ..., c+N-1
 * (mod N) — the order of a ring reduce-scatter started by rank c — one
 * binary32 addition at a time, then the residual is added:
 *     out[i] = (((p_c[i] + p_{c+1}[i]) + ...) + p_{c+N-1}[i]) + residual[i]
 * Bit-exact: no fused or reassociated arithmetic, denormals kept.
 *   partials fp32 [N][batch][hidden] rank-major
 *   residual fp32 [batch][hidden]; out fp32 [batch][hidden] (may alias residual)
 *   out_bf16 bf16 [batch][hidden] or NULL: out rounded to nearest-even bf16
 */
tp_status tp_ring_reduce(tp_plan_t plan, const float* partials, const float* residual,
                         float* out, void* out_bf16, void* stream);

/*
 * One rank's share of a decode step over n_layers layers: for each layer,
 * for the mixer output point and then the FFN down point, compute this
 * rank's partial into its slot and set hidden <- ring_sum(slot) + hidden
 * (lesson 9.9, Conceito: two reconciliation points per layer, each an
 * all-reduce of one hidden vector per decoded token). Each point's
 * activation slice is an input (the operations between the points are
 * not part of this path).
 *   x_attn bf16 [L][batch][k_attn/N]   w_o    bf16 [L][k_attn/N][hidden]
 *   x_ffn  bf16 [L][batch][inter/N]    w_down bf16 [L][inter/N][hidden]
 *   slots  fp32 [L][2][N][batch][hidden]: the other N-1 ranks' partials are
 *          inputs; entry [l][point][rank] is overwritten with this rank's
 *   hidden fp32 [batch][hidden], in/out (the residual stream)
 * The whole step is one cooperative (persistent) launch over tiles of long
 * row ranges, streamed. Below 16 tokens the vector-ALU step, unless the
 * points are small (an FFN slice of at most 2048 rows, or batch >= 8 with
 * hidden < 5120; "step_kind"), where the matrix-core step is faster. The
 * vector-ALU step: tiles of 512 columns
 * (256 where hidden < 5120; "valu_cols") by at most "step_rows" rows (2048
 * for 512 columns, 1024 for 256) and about 16384 / batch; with the same
 * tiles as the per-point launches (valu_cols and splits_attn / splits_ffn
 * set so that both take the same rows) the bits equal those of
 * tp_rowparallel_partial followed by tp_ring_reduce at each point. The
 * matrix-core step: tiles of 128 columns by at most 2048 rows
 * ("step_rows"), whose fp32 sums are ordered differently from
 * tp_rowparallel_partial's (both within the partial tolerance). With
 * "decode_mode" = 1 each point is one launch and the results equal
 * tp_rowparallel_partial followed by tp_ring_reduce, bit for bit. Point order as in
 * tp_decode_layers_packed: by default each hidden-state element follows its
 * own chain; "serial_points" = 1 makes every point wait for all of the
 * previous one. Both give the same bits. The workspace's error word
 * (tp_workspace_status) reports a wait that timed out.
 */
tp_status tp_decode_layers(tp_plan_t plan, int32_t n_layers, int32_t rank,
                           const void* x_attn, const void* w_o,
                           const void* x_ffn, const void* w_down,
                           float* slots, float* hidden, void* workspace, void* stream);

/*
 * One reconciliation point: the rank's partial of `point` into its slot, then
 * hidden <- ring_sum(slots) + hidden (lesson 9.9, Conceito). For batch < 16
 * in one launch (a split-K projection's last-arriving split does the ring
 * for its columns); for batch >= 16 the ring is a second launch, which is
 * faster there.
 *   x bf16 [batch][K_r], w bf16 [K_r][hidden] (row-major slice),
 *   slots fp32 [N][batch][hidden]: the other N-1 ranks' partials are inputs,
 *   entry [rank] is overwritten; hidden fp32 [batch][hidden], in/out.
 * Same results as tp_rowparallel_partial followed by tp_ring_reduce, bit
 * for bit. Errors as tp_rowparallel_partial.
 */
tp_status tp_decode_point(tp_plan_t plan, int32_t point, int32_t rank, const void* x, const void* w,
                          float* slots, float* hidden, void* workspace, void* stream);

/*
 * Packed weights for the streamed decode step. A rank's weight slice
 * W_r[K_r][H] (row-major, as tp_rowparallel_partial takes it) is stored
 * once, when the weights are loaded (not part of the decode step), in the
 * layout of the plan's packed_kind (see tp_plan_info):
 *  1, pair strips (vector-ALU stream):
 *     P[s][kp][c][q] = W_r[2kp + q][4s + c]
 *     s < H/4, kp < ceil(K_r/2), c < 4, q < 2   (rows past K_r are zero)
 *     H/4 strips of 4 columns; each 16-byte vector holds rows 2kp and 2kp+1
 *     of its strip as one bf16 pair per column; a strip's rows are
 *     contiguous. w_packed bf16 [n_layers][H/4][ceil(K_r/2)][8].
 *  2, MFMA tiles (matrix-core stream, v_mfma_f32_16x16x32_bf16 B operands):
 *     T[s][kb][h][l][i] = W_r[64kb + 16(l/16) + 8h + i][16s + l%16]
 *     s < H/16, kb < ceil(K_r/64), h < 2, lane l < 64, i < 8 (rows past
 *     K_r are zero): 2 KB tiles of 64 rows x 16 columns.
 *     w_packed bf16 [n_layers][H/16][ceil(K_r/64)][2][64][8].
 * tp_pack_weights: w bf16 [n_layers][K_r][hidden] -> w_packed for `point`.
 * w and w_packed must not overlap. TP_ERR_UNSUPPORTED if packed_kind is 0
 * or the plan's weights are MX (tp_quantize_mx, tp_pack_weights_mx).
 */
tp_status tp_pack_weights(tp_plan_t plan, int32_t point, int32_t n_layers, const void* w,
                          void* w_packed, void* stream);

/*
 * Static conversion of a point's bf16 weight stack to the plan's MX format
 * ("Hosting Qwen on Blackwell", Quantization), block by block (32 rows of a
 * column): the scale E = floor(log2(max |w|)) - emax + 127, emax = 8 (E4M3)
 * or 2 (E2M1), clamped to [0, 254] (0 for an all-zero block; 255, NaN,
 * with zero codes if the block holds a NaN or an infinity); each element
 * w * 2^(127-E) rounded to the nearest element value, ties to the even
 * code, saturating at the largest finite value (448 or 6), sign kept.
 *   w      bf16 [n_layers][K_r][hidden] (the rank's slices, row-major)
 *   codes  uint8, MXFP8: [n_layers][K_r][hidden]; MXFP4: [n_layers][K_r/2][hidden],
 *          two rows of a column per byte, the even row in the low nibble
 *   scales uint8 [n_layers][K_r/32][hidden] (E of rows 32kb..32kb+31)
 * TP_ERR_UNSUPPORTED unless the plan's format is MX and 32 divides K_r.
 */
tp_status tp_quantize_mx(tp_plan_t plan, int32_t point, int32_t n_layers, const void* w, void* codes,
                         void* scales, void* stream);

/*
 * Pack a point's MX weight stack (tp_quantize_mx's layout) for the packed
 * step, once, at load time: w_packed holds info.packed_layer_bytes[point] *
 * n_layers bytes.
 *  packed_kind 1: first, for every layer, the 16-byte vectors
 *   [hidden/4][K_r/R][4 columns][R rows] (R = 4 FP8 codes, or 8 FP4 codes as
 *   4 bytes of two rows each), then, for every layer, the scale words
 *   [hidden/4][K_r/32], the 4 columns' E in bytes 0..3.
 *  packed_kind 2: tiles [n_layers][hidden/16][ceil(K_r/64)] of 64 rows x 16
 *   columns: the codes lane-major, lane l holding rows 16(l/16) .. +15 of
 *   column l%16 (16 FP8 bytes, or 8 bytes of two FP4 rows, the even row in
 *   the low nibble), then 32 scale bytes [2 blocks][16 columns]; codes and
 *   scales past K_r are zero (1056 bytes a tile for FP8, 544 for FP4).
 * TP_ERR_UNSUPPORTED unless the plan's format is MX and packed_kind is 1 or 2.
 */
tp_status tp_pack_weights_mx(tp_plan_t plan, int32_t point, int32_t n_layers, const void* codes,
                             const void* scales, void* w_packed, void* stream);

/*
 * The activation slices of a step in the order tp_decode_layers_packed
 * reads them (part of the decode step: call it once per step).
 *  info.acts_layout 0 (packed_kind 1, and packed_kind 2 up to 4 tokens):
 *     row-major, as given (the bytes are copied); the matrix-core stream
 *     then reads each token's row directly.
 *  info.acts_layout 1 (packed_kind 2 from 9 tokens on): A-operand order of
 *     the matrix-core stream,
 *     X[kb][tt][h][l][i] = x[16tt + l%16][64kb + 16(l/16) + 8h + i]
 *     kb < ceil(K_r/64), tt < ceil(b/16), h < 2, lane l < 64, i < 8 (zero
 *     for rows past K_r; entries of tokens past b are left unwritten and
 *     never read): each 16-byte-per-lane load of the step then reads 1 KB
 *     (b >= 16) of contiguous memory.
 *     x*_packed bf16 [n_layers][ceil(K_r/64)][ceil(b/16)][2][64][8].
 * x_attn bf16 [n_layers][batch][k_attn/N], x_ffn bf16 [n_layers][batch][inter/N]
 * in; xa_packed, xf_packed out (distinct from each other and the inputs).
 * TP_ERR_UNSUPPORTED if packed_kind is 0.
 */
tp_status tp_pack_activations(tp_plan_t plan, int32_t n_layers, const void* x_attn, const void* x_ffn,
                              void* xa_packed, void* xf_packed, void* stream);

/*
 * The decode step of tp_decode_layers on packed weights and activations
 * (tp_pack_weights, tp_pack_activations): same results (the projections
 * within their fp tolerance, the ring stage the same binary32 additions in
 * the same order). One launch per step; per point it writes the rank's
 * partial into its slot and sets hidden <- ring_sum(slot) + hidden
 * (lesson 9.9, Conceito), keeping its columns of the hidden state on chip
 * between points.
 *  packed_kind 1: each workgroup owns a set of 4-column strips for every
 *     point and streams their weights over all of K_r.
 *  packed_kind 2: each point's 64-row tiles, in strip-major order, are cut
 *     into equal contiguous ranges, one per workgroup (one per CU; info
 *     stream_wgs); a 16-column strip cut between two workgroups is summed
 *     by the one holding its first rows, its own rows first, then the other
 *     workgroup's partial (handed over through the workspace). The result
 *     is deterministic for a given stream_wgs. Needs that many compute
 *     units on the device (TP_ERR_UNSUPPORTED otherwise).
 *
 * Point order. Every element of the hidden state is updated point after
 * point, each update reading the previous one; since each point's
 * activation slice is an input, no point has to wait for other columns.
 * With the plan knob "serial_points" = 1 (packed_kind 1 only) the step also
 * emulates a model in which a point's activation depends on the whole
 * previous hidden state: point j+1's activation is read only after every
 * column of point j is complete (a grid-wide wait per point; cooperative
 * launch). Both orders give the same bits. The workspace's error word
 * (tp_workspace_status) reports a wait that timed out.
 *
 * TP_ERR_UNSUPPORTED if packed_kind is 0 (packed_kind 1 needs batch <= 8,
 * n_ranks <= 8, K_r even for both points, batch * K_r a multiple of 8, the
 * activation slices of a point within about 150 KiB of on-chip buffers and
 * 16 * batch * ceil(hidden / 1024) <= 192; packed_kind 2 needs batch <= 64,
 * n_ranks <= 8, hidden a multiple of 16, K_r a multiple of 8 and
 * hidden/16 <= 2 * stream_wgs), or with "serial_points" = 1 on packed_kind 2
 * or on a packed_kind 1 stream of more than 256 workgroups (hidden above
 * 15,360: one cooperative workgroup per compute unit).
 */
tp_status tp_decode_layers_packed(tp_plan_t plan, int32_t n_layers, int32_t rank,
                                  const void* x_attn, const void* w_o_packed,
                                  const void* x_ffn, const void* w_down_packed,
                                  float* slots, float* hidden, void* workspace, void* stream);

/*
 * tp_decode_layers_packed without a workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc). Same arguments, kernels and
 * results (bit for bit) as tp_decode_layers_packed, minus `workspace`.
 * Instead of a workspace the kernels use a scratch array the library keeps
 * in device memory, one per GPU, held until the process ends: 8.25 MiB
 * (a 256 KiB region of completion, exchange and error words, and 8 MiB of
 * exchange buffers for the matrix-core stream). The call allocates nothing
 * (no hipMalloc, hipFree or allocating library routine); its first call on
 * a GPU looks the array up and clears its words with a kernel on `stream`.
 * Each call clears the array's error word (a kernel, in stream order) and
 * the kernels leave every other word ready for the next call.
 * All calls on one GPU share that GPU's array: calls that overlap in time
 * on one GPU (on different streams or threads) race on it and must not be
 * issued. tp_workspace_status(plan, NULL, &flags) reads the error word of
 * the latest call on the current device.
 * Errors as tp_decode_layers_packed, and TP_ERR_UNSUPPORTED where the plan
 * needs more scratch than the array holds: packed_kind 2 with
 * 2 * 4 * (hidden/16) * ceil(batch/16) KiB of exchange buffers above 8 MiB
 * (e.g. hidden 5120 with batch > 48; hidden 4096 fits every batch).
 */
tp_status tp_decode_layers_packed_noalloc(tp_plan_t plan, int32_t n_layers, int32_t rank,
                                          const void* x_attn, const void* w_o_packed,
                                          const void* x_ffn, const void* w_down_packed,
                                          float* slots, float* hidden, void* stream);

/*
 * The partial projections of a layer stack on weights packed by
 * tp_pack_weights, in layer order, in one call (lesson 9.9, Conceito; as
 * tp_rowparallel_partials, no reduction, no residual): the vector-ALU
 * stream of tp_decode_layers_packed with packed_kind 1, writing each
 * point's partial instead of the ring sum.
 *   x_attn, w_o_packed, x_ffn, w_down_packed as tp_decode_layers_packed
 *   p fp32 [L][2][batch][hidden] (output)
 * p[l][point] equals the slot tp_decode_layers_packed writes for this rank
 * with the same plan, bit for bit. n_layers = 0 does nothing (the pointers
 * may then be null). TP_ERR_UNSUPPORTED unless packed_kind is 1; other
 * errors as tp_decode_layers_packed.
 */
tp_status tp_rowparallel_partials_packed(tp_plan_t plan, int32_t n_layers, const void* x_attn,
                                         const void* w_o_packed, const void* x_ffn,
                                         const void* w_down_packed, float* p, void* workspace,
                                         void* stream);

/*
 * Pack a point's bf16 weight stack for tp_prefill_layers, once, at load
 * time: the matrix-core tile layout of tp_pack_weights' packed_kind 2,
 *     T[l][s][kb][h][lane][i] = W[l][64kb + 16(lane/16) + 8h + i][16s + lane%16]
 * (rows past K_r zero), whatever the plan's decode batch.
 *   w bf16 [n_layers][K_r][hidden] -> w_packed bf16 [n_layers][hidden/16][ceil(K_r/64)][2][64][8]
 * TP_ERR_UNSUPPORTED if hidden is not a multiple of 16.
 */
tp_status tp_prefill_pack_weights(tp_plan_t plan, int32_t point, int32_t n_layers, const void* w,
                                  void* w_packed, void* stream);

/*
 * The prefill of a prompt of `tokens` tokens through the layer stack, for
 * rank `rank`: the same two reconciliation points per layer as the decode
 * step, each carrying one hidden vector per token (lesson 9.9, Conceito: a
 * 4,096-token prompt runs every position at once, so every collective
 * carries 4,096 hidden vectors and bandwidth, not latency, governs). Per
 * point: the rank's partial P = X . W_r (T x hidden, fp32 accumulation on
 * the bf16 matrix cores) into its slot, then hidden <- ring_sum(slot) +
 * hidden, the ring order of tp_ring_reduce over the flattened [T x hidden]
 * payload (chunks of T*hidden/N).
 *   x_attn bf16 [L][tokens][k_attn/N]   x_ffn bf16 [L][tokens][inter/N]
 *   w_o_packed, w_down_packed: tp_prefill_pack_weights' layout
 *   slots  fp32 [L][2][N][tokens][hidden]: the other ranks' partials are
 *          inputs; entry [l][point][rank] is overwritten
 *   hidden fp32 [tokens][hidden], in/out
 * One cooperative launch over tiles of 128 tokens x 256 columns of every
 * point; a tile's ring sum waits (bounded) for the previous point's sum of
 * the same tile; the workspace's error word reports a wait that timed out.
 * Errors: TP_ERR_INVALID_ARG (null pointer, tokens < 1, rank out of range,
 * N not dividing tokens*hidden), TP_ERR_ALIGNMENT, TP_ERR_UNSUPPORTED
 * (hidden not a multiple of 16, K_r not a multiple of 8, n_ranks > 8, a
 * point's X of 2 GiB or more, more than 1024 tiles per point).
 */
tp_status tp_prefill_layers(tp_plan_t plan, int32_t n_layers, int32_t rank, int32_t tokens,
                            const void* x_attn, const void* w_o_packed, const void* x_ffn,
                            const void* w_down_packed, float* slots, float* hidden, void* workspace,
                            void* stream);

/*
 * Top-k routing of decode tokens ("Hosting Qwen on Blackwell", Prefillers:
 * each token goes to top_k of the experts). Per token: softmax over the
 * experts' logits (computed in double), the top_k experts by probability
 * (ties to the lower index), their probabilities renormalised to sum to 1
 * (renorm != 0) or left as they are; listed in ascending expert order.
 *   logits fp32 [tokens][n_experts] (finite or -inf; NaN is not allowed)
 *   sel_expert int32 [tokens][top_k], sel_weight fp32 [tokens][top_k] (outputs)
 * The expert choice compares the fp32 logits directly (softmax is
 * monotone), so it is exact. TP_ERR_INVALID_ARG if the plan has no MoE
 * share or tokens > max_tokens; TP_ERR_UNSUPPORTED if n_experts > 2048.
 */
tp_status tp_moe_route(tp_plan_t plan, const float* logits, int32_t tokens, int32_t renorm,
                       int32_t* sel_expert, float* sel_weight, void* stream);

/*
 * Pack one rank's experts for tp_moe_partial, once, at load time:
 *     w_local  bf16 [E/ep][moe_inter][hidden] (row-major, as trained)
 *     w_packed bf16 [E/ep][hidden/16][ceil(moe_inter/64)][1024], with
 *     w_packed[e][s][kb][512h + 8l + i] = w_local[e][64kb + 16(l/16) + 8h + i][16s + l%16]
 *     (h < 2, l < 64, i < 8; rows past moe_inter are zero)
 * the matrix-core tiles of the dense decode step (tp_pack_weights with
 * packed_kind 2), one expert per matrix: 2 KB per 64 rows x 16 columns.
 * TP_ERR_UNSUPPORTED if hidden is not a multiple of 16.
 */
tp_status tp_moe_pack_experts(tp_plan_t plan, const void* w_local, void* w_packed, void* stream);

/*
 * Expert-parallel down projection and local weighted combine for rank
 * `rank` ("Hosting Qwen on Blackwell", MoE Dispatch-Combine and Expert
 * Parallel: the combine first accumulates, per token, the contributions of
 * the experts on this rank, weighted by the routing weights; the all-reduce
 * over ranks follows, e.g. tp_ring_reduce over the ep ranks' parts):
 *     part[t, :] = sum over s with sel_expert[t,s] on this rank, in
 *                  ascending expert order, of sel_weight[t,s] * (u[t,s,:] . W_e)
 *   sel_expert int32 [tokens][top_k], sel_weight fp32 [tokens][top_k]
 *   u        bf16 [tokens][top_k][moe_inter]: one activation per selection
 *   w_packed this rank's experts packed by tp_moe_pack_experts
 *   part     fp32 [tokens][hidden] (output; rows of tokens with no local
 *            expert are zero)
 * Each projection accumulates in fp32 (fixed order); the combine adds the
 * local experts' weighted rows in ascending expert order. Experts that no
 * token selected are not read. Expert ids outside this rank's range are
 * skipped. Uses the workspace (one projected row per selection).
 * TP_ERR_UNSUPPORTED if moe_inter is not a multiple of 8, hidden not a
 * multiple of 16, or one expert's packed tiles reach 2 GiB.
 */
tp_status tp_moe_partial(tp_plan_t plan, int32_t rank, const int32_t* sel_expert,
                         const float* sel_weight, int32_t tokens, const void* u,
                         const void* w_packed, float* part, void* workspace, void* stream);

/*
 * The MoE share's reconciliation point: tp_moe_partial for the plan's batch
 * of tokens (the rank's experts), with the combine writing the rank's
 * partial into its slot and, in the same launch, hidden <- ring_sum(slots) +
 * hidden (lesson 9.9, Conceito; "Hosting Qwen on Blackwell", MoE
 * Dispatch-Combine: the combine's all-reduce).
 *   sel_expert, sel_weight [batch][top_k] (tp_moe_route), u bf16
 *   [batch][top_k][moe_inter], w_packed as tp_moe_partial,
 *   slots fp32 [N][batch][hidden] (entry [rank] overwritten), hidden fp32
 *   [batch][hidden] in/out.
 * The partial equals tp_moe_partial's bit for bit and the ring stage
 * tp_ring_reduce's. TP_ERR_INVALID_ARG also if ep != n_ranks or batch >
 * max_tokens.
 */
tp_status tp_moe_decode(tp_plan_t plan, int32_t rank, const int32_t* sel_expert,
                        const float* sel_weight, const void* u, const void* w_packed,
                        float* slots, float* hidden, void* workspace, void* stream);

/*
 * Pack the rank's attention output slice for tp_moe_layer_decode, once, at
 * load time: w bf16 [k_attn/N][hidden] (row-major) -> w_packed bf16
 * [hidden/16][ceil(k_attn/N / 64)][1024], the tile layout of
 * tp_moe_pack_experts for a single matrix. TP_ERR_INVALID_ARG if the plan
 * has no MoE share or no attention dimension; TP_ERR_UNSUPPORTED if hidden
 * is not a multiple of 16.
 */
tp_status tp_moe_pack_attn(tp_plan_t plan, const void* w, void* w_packed, void* stream);

/*
 * One MoE layer's whole decode share for rank `rank` ("Hosting Qwen on
 * Blackwell", MoE Dispatch-Combine and Expert Parallel; lesson 9.9,
 * Conceito, for the two ring sums), for the plan's batch of T tokens:
 *   1. routing (tp_moe_route): sel_expert, sel_weight [T][top_k] written;
 *   2. the attention output slice's partial x_attn . W_attn into
 *      slots_attn[rank], then hidden <- ring_sum(slots_attn) + hidden;
 *   3. the rank's experts and local combine (tp_moe_partial) into
 *      slots_moe[rank], then hidden <- ring_sum(slots_moe) + hidden.
 *   logits fp32 [T][n_experts]; x_attn bf16 [T][k_attn/N];
 *   w_attn_packed: tp_moe_pack_attn's tiles; u bf16 [T][top_k][moe_inter];
 *   w_packed: tp_moe_pack_experts's tiles; slots_attn, slots_moe fp32
 *   [N][T][hidden] (entry [rank] of each overwritten); hidden fp32
 *   [T][hidden] in/out.
 * Two launches: routing, the attention slice and the experts share one
 * (the expert workgroups wait, bounded, for the routing workgroups, which
 * come first in dispatch order; a timeout sets bit 0 of the workspace's
 * error word), and one for both ring sums. The routing equals
 * tp_moe_route's and slots_moe[rank] tp_moe_partial's bit for bit; the
 * attention partial accumulates each column in fp32 over 64-row tiles
 * split among four waves, then sums the waves in order; both ring stages
 * equal tp_ring_reduce's bit for bit given the same slots. Calls that
 * overlap on one workspace race. TP_ERR_INVALID_ARG also if ep != n_ranks,
 * batch > max_tokens or the plan has no attention dimension;
 * TP_ERR_UNSUPPORTED if n_experts > 512, top_k > 64, moe_inter or
 * k_attn/N is not a multiple of 8, or hidden not a multiple of 16.
 */
tp_status tp_moe_layer_decode(tp_plan_t plan, int32_t rank, const float* logits, int32_t renorm,
                              const void* x_attn, const void* w_attn_packed, const void* u,
                              const void* w_packed, int32_t* sel_expert, float* sel_weight,
                              float* slots_attn, float* slots_moe, float* hidden,
                              void* workspace, void* stream);

/*
 * Measurement: the device's streaming-read ceiling. Reads `bytes` of `buf`
 * with 16-byte nontemporal loads (the access the decode kernels make of
 * their weights: "Hosting Qwen on Blackwell", Decoders, a decode matmul
 * costs what loading its weights costs), `workgroups` workgroups of 512
 * threads in a grid-stride walk (16 loads in flight per thread), and stores one XOR fold of the data per
 * workgroup into sink[0 .. workgroups) so that no load is dropped. No
 * arithmetic of the method. bytes a multiple of 16, buf and sink 16-byte
 * aligned (TP_ERR_ALIGNMENT); TP_ERR_INVALID_ARG for a null pointer,
 * bytes < 0 or workgroups outside 1 .. 65536.
 */
tp_status tp_stream_read_probe(const void* buf, int64_t bytes, uint32_t* sink, int32_t workgroups,
                               void* stream);

/*
 * Debug mode, process-wide: with on = 1 every entry point waits for its
 * stream after each kernel launch and returns TP_ERR_DEVICE from the call
 * whose kernel failed (a fault, an abort, a launch error), rather than
 * leaving it to a later call; nothing waits while the stream is being
 * captured into a graph. Off by default; on from the first launch if the
 * environment variable TP_DEBUG_SYNC is set to a value other than "0".
 * Slows every call down by a host round trip. TP_ERR_INVALID_ARG unless on
 * is 0 or 1.
 */
tp_status tp_set_debug_sync(int32_t on);

#ifdef __cplusplus
}
#endif

#endif /* TP_DECODE_H */
