// Pair-strip weight layout and the decode step that streams it.
//
// The decode projections are bound by streaming the weights from HBM
// ("Hosting Qwen on Blackwell", section Decoders: the decode matmuls depend
// on the cost of loading the weights); each reconciliation point is followed
// by the sum of the ranks' partials before the residual stream continues
// (lesson 9.9 "Interconnects e clusters", section 01 · Conceito).
//
// Layout. A rank's slice W_r[K][H] is stored once, at load time, as
//
//     P[s][kp][c][q] = W_r[2kp + q][4s + c]   s < H/4, kp < ceil(K/2), c < 4, q < 2
//
// (rows past K read as zero). Same bytes as the row-major slice. A 16-byte
// vector holds two consecutive rows of a 4-column strip, column by column,
// so each of its dwords is a (row 2kp, row 2kp+1) bf16 pair that one
// v_dot2c_f32_bf16 multiplies by the matching pair of x. A strip's K rows
// are K*8 contiguous bytes: a wave streams 128 rows of a strip per 1 KB
// load, and one workgroup reduces whole strips over K, so no partial leaves
// the workgroup.
//
// decode_stream: one launch per decode step. Workgroup g of G owns strips
// g, g+G, g+2G, ... (NS of them: H/4 strips spread evenly, one workgroup
// per CU at the page-1 shapes) for every point of the step, and keeps the
// hidden state of its columns in registers for the whole step. It runs
//   - NS*WPS compute waves: WPS waves share a strip, interleaving its
//     1 KB row blocks. Each wave streams its blocks of every point through
//     two banks of SL 16-byte loads per lane: while one bank is multiplied,
//     the other is in flight, and a consumed bank is refilled at once with
//     the blocks two segments ahead, across point boundaries. The bank
//     loads are never conditional: blocks past a strip (or past the step)
//     go through a buffer descriptor whose range makes them read zero
//     without touching memory, so the wait counts stay exact and no point
//     boundary drains the pipeline.
//   - one control wave: stages each point's x into LDS with direct
//     global->LDS loads (x of the next point of the same kind is staged
//     while the current one is multiplied), and at the end of each point
//     sums the compute waves' partials, writes the rank's partial to its
//     slot, forms the ring-order sum of the N ranks' values plus the
//     residual, and keeps the result as the next residual.
//
// Point order. The hidden state is chained element by element (a point's
// residual is the previous point's output at the same element), which the
// ownership of columns by one workgroup preserves without any grid-wide
// synchronisation. With `serial` set, the step also emulates a model in
// which each point's activation is a function of the whole previous hidden
// state: after point j every workgroup publishes its completion, and point
// j+1's x is staged only once all workgroups have completed point j (a
// flag barrier; needs a cooperative launch). The results are the same bits
// in both orders.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tp_device.h"
#include "tp_internal.h"

namespace {

using namespace tpdev;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;

// ------------------------------------------------------------- packing --

// P[l][s][kp][c][q] = W[l][2kp+q][4s+c]: one 16-byte output vector per thread.
__global__ void pack_pairs_kernel(const uint16_t* __restrict__ w, uint16_t* __restrict__ p,
                                  int64_t layers, int64_t K, int64_t H) {
    const int64_t strips = H / 4;
    const int64_t kh = (K + 1) / 2;
    const int64_t per_layer = strips * kh;
    const int64_t total = layers * per_layer;
    for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < total;
         v += (int64_t)gridDim.x * blockDim.x) {
        const int64_t l = v / per_layer;
        const int64_t rem = v - l * per_layer;
        const int64_t s = rem / kh;
        const int64_t kp = rem - s * kh;
        const uint16_t* r0 = w + (l * K + 2 * kp) * H + 4 * s;
        uint16_t a[4], b[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            a[c] = r0[c];
            b[c] = 2 * kp + 1 < K ? r0[H + c] : (uint16_t)0;
        }
        u32x4_t out;
        out.x = a[0] | ((uint32_t)b[0] << 16);
        out.y = a[1] | ((uint32_t)b[1] << 16);
        out.z = a[2] | ((uint32_t)b[2] << 16);
        out.w = a[3] | ((uint32_t)b[3] << 16);
        *reinterpret_cast<u32x4_t*>(p + v * 8) = out;
    }
}

// ------------------------------------------------------- decode step --

constexpr int kStreamMaxWaves = 16;   // 1 control + up to 15 compute waves
constexpr int kStreamMaxNS = 15;      // strips per workgroup
constexpr int kBlockBytes = 1024;     // one wave load: 64 lanes x 16 bytes = 128 rows of a strip

struct StreamArgs {
    const uint16_t* x0;     // x_attn [L][B][K0]
    const uint16_t* x1;     // x_ffn  [L][B][K1]
    const uint16_t* w0;     // packed w_o    [L][S][Kv0][8] (16-byte vectors)
    const uint16_t* w1;     // packed w_down [L][S][Kv1][8]
    const uint32_t* sc0;    // MX weights: scales of w_o [L][S][K0/32] (4 columns' E8M0 bytes)
    const uint32_t* sc1;    // MX weights: scales of w_down [L][S][K1/32]
    float* slots;           // [L][2][N][B][H]
    float* hidden;          // [B][H]
    uint32_t* flags;        // serial order: G completion words, then the exit counter
    uint32_t* err;          // error word (bit 0: a bounded wait timed out)
    int32_t H, S, NS, WPS;
    int32_t K0, K1, Kh0, Kh1;
    int32_t Kv0, Kv1;       // 16-byte weight vectors per strip per point kind
    int32_t bpw0, bpw1;     // row blocks per compute wave per point (same for every wave)
    int32_t layers, n_ranks, rank, chunk;
    int32_t xoff1;          // dword offset of the second x buffer in LDS
    int32_t xdwords;        // total LDS dwords of the x buffers
    int32_t xpair;          // FLAT: dword offset of the second pair of x buffers
    uint32_t spin_limit;
};

// Flag words (serial order): [0, G) completion of each workgroup (G <= 256),
// then the exit counter on a line of its own.
constexpr int kFlagExit = 1024;

// Hidden-state elements of a workgroup (NS * 4 * B) held per control lane:
// at most 3, so the control wave's registers stay few (the host keeps NS
// small enough).
constexpr int stream_elems_per_lane(int b) {
    return (kStreamMaxNS * 4 * b + 63) / 64 < 3 ? (kStreamMaxNS * 4 * b + 63) / 64 : 3;
}

// An E8M0 block scale as the scale operand of gfx950's scaled conversions
// (v_cvt_scalef32_pk_bf16_fp8 / _fp4). Those read only the binary32's
// exponent field, as an E8M0 value: field E scales by 2^(E-127), field 0 by
// 2^-127, field 255 gives NaN, and the mantissa is ignored; the product is
// rounded to bf16 nearest-even (measured over every code at scales 2^-127 ..
// 2^120). So the byte goes straight into the exponent field.
__device__ __forceinline__ float mx_scale_f32(uint32_t e) { return __uint_as_float(e << 23); }

// PART: the partials only (tp_rowparallel_partials_packed): the control wave
// writes each point's partial to slots[j] ([L][2][b][H]) and forms no ring
// sum; the hidden state is neither read nor written.
// WF: the weights' element format (tp_weight_format). A 16-byte vector holds
// 4 columns of a strip and RV = 2 (bf16), 4 (FP8) or 8 (FP4) consecutive
// rows per column; with MX weights every 32 rows of a column share a scale.
template <int B, int SL, bool SERIAL, bool PART = false, int WF = TP_WEIGHTS_BF16, bool FLAT = false>
__global__ __launch_bounds__(kStreamMaxWaves * 64) void decode_stream(StreamArgs a) {
    extern __shared__ __align__(16) uint32_t xs[];             // x buffers, bf16 pairs
    // the compute waves' sums of a point: per point parity, or (FLAT) per
    // point mod 4
    constexpr int NRED = FLAT ? 4 : 2;
    __shared__ float red[NRED][kStreamMaxWaves - 1][B * 4];
    // FLAT: arrivals of the compute waves per red buffer, points consumed by
    // the control wave, points whose x is staged
    __shared__ int fl[6];
    constexpr int kFlConsumed = 4, kFlXready = 5;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = blockIdx.x, G = gridDim.x;
    const int n_points = 2 * a.layers;
    const int len = B * a.H;
    // the LDS x buffer of point j: one per kind, or (FLAT) two per kind,
    // used by every other point of that kind
    auto xoff_of = [&](int j) {
        return (j & 1 ? a.xoff1 : 0) + (FLAT && (j & 2) ? a.xpair : 0);
    };

    // zero the x buffers: rows past a point's K are multiplied by zero
    // weights and must hold finite values
    for (int i = tid; i < a.xdwords; i += blockDim.x) xs[i] = 0u;
    if (tid < 6) fl[tid] = 0;
    __syncthreads();

    if (wave == 0) {
        // ---------------------------------------------------- control wave
        __builtin_amdgcn_s_setprio(3);
        constexpr int EQ_MAX = stream_elems_per_lane(B);
        const int n_el = a.NS * 4 * B;
        // element e = (b * NS + si) * 4 + c -> hidden index b*H + 4*(g + si*G) + c
        int idx[EQ_MAX];
        bool valid[EQ_MAX];
        float h[EQ_MAX];
        float oth[EQ_MAX][8];
#pragma unroll
        for (int q = 0; q < EQ_MAX; ++q) {
            const int e = lane + 64 * q;
            const int c = e & 3, si = (e >> 2) % a.NS, b = (e >> 2) / a.NS;
            const int s = g + si * G;
            valid[q] = e < n_el && s < a.S;
            idx[q] = valid[q] ? b * a.H + 4 * s + c : 0;
            h[q] = valid[q] && !PART ? a.hidden[idx[q]] : 0.f;
        }
        // the other ranks' values of point j, in ring order from the
        // element's chunk: every load is issued, unconditionally, before any
        // is used (one memory round trip); the entries that are not needed
        // (past N, our own rank, lanes without an element) read zero through
        // the buffer range without touching memory
        auto fetch_others = [&](int j, float (&oth)[EQ_MAX][8]) {
            if (PART) return;
            const float* slot = a.slots + (int64_t)j * a.n_ranks * len;
            const __amdgpu_buffer_rsrc_t rsl = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<float*>(slot), (short)0, a.n_ranks * len * 4, kBufferRsrcWord3);
#pragma unroll
            for (int q = 0; q < EQ_MAX; ++q) {
                const int cidx = idx[q] / a.chunk;
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    int r = cidx + u;
                    r = r >= a.n_ranks ? r - a.n_ranks : r;
                    const bool need = valid[q] && u < a.n_ranks && r != a.rank;
                    const uint32_t off = need ? (uint32_t)(r * len + idx[q]) * 4u : 0xfffffff0u;
                    oth[q][u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsl, off, 0, 0));
                }
            }
        };
        // x of point j -> its buffer (j & 1), as 1 KB direct-to-LDS copies;
        // lanes past the end re-read the last vector into the buffer's pad
        auto stage_x = [&](int j) {
            const int t = j & 1, l = j >> 1;
            const int K = t ? a.K1 : a.K0;
            const uint16_t* src = (t ? a.x1 : a.x0) + (int64_t)l * B * K;
            const int n16 = B * K / 8;
            uint32_t* dst = xs + xoff_of(j);
            // start at a workgroup-dependent piece, so that the workgroups do
            // not all read the same lines of x at the same moment
            const int pieces = (n16 + 63) / 64;
            const int rot = g % pieces;
            for (int q = 0; q < pieces; ++q) {
                const int v0 = (q + rot < pieces ? q + rot : q + rot - pieces) * 64;
                int v = v0 + lane;
                v = v < n16 ? v : n16 - 1;
                __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src + (int64_t)v * 8),
                                                 (lds_void_t*)(dst + v0 * 4), 16, 0, 0);
            }
        };
        uint32_t* err = a.err;
        int ok = 1;
        // serial order: wait until every workgroup has completed point j
        // (the G <= 256 completion words, 4 per lane; words past G read as
        // complete)
        auto grid_wait = [&](int j) {
            if (!ok) return;
            const uint32_t target = (uint32_t)(j + 1);
            const __amdgpu_buffer_rsrc_t rf = dev_rsrc(a.flags, (uint32_t)G * 4);
            for (uint32_t n = 0;; ++n) {
                uint32_t mn = 0xffffffffu;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t f = ld_dev_u32_buf(rf, (uint32_t)(lane + 64 * i) * 4);
                    mn = lane + 64 * i < G && f < mn ? f : mn;
                }
                if (__builtin_amdgcn_ballot_w64(mn < target) == 0) return;
                if ((n & 15) == 15 && __builtin_amdgcn_readfirstlane(ld_dev_u32(err))) { ok = 0; return; }
                if (n >= a.spin_limit) {
                    if (lane == 0) __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    ok = 0;
                    return;
                }
                __builtin_amdgcn_s_sleep(1);
            }
        };

        // point j's partial from the compute waves' sums in red[rb], to the
        // rank's slot, then the ring-order sum of the N ranks' values plus the
        // residual
        auto ring = [&](int j, int rb, const float (&oth)[EQ_MAX][8]) {
            float* slot = PART ? a.slots + (int64_t)j * len
                               : a.slots + (int64_t)j * a.n_ranks * len + (int64_t)a.rank * len;
#pragma unroll
            for (int q = 0; q < EQ_MAX; ++q) {
#pragma clang fp contract(off)
                if (!valid[q]) continue;
                const int e = lane + 64 * q;
                const int c = e & 3, si = (e >> 2) % a.NS, b = (e >> 2) / a.NS;
                float v = red[rb][si * a.WPS][b * 4 + c];
                for (int wi = 1; wi < a.WPS; ++wi) v += red[rb][si * a.WPS + wi][b * 4 + c];
                slot[idx[q]] = v;
                if (PART) continue;
                // ring order: chunk c starts at rank c, then c+1, ... (mod N)
                const int cidx = idx[q] / a.chunk;
                float sum = 0.f;
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    if (u < a.n_ranks) {
                        int r = cidx + u;
                        if (r >= a.n_ranks) r -= a.n_ranks;
                        const float val = r == a.rank ? v : oth[q][u];
                        sum = u == 0 ? val : sum + val;
                    }
                }
                h[q] = sum + h[q];
            }
        };

        if constexpr (FLAT) {
            // The compute waves deposit each point's sums in red[j % 4] and
            // count themselves; nothing meets at a barrier. After point j's
            // ring sum the wave issues x of point j+4 (into point j's buffer:
            // every compute wave is done with it) and then the other ranks'
            // values of point j+2, into the register set point j used. The
            // ring sum of point j+2 waits for those values, and so (loads
            // complete in order) for that x too: x of point j+4 is marked
            // staged after it. Two points of work cover every round trip.
            const int ncw = (int)(blockDim.x / 64) - 1;
            const int npre = n_points < 4 ? n_points : 4;
            float othA[EQ_MAX][8], othB[EQ_MAX][8];
            for (int j = 0; j < npre; ++j) stage_x(j);
            fetch_others(0, othA);
            if (n_points > 1) fetch_others(1, othB);
            wait_mem();
            if (lane == 0) lds_st(&fl[kFlXready], npre);
            __syncthreads();  // start
            auto point = [&](int j, float (&o)[EQ_MAX][8]) {
                wait_flag(&fl[j & 3], ncw * (j / 4 + 1), a.err);  // every compute wave's sums of point j
                lds_wait();
                ring(j, j & 3, o);
                // the values are in (their first load waited for, and so
                // everything issued before it)
                asm volatile("" ::"v"(o[0][0]) : "memory");
                lds_wait();
                if (lane == 0) {
                    lds_st(&fl[kFlConsumed], j + 1);  // red[j % 4] may be refilled
                    // x of point j+2 (issued before the values just used)
                    if (j >= 2 && j + 2 < n_points) lds_st(&fl[kFlXready], j + 3);
                }
                if (j + 4 < n_points) stage_x(j + 4);
                if (j + 2 < n_points) fetch_others(j + 2, o);
            };
            for (int j = 0; j < n_points; j += 2) {
                point(j, othA);
                if (j + 1 < n_points) point(j + 1, othB);
            }
            wait_mem();
        } else {
        stage_x(0);
        if (!SERIAL && n_points > 1) stage_x(1);
        fetch_others(0, oth);
        wait_mem();
        __syncthreads();  // start: x of the first point(s) is in LDS

        for (int j = 0; j < n_points; ++j) {
            __syncthreads();  // P_j: the compute waves' sums of point j are in red[j & 1]
            ring(j, j & 1, oth);
            if (j + 1 < n_points) fetch_others(j + 1, oth);
            if (SERIAL) {
                if (j + 1 < n_points) {
                    wait_mem();
                    if (lane == 0) st_dev_u32(a.flags + g, (uint32_t)(j + 1));
                    grid_wait(j);
                    stage_x(j + 1);
                    wait_mem();
                    __syncthreads();  // A_{j+1}: x of point j+1 is in LDS
                }
            } else {
                if (j + 2 < n_points) stage_x(j + 2);
                wait_mem();  // x staged before P_{j+1}; needed from P_{j+1} on
            }
        }
        }
#pragma unroll
        for (int q = 0; q < EQ_MAX; ++q)
            if (valid[q] && !PART) a.hidden[idx[q]] = h[q];
        if (SERIAL) {
            // the last workgroup to leave clears the flags for the next launch
            wait_mem();
            int last = 0;
            if (lane == 0) last = add_dev_u32(a.flags + kFlagExit, 1u) == (uint32_t)G - 1;
            if (__builtin_amdgcn_readfirstlane(last)) {
                for (int w0 = lane; w0 < G; w0 += 64) st_dev_u32(a.flags + w0, 0u);
                if (lane == 0) st_dev_u32(a.flags + kFlagExit, 0u);
            }

        }
    } else {
        // --------------------------------------------------- compute waves
        const int cw = wave - 1;
        const int si = cw / a.WPS, wi = cw - si * a.WPS;
        const bool active = si < a.NS && g + si * G < a.S;
        const int s = g + si * G;
        const int voff = lane * 16 + wi * kBlockBytes;  // + block offset: all in the VGPR
                                                        // offset, which the range check covers
        const int stride = a.WPS * kBlockBytes;

        constexpr int RV = WF == TP_WEIGHTS_MXFP8 ? 4 : WF == TP_WEIGHTS_MXFP4 ? 8 : 2;
        constexpr int VPB = kMxBlock / RV;  // vectors per scale block (MX)
        auto bpw = [&](int j) { return (j & 1) ? a.bpw1 : a.bpw0; };
        // A wave takes row blocks m = 0 .. bpw-1 of its strip in every point
        // (block wi + m * WPS of the strip); bpw is the same for every wave,
        // so all waves meet the same point boundaries.

        // The descriptors of point j's weight (and MX scale) stream of this
        // wave's strip: an empty range past the step or for an idle wave
        // (loads through it read zeros without a memory access).
        auto wdesc = [&](int j) {
            const int t = j & 1, l = j >> 1;
            const bool live = active && j < n_points;
            const int kv = t ? a.Kv1 : a.Kv0;
            const uint16_t* base = (t ? a.w1 : a.w0) + ((int64_t)l * a.S + s) * kv * 8;
            return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(live ? base : a.w0), (short)0,
                                                     live ? kv * 16 : 0, kBufferRsrcWord3);
        };
        auto sdesc = [&](int j) {
            const int t = j & 1, l = j >> 1;
            const bool live = active && j < n_points;
            const int nsb = (t ? a.Kv1 : a.Kv0) / VPB;
            const uint32_t* sb = (t ? a.sc1 : a.sc0) + ((int64_t)l * a.S + s) * nsb;
            return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(live ? sb : a.sc0), (short)0,
                                                     live ? nsb * 4 : 0, kBufferRsrcWord3);
        };
        auto load_w = [&](__amdgpu_buffer_rsrc_t rs, int m) {
            return __builtin_bit_cast(u32x4_t,
                                      __builtin_amdgcn_raw_buffer_load_b128(rs, voff + m * stride, 0, kCachePolicyNT));
        };
        auto load_s = [&](__amdgpu_buffer_rsrc_t rsc, int m) {
            const int v = (wi + m * a.WPS) * 64 + lane;
            return __builtin_amdgcn_raw_buffer_load_b32(rsc, (v / VPB) * 4, 0, 0);
        };

        float acc[B][4];
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[b][c] = 0.f;
        // one block (16-byte vector per lane) of a point into acc: the
        // point's x buffer xb (kh pairs per token), kvt vectors per strip
        auto block = [&](const u32x4_t wq, const uint32_t sw, const uint32_t* xb, int kh, int kvt, int m) {
            const int v = (wi + m * a.WPS) * 64 + lane;  // vector index in the strip
            const uint32_t wd[4] = {wq.x, wq.y, wq.z, wq.w};
            if constexpr (WF == TP_WEIGHTS_BF16) {
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    const bf16x2_t xv = __builtin_bit_cast(bf16x2_t, xb[b * kh + v]);
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        acc[b][c] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, wd[c]), xv,
                                                                    acc[b][c], false);
                }
            } else {
                // rows RV*v .. RV*v + RV-1 of each column: the codes widened
                // to bf16 pairs with the block scale applied (exact: a
                // power of two times at most 4 significant bits), then the
                // same pair products as the bf16 weights
                constexpr int NP = RV / 2;  // row pairs per vector
                // slots past the strip's vectors read zero weights: any
                // staged x will do, so the index is clamped into the buffer
                const int vx = v < kvt ? v : kvt - 1;
                // the vector's 4 columns widened once, then x token by token
                bf16x2_t wp[4][NP];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const float sc = mx_scale_f32((sw >> (8 * c)) & 0xffu);
                    if constexpr (WF == TP_WEIGHTS_MXFP8) {
                        wp[c][0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wd[c], sc, false);
                        wp[c][1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wd[c], sc, true);
                    } else {
                        wp[c][0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[c], sc, 0);
                        wp[c][1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[c], sc, 1);
                        wp[c][2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[c], sc, 2);
                        wp[c][3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[c], sc, 3);
                    }
                }
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    uint32_t xv[NP];
#pragma unroll
                    for (int q = 0; q < NP; ++q) xv[q] = xb[b * kh + NP * vx + q];
#pragma unroll
                    for (int c = 0; c < 4; ++c)
#pragma unroll
                        for (int q = 0; q < NP; ++q)
                            acc[b][c] = __builtin_amdgcn_fdot2_f32_bf16(
                                wp[c][q], __builtin_bit_cast(bf16x2_t, xv[q]), acc[b][c], false);
                }
            }
        };
        auto point_end = [&](int j) {
#pragma unroll
            for (int b = 0; b < B; ++b)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const float v = wave_sum(acc[b][c]);
                    if (lane == 0) red[j & 1][cw][b * 4 + c] = v;
                    acc[b][c] = 0.f;
                }
            __syncthreads();                                   // P_j
            if (SERIAL && j + 1 < n_points) __syncthreads();   // A_{j+1}
        };

        u32x4_t bank0[SL], bank1[SL];
        uint32_t sbank0[SL], sbank1[SL];  // MX scale words (unused for bf16)
        if constexpr (FLAT) {
            // Small points (a layer's blocks fit one bank): the stream is
            // taken block by block across points, so that a bank's loads are
            // never empty; each register slot is refilled with the block 2 SL
            // further on as soon as it is consumed, so every slot is in
            // flight again before a point's end. No early exit: blocks past
            // the step read zero weights, every path issues the same loads
            // and the compiler's waits stay exact.
            struct Pos {
                int j, m;
            };
            auto step = [&](Pos& c) {
                if (++c.m == bpw(c.j)) {
                    c.m = 0;
                    ++c.j;
                }
            };
            int cur = -1;
            __amdgpu_buffer_rsrc_t rs = wdesc(n_points), rsc = sdesc(n_points);
            auto issue = [&](u32x4_t& wv, uint32_t& sv, Pos& c) {
                if (c.j != cur) {  // descriptors made again only when the point changes
                    cur = c.j;
                    rs = wdesc(c.j);
                    if constexpr (WF != TP_WEIGHTS_BF16) rsc = sdesc(c.j);
                }
                wv = load_w(rs, c.m);
                if constexpr (WF != TP_WEIGHTS_BF16) sv = load_s(rsc, c.m);
                step(c);
            };
            // a point's end without a barrier: the sums go to red[j % 4] once
            // the control wave has consumed point j-4, and the wave counts
            // itself in that buffer's arrivals
            auto deposit = [&](int j) {
                float v[B][4];
#pragma unroll
                for (int b = 0; b < B; ++b)
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        v[b][c] = wave_sum(acc[b][c]);
                        acc[b][c] = 0.f;
                    }
                wait_flag(&fl[kFlConsumed], j - 3, a.err);
                lds_wait();
                if (lane == 0) {
#pragma unroll
                    for (int b = 0; b < B; ++b)
#pragma unroll
                        for (int c = 0; c < 4; ++c) red[j & 3][cw][b * 4 + c] = v[b][c];
                }
                lds_wait();
                if (lane == 0) lds_add(&fl[j & 3], 1);
            };
            int xchk = -1;  // the last point whose x was seen staged
            auto consume = [&](u32x4_t (&bank)[SL], uint32_t (&sbank)[SL], Pos& c, Pos& ci) {
#pragma unroll
                for (int i = 0; i < SL; ++i) {
                    const int j = c.j, t = j & 1;
                    if (j > xchk && j < n_points) {
                        wait_flag(&fl[kFlXready], j + 1, a.err);  // x of point j is in LDS
                        lds_wait();
                        xchk = j;
                    }
                    block(bank[i], sbank[i], xs + xoff_of(j), t ? a.Kh1 : a.Kh0, t ? a.Kv1 : a.Kv0, c.m);
                    issue(bank[i], sbank[i], ci);
                    step(c);
                    if (c.j != j && j < n_points) deposit(j);  // the point's last block
                }
            };
            Pos ci{0, 0}, cc{0, 0};
#pragma unroll
            for (int i = 0; i < SL; ++i) issue(bank0[i], sbank0[i], ci);
#pragma unroll
            for (int i = 0; i < SL; ++i) issue(bank1[i], sbank1[i], ci);
            __syncthreads();  // start
            while (cc.j < n_points) {  // (past the last point the blocks are zero)
                consume(bank0, sbank0, cc, ci);
                consume(bank1, sbank1, cc, ci);
            }
        } else {
            // Segments: blocks m0 .. m0+SL-1 of one point per bank (the
            // point's remaining blocks, the rest of the bank reading zero);
            // a point ends after its last segment, once the bank is refilled.
            struct Cursor {
                int j, m0;
            };
            auto advance = [&](Cursor& cu) {
                cu.m0 += SL;
                if (cu.m0 >= bpw(cu.j)) {
                    cu.j += 1;
                    cu.m0 = 0;
                }
            };
            auto issue = [&](u32x4_t (&bank)[SL], uint32_t (&sbank)[SL], const Cursor& cu) {
                const __amdgpu_buffer_rsrc_t rs = wdesc(cu.j);
#pragma unroll
                for (int i = 0; i < SL; ++i) bank[i] = load_w(rs, cu.m0 + i);
                if constexpr (WF != TP_WEIGHTS_BF16) {
                    const __amdgpu_buffer_rsrc_t rsc = sdesc(cu.j);
#pragma unroll
                    for (int i = 0; i < SL; ++i) sbank[i] = load_s(rsc, cu.m0 + i);
                }
            };
            auto consume = [&](const u32x4_t (&bank)[SL], const uint32_t (&sbank)[SL], const Cursor& cu) {
                const int t = cu.j & 1;
                const uint32_t* xb = xs + xoff_of(cu.j);
                const int kh = t ? a.Kh1 : a.Kh0, kvt = t ? a.Kv1 : a.Kv0;
#pragma unroll
                for (int i = 0; i < SL; ++i) block(bank[i], sbank[i], xb, kh, kvt, cu.m0 + i);
            };
            Cursor ci{0, 0}, cc{0, 0};
            issue(bank0, sbank0, ci);
            advance(ci);
            issue(bank1, sbank1, ci);
            advance(ci);
            __syncthreads();  // start
            while (cc.j < n_points) {
                {
                    consume(bank0, sbank0, cc);
                    const int j = cc.j;
                    const bool last = cc.m0 + SL >= bpw(j);
                    advance(cc);
                    issue(bank0, sbank0, ci);
                    advance(ci);
                    if (last) point_end(j);
                }
                {
                    const bool live = cc.j < n_points;
                    int j = cc.j;
                    bool last = false;
                    if (live) {
                        consume(bank1, sbank1, cc);
                        last = cc.m0 + SL >= bpw(j);
                        advance(cc);
                    }
                    issue(bank1, sbank1, ci);
                    advance(ci);
                    if (last) point_end(j);
                }
            }
        }
    }
}

typedef void (*stream_fn)(StreamArgs);

template <int SL, bool SERIAL, bool PART, int WF, bool FLAT = false>
stream_fn stream_kernel_for(int b) {
    switch (b) {
        case 1: return decode_stream<1, SL, SERIAL, PART, WF, FLAT>;
        case 2: return decode_stream<2, SL, SERIAL, PART, WF, FLAT>;
        case 3: return decode_stream<3, SL, SERIAL, PART, WF, FLAT>;
        case 4: return decode_stream<4, SL, SERIAL, PART, WF, FLAT>;
        case 5: return decode_stream<5, SL, SERIAL, PART, WF, FLAT>;
        case 6: return decode_stream<6, SL, SERIAL, PART, WF, FLAT>;
        case 7: return decode_stream<7, SL, SERIAL, PART, WF, FLAT>;
        case 8: return decode_stream<8, SL, SERIAL, PART, WF, FLAT>;
    }
    return nullptr;
}

// 8-load banks only for batch <= 4 (beyond, the registers would spill).
template <bool SERIAL, bool PART, int WF, bool FLAT = false>
stream_fn stream_kernel_sl8(int b) {
    switch (b) {
        case 1: return decode_stream<1, 8, SERIAL, PART, WF, FLAT>;
        case 2: return decode_stream<2, 8, SERIAL, PART, WF, FLAT>;
        case 3: return decode_stream<3, 8, SERIAL, PART, WF, FLAT>;
        case 4: return decode_stream<4, 8, SERIAL, PART, WF, FLAT>;
    }
    return nullptr;
}

// mode 0: dataflow point order, 1: serial point order, 2: partials only,
// 3: dataflow order with the stream taken block by block across points
template <int WF>
stream_fn stream_kernel_wf(int b, int sl, int mode) {
    if (sl == 4)
        return mode == 1 ? stream_kernel_for<4, true, false, WF>(b)
               : mode == 2 ? stream_kernel_for<4, false, true, WF>(b)
               : mode == 3 ? stream_kernel_for<4, false, false, WF, true>(b)
                           : stream_kernel_for<4, false, false, WF>(b);
    if constexpr (WF == TP_WEIGHTS_BF16) {
        if (sl == 8)
            return mode == 1 ? stream_kernel_sl8<true, false, WF>(b)
                   : mode == 2 ? stream_kernel_sl8<false, true, WF>(b)
                   : mode == 3 ? stream_kernel_sl8<false, false, WF, true>(b)
                               : stream_kernel_sl8<false, false, WF>(b);
    }
    return nullptr;
}

stream_fn stream_kernel(int b, int sl, int mode, int wf) {
    switch (wf) {
        case TP_WEIGHTS_BF16: return stream_kernel_wf<TP_WEIGHTS_BF16>(b, sl, mode);
        case TP_WEIGHTS_MXFP8: return stream_kernel_wf<TP_WEIGHTS_MXFP8>(b, sl, mode);
        case TP_WEIGHTS_MXFP4: return stream_kernel_wf<TP_WEIGHTS_MXFP4>(b, sl, mode);
    }
    return nullptr;
}

// ------------------------------------------------------- MX weights --

// Static conversion of bf16 weights to an MX format ("Hosting Qwen on
// Blackwell", Quantization: the weights are converted once to MXFP8). One
// thread per block of 32 rows of a column: the block scale
// E = floor(log2(max |w|)) - emax + 127 (clamped to [0, 254]; 0 for an
// all-zero block; 255 and zero codes for a block holding a NaN or an
// infinity), then each element w * 2^(127-E) rounded to the nearest
// element value, ties to the even code, saturating at the largest finite
// value, sign kept. Interchange layout: codes [L][K][H] (FP8) or
// [L][K/2][H] (FP4, the even row in the low nibble), scales [L][K/32][H].
template <int WF>
__global__ void mx_quantize_kernel(const uint16_t* __restrict__ w, uint8_t* __restrict__ codes,
                                   uint8_t* __restrict__ scales, int64_t layers, int64_t K, int64_t H) {
    constexpr int emax = WF == TP_WEIGHTS_MXFP8 ? 8 : 2;
    const int64_t nblk = K / kMxBlock;
    const int64_t total = layers * nblk * H;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t n = t % H, kb = (t / H) % nblk, l = t / (H * nblk);
        const uint16_t* col = w + (l * K + kb * kMxBlock) * H + n;
        uint32_t amax = 0;  // |w| as binary32 bits: ordered like the values
        bool finite = true;
        for (int i = 0; i < kMxBlock; ++i) {
            const uint32_t u = ((uint32_t)col[(int64_t)i * H] << 16) & 0x7fffffffu;
            if (u >= 0x7f800000u) finite = false;
            amax = u > amax ? u : amax;
        }
        uint32_t E;
        if (!finite) {
            E = 255;
        } else if (amax == 0) {
            E = 0;
        } else {
            // floor(log2(amax)): the exponent field, or for a subnormal the
            // position of the top mantissa bit
            const int fl = (amax >> 23) ? (int)(amax >> 23) - 127 : (31 - __clz((int)amax)) - 149;
            const int se = fl - emax + 127;
            E = se < 0 ? 0u : se > 254 ? 254u : (uint32_t)se;
        }
        scales[(l * nblk + kb) * H + n] = (uint8_t)E;
        // 2^(127-E), an exact binary32 for E in [0, 254]
        const float inv = __uint_as_float(E >= 1 && E <= 253 ? (254u - E) << 23 : E == 0 ? 0x7f000000u : 0x00400000u);
        uint8_t prev = 0;
        for (int i = 0; i < kMxBlock; ++i) {
            const uint32_t wb = (uint32_t)col[(int64_t)i * H] << 16;
            uint32_t code = 0;
            if (E != 255) {
                const float v = __uint_as_float(wb) * inv;  // exact: a power-of-two scaling
                const uint32_t sign = __float_as_uint(v) >> 31;
                const float av = __builtin_fabsf(v);
                const uint32_t ua = __float_as_uint(av);
                if (WF == TP_WEIGHTS_MXFP8) {
                    if (av >= 448.0f) {
                        code = 0x7e;
                    } else if (av < 0.015625f) {  // below 2^-6: multiples of 2^-9
                        code = (uint32_t)__builtin_rintf(av * 512.0f);
                    } else {  // 3 mantissa bits, nearest even
                        code = ((ua + 0x7ffffu + ((ua >> 20) & 1u)) >> 20) - (120u << 3);
                    }
                    code |= sign << 7;
                } else {
                    if (av >= 6.0f) {
                        code = 0x7;
                    } else if (av < 1.0f) {  // below 1: multiples of 0.5
                        code = (uint32_t)__builtin_rintf(av * 2.0f);
                    } else {  // 1 mantissa bit, nearest even
                        code = ((ua + 0x1fffffu + ((ua >> 22) & 1u)) >> 22) - (126u << 1);
                    }
                    code |= sign << 3;
                }
            }
            const int64_t k = kb * kMxBlock + i;
            if (WF == TP_WEIGHTS_MXFP8) {
                codes[(l * K + k) * H + n] = (uint8_t)code;
            } else if (i & 1) {
                codes[(l * (K / 2) + k / 2) * H + n] = (uint8_t)(prev | (code << 4));
            } else {
                prev = (uint8_t)code;
            }
        }
    }
}

// Interchange -> the stream's layout, per layer: the 16-byte code vectors
// [S][Kv][4 columns][RV rows] (FP8: one byte per row; FP4: one byte per two
// rows, the even row in the low nibble, as in the interchange), then the
// scale words [S][K/32] holding the block's 4 column scales, column c in
// byte c. One 16-byte vector or one scale word per thread.
template <int WF>
__global__ void mx_pack_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                               uint8_t* __restrict__ out, int64_t layers, int64_t K, int64_t H) {
    constexpr int RV = WF == TP_WEIGHTS_MXFP8 ? 4 : 8;
    constexpr int BPV = WF == TP_WEIGHTS_MXFP8 ? 4 : 4;  // code bytes per column per vector
    const int64_t S = H / 4, kv = K / RV, nblk = K / kMxBlock;
    const int64_t nvec = layers * S * kv, total = nvec + layers * S * nblk;
    const int64_t crow = WF == TP_WEIGHTS_MXFP8 ? K : K / 2;  // interchange code rows per layer
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        if (t < nvec) {
            const int64_t v = t % kv, s = (t / kv) % S, l = t / (kv * S);
            uint32_t d[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                uint32_t word = 0;
#pragma unroll
                for (int j = 0; j < BPV; ++j)  // interchange row BPV*v + j of column 4s + c
                    word |= (uint32_t)codes[(l * crow + BPV * v + j) * H + 4 * s + c] << (8 * j);
                d[c] = word;
            }
            *reinterpret_cast<u32x4_t*>(out + t * 16) = u32x4_t{d[0], d[1], d[2], d[3]};
        } else {
            const int64_t u = t - nvec;
            const int64_t kb = u % nblk, s = (u / nblk) % S, l = u / (nblk * S);
            const uint8_t* e = scales + (l * nblk + kb) * H + 4 * s;
            *reinterpret_cast<uint32_t*>(out + nvec * 16 + u * 4) =
                (uint32_t)e[0] | ((uint32_t)e[1] << 8) | ((uint32_t)e[2] << 16) | ((uint32_t)e[3] << 24);
        }
    }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

// Geometry of the streamed step for a plan (host side; see tp_internal.h).
bool tp_stream_geometry(const tp_plan_s* p, StreamGeom* g) {
    if (p->batch < 1 || p->batch > kStripMaxBatch || p->n_ranks > 8) return false;
    if (p->hidden % 4) return false;
    const int64_t k0 = p->k_attn / p->n_ranks, k1 = p->inter / p->n_ranks;
    if (k0 < 2 || k1 < 2 || (k0 & 1) || (k1 & 1)) return false;
    const int rv = stream_rows_per_vec(p->weight_format);
    if (p->weight_format != TP_WEIGHTS_BF16 && (k0 % kMxBlock || k1 % kMxBlock)) return false;
    if ((k0 * p->batch) % 8 || (k1 * p->batch) % 8) return false;
    const int64_t S = p->hidden / 4;
    int64_t ns = (S + kTargetCUs - 1) / kTargetCUs;
    if (ns > kStreamMaxNS) ns = kStreamMaxNS;
    const int64_t G = (S + ns - 1) / ns;
    if (ns * 4 * p->batch > 64 * stream_elems_per_lane(p->batch)) return false;
    const int wps = (int)((kStreamMaxWaves - 1) / ns);
    // 8-load banks (more bytes in flight) where the registers allow it (bf16
    // weights up to 4 tokens; MX weights, whose vectors are widened in
    // registers, always take 4)
    const int sl = p->segment_loads == 4 || p->batch > 4 || p->weight_format != TP_WEIGHTS_BF16 ? 4 : 8;
    const int64_t kh0 = k0 / 2, kh1 = k1 / 2;
    const int64_t kv0 = k0 / rv, kv1 = k1 / rv;  // (K even; a multiple of 32 for MX)
    const int64_t nb0 = (kv0 + 63) / 64, nb1 = (kv1 + 63) / 64;
    const int64_t bpw0 = (nb0 + wps - 1) / wps, bpw1 = (nb1 + wps - 1) / wps;
    // x buffer t: B*Kh_t dwords staged in 1 KB pieces, and every pair index a
    // compute lane reads (rv/2 pairs per vector, up to the last block of its
    // last segment)
    auto xbuf = [&](int64_t kh, int64_t bpw) {
        const int64_t n16 = p->batch * kh * 4 / 16;
        const int64_t staged = (n16 + 63) / 64 * 256;
        const int64_t segs = (bpw + sl - 1) / sl;
        // (MX weights: the compute lanes clamp their x index to the last vector)
        const int64_t read = p->weight_format != TP_WEIGHTS_BF16
                                 ? p->batch * kh
                                 : (p->batch - 1) * kh + ((wps - 1) + (segs * sl - 1) * wps) * 64 + 64;
        const int64_t d = staged > read ? staged : read;
        return (d + 255) / 256 * 256;
    };
    const int64_t xb0 = xbuf(kh0, bpw0), xb1 = xbuf(kh1, bpw1);
    g->xoff1 = (int32_t)xb0;
    g->xdwords = (int32_t)(xb0 + xb1);
    g->grid = (int32_t)G;
    g->ns = (int32_t)ns;
    g->wps = wps;
    g->sl = sl;
    g->block = (int32_t)(1 + ns * wps) * 64;
    g->kh0 = (int32_t)kh0;
    g->kh1 = (int32_t)kh1;
    g->kv0 = (int32_t)kv0;
    g->kv1 = (int32_t)kv1;
    g->bpw0 = (int32_t)bpw0;
    g->bpw1 = (int32_t)bpw1;
    g->lds_bytes = g->xdwords * 4;
    return g->lds_bytes <= kStreamMaxLdsBytes;
}

int64_t tp_stream_packed_bytes(const tp_plan_s* p, int point, int64_t n_layers) {
    const int64_t K = (point == TP_POINT_ATTN_OUT ? p->k_attn : p->inter) / p->n_ranks;
    const int64_t S = p->hidden / 4;
    if (p->weight_format == TP_WEIGHTS_BF16) return n_layers * S * ((K + 1) / 2) * 16;
    const int rv = stream_rows_per_vec(p->weight_format);
    return n_layers * S * (K / rv * 16 + K / kMxBlock * 4);
}

tp_status tp_mx_quantize(const tp_plan_s* p, int point, int n_layers, const void* w, void* codes,
                         void* scales, void* stream) {
    const int64_t K = (point == TP_POINT_ATTN_OUT ? p->k_attn : p->inter) / p->n_ranks;
    if (K % kMxBlock) return TP_ERR_UNSUPPORTED;
    const int64_t total = (int64_t)n_layers * (K / kMxBlock) * p->hidden;
    if (total == 0) return TP_OK;
    const int64_t blocks = (total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536;
    auto k = p->weight_format == TP_WEIGHTS_MXFP8 ? mx_quantize_kernel<TP_WEIGHTS_MXFP8>
                                                  : mx_quantize_kernel<TP_WEIGHTS_MXFP4>;
    hipLaunchKernelGGL(k, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       static_cast<const uint16_t*>(w), static_cast<uint8_t*>(codes),
                       static_cast<uint8_t*>(scales), (int64_t)n_layers, K, p->hidden);
    return tp_launch_status(stream);
}

tp_status tp_mx_pack(const tp_plan_s* p, int point, int n_layers, const void* codes, const void* scales,
                     void* w_packed, void* stream) {
    const int64_t K = (point == TP_POINT_ATTN_OUT ? p->k_attn : p->inter) / p->n_ranks;
    if (K % kMxBlock || p->hidden % 4) return TP_ERR_UNSUPPORTED;
    const int rv = stream_rows_per_vec(p->weight_format);
    const int64_t S = p->hidden / 4;
    const int64_t total = (int64_t)n_layers * S * (K / rv + K / kMxBlock);
    if (total == 0) return TP_OK;
    const int64_t blocks = (total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536;
    auto k = p->weight_format == TP_WEIGHTS_MXFP8 ? mx_pack_kernel<TP_WEIGHTS_MXFP8>
                                                  : mx_pack_kernel<TP_WEIGHTS_MXFP4>;
    hipLaunchKernelGGL(k, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       static_cast<const uint8_t*>(codes), static_cast<const uint8_t*>(scales),
                       static_cast<uint8_t*>(w_packed), (int64_t)n_layers, K, p->hidden);
    return tp_launch_status(stream);
}

tp_status tp_pack_pairs(const tp_plan_s* p, int point, int n_layers, const void* w, void* w_packed,
                        void* stream) {
    const int64_t K = (point == TP_POINT_ATTN_OUT ? p->k_attn : p->inter) / p->n_ranks;
    const int64_t total = (int64_t)n_layers * ((K + 1) / 2) * (p->hidden / 4);
    if (total == 0) return TP_OK;
    const int64_t blocks = (total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536;
    hipLaunchKernelGGL(pack_pairs_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       static_cast<const uint16_t*>(w), static_cast<uint16_t*>(w_packed),
                       (int64_t)n_layers, K, p->hidden);
    return tp_launch_status(stream);
}

tp_status tp_decode_stream(const tp_plan_s* p, int32_t n_layers, int32_t rank, const void* x_attn,
                           const void* w_o_packed, const void* x_ffn, const void* w_down_packed,
                           float* slots, float* hidden, float* partials, void* ws, void* stream) {
    StreamGeom geo;
    if (!tp_stream_geometry(p, &geo)) return TP_ERR_UNSUPPORTED;
    if ((int64_t)n_layers * 2 >= ((int64_t)1 << 30)) return TP_ERR_UNSUPPORTED;
    if ((int64_t)p->batch * p->hidden >= ((int64_t)1 << 31)) return TP_ERR_UNSUPPORTED;
    // the slots of one point through one buffer range
    if ((int64_t)p->n_ranks * p->batch * p->hidden * 4 >= ((int64_t)1 << 31)) return TP_ERR_UNSUPPORTED;
    if ((int64_t)n_layers * geo.grid * (int64_t)(geo.kh0 > geo.kh1 ? geo.kh0 : geo.kh1) * 8 >=
        ((int64_t)1 << 62))
        return TP_ERR_UNSUPPORTED;
    if ((((uintptr_t)w_o_packed | (uintptr_t)w_down_packed) & 15) != 0) return TP_ERR_ALIGNMENT;
    if (geo.grid > 1024) return TP_ERR_UNSUPPORTED;  // completion words of the serial order
    if (n_layers == 0) return TP_OK;
    const bool serial = p->serial_points != 0 && !partials;
    // the serial order's cooperative launch holds one workgroup per compute
    // unit, and its wait reads 256 completion words
    if (serial && geo.grid > kTargetCUs) return TP_ERR_UNSUPPORTED;
    // the dataflow order takes the stream block by block across points where
    // a layer's blocks fit one bank (small points: measured up to 33 %
    // faster; larger points, up to 5 % slower that way, keep a point per
    // bank), and with bf16 weights from 4 tokens, where the compute waves'
    // skew at the per-point barriers weighs (page-1 N=4 b=4 6 % faster, N=2
    // b=4 the same; at 2 tokens 1 % slower). FLAT keeps two x buffers per kind
    const bool flat = !serial && !partials && 2 * (int64_t)geo.lds_bytes <= kStreamMaxLdsBytes &&
                      (p->stream_flat >= 0 ? p->stream_flat == 1
                                           : geo.bpw0 + geo.bpw1 <= geo.sl ||
                                                 (p->batch >= 4 && p->weight_format == TP_WEIGHTS_BF16));
    const int32_t xpair = geo.xdwords;
    if (flat) {
        geo.xdwords *= 2;
        geo.lds_bytes *= 2;
    }
    stream_fn k = stream_kernel(p->batch, geo.sl, partials ? 2 : serial ? 1 : flat ? 3 : 0, p->weight_format);
    if (!k) return TP_ERR_UNSUPPORTED;
    StreamArgs a;
    a.x0 = static_cast<const uint16_t*>(x_attn);
    a.x1 = static_cast<const uint16_t*>(x_ffn);
    a.w0 = static_cast<const uint16_t*>(w_o_packed);
    a.w1 = static_cast<const uint16_t*>(w_down_packed);
    // MX weights: each stack's scale words follow its code vectors
    a.sc0 = reinterpret_cast<const uint32_t*>(static_cast<const char*>(w_o_packed) +
                                              (int64_t)n_layers * (p->hidden / 4) * geo.kv0 * 16);
    a.sc1 = reinterpret_cast<const uint32_t*>(static_cast<const char*>(w_down_packed) +
                                              (int64_t)n_layers * (p->hidden / 4) * geo.kv1 * 16);
    a.slots = partials ? partials : slots;
    a.hidden = hidden;
    a.flags = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + kStreamFlagOffset);
    a.err = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + kSyncOffset) + kSyncErr;
    a.H = (int32_t)p->hidden;
    a.S = (int32_t)(p->hidden / 4);
    a.NS = geo.ns;
    a.WPS = geo.wps;
    a.K0 = (int32_t)(p->k_attn / p->n_ranks);
    a.K1 = (int32_t)(p->inter / p->n_ranks);
    a.Kh0 = geo.kh0;
    a.Kh1 = geo.kh1;
    a.Kv0 = geo.kv0;
    a.Kv1 = geo.kv1;
    a.bpw0 = geo.bpw0;
    a.bpw1 = geo.bpw1;
    a.layers = n_layers;
    a.n_ranks = p->n_ranks;
    a.rank = rank;
    a.chunk = (int32_t)((int64_t)p->batch * p->hidden / p->n_ranks);
    a.xoff1 = geo.xoff1;
    a.xdwords = geo.xdwords;
    a.xpair = xpair;

    a.spin_limit = 1u << 20;
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                            hipFuncAttributeMaxDynamicSharedMemorySize, geo.lds_bytes) != hipSuccess)
        return TP_ERR_DEVICE;
    if (serial) {
        void* args[] = {&a};
        if (hipLaunchCooperativeKernel(reinterpret_cast<const void*>(k), dim3((unsigned)geo.grid),
                                       dim3((unsigned)geo.block), args, (unsigned)geo.lds_bytes,
                                       (hipStream_t)stream) != hipSuccess)
            return TP_ERR_DEVICE;
    } else {
        hipLaunchKernelGGL(k, dim3((unsigned)geo.grid), dim3((unsigned)geo.block),
                           (unsigned)geo.lds_bytes, (hipStream_t)stream, a);
    }
    return tp_launch_status(stream);
}

