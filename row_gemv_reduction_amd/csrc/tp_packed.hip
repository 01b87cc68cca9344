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
    const uint16_t* w0;     // packed w_o    [L][S][Kh0][8]
    const uint16_t* w1;     // packed w_down [L][S][Kh1][8]
    float* slots;           // [L][2][N][B][H]
    float* hidden;          // [B][H]
    uint32_t* flags;        // serial order: G completion words, then the exit counter
    uint32_t* err;          // error word (bit 0: a bounded wait timed out)
    int32_t H, S, NS, WPS;
    int32_t K0, K1, Kh0, Kh1;
    int32_t bpw0, bpw1;     // row blocks per compute wave per point (same for every wave)
    int32_t layers, n_ranks, rank, chunk;
    int32_t xoff1;          // dword offset of the second x buffer in LDS
    int32_t xdwords;        // total LDS dwords of the two x buffers
    uint32_t spin_limit;
};

// Flag words (serial order): [0, G) completion of each workgroup, then the
// exit counter on a line of its own.
constexpr int kFlagExit = 1024;

// Hidden-state elements of a workgroup (NS * 4 * B) held per control lane:
// at most 3, so the control wave's registers stay few (the host keeps NS
// small enough).
constexpr int stream_elems_per_lane(int b) {
    return (kStreamMaxNS * 4 * b + 63) / 64 < 3 ? (kStreamMaxNS * 4 * b + 63) / 64 : 3;
}

// Wave-uniform cursor over a compute wave's stream of segments: segment
// (j, m0) is row blocks m0 .. m0+SL-1 of this wave's blocks of point j.
struct Cursor {
    int j, m0;
};

// PART: the partials only (tp_rowparallel_partials_packed): the control wave
// writes each point's partial to slots[j] ([L][2][b][H]) and forms no ring
// sum; the hidden state is neither read nor written.
template <int B, int SL, bool SERIAL, bool PART = false>
__global__ __launch_bounds__(kStreamMaxWaves * 64) void decode_stream(StreamArgs a) {
    extern __shared__ __align__(16) uint32_t xs[];             // two x buffers, bf16 pairs
    __shared__ float red[2][kStreamMaxWaves - 1][B * 4];        // per point parity

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = blockIdx.x, G = gridDim.x;
    const int n_points = 2 * a.layers;
    const int len = B * a.H;

    // zero both x buffers: rows past a point's K are multiplied by zero
    // weights and must hold finite values
    for (int i = tid; i < a.xdwords; i += blockDim.x) xs[i] = 0u;
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
        auto fetch_others = [&](int j) {
            if (PART) return;
            const float* slot = a.slots + (int64_t)j * a.n_ranks * len;
#pragma unroll
            for (int q = 0; q < EQ_MAX; ++q) {
                const int cidx = idx[q] / a.chunk;
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    int r = cidx + u;
                    if (r >= a.n_ranks) r -= a.n_ranks;
                    oth[q][u] = (valid[q] && u < a.n_ranks && r != a.rank)
                                    ? slot[(int64_t)r * len + idx[q]] : 0.f;
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
            uint32_t* dst = xs + (t ? a.xoff1 : 0);
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
        auto grid_wait = [&](int j) {
            if (!ok) return;
            const uint32_t target = (uint32_t)(j + 1);
            for (uint32_t n = 0;; ++n) {
                uint32_t mn = 0xffffffffu;
                for (int w0 = lane; w0 < G; w0 += 64) {
                    const uint32_t f = ld_dev_u32(a.flags + w0);
                    mn = f < mn ? f : mn;
                }
                const bool done = __builtin_amdgcn_ballot_w64(mn < target) == 0;
                if (done) return;
                if ((n & 15) == 15 && __builtin_amdgcn_readfirstlane(ld_dev_u32(err))) { ok = 0; return; }
                if (n >= a.spin_limit) {
                    if (lane == 0) __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    ok = 0;
                    return;
                }
                __builtin_amdgcn_s_sleep(1);
            }
        };

        stage_x(0);
        if (!SERIAL && n_points > 1) stage_x(1);
        fetch_others(0);
        wait_mem();
        __syncthreads();  // start: x of the first point(s) is in LDS

        for (int j = 0; j < n_points; ++j) {
            __syncthreads();  // P_j: the compute waves' sums of point j are in red[j & 1]
            float* slot = PART ? a.slots + (int64_t)j * len
                               : a.slots + (int64_t)j * a.n_ranks * len + (int64_t)a.rank * len;
#pragma unroll
            for (int q = 0; q < EQ_MAX; ++q) {
#pragma clang fp contract(off)
                if (!valid[q]) continue;
                const int e = lane + 64 * q;
                const int c = e & 3, si = (e >> 2) % a.NS, b = (e >> 2) / a.NS;
                float v = red[j & 1][si * a.WPS][b * 4 + c];
                for (int wi = 1; wi < a.WPS; ++wi) v += red[j & 1][si * a.WPS + wi][b * 4 + c];
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
            if (j + 1 < n_points) fetch_others(j + 1);
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

        auto bpw = [&](int j) { return (j & 1) ? a.bpw1 : a.bpw0; };
        auto advance = [&](Cursor& cu) {
            cu.m0 += SL;
            if (cu.m0 >= bpw(cu.j)) { cu.j += 1; cu.m0 = 0; }
        };
        // SL loads, always issued; a segment past the strip or the step has
        // an empty range and reads zeros without a memory access
        auto issue = [&](u32x4_t (&bank)[SL], const Cursor& cu) {
            const int t = cu.j & 1, l = cu.j >> 1;
            const int kh = t ? a.Kh1 : a.Kh0;
            const bool live = active && cu.j < n_points;
            const uint16_t* base = (t ? a.w1 : a.w0) + ((int64_t)l * a.S + s) * kh * 8;
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint16_t*>(live ? base : a.w0), (short)0, live ? kh * 16 : 0,
                kBufferRsrcWord3);
#pragma unroll
            for (int i = 0; i < SL; ++i)
                bank[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                          rs, voff + (cu.m0 + i) * stride, 0, kCachePolicyNT));
        };
        float acc[B][4];
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[b][c] = 0.f;
        auto consume = [&](const u32x4_t (&bank)[SL], const Cursor& cu) {
            const int t = cu.j & 1;
            const int kh = t ? a.Kh1 : a.Kh0;
            const uint32_t* xb = xs + (t ? a.xoff1 : 0);
#pragma unroll
            for (int i = 0; i < SL; ++i) {
                const int kp = (wi + (cu.m0 + i) * a.WPS) * 64 + lane;
                const u32x4_t wq = bank[i];
                const uint32_t wd[4] = {wq.x, wq.y, wq.z, wq.w};
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    const bf16x2_t xv = __builtin_bit_cast(bf16x2_t, xb[b * kh + kp]);
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        acc[b][c] = __builtin_amdgcn_fdot2_f32_bf16(
                            __builtin_bit_cast(bf16x2_t, wd[c]), xv, acc[b][c], false);
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
        Cursor ci{0, 0}, cc{0, 0};
        issue(bank0, ci);
        advance(ci);
        issue(bank1, ci);
        advance(ci);
        __syncthreads();  // start
        while (cc.j < n_points) {
            {
                consume(bank0, cc);
                const int j = cc.j;
                const bool last = cc.m0 + SL >= bpw(j);
                advance(cc);
                issue(bank0, ci);
                advance(ci);
                if (last) point_end(j);
            }
            {
                const bool live = cc.j < n_points;
                int j = cc.j;
                bool last = false;
                if (live) {
                    consume(bank1, cc);
                    last = cc.m0 + SL >= bpw(j);
                    advance(cc);
                }
                issue(bank1, ci);
                advance(ci);
                if (last) point_end(j);
            }
        }
    }
}

typedef void (*stream_fn)(StreamArgs);

template <int SL, bool SERIAL, bool PART>
stream_fn stream_kernel_for(int b) {
    switch (b) {
        case 1: return decode_stream<1, SL, SERIAL, PART>;
        case 2: return decode_stream<2, SL, SERIAL, PART>;
        case 3: return decode_stream<3, SL, SERIAL, PART>;
        case 4: return decode_stream<4, SL, SERIAL, PART>;
        case 5: return decode_stream<5, SL, SERIAL, PART>;
        case 6: return decode_stream<6, SL, SERIAL, PART>;
        case 7: return decode_stream<7, SL, SERIAL, PART>;
        case 8: return decode_stream<8, SL, SERIAL, PART>;
    }
    return nullptr;
}

// 8-load banks only for batch <= 4 (beyond, the registers would spill).
template <bool SERIAL, bool PART>
stream_fn stream_kernel_sl8(int b) {
    switch (b) {
        case 1: return decode_stream<1, 8, SERIAL, PART>;
        case 2: return decode_stream<2, 8, SERIAL, PART>;
        case 3: return decode_stream<3, 8, SERIAL, PART>;
        case 4: return decode_stream<4, 8, SERIAL, PART>;
    }
    return nullptr;
}

// mode 0: dataflow point order, 1: serial point order, 2: partials only
stream_fn stream_kernel(int b, int sl, int mode) {
    if (sl == 4)
        return mode == 1 ? stream_kernel_for<4, true, false>(b)
                         : mode == 2 ? stream_kernel_for<4, false, true>(b) : stream_kernel_for<4, false, false>(b);
    if (sl == 8)
        return mode == 1 ? stream_kernel_sl8<true, false>(b)
                         : mode == 2 ? stream_kernel_sl8<false, true>(b) : stream_kernel_sl8<false, false>(b);
    return nullptr;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

// Geometry of the streamed step for a plan (host side; see tp_internal.h).
bool tp_stream_geometry(const tp_plan_s* p, StreamGeom* g) {
    if (p->batch < 1 || p->batch > kStripMaxBatch || p->n_ranks > 8) return false;
    if (p->hidden % 4) return false;
    const int64_t k0 = p->k_attn / p->n_ranks, k1 = p->inter / p->n_ranks;
    if (k0 < 2 || k1 < 2 || (k0 & 1) || (k1 & 1)) return false;
    if ((k0 * p->batch) % 8 || (k1 * p->batch) % 8) return false;
    const int64_t S = p->hidden / 4;
    int64_t ns = (S + kTargetCUs - 1) / kTargetCUs;
    if (ns > kStreamMaxNS) ns = kStreamMaxNS;
    const int64_t G = (S + ns - 1) / ns;
    if (ns * 4 * p->batch > 64 * stream_elems_per_lane(p->batch)) return false;
    const int wps = (int)((kStreamMaxWaves - 1) / ns);
    // 8-load banks (more bytes in flight) where the registers allow it
    const int sl = p->segment_loads == 4 || p->batch > 4 ? 4 : 8;
    const int64_t kh0 = k0 / 2, kh1 = k1 / 2;
    const int64_t nb0 = (kh0 + 63) / 64, nb1 = (kh1 + 63) / 64;
    const int64_t bpw0 = (nb0 + wps - 1) / wps, bpw1 = (nb1 + wps - 1) / wps;
    // x buffer t: B*Kh_t dwords staged in 1 KB pieces, and every pair index a
    // compute lane reads (up to the last block of its last segment)
    auto xbuf = [&](int64_t kh, int64_t bpw) {
        const int64_t n16 = p->batch * kh * 4 / 16;
        const int64_t staged = (n16 + 63) / 64 * 256;
        const int64_t segs = (bpw + sl - 1) / sl;
        const int64_t read = (p->batch - 1) * kh + ((wps - 1) + (segs * sl - 1) * wps) * 64 + 64;
        const int64_t d = staged > read ? staged : read;
        return (d + 255) / 256 * 256;
    };
    g->xoff1 = xbuf(kh0, bpw0);
    g->xdwords = g->xoff1 + xbuf(kh1, bpw1);
    g->grid = (int32_t)G;
    g->ns = (int32_t)ns;
    g->wps = wps;
    g->sl = sl;
    g->block = (int32_t)(1 + ns * wps) * 64;
    g->kh0 = (int32_t)kh0;
    g->kh1 = (int32_t)kh1;
    g->bpw0 = (int32_t)bpw0;
    g->bpw1 = (int32_t)bpw1;
    g->lds_bytes = g->xdwords * 4;
    return g->lds_bytes <= kStreamMaxLdsBytes;
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
    return hipGetLastError() == hipSuccess ? TP_OK : TP_ERR_DEVICE;
}

tp_status tp_decode_stream(const tp_plan_s* p, int32_t n_layers, int32_t rank, const void* x_attn,
                           const void* w_o_packed, const void* x_ffn, const void* w_down_packed,
                           float* slots, float* hidden, float* partials, void* ws, void* stream) {
    StreamGeom geo;
    if (!tp_stream_geometry(p, &geo)) return TP_ERR_UNSUPPORTED;
    if ((int64_t)n_layers * 2 >= ((int64_t)1 << 30)) return TP_ERR_UNSUPPORTED;
    if ((int64_t)p->batch * p->hidden >= ((int64_t)1 << 31)) return TP_ERR_UNSUPPORTED;
    if ((int64_t)n_layers * geo.grid * (int64_t)(geo.kh0 > geo.kh1 ? geo.kh0 : geo.kh1) * 8 >=
        ((int64_t)1 << 62))
        return TP_ERR_UNSUPPORTED;
    if (geo.grid > 1024) return TP_ERR_UNSUPPORTED;  // completion words of the serial order
    if (n_layers == 0) return TP_OK;
    const bool serial = p->serial_points != 0 && !partials;
    stream_fn k = stream_kernel(p->batch, geo.sl, partials ? 2 : serial ? 1 : 0);
    if (!k) return TP_ERR_UNSUPPORTED;
    StreamArgs a;
    a.x0 = static_cast<const uint16_t*>(x_attn);
    a.x1 = static_cast<const uint16_t*>(x_ffn);
    a.w0 = static_cast<const uint16_t*>(w_o_packed);
    a.w1 = static_cast<const uint16_t*>(w_down_packed);
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
    a.bpw0 = geo.bpw0;
    a.bpw1 = geo.bpw1;
    a.layers = n_layers;
    a.n_ranks = p->n_ranks;
    a.rank = rank;
    a.chunk = (int32_t)((int64_t)p->batch * p->hidden / p->n_ranks);
    a.xoff1 = geo.xoff1;
    a.xdwords = geo.xdwords;
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
    return hipGetLastError() == hipSuccess ? TP_OK : TP_ERR_DEVICE;
}

