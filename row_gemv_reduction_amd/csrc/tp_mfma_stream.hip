// The decode step on the bf16 matrix cores, for batches of several tokens.
//
// Same computation as decode_stream (tp_packed.hip): per reconciliation
// point the rank's partial of its weight slice, written to its slot, then
// the ring-order sum of the N ranks' values plus the residual (lesson 9.9
// "Interconnects e clusters", section 01 · Conceito). With b tokens a weight
// byte feeds b multiply-adds; from b ~ 5 on, the vector ALUs would need
// more issue slots than the weight stream leaves, so the products run on
// v_mfma_f32_16x16x32_bf16 (16 tokens x 32 rows x 16 columns per
// instruction). The step stays bound by streaming the weights from HBM.
//
// Layout ("MFMA tiles"): a rank's slice W_r[K][H] is stored once, at load
// time, as 2 KB tiles of 64 rows x 16 columns, each two halves of the
// matrix-core B operand:
//     T[s][kb][h][l][i] = W_r[64kb + 16(l/16) + 8h + i][16s + l%16]
//     s < H/16, kb < ceil(K/64), h < 2, lane l < 64, i < 8   (rows past K are zero)
// One 16-byte load per lane and half hands lane l its B operand (8
// consecutive rows of one column). The two halves of lane group g = l/16
// hold rows 16g .. 16g+15, so the A operands of the two MFMAs of a tile
// (x rows 16g+8h .. +8) cover, per token, one whole 128-byte line of x
// between them: the second load of the line hits L1.
//
// decode_stream_mfma: one launch per step; workgroup s owns the 16-column
// strip s for every point (one workgroup per strip; at most two per CU).
//   - WPS compute waves interleave the strip's tiles. Each wave streams its
//     tiles through two register banks of SL tiles: the weight tile and, per
//     16-token block, the matching A operand (the x rows, 16 bytes per lane,
//     read straight from x; x is small and shared by every workgroup, so it
//     comes from L2). Loads are never conditional (empty buffer ranges read
//     zero), so consuming one bank never waits for the other. Tokens past b
//     and rows past K read zero.
//   - one control wave: at each point's end sums the waves' D tiles in wave
//     order, writes the rank's partial to its slot and forms the ring-order
//     sum with the other ranks' values (staged into LDS a point ahead with
//     direct global->LDS loads) plus the residual, which stays in LDS for the
//     whole step.
// Point order: as decode_stream's default (each hidden-state element follows
// its own chain; no grid-wide synchronisation).
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tp_device.h"
#include "tp_internal.h"

namespace {

using namespace tpdev;

typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kTileBytes = 2048;   // 64 rows x 16 columns of bf16, two operand halves
constexpr int kTileRows = 64;

// T[l][s][kb][h][lane][i] = W[l][64kb + 16(lane/16) + 8h + i][16s + lane%16]
__global__ void pack_tiles_kernel(const uint16_t* __restrict__ w, uint16_t* __restrict__ p,
                                  int64_t layers, int64_t K, int64_t H) {
    const int64_t strips = H / 16, nkb = (K + kTileRows - 1) / kTileRows;
    const int64_t per_layer = strips * nkb * 128;
    const int64_t total = layers * per_layer;
    for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < total;
         v += (int64_t)gridDim.x * blockDim.x) {
        const int64_t l = v / per_layer;
        int64_t rem = v - l * per_layer;
        const int64_t s = rem / (nkb * 128);
        rem -= s * nkb * 128;
        const int64_t kb = rem / 128, h = (rem / 64) % 2, lane = rem % 64;
        const int64_t k0 = kTileRows * kb + 16 * (lane / 16) + 8 * h, n = 16 * s + lane % 16;
        uint16_t e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = k0 + i < K ? w[(l * K + k0 + i) * H + n] : (uint16_t)0;
        u32x4_t out;
        out.x = e[0] | ((uint32_t)e[1] << 16);
        out.y = e[2] | ((uint32_t)e[3] << 16);
        out.z = e[4] | ((uint32_t)e[5] << 16);
        out.w = e[6] | ((uint32_t)e[7] << 16);
        *reinterpret_cast<u32x4_t*>(p + v * 8) = out;
    }
}

struct MfmaArgs {
    const uint16_t* x0;     // x_attn [L][B][K0]
    const uint16_t* x1;     // x_ffn  [L][B][K1]
    const uint16_t* w0;     // tiles of w_o    [L][H/16][nkb0][2][64][8]
    const uint16_t* w1;     // tiles of w_down [L][H/16][nkb1][2][64][8]
    float* slots;           // [L][2][N][B][H]
    float* hidden;          // [B][H]
    int32_t H, S16, WPS, batch;
    int32_t K0, K1, nkb0, nkb1, bpw0, bpw1;
    int32_t layers, n_ranks, rank, chunk;
    int32_t red_floats;     // LDS floats of one parity of the waves' D tiles
    int32_t oth_floats;     // LDS floats of one parity of the other ranks' values
};

struct Cursor {
    int j, m0;
};

template <int BT, int SL>
__global__ __launch_bounds__(1024) void decode_stream_mfma(MfmaArgs a) {
    // [2][WPS][BT][64][4] D tiles | [2][(N-1) * B][16] other ranks | [B][16] hidden
    extern __shared__ __align__(16) float sh[];
    float* red = sh;
    float* oth = sh + 2 * a.red_floats;
    float* hs = oth + 2 * a.oth_floats;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int s = blockIdx.x;
    const int n_points = 2 * a.layers;
    const int B = a.batch;
    const int len = B * a.H;

    if (wave == 0) {
        // ---------------------------------------------------- control wave
        __builtin_amdgcn_s_setprio(3);
        const int n_el = 16 * B;
        for (int e = lane; e < n_el; e += 64) hs[e] = a.hidden[(e >> 4) * a.H + 16 * s + (e & 15)];
        // the other ranks' 16 values per token, rows ordered (other rank, token)
        auto stage_others = [&](int j) {
            const float* slot = a.slots + (int64_t)j * a.n_ranks * len;
            float* dst = oth + (j & 1) * a.oth_floats;
            const int rows = (a.n_ranks - 1) * B;
            for (int r0 = 0; r0 < rows; r0 += 16) {
                int row = r0 + lane / 4;
                row = row < rows ? row : rows - 1;
                const int ro = row / B, tok = row - ro * B;
                const int r = ro < a.rank ? ro : ro + 1;
                const float* src = slot + (int64_t)r * len + (int64_t)tok * a.H + 16 * s + 4 * (lane & 3);
                __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src),
                                                 (lds_void_t*)(dst + r0 * 16), 16, 0, 0);
            }
        };
        if (a.n_ranks > 1) stage_others(0);
        wait_mem();
        __syncthreads();  // start: hidden columns and the first point's other values are in LDS
        for (int j = 0; j < n_points; ++j) {
            __syncthreads();  // P_j: the waves' D tiles of point j are in red[j & 1]
            if (a.n_ranks > 1 && j + 1 < n_points) stage_others(j + 1);
            const float* rj = red + (j & 1) * a.red_floats;
            const float* oj = oth + (j & 1) * a.oth_floats;
            float* slot = a.slots + (int64_t)j * a.n_ranks * len + (int64_t)a.rank * len;
            for (int e = lane; e < n_el; e += 64) {
#pragma clang fp contract(off)
                const int tok = e >> 4, col = e & 15;
                const int tt = tok >> 4, m = tok & 15;
                const int d = ((tt * 64) + 16 * (m >> 2) + col) * 4 + (m & 3);
                float v = rj[d];
                for (int wi = 1; wi < a.WPS; ++wi) v += rj[wi * BT * 256 + d];
                const int i = tok * a.H + 16 * s + col;
                slot[i] = v;
                // ring order: chunk c starts at rank c, then c+1, ... (mod N)
                const int cidx = i / a.chunk;
                float sum = 0.f;
                for (int u = 0; u < a.n_ranks; ++u) {
                    int r = cidx + u;
                    if (r >= a.n_ranks) r -= a.n_ranks;
                    const int ro = r < a.rank ? r : r - 1;
                    const float val = r == a.rank ? v : oj[(ro * B + tok) * 16 + col];
                    sum = u == 0 ? val : sum + val;
                }
                hs[e] = sum + hs[e];
            }
            wait_mem();  // the next point's other values are staged before P_{j+1}
        }
        for (int e = lane; e < n_el; e += 64) a.hidden[(e >> 4) * a.H + 16 * s + (e & 15)] = hs[e];
    } else {
        // --------------------------------------------------- compute waves
        const int wi = wave - 1;
        auto bpw = [&](int j) { return (j & 1) ? a.bpw1 : a.bpw0; };
        auto advance = [&](Cursor& cu) {
            cu.m0 += SL;
            if (cu.m0 >= bpw(cu.j)) { cu.j += 1; cu.m0 = 0; }
        };
        // A operand of lane l: token 16*tt + l%16, rows 16*(l/16) + 8h .. +7 of the tile
        const int xo = lane & 15, xk = 16 * (lane >> 4);
        auto issue = [&](u32x4_t (&wv)[SL][2], u32x4_t (&xv)[SL][2][BT], const Cursor& cu) {
            const int t = cu.j & 1, l = cu.j >> 1;
            const bool live = cu.j < n_points;
            const int K = t ? a.K1 : a.K0, nkb = t ? a.nkb1 : a.nkb0;
            const uint16_t* wb = (t ? a.w1 : a.w0) + ((int64_t)l * a.S16 + s) * nkb * (kTileBytes / 2);
            const uint16_t* xb = (t ? a.x1 : a.x0) + (int64_t)l * B * K;
            const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint16_t*>(live ? wb : a.w0), (short)0, live ? nkb * kTileBytes : 0,
                kBufferRsrcWord3);
            const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint16_t*>(live ? xb : a.x0), (short)0, live ? B * K * 2 : 0,
                kBufferRsrcWord3);
            // Workgroups start their walk over a point's tiles at different
            // places (a rotation by whole rounds of WPS tiles), so that they do
            // not all read the same rows of x at the same moment. Slots past
            // the wave's bpw tiles (the tail of the last segment) stay past the
            // span, which reads zero.
            const int bpw = t ? a.bpw1 : a.bpw0;
            const int span = bpw * a.WPS;
            const int rot = (s % bpw) * a.WPS;
#pragma unroll
            for (int i = 0; i < SL; ++i) {
                int kb = wi + (cu.m0 + i) * a.WPS + rot;
                kb = cu.m0 + i >= bpw ? span : kb >= span ? kb - span : kb;
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    wv[i][h] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                               wr, kb * kTileBytes + h * 1024 + lane * 16, 0,
                                                               kCachePolicyNT));
#pragma unroll
                for (int tt = 0; tt < BT; ++tt)
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        xv[i][h][tt] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                                       xr, ((16 * tt + xo) * K + kTileRows * kb + xk + 8 * h) * 2,
                                                                       0, 0));
            }
        };
        floatx4_t acc[BT];
#pragma unroll
        for (int tt = 0; tt < BT; ++tt) acc[tt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
        auto consume = [&](const u32x4_t (&wv)[SL][2], const u32x4_t (&xv)[SL][2][BT]) {
#pragma unroll
            for (int i = 0; i < SL; ++i)
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int tt = 0; tt < BT; ++tt)
                        acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8_t, xv[i][h][tt]), __builtin_bit_cast(bf16x8_t, wv[i][h]),
                            acc[tt], 0, 0, 0);
        };
        auto point_end = [&](int j) {
            float* rj = red + (j & 1) * a.red_floats + wi * BT * 256;
#pragma unroll
            for (int tt = 0; tt < BT; ++tt) {
                *reinterpret_cast<floatx4_t*>(rj + (tt * 64 + lane) * 4) = acc[tt];
                acc[tt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
            }
            __syncthreads();  // P_j
        };

        u32x4_t w0[SL][2], w1[SL][2], x0[SL][2][BT], x1[SL][2][BT];
        Cursor ci{0, 0}, cc{0, 0};
        issue(w0, x0, ci);
        advance(ci);
        issue(w1, x1, ci);
        advance(ci);
        __syncthreads();  // start
        while (cc.j < n_points) {
            {
                consume(w0, x0);
                const int j = cc.j;
                const bool last = cc.m0 + SL >= bpw(j);
                advance(cc);
                issue(w0, x0, ci);
                advance(ci);
                if (last) point_end(j);
            }
            {
                const bool live = cc.j < n_points;
                const int j = cc.j;
                bool last = false;
                if (live) {
                    consume(w1, x1);
                    last = cc.m0 + SL >= bpw(j);
                    advance(cc);
                }
                issue(w1, x1, ci);
                advance(ci);
                if (last) point_end(j);
            }
        }
    }
}

typedef void (*mfma_stream_fn)(MfmaArgs);

// Tiles per bank: fewer for more token blocks (each tile also carries 2*BT
// A operands), so the banks fit the registers.
mfma_stream_fn mfma_stream_kernel(int bt) {
    switch (bt) {
        case 1: return decode_stream_mfma<1, 2>;
        case 2: return decode_stream_mfma<2, 2>;
        case 3: return decode_stream_mfma<3, 1>;
        case 4: return decode_stream_mfma<4, 1>;
    }
    return nullptr;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

bool tp_mfma_geometry(const tp_plan_s* p, MfmaGeom* g) {
    const int b = p->batch;
    if (b < 1 || b > kMfmaMaxBatch || p->n_ranks > 8 || p->hidden % 16) return false;
    const int64_t k0 = p->k_attn / p->n_ranks, k1 = p->inter / p->n_ranks;
    if (k0 % 8 || k1 % 8) return false;
    const int64_t S16 = p->hidden / 16;
    if (S16 > 2 * kTargetCUs) return false;  // one strip per workgroup, at most two per CU
    const int per_cu = S16 > kTargetCUs ? 2 : 1;
    const int bt = (b + 15) / 16;
    int wps = per_cu == 2 ? 7 : (bt <= 2 ? 15 : 7);
    const int sl = bt <= 2 ? 2 : 1;
    const int64_t nkb0 = (k0 + kTileRows - 1) / kTileRows, nkb1 = (k1 + kTileRows - 1) / kTileRows;
    g->red_floats = wps * bt * 256;
    g->oth_floats = (p->n_ranks - 1) * b * 16 > 0 ? ((p->n_ranks - 1) * b * 16 + 255) / 256 * 256 : 0;
    g->lds_bytes = (2 * g->red_floats + 2 * g->oth_floats + ((16 * b + 63) / 64) * 64) * 4;
    if (g->lds_bytes > (per_cu == 2 ? 76 : 152) * 1024) return false;
    // the largest buffer offsets must fit 32 bits
    if ((int64_t)b * (k0 > k1 ? k0 : k1) * 2 >= ((int64_t)1 << 31)) return false;
    if ((nkb0 > nkb1 ? nkb0 : nkb1) * kTileBytes >= ((int64_t)1 << 31)) return false;
    g->grid = (int32_t)S16;
    g->wps = wps;
    g->bt = bt;
    g->sl = sl;
    g->block = (1 + wps) * 64;
    g->nkb0 = (int32_t)nkb0;
    g->nkb1 = (int32_t)nkb1;
    g->bpw0 = (int32_t)((nkb0 + wps - 1) / wps);
    g->bpw1 = (int32_t)((nkb1 + wps - 1) / wps);
    return true;
}

tp_status tp_pack_tiles(const tp_plan_s* p, int point, int n_layers, const void* w, void* w_packed,
                        void* stream) {
    const int64_t K = (point == TP_POINT_ATTN_OUT ? p->k_attn : p->inter) / p->n_ranks;
    const int64_t total = (int64_t)n_layers * (p->hidden / 16) * ((K + kTileRows - 1) / kTileRows) * 128;
    if (total == 0) return TP_OK;
    const int64_t blocks = (total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536;
    hipLaunchKernelGGL(pack_tiles_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       static_cast<const uint16_t*>(w), static_cast<uint16_t*>(w_packed),
                       (int64_t)n_layers, K, p->hidden);
    return hipGetLastError() == hipSuccess ? TP_OK : TP_ERR_DEVICE;
}

tp_status tp_decode_mfma_stream(const tp_plan_s* p, int32_t n_layers, int32_t rank,
                                const void* x_attn, const void* w_o_tiles, const void* x_ffn,
                                const void* w_down_tiles, float* slots, float* hidden, void* stream) {
    MfmaGeom geo;
    if (!tp_mfma_geometry(p, &geo)) return TP_ERR_UNSUPPORTED;
    if (!aligned16(x_attn) || !aligned16(x_ffn) || !aligned16(w_o_tiles) || !aligned16(w_down_tiles) ||
        !aligned16(slots) || !aligned16(hidden))
        return TP_ERR_ALIGNMENT;
    if ((int64_t)p->batch * p->hidden >= ((int64_t)1 << 31)) return TP_ERR_UNSUPPORTED;
    if (n_layers == 0) return TP_OK;
    mfma_stream_fn k = mfma_stream_kernel(geo.bt);
    if (!k) return TP_ERR_UNSUPPORTED;
    MfmaArgs a;
    a.x0 = static_cast<const uint16_t*>(x_attn);
    a.x1 = static_cast<const uint16_t*>(x_ffn);
    a.w0 = static_cast<const uint16_t*>(w_o_tiles);
    a.w1 = static_cast<const uint16_t*>(w_down_tiles);
    a.slots = slots;
    a.hidden = hidden;
    a.H = (int32_t)p->hidden;
    a.S16 = (int32_t)(p->hidden / 16);
    a.WPS = geo.wps;
    a.batch = p->batch;
    a.K0 = (int32_t)(p->k_attn / p->n_ranks);
    a.K1 = (int32_t)(p->inter / p->n_ranks);
    a.nkb0 = geo.nkb0;
    a.nkb1 = geo.nkb1;
    a.bpw0 = geo.bpw0;
    a.bpw1 = geo.bpw1;
    a.layers = n_layers;
    a.n_ranks = p->n_ranks;
    a.rank = rank;
    a.chunk = (int32_t)((int64_t)p->batch * p->hidden / p->n_ranks);
    a.red_floats = geo.red_floats;
    a.oth_floats = geo.oth_floats;
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                            hipFuncAttributeMaxDynamicSharedMemorySize, geo.lds_bytes) != hipSuccess)
        return TP_ERR_DEVICE;
    hipLaunchKernelGGL(k, dim3((unsigned)geo.grid), dim3((unsigned)geo.block), (unsigned)geo.lds_bytes,
                       (hipStream_t)stream, a);
    return hipGetLastError() == hipSuccess ? TP_OK : TP_ERR_DEVICE;
}
