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
// decode_stream_mfma: one launch per step, G workgroups (one per CU).
// Work is balanced by tiles, not by strips: per point the S16 * nkb tiles,
// taken in strip-major order, are cut into G equal contiguous ranges, one
// per workgroup (with H = 5120 there are 320 strips for 256 CUs, so whole
// strips would leave a quarter of the CUs doing twice the work). A range
// falls into segments, one per strip it touches; a strip cut between two
// workgroups is owned by the one that holds its first tile (that owner is
// the same for both kinds of point), and the other one, its contributor,
// hands over the partial of the remaining rows through device memory.
//   - WPS compute waves interleave each segment's tiles. Each wave streams
//     its tiles through two register banks of SL tiles: the weight tile and,
//     per 16-token block, the matching A operand (the x rows, 16 bytes per
//     lane, read straight from x, which every workgroup reads and L2 keeps).
//     Loads are never conditional (empty buffer ranges read zero), so
//     consuming one bank never waits for the other. Tokens past b and rows
//     past K read zero. At a segment's end a wave stores its D tiles to LDS,
//     counts itself and streams on (no barrier).
//   - a reducer wave sums each segment's D tiles in wave order into one of
//     two LDS partial buffers and frees the D-tile buffer at once;
//   - the control wave takes the segments' partials in order: a contributor
//     publishes its partial; an owner adds the contributor's partial (its
//     own rows first), writes the rank's partial to its slot and forms the
//     ring-order sum with the other ranks' values (staged into LDS a point
//     ahead by two stager waves with direct global->LDS loads) plus the
//     residual, which stays in LDS for the whole step.
// Point order: as decode_stream's default (each hidden-state element follows
// its own chain, kept by the strip's owner; no grid-wide synchronisation).
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

// Microscaled weights on the matrix cores: a tile of 64 rows x 16 columns
// holds the codes lane-major (lane l: the 16 consecutive rows 16(l/16) ..
// +15 of column l%16, 16 bytes of FP8 or 8 of FP4, the even row of a byte in
// its low nibble), then the 32 scale bytes of its two 32-row blocks
// ([block][column]). Lane l's rows lie in block l/32. In registers each
// half of a lane's rows is widened to the bf16 B operand by gfx950's scaled
// conversions (the block scale as their scale operand), then multiplied on
// the bf16 matrix cores like bf16 weights.
template <int WF>
constexpr int tile_bytes() {
    return WF == TP_WEIGHTS_MXFP8 ? 1024 + 32 : WF == TP_WEIGHTS_MXFP4 ? 512 + 32 : kTileBytes;
}

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// One tile's weights for lane `lane` (tile kb of the range; past the range
// it reads zero): bf16, both operand halves; MX, the codes and the scale.
template <int WF>
__device__ __forceinline__ void load_w_tile(__amdgpu_buffer_rsrc_t wr, int kb, int lane, u32x4_t (&wv)[2],
                                            uint32_t& sv) {
    constexpr int TB = tile_bytes<WF>();
    if constexpr (WF == TP_WEIGHTS_BF16) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
            wv[h] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                    wr, kb * TB + h * 1024 + lane * 16, 0, kCachePolicyNT));
        sv = 0u;
    } else {
        constexpr int CB = WF == TP_WEIGHTS_MXFP8 ? 16 : 8;  // code bytes per lane
        if constexpr (WF == TP_WEIGHTS_MXFP8) {
            wv[0] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                    wr, kb * TB + lane * CB, 0, kCachePolicyNT));
        } else {
            const u32x2_t c = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(
                                                              wr, kb * TB + lane * CB, 0, kCachePolicyNT));
            wv[0] = u32x4_t{c.x, c.y, 0u, 0u};
        }
        wv[1] = u32x4_t{0u, 0u, 0u, 0u};
        sv = __builtin_amdgcn_raw_buffer_load_b8(wr, kb * TB + 64 * CB + (lane >> 5) * 16 + (lane & 15), 0,
                                                 kCachePolicyNT);
    }
}

// Half h (rows 8h .. 8h+7 of the lane's 16) as the bf16 B operand.
template <int WF>
__device__ __forceinline__ bf16x8_t b_operand(const u32x4_t (&wv)[2], uint32_t sv, int h) {
    if constexpr (WF == TP_WEIGHTS_BF16) {
        return __builtin_bit_cast(bf16x8_t, wv[h]);
    } else {
        // the E8M0 byte as the conversions' scale operand: they read the
        // binary32's exponent field as E8M0 (the mantissa is ignored)
        const float sc = __uint_as_float(sv << 23);
        bf16x2_t q[4];
        if constexpr (WF == TP_WEIGHTS_MXFP8) {
            const uint32_t d0 = h ? wv[0].z : wv[0].x, d1 = h ? wv[0].w : wv[0].y;
            q[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, sc, false);
            q[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, sc, true);
            q[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, sc, false);
            q[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, sc, true);
        } else {
            const uint32_t d = h ? wv[0].y : wv[0].x;
            q[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 0);
            q[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 1);
            q[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 2);
            q[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 3);
        }
        const u32x4_t r{__builtin_bit_cast(uint32_t, q[0]), __builtin_bit_cast(uint32_t, q[1]),
                        __builtin_bit_cast(uint32_t, q[2]), __builtin_bit_cast(uint32_t, q[3])};
        return __builtin_bit_cast(bf16x8_t, r);
    }
}

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

// Activations in A-operand order, so that every 16-byte-per-lane load of
// the step reads 1 KB of contiguous memory (row-major x would give each
// load 16 tokens x 64 bytes, half of 16 different cache lines):
//     X[l][kb][tt][h][lane][i] = x[l][16tt + lane%16][64kb + 16(lane/16) + 8h + i]
// (zero for rows past K; entries of tokens past b are not written: the
// step never reads them).
__global__ void pack_acts_kernel(const uint16_t* __restrict__ x0, const uint16_t* __restrict__ x1,
                                 uint16_t* __restrict__ p0, uint16_t* __restrict__ p1, int64_t layers,
                                 int64_t B, int64_t K0, int64_t K1, int64_t bt) {
    const int64_t nkb0 = (K0 + kTileRows - 1) / kTileRows, nkb1 = (K1 + kTileRows - 1) / kTileRows;
    const int64_t per0 = nkb0 * bt * 128, per1 = nkb1 * bt * 128;  // 16-byte vectors per layer
    const int64_t total = layers * (per0 + per1);
    for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < total;
         v += (int64_t)gridDim.x * blockDim.x) {
        const bool second = v >= layers * per0;
        const int64_t w = second ? v - layers * per0 : v;
        const int64_t per = second ? per1 : per0, K = second ? K1 : K0;
        const int64_t l = w / per;
        int64_t rem = w - l * per;
        const int64_t kb = rem / (bt * 128);
        rem -= kb * bt * 128;
        const int64_t tt = rem / 128, h = (rem / 64) % 2, lane = rem % 64;
        const int64_t tok = 16 * tt + lane % 16, k0 = kTileRows * kb + 16 * (lane / 16) + 8 * h;
        if (tok >= B) continue;
        u32x4_t out = u32x4_t{0u, 0u, 0u, 0u};
        if (k0 < K)  // K is a multiple of 8: the 8 rows are all inside or all past
            out = *reinterpret_cast<const u32x4_t*>((second ? x1 : x0) + (l * B + tok) * K + k0);
        *reinterpret_cast<u32x4_t*>((second ? p1 : p0) + w * 8) = out;
    }
}

// MX codes [L][K][H] (FP8) or [L][K/2][H] (FP4) and scales [L][K/32][H]
// -> MX tiles [L][H/16][ceil(K/64)] (codes lane-major, then the 32 scale
// bytes), zero past K. One thread per (tile, lane): its code bytes, and for
// lanes < 32 the scale byte (block lane/16, column lane%16).
template <int WF>
__global__ void pack_mx_tiles_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                     uint8_t* __restrict__ p, int64_t layers, int64_t K, int64_t H) {
    constexpr int TB = tile_bytes<WF>(), CB = WF == TP_WEIGHTS_MXFP8 ? 16 : 8;
    const int64_t strips = H / 16, nkb = (K + kTileRows - 1) / kTileRows;
    const int64_t crows = WF == TP_WEIGHTS_MXFP8 ? K : K / 2;  // code rows per layer
    const int64_t total = layers * strips * nkb * 64;
    for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < total;
         v += (int64_t)gridDim.x * blockDim.x) {
        const int64_t tile = v / 64, lane = v % 64;
        const int64_t kb = tile % nkb, s = (tile / nkb) % strips, l = tile / (nkb * strips);
        const int64_t n = 16 * s + lane % 16, r0 = kTileRows * kb + 16 * (lane / 16);
        uint8_t* out = p + tile * TB;
#pragma unroll
        for (int i = 0; i < CB; ++i) {
            // FP8: byte i = row r0 + i; FP4: byte i = rows r0 + 2i (low nibble), r0 + 2i + 1
            const int64_t r = WF == TP_WEIGHTS_MXFP8 ? r0 + i : r0 + 2 * i;
            const int64_t cr = WF == TP_WEIGHTS_MXFP8 ? r : r / 2;
            out[lane * CB + i] = r < K ? codes[(l * crows + cr) * H + n] : (uint8_t)0;
        }
        if (lane < 32) {
            const int64_t blk = 2 * kb + lane / 16, c = 16 * s + lane % 16;
            out[64 * CB + lane] = 32 * blk < K ? scales[(l * (K / 32) + blk) * H + c] : (uint8_t)0;
        }
    }
}

struct MfmaArgs {
    const uint16_t* x0;     // x_attn in A-operand order [L][nkb0][BT][2][64][8]
    const uint16_t* x1;     // x_ffn  in A-operand order [L][nkb1][BT][2][64][8]
    const uint16_t* w0;     // tiles of w_o    [L][H/16][nkb0][2][64][8]
    const uint16_t* w1;     // tiles of w_down [L][H/16][nkb1][2][64][8]
    float* slots;           // [L][2][N][B][H]
    float* hidden;          // [B][H]
    float* xpart;           // [2][kXchgRing][S16][BT][64][4] contributors' partials
    uint32_t* pub;          // [2][S16] contributor has published point j: j + 1
    uint32_t* ack;          // [2][S16] owner has read point j: j + 1
    uint32_t* exit_ctr;     // workgroups that have left
    uint32_t* err;          // error word (bit 0: an exchange wait timed out, bit 1: a wave wait)
    int32_t H, S16, G, batch;
    int32_t K0, K1, nkb0, nkb1;
    int32_t layers, n_ranks, rank, chunk;
    int32_t oth_strip;      // LDS floats of the other ranks' values per owned strip
    int32_t own_max;        // owned strips per workgroup at most (their buffers per staged point)
    int32_t oth_lg;         // the other ranks' values are staged in 1 << oth_lg buffers
    uint32_t spin_limit;
};

// A workgroup's work for one kind of point: up to kMaxSeg segments (strip,
// first tile, tiles, role).
constexpr int kMaxSeg = 4;
constexpr int kMaxOwn = 2;  // strips whose hidden state a workgroup keeps
enum { kFull = 0, kOwnerPart = 1, kContrib = 2 };

// Tiles u = s * nkb + kb of one kind of point, in strip-major order; workgroup
// g takes u in [ceil(g T / G), ceil((g+1) T / G)), T = S16 * nkb. The tile
// kb = 0 of strip s falls to workgroup floor(s G / S16) whatever nkb is, so
// a strip has the same owner for both kinds of point; with G <= S16 every
// range holds at least nkb tiles, so a strip is cut at most once.
__device__ int wg_segments(int g, int G, int S16, int nkb, int (*out)[4]) {
    const int64_t T = (int64_t)S16 * nkb;
    const int64_t u0 = ((int64_t)g * T + G - 1) / G, u1 = ((int64_t)(g + 1) * T + G - 1) / G;
    int n = 0;
    for (int64_t u = u0; u < u1 && n < kMaxSeg;) {
        const int s = (int)(u / nkb);
        const int kb0 = (int)(u - (int64_t)s * nkb);
        const int64_t e = u1 < (int64_t)(s + 1) * nkb ? u1 : (int64_t)(s + 1) * nkb;
        out[n][0] = s;
        out[n][1] = kb0;
        out[n][2] = (int)(e - u);
        out[n][3] = kb0 > 0 ? kContrib : (e - u == nkb ? kFull : kOwnerPart);
        ++n;
        u = e;
    }
    return n;
}

// Index of workgroup w among the G when those on XCD x = w % 8 take the
// x-th block of consecutive indices (blocks of G/8, the first G % 8 one
// larger). A bijection of [0, G).
__device__ __forceinline__ int xcd_range_index(int w, int G) {
    const int x = w % kXCDs, q = G / kXCDs, r = G % kXCDs;
    return x * q + (x < r ? x : r) + w / kXCDs;
}

struct Cursor {
    int j, i, m0;            // point, segment, first slot of the bank
    int s, kb0, len, bpw, rot;  // the segment's strip, tiles, slots per wave, walk rotation
};

// A compute wave's place in its own stream of tiles, for register slots
// that run across segment and point boundaries: the wave's m-th tile of
// segment i of point j. nr = its tiles in the segment (wi + m WPS < len),
// ns = max(nr, 1) slots (a segment without a tile of this wave still takes
// one empty slot, so that the wave counts itself there), r0 = rotation.
struct SlotCursor {
    int j, i, m;
    int s, kb0, nr, ns, r0;
};

// The waves of a workgroup meet through LDS flags, not barriers: a compute
// wave stores its D tiles of segment e into buffer e % NBUF, counts itself
// in that buffer's arrivals and goes on streaming; the control wave starts
// on segment e once all WPS waves have counted, and publishes `consumed` =
// e + 1 once it has read their tiles, which frees the buffer for segment
// e + NBUF. So a wave waits for its slowest sibling only when it is NBUF
// segments ahead of it.
// The other ranks' values are staged up to kMaxOth points ahead (a ring of
// 1 << oth_lg LDS buffers, one staged count each).
constexpr int kMaxOth = 8;
constexpr int kMaxDBufs = 8;  // D-tile buffers (arrival counts) at most
constexpr int kFlagArrived = 0, kFlagConsumed = kMaxDBufs, kFlagStaged = kMaxDBufs + 1,
              kFlagOthFree = kFlagStaged + kMaxOth,
              kFlagReduced = kFlagOthFree + 1, kFlagDone = kFlagOthFree + 2, kFlagCount = kFlagOthFree + 3;
template <int BT, int SL, int WPS, int NSTG, int NBUF, bool XRM, bool FLAT, int WF = TP_WEIGHTS_BF16>
__global__ __launch_bounds__((2 + NSTG + WPS) * 64) void decode_stream_mfma(MfmaArgs a) {
    constexpr int TB = tile_bytes<WF>();
    static_assert(NBUF <= kMaxDBufs, "one arrival count per D-tile buffer");
    constexpr int kRed = WPS * BT * 256;                  // floats of one buffer
    __shared__ __align__(16) float red[NBUF * kRed];       // [NBUF][WPS][BT][64][4] D tiles
    __shared__ __align__(16) float hs[kMaxOwn * BT * 256]; // owned strips' hidden state, [token][16]
    __shared__ __align__(16) float vr[2 * BT * 256];       // segment e's partial in vr[e & 1], [token][16]
    // LDS flags: arrivals per D-tile buffer, segments consumed, stagers done
    // per parity of point, points whose other values have been read
    __shared__ int flags[kFlagCount];
    __shared__ int segtab[2][kMaxSeg][4];
    __shared__ int nseg[2];
    __shared__ int s_last;
    extern __shared__ __align__(16) float oth[];           // [1 << oth_lg][own][(N-1) * B][16] other ranks

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Workgroups are dealt to the 8 XCDs in turn (workgroup w runs on XCD
    // w % 8); neighbouring ranges of tiles go to the same XCD, so that the
    // 128-byte lines that two neighbouring strips share (16 columns are 64
    // bytes of a row of the fp32 slots and of the hidden state) are fetched
    // into one L2 rather than two.
    const int g = xcd_range_index((int)blockIdx.x, (int)gridDim.x);
    const int n_points = 2 * a.layers;
    const int B = a.batch;
    const int len = B * a.H;
    const int noth = 1 << a.oth_lg;  // buffers of the other ranks' values (points staged ahead)
    // strips whose kb = 0 tile is ours: [own0, own0 + nown)
    const int own0 = (int)(((int64_t)g * a.S16 + a.G - 1) / a.G);
    const int nown = (int)(((int64_t)(g + 1) * a.S16 + a.G - 1) / a.G) - own0;

    if (tid == 0) {
        nseg[0] = wg_segments(g, a.G, a.S16, a.nkb0, segtab[0]);
        nseg[1] = wg_segments(g, a.G, a.S16, a.nkb1, segtab[1]);
        for (int f = 0; f < kFlagCount; ++f) flags[f] = 0;
    }

    if (wave == 0) {
        // ---------------------------------------------------- reducer wave
        // Sums each segment's D tiles in wave order into vr[e & 1] as
        // [token][16 columns] (lane l of a D tile holds tokens 16tt +
        // 4(l/16) + k of column l % 16) and frees the D-tile buffer at once;
        // the control wave takes the partial from there, so the compute
        // waves never wait on the ring.
        __builtin_amdgcn_s_setprio(3);
        __syncthreads();  // start
        int e = 0;
        for (int j = 0; j < n_points; ++j) {
            const int ns = nseg[j & 1];
            for (int i = 0; i < ns; ++i, ++e) {
                wait_flag(&flags[kFlagArrived + e % NBUF], (e / NBUF + 1) * WPS, a.err);
                wait_flag(&flags[kFlagDone], e - 1, a.err);  // vr[e & 1] was read for segment e - 2
                lds_wait();
                const float* re = red + (e % NBUF) * kRed;
                float* ve = vr + (e & 1) * BT * 256;
#pragma unroll
                for (int tt = 0; tt < BT; ++tt) {
                    floatx4_t part[WPS];
#pragma unroll
                    for (int wi = 0; wi < WPS; ++wi)
                        part[wi] = *reinterpret_cast<const floatx4_t*>(re + (wi * BT + tt) * 256 + lane * 4);
                    floatx4_t v = part[0];
#pragma unroll
                    for (int wi = 1; wi < WPS; ++wi) v = v + part[wi];
#pragma unroll
                    for (int k = 0; k < 4; ++k) ve[(16 * tt + 4 * (lane >> 4) + k) * 16 + (lane & 15)] = v[k];
                }
                lds_wait();
                if (lane == 0) {
                    lds_st(&flags[kFlagConsumed], e + 1);  // its D-tile buffer is free again
                    lds_st(&flags[kFlagReduced], e + 1);
                }
            }
        }
    } else if (wave == 1) {
        // ---------------------------------------------------- control wave
        // Works in the [token][16 columns] layout: lane l takes token
        // 16tt + l/4 and columns 4(l%4) .. +3 of a strip (16-byte LDS and
        // global accesses throughout).
        __builtin_amdgcn_s_setprio(2);
        const int tl = lane >> 2, c4 = 4 * (lane & 3);
        for (int o = 0; o < nown; ++o)
#pragma unroll
            for (int tt = 0; tt < BT; ++tt) {
                const int tok = 16 * tt + tl;
                floatx4_t h = floatx4_t{0.f, 0.f, 0.f, 0.f};
                if (tok < B)
                    h = *reinterpret_cast<const floatx4_t*>(a.hidden + (int64_t)tok * a.H + 16 * (own0 + o) + c4);
                *reinterpret_cast<floatx4_t*>(hs + (o * BT + tt) * 256 + lane * 4) = h;
            }
        const uint32_t xbytes = (uint32_t)((int64_t)2 * kXchgRing * a.S16 * BT * 1024);
        const __amdgpu_buffer_rsrc_t rx = dev_rsrc(a.xpart, xbytes);
        const int N = a.n_ranks;
        const int bs = B * 16;                 // LDS floats per other rank
        const bool quad_chunks = a.chunk % 4 == 0;  // a lane's four columns lie in one chunk
        int ok = 1;
        __syncthreads();  // start: segment tables, flags and hidden columns are in LDS
        int e = 0;
        for (int j = 0; j < n_points; ++j) {
            const int t = j & 1;
            const int ns = nseg[t];
            bool staged = false;
            for (int i = 0; i < ns; ++i, ++e) {
                const int s = segtab[t][i][0], role = segtab[t][i][3];
                wait_flag(&flags[kFlagReduced], e + 1, a.err);  // segment e's partial is in vr[e & 1]
                lds_wait();
                float* ve = vr + (e & 1) * BT * 256;
                // exchange buffer of this kind of point and strip: slot (j/2) mod R,
                // last used at point j - 2R
                const int jj = j >> 1;
                const uint32_t xoff = (uint32_t)((((int64_t)t * kXchgRing + jj % kXchgRing) * a.S16 + s) * BT * 1024);
                uint32_t* pub = a.pub + t * a.S16 + s;
                uint32_t* ack = a.ack + t * a.S16 + s;
                if (role == kContrib) {
                    if (jj >= kXchgRing && ok) {
                        if (lane == 0) ok = wait_at_least(ack, (uint32_t)(j - 2 * kXchgRing + 1), a.err, a.spin_limit);
                        ok = __builtin_amdgcn_readfirstlane(ok);
                    }
#pragma unroll
                    for (int tt = 0; tt < BT; ++tt)
                        st_dev4(rx, xoff + (uint32_t)((tt * 64 + lane) * 16),
                                *reinterpret_cast<const floatx4_t*>(ve + tt * 256 + lane * 4));
                    wait_mem();
                    if (lane == 0) {
                        st_dev_u32(pub, (uint32_t)(j + 1));
                        lds_st(&flags[kFlagDone], e + 1);  // vr[e & 1] may be refilled
                    }
                    continue;
                }
                if (role == kOwnerPart) {
                    // the contributor's rows come after ours
                    if (ok) {
                        if (lane == 0) ok = wait_at_least(pub, (uint32_t)(j + 1), a.err, a.spin_limit);
                        ok = __builtin_amdgcn_readfirstlane(ok);
                    }
                    floatx4_t c[BT];
#pragma unroll
                    for (int tt = 0; tt < BT; ++tt) c[tt] = ld_dev4(rx, xoff + (uint32_t)((tt * 64 + lane) * 16));
                    wait_mem();
                    if (lane == 0) st_dev_u32(ack, (uint32_t)(j + 1));
#pragma unroll
                    for (int tt = 0; tt < BT; ++tt) {
                        float* vp = ve + tt * 256 + lane * 4;
                        *reinterpret_cast<floatx4_t*>(vp) = *reinterpret_cast<const floatx4_t*>(vp) + c[tt];
                    }
                }
                if (!staged) {
                    // point j's other values are in LDS (every stager has counted
                    // its buffer's rounds up to point j)
                    wait_flag(&flags[kFlagStaged + (j & (noth - 1))], NSTG * ((j >> a.oth_lg) + 1), a.err);
                    lds_wait();
                    staged = true;
                }
                // Ring order: chunk c starts at rank c, then c+1, ... (mod N); then
                // the residual. Along that order the other ranks come as a rotation
                // of their rows 0 .. N-2 (row q = rank q, or q+1 past our rank)
                // starting at row c (c - 1 past our rank; row 0 if that is N - 1),
                // and our own value sits at position (rank - c) mod N.
                const int o = s - own0;
                const float* oj = oth + ((j & (noth - 1)) * a.own_max + o) * a.oth_strip;
                float* slot = a.slots + (int64_t)j * a.n_ranks * len + (int64_t)a.rank * len;
                float* hso = hs + o * BT * 256;
#pragma unroll 1
                for (int tt = 0; tt < BT; ++tt) {
#pragma clang fp contract(off)
                    const int tok = 16 * tt + tl;
                    const int tokc = tok < B ? tok : B - 1;
                    const floatx4_t v = *reinterpret_cast<const floatx4_t*>(ve + tt * 256 + lane * 4);
                    const floatx4_t h = *reinterpret_cast<const floatx4_t*>(hso + tt * 256 + lane * 4);
                    const float* ob = oj + tokc * 16 + c4;
                    const int idx = tokc * a.H + 16 * s + c4;
                    floatx4_t sum;
                    if (quad_chunks) {
                        const int cc = idx / a.chunk;
                        int p = a.rank - cc;
                        p = p < 0 ? p + N : p;
                        int q = cc > a.rank ? cc - 1 : cc;
                        q = q >= N - 1 ? 0 : q;
                        // all eight loads are issued before the first add (q stays
                        // within rows 0 .. max(N - 2, 0); positions u >= N are unused)
                        floatx4_t x[8];
#pragma unroll
                        for (int u = 0; u < 8; ++u) {
                            x[u] = *reinterpret_cast<const floatx4_t*>(ob + q * bs);
                            if (u != p) q = q + 1 >= N - 1 ? 0 : q + 1;
                        }
#pragma unroll
                        for (int k = 0; k < 4; ++k) sum[k] = p == 0 ? v[k] : x[0][k];
#pragma unroll
                        for (int u = 1; u < 8; ++u)
                            if (u < N) {
                                floatx4_t y;
#pragma unroll
                                for (int k = 0; k < 4; ++k) y[k] = u == p ? v[k] : x[u][k];
                                sum = sum + y;
                            }
                    } else {
                        // a chunk boundary may fall between a lane's columns
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            const int cc = (idx + k) / a.chunk;
                            int p = a.rank - cc;
                            p = p < 0 ? p + N : p;
                            int q = cc > a.rank ? cc - 1 : cc;
                            q = q == N - 1 ? 0 : q;
                            float sk = v[k];
                            for (int u = 0; u < N; ++u) {
                                const bool own = u == p;
                                const float y = own ? v[k] : ob[q * bs + k];
                                sk = u > 0 ? sk + y : y;
                                if (!own) q = q + 1 == N - 1 ? 0 : q + 1;
                            }
                            sum[k] = sk;
                        }
                    }
                    if (tok < B) {
                        *reinterpret_cast<floatx4_t*>(hso + tt * 256 + lane * 4) = sum + h;
                        *reinterpret_cast<floatx4_t*>(slot + (int64_t)tok * a.H + 16 * s + c4) = v;
                    }
                }
                lds_wait();
                if (lane == 0) lds_st(&flags[kFlagDone], e + 1);  // vr[e & 1] may be refilled
            }
            // the other values of point j have been read: their buffer may be refilled (point j + noth)
            lds_wait();
            if (lane == 0) lds_st(&flags[kFlagOthFree], j + 1);
        }
        lds_wait();
        for (int o = 0; o < nown; ++o)
#pragma unroll
            for (int tt = 0; tt < BT; ++tt) {
                const int tok = 16 * tt + tl;
                if (tok < B)
                    *reinterpret_cast<floatx4_t*>(a.hidden + (int64_t)tok * a.H + 16 * (own0 + o) + c4) =
                        *reinterpret_cast<const floatx4_t*>(hs + (o * BT + tt) * 256 + lane * 4);
            }
        wait_mem();
    } else if (wave <= 1 + NSTG) {
        // ---------------------------------------------------- stager waves
        // The other ranks' 16 values per token of each owned strip, rows
        // ordered (other rank, token), staged with direct global->LDS loads
        // into buffer j mod noth, up to noth - 1 points ahead of the control
        // wave (a load waits behind the weight stream's loads in flight,
        // several microseconds, longer than two small points take); stager
        // q issues every NSTG-th load.
        const int q = wave - 2;
        __syncthreads();  // start
        const int rows = (a.n_ranks - 1) * B;
        const int per_strip = (rows + 15) / 16;
        for (int j = 0; j < n_points; ++j) {
            // buffer j mod noth was last read at point j - noth
            wait_flag(&flags[kFlagOthFree], j - (noth - 1), a.err);
            const float* slot = a.slots + (int64_t)j * a.n_ranks * len;
            for (int n = q; n < nown * per_strip; n += NSTG) {
                const int o = n / per_strip, r0 = (n - o * per_strip) * 16;
                int row = r0 + lane / 4;
                row = row < rows ? row : rows - 1;
                const int ro = row / B, tok = row - ro * B;
                const int r = ro < a.rank ? ro : ro + 1;
                const float* src = slot + (int64_t)r * len + (int64_t)tok * a.H + 16 * (own0 + o) + 4 * (lane & 3);
                float* dst = oth + ((j & (noth - 1)) * a.own_max + o) * a.oth_strip + r0 * 16;
                __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src), (lds_void_t*)dst, 16, 0, 0);
            }
            wait_mem();
            if (lane == 0) lds_add(&flags[kFlagStaged + (j & (noth - 1))], 1);
        }
    } else {
        // --------------------------------------------------- compute waves
        const int wi = wave - 2 - NSTG;
        __syncthreads();  // start: the segment tables are in LDS
        // whole strips start their walk at different places (a rotation by
        // whole rounds of WPS tiles), so that workgroups do not all read the
        // same rows of x at the same moment
        auto seg_fields = [&](const int* tb, Cursor& c) {
            c.s = tb[0];
            c.kb0 = tb[1];
            c.len = tb[2];
            c.bpw = (c.len + WPS - 1) / WPS;
            c.rot = tb[3] == kFull ? (g % c.bpw) * WPS : 0;
        };
        // The first segment of each kind of point (every segment where
        // strips stay whole) is read and its walk worked out once, so that
        // a bank's issue needs no LDS read or division at small points.
        Cursor first0{}, first1{};
        seg_fields(segtab[0][0], first0);
        seg_fields(segtab[1][0], first1);
        const int nseg0 = nseg[0], nseg1 = nseg[1];  // segments per kind of point
        auto set_seg = [&](Cursor& c) {
            if (c.j >= n_points) return;
            if (c.i == 0) {
                const Cursor& f = (c.j & 1) ? first1 : first0;
                c.s = f.s;
                c.kb0 = f.kb0;
                c.len = f.len;
                c.bpw = f.bpw;
                c.rot = f.rot;
                return;
            }
            seg_fields(segtab[c.j & 1][c.i], c);
        };
        auto advance = [&](Cursor& c) {
            c.m0 += SL;
            if (c.m0 >= c.bpw) {
                c.m0 = 0;
                if (++c.i >= ((c.j & 1) ? nseg1 : nseg0)) {
                    c.i = 0;
                    ++c.j;
                }
                set_seg(c);
            }
        };
        // A operand of lane l: token 16*tt + l%16, rows 16*(l/16) + 8h .. +7 of
        // the tile, 16 contiguous bytes of the packed activations (XRM: of
        // the token's row of x; the 4 lanes of a token and both halves then
        // read one 128-byte line)
        auto issue = [&](u32x4_t (&wv)[SL][2], uint32_t (&sv)[SL], u32x4_t (&xv)[SL][2][BT], const Cursor& c) {
            const int t = c.j & 1, l = c.j >> 1;
            const bool live = c.j < n_points;
            const int nkb = t ? a.nkb1 : a.nkb0;
            const int K = t ? a.K1 : a.K0;
            const char* wb = reinterpret_cast<const char*>(t ? a.w1 : a.w0) + ((int64_t)l * a.S16 + c.s) * nkb * TB;
            const uint16_t* xb = (t ? a.x1 : a.x0) + (XRM ? (int64_t)l * B * K : (int64_t)l * nkb * BT * 1024);
            const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<char*>(live ? wb : reinterpret_cast<const char*>(a.w0)), (short)0, live ? nkb * TB : 0,
                kBufferRsrcWord3);
            const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint16_t*>(live ? xb : a.x0), (short)0,
                live ? (XRM ? B * K * 2 : nkb * BT * 2048) : 0, kBufferRsrcWord3);
            // slots past the segment's tiles read zero (tile nkb is past the
            // strip), and so do the lanes of tokens past b (an offset past the
            // range: their packed entries are never read)
            const int span = c.bpw * WPS;
#pragma unroll
            for (int i = 0; i < SL; ++i) {
                int kl = wi + (c.m0 + i) * WPS + c.rot;
                kl = kl >= span ? kl - span : kl;
                const int kb = (c.m0 + i < c.bpw && kl < c.len) ? c.kb0 + kl : nkb;
                load_w_tile<WF>(wr, kb, lane, wv[i], sv[i]);
#pragma unroll
                for (int tt = 0; tt < BT; ++tt)
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        // rows past K (K is a multiple of 8: a lane's 8 rows are all
                        // inside or all past) and tokens past b read zero
                        const int tok = 16 * tt + (lane & 15);
                        const int k = kb * kTileRows + 16 * (lane >> 4) + 8 * h;
                        const int off = XRM ? (tok < B && k < K ? (tok * K + k) * 2 : 0x7ffffff0)
                                            : (tok < B ? ((kb * BT + tt) * 2 + h) * 1024 + lane * 16 : 0x7ffffff0);
                        xv[i][h][tt] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                                       xr, off, 0, 0));
                    }
            }
        };
        floatx4_t acc[BT];
#pragma unroll
        for (int tt = 0; tt < BT; ++tt) acc[tt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
        auto consume = [&](const u32x4_t (&wv)[SL][2], const uint32_t (&sv)[SL], const u32x4_t (&xv)[SL][2][BT]) {
#pragma unroll
            for (int i = 0; i < SL; ++i)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const bf16x8_t wb = b_operand<WF>(wv[i], sv[i], h);
#pragma unroll
                    for (int tt = 0; tt < BT; ++tt)
                        acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8_t, xv[i][h][tt]), wb, acc[tt], 0, 0, 0);
                }
        };
        int e = 0;
        auto seg_end = [&]() {
            // D-tile buffer e % NBUF is free once the control wave has read segment e - NBUF
            wait_flag(&flags[kFlagConsumed], e - (NBUF - 1), a.err);
            float* re = red + (e % NBUF) * kRed + wi * BT * 256;
#pragma unroll
            for (int tt = 0; tt < BT; ++tt) {
                *reinterpret_cast<floatx4_t*>(re + (tt * 64 + lane) * 4) = acc[tt];
                acc[tt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
            }
            lds_wait();
            if (lane == 0) lds_add(&flags[kFlagArrived + e % NBUF], 1);
            ++e;
        };

        if constexpr (FLAT) {
            // A ring of 2 SL tile slots, each refilled with the wave's tile
            // 2 SL further on as soon as it is consumed, across segment and
            // point boundaries (small segments would leave most of a bank
            // empty). Every slot issues the same loads (empty ranges past a
            // segment's tiles or past the step), so the waits stay exact.
            auto slot_fields = [&](const int* tb, SlotCursor& c) {
                c.s = tb[0];
                c.kb0 = tb[1];
                const int len = tb[2];
                c.nr = len > wi ? (len - wi + WPS - 1) / WPS : 0;
                c.ns = c.nr > 0 ? c.nr : 1;
                c.r0 = tb[3] == kFull && c.nr > 0 ? g % c.nr : 0;
            };
            // the first segment of each kind worked out once (as for the banks)
            SlotCursor sfirst0{}, sfirst1{};
            slot_fields(segtab[0][0], sfirst0);
            slot_fields(segtab[1][0], sfirst1);
            auto fset = [&](SlotCursor& c) {
                if (c.j >= n_points) return;
                if (c.i == 0) {
                    const SlotCursor& f = (c.j & 1) ? sfirst1 : sfirst0;
                    c.s = f.s;
                    c.kb0 = f.kb0;
                    c.nr = f.nr;
                    c.ns = f.ns;
                    c.r0 = f.r0;
                    return;
                }
                slot_fields(segtab[c.j & 1][c.i], c);
            };
            auto fadv = [&](SlotCursor& c) {
                if (c.j >= n_points) return;
                if (++c.m >= c.ns) {
                    c.m = 0;
                    if (++c.i >= ((c.j & 1) ? nseg1 : nseg0)) {
                        c.i = 0;
                        ++c.j;
                    }
                    fset(c);
                }
            };
            auto fissue = [&](u32x4_t (&wv)[2], uint32_t& sv, u32x4_t (&xv)[2][BT], const SlotCursor& c) {
                const int t = c.j & 1, l = c.j >> 1;
                const bool live = c.j < n_points;
                const int nkb = t ? a.nkb1 : a.nkb0;
                const int K = t ? a.K1 : a.K0;
                const char* wb = reinterpret_cast<const char*>(t ? a.w1 : a.w0) + ((int64_t)l * a.S16 + c.s) * nkb * TB;
                const uint16_t* xb = (t ? a.x1 : a.x0) + (XRM ? (int64_t)l * B * K : (int64_t)l * nkb * BT * 1024);
                const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
                    const_cast<char*>(live ? wb : reinterpret_cast<const char*>(a.w0)), (short)0,
                    live ? nkb * TB : 0, kBufferRsrcWord3);
                const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
                    const_cast<uint16_t*>(live ? xb : a.x0), (short)0,
                    live ? (XRM ? B * K * 2 : nkb * BT * 2048) : 0, kBufferRsrcWord3);
                int kb = nkb;  // an empty slot: past the strip, reads zero
                if (c.nr > 0) {
                    int mm = c.m + c.r0;
                    mm = mm >= c.nr ? mm - c.nr : mm;
                    kb = c.kb0 + wi + mm * WPS;
                }
                load_w_tile<WF>(wr, kb, lane, wv, sv);
#pragma unroll
                for (int tt = 0; tt < BT; ++tt)
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int tok = 16 * tt + (lane & 15);
                        const int k = kb * kTileRows + 16 * (lane >> 4) + 8 * h;
                        const int off = XRM ? (tok < B && k < K ? (tok * K + k) * 2 : 0x7ffffff0)
                                            : (tok < B ? ((kb * BT + tt) * 2 + h) * 1024 + lane * 16 : 0x7ffffff0);
                        xv[h][tt] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                                    xr, off, 0, 0));
                    }
            };
            u32x4_t wr_[2 * SL][2], xr_[2 * SL][2][BT];
            uint32_t sr_[2 * SL];
            SlotCursor fi{0, 0, 0, 0, 0, 0, 0, 0}, fc;
            fset(fi);
            fc = fi;
#pragma unroll
            for (int q = 0; q < 2 * SL; ++q) {
                fissue(wr_[q], sr_[q], xr_[q], fi);
                fadv(fi);
            }
            while (fc.j < n_points) {
#pragma unroll
                for (int q = 0; q < 2 * SL; ++q) {
                    bool last = false;
                    if (fc.j < n_points) {
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const bf16x8_t wb = b_operand<WF>(wr_[q], sr_[q], h);
#pragma unroll
                            for (int tt = 0; tt < BT; ++tt)
                                acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    __builtin_bit_cast(bf16x8_t, xr_[q][h][tt]), wb, acc[tt], 0, 0, 0);
                        }
                        last = fc.m == fc.ns - 1;
                        fadv(fc);
                    }
                    fissue(wr_[q], sr_[q], xr_[q], fi);
                    fadv(fi);
                    if (last) seg_end();
                }
            }
        } else {
        u32x4_t w0[SL][2], w1[SL][2], x0[SL][2][BT], x1[SL][2][BT];
        uint32_t s0[SL], s1[SL];
        Cursor ci{0, 0, 0, 0, 0, 0, 0, 0}, cc;
        set_seg(ci);
        cc = ci;
        issue(w0, s0, x0, ci);
        advance(ci);
        issue(w1, s1, x1, ci);
        advance(ci);
        while (cc.j < n_points) {
            {
                consume(w0, s0, x0);
                const bool last = cc.m0 + SL >= cc.bpw;
                advance(cc);
                issue(w0, s0, x0, ci);
                advance(ci);
                if (last) seg_end();
            }
            {
                const bool live = cc.j < n_points;
                bool last = false;
                if (live) {
                    consume(w1, s1, x1);
                    last = cc.m0 + SL >= cc.bpw;
                    advance(cc);
                }
                issue(w1, s1, x1, ci);
                advance(ci);
                if (last) seg_end();
            }
        }
        }
    }
    // The last workgroup to leave clears the exchange flags for the next
    // launch (no workgroup reads them any more).
    __syncthreads();
    if (tid == 0) s_last = add_dev_u32(a.exit_ctr, 1u) == gridDim.x - 1;
    __syncthreads();
    if (s_last) {
        for (int w = tid; w < 2 * a.S16; w += blockDim.x) {
            st_dev_u32(a.pub + w, 0u);
            st_dev_u32(a.ack + w, 0u);
        }
        if (tid == 0) st_dev_u32(a.exit_ctr, 0u);
    }
}

typedef void (*mfma_stream_fn)(MfmaArgs);

// Tiles per bank: fewer for more token blocks (each tile also carries 2*BT
// A operands), so the banks fit the registers. The waves of a workgroup are
// spread over the CU's four SIMDs in turn, and on each SIMD the oldest wave
// is served first: with one reducer, control or stager wave per SIMD and the same
// number of compute waves on every SIMD (12, or 8 for three and four token
// blocks, where the LDS of their D tiles is short), no SIMD carries more of
// the stream than another. D-tile buffers: 4, or fewer where the LDS is short.
constexpr int kWps[5] = {0, 8, 12, 8, 8};
constexpr int kSl[5] = {0, 3, 2, 1, 1};
constexpr int kFlatFromBatch = 8;  // one token block: the slot ring from this batch on
constexpr int kStagers[5] = {0, 2, 2, 2, 2};
constexpr int kDBufs[5] = {0, 4, 3, 2, 2};  // D-tile buffers (LDS)
// One token block: tiles per bank and compute waves may be chosen (plan
// knobs), and so may the activations' layout (row-major or A-operand order).
// One and two token blocks: banks of 2 tiles on 12 compute waves, or of
// 3 on 8 (fewer waves per SIMD, the same tiles in flight), each with a bank
// per segment or a ring of slots across segments (FLAT); one token block may
// read row-major activations (XRM).
template <int BT, bool XRM, bool FLAT>
mfma_stream_fn mfma_stream_kernel_v(int sl, int wps) {
    if (wps == 12 && sl == 2) return decode_stream_mfma<BT, 2, 12, kStagers[BT], kDBufs[BT], XRM, FLAT>;
    if (wps == 8 && sl == 3) return decode_stream_mfma<BT, 3, 8, kStagers[BT], kDBufs[BT], XRM, FLAT>;
    return nullptr;
}
// Microscaled weights: one token block, banks of 3 tiles on 8 waves.
template <int WF>
mfma_stream_fn mfma_stream_kernel_mx(const MfmaGeom& g) {
    if (g.bt != 1 || g.sl != 3 || g.wps != 8) return nullptr;
    if (g.flat) return g.acts_rm ? decode_stream_mfma<1, 3, 8, kStagers[1], kDBufs[1], true, true, WF>
                                 : decode_stream_mfma<1, 3, 8, kStagers[1], kDBufs[1], false, true, WF>;
    return g.acts_rm ? decode_stream_mfma<1, 3, 8, kStagers[1], kDBufs[1], true, false, WF>
                     : decode_stream_mfma<1, 3, 8, kStagers[1], kDBufs[1], false, false, WF>;
}
mfma_stream_fn mfma_stream_kernel(const MfmaGeom& g) {
    if (g.wf == TP_WEIGHTS_MXFP8) return mfma_stream_kernel_mx<TP_WEIGHTS_MXFP8>(g);
    if (g.wf == TP_WEIGHTS_MXFP4) return mfma_stream_kernel_mx<TP_WEIGHTS_MXFP4>(g);
    switch (g.bt) {
        case 1:
            if (g.flat) return g.acts_rm ? mfma_stream_kernel_v<1, true, true>(g.sl, g.wps)
                                         : mfma_stream_kernel_v<1, false, true>(g.sl, g.wps);
            return g.acts_rm ? mfma_stream_kernel_v<1, true, false>(g.sl, g.wps)
                             : mfma_stream_kernel_v<1, false, false>(g.sl, g.wps);
        case 2:
            return g.flat ? mfma_stream_kernel_v<2, false, true>(g.sl, g.wps)
                          : mfma_stream_kernel_v<2, false, false>(g.sl, g.wps);
        case 3: return decode_stream_mfma<3, kSl[3], kWps[3], kStagers[3], kDBufs[3], false, false>;
        case 4: return decode_stream_mfma<4, kSl[4], kWps[4], kStagers[4], kDBufs[4], false, false>;
    }
    return nullptr;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Compute units of the current device (cached per device).
int device_cus() {
    static int cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (cus[dev] <= 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cus[dev] = n;
    }
    return cus[dev];
}

}  // namespace

bool tp_mfma_geometry(const tp_plan_s* p, MfmaGeom* g) {
    const int b = p->batch;
    if (b < 1 || b > kMfmaMaxBatch || p->n_ranks > 8 || p->hidden % 16) return false;
    const int64_t k0 = p->k_attn / p->n_ranks, k1 = p->inter / p->n_ranks;
    if (k0 % 8 || k1 % 8) return false;
    const int64_t S16 = p->hidden / 16;
    int64_t G = p->stream_wgs > 0 ? p->stream_wgs : kTargetCUs;
    if (G > S16) G = S16;
    // every workgroup's range covers at least one strip's tiles and at most
    // two strips' (at most kMaxSeg segments, kMaxOwn owned strips)
    if (S16 > 2 * G || S16 > kXchgMaxStrips) return false;
    const int bt = (b + 15) / 16;
    // knobs for one and two token blocks (the kernel has those variants only)
    const bool knobs = bt <= 2;
    const int wps = knobs && p->mfma_wps ? p->mfma_wps : kWps[bt], nstg = kStagers[bt];
    const int sl = knobs && p->mfma_sl ? p->mfma_sl : kSl[bt];
    if (knobs && !((wps == 12 && sl == 2) || (wps == 8 && sl == 3))) return false;
    // microscaled weights: up to 16 tokens, banks of 3 on 8 waves, K_r in
    // whole 32-row scale blocks
    const int wf = p->weight_format;
    if (wf != TP_WEIGHTS_BF16 && (bt != 1 || sl != 3 || wps != 8 || k0 % 32 || k1 % 32)) return false;
    const int tbytes = wf == TP_WEIGHTS_MXFP8 ? tile_bytes<TP_WEIGHTS_MXFP8>()
                       : wf == TP_WEIGHTS_MXFP4 ? tile_bytes<TP_WEIGHTS_MXFP4>() : kTileBytes;
    const int nbuf = kDBufs[bt];
    // activations: row-major up to 8 tokens (read directly, no layout
    // launch per step), else in A-operand order (1 KB per operand load)
    const bool acts_rm = p->mfma_acts == 1 || (p->mfma_acts == 0 && b <= kMfmaRowMajorActsMax);
    if (acts_rm && bt != 1) return false;
    const int64_t nkb0 = (k0 + kTileRows - 1) / kTileRows, nkb1 = (k1 + kTileRows - 1) / kTileRows;
    // the ring of slots: from kFlatFromBatch tokens, and for bf16 weights
    // where a layer's tiles per compute wave (whole strips) fit its 2 SL
    // slots (small points: measured 1-6 % faster at H4096 N=8, 1-4 tokens;
    // 1-2 % slower at N=4, whose points fill the banks)
    const bool small_layer = (nkb0 + wps - 1) / wps + (nkb1 + wps - 1) / wps <= 2 * sl;
    const bool flat = knobs && (p->mfma_flat == 1 ||
                                (p->mfma_flat < 0 && bt == 1 &&
                                 (b >= kFlatFromBatch || (small_layer && wf == TP_WEIGHTS_BF16))));
    // static LDS: D tiles of both parities, owned hidden state, a segment's
    // partial, tables; dynamic: the other ranks' values of the owned strips
    // (room for one rank's values even with N = 1, so that the clamped reads
    // of a single-rank plan stay inside the allocation)
    const int own_max = (int)((S16 + G - 1) / G);
    g->oth_strip = (int32_t)(((p->n_ranks > 1 ? p->n_ranks - 1 : 1) * b * 16 + 255) / 256 * 256);
    g->own_max = own_max;
    // staged points: the knob, else 2 (deeper staging measured no faster)
    int noth = p->mfma_oth ? p->mfma_oth : 2;
    g->lds_bytes = noth * own_max * g->oth_strip * 4;
    const int64_t stat = (nbuf * wps * bt * 256 + kMaxOwn * bt * 256 + 2 * bt * 256) * 4 + 1024;
    while (!p->mfma_oth && noth > 2 && g->lds_bytes + stat > 152 * 1024) {
        noth /= 2;
        g->lds_bytes = noth * own_max * g->oth_strip * 4;
    }
    if (g->lds_bytes + stat > 152 * 1024) return false;
    g->oth_lg = noth == 8 ? 3 : noth == 4 ? 2 : 1;
    // the largest buffer offsets must fit 32 bits
    if ((nkb0 > nkb1 ? nkb0 : nkb1) * (int64_t)(tbytes > kTileBytes * bt ? tbytes : kTileBytes * bt) >=
        ((int64_t)1 << 31))
        return false;
    if ((int64_t)b * p->hidden >= ((int64_t)1 << 31)) return false;
    if (acts_rm && (int64_t)b * (k0 > k1 ? k0 : k1) * 2 >= ((int64_t)1 << 31)) return false;
    g->grid = (int32_t)G;
    g->wps = wps;
    g->bt = bt;
    g->sl = sl;
    g->acts_rm = acts_rm ? 1 : 0;
    g->flat = flat ? 1 : 0;
    g->wf = wf;
    g->tile_bytes = tbytes;
    g->block = (2 + nstg + wps) * 64;
    g->nkb0 = (int32_t)nkb0;
    g->nkb1 = (int32_t)nkb1;
    return true;
}

int64_t tp_xchg_bytes(const tp_plan_s* p) {
    if (p->batch < 1 || p->batch > kMfmaMaxBatch || p->hidden % 16) return 0;
    const int64_t S16 = p->hidden / 16;
    if (S16 > kXchgMaxStrips) return 0;
    return 2 * kXchgRing * S16 * ((p->batch + 15) / 16) * 1024;
}

tp_status tp_pack_acts(const tp_plan_s* p, int n_layers, const void* x_attn, const void* x_ffn,
                       void* xa_packed, void* xf_packed, void* stream) {
    const int64_t K0 = p->k_attn / p->n_ranks, K1 = p->inter / p->n_ranks;
    const int64_t bt = (p->batch + 15) / 16;
    const int64_t total = (int64_t)n_layers * ((K0 + kTileRows - 1) / kTileRows + (K1 + kTileRows - 1) / kTileRows) * bt * 128;
    if (total == 0) return TP_OK;
    const int64_t blocks = (total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536;
    hipLaunchKernelGGL(pack_acts_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       static_cast<const uint16_t*>(x_attn), static_cast<const uint16_t*>(x_ffn),
                       static_cast<uint16_t*>(xa_packed), static_cast<uint16_t*>(xf_packed),
                       (int64_t)n_layers, (int64_t)p->batch, K0, K1, bt);
    return tp_launch_status(stream);
}

tp_status tp_pack_tile_stack(int64_t n_mats, int64_t K, int64_t H, const void* w, void* w_packed,
                             void* stream) {
    const int64_t total = n_mats * (H / 16) * ((K + kTileRows - 1) / kTileRows) * 128;
    if (total == 0) return TP_OK;
    const int64_t blocks = (total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536;
    hipLaunchKernelGGL(pack_tiles_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       static_cast<const uint16_t*>(w), static_cast<uint16_t*>(w_packed), n_mats, K, H);
    return tp_launch_status(stream);
}

tp_status tp_pack_tiles(const tp_plan_s* p, int point, int n_layers, const void* w, void* w_packed,
                        void* stream) {
    const int64_t K = (point == TP_POINT_ATTN_OUT ? p->k_attn : p->inter) / p->n_ranks;
    return tp_pack_tile_stack(n_layers, K, p->hidden, w, w_packed, stream);
}

tp_status tp_mx_pack_tiles(const tp_plan_s* p, int point, int n_layers, const void* codes,
                           const void* scales, void* w_packed, void* stream) {
    const int64_t K = (point == TP_POINT_ATTN_OUT ? p->k_attn : p->inter) / p->n_ranks;
    const int64_t total = (int64_t)n_layers * (p->hidden / 16) * ((K + kTileRows - 1) / kTileRows) * 64;
    if (total == 0) return TP_OK;
    const int64_t blocks = (total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536;
    auto k = p->weight_format == TP_WEIGHTS_MXFP8 ? pack_mx_tiles_kernel<TP_WEIGHTS_MXFP8>
                                                  : pack_mx_tiles_kernel<TP_WEIGHTS_MXFP4>;
    hipLaunchKernelGGL(k, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       static_cast<const uint8_t*>(codes), static_cast<const uint8_t*>(scales),
                       static_cast<uint8_t*>(w_packed), (int64_t)n_layers, K, p->hidden);
    return tp_launch_status(stream);
}

int64_t tp_mfma_packed_bytes(const tp_plan_s* p, int point, int64_t n_layers) {
    MfmaGeom g;
    if (!tp_mfma_geometry(p, &g)) return 0;
    return n_layers * (p->hidden / 16) * (point == TP_POINT_ATTN_OUT ? g.nkb0 : g.nkb1) * g.tile_bytes;
}

tp_status tp_decode_mfma_stream(const tp_plan_s* p, int32_t n_layers, int32_t rank,
                                const void* x_attn, const void* w_o_tiles, const void* x_ffn,
                                const void* w_down_tiles, float* slots, float* hidden, void* ws,
                                void* stream) {
    return tp_decode_mfma_stream_at(p, n_layers, rank, x_attn, w_o_tiles, x_ffn, w_down_tiles, slots,
                                    hidden, ws,
                                    reinterpret_cast<float*>(static_cast<char*>(ws) + tp_ws_xchg_offset(p)),
                                    stream);
}

tp_status tp_decode_mfma_stream_at(const tp_plan_s* p, int32_t n_layers, int32_t rank,
                                   const void* x_attn, const void* w_o_tiles, const void* x_ffn,
                                   const void* w_down_tiles, float* slots, float* hidden, void* ws,
                                   float* xpart, void* stream) {
    MfmaGeom geo;
    if (!tp_mfma_geometry(p, &geo)) return TP_ERR_UNSUPPORTED;
    if (!aligned16(x_attn) || !aligned16(x_ffn) || !aligned16(w_o_tiles) || !aligned16(w_down_tiles) ||
        !aligned16(slots) || !aligned16(hidden) || !aligned16(ws) || !aligned16(xpart))
        return TP_ERR_ALIGNMENT;
    if (n_layers == 0) return TP_OK;
    mfma_stream_fn k = mfma_stream_kernel(geo);
    if (!k) return TP_ERR_UNSUPPORTED;
    MfmaArgs a;
    a.x0 = static_cast<const uint16_t*>(x_attn);
    a.x1 = static_cast<const uint16_t*>(x_ffn);
    a.w0 = static_cast<const uint16_t*>(w_o_tiles);
    a.w1 = static_cast<const uint16_t*>(w_down_tiles);
    a.slots = slots;
    a.hidden = hidden;
    char* base = static_cast<char*>(ws);
    a.xpart = xpart;
    a.pub = reinterpret_cast<uint32_t*>(base + kXchgFlagOffset);
    a.ack = a.pub + 2 * kXchgMaxStrips;
    a.exit_ctr = reinterpret_cast<uint32_t*>(base + kXchgExitOffset);
    a.err = reinterpret_cast<uint32_t*>(base + kSyncOffset) + kSyncErr;
    a.H = (int32_t)p->hidden;
    a.S16 = (int32_t)(p->hidden / 16);
    a.G = geo.grid;
    a.batch = p->batch;
    a.K0 = (int32_t)(p->k_attn / p->n_ranks);
    a.K1 = (int32_t)(p->inter / p->n_ranks);
    a.nkb0 = geo.nkb0;
    a.nkb1 = geo.nkb1;
    a.layers = n_layers;
    a.n_ranks = p->n_ranks;
    a.rank = rank;
    a.chunk = (int32_t)((int64_t)p->batch * p->hidden / p->n_ranks);
    a.oth_strip = geo.oth_strip;
    a.own_max = geo.own_max;
    a.oth_lg = geo.oth_lg;
    a.spin_limit = 1u << 20;
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                            hipFuncAttributeMaxDynamicSharedMemorySize, geo.lds_bytes) != hipSuccess)
        return TP_ERR_DEVICE;
    // The exchange waits need every workgroup resident at once: one per CU,
    // so the device must have at least G of them (a partitioned device may
    // have fewer). The waits are bounded either way.
    if (geo.grid > device_cus()) return TP_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(k, dim3((unsigned)geo.grid), dim3((unsigned)geo.block), (unsigned)geo.lds_bytes,
                       (hipStream_t)stream, a);
    return tp_launch_status(stream);
}
