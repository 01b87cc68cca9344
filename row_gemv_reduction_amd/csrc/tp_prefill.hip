// Prefill: the same reconciliation points with a whole prompt of T tokens
// at once ("Interconnects e clusters", lesson 9.9, section 01 · Conceito: a
// 4,096-token prompt runs every position together, so each of the 128
// collectives carries 4,096 hidden vectors; the bytes matter and bandwidth
// governs). Per point the rank's partial is a dense product
//     P[t, n] = sum_k X[t, k] * W[k, n]      (T tokens x H columns, K = K_r)
// on the bf16 matrix cores, written to the rank's slot, and the ring-order
// sum of the N ranks' partials plus the residual updates the hidden state,
// fused into the product's epilogue.
//
// prefill_step: one persistent launch over every point of the stack. The
// tiles of 128 tokens x 256 columns are taken in point order by all resident
// workgroups (two per CU). A workgroup of 4 waves (2 x 2, each 64 tokens x
// 128 columns: 4 x 8 blocks of v_mfma_f32_16x16x32_bf16) stages 32 rows of
// K at a time into LDS with direct buffer->LDS copies, three stages deep:
//   - the weights as the matrix-core stream's packed tiles (one 1 KB half
//     tile per 16-column strip: already the B operand order);
//   - X in A-operand order (lane l of a half block: token l%16, the 8 rows
//     16(l/16) + 8h .. +7 of the tile), gathered from row-major X.
// Both are read back with one 16-byte LDS read per lane and operand, in
// lane order. Rows past K and tokens past T read zero (range-checked
// loads). The products are formed transposed (P^T blocks), so that each lane
// ends with 4 consecutive columns of one token. The epilogue of tile (point
// j, m, n) waits until tile (j-1, m, n) has updated its hidden state (a
// counter per tile, bounded wait), then writes the partial to the rank's
// slot, reads the other ranks' partials and the residual (16 bytes per lane
// and access, a batch of blocks in flight at once), and forms the ring-order
// sum: chunk c of the flattened [T x H] payload is summed over ranks c, c+1,
// ... (mod N), one binary32 addition at a time, then the residual is added.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tp_device.h"
#include "tp_internal.h"

namespace {

using namespace tpdev;

typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kPfWavesM = 2, kPfWavesN = 2;
constexpr int kPfMB = 4;   // 16-token blocks per wave
constexpr int kPfNB = 8;   // 16-column strips per wave
constexpr int kPfTileM = kPfWavesM * kPfMB * 16;  // 128 tokens
constexpr int kPfTileN = kPfWavesN * kPfNB * 16;  // 256 columns
constexpr int kPfThreads = kPfWavesM * kPfWavesN * 64;
constexpr int kPfABytes = kPfTileM / 16 * 1024;   // one stage of A: 8 KB
constexpr int kPfBBytes = kPfTileN / 16 * 1024;   // one stage of B: 16 KB
static_assert(kPfMB == 4 && kPfNB == 8, "the stage's LDS reads are written out for 4 x 8 blocks");
constexpr int kPfStages = 3;  // LDS stages (separate objects: see the K loop)
constexpr int kPfLoadsPerStage = kPfTileM / 16 / 4 + kPfTileN / 16 / 4;  // copies per wave and stage (6)

// The LDS address (a 32-bit offset) of a pointer into a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)(p);
}

struct PrefillArgs {
    const uint16_t* x[2];   // X per point kind: [L][T][K] bf16 row-major
    const uint16_t* w[2];   // packed tiles per point kind: [L][H/16][nkb][2][64][8]
    float* slots;           // [L][2][N][T][H]
    float* hidden;          // [T][H]
    uint32_t* done;         // per (m, n) tile: points whose epilogue is complete (stride 16)
    uint32_t* exit_ctr;     // workgroups that have left
    uint32_t* err;          // error word (bit 0: a wait timed out)
    int32_t T, H, layers, n_ranks, rank;
    int32_t K[2], nkb[2];
    int32_t mt, nt;         // tiles along tokens and columns
    int32_t parts_m, parts_n;  // XCD blocks along tokens and columns (parts_m * parts_n = 8), or 0
    int64_t chunk;          // T*H/N
    uint32_t spin_limit;
};

// NR: the number of ranks (a template argument, so that the epilogue holds
// exactly the other ranks' values).
template <int NR>
__global__ __launch_bounds__(kPfThreads, 2) void prefill_step(PrefillArgs a) {
    // One LDS object per stage, three stages (72 KB: two workgroups per CU,
    // so that one's products overlap the other's epilogue; measured 15 %
    // faster than one workgroup with five stages). Separate objects let the
    // compiler see that a copy into stage s+2 does not write what the MFMAs
    // read from stage s.
    __shared__ __align__(16) uint8_t lds0[kPfABytes + kPfBBytes];
    __shared__ __align__(16) uint8_t lds1[kPfABytes + kPfBBytes];
    __shared__ __align__(16) uint8_t lds2[kPfABytes + kPfBBytes];
    __shared__ int s_ok, s_last;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / kPfWavesN, wn = wave % kPfWavesN;
    const int tiles_per_point = a.mt * a.nt;
    const int64_t total = (int64_t)2 * a.layers * tiles_per_point;
    const int64_t len = (int64_t)a.T * a.H;
    int ok = 1;

    // The walk. Workgroup w runs on XCD w % 8, and the 8 XCDs have an L2
    // each. With parts_m > 0 every point's tiles are cut into the same 8
    // blocks (parts_m along tokens x parts_n along columns) and XCD x's
    // workgroups walk block x of every point in point order: an XCD then
    // fetches only its block's rows of X and columns of W into its L2,
    // which all its tiles share (the host picks the cut that fetches the
    // fewest bytes). Tile (j, m, n) always falls to the same XCD, so the
    // chain of waits stays inside it. Without the cut (a grid that is not a
    // multiple of 8, or fewer tiles than blocks), all workgroups walk all
    // tiles.
    const int G = (int)gridDim.x, bx = (int)blockIdx.x;
    int64_t q0 = bx, qstep = G, qend = total;
    int mlo = 0, nlo = 0, nbx = a.nt, px = tiles_per_point;
    if (a.parts_m > 0) {
        const int x = bx % kXCDs, xm = x / a.parts_n, xn = x - xm * a.parts_n;
        mlo = xm * a.mt / a.parts_m;
        nlo = xn * a.nt / a.parts_n;
        nbx = (xn + 1) * a.nt / a.parts_n - nlo;
        px = ((xm + 1) * a.mt / a.parts_m - mlo) * nbx;
        q0 = bx / kXCDs;
        qstep = G / kXCDs;
        qend = (int64_t)2 * a.layers * px;
    }
    for (int64_t q = q0; q < qend; q += qstep) {
        const int j = (int)(q / px);
        const int lt = (int)(q - (int64_t)j * px);
        const int mbx = px / nbx;  // column-major inside the block
        const int mi = mlo + lt % mbx, ni = nlo + lt / mbx;
        const int tile = mi * a.nt + ni;
        const int pt = j & 1, l = j >> 1;
        const int K = a.K[pt], nkb = a.nkb[pt];
        const int m0 = mi * kPfTileM, n0 = ni * kPfTileN;
        // operand sources: X of the point (range T*K*2 bytes) and the
        // packed tiles of the tile's 16 strips (range: the strips inside H)
        const uint16_t* xp = a.x[pt] + (int64_t)l * a.T * K;
        const __amdgpu_buffer_rsrc_t xr =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(xp), (short)0, a.T * K * 2, kBufferRsrcWord3);
        const int s0 = n0 / 16;
        const int strips = a.H / 16 - s0 < kPfTileN / 16 ? a.H / 16 - s0 : kPfTileN / 16;
        const uint16_t* wp = a.w[pt] + ((int64_t)l * (a.H / 16) + s0) * nkb * 1024;
        const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(wp), (short)0, strips * nkb * 2048, kBufferRsrcWord3);
        // one stage: 32 rows of K (half h of 64-row block kb), A and B; every
        // wave issues exactly kPfLoadsPerStage copies
        auto stage = [&](int st, uint8_t* ab) {
            const int kb = st >> 1, h = st & 1;
            uint8_t* bb = ab + kPfABytes;
            // A: 8 half blocks of 16 tokens, two per wave
#pragma unroll
            for (int u0 = 0; u0 < kPfTileM / 16; u0 += kPfThreads / 64) {
                const int u = u0 + wave;
                const int tok = m0 + 16 * u + (lane & 15);
                const int k = 64 * kb + 16 * (lane >> 4) + 8 * h;
                const uint32_t off = tok < a.T && k < K ? (uint32_t)(((int64_t)tok * K + k) * 2) : 0x7ffffff0u;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void_t*)(ab + u * 1024), 16, off, 0, 0, 0);
            }
            // B: 16 half tiles (one per strip), four per wave
#pragma unroll
            for (int u0 = 0; u0 < kPfTileN / 16; u0 += kPfThreads / 64) {
                const int u = u0 + wave;
                const uint32_t off = (uint32_t)((u * nkb + kb) * 2048 + h * 1024 + lane * 16);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_void_t*)(bb + u * 1024), 16, off, 0, 0, 0);
            }
        };
        floatx4_t acc[kPfMB][kPfNB];
#pragma unroll
        for (int mb = 0; mb < kPfMB; ++mb)
#pragma unroll
            for (int nb = 0; nb < kPfNB; ++nb) acc[mb][nb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
        const int nst = 2 * nkb;
        uint8_t* const bufs[kPfStages] = {lds0, lds1, lds2};
        // prologue: stages 0 .. kPfStages-2 in flight
#pragma unroll
        for (int i = 0; i < kPfStages - 1; ++i)
            if (i < nst) stage(i, bufs[i]);
        // stage st: wait for its copies (later stages may stay in flight),
        // meet (every wave is done with stage st-1, whose buffer is refilled
        // with stage st + kPfStages - 1), then multiply
        auto step = [&](int st, uint8_t* cur, uint8_t* refill) {
            const int later = nst - 1 - st < kPfStages - 2 ? nst - 1 - st : kPfStages - 2;
            if (later >= kPfStages - 2)
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kPfLoadsPerStage * (kPfStages - 2)) : "memory");
            else
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            // a bare barrier: __syncthreads' release fence would wait for every
            // copy in flight. The wait above covers this wave's copies of
            // stage st; its reads of stage st-1 have been consumed by the
            // MFMAs before it arrives.
            compiler_barrier();
            __builtin_amdgcn_s_barrier();
            compiler_barrier();
            if (st + kPfStages - 1 < nst) stage(st + kPfStages - 1, refill);
            // the stage's 12 operands, read in one block that waits for its
            // own reads: the compiler, which cannot tell these reads from the
            // copies still in flight to other stages, would otherwise wait
            // for all of those first
            bf16x8_t A[kPfMB], B[kPfNB];
            const uint32_t aa = lds_addr(cur + (wm * kPfMB) * 1024 + lane * 16);
            const uint32_t ba = lds_addr(cur + kPfABytes + (wn * kPfNB) * 1024 + lane * 16);
            asm volatile(
                "ds_read_b128 %0, %12\n"
                "ds_read_b128 %1, %12 offset:1024\n"
                "ds_read_b128 %2, %12 offset:2048\n"
                "ds_read_b128 %3, %12 offset:3072\n"
                "ds_read_b128 %4, %13\n"
                "ds_read_b128 %5, %13 offset:1024\n"
                "ds_read_b128 %6, %13 offset:2048\n"
                "ds_read_b128 %7, %13 offset:3072\n"
                "ds_read_b128 %8, %13 offset:4096\n"
                "ds_read_b128 %9, %13 offset:5120\n"
                "ds_read_b128 %10, %13 offset:6144\n"
                "ds_read_b128 %11, %13 offset:7168\n"
                "s_waitcnt lgkmcnt(0)"
                : "=v"(A[0]), "=v"(A[1]), "=v"(A[2]), "=v"(A[3]), "=v"(B[0]), "=v"(B[1]), "=v"(B[2]),
                  "=v"(B[3]), "=v"(B[4]), "=v"(B[5]), "=v"(B[6]), "=v"(B[7])
                : "v"(aa), "v"(ba));
            // the transposed block P^T = W^T X^T: lane l then holds 4
            // consecutive columns 4(l/16) .. +3 of token l%16, so that the
            // epilogue moves 16 bytes per lane and access
#pragma unroll
            for (int mb = 0; mb < kPfMB; ++mb)
#pragma unroll
                for (int nb = 0; nb < kPfNB; ++nb)
                    acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(B[nb], A[mb], acc[mb][nb], 0, 0, 0);
        };
        for (int st = 0; st < nst; st += kPfStages) {
            step(st, lds0, lds2);
            if (st + 1 < nst) step(st + 1, lds1, lds0);
            if (st + 2 < nst) step(st + 2, lds2, lds1);
        }
        // epilogue: wait for point j-1 of this tile, then slot + ring + residual
        uint32_t* done = a.done + (int64_t)tile * kCounterStride;
        if (tid == 0) s_ok = ok && wait_at_least(done, (uint32_t)j, a.err, a.spin_limit);
        __syncthreads();
        ok = s_ok;
        float* slot = a.slots + (int64_t)j * NR * len;
        float* own = slot + (int64_t)a.rank * len;
        const __amdgpu_buffer_rsrc_t hr = dev_rsrc(a.hidden, (uint32_t)(len * 4 < 0x7fffffff ? len * 4 : 0x7fffffff));
        if (ok) {
            // batches of EB blocks of 16 tokens x 16 columns: every load of a
            // batch (the other ranks' partials and the residual, 16 bytes per
            // lane) is issued before the first addition
            constexpr int EB = NR <= 4 ? 4 : 2;
#pragma unroll
            for (int g = 0; g < kPfMB * kPfNB / EB; ++g) {
                floatx4_t oth[EB][NR > 1 ? NR - 1 : 1];
                floatx4_t res[EB];
                int64_t eo[EB];
                bool in[EB];
#pragma unroll
                for (int i = 0; i < EB; ++i) {
                    const int blk = g * EB + i, mb = blk / kPfNB, nb = blk % kPfNB;
                    const int t = m0 + (wm * kPfMB + mb) * 16 + (lane & 15);
                    const int n = n0 + (wn * kPfNB + nb) * 16 + 4 * (lane >> 4);
                    in[i] = t < a.T && n < a.H;  // a strip lies wholly inside H or past it
                    eo[i] = in[i] ? (int64_t)t * a.H + n : 0;
#pragma unroll
                    for (int u = 0; u < NR - 1; ++u) {  // the other ranks in rank order
                        const int rr = u < a.rank ? u : u + 1;
                        oth[i][u] = *reinterpret_cast<const floatx4_t*>(slot + (int64_t)rr * len + eo[i]);
                    }
                    res[i] = ld_dev4(hr, (uint32_t)(eo[i] * 4));
                }
#pragma unroll
                for (int i = 0; i < EB; ++i) {
#pragma clang fp contract(off)
                    if (!in[i]) continue;
                    const int blk = g * EB + i, mb = blk / kPfNB, nb = blk % kPfNB;
                    const floatx4_t v = acc[mb][nb];
                    *reinterpret_cast<floatx4_t*>(own + eo[i]) = v;
                    floatx4_t out;
                    // the chunk of the first column (32-bit: T*H < 2^29), and
                    // where the next chunk starts (4 columns span at most two
                    // chunks of 4 or more elements)
                    const uint32_t e0 = (uint32_t)eo[i];
                    const uint32_t c0 = e0 / (uint32_t)a.chunk;
                    const uint32_t next = (c0 + 1) * (uint32_t)a.chunk;
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        // ring order: ranks c, c+1, ... (mod N) of this element's
                        // chunk; our value at position (rank - c) mod N
                        const int c = a.chunk >= 4 ? (int)(e0 + k < next ? c0 : c0 + 1)
                                                   : (int)((e0 + k) / (uint32_t)a.chunk);
                        float sum = 0.f;
#pragma unroll
                        for (int u = 0; u < NR; ++u) {
                            int rr = c + u;
                            rr = rr >= NR ? rr - NR : rr;
                            const int q = rr < a.rank ? rr : rr - 1;  // among the other ranks
                            float val = v[k];                          // (selects, not an indexed array)
#pragma unroll
                            for (int w = 0; w < NR - 1; ++w) val = (rr != a.rank && w == q) ? oth[i][w][k] : val;
                            sum = u == 0 ? val : sum + val;
                        }
                        out[k] = sum + res[i][k];
                    }
                    st_dev4(hr, (uint32_t)(eo[i] * 4), out);
                }
            }
        }
        wait_mem();        // this wave's hidden-state stores are complete
        __syncthreads();
        if (tid == 0 && ok) add_dev_u32(done, 1u);
    }
    // the last workgroup to leave clears the tile counters for the next launch
    __syncthreads();
    if (tid == 0) s_last = add_dev_u32(a.exit_ctr, 1u) == gridDim.x - 1;
    __syncthreads();
    if (s_last) {
        for (int t = tid; t < tiles_per_point; t += blockDim.x) st_dev_u32(a.done + (int64_t)t * kCounterStride, 0u);
        if (tid == 0) st_dev_u32(a.exit_ctr, 0u);
    }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

typedef void (*prefill_fn)(PrefillArgs);
prefill_fn prefill_kernel(int n) {
    switch (n) {
        case 1: return prefill_step<1>;
        case 2: return prefill_step<2>;
        case 3: return prefill_step<3>;
        case 4: return prefill_step<4>;
        case 5: return prefill_step<5>;
        case 6: return prefill_step<6>;
        case 7: return prefill_step<7>;
        case 8: return prefill_step<8>;
    }
    return nullptr;
}

int prefill_grid(prefill_fn k) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(k), kPfThreads,
                                                     0) != hipSuccess)
        return 0;
    return per_cu * cus;
}

}  // namespace

extern "C" {

tp_status tp_prefill_pack_weights(tp_plan_t p, int32_t point, int32_t n_layers, const void* w,
                                  void* w_packed, void* stream) {
    if (!p || !w || !w_packed || n_layers < 0) return TP_ERR_INVALID_ARG;
    if (point != TP_POINT_ATTN_OUT && point != TP_POINT_FFN_DOWN) return TP_ERR_INVALID_ARG;
    if (!aligned16(w) || !aligned16(w_packed)) return TP_ERR_ALIGNMENT;
    if (w == w_packed) return TP_ERR_INVALID_ARG;
    if (p->hidden % 16) return TP_ERR_UNSUPPORTED;
    const int64_t K = (point == TP_POINT_ATTN_OUT ? p->k_attn : p->inter) / p->n_ranks;
    return tp_pack_tile_stack(n_layers, K, p->hidden, w, w_packed, stream);
}

tp_status tp_prefill_layers(tp_plan_t p, int32_t n_layers, int32_t rank, int32_t tokens,
                            const void* x_attn, const void* w_o_packed, const void* x_ffn,
                            const void* w_down_packed, float* slots, float* hidden, void* ws,
                            void* stream) {
    if (!p || n_layers < 0 || tokens < 1 || rank < 0 || rank >= p->n_ranks) return TP_ERR_INVALID_ARG;
    if (!x_attn || !w_o_packed || !x_ffn || !w_down_packed || !slots || !hidden || !ws)
        return TP_ERR_INVALID_ARG;
    if (!aligned16(x_attn) || !aligned16(w_o_packed) || !aligned16(x_ffn) || !aligned16(w_down_packed) ||
        !aligned16(slots) || !aligned16(hidden) || !aligned16(ws))
        return TP_ERR_ALIGNMENT;
    const int64_t T = tokens, H = p->hidden;
    const int64_t K0 = p->k_attn / p->n_ranks, K1 = p->inter / p->n_ranks;
    if (((int64_t)T * H) % p->n_ranks) return TP_ERR_INVALID_ARG;  // the ring's N equal chunks
    if (H % 16 || K0 % 8 || K1 % 8 || p->n_ranks > 8) return TP_ERR_UNSUPPORTED;
    // 32-bit buffer ranges: X of a point and a tile's 16 strips of packed weights
    const int64_t nkb0 = (K0 + 63) / 64, nkb1 = (K1 + 63) / 64;
    if (T * (K0 > K1 ? K0 : K1) * 2 > 0x7fff0000LL ||
        (int64_t)(kPfTileN / 16) * (nkb0 > nkb1 ? nkb0 : nkb1) * 2048 >= ((int64_t)1 << 31))
        return TP_ERR_UNSUPPORTED;
    const int64_t mt = (T + kPfTileM - 1) / kPfTileM, nt = (H + kPfTileN - 1) / kPfTileN;
    if (mt * nt > kMaxCounters) return TP_ERR_UNSUPPORTED;  // tile counters in the workspace
    if (T * H * 4 >= ((int64_t)1 << 31)) return TP_ERR_UNSUPPORTED;  // hidden state through a 32-bit buffer range
    if (n_layers == 0) return TP_OK;
    if ((int64_t)2 * n_layers * mt * nt >= ((int64_t)1 << 62)) return TP_ERR_UNSUPPORTED;
    PrefillArgs a;
    a.x[0] = static_cast<const uint16_t*>(x_attn);
    a.x[1] = static_cast<const uint16_t*>(x_ffn);
    a.w[0] = static_cast<const uint16_t*>(w_o_packed);
    a.w[1] = static_cast<const uint16_t*>(w_down_packed);
    a.slots = slots;
    a.hidden = hidden;
    char* base = static_cast<char*>(ws);
    a.done = reinterpret_cast<uint32_t*>(base);  // the column-tile counters' region
    a.exit_ctr = reinterpret_cast<uint32_t*>(base + kSyncOffset) + kSyncExit;
    a.err = reinterpret_cast<uint32_t*>(base + kSyncOffset) + kSyncErr;
    a.T = (int32_t)T;
    a.H = (int32_t)H;
    a.layers = n_layers;
    a.n_ranks = p->n_ranks;
    a.rank = rank;
    a.K[0] = (int32_t)K0;
    a.K[1] = (int32_t)K1;
    a.nkb[0] = (int32_t)nkb0;
    a.nkb[1] = (int32_t)nkb1;
    a.mt = (int32_t)mt;
    a.nt = (int32_t)nt;
    a.chunk = T * H / p->n_ranks;
    a.parts_m = 0;
    a.parts_n = 0;
    a.spin_limit = 1u << 22;
    prefill_fn k = prefill_kernel(p->n_ranks);
    if (!k) return TP_ERR_UNSUPPORTED;
    const int cap = prefill_grid(k);
    if (cap < 1) return TP_ERR_DEVICE;
    const int64_t total = 2 * (int64_t)n_layers * mt * nt;
    const int grid = total < cap ? (int)total : cap;
    if (grid % kXCDs == 0) {
        // the XCD blocks: the cut whose operand fetches (every block reads
        // its rows of X and its columns of W once per point) are fewest
        const double xb = (double)T * (K0 + K1) * 2, wb = (double)(K0 + K1) * H * 2;
        double best = 0;
        for (int pm = 1; pm <= kXCDs; pm *= 2) {
            const int pn = kXCDs / pm;
            if (pm > mt || pn > nt) continue;
            const double cost = pn * xb + pm * wb;
            if (a.parts_m == 0 || cost < best) {
                best = cost;
                a.parts_m = pm;
                a.parts_n = pn;
            }
        }
    }
    void* args[] = {&a};
    if (hipLaunchCooperativeKernel(reinterpret_cast<const void*>(k), dim3(grid), dim3(kPfThreads), args, 0,
                                   (hipStream_t)stream) != hipSuccess)
        return TP_ERR_DEVICE;
    return tp_launch_status(stream);
}

}  // extern "C"
