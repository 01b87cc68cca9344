// HIP kernels for gfx950 (MI355X) and the entry points that launch them.
//
// Path ("Interconnects e clusters", llmdeepdive.com lesson 9.9, section
// 01 · Conceito): at each of a layer's two reconciliation points the rank
// computes its row-parallel partial p_r = x[:, K_r] . W[K_r, :] and the
// partials of all ranks are summed, ring-style, before the residual stream
// continues. Decode projections are bound by streaming the weights from HBM
// ("Hosting Qwen on Blackwell", section Decoders), so the kernels are built
// around moving each weight byte once, in 16-byte coalesced nontemporal
// loads, with enough loads in flight to cover HBM latency on 256 CUs.
//
// Kernels:
//   valu_gemv       batch 1..15, one projection. A workgroup owns a tile of
//                   COLS columns x `rows` rows (split-K). Each lane loads
//                   all of its rows' 16-byte weight vectors (8 columns each)
//                   into registers at once, then multiplies them by x
//                   staged as fp32 in LDS, accumulating in fp32.
//   decode_step     batch 1..15, the whole decode step in one cooperative
//                   (persistent) launch: workgroups walk the step's tiles in
//                   point order. A workgroup issues the weight loads of its
//                   next tile before it waits for the previous point's
//                   hidden state to complete, so the weight stream of point
//                   j+1 overlaps the reduction of point j; the launch gap
//                   between points disappears.
//   mfma_gemm       batch 16..64: the tile streamed as 8 rows x 16 bytes per
//                   lane, transposed in registers with v_perm into k-major
//                   bf16x8 operands, multiplied on the bf16 matrix cores
//                   (v_mfma_f32_16x16x32_bf16).
//   ring_reduce     the stand-alone ring-order sum + residual.
//
// Split-K fixup: every workgroup publishes its fp32 partial tile; the last
// workgroup of a column tile (arrival counter) sums the splits in split
// order, so the result does not depend on scheduling. With the ring
// epilogue (decode) it then sums the N ranks' partials in ring order and
// adds the residual.
//
// Cross-workgroup visibility inside a launch: see tp_device.h.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>

#include "tp_device.h"
#include "tp_internal.h"

namespace {

using namespace tpdev;

// ------------------------------------------------------------ epilogue --

struct Epilogue {
    float* p;                 // final partial [B][H] (the rank's slot when fused)
    float* ws_part;           // split partials [S][B][H]
    uint32_t* counters;       // one per column tile, stride kCounterStride
    int32_t splits;
    // ring epilogue (decode); ring_slots == nullptr disables it
    const float* ring_slots;  // this point's [N][B][H]
    float* hidden;            // [B][H] residual stream, updated in place
    int32_t n_ranks, rank;
    int64_t chunk;            // B*H / N
    // spread fix-up: every split's workgroup is resident (cooperative
    // launch) and sums a share of its column tile (0: the last arrival sums
    // all of it)
    int32_t spread;
    uint32_t* err;            // error word (bounded waits)
    uint32_t spin_limit;
};

// Publish this split's partial tile [batch][COLS] (LDS) and find out whether
// this workgroup arrived last for its column tile. Returns true for the
// last arrival (and always when there is a single split). Four columns per
// device-coherent 16-byte store (H and COLS are multiples of 4).
template <int COLS, int NT>
__device__ bool publish_split(const Epilogue& e, const float* tile, int batch, int64_t H, int ct,
                              int sp, int tid, int* s_flag) {
    if (e.splits == 1) return true;
    const int64_t n0 = (int64_t)ct * COLS;
    const __amdgpu_buffer_rsrc_t rs =
        dev_rsrc(e.ws_part, (uint32_t)((int64_t)e.splits * batch * H * 4));
    for (int idx = tid; idx < batch * COLS / 4; idx += NT) {
        const int bb = idx / (COLS / 4), c = (idx - bb * (COLS / 4)) * 4;
        const int64_t n = n0 + c;
        if (n < H)
            st_dev4(rs, (uint32_t)((((int64_t)sp * batch + bb) * H + n) * 4),
                    *reinterpret_cast<const floatx4_t*>(tile + bb * COLS + c));
    }
    wait_mem();
    __syncthreads();
    if (tid == 0) {
        uint32_t prev = add_dev_u32(&e.counters[ct * kCounterStride], 1u);
        *s_flag = prev == (uint32_t)(e.splits - 1);
    }
    __syncthreads();
    compiler_barrier();
    return *s_flag != 0;
}

// Ring-order sum (no residual) of four consecutive elements i..i+3 that
// share ring chunk c0: the other ranks' values as 16-byte loads, a group of
// up to 8 ranks in flight at once, added in ring order element by element
// (the same bits as ring_element for each). `own` is this rank's vector.
__device__ __forceinline__ floatx4_t ring_vector(const float* slots, int64_t len, int64_t i, int c0,
                                                 int n_ranks, int rank, floatx4_t own) {
#pragma clang fp contract(off)
    floatx4_t sum;
    for (int j0 = 0; j0 < n_ranks; j0 += 8) {
        floatx4_t t[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int jj = j0 + k < n_ranks ? j0 + k : n_ranks - 1;
            int r = c0 + jj;
            if (r >= n_ranks) r -= n_ranks;
            t[k] = r == rank ? own : *reinterpret_cast<const floatx4_t*>(slots + (int64_t)r * len + i);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (j0 + k < n_ranks) sum = (j0 + k == 0) ? t[k] : sum + t[k];
    }
    return sum;
}

// One 16-byte vector (4 columns) of the final partial: the splits summed in
// split order, written to the partial and, with the ring epilogue, the
// ring-order sum + residual into the hidden state. The residual load goes
// out with the split loads (one round trip).
__device__ __forceinline__ void fixup_vector(const Epilogue& e, const float* tile_vec, int64_t i,
                                             int64_t len, __amdgpu_buffer_rsrc_t rp,
                                             __amdgpu_buffer_rsrc_t rh) {
#pragma clang fp contract(off)
    const floatx4_t res = e.ring_slots ? ld_dev4(rh, (uint32_t)(i * 4)) : floatx4_t{0.f, 0.f, 0.f, 0.f};
    floatx4_t v;
    if (e.splits > 1) {
        floatx4_t l[8];
        for (int s0 = 0; s0 < e.splits; s0 += 8) {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int sp = s0 + u < e.splits ? s0 + u : e.splits - 1;
                l[u] = ld_dev4(rp, (uint32_t)(((int64_t)sp * len + i) * 4));
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (s0 + u < e.splits) v = (s0 + u == 0) ? l[u] : v + l[u];
        }
    } else {
        v = *reinterpret_cast<const floatx4_t*>(tile_vec);
    }
    *reinterpret_cast<floatx4_t*>(e.p + i) = v;
    if (e.ring_slots) {
        floatx4_t o;
        const int c0 = (int)(i / e.chunk);
        if (c0 == (int)((i + 3) / e.chunk)) {
            o = ring_vector(e.ring_slots, len, i, c0, e.n_ranks, e.rank, v) + res;
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                o[k] = ring_element(e.ring_slots, len, i + k, e.chunk, e.n_ranks, e.rank, v[k], res[k]);
        }
        st_dev4(rh, (uint32_t)(i * 4), o);
    }
}

// Last arrival: sum the splits in split order, write the partial and, with
// the ring epilogue, the ring-order sum + residual into the hidden state.
// Four columns at a time; every element is still summed in split order.
template <int COLS, int NT>
__device__ void fixup_tile(const Epilogue& e, const float* tile, int batch, int64_t H, int ct,
                           int tid) {
    const int64_t n0 = (int64_t)ct * COLS;
    const int64_t len = (int64_t)batch * H;
    const __amdgpu_buffer_rsrc_t rp = dev_rsrc(e.ws_part, (uint32_t)((int64_t)e.splits * len * 4));
    const __amdgpu_buffer_rsrc_t rh = dev_rsrc(e.hidden, (uint32_t)(len * 4));
    for (int idx = tid; idx < batch * COLS / 4; idx += NT) {
        const int bb = idx / (COLS / 4), c = (idx - bb * (COLS / 4)) * 4;
        const int64_t n = n0 + c;
        if (n >= H) continue;
        fixup_vector(e, tile + bb * COLS + c, (int64_t)bb * H + n, len, rp, rh);
    }
    if (e.splits > 1 && tid == 0) st_dev_u32(&e.counters[ct * kCounterStride], 0u);
    wait_mem();
}

// Last arrival of a persistent-step tile (point j, column tile ct): the
// splits summed in split order, the rank's slot written and the ring-order
// sum over the N ranks formed in registers (ring_element with a residual of
// -0.0, which leaves every value as it is), all before `wait_prev` waits for
// (j-1, ct); only the residual's read, one addition and the store of the
// hidden state follow it. Same bits as fixup_tile. Without ring slots
// (partials only) it writes the partial and returns. Returns false if the
// wait failed.
template <int BMAX, int COLS, int NT, typename Wait>
__device__ bool step_fixup(const Epilogue& e, const float* tile, int batch, int64_t H, int ct,
                           int tid, Wait wait_prev) {
#pragma clang fp contract(off)
    constexpr int VPT = (BMAX * COLS / 4 + NT - 1) / NT;
    const int NV = batch * COLS / 4;  // 16-byte vectors in the tile
    const int64_t n0 = (int64_t)ct * COLS;
    const int64_t len = (int64_t)batch * H;
    const __amdgpu_buffer_rsrc_t rp = dev_rsrc(e.ws_part, (uint32_t)((int64_t)e.splits * len * 4));
    const __amdgpu_buffer_rsrc_t rh = dev_rsrc(e.hidden, (uint32_t)(len * 4));
    floatx4_t ring[VPT];
    int64_t at[VPT];
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
        const int idx = tid + u * NT;
        at[u] = -1;
        if (idx >= NV) continue;
        const int bb = idx / (COLS / 4), c = (idx - bb * (COLS / 4)) * 4;
        if (n0 + c >= H) continue;
        const int64_t i = (int64_t)bb * H + n0 + c;
        at[u] = i;
        floatx4_t v;
        if (e.splits > 1) {
            floatx4_t l[8];
            for (int s0 = 0; s0 < e.splits; s0 += 8) {
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int sp = s0 + k < e.splits ? s0 + k : e.splits - 1;
                    l[k] = ld_dev4(rp, (uint32_t)(((int64_t)sp * len + i) * 4));
                }
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    if (s0 + k < e.splits) v = (s0 + k == 0) ? l[k] : v + l[k];
            }
        } else {
            v = *reinterpret_cast<const floatx4_t*>(tile + bb * COLS + c);
        }
        *reinterpret_cast<floatx4_t*>(e.p + i) = v;
        if (!e.ring_slots) continue;
        const int c0 = (int)(i / e.chunk);
        if (c0 == (int)((i + 3) / e.chunk)) {
            ring[u] = ring_vector(e.ring_slots, len, i, c0, e.n_ranks, e.rank, v);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                ring[u][k] = ring_element(e.ring_slots, len, i + k, e.chunk, e.n_ranks, e.rank, v[k], -0.0f);
        }
    }
    if (e.splits > 1 && tid == 0) st_dev_u32(&e.counters[ct * kCounterStride], 0u);
    if (!e.ring_slots) {  // partials only: no residual chain
        wait_mem();
        return true;
    }
    if (!wait_prev()) return false;
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
        if (at[u] < 0) continue;
        const floatx4_t res = ld_dev4(rh, (uint32_t)(at[u] * 4));
        st_dev4(rh, (uint32_t)(at[u] * 4), ring[u] + res);
    }
    wait_mem();
    return true;
}

// Spread fix-up (all of a column tile's splits resident): once every split
// has published, split sp's workgroup takes the sp-th of S equal shares of
// the tile's vectors (each still summed in split order, so the result is
// the last-arrival fix-up's, bit for bit); the last one to finish clears
// the tile's counters for the next launch. The arrival wait is bounded.
template <int COLS, int NT>
__device__ void spread_fixup(const Epilogue& e, int batch, int64_t H, int ct, int sp, int tid) {
    uint32_t* arrive = &e.counters[ct * kCounterStride];
    uint32_t* leave = arrive + 1;
    if (tid == 0) wait_at_least(arrive, (uint32_t)e.splits, e.err, e.spin_limit);
    __syncthreads();
    compiler_barrier();
    const int64_t n0 = (int64_t)ct * COLS;
    const int64_t len = (int64_t)batch * H;
    const __amdgpu_buffer_rsrc_t rp = dev_rsrc(e.ws_part, (uint32_t)((int64_t)e.splits * len * 4));
    const __amdgpu_buffer_rsrc_t rh = dev_rsrc(e.hidden, (uint32_t)(len * 4));
    const int total = batch * COLS / 4;
    const int share = (total + e.splits - 1) / e.splits;
    const int hi = (sp + 1) * share < total ? (sp + 1) * share : total;
    for (int idx = sp * share + tid; idx < hi; idx += NT) {
        const int bb = idx / (COLS / 4), c = (idx - bb * (COLS / 4)) * 4;
        const int64_t n = n0 + c;
        if (n >= H) continue;
        fixup_vector(e, nullptr, (int64_t)bb * H + n, len, rp, rh);
    }
    wait_mem();
    __syncthreads();
    if (tid == 0 && add_dev_u32(leave, 1u) == (uint32_t)(e.splits - 1)) {
        st_dev_u32(arrive, 0u);
        st_dev_u32(leave, 0u);
    }
}

// ------------------------------------------------------------ VALU tile --

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

// Select the low (even column) or high (odd column) bf16 of two row words
// into one k-major pair: result = {row0 half, row1 half}.
__device__ __forceinline__ uint32_t pair_rows(uint32_t row0, uint32_t row1, bool high) {
    return __builtin_amdgcn_perm(row1, row0, high ? 0x07060302u : 0x05040100u);
}

// Two of a lane's rows (ra, rb; 8 columns each) against x at those rows:
// per column and batch row, one v_dot2c_f32_bf16 adds both exact bf16
// products to the fp32 accumulator. xp[bb] = {x[bb][ra], x[bb][rb]}.
template <int B>
__device__ __forceinline__ void dot2_rows(float (&acc)[B][8], const u32x4_t& ra, const u32x4_t& rb,
                                          const uint32_t* xp) {
    const uint32_t pr[8] = {pair_rows(ra.x, rb.x, false), pair_rows(ra.x, rb.x, true),
                            pair_rows(ra.y, rb.y, false), pair_rows(ra.y, rb.y, true),
                            pair_rows(ra.z, rb.z, false), pair_rows(ra.z, rb.z, true),
                            pair_rows(ra.w, rb.w, false), pair_rows(ra.w, rb.w, true)};
#pragma unroll
    for (int bb = 0; bb < B; ++bb) {
        const bf16x2_t xv = __builtin_bit_cast(bf16x2_t, xp[bb]);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            acc[bb][j] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pr[j]), xv,
                                                         acc[bb][j], false);
    }
}

// Stage x[:, k0 .. k0+nr) for dot2_rows: a lane's rows are r0 + i*RSTEP,
// taken in pairs (i even, i+1). Rows a with a / RSTEP even start a pair;
// pair p = (a / (2*RSTEP))*RSTEP + a % RSTEP is stored densely at
// xp[p*B + bb] = {x[bb][k0+a], x[bb][k0+a+RSTEP]} (pair_index gives p). A
// partner row past the tile reads as zero (its weights are zero too, and
// nothing stale in LDS is ever multiplied).
template <int B, int RSTEP, int NT>
__device__ __forceinline__ void stage_x_pairs(uint32_t* xp, const uint16_t* x, int64_t K, int64_t k0,
                                              int nr) {
    const int nblk = (nr + 2 * RSTEP - 1) / (2 * RSTEP);
    const int per_b = nblk * RSTEP;
    for (int i = threadIdx.x; i < per_b * B; i += NT) {
        const int bb = i / per_b, p = i - bb * per_b;
        const int ra = (p / RSTEP) * 2 * RSTEP + p % RSTEP;
        if (ra >= nr) continue;
        const uint16_t* xr = x + (int64_t)bb * K + k0;
        const uint32_t lo = xr[ra];
        const uint32_t hi = ra + RSTEP < nr ? xr[ra + RSTEP] : 0u;
        xp[p * B + bb] = lo | (hi << 16);
    }
}

// Pair index of the pair starting at row r0 + m*RSTEP (m even, r0 < RSTEP).
template <int RSTEP>
__device__ __forceinline__ int pair_index(int r0, int m) { return (m / 2) * RSTEP + r0; }

template <int B, int COLS>
struct ValuShared {
    static constexpr int XS = valu_rows_max(B, COLS) * B;
    uint32_t xs[XS];  // x row pairs, see stage_x_pairs
    float red[kValuWaves * COLS];
    __attribute__((aligned(16))) float tile[B * COLS];
    int flag;
    int wflag;  // outcome of the decode step's waits
};

// Issue the weight loads of one VALU tile: columns [ct*COLS, +COLS) x rows
// [k0, k0+nr) of W[K][H]. Every 16-byte vector (8 columns) of the lane's
// rows goes out at once; lanes past the tile get zeros.
template <int B, int COLS>
__device__ __forceinline__ void valu_issue(u32x4_t (&wv)[kValuLoadsPerLane], const uint16_t* w,
                                           int64_t H, int64_t k0, int nr, int ct) {
    constexpr int LPR = COLS / 8;   // lanes per row segment
    constexpr int RPW = 64 / LPR;   // row groups per wave
    constexpr int RSTEP = kValuWaves * RPW;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t n = (int64_t)ct * COLS + (lane % LPR) * 8;
    const bool col_ok = n < H;
    const int r0 = wave * RPW + lane / LPR;
    const uint16_t* wp = w + (k0 + r0) * H + n;
#pragma unroll
    for (int i = 0; i < kValuLoadsPerLane; ++i) {
        if (col_ok && r0 + i * RSTEP < nr) wv[i] = load_stream16(wp + (int64_t)i * RSTEP * H);
        else wv[i] = u32x4_t{0u, 0u, 0u, 0u};
    }
}

// Sum a tile's per-lane accumulators (lane rows r0 + i*RSTEP, taken in
// pairs in i order) into tile[B][COLS]: first the wave's row groups (lanes that share
// columns; an xor pair adds the same two values, so both lanes hold
// identical bits), then the waves in wave order, one batch row at a time.
template <int B, int COLS>
__device__ __forceinline__ void reduce_tile(float (&acc)[B][8], float* red, float* tile) {
    constexpr int NT = kValuWaves * 64;
    constexpr int LPR = COLS / 8;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int m = LPR; m < 64; m <<= 1)
#pragma unroll
        for (int bb = 0; bb < B; ++bb)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[bb][j] += __shfl_xor(acc[bb][j], m);
    for (int bb = 0; bb < B; ++bb) {
        if (lane < LPR) {
#pragma unroll
            for (int j = 0; j < 8; ++j) red[wave * COLS + lane * 8 + j] = acc[bb][j];
        }
        __syncthreads();
        for (int c = tid; c < COLS; c += NT) {
            float s = red[c];
#pragma unroll
            for (int wq = 1; wq < kValuWaves; ++wq) s += red[wq * COLS + c];
            tile[bb * COLS + c] = s;
        }
        __syncthreads();
    }
}

// Finish one VALU tile whose loads valu_issue put in `wv`, x [B][K]: stage
// x row pairs in LDS, multiply (rows in pairs, dot2_rows), and leave the
// workgroup's partial in sh.tile.
template <int B, int COLS>
__device__ void valu_finish(ValuShared<B, COLS>& sh, const u32x4_t (&wv)[kValuLoadsPerLane],
                            const uint16_t* x, int64_t K, int64_t k0, int nr) {
    constexpr int NT = kValuWaves * 64;
    constexpr int LPR = COLS / 8;
    constexpr int RPW = 64 / LPR;
    constexpr int RSTEP = kValuWaves * RPW;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r0 = wave * RPW + lane / LPR;

    stage_x_pairs<B, RSTEP, NT>(sh.xs, x, K, k0, nr);
    __syncthreads();

    float acc[B][8];
#pragma unroll
    for (int bb = 0; bb < B; ++bb)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[bb][j] = 0.f;
    static_assert(kValuLoadsPerLane % 2 == 0, "rows are taken in pairs");
#pragma unroll
    for (int i = 0; i < kValuLoadsPerLane; i += 2) {
        int r = r0 + i * RSTEP;
        if (r < nr) dot2_rows<B>(acc, wv[i], wv[i + 1], &sh.xs[pair_index<RSTEP>(r0, i) * B]);
    }
    reduce_tile<B, COLS>(acc, sh.red, sh.tile);
}

struct GemvArgs {
    const uint16_t* x;  // [B][K]
    const uint16_t* w;  // [K][H]
    int64_t K, H;
    int32_t rows;       // rows per split
    int32_t col_tiles;
    Epilogue epi;
};

template <int B, int COLS>
__global__ __launch_bounds__(kValuWaves * 64) void valu_gemv(GemvArgs a) {
    constexpr int NT = kValuWaves * 64;
    __shared__ ValuShared<B, COLS> sh;
    const int ct = blockIdx.x % a.col_tiles;
    const int sp = blockIdx.x / a.col_tiles;
    const int64_t k0 = (int64_t)sp * a.rows;
    const int nr = (int)(a.K - k0 < a.rows ? a.K - k0 : a.rows);
    u32x4_t wv[kValuLoadsPerLane];
    valu_issue<B, COLS>(wv, a.w, a.H, k0, nr, ct);
    valu_finish<B, COLS>(sh, wv, a.x, a.K, k0, nr);
    if (publish_split<COLS, NT>(a.epi, sh.tile, B, a.H, ct, sp, threadIdx.x, &sh.flag))
        fixup_tile<COLS, NT>(a.epi, sh.tile, B, a.H, ct, threadIdx.x);
}

// ------------------------------------------------------- decode step --

struct StepArgs {
    const uint16_t* x[2];   // x_attn [L][b][K0], x_ffn [L][b][K1]
    const uint16_t* w[2];   // w_o [L][K0][H], w_down [L][K1][H]
    float* slots;           // [L][2][N][b][H]
    float* hidden;          // [b][H]
    float* partials;        // partials only (no ring, no residual): [L][2][b][H]
    float* ws_part;         // kStepBufs split-partial buffers
    int64_t part_stride;    // floats between two buffers
    uint32_t* counters;     // column-tile arrival counters, kStepBufs sets
    uint32_t* fixed;        // per column tile: points whose fix-up is done
    uint32_t* sync;         // done / exit / error words
    int64_t H, K[2];
    int32_t rows[2], splits[2], tiles[2];
    int32_t col_tiles, layers, n_ranks, rank;
    int32_t batch;
    int32_t serial;         // 1: point j+1 reads its activation after all of point j
    int32_t xcd_walk;       // 1: each XCD's workgroups take contiguous tiles per round
    int32_t lstep;          // layers of x and W between two layers of the step (1, or 2
                            // when two consecutive layers are its two points)
    int64_t chunk;
    uint32_t spin_limit;
};

// Tile q of a step: (layer, point kind) in order, then split-major over the
// column tiles.
struct StepTile {
    int pt, ct, sp, j, nr, splits;
    int64_t K, k0;
    const uint16_t* x;  // the point's x [b][K]
    const uint16_t* w;  // the point's W [K][H]
};
__device__ __forceinline__ StepTile step_tile(const StepArgs& a, int64_t q) {
    StepTile t;
    const int per_layer = a.tiles[0] + a.tiles[1];
    const int l = (int)(q / per_layer);
    const int rem = (int)(q - (int64_t)l * per_layer);
    t.pt = rem >= a.tiles[0];
    const int r = t.pt ? rem - a.tiles[0] : rem;
    t.ct = r % a.col_tiles;
    t.sp = r / a.col_tiles;
    t.j = 2 * l + t.pt;  // point index in the step
    t.K = a.K[t.pt];
    t.k0 = (int64_t)t.sp * a.rows[t.pt];
    t.nr = (int)(t.K - t.k0 < a.rows[t.pt] ? t.K - t.k0 : a.rows[t.pt]);
    t.splits = a.splits[t.pt];
    t.x = a.x[t.pt] + (int64_t)l * a.lstep * a.batch * t.K;
    t.w = a.w[t.pt] + (int64_t)l * a.lstep * t.K * a.H;
    return t;
}

// The first tile of a workgroup's walk (then every gridDim.x-th). The
// hardware deals workgroups to the 8 XCDs round-robin (blockIdx.x mod 8),
// each XCD with its own L2. With xcd_walk set, each XCD's workgroups take a
// contiguous range of the tile indices of every round, so that neighbouring
// column tiles of a point, which read the same x, share one L2. Every
// workgroup still walks its tiles in increasing order, one per round, so
// the waits between points resolve as in the plain walk, and no sum
// changes order.
__device__ __forceinline__ int64_t step_first_tile(const StepArgs& a) {
    constexpr int kXcds = 8;
    const int g = (int)gridDim.x, bid = (int)blockIdx.x;
    if (!a.xcd_walk || g % kXcds) return bid;
    return (int64_t)(bid % kXcds) * (g / kXcds) + bid / kXcds;
}

// After a tile's partial is in LDS (tile[b][COLS]): publish it to this
// point's split set, and the last arrival fixes the column tile (splits in
// split order, the rank's slot, the ring and the residual, or the partial
// alone). `wait_all(ctr, target)` is the workgroup's bounded wait. Returns
// false if a wait failed (the caller stops its walk).
template <int BMAX, int COLS, int NT, typename WaitAll>
__device__ bool step_tile_epilogue(const StepArgs& a, const StepTile& t, const float* tile,
                                   int* s_flag, WaitAll wait_all) {
    const int tid = threadIdx.x, j = t.j, ct = t.ct;
    const int64_t len = (int64_t)a.batch * a.H;
    uint32_t* fixed = a.fixed + ct * kCounterStride;
    // The split set of point j was last used by point j - kStepBufs:
    // publish once this set's earlier rounds are fixed for this column tile
    // (word 2 of the tile's counter line counts them, in whatever order the
    // points' fix-ups complete). A single split uses no set.
    const int set = j % kStepBufs;
    uint32_t* rounds = a.counters + ((int64_t)set * a.col_tiles + ct) * kCounterStride + 2;
    if (t.splits > 1 && j >= kStepBufs && !wait_all(rounds, (uint32_t)(j / kStepBufs))) return false;

    float* slot = a.partials ? nullptr : a.slots + (int64_t)j * a.n_ranks * len;
    Epilogue e{};
    e.p = a.partials ? a.partials + (int64_t)j * len : slot + (int64_t)a.rank * len;
    e.ws_part = a.ws_part + (int64_t)set * a.part_stride;
    e.counters = a.counters + (int64_t)set * a.col_tiles * kCounterStride;
    e.splits = t.splits;
    e.ring_slots = slot;
    e.hidden = a.hidden;
    e.n_ranks = a.n_ranks;
    e.rank = a.rank;
    e.chunk = a.chunk;
    if (publish_split<COLS, NT>(e, tile, a.batch, a.H, ct, t.sp, tid, s_flag)) {
        // the residual columns of this tile are those (j-1, ct) wrote
        // (partials only: step_fixup returns before waiting)
        auto wait_prev = [&]() -> bool { return a.serial || j == 0 || wait_all(fixed, (uint32_t)j); };
        if (!step_fixup<BMAX, COLS, NT>(e, tile, a.batch, a.H, ct, tid, wait_prev)) return false;
        __syncthreads();
        if (tid == 0) {
            if (t.splits > 1) add_dev_u32(rounds, 1u);  // after the arrival counter's reset
            add_dev_u32(a.serial ? a.sync + kSyncDone : fixed, 1u);
            wait_mem();
        }
    }
    return true;
}

// The last workgroup to leave resets the step's sync words for the next
// launch (no workgroup waits on them any more).
template <int NT>
__device__ void step_exit(const StepArgs& a, int* s_flag) {
    const int tid = threadIdx.x;
    __syncthreads();
    if (tid == 0) *s_flag = add_dev_u32(a.sync + kSyncExit, 1u) == gridDim.x - 1;
    __syncthreads();
    if (*s_flag) {
        for (int c = tid; c < a.col_tiles; c += NT) st_dev_u32(a.fixed + c * kCounterStride, 0u);
        for (int c = tid; c < kStepBufs * a.col_tiles; c += NT)
            st_dev_u32(a.counters + (int64_t)c * kCounterStride + 2, 0u);
        if (tid == 0) {
            st_dev_u32(a.sync + kSyncDone, 0u);
            st_dev_u32(a.sync + kSyncExit, 0u);
        }
    }
}

template <int B, int COLS>
struct StepShared {
    uint32_t xs[kStepXsWords];  // the tile's x row pairs (dense), see stage_x_pairs
    float red[kValuWaves * COLS];
    __attribute__((aligned(16))) float tile[B * COLS];
    int flag;
    int wflag;  // outcome of the waits
};

// 16-byte weight loads per lane in each of the two register banks.
constexpr int step_bank_loads(int b) { return b <= 8 ? 12 : b <= 10 ? 8 : b <= 11 ? 6 : 4; }

// Stream rows [k0, k0+nr) of a column tile through two register banks of
// NB loads per lane: while one bank is multiplied the other is in flight,
// and the oldest loads are always the ones waited for. The lane's rows are
// r0 + i*RSTEP for i = 0, 1, ..., in pairs in order, as in valu_finish, so a
// tile of the same rows gives the same bits. stream_issue loads a tile's
// first two banks (the decode step issues them for its next tile before it
// reduces the current one); stream_run multiplies the tile, streaming the
// rest, and leaves both banks consumed.
template <int COLS>
struct LaneRows {
    static constexpr int LPR = COLS / 8;
    static constexpr int RPW = 64 / LPR;
    static constexpr int RSTEP = kValuWaves * RPW;
    // Rows [k0, k0+nr) of the matrix as a raw buffer: a 16-byte load past
    // row nr reads zero. The lane's byte offset of its first row and
    // column; lanes past column H start beyond the buffer (reads are zero).
    __amdgpu_buffer_rsrc_t rs;
    uint32_t voff, row_bytes;
    int r0, nr;
    __device__ __forceinline__ LaneRows(const uint16_t* w, int64_t H, int64_t k0, int nr_, int ct) {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int64_t n = (int64_t)ct * COLS + (lane % LPR) * 8;
        r0 = wave * RPW + lane / LPR;
        nr = nr_;
        row_bytes = (uint32_t)(H * 2);
        rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(w + k0 * H), (short)0,
                                               (int)((int64_t)nr * H * 2), kBufferRsrcWord3);
        voff = n < H ? (uint32_t)(r0 * H + n) * 2u : 0x80000000u;
    }
};

template <int COLS, int NB>
__device__ __forceinline__ void stream_bank(u32x4_t (&v)[NB], const LaneRows<COLS>& t, int64_t H,
                                            int base) {
    constexpr int RSTEP = LaneRows<COLS>::RSTEP;
    (void)H;
#pragma unroll
    for (int i = 0; i < NB; ++i)
        v[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                               t.rs, t.voff + (uint32_t)(base + i * RSTEP) * t.row_bytes,
                                               0, kCachePolicyNT));
}

template <int COLS, int NB>
__device__ __forceinline__ void stream_issue(u32x4_t (&va)[NB], u32x4_t (&vb)[NB],
                                             const LaneRows<COLS>& t, int64_t H) {
    stream_bank<COLS, NB>(va, t, H, 0);
    stream_bank<COLS, NB>(vb, t, H, LaneRows<COLS>::RSTEP * NB);
}

template <int B, int COLS, int NB>
__device__ __forceinline__ void stream_run(u32x4_t (&va)[NB], u32x4_t (&vb)[NB],
                                           const LaneRows<COLS>& t, int64_t H, const uint32_t* xs,
                                           float (&acc)[B][8]) {
    constexpr int RSTEP = LaneRows<COLS>::RSTEP;
    constexpr int BR = RSTEP * NB;  // rows per bank
    static_assert(NB % 2 == 0, "rows are taken in pairs");
    auto fma_bank = [&](const u32x4_t (&v)[NB], int base) {
        // base is a multiple of 2*RSTEP (banks hold an even number of loads)
#pragma unroll
        for (int i = 0; i < NB; i += 2) {
            const int r = t.r0 + base + i * RSTEP;
            if (r < t.nr) dot2_rows<B>(acc, v[i], v[i + 1], &xs[pair_index<RSTEP>(t.r0, base / RSTEP + i) * B]);
        }
    };
    for (int base = 0; base < t.nr; base += 2 * BR) {
        fma_bank(va, base);
        if (base + 2 * BR < t.nr) stream_bank<COLS, NB>(va, t, H, base + 2 * BR);
        fma_bank(vb, base + BR);
        if (base + 3 * BR < t.nr) stream_bank<COLS, NB>(vb, t, H, base + 3 * BR);
    }
}

// The whole decode step in one cooperative launch. Tiles are (point,
// column tile, split), walked in point order with a grid stride; a tile
// covers a long row range, streamed, with its x slice staged in LDS.
//
// Point order. The residual chain runs element by element: the fix-up of
// (point j, column tile c) reads the hidden-state columns of tile c that
// (j-1, c) wrote, and nothing else of earlier points, so by default a
// workgroup waits only for that (per-tile `fixed` counters) and tiles of
// later points stream while earlier ones are reduced. Points rotate over
// kStepBufs sets of split buffers and arrival counters; a split of point j
// publishes only once (j - kStepBufs, c) has been fixed, which frees its
// set (counted per set and column tile, so that this holds also where
// fix-ups complete out of point order: the partials-only mode has no
// residual chain). With `serial` the step also emulates a model whose activation at
// point j depends on the whole hidden state after j-1: every tile of point
// j waits, before it reads x, until all column tiles of j-1 are fixed. Each
// wait targets tiles earlier in the grid-stride order, and the launch is
// cooperative (all workgroups resident), so the earliest pending tile
// always proceeds. Both orders sum the same values in the same order: the
// bits do not depend on it.
template <int B, int COLS>
__global__ __launch_bounds__(kValuWaves * 64) void decode_step(StepArgs a) {
    constexpr int NT = kValuWaves * 64;
    constexpr int NB = step_bank_loads(B);
    __shared__ StepShared<B, COLS> sh;
    const int tid = threadIdx.x;
    const int64_t total = (int64_t)a.layers * (a.tiles[0] + a.tiles[1]);

    // tid 0 waits until *ctr >= target; every thread gets the outcome
    auto wait_all = [&](uint32_t* ctr, uint32_t target) -> bool {
        if (tid == 0) sh.wflag = wait_at_least(ctr, target, a.sync + kSyncErr, a.spin_limit);
        __syncthreads();
        compiler_barrier();
        return sh.wflag != 0;
    };

    // The workgroup's tiles q = q0 + m*gridDim.x. A tile's first two
    // banks are issued before the previous tile is reduced and published.
    u32x4_t va[NB], vb[NB];
    const int64_t q0 = step_first_tile(a);
    if (q0 < total) {
        const StepTile t0 = step_tile(a, q0);
        stream_issue<COLS, NB>(va, vb, LaneRows<COLS>(t0.w, a.H, t0.k0, t0.nr, t0.ct), a.H);
    }
    for (int64_t q = q0; q < total; q += gridDim.x) {
        const StepTile tq = step_tile(a, q);

        __syncthreads();  // LDS of the previous tile is no longer read
        // A failed wait (error word set) ends the workgroup's walk; every
        // later wait fails at once, so the grid drains.
        if (a.serial && !wait_all(a.sync + kSyncDone, (uint32_t)tq.j * a.col_tiles)) break;

        constexpr int RSTEP = LaneRows<COLS>::RSTEP;
        stage_x_pairs<B, RSTEP, NT>(sh.xs, tq.x, tq.K, tq.k0, tq.nr);
        __syncthreads();

        float acc[B][8];
#pragma unroll
        for (int bb = 0; bb < B; ++bb)
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[bb][c] = 0.f;
        stream_run<B, COLS, NB>(va, vb, LaneRows<COLS>(tq.w, a.H, tq.k0, tq.nr, tq.ct), a.H, sh.xs, acc);
        if (q + gridDim.x < total) {
            const StepTile tn = step_tile(a, q + gridDim.x);
            stream_issue<COLS, NB>(va, vb, LaneRows<COLS>(tn.w, a.H, tn.k0, tn.nr, tn.ct), a.H);
        }
        reduce_tile<B, COLS>(acc, sh.red, sh.tile);
        if (!step_tile_epilogue<B, COLS, NT>(a, tq, sh.tile, &sh.flag, wait_all)) break;
    }
    step_exit<NT>(a, &sh.flag);
}

// The matrix-core decode step (b = 16..64, BT tiles of 16 tokens), on the
// same tiles, point order, split sets and epilogue as decode_step. A tile
// is 128 columns by the plan's tile length in rows (2048 by default, a
// whole K in the up projection). Each of the kStepMfmaWaves waves takes
// 32-row steps (wave w: steps w, w + NW, ...): per lane 8 rows x 16 bytes
// of weights, transposed with v_perm into k-major B operands, and one
// 16-byte A operand (8 rows of x) per 16 tokens, both loaded one step
// ahead, multiplied on v_mfma_f32_16x16x32_bf16. Each row of x is read
// once per tile (b/128 bytes per weight byte), as staging it would read
// it, without the staging's wait or its bound on the tile length. The
// waves' D tiles are summed in wave order in LDS.
template <int BT>
struct StepMfmaShared {
    float red[kStepMfmaWaves * 16 * kMfmaCols];
    __attribute__((aligned(16))) float tile[BT * 16 * kMfmaCols];
    int flag;
    int wflag;
};

template <int BT>
__global__ __launch_bounds__(kStepMfmaWaves * 64) void decode_step_mfma(StepArgs a) {
    constexpr int NW = kStepMfmaWaves;
    constexpr int NT = NW * 64;
    constexpr int COLS = kMfmaCols;
    __shared__ StepMfmaShared<BT> sh;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4;   // k group: rows 8g .. 8g+7 of a 32-row step
    const int i = lane & 15;   // column group (B operand) / token row (A operand)
    const int64_t total = (int64_t)a.layers * (a.tiles[0] + a.tiles[1]);

    auto wait_all = [&](uint32_t* ctr, uint32_t target) -> bool {
        if (tid == 0) sh.wflag = wait_at_least(ctr, target, a.sync + kSyncErr, a.spin_limit);
        __syncthreads();
        compiler_barrier();
        return sh.wflag != 0;
    };

    for (int64_t q = step_first_tile(a); q < total; q += gridDim.x) {
        const StepTile tq = step_tile(a, q);
        const int nr = tq.nr;

        __syncthreads();  // LDS of the previous tile is no longer read
        if (a.serial && !wait_all(a.sync + kSyncDone, (uint32_t)tq.j * a.col_tiles)) break;

        // The tile's weight rows as a raw buffer (rows past nr and columns
        // past H read zero); x [b][K] as another (tokens past b read zero).
        const int64_t n = (int64_t)tq.ct * COLS + i * 8;
        const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(tq.w + tq.k0 * a.H), (short)0, (int)((int64_t)nr * a.H * 2),
            kBufferRsrcWord3);
        const uint32_t row_bytes = (uint32_t)(a.H * 2);
        const uint32_t voff = n < a.H ? (uint32_t)((8 * g) * a.H + n) * 2u : 0x80000000u;
        const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(tq.x), (short)0, (int)((int64_t)a.batch * tq.K * 2), kBufferRsrcWord3);
        const bool x_vec = (tq.K & 7) == 0;
        auto load_step = [&](u32x4_t (&wv)[8], u32x4_t (&xv)[BT], int step) {
#pragma unroll
            for (int r = 0; r < 8; ++r)
                wv[r] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                        rw, voff + (uint32_t)(step + r) * row_bytes, 0,
                                                        kCachePolicyNT));
            // A operands: x[bt*16 + i][k0 + step + 8g .. +7]; rows past the
            // tile read as zero (their weights are zero too)
            const int r0 = step + 8 * g;
#pragma unroll
            for (int bt = 0; bt < BT; ++bt) {
                const uint32_t xo = (uint32_t)(((int64_t)(bt * 16 + i) * tq.K + tq.k0 + r0) * 2);
                if (x_vec && r0 + 8 <= nr) {
                    xv[bt] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rx, xo, 0, 0));
                } else {
                    uint32_t h[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        h[u] = r0 + u < nr ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rx, xo + 2 * u, 0, 0)
                                           : 0u;
                    xv[bt] = u32x4_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                                     h[6] | (h[7] << 16)};
                }
            }
        };

        floatx4_t acc[BT][8];
#pragma unroll
        for (int bt = 0; bt < BT; ++bt)
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[bt][c] = floatx4_t{0.f, 0.f, 0.f, 0.f};
        u32x4_t wv[8], xv[BT];
        if (wave * 32 < nr) load_step(wv, xv, wave * 32);
        for (int step = wave * 32; step < nr; step += NW * 32) {
            // column c's B operand (its 8 rows, k-major) just before its MFMAs
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const bool hi = c & 1;
                u32x4_t bw;
                bw.x = pair_rows(wv[0][c >> 1], wv[1][c >> 1], hi);
                bw.y = pair_rows(wv[2][c >> 1], wv[3][c >> 1], hi);
                bw.z = pair_rows(wv[4][c >> 1], wv[5][c >> 1], hi);
                bw.w = pair_rows(wv[6][c >> 1], wv[7][c >> 1], hi);
                const bf16x8_t bop = __builtin_bit_cast(bf16x8_t, bw);
#pragma unroll
                for (int bt = 0; bt < BT; ++bt)
                    acc[bt][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, xv[bt]), bop, acc[bt][c], 0, 0, 0);
            }
            if (step + NW * 32 < nr) load_step(wv, xv, step + NW * 32);
        }

        // D layout of a 16x16 fp32 MFMA tile: lane holds rows 4*(lane/16)+q,
        // column lane%16; here rows are tokens and MFMA column i' is tile
        // column 8*i' + c. Waves summed in wave order.
        for (int bt = 0; bt < BT; ++bt) {
#pragma unroll
            for (int c = 0; c < 8; ++c)
#pragma unroll
                for (int qq = 0; qq < 4; ++qq)
                    sh.red[(wave * 16 + 4 * g + qq) * COLS + i * 8 + c] = acc[bt][c][qq];
            __syncthreads();
            for (int idx = tid; idx < 16 * COLS; idx += NT) {
                float sum = sh.red[idx];
#pragma unroll
                for (int wq = 1; wq < NW; ++wq) sum += sh.red[wq * 16 * COLS + idx];
                sh.tile[bt * 16 * COLS + idx] = sum;
            }
            __syncthreads();
        }
        if (!step_tile_epilogue<BT * 16, COLS, NT>(a, tq, sh.tile, &sh.flag, wait_all)) break;
    }
    step_exit<NT>(a, &sh.flag);
}

// -------------------------------------------- column-parallel SwiGLU --

// a = silu(g) * u elementwise, rounded to bf16 nearest-even (the down
// projection's x slice), for `layers` layers: sums fp32 [layers][2][len]
// (the gate's, then the up's), out bf16 [layers][len].
__global__ __launch_bounds__(256) void swiglu_kernel(const float* sums, uint16_t* out, int64_t len,
                                                     int64_t total) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    const int64_t l = i / len, e = i - l * len;
    const float gv = sums[(2 * l) * len + e];
    const float silu = gv / (1.0f + expf(-gv));
    out[i] = f32_to_bf16_rne(silu * sums[(2 * l + 1) * len + e]);
}

// fp32 sums rounded to bf16 nearest-even (the QKV projection's output).
__global__ __launch_bounds__(256) void round_bf16_kernel(const float* sums, uint16_t* out,
                                                         int64_t total) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < total) out[i] = f32_to_bf16_rne(sums[i]);
}

// ------------------------------------------------------------ MFMA GEMM --

template <int BT>  // batch tiles of 16 rows
__global__ __launch_bounds__(kMfmaWaves * 64) void mfma_gemm(GemvArgs a, int batch) {
    constexpr int NT = kMfmaWaves * 64;
    constexpr int COLS = kMfmaCols;
    __shared__ float red[kMfmaWaves * 16 * COLS];  // 32 KB
    __shared__ __align__(16) float tile[BT * 16 * COLS];
    __shared__ int s_flag;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ct = blockIdx.x % a.col_tiles;
    const int sp = blockIdx.x / a.col_tiles;
    const int64_t k0 = (int64_t)sp * a.rows;
    const int rows = (int)(a.K - k0 < a.rows ? a.K - k0 : a.rows);
    const int g = lane >> 4;   // k group: rows 8g .. 8g+7 of a 32-row step
    const int i = lane & 15;   // column group: columns 8i .. 8i+7 of the tile
    const int64_t n = (int64_t)ct * COLS + i * 8;
    const bool col_ok = n < a.H;
    const bool x_vec = (a.K & 7) == 0;

    floatx4_t acc[BT][8];
#pragma unroll
    for (int bt = 0; bt < BT; ++bt)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[bt][c] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    // The wave's 32-row steps. Once a step's weight rows are rearranged into
    // B operands, the next step's rows (s + 4*32) are loaded into the same
    // registers while this step is multiplied (rows past the split read
    // nothing and give zeros).
    auto load_w = [&](u32x4_t (&wv)[8], int step) {
        const int64_t kr = k0 + step + 8 * g;  // first of this lane's 8 rows
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const bool ok = col_ok && (step + 8 * g + j) < rows;
            wv[j] = ok ? load_stream16(a.w + (kr + j) * a.H + n) : u32x4_t{0u, 0u, 0u, 0u};
        }
    };
    u32x4_t wv[8];
    load_w(wv, wave * 32);
    for (int step = wave * 32; step < rows; step += kMfmaWaves * 32) {
        const int64_t kr = k0 + step + 8 * g;
        // A operands: x[bt*16 + i][kr .. kr+7]
        bf16x8_t xa[BT];
#pragma unroll
        for (int bt = 0; bt < BT; ++bt) {
            int brow = bt * 16 + i;
            u32x4_t xv = u32x4_t{0u, 0u, 0u, 0u};
            if (brow < batch) {
                const uint16_t* xp = a.x + (int64_t)brow * a.K + kr;
                int left = rows - (step + 8 * g);
                if (x_vec && left >= 8) {
                    xv = *reinterpret_cast<const u32x4_t*>(xp);
                } else {
                    uint16_t t[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) t[j] = j < left ? xp[j] : (uint16_t)0;
                    xv.x = t[0] | ((uint32_t)t[1] << 16);
                    xv.y = t[2] | ((uint32_t)t[3] << 16);
                    xv.z = t[4] | ((uint32_t)t[5] << 16);
                    xv.w = t[6] | ((uint32_t)t[7] << 16);
                }
            }
            xa[bt] = __builtin_bit_cast(bf16x8_t, xv);
        }
        // B operands: for each of the lane's 8 columns c, its 8 rows as k-major bf16x8
        bf16x8_t bop[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const bool hi = c & 1;
            u32x4_t bw;
            bw.x = pair_rows(wv[0][c >> 1], wv[1][c >> 1], hi);
            bw.y = pair_rows(wv[2][c >> 1], wv[3][c >> 1], hi);
            bw.z = pair_rows(wv[4][c >> 1], wv[5][c >> 1], hi);
            bw.w = pair_rows(wv[6][c >> 1], wv[7][c >> 1], hi);
            bop[c] = __builtin_bit_cast(bf16x8_t, bw);
        }
        load_w(wv, step + kMfmaWaves * 32);
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
            for (int bt = 0; bt < BT; ++bt)
                acc[bt][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[bt], bop[c], acc[bt][c], 0, 0, 0);
    }

    // D layout of a 16x16 fp32 MFMA tile: lane holds rows 4*(lane/16)+q,
    // column lane%16. Here rows are batch rows and MFMA column i' is
    // tile column 8*i' + c.
    for (int bt = 0; bt < BT; ++bt) {
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                red[(wave * 16 + 4 * g + q) * COLS + i * 8 + c] = acc[bt][c][q];
        __syncthreads();
        for (int idx = tid; idx < 16 * COLS; idx += NT) {
            float s = red[idx];
#pragma unroll
            for (int wq = 1; wq < kMfmaWaves; ++wq) s += red[wq * 16 * COLS + idx];
            tile[bt * 16 * COLS + idx] = s;
        }
        __syncthreads();
    }
    const bool last = publish_split<COLS, NT>(a.epi, tile, batch, a.H, ct, sp, tid, &s_flag);
    if (a.epi.spread && a.epi.splits > 1)
        spread_fixup<COLS, NT>(a.epi, batch, a.H, ct, sp, tid);
    else if (last)
        fixup_tile<COLS, NT>(a.epi, tile, batch, a.H, ct, tid);
}

// ----------------------------------------------------------- ring reduce --

__global__ void ring_reduce_kernel(const float* partials, const float* residual, float* out,
                                   uint16_t* out_bf16, int64_t len, int64_t chunk, int n_ranks) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= len) return;
    float o = ring_element(partials, len, i, chunk, n_ranks, -1, 0.f, residual[i]);
    out[i] = o;
    if (out_bf16) out_bf16[i] = f32_to_bf16_rne(o);
}

__global__ void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t v) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

// ------------------------------------------------------------- dispatch --

typedef void (*valu_fn)(GemvArgs);
typedef void (*step_fn)(StepArgs);

template <int COLS>
valu_fn valu_kernel_for(int b) {
    switch (b) {
        case 1: return valu_gemv<1, COLS>;   case 2: return valu_gemv<2, COLS>;
        case 3: return valu_gemv<3, COLS>;   case 4: return valu_gemv<4, COLS>;
        case 5: return valu_gemv<5, COLS>;   case 6: return valu_gemv<6, COLS>;
        case 7: return valu_gemv<7, COLS>;   case 8: return valu_gemv<8, COLS>;
        case 9: return valu_gemv<9, COLS>;   case 10: return valu_gemv<10, COLS>;
        case 11: return valu_gemv<11, COLS>; case 12: return valu_gemv<12, COLS>;
        case 13: return valu_gemv<13, COLS>; case 14: return valu_gemv<14, COLS>;
        case 15: return valu_gemv<15, COLS>;
    }
    return nullptr;
}

template <int COLS>
step_fn step_kernel_for(int b) {
    switch (b) {
        case 1: return decode_step<1, COLS>;   case 2: return decode_step<2, COLS>;
        case 3: return decode_step<3, COLS>;   case 4: return decode_step<4, COLS>;
        case 5: return decode_step<5, COLS>;   case 6: return decode_step<6, COLS>;
        case 7: return decode_step<7, COLS>;   case 8: return decode_step<8, COLS>;
        case 9: return decode_step<9, COLS>;   case 10: return decode_step<10, COLS>;
        case 11: return decode_step<11, COLS>; case 12: return decode_step<12, COLS>;
        case 13: return decode_step<13, COLS>; case 14: return decode_step<14, COLS>;
        case 15: return decode_step<15, COLS>;
    }
    return nullptr;
}

step_fn step_mfma_kernel(int b) {
    switch ((b + 15) / 16) {
        case 1: return decode_step_mfma<1>;
        case 2: return decode_step_mfma<2>;
        case 3: return decode_step_mfma<3>;
        case 4: return decode_step_mfma<4>;
    }
    return nullptr;
}

valu_fn valu_kernel(int b, int cols) {
    switch (cols) {
        case 128: return valu_kernel_for<128>(b);
        case 256: return valu_kernel_for<256>(b);
        case 512: return valu_kernel_for<512>(b);
    }
    return nullptr;
}

step_fn step_kernel(int b, int cols) {
    switch (cols) {
        case 128: return step_kernel_for<128>(b);
        case 256: return step_kernel_for<256>(b);
        case 512: return step_kernel_for<512>(b);
    }
    return nullptr;
}

typedef void (*mfma_fn)(GemvArgs, int);
mfma_fn mfma_kernel(int b) {
    switch ((b + 15) / 16) {
        case 1: return mfma_gemm<1>;
        case 2: return mfma_gemm<2>;
        case 3: return mfma_gemm<3>;
        case 4: return mfma_gemm<4>;
    }
    return nullptr;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

uint32_t* ws_counters(void* ws) { return reinterpret_cast<uint32_t*>(ws); }
uint32_t* ws_sync(void* ws) {
    return reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(ws) + kSyncOffset);
}
float* ws_partials(void* ws) {
    return reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + tp_ws_partials_offset());
}

// Resident workgroups of a kernel on the current device (cooperative grid).
int resident_grid(const void* kernel, int block) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, 0) != hipSuccess) return 0;
    return per_cu * cus;
}

// Whether the matrix-core projection of geometry g spreads its split-K
// fix-up over all splits: only where every workgroup of the grid can be
// resident at once on an idle device (the kernel's occupancy, cached per
// device and token blocks), since a split waits for the others' partials.
// The wait is bounded: should other work hold CUs for long, the error word
// is set and the launch still ends. (A cooperative launch would guarantee
// residency but costs more host time per launch than the fix-up saves.)
bool mfma_spread(const PointGeom& g, int batch) {
    if (g.path != TP_PATH_MFMA || g.splits < 2) return false;
    const int bt = (batch + 15) / 16;
    if (bt < 1 || bt > 4) return false;
    static int cap[16][5];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) return false;
    if (cap[dev][bt] == 0) {
        const int c = resident_grid(reinterpret_cast<const void*>(mfma_kernel(batch)), kMfmaWaves * 64);
        cap[dev][bt] = c > 0 ? c : -1;
    }
    return g.grid <= cap[dev][bt];
}

// Launch one projection (and its optional ring epilogue).
tp_status launch_projection(const tp_plan_s* p, const PointGeom& g, int batch, const void* x,
                            const void* w, const Epilogue& epi, hipStream_t st) {
    GemvArgs a;
    a.x = static_cast<const uint16_t*>(x);
    a.w = static_cast<const uint16_t*>(w);
    a.K = g.k_r;
    a.H = p->hidden;
    a.rows = g.rows;
    a.col_tiles = g.col_tiles;
    a.epi = epi;
    a.epi.err = ws_sync(epi.counters) + kSyncErr;
    a.epi.spin_limit = 1u << 21;
    a.epi.spread = mfma_spread(g, batch) ? 1 : 0;
    // host-side checks of what the kernels assume
    if (g.splits < 1 || g.col_tiles < 1 || (int64_t)g.rows * g.splits < g.k_r) return TP_ERR_INVALID_ARG;
    if ((int64_t)g.splits * batch * p->hidden * 4 >= ((int64_t)1 << 31)) return TP_ERR_UNSUPPORTED;
    if (g.col_tiles > kMaxCounters) return TP_ERR_UNSUPPORTED;
    if (g.path == TP_PATH_VALU) {
        if (batch < 1 || batch > kValuMaxBatch || g.rows > valu_rows_max(batch, g.cols))
            return TP_ERR_UNSUPPORTED;
        valu_fn k = valu_kernel(batch, g.cols);
        if (!k) return TP_ERR_UNSUPPORTED;
        hipLaunchKernelGGL(k, dim3(g.grid), dim3(kValuWaves * 64), 0, st, a);
    } else {
        if (batch < kMfmaMinBatch || batch > kMfmaMaxBatch || g.cols != kMfmaCols) return TP_ERR_UNSUPPORTED;
        mfma_fn k = mfma_kernel(batch);
        if (!k) return TP_ERR_UNSUPPORTED;
        hipLaunchKernelGGL(k, dim3(g.grid), dim3(kMfmaWaves * 64), 0, st, a, batch);
    }
    return tp_launch_status(st);
}

// The persistent step; with `partials` set, only the 2L partials (no ring,
// no residual) into partials [L][2][b][H].
tp_status decode_persistent(const tp_plan_s* p, int32_t n_layers, int32_t rank, const void* x_attn,
                            const void* w_o, const void* x_ffn, const void* w_down, float* slots,
                            float* hidden, float* partials, void* ws, hipStream_t st,
                            int32_t lstep = 1) {
    const int b = p->batch;
    if (b < 1 || b > kMfmaMaxBatch) return TP_ERR_UNSUPPORTED;
    const bool mfma = tp_step_mfma(p);
    PointGeom geo[2] = {tp_step_geom(p, 0), tp_step_geom(p, 1)};
    if (geo[0].cols != geo[1].cols || geo[0].col_tiles != geo[1].col_tiles) return TP_ERR_UNSUPPORTED;
    // kStepBufs sets of arrival counters in [0, kSyncOffset); the fixed
    // counters in [kFixedOffset, kCounterBytes)
    if ((int64_t)kStepBufs * geo[0].col_tiles > kMaxCounters ||
        kFixedOffset + (int64_t)geo[0].col_tiles * kCounterStride * 4 > kCounterBytes)
        return TP_ERR_UNSUPPORTED;
    // the matrix-core step reads x through a buffer of b*K*2 bytes
    if (mfma && ((int64_t)b * geo[1].k_r * 2 >= ((int64_t)1 << 31) ||
                 (int64_t)b * geo[0].k_r * 2 >= ((int64_t)1 << 31)))
        return TP_ERR_UNSUPPORTED;
    for (int pt = 0; pt < 2; ++pt)
        // (the lanes' 32-bit buffer offsets, rows read ahead included, stay
        // below 2^31, so that a lane past column H stays out of range)
        if (geo[pt].rows < 1 || (!mfma && (int64_t)(geo[pt].rows / 2 + 16) * b > kStepXsWords) ||
            (int64_t)(geo[pt].rows + 1024) * p->hidden * 2 >= ((int64_t)1 << 31) ||
            (int64_t)geo[pt].rows * geo[pt].splits < geo[pt].k_r)
            return TP_ERR_UNSUPPORTED;
    if ((int64_t)n_layers * (geo[0].grid + geo[1].grid) >= (int64_t)1 << 31) return TP_ERR_UNSUPPORTED;
    const int64_t part_stride = tp_step_partial_buffer_bytes(p) / 4;
    if (part_stride * 4 * kStepBufs >= ((int64_t)1 << 31)) return TP_ERR_UNSUPPORTED;
    step_fn k = mfma ? step_mfma_kernel(b) : step_kernel(b, geo[0].cols);
    const int block = mfma ? kStepMfmaWaves * 64 : kValuWaves * 64;
    if (!k) return TP_ERR_UNSUPPORTED;
    StepArgs a;
    a.batch = b;
    a.x[0] = static_cast<const uint16_t*>(x_attn);
    a.x[1] = static_cast<const uint16_t*>(x_ffn);
    a.w[0] = static_cast<const uint16_t*>(w_o);
    a.w[1] = static_cast<const uint16_t*>(w_down);
    a.slots = slots;
    a.hidden = hidden;
    a.partials = partials;
    a.ws_part = ws_partials(ws);
    a.part_stride = part_stride;
    a.counters = ws_counters(ws);
    a.fixed = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + kFixedOffset);
    a.sync = ws_sync(ws);
    a.serial = p->serial_points && !partials ? 1 : 0;
    a.H = p->hidden;
    for (int pt = 0; pt < 2; ++pt) {
        a.K[pt] = geo[pt].k_r;
        a.rows[pt] = geo[pt].rows;
        a.splits[pt] = geo[pt].splits;
        a.tiles[pt] = geo[pt].grid;
    }
    a.col_tiles = geo[0].col_tiles;
    a.layers = n_layers;
    a.lstep = lstep;
    a.xcd_walk = p->xcd_walk > 0 ? 1 : 0;
    a.n_ranks = p->n_ranks;
    a.rank = rank;
    a.chunk = (int64_t)b * p->hidden / p->n_ranks;
    a.spin_limit = 1u << 21;
    if (n_layers == 0) return TP_OK;
    int cap = resident_grid(reinterpret_cast<const void*>(k), block);
    if (cap < 1) return TP_ERR_DEVICE;
    // Every resident workgroup: the tiles of later points are taken up while
    // earlier ones are reduced (the waits order what must be ordered).
    const int64_t total = (int64_t)n_layers * (geo[0].grid + geo[1].grid);
    int grid = total < cap ? (int)total : cap;
    void* args[] = {&a};
    if (hipLaunchCooperativeKernel(reinterpret_cast<const void*>(k), dim3(grid), dim3(block), args,
                                   0, st) != hipSuccess)
        return TP_ERR_DEVICE;
    return tp_launch_status(st);
}

}  // namespace

tp_status tp_fill_u32(uint32_t* p, int64_t n, uint32_t v, void* stream) {
    if (n <= 0) return TP_OK;
    hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       (hipStream_t)stream, p, n, v);
    return tp_launch_status(stream);
}

// Debug mode: -1 until first read (then the environment decides), 0 or 1.
static std::atomic<int> g_debug_sync{-1};

static bool debug_sync_on() {
    int v = g_debug_sync.load(std::memory_order_relaxed);
    if (v < 0) {
        const char* e = getenv("TP_DEBUG_SYNC");
        int want = e && e[0] && strcmp(e, "0") != 0 ? 1 : 0;
        g_debug_sync.compare_exchange_strong(v, want);
        v = g_debug_sync.load(std::memory_order_relaxed);
    }
    return v == 1;
}

tp_status tp_launch_status(void* stream) {
    if (hipGetLastError() != hipSuccess) return TP_ERR_DEVICE;
    if (!debug_sync_on()) return TP_OK;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing((hipStream_t)stream, &cs) != hipSuccess) return TP_ERR_DEVICE;
    if (cs != hipStreamCaptureStatusNone) return TP_OK;
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return TP_ERR_DEVICE;
    return hipGetLastError() == hipSuccess ? TP_OK : TP_ERR_DEVICE;
}

extern "C" {

tp_status tp_set_debug_sync(int32_t on) {
    if (on != 0 && on != 1) return TP_ERR_INVALID_ARG;
    g_debug_sync.store(on, std::memory_order_relaxed);
    return TP_OK;
}

tp_status tp_workspace_init(tp_plan_t p, void* ws, void* stream) {
    if (!p || !ws) return TP_ERR_INVALID_ARG;
    if (!aligned16(ws)) return TP_ERR_ALIGNMENT;
    int64_t n = kCounterBytes / 4;
    hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       (hipStream_t)stream, ws_counters(ws), n, 0u);
    return tp_launch_status(stream);
}

tp_status tp_workspace_status(tp_plan_t p, const void* ws, int32_t* flags) {
    if (!p || !flags) return TP_ERR_INVALID_ARG;
    if (!ws) return tp_scratch_status(flags);  // the no-alloc entry point's scratch
    if (!aligned16(ws)) return TP_ERR_ALIGNMENT;
    uint32_t v = 0;
    if (hipMemcpy(&v, static_cast<const char*>(ws) + kSyncOffset + 4 * kSyncErr, 4,
                  hipMemcpyDeviceToHost) != hipSuccess)
        return TP_ERR_DEVICE;
    *flags = (int32_t)v;
    return TP_OK;
}

tp_status tp_rowparallel_partial(tp_plan_t p, int32_t point, const void* x, const void* w,
                                 float* out, void* ws, void* stream) {
    if (!p || !x || !w || !out || !ws) return TP_ERR_INVALID_ARG;
    if (point != TP_POINT_ATTN_OUT && point != TP_POINT_FFN_DOWN) return TP_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(w) || !aligned16(out) || !aligned16(ws)) return TP_ERR_ALIGNMENT;
    PointGeom g = tp_point_geom(p, point);
    Epilogue e{};
    e.p = out;
    e.ws_part = ws_partials(ws);
    e.counters = ws_counters(ws);
    e.splits = g.splits;
    return launch_projection(p, g, p->batch, x, w, e, (hipStream_t)stream);
}

tp_status tp_gate_up_swiglu(tp_plan_t p, int32_t n_layers, const void* x, const void* w_gate,
                            const void* w_up, void* out, void* ws, void* stream) {
    if (!p || n_layers < 0) return TP_ERR_INVALID_ARG;
    if (n_layers == 0) return TP_OK;  // nothing is read or written
    if (!x || !w_gate || !w_up || !out || !ws) return TP_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(w_gate) || !aligned16(w_up) || !aligned16(out) || !aligned16(ws))
        return TP_ERR_ALIGNMENT;
    if (!tp_swiglu_ok(p)) return TP_ERR_UNSUPPORTED;
    const int64_t b = p->batch, H = p->hidden, C = p->inter / p->n_ranks;
    if ((b * C) % 8) return TP_ERR_ALIGNMENT;  // each layer's output slice stays 16-byte aligned
    const tp_plan_s q = tp_swiglu_plan(p);
    float* gu = reinterpret_cast<float*>(static_cast<char*>(ws) + tp_ws_swiglu_offset(p));
    const int32_t per = tp_swiglu_layers_per_launch(p);
    // as few launches as the sums region allows, with the layers spread
    // evenly over them (no short last launch that leaves the chip idle)
    const int32_t launches = (n_layers + per - 1) / per;
    hipStream_t st = (hipStream_t)stream;
    for (int32_t k = 0; k < launches; ++k) {
        const int32_t l0 = (int32_t)((int64_t)k * n_layers / launches);
        const int32_t nl = (int32_t)((int64_t)(k + 1) * n_layers / launches) - l0;
        const uint16_t* xl = static_cast<const uint16_t*>(x) + (int64_t)l0 * b * H;
        const uint16_t* wg = static_cast<const uint16_t*>(w_gate) + (int64_t)l0 * H * C;
        const uint16_t* wu = static_cast<const uint16_t*>(w_up) + (int64_t)l0 * H * C;
        // the gate and up sums of nl layers: the two points of each layer of
        // one persistent partials launch (x is the same for both)
        tp_status s = decode_persistent(&q, nl, 0, xl, wg, xl, wu, nullptr, nullptr, gu, ws, st);
        if (s != TP_OK) return s;
        const int64_t total = (int64_t)nl * b * C;
        hipLaunchKernelGGL(swiglu_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, gu,
                           static_cast<uint16_t*>(out) + (int64_t)l0 * b * C, b * C, total);
        if (hipGetLastError() != hipSuccess) return TP_ERR_DEVICE;
    }
    return TP_OK;
}

tp_status tp_qkv_proj(tp_plan_t p, int32_t n_layers, const void* x, const void* w_qkv, void* out,
                      void* ws, void* stream) {
    if (!p || n_layers < 0) return TP_ERR_INVALID_ARG;
    if (n_layers == 0) return TP_OK;  // nothing is read or written
    if (!x || !w_qkv || !out || !ws) return TP_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(w_qkv) || !aligned16(out) || !aligned16(ws))
        return TP_ERR_ALIGNMENT;
    if (!tp_qkv_ok(p)) return TP_ERR_UNSUPPORTED;
    const int64_t b = p->batch, H = p->hidden, C = p->qkv_cols;
    if ((b * C) % 8) return TP_ERR_ALIGNMENT;  // each layer's output slice stays 16-byte aligned
    tp_plan_s q = tp_colproj_plan(p, C);
    // From 16 tokens on, a narrow point's few column tiles each re-read a
    // wide x: by default each XCD's workgroups then take contiguous tiles of
    // a round, so that a point's tiles share one L2 (the same bits either
    // way). Measured on MI355X: +6-8 % at 768 and 1280 columns, -3 % at
    // 3072 (more tiles per point already share x).
    if (q.xcd_walk < 0) q.xcd_walk = b >= 16 && C <= 2048 ? 1 : 0;
    float* sums = reinterpret_cast<float*>(static_cast<char*>(ws) + tp_ws_qkv_offset(p));
    const int32_t per = tp_qkv_layers_per_launch(p);  // even
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    const uint16_t* wb = static_cast<const uint16_t*>(w_qkv);
    uint16_t* ob = static_cast<uint16_t*>(out);
    hipStream_t st = (hipStream_t)stream;
    // Layers 2u and 2u+1 of a launch are the two points of the step's layer
    // u (layer stride 2), so their sums land in layer order. An odd last
    // layer takes a launch of its own, as both points (the second's sums
    // are not used).
    const int32_t even = n_layers - n_layers % 2;
    const int32_t launches = (even + per - 1) / per;
    auto run = [&](int32_t l0, int32_t units, int32_t lstep) -> tp_status {
        const uint16_t* x0 = xb + (int64_t)l0 * b * H;
        const uint16_t* w0 = wb + (int64_t)l0 * H * C;
        const uint16_t* x1 = lstep == 2 ? x0 + b * H : x0;
        const uint16_t* w1 = lstep == 2 ? w0 + H * C : w0;
        tp_status s = decode_persistent(&q, units, 0, x0, w0, x1, w1, nullptr, nullptr, sums, ws, st,
                                        lstep);
        if (s != TP_OK) return s;
        const int64_t total = (int64_t)(lstep == 2 ? 2 * units : 1) * b * C;
        hipLaunchKernelGGL(round_bf16_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, sums,
                           ob + (int64_t)l0 * b * C, total);
        return tp_launch_status(stream);
    };
    for (int32_t k = 0; k < launches; ++k) {
        // layer pairs spread evenly over the launches
        const int32_t u0 = (int32_t)((int64_t)k * (even / 2) / launches);
        const int32_t u1 = (int32_t)((int64_t)(k + 1) * (even / 2) / launches);
        tp_status s = run(2 * u0, u1 - u0, 2);
        if (s != TP_OK) return s;
    }
    if (n_layers % 2) return run(n_layers - 1, 1, 1);
    return TP_OK;
}

tp_status tp_rowparallel_partials(tp_plan_t p, int32_t n_layers, const void* x_attn, const void* w_o,
                                  const void* x_ffn, const void* w_down, float* out, void* ws,
                                  void* stream) {
    if (!p || n_layers < 0) return TP_ERR_INVALID_ARG;
    if (n_layers == 0) return TP_OK;  // nothing is read or written
    if (!x_attn || !w_o || !x_ffn || !w_down || !out || !ws) return TP_ERR_INVALID_ARG;
    if (!aligned16(x_attn) || !aligned16(w_o) || !aligned16(x_ffn) || !aligned16(w_down) ||
        !aligned16(out) || !aligned16(ws))
        return TP_ERR_ALIGNMENT;
    const int64_t b = p->batch, H = p->hidden, len = b * H;
    PointGeom geo[2] = {tp_point_geom(p, 0), tp_point_geom(p, 1)};
    // every slice of the stacked inputs must stay 16-byte aligned
    for (int pt = 0; pt < 2; ++pt)
        if ((b * geo[pt].k_r) % 8) return TP_ERR_ALIGNMENT;
    hipStream_t st = (hipStream_t)stream;
    if (tp_decode_mode(p) == 2)
        return decode_persistent(p, n_layers, 0, x_attn, w_o, x_ffn, w_down, nullptr, nullptr, out,
                                 ws, st);
    for (int32_t l = 0; l < n_layers; ++l)
        for (int pt = 0; pt < 2; ++pt) {
            const PointGeom& g = geo[pt];
            const uint16_t* xb = static_cast<const uint16_t*>(pt == 0 ? x_attn : x_ffn);
            const uint16_t* wb = static_cast<const uint16_t*>(pt == 0 ? w_o : w_down);
            Epilogue e{};
            e.p = out + ((int64_t)l * 2 + pt) * len;
            e.ws_part = ws_partials(ws);
            e.counters = ws_counters(ws);
            e.splits = g.splits;
            tp_status s = launch_projection(p, g, (int)b, xb + (int64_t)l * b * g.k_r,
                                            wb + (int64_t)l * g.k_r * H, e, st);
            if (s != TP_OK) return s;
        }
    return TP_OK;
}

tp_status tp_ring_reduce(tp_plan_t p, const float* partials, const float* residual, float* out,
                         void* out_bf16, void* stream) {
    if (!p || !partials || !residual || !out) return TP_ERR_INVALID_ARG;
    if (!aligned16(partials) || !aligned16(residual) || !aligned16(out) ||
        (out_bf16 && !aligned16(out_bf16)))
        return TP_ERR_ALIGNMENT;
    int64_t len = (int64_t)p->batch * p->hidden;
    int64_t chunk = len / p->n_ranks;
    hipLaunchKernelGGL(ring_reduce_kernel, dim3((unsigned)((len + 255) / 256)), dim3(256), 0,
                       (hipStream_t)stream, partials, residual, out,
                       static_cast<uint16_t*>(out_bf16), len, chunk, (int)p->n_ranks);
    return tp_launch_status(stream);
}

tp_status tp_decode_point(tp_plan_t p, int32_t point, int32_t rank, const void* x, const void* w,
                          float* slots, float* hidden, void* ws, void* stream) {
    if (!p || !x || !w || !slots || !hidden || !ws) return TP_ERR_INVALID_ARG;
    if (point != TP_POINT_ATTN_OUT && point != TP_POINT_FFN_DOWN) return TP_ERR_INVALID_ARG;
    if (rank < 0 || rank >= p->n_ranks) return TP_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(w) || !aligned16(slots) || !aligned16(hidden) || !aligned16(ws))
        return TP_ERR_ALIGNMENT;
    const int64_t b = p->batch, len = b * p->hidden, N = p->n_ranks;
    const PointGeom g = tp_point_geom(p, point);
    Epilogue e{};
    e.p = slots + rank * len;
    e.ws_part = ws_partials(ws);
    e.counters = ws_counters(ws);
    e.splits = g.splits;
    if (g.path == TP_PATH_MFMA && !mfma_spread(g, (int)b)) {
        // Measured: at b >= 16 the ring is faster as its own pass than in
        // the last-arriving split's epilogue (64 tokens, K_r = 2048, H = 4096:
        // 20 us against 40 us); with the fix-up spread over all splits the
        // epilogue carries it.
        tp_status s = launch_projection(p, g, (int)b, static_cast<const uint16_t*>(x),
                                        static_cast<const uint16_t*>(w), e, (hipStream_t)stream);
        if (s != TP_OK) return s;
        return tp_ring_reduce(p, slots, hidden, hidden, nullptr, stream);
    }
    e.ring_slots = slots;
    e.hidden = hidden;
    e.n_ranks = (int32_t)N;
    e.rank = rank;
    e.chunk = len / N;
    return launch_projection(p, g, (int)b, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w),
                             e, (hipStream_t)stream);
}

tp_status tp_decode_layers(tp_plan_t p, int32_t n_layers, int32_t rank, const void* x_attn,
                           const void* w_o, const void* x_ffn, const void* w_down, float* slots,
                           float* hidden, void* ws, void* stream) {
    if (!p || !x_attn || !w_o || !x_ffn || !w_down || !slots || !hidden || !ws)
        return TP_ERR_INVALID_ARG;
    if (n_layers < 0 || rank < 0 || rank >= p->n_ranks) return TP_ERR_INVALID_ARG;
    if (!aligned16(x_attn) || !aligned16(w_o) || !aligned16(x_ffn) || !aligned16(w_down) ||
        !aligned16(slots) || !aligned16(hidden) || !aligned16(ws))
        return TP_ERR_ALIGNMENT;
    const int64_t b = p->batch, H = p->hidden, N = p->n_ranks;
    const int64_t len = b * H;
    PointGeom geo[2] = {tp_point_geom(p, 0), tp_point_geom(p, 1)};
    // every slice of the stacked inputs must stay 16-byte aligned
    for (int pt = 0; pt < 2; ++pt)
        if ((b * geo[pt].k_r) % 8) return TP_ERR_ALIGNMENT;
    hipStream_t st = (hipStream_t)stream;
    if (tp_decode_mode(p) == 2)
        return decode_persistent(p, n_layers, rank, x_attn, w_o, x_ffn, w_down, slots, hidden,
                                 nullptr, ws, st);
    for (int32_t l = 0; l < n_layers; ++l) {
        for (int pt = 0; pt < 2; ++pt) {
            const PointGeom& g = geo[pt];
            const uint16_t* xb = static_cast<const uint16_t*>(pt == 0 ? x_attn : x_ffn);
            const uint16_t* wb = static_cast<const uint16_t*>(pt == 0 ? w_o : w_down);
            float* slot = slots + ((int64_t)l * 2 + pt) * N * len;
            Epilogue e{};
            e.p = slot + rank * len;
            e.ws_part = ws_partials(ws);
            e.counters = ws_counters(ws);
            e.splits = g.splits;
            e.ring_slots = slot;
            e.hidden = hidden;
            e.n_ranks = (int32_t)N;
            e.rank = rank;
            e.chunk = len / N;
            tp_status s = launch_projection(p, g, (int)b, xb + (int64_t)l * b * g.k_r,
                                            wb + (int64_t)l * g.k_r * H, e, st);
            if (s != TP_OK) return s;
        }
    }
    return TP_OK;
}

}  // extern "C"
