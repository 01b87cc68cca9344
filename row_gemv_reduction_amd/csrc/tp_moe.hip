// Expert-parallel MoE share of a decode step: routing, the down projection
// of this rank's experts and the local weighted combine.
//
// "Hosting Qwen on Blackwell" (sections Prefillers, MoE Dispatch-Combine and
// Expert Parallel): each token is sent to top_k of the experts; experts are
// spread over the expert-parallel ranks; a rank's combine first accumulates,
// per token, the contributions of the experts it holds, weighted by the
// routing weights, and the all-reduce over ranks then sums the ranks'
// partials (here: tp_ring_reduce). With 64 decode tokens, top-8 of 128
// experts and 32 experts per rank, almost every local expert is selected by
// a few tokens (4 on average), so the down projection is a grouped GEMV:
// every active expert's weights are streamed from HBM once and multiplied by
// the handful of activation rows routed to it.
//
// Kernels:
//   moe_route      one wave per token: softmax over the experts' logits (in
//                  double), top_k by logit with ties to the lower index,
//                  optional renormalisation, listed in ascending expert order.
//   moe_expert     one workgroup per (local expert, block of 8 16-column
//                  strips): the expert's rows are the (token, selection)
//                  pairs that chose it, found by scanning the selections in
//                  pair order (no table launch); up to 16 of them at a time
//                  are the A operand of v_mfma_f32_16x16x32_bf16 (each weight
//                  tile is read once per 16 rows; an expert has 4 rows on
//                  average), the waves split the expert's K rows, their D
//                  tiles are summed in LDS in wave order, and pair p's
//                  projection lands in Y[p]. A dot-product (vector ALU)
//                  version of the same GEMV spent more time in its
//                  multiply-adds than in streaming the weights; the matrix
//                  cores take them off the issue slots.
//   moe_combine    part[t, n] = sum over the token's selections s, in order
//                  (ascending expert), of weight * Y[t * top_k + s, n] for
//                  the local ones.
//
// Expert weights are packed once at load time as the matrix-core tiles of
// the dense decode step (one expert per matrix):
//     T[e][s][kb][h][l][i] = W_e[64kb + 16(l/16) + 8h + i][16s + l%16]
// (rows past I zero), so that one 16-byte load per lane and half hands each
// lane its B operand and a tile is 2 KB of contiguous memory.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tp_device.h"
#include "tp_internal.h"

namespace {

using namespace tpdev;


constexpr int kRouteMaxPerLane = 32;   // experts per lane in the routing wave (E <= 2048)

// ------------------------------------------------------------- routing --

// (value, index) arg-max over the wave: larger value wins, ties go to the
// lower index. Every lane ends with the same pair. The combine is
// associative and commutative, so any pairing of lane groups gives the same
// result: within rows of 16 lanes the partners come from DPP permutes
// (quads, then half-rows and rows mirrored), across rows from two shuffles.
template <int CTRL>
__device__ __forceinline__ void argmax_dpp(float& v, int& e) {
    const float ov = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
    const int oe = __builtin_amdgcn_update_dpp(0, e, CTRL, 0xF, 0xF, false);
    if (ov > v || (ov == v && oe < e)) { v = ov; e = oe; }
}
__device__ __forceinline__ void wave_argmax(float& v, int& e) {
    argmax_dpp<0xB1>(v, e);   // quad_perm 1,0,3,2
    argmax_dpp<0x4E>(v, e);   // quad_perm 2,3,0,1
    argmax_dpp<0x141>(v, e);  // row_half_mirror: quad 0 with quad 1 of each half-row
    argmax_dpp<0x140>(v, e);  // row_mirror: the two half-rows
#pragma unroll
    for (int m = 16; m < 64; m <<= 1) {
        const float ov = __shfl_xor(v, m);
        const int oe = __shfl_xor(e, m);
        if (ov > v || (ov == v && oe < e)) { v = ov; e = oe; }
    }
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m);
    return v;
}

template <int EPL>  // experts per lane (E <= 64 * EPL)
__global__ __launch_bounds__(256) void moe_route_kernel(const float* __restrict__ logits, int tokens,
                                                        int E, int top_k, int renorm,
                                                        int32_t* __restrict__ sel_expert,
                                                        float* __restrict__ sel_weight) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= tokens) return;
    const float* z = logits + (int64_t)t * E;
    float zl[EPL];
    uint32_t taken = 0;
    float zmax = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        zl[i] = e < E ? z[e] : -__builtin_inff();
        zmax = e < E && zl[i] > zmax ? zl[i] : zmax;
    }
    {
        int dummy = 0;
        wave_argmax(zmax, dummy);
    }
    // top_k rounds of arg-max over the experts not yet taken
    int my_e = 0x7fffffff;
    float my_z = 0.f;
    for (int r = 0; r < top_k; ++r) {
        float bv = -__builtin_inff();
        int be = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane + 64 * i;
            if (e < E && !(taken >> i & 1u) && (zl[i] > bv || be == 0x7fffffff)) {
                bv = zl[i];
                be = e;
            }
        }
        wave_argmax(bv, be);
        if ((be & 63) == lane) taken |= 1u << (be >> 6);
        if (lane == r) { my_e = be; my_z = bv; }
    }
    const bool mine = lane < top_k;
    const double p = mine ? exp((double)my_z - (double)zmax) : 0.0;
    double denom;
    if (renorm) {
        denom = wave_sum_f64(p);
    } else {
        // softmax denominator over all experts (double)
        double part = 0.0;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (lane + 64 * i < E) part += exp((double)zl[i] - (double)zmax);
        denom = wave_sum_f64(part);
    }
    // ascending expert order: the rank of my expert among the selected ones
    int rank = 0;
    for (int s = 0; s < top_k; ++s) {
        const int es = __shfl(my_e, s);
        rank += es < my_e;
    }
    if (mine) {
        sel_expert[(int64_t)t * top_k + rank] = my_e;
        sel_weight[(int64_t)t * top_k + rank] = (float)(p / denom);
    }
}

typedef void (*route_fn)(const float*, int, int, int, int, int32_t*, float*);
route_fn route_kernel(int E) {
    if (E <= 64) return moe_route_kernel<1>;
    if (E <= 128) return moe_route_kernel<2>;
    if (E <= 256) return moe_route_kernel<4>;
    if (E <= 512) return moe_route_kernel<8>;
    if (E <= 1024) return moe_route_kernel<16>;
    if (E <= 2048) return moe_route_kernel<32>;
    return nullptr;
}

// ------------------------------------------------------- expert GEMV --

struct ExpertArgs {
    const uint16_t* u;       // [T][k][I] bf16, row of pair p = t * k + s at u + p * I
    const uint16_t* w;       // tiles [EL][S16][nkb][2][64][8]
    const int32_t* sel;      // [T * k] selected expert of each pair
    float* y;                // [T * k][H] projection of each local pair's row
    int32_t n_pairs, e0;     // pairs; global id of local expert 0
    int32_t H, S16, I, nkb;
    int32_t col_blocks;      // ceil(S16 / SB)
};

constexpr int kMoeTileBytes = 2048;  // 64 rows x 16 columns of bf16

// One workgroup per (local expert, block of SB 16-column strips). The
// expert's rows are the pairs that selected it, in ascending pair order
// (found by scanning the selections: ranks from wave ballots); a pass takes
// up to 16 of them as the A operand (token m = lane % 16), and row p's
// projection lands in Y[p] (so the combine needs no table). Wave w takes the row tiles kb = w, w + NW,
// ... of the expert and, per tile, the block's SB strips in two register
// banks of SL = SB/2 tiles, loading each A operand once per 64 rows and the
// next tile's operands while it multiplies the current ones. The waves' D
// tiles are then summed in wave order in LDS. Strips past the block's last and rows past the expert's read
// zero (offsets past the buffer range); A operands of empty token slots and
// of rows past I are zero.
template <int SB, int NW>
__global__ __launch_bounds__(NW * 64) void moe_expert_kernel(ExpertArgs a) {
    constexpr int SL = SB / 2;
    constexpr int NT = NW * 64;
    __shared__ __align__(16) float red[NW * SB * 256];  // [NW][SB][64][4] D tiles
    __shared__ int rows[16];                            // the pass's pairs
    __shared__ int wcount[NW];
    __shared__ int s_rows;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int le = blockIdx.x / a.col_blocks, cb = blockIdx.x % a.col_blocks;
    const int eg = a.e0 + le;
    if (tid == 0) s_rows = 0;
    __syncthreads();
    {
        int c = 0;
        for (int p = tid; p < a.n_pairs; p += NT) c += a.sel[p] == eg;
        if (c) atomicAdd(&s_rows, c);
    }
    __syncthreads();
    const int n_rows = s_rows;
    if (n_rows == 0) return;  // expert not selected by any token: not read
    const int s0 = cb * SB;
    const int ns = a.S16 - s0 < SB ? a.S16 - s0 : SB;
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.w) + ((int64_t)le * a.S16 + s0) * a.nkb * (kMoeTileBytes / 2), (short)0,
        ns * a.nkb * kMoeTileBytes, kBufferRsrcWord3);
    const int past = ns * a.nkb * kMoeTileBytes;  // an offset past the range: reads zero
    const int nkw = a.nkb > wave ? (a.nkb - wave + NW - 1) / NW : 0;  // this wave's row tiles
    const int g16 = 16 * (lane >> 4);

    for (int r0 = 0; r0 < n_rows; r0 += 16) {
        const int nr = n_rows - r0 < 16 ? n_rows - r0 : 16;
        // the pass's rows: the expert's pairs of rank r0 .. r0 + 15
        if (r0 > 0) __syncthreads();  // the previous pass has read rows
        int base = 0;  // matches before the chunk
        for (int c0 = 0; c0 < a.n_pairs && base < r0 + 16; c0 += NT) {
            const int p = c0 + tid;
            const bool hit = p < a.n_pairs && a.sel[p] == eg;
            const uint64_t bal = __ballot(hit);
            if (lane == 0) wcount[wave] = __popcll(bal);
            __syncthreads();
            int rank = base + __popcll(bal & ((1ull << lane) - 1)), total = base;
            for (int w = 0; w < NW; ++w) {
                rank += w < wave ? wcount[w] : 0;
                total += wcount[w];
            }
            if (hit && rank >= r0 && rank < r0 + 16) rows[rank - r0] = p;
            __syncthreads();  // wcount is rewritten by the next chunk
            base = total;
        }
        const int m = lane & 15;
        const int pr = m < nr ? rows[m] : -1;
        const uint16_t* up = a.u + (int64_t)(pr < 0 ? 0 : pr) * a.I;
        // B operands of bank j (strips j*SL .. j*SL + SL - 1) of row tile kb (< 0: none)
        auto issue_w = [&](u32x4_t (&bv)[SL][2], int j, int kb) {
#pragma unroll
            for (int i = 0; i < SL; ++i) {
                const int s = j * SL + i;
                const int off = kb >= 0 && s < ns ? (s * a.nkb + kb) * kMoeTileBytes : past;
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    bv[i][h] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                               wr, off + h * 1024 + lane * 16, 0, kCachePolicyNT));
            }
        };
        // A operands of row tile kb: token m, rows 64kb + 16(lane/16) + 8h .. +7
        auto issue_x = [&](u32x4_t (&xv)[2], int kb) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int k0 = 64 * kb + g16 + 8 * h;
                xv[h] = kb >= 0 && pr >= 0 && k0 < a.I ? *reinterpret_cast<const u32x4_t*>(up + k0)
                                                       : u32x4_t{0u, 0u, 0u, 0u};
            }
        };
        floatx4_t acc[SB];
#pragma unroll
        for (int s = 0; s < SB; ++s) acc[s] = floatx4_t{0.f, 0.f, 0.f, 0.f};
        auto consume = [&](const u32x4_t (&bv)[SL][2], const u32x4_t (&xv)[2], int j) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < SL; ++i)
                    acc[j * SL + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, xv[h]), __builtin_bit_cast(bf16x8_t, bv[i][h]),
                        acc[j * SL + i], 0, 0, 0);
        };
        u32x4_t b0[SL][2], b1[SL][2], xa[2], xb[2];
        const int kb_first = nkw > 0 ? wave : -1;
        issue_x(xa, kb_first);
        issue_w(b0, 0, kb_first);
        issue_w(b1, 1, kb_first);
        // row tile n of this wave: its operands are in (xc, b0, b1); the next
        // tile's are loaded behind them into (xn, b0, b1)
        auto step = [&](u32x4_t (&xc)[2], u32x4_t (&xn)[2], int n) {
            const int kbn = n + 1 < nkw ? wave + (n + 1) * NW : -1;
            issue_x(xn, kbn);
            consume(b0, xc, 0);
            issue_w(b0, 0, kbn);
            consume(b1, xc, 1);
            issue_w(b1, 1, kbn);
        };
        int n = 0;
        for (; n + 1 < nkw; n += 2) {
            step(xa, xb, n);
            step(xb, xa, n + 1);
        }
        if (n < nkw) step(xa, xb, n);
        // the waves' D tiles (lane l: tokens 4(l/16) + q of column l % 16),
        // summed in wave order
        if (r0 > 0) __syncthreads();  // the previous pass has read red
#pragma unroll
        for (int s = 0; s < SB; ++s)
            *reinterpret_cast<floatx4_t*>(red + (wave * SB + s) * 256 + lane * 4) = acc[s];
        __syncthreads();
        for (int idx = tid; idx < ns * nr * 16; idx += NW * 64) {
            const int s = idx / (nr * 16), rem = idx - s * nr * 16;
            const int row = rem >> 4, col = rem & 15;
            const int e = (16 * (row >> 2) + col) * 4 + (row & 3);
            float v = red[s * 256 + e];
#pragma unroll
            for (int w = 1; w < NW; ++w) v += red[(w * SB + s) * 256 + e];
            a.y[(int64_t)rows[row] * a.H + 16 * (s0 + s) + col] = v;
        }
    }
}

// ------------------------------------------------------------ combine --

// Four columns per thread (H is a multiple of 16): each element sums the
// token's local selections in order, as one fused multiply-add each.
__device__ __forceinline__ floatx4_t combine4(const int32_t* __restrict__ sel_expert,
                                              const float* __restrict__ sel_weight,
                                              const float* __restrict__ y, int e0, int el, int t,
                                              int top_k, int H, int n) {
    floatx4_t acc = floatx4_t{0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < top_k; ++s) {
        const int q = t * top_k + s;
        const int le = sel_expert[q] - e0;
        if (le >= 0 && le < el) {
            const float w = sel_weight[q];
            const floatx4_t yv = *reinterpret_cast<const floatx4_t*>(y + (int64_t)q * H + n);
#pragma unroll
            for (int k = 0; k < 4; ++k) acc[k] = __builtin_fmaf(w, yv[k], acc[k]);
        }
    }
    return acc;
}

__global__ void moe_combine_kernel(const int32_t* __restrict__ sel_expert, const float* __restrict__ sel_weight,
                                   const float* __restrict__ y, int e0, int el, int tokens, int top_k, int H,
                                   float* __restrict__ part) {
    const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int H4 = H / 4;
    if (v >= (int64_t)tokens * H4) return;
    const int t = (int)(v / H4), n = 4 * (int)(v - (int64_t)t * H4);
    *reinterpret_cast<floatx4_t*>(part + (int64_t)t * H + n) =
        combine4(sel_expert, sel_weight, y, e0, el, t, top_k, H, n);
}

// The same combine, then the rank's partial to its slot and the ring-order
// sum of the N ranks' values of the point plus the residual (lesson 9.9
// "Interconnects e clusters", section 01 · Conceito). Four elements per
// thread: where they lie in one ring chunk (chunk a multiple of 4) the
// ranks' values come as 16-byte loads, all issued before the first add;
// otherwise element by element.
__global__ void moe_combine_ring_kernel(const int32_t* __restrict__ sel_expert,
                                        const float* __restrict__ sel_weight, const float* __restrict__ y,
                                        int e0, int el, int tokens, int top_k, int H,
                                        float* __restrict__ slots, float* hidden, int n_ranks, int rank,
                                        int64_t chunk) {
#pragma clang fp contract(off)
    const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t len = (int64_t)tokens * H;
    const int H4 = H / 4;
    if (v >= (int64_t)tokens * H4) return;
    const int t = (int)(v / H4), n = 4 * (int)(v - (int64_t)t * H4);
    const int64_t i = (int64_t)t * H + n;
    const floatx4_t acc = combine4(sel_expert, sel_weight, y, e0, el, t, top_k, H, n);
    *reinterpret_cast<floatx4_t*>(slots + (int64_t)rank * len + i) = acc;
    const floatx4_t res = *reinterpret_cast<const floatx4_t*>(hidden + i);
    floatx4_t out;
    if (chunk % 4 == 0) {
        const int c = (int)(i / chunk);
        floatx4_t sum = acc;
        for (int u0 = 0; u0 < n_ranks; u0 += 8) {
            floatx4_t x[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                int r = c + (u0 + u < n_ranks ? u0 + u : n_ranks - 1);
                r = r >= n_ranks ? r - n_ranks : r;
                x[u] = r == rank ? acc : *reinterpret_cast<const floatx4_t*>(slots + (int64_t)r * len + i);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (u0 + u < n_ranks) sum = u0 + u == 0 ? x[u] : sum + x[u];
        }
        out = sum + res;
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            out[k] = ring_element(slots, len, i + k, chunk, n_ranks, rank, acc[k], res[k]);
    }
    *reinterpret_cast<floatx4_t*>(hidden + i) = out;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

struct ExpertVariant {
    int sb, nw;
    void (*fn)(ExpertArgs);
};
// The plan knob "moe_variant" picks one (1-based; 0 = the first, the
// fastest measured at 128 experts of 1536 x 4096, 64 tokens, top-8, EP=4).
const ExpertVariant kExpertVariants[] = {
    {8, 4, moe_expert_kernel<8, 4>},
    {4, 4, moe_expert_kernel<4, 4>},
    {6, 4, moe_expert_kernel<6, 4>},
    {8, 8, moe_expert_kernel<8, 8>},
    {4, 8, moe_expert_kernel<4, 8>},
    {8, 2, moe_expert_kernel<8, 2>},
    {16, 4, moe_expert_kernel<16, 4>},
};

// Projections of the pairs' rows, [T * k][H] fp32, in the workspace.
float* moe_rows(const tp_plan_s* p, void* ws) {
    return reinterpret_cast<float*>(static_cast<char*>(ws) + tp_ws_moe_offset(p));
}

}  // namespace

int64_t tp_moe_workspace_bytes(const tp_plan_s* p) {
    if (!p->n_experts) return 0;
    const int64_t pairs = (int64_t)p->max_tokens * p->top_k;
    return pairs * p->hidden * 4;
}

extern "C" {

tp_status tp_moe_route(tp_plan_t p, const float* logits, int32_t tokens, int32_t renorm,
                       int32_t* sel_expert, float* sel_weight, void* stream) {
    if (!p || !logits || !sel_expert || !sel_weight) return TP_ERR_INVALID_ARG;
    if (!p->n_experts) return TP_ERR_INVALID_ARG;
    if (tokens < 0 || tokens > p->max_tokens) return TP_ERR_INVALID_ARG;
    if (!aligned16(logits) || !aligned16(sel_expert) || !aligned16(sel_weight)) return TP_ERR_ALIGNMENT;
    if (p->n_experts > 64 * kRouteMaxPerLane || p->top_k > 64) return TP_ERR_UNSUPPORTED;
    if (tokens == 0) return TP_OK;
    route_fn k = route_kernel((int)p->n_experts);
    if (!k) return TP_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(k, dim3((unsigned)((tokens + 3) / 4)), dim3(256), 0, (hipStream_t)stream, logits,
                       (int)tokens, (int)p->n_experts, (int)p->top_k, (int)(renorm != 0), sel_expert,
                       sel_weight);
    return hipGetLastError() == hipSuccess ? TP_OK : TP_ERR_DEVICE;
}

tp_status tp_moe_pack_experts(tp_plan_t p, const void* w_local, void* w_packed, void* stream) {
    if (!p || !w_local || !w_packed) return TP_ERR_INVALID_ARG;
    if (!p->n_experts) return TP_ERR_INVALID_ARG;
    if (!aligned16(w_local) || !aligned16(w_packed)) return TP_ERR_ALIGNMENT;
    if (w_local == w_packed) return TP_ERR_INVALID_ARG;
    if (p->hidden % 16) return TP_ERR_UNSUPPORTED;
    return tp_pack_tile_stack(p->n_experts / p->ep, p->moe_inter, p->hidden, w_local, w_packed, stream);
}

}  // extern "C"

namespace {

// The projections of the local pairs' rows (the grouped GEMV) for tokens
// 0 .. tokens-1, into moe_rows; the caller combines them.
tp_status moe_experts(const tp_plan_s* p, int32_t rank, const int32_t* sel_expert, int32_t tokens,
                      const void* u, const void* w_packed, void* ws, hipStream_t st) {
    const int64_t I = p->moe_inter, H = p->hidden, el = p->n_experts / p->ep;
    if (I % 8 || H % 16) return TP_ERR_UNSUPPORTED;
    const int64_t S16 = H / 16, nkb = (I + 63) / 64;
    const ExpertVariant v = kExpertVariants[p->moe_variant > 0 ? p->moe_variant - 1 : 0];
    if (S16 * nkb * kMoeTileBytes >= ((int64_t)1 << 31)) return TP_ERR_UNSUPPORTED;  // one expert's bytes
    if (tokens == 0) return TP_OK;
    ExpertArgs a;
    a.u = static_cast<const uint16_t*>(u);
    a.w = static_cast<const uint16_t*>(w_packed);
    a.sel = sel_expert;
    a.y = moe_rows(p, ws);
    a.n_pairs = tokens * p->top_k;
    a.e0 = (int32_t)(rank * el);
    a.H = (int32_t)H;
    a.S16 = (int32_t)S16;
    a.I = (int32_t)I;
    a.nkb = (int32_t)nkb;
    a.col_blocks = (int32_t)((S16 + v.sb - 1) / v.sb);
    const int64_t grid = el * a.col_blocks;
    hipLaunchKernelGGL(v.fn, dim3((unsigned)grid), dim3(v.nw * 64), 0, st, a);
    return hipGetLastError() == hipSuccess ? TP_OK : TP_ERR_DEVICE;
}

}  // namespace

extern "C" {

tp_status tp_moe_partial(tp_plan_t p, int32_t rank, const int32_t* sel_expert,
                         const float* sel_weight, int32_t tokens, const void* u,
                         const void* w_packed, float* part, void* ws, void* stream) {
    if (!p || !sel_expert || !sel_weight || !u || !w_packed || !part || !ws) return TP_ERR_INVALID_ARG;
    if (!p->n_experts) return TP_ERR_INVALID_ARG;
    if (rank < 0 || rank >= p->ep || tokens < 0 || tokens > p->max_tokens) return TP_ERR_INVALID_ARG;
    if (!aligned16(sel_expert) || !aligned16(sel_weight) || !aligned16(u) || !aligned16(w_packed) ||
        !aligned16(part) || !aligned16(ws))
        return TP_ERR_ALIGNMENT;
    hipStream_t st = (hipStream_t)stream;
    tp_status s = moe_experts(p, rank, sel_expert, tokens, u, w_packed, ws, st);
    if (s != TP_OK || tokens == 0) return s;
    const int64_t H = p->hidden, n_out = (int64_t)tokens * H, el = p->n_experts / p->ep;
    hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)((n_out / 4 + 255) / 256)), dim3(256), 0, st,
                       sel_expert, sel_weight, moe_rows(p, ws), (int)(rank * el), (int)el, (int)tokens,
                       (int)p->top_k, (int)H, part);
    return hipGetLastError() == hipSuccess ? TP_OK : TP_ERR_DEVICE;
}

tp_status tp_moe_decode(tp_plan_t p, int32_t rank, const int32_t* sel_expert, const float* sel_weight,
                        const void* u, const void* w_packed, float* slots, float* hidden, void* ws,
                        void* stream) {
    if (!p || !sel_expert || !sel_weight || !u || !w_packed || !slots || !hidden || !ws)
        return TP_ERR_INVALID_ARG;
    if (!p->n_experts) return TP_ERR_INVALID_ARG;
    // the ring spans the plan's N ranks; the experts are spread over ep of them
    if (p->ep != p->n_ranks || rank < 0 || rank >= p->ep || p->batch > p->max_tokens)
        return TP_ERR_INVALID_ARG;
    if (!aligned16(sel_expert) || !aligned16(sel_weight) || !aligned16(u) || !aligned16(w_packed) ||
        !aligned16(slots) || !aligned16(hidden) || !aligned16(ws))
        return TP_ERR_ALIGNMENT;
    hipStream_t st = (hipStream_t)stream;
    const int32_t tokens = p->batch;
    tp_status s = moe_experts(p, rank, sel_expert, tokens, u, w_packed, ws, st);
    if (s != TP_OK) return s;
    const int64_t H = p->hidden, len = (int64_t)tokens * H, el = p->n_experts / p->ep;
    hipLaunchKernelGGL(moe_combine_ring_kernel, dim3((unsigned)((len / 4 + 255) / 256)), dim3(256), 0, st,
                       sel_expert, sel_weight, moe_rows(p, ws), (int)(rank * el), (int)el, (int)tokens,
                       (int)p->top_k, (int)H, slots, hidden, (int)p->n_ranks, (int)rank, len / p->n_ranks);
    return hipGetLastError() == hipSuccess ? TP_OK : TP_ERR_DEVICE;
}

}  // extern "C"
