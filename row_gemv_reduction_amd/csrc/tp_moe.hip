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
//   moe_table      one workgroup: the local pairs (token, selection) grouped
//                  by local expert: counts, offsets and a slot per pair. The
//                  order of pairs inside an expert's group only decides which
//                  slot holds which row, never any arithmetic.
//   moe_expert     one workgroup per (local expert, block of 256 columns):
//                  the expert's rows are staged in LDS as bf16 pairs, each lane
//                  owns 4 columns and accumulates over its wave's share of
//                  the expert's K rows (no cross-lane reduction), the waves'
//                  K shares are summed in LDS in wave order, and the rows'
//                  projections land in Y[slot].
//   moe_combine    part[t, n] = sum over the token's selections s, in order
//                  (ascending expert), of weight * Y[slot(t, s), n] for the
//                  local ones.
//
// Expert weights are packed once at load time ("pair rows"):
//     P[e][kp][g][c][q] = W_e[2kp + q][4g + c]     kp < ceil(I/2), g < H/4
// so a wave streams one row pair across 256 columns per 1 KB load.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tp_device.h"
#include "tp_internal.h"

namespace {

using namespace tpdev;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kRouteMaxPerLane = 32;   // experts per lane in the routing wave (E <= 2048)
constexpr int kMoeCols = 256;          // columns per expert workgroup: 64 lanes x 4

// ------------------------------------------------------------- routing --

// (value, index) arg-max over the wave: larger value wins, ties go to the
// lower index. Every lane ends with the same pair.
__device__ __forceinline__ void wave_argmax(float& v, int& e) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
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

// ---------------------------------------------------------- pair table --

struct MoeTable {
    int32_t* off;       // [EL + 1] start of each local expert's slots
    int32_t* slot;      // [T * k] slot of each pair, -1 if its expert is not local
    int32_t* pair;      // [T * k] pair id (t * k + s) of each slot
    float* y;           // [T * k][H] projection of each slot's row
};

__global__ __launch_bounds__(1024) void moe_table_kernel(const int32_t* __restrict__ sel_expert,
                                                         int n_pairs, int e0, int EL, MoeTable tb) {
    extern __shared__ int32_t cnt[];  // [EL] counts, then [EL] cursors
    int32_t* cur = cnt + EL;
    for (int e = threadIdx.x; e < EL; e += blockDim.x) cnt[e] = 0;
    __syncthreads();
    for (int p = threadIdx.x; p < n_pairs; p += blockDim.x) {
        const int le = sel_expert[p] - e0;
        if (le >= 0 && le < EL) atomicAdd(&cnt[le], 1);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int run = 0;
        for (int e = 0; e < EL; ++e) {
            tb.off[e] = run;
            cur[e] = run;
            run += cnt[e];
        }
        tb.off[EL] = run;
    }
    __syncthreads();
    for (int p = threadIdx.x; p < n_pairs; p += blockDim.x) {
        const int ex = sel_expert[p];
        const int le = ex - e0;
        int s = -1;
        if (le >= 0 && le < EL) {
            s = atomicAdd(&cur[le], 1);
            tb.pair[s] = p;
        }
        tb.slot[p] = s;  // ids of other ranks' experts (or invalid ids) are skipped
    }
}

// ------------------------------------------------------- expert GEMV --

struct ExpertArgs {
    const uint16_t* u;       // [T][k][I] bf16, row of pair p at u + p * I
    const uint16_t* w;       // packed [EL][Kh][H/4][8]
    MoeTable tb;
    int32_t H, G4, I, Kh;    // G4 = H / 4 column groups
    int32_t rows_per_wave;   // row pairs per wave (multiple of 2 * kMoeSL)
    int32_t col_blocks;      // ceil(G4 / 64)
};

// MT activation rows per pass (more rows: more passes over the weights),
// NW waves per workgroup (the K split), SL loads per lane per register bank.
template <int MT, int NW, int SL>
__global__ __launch_bounds__(NW * 64) void moe_expert_kernel(ExpertArgs a) {
    constexpr int kMoeWaves = NW;
    constexpr int kMoeSL = SL;
    // x rows of the pass as bf16 pairs [MT][Kh]; reused afterwards for the
    // waves' column sums [kMoeWaves][MT][kMoeCols]
    extern __shared__ __align__(16) uint32_t sh[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int le = blockIdx.x / a.col_blocks, cb = blockIdx.x % a.col_blocks;
    const int q0 = a.tb.off[le], n_rows = a.tb.off[le + 1] - q0;
    if (n_rows == 0) return;  // expert not selected by any token: not read
    const int g = cb * 64 + lane;  // this lane's column group
    const int kp0 = wave * a.rows_per_wave;
    const int64_t slab = (int64_t)a.Kh * a.G4 * 16;  // bytes of one expert
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.w) + (int64_t)le * a.Kh * a.G4 * 8, (short)0, (int)slab,
        kBufferRsrcWord3);
    // lanes past the last column group read the next row's columns (or
    // zeros at the end of the slab); their sums are never stored
    const int voff = (kp0 * a.G4 + g) * 16;
    const int rstride = a.G4 * 16;
    float* red = reinterpret_cast<float*>(sh);

    for (int r0 = 0; r0 < n_rows; r0 += MT) {
        const int nr = n_rows - r0 < MT ? n_rows - r0 : MT;
        __syncthreads();  // the previous pass is done with the LDS
        // stage the pass's rows: [row][kp] dwords, 16 bytes per thread step
        for (int v = tid; v < nr * (a.I / 8); v += kMoeWaves * 64) {
            const int row = v / (a.I / 8), c = v - row * (a.I / 8);
            const int p = a.tb.pair[q0 + r0 + row];
            const u32x4_t val = *reinterpret_cast<const u32x4_t*>(a.u + (int64_t)p * a.I + c * 8);
            *reinterpret_cast<u32x4_t*>(sh + row * a.Kh + c * 4) = val;
        }
        __syncthreads();

        float acc[MT][4];
#pragma unroll
        for (int r = 0; r < MT; ++r)
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[r][c] = 0.f;
        u32x4_t bank0[kMoeSL], bank1[kMoeSL];
        auto issue = [&](u32x4_t (&bank)[kMoeSL], int k) {
#pragma unroll
            for (int i = 0; i < kMoeSL; ++i)
                bank[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                          rs, voff + (k + i) * rstride, 0, kCachePolicyNT));
        };
        // row pairs past Kh read zero weights; their x index is clamped to the
        // last staged pair, so the product is zero (x is finite)
        auto consume = [&](const u32x4_t (&bank)[kMoeSL], int k) {
#pragma unroll
            for (int i = 0; i < kMoeSL; ++i) {
                const u32x4_t wq = bank[i];
                const uint32_t wd[4] = {wq.x, wq.y, wq.z, wq.w};
                int kp = kp0 + k + i;
                kp = kp < a.Kh ? kp : a.Kh - 1;
#pragma unroll
                for (int r = 0; r < MT; ++r) {
                    if (r < nr) {
                        const bf16x2_t xv = __builtin_bit_cast(bf16x2_t, sh[r * a.Kh + kp]);
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            acc[r][c] = __builtin_amdgcn_fdot2_f32_bf16(
                                __builtin_bit_cast(bf16x2_t, wd[c]), xv, acc[r][c], false);
                    }
                }
            }
        };
        const int n = a.rows_per_wave;  // multiple of 2 * kMoeSL
        issue(bank0, 0);
        issue(bank1, kMoeSL);
        for (int k = 0; k < n; k += 2 * kMoeSL) {
            consume(bank0, k);
            issue(bank0, k + 2 * kMoeSL < n ? k + 2 * kMoeSL : a.Kh);
            consume(bank1, k + kMoeSL);
            issue(bank1, k + 3 * kMoeSL < n ? k + 3 * kMoeSL : a.Kh);
        }
        __syncthreads();  // every wave is done reading x: reuse the LDS
#pragma unroll
        for (int r = 0; r < MT; ++r)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                red[(wave * MT + r) * kMoeCols + lane * 4 + c] = acc[r][c];
        __syncthreads();
        // sum the waves' K shares in wave order; store the pass's rows
        for (int idx = tid; idx < nr * kMoeCols; idx += kMoeWaves * 64) {
            const int r = idx / kMoeCols, col = idx - r * kMoeCols;
            const int n_col = cb * kMoeCols + col;
            if (n_col >= a.H) continue;
            float v = red[r * kMoeCols + col];
#pragma unroll
            for (int w = 1; w < kMoeWaves; ++w) v += red[(w * MT + r) * kMoeCols + col];
            a.tb.y[(int64_t)(q0 + r0 + r) * a.H + n_col] = v;
        }
    }
}

// ------------------------------------------------------------ combine --

__global__ void moe_combine_kernel(const float* __restrict__ sel_weight, MoeTable tb, int tokens,
                                   int top_k, int H, float* __restrict__ part) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)tokens * H) return;
    const int t = (int)(i / H), n = (int)(i - (int64_t)t * H);
    float acc = 0.f;
    for (int s = 0; s < top_k; ++s) {
        const int q = tb.slot[t * top_k + s];
        if (q >= 0) acc = __builtin_fmaf(sel_weight[t * top_k + s], tb.y[(int64_t)q * H + n], acc);
    }
    part[i] = acc;
}

// The same combine, then the rank's partial to its slot and the ring-order
// sum of the N ranks' values of the point plus the residual (lesson 9.9
// "Interconnects e clusters", section 01 · Conceito), one element per thread.
__global__ void moe_combine_ring_kernel(const float* __restrict__ sel_weight, MoeTable tb, int tokens,
                                        int top_k, int H, float* __restrict__ slots, float* hidden,
                                        int n_ranks, int rank, int64_t chunk) {
#pragma clang fp contract(off)
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t len = (int64_t)tokens * H;
    if (i >= len) return;
    const int t = (int)(i / H), n = (int)(i - (int64_t)t * H);
    float acc = 0.f;
    for (int s = 0; s < top_k; ++s) {
        const int q = tb.slot[t * top_k + s];
        if (q >= 0) acc = __builtin_fmaf(sel_weight[t * top_k + s], tb.y[(int64_t)q * H + n], acc);
    }
    slots[(int64_t)rank * len + i] = acc;
    hidden[i] = ring_element(slots, len, i, chunk, n_ranks, rank, acc, hidden[i]);
}

// ------------------------------------------------------------- packing --

// P[e][kp][g][c][q] = W[e][2kp+q][4g+c]: one 16-byte output vector per thread.
__global__ void pack_experts_kernel(const uint16_t* __restrict__ w, uint16_t* __restrict__ p,
                                    int64_t experts, int64_t I, int64_t H) {
    const int64_t g4 = H / 4, kh = (I + 1) / 2;
    const int64_t total = experts * kh * g4;
    for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < total;
         v += (int64_t)gridDim.x * blockDim.x) {
        const int64_t e = v / (kh * g4);
        const int64_t rem = v - e * kh * g4;
        const int64_t kp = rem / g4, gg = rem - kp * g4;
        const uint16_t* r0 = w + (e * I + 2 * kp) * H + 4 * gg;
        uint16_t lo[4], hi[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            lo[c] = r0[c];
            hi[c] = 2 * kp + 1 < I ? r0[H + c] : (uint16_t)0;
        }
        u32x4_t out;
        out.x = lo[0] | ((uint32_t)hi[0] << 16);
        out.y = lo[1] | ((uint32_t)hi[1] << 16);
        out.z = lo[2] | ((uint32_t)hi[2] << 16);
        out.w = lo[3] | ((uint32_t)hi[3] << 16);
        *reinterpret_cast<u32x4_t*>(p + v * 8) = out;
    }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

struct ExpertVariant {
    int mt, nw, sl;
    void (*fn)(ExpertArgs);
};
// The plan knob "moe_variant" picks one (1-based; 0 = the first, the
// fastest measured at 128 experts of 1536 x 4096, 64 tokens, top-8, EP=4).
const ExpertVariant kExpertVariants[] = {
    {8, 8, 4, moe_expert_kernel<8, 8, 4>},
    {8, 4, 4, moe_expert_kernel<8, 4, 4>},
    {8, 4, 8, moe_expert_kernel<8, 4, 8>},
    {4, 4, 8, moe_expert_kernel<4, 4, 8>},
    {4, 8, 8, moe_expert_kernel<4, 8, 8>},
    {8, 16, 4, moe_expert_kernel<8, 16, 4>},
    {8, 16, 2, moe_expert_kernel<8, 16, 2>},
};

MoeTable table_in(const tp_plan_s* p, void* ws) {
    const int64_t pairs = (int64_t)p->max_tokens * p->top_k;
    const int64_t el = p->n_experts / p->ep;
    char* base = static_cast<char*>(ws) + tp_ws_moe_offset(p);
    MoeTable t;
    t.off = reinterpret_cast<int32_t*>(base);
    base += (el + 1 + 63) / 64 * 256;
    t.slot = reinterpret_cast<int32_t*>(base);
    base += (pairs + 63) / 64 * 256;
    t.pair = reinterpret_cast<int32_t*>(base);
    base += (pairs + 63) / 64 * 256;
    t.y = reinterpret_cast<float*>(base);
    return t;
}

}  // namespace

int64_t tp_moe_workspace_bytes(const tp_plan_s* p) {
    if (!p->n_experts) return 0;
    const int64_t pairs = (int64_t)p->max_tokens * p->top_k;
    const int64_t el = p->n_experts / p->ep;
    return (el + 1 + 63) / 64 * 256 + 2 * ((pairs + 63) / 64 * 256) + pairs * p->hidden * 4;
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
    const int64_t el = p->n_experts / p->ep;
    const int64_t total = el * ((p->moe_inter + 1) / 2) * (p->hidden / 4);
    const int64_t blocks = (total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536;
    hipLaunchKernelGGL(pack_experts_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       static_cast<const uint16_t*>(w_local), static_cast<uint16_t*>(w_packed), el,
                       p->moe_inter, p->hidden);
    return hipGetLastError() == hipSuccess ? TP_OK : TP_ERR_DEVICE;
}

}  // extern "C"

namespace {

// The rank's expert rows y (pair table, then the grouped GEMV) for tokens
// 0 .. tokens-1; the caller combines them.
tp_status moe_experts(const tp_plan_s* p, int32_t rank, const int32_t* sel_expert, int32_t tokens,
                      const void* u, const void* w_packed, void* ws, hipStream_t st, MoeTable* tb_out) {
    const int64_t I = p->moe_inter, H = p->hidden, el = p->n_experts / p->ep;
    if (I % 8) return TP_ERR_UNSUPPORTED;
    const int64_t kh = I / 2;
    const ExpertVariant v = kExpertVariants[p->moe_variant > 0 ? p->moe_variant - 1 : 0];
    // LDS: the pass's rows (MT x I bf16) and the waves' sums
    const int64_t lds_x = (int64_t)v.mt * kh * 4;
    const int64_t lds_red = (int64_t)v.nw * v.mt * kMoeCols * 4;
    const int64_t lds = lds_x > lds_red ? lds_x : lds_red;
    if (lds > 150 * 1024 || el * 8 > 64 * 1024) return TP_ERR_UNSUPPORTED;
    if (kh * (H / 4) * 16 >= ((int64_t)1 << 31)) return TP_ERR_UNSUPPORTED;  // one expert's bytes
    MoeTable tb = table_in(p, ws);
    *tb_out = tb;
    if (tokens == 0) return TP_OK;
    const int n_pairs = tokens * p->top_k;
    hipLaunchKernelGGL(moe_table_kernel, dim3(1), dim3(1024), (unsigned)(el * 8), st, sel_expert,
                       n_pairs, (int)(rank * el), (int)el, tb);
    if (hipGetLastError() != hipSuccess) return TP_ERR_DEVICE;
    ExpertArgs a;
    a.u = static_cast<const uint16_t*>(u);
    a.w = static_cast<const uint16_t*>(w_packed);
    a.tb = tb;
    a.H = (int32_t)H;
    a.G4 = (int32_t)(H / 4);
    a.I = (int32_t)I;
    a.Kh = (int32_t)kh;
    const int64_t per_wave = (kh + v.nw - 1) / v.nw;
    a.rows_per_wave = (int32_t)((per_wave + 2 * v.sl - 1) / (2 * v.sl) * (2 * v.sl));
    a.col_blocks = (int32_t)((H / 4 + 63) / 64);
    const int64_t grid = el * a.col_blocks;
    if (lds > 64 * 1024 && hipFuncSetAttribute(reinterpret_cast<const void*>(v.fn),
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)lds) != hipSuccess)
        return TP_ERR_DEVICE;
    hipLaunchKernelGGL(v.fn, dim3((unsigned)grid), dim3(v.nw * 64), (unsigned)lds, st, a);
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
    MoeTable tb;
    tp_status s = moe_experts(p, rank, sel_expert, tokens, u, w_packed, ws, st, &tb);
    if (s != TP_OK || tokens == 0) return s;
    const int64_t H = p->hidden, n_out = (int64_t)tokens * H;
    hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)((n_out + 255) / 256)), dim3(256), 0, st,
                       sel_weight, tb, (int)tokens, (int)p->top_k, (int)H, part);
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
    MoeTable tb;
    const int32_t tokens = p->batch;
    tp_status s = moe_experts(p, rank, sel_expert, tokens, u, w_packed, ws, st, &tb);
    if (s != TP_OK) return s;
    const int64_t H = p->hidden, len = (int64_t)tokens * H;
    hipLaunchKernelGGL(moe_combine_ring_kernel, dim3((unsigned)((len + 255) / 256)), dim3(256), 0, st,
                       sel_weight, tb, (int)tokens, (int)p->top_k, (int)H, slots, hidden,
                       (int)p->n_ranks, (int)rank, len / p->n_ranks);
    return hipGetLastError() == hipSuccess ? TP_OK : TP_ERR_DEVICE;
}

}  // extern "C"
