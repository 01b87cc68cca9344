// Column-strip weight layout and the decode step that streams it.
//
// The decode projections are weight-streaming bound ("Hosting Qwen on
// Blackwell", section Decoders); the reconciliation after each one is a
// short serial dependency (lesson 9.9 "Interconnects e clusters", section
// 01 · Conceito: every point is a blocking round trip). Row-major W[K][H]
// forces a split of K over workgroups, and the split partials then have to
// meet in memory (publish, count arrivals, gather) on that serial path. The
// strip layout removes that exchange: the rank's slice W_r[K][H] is stored
// once, at load time, as
//
//     P[s][k][c] = W_r[k][8s + c]      s < H/8, k < K, c < 8
//
// (same bytes, 16 contiguous bytes per row of a strip), so one workgroup
// streams a whole strip of 8 columns over all K rows as contiguous 1 KB
// wave loads and reduces over K inside the workgroup: lanes by a shuffle
// butterfly, waves through LDS. No partial leaves the workgroup.
//
// decode_strips: one cooperative (persistent) launch per decode step. Each
// workgroup owns strips g, g+G, ... for every point of the step and runs
//   - NW compute waves: hold the weights of the current task in registers,
//     multiply them by x (staged in LDS), reduce, and issue the loads of
//     their next task right away, so those are in flight while the current
//     point is reduced and the next point is waited for;
//   - one control wave: waits for the previous point, stages x, forms the
//     ring-order sum of the N ranks' values plus the residual for its strip
//     (the strip's hidden state stays in LDS between points), stores it
//     device-coherently and signals completion. Its memory counter never
//     waits behind the bulk weight loads.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tp_device.h"
#include "tp_internal.h"

namespace {

using namespace tpdev;

// ------------------------------------------------------------- packing --

// P[l][s][k][0..8) = W[l][k][8s .. 8s+8): one 16-byte vector per thread.
__global__ void pack_strips_kernel(const uint16_t* __restrict__ w, uint16_t* __restrict__ p,
                                   int64_t layers, int64_t K, int64_t H) {
    const int64_t strips = H / 8;
    const int64_t per_layer = K * strips;
    const int64_t total = layers * per_layer;
    for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < total;
         v += (int64_t)gridDim.x * blockDim.x) {
        const int64_t l = v / per_layer;
        const int64_t rem = v - l * per_layer;
        const int64_t k = rem / strips;
        const int64_t s = rem - k * strips;
        const u32x4_t val = *reinterpret_cast<const u32x4_t*>(w + (l * K + k) * H + s * 8);
        *reinterpret_cast<u32x4_t*>(p + ((l * strips + s) * K + k) * 8) = val;
    }
}

// ------------------------------------------------------- decode step --

// Per-point fields are separate scalars (not arrays indexed by the point),
// so the compiler keeps them, and the buffer descriptors built from them,
// in scalar registers.
struct StripArgs {
    const uint16_t* x0;     // x_attn [L][B][K0]
    const uint16_t* x1;     // x_ffn  [L][B][K1]
    const uint16_t* w0;     // strip-packed w_o    [L][H/8][K0][8]
    const uint16_t* w1;     // strip-packed w_down [L][H/8][K1][8]
    float* slots;           // [L][2][N][B][H]
    float* hidden;          // [B][H]
    uint32_t* sync;         // done / exit / error words
    int32_t H, K0, K1;
    int32_t strips, layers, n_ranks, rank;
    int32_t chunk;
    uint32_t spin_limit;
    int32_t xs_bytes;       // dynamic LDS for x: rows padded to NW * 64, * B * 2
};

// An opaque 0 that the compiler can only produce after every accumulator
// value is final (inline asm consuming them, 8 at a time). Loads whose
// offsets take it cannot be hoisted above the multiplies.
template <int B>
__device__ __forceinline__ int after_all(const float (&acc)[B][8]) {
    int z = 0;
#pragma unroll
    for (int bb = 0; bb < B; ++bb)
        asm volatile("; wait for %1..%8\n\tv_mov_b32 %0, 0"
                     : "=v"(z)
                     : "v"(acc[bb][0]), "v"(acc[bb][1]), "v"(acc[bb][2]), "v"(acc[bb][3]),
                       "v"(acc[bb][4]), "v"(acc[bb][5]), "v"(acc[bb][6]), "v"(acc[bb][7]), "0"(z));
    return z;
}

// Grid-wide "point complete" signal as a two-level tree. A single counter
// that every workgroup increments and polls serialises hundreds of atomics
// and loads on one address (microseconds per point). Here workgroup g
// arrives on group counter g % M; the last arrival of a group arrives on the
// top counter; the last group's arrival writes every group's release word;
// workgroups wait on their own group's release word. Counters only grow
// during a launch (point j is complete when a counter reaches (j+1) x its
// arrivals per point); the last workgroup to leave resets them.
struct TreeBarrier {
    uint32_t* sync;
    int groups;  // active groups: min(kTreeGroups, grid)
    __device__ uint32_t* group_ctr(int q) const { return sync + kTreeGroupBase + q * kTreeLine; }
    __device__ uint32_t* release(int q) const { return sync + kTreeReleaseBase + q * kTreeLine; }
    __device__ uint32_t* top() const { return sync + kTreeTop; }
};

// Control wave of workgroup g: point j's strips of this workgroup are done.
__device__ __forceinline__ void tree_arrive(const TreeBarrier& tb, int g, int G, int j, int lane) {
    const int q = g % tb.groups;
    const uint32_t members = (uint32_t)((G - 1 - q) / tb.groups + 1);
    int last = 0;
    if (lane == 0) {
        const uint32_t old = add_dev_u32(tb.group_ctr(q), 1u);
        if (old + 1 == members * (uint32_t)(j + 1)) {
            const uint32_t t = add_dev_u32(tb.top(), 1u);
            last = t + 1 == (uint32_t)tb.groups * (uint32_t)(j + 1);
        }
    }
    if (__builtin_amdgcn_readfirstlane(last)) {
        for (int r = lane; r < tb.groups; r += 64) st_dev_u32(tb.release(r), (uint32_t)(j + 1));
    }
}

// Lane 0: wait until point j-1 is complete (release word of my group >= j).
__device__ __forceinline__ bool tree_wait(const TreeBarrier& tb, int g, int j, uint32_t* err,
                                          uint32_t limit) {
    return wait_at_least(tb.release(g % tb.groups), (uint32_t)j, err, limit);
}

template <int B, int NW, int NI>
__global__ __launch_bounds__((NW + 1) * 64) void decode_strips(StripArgs a) {
    extern __shared__ __align__(16) uint16_t xs[];    // x of the current point, [rows][B] bf16
    __shared__ float red[NW * B * 8];
    __shared__ float h_strip[kStripMaxPerWg * B * 8]; // this workgroup's strips of the hidden state
    __shared__ int flag;

    // The wave index and everything derived from the task index are
    // wave-uniform; readfirstlane tells the compiler, which then keeps them
    // in scalar registers.
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    uint32_t* err = a.sync + kSyncErr;
    const int len = B * a.H;
    const int G = gridDim.x;
    TreeBarrier tb;
    tb.sync = a.sync;
    tb.groups = G < kTreeGroups ? G : kTreeGroups;
    const int my_strips = (a.strips - (int)blockIdx.x + G - 1) / G;
    // task t of this workgroup: point j = t / my_strips, strip s = g + (t % my_strips) * G
    // (all task, row and element indices fit in 32 bits; the host checks)
    const int n_tasks = a.layers * 2 * my_strips;
    auto task_point = [&](int t) { return t / my_strips; };
    auto task_strip = [&](int t) { return (int)blockIdx.x + (t % my_strips) * G; };
    auto task_k = [&](int t) { return (task_point(t) & 1) ? a.K1 : a.K0; };

    // Per task: barrier A (x of the point staged, or the wait failed), then
    // barrier B (the compute waves' sums are in LDS). The two roles run
    // separate loops with the same barriers, so neither role's registers
    // are live in the other's code.
    if (wave == 0) {
        // ---------------------------------------------------- control wave
        // Its few memory operations (wait, x, signal) are the serial path of
        // the step: give them issue priority over the compute waves' bulk
        // weight loads in this CU.
        __builtin_amdgcn_s_setprio(3);
        for (int e = lane; e < my_strips * B * 8; e += 64) {
            const int k = e / (B * 8), bb = (e / 8) % B, c = e % 8;
            const int64_t s = blockIdx.x + (int64_t)k * G;
            h_strip[e] = a.hidden[(int64_t)bb * a.H + s * 8 + c];
        }
        // the other ranks' values of the task, loaded ahead, in ring order
        float others[8];
        auto fetch_others = [&](int t) {
            if (lane >= B * 8) return;
            const int j = task_point(t), s = task_strip(t);
            const int i = (lane / 8) * a.H + s * 8 + (lane % 8);
            const float* slot = a.slots + (int64_t)j * a.n_ranks * len;
            const int c = i / a.chunk;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                int r = c + u;
                if (r >= a.n_ranks) r -= a.n_ranks;
                others[u] = (u < a.n_ranks && r != a.rank) ? slot[(int64_t)r * len + i] : 0.f;
            }
        };
        if (n_tasks > 0) fetch_others(0);
        for (int t = 0; t < n_tasks; ++t) {
            const int j = task_point(t), s = task_strip(t), K = task_k(t);
            // point j reads its activation only after point j-1 is complete
            int ok = 1;
            if (lane == 0 && t % my_strips == 0) ok = tree_wait(tb, blockIdx.x, j, err, a.spin_limit);
            ok = __builtin_amdgcn_readfirstlane(ok);
            if (ok) {
                // stage x_j as [rows][B] bf16; rows past K (up to the padded
                // row count the compute lanes walk) are zero, so the multiply
                // loop needs no per-row test (the weights there read as zero)
                const uint16_t* x = ((j & 1) ? a.x1 : a.x0) + (int64_t)(j >> 1) * B * K;
                const int rows = (K + NW * 64 - 1) / (NW * 64) * (NW * 64);
                if (B == 1) {
                    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x);
                    u32x4_t* dst = reinterpret_cast<u32x4_t*>(xs);
                    for (int v = lane; v < rows / 8; v += 64)
                        dst[v] = v < K / 8 ? src[v] : u32x4_t{0u, 0u, 0u, 0u};
                } else {
                    for (int e = lane; e < K * B; e += 64) {
                        const int bb = e / K, r = e - bb * K;
                        xs[r * B + bb] = x[e];
                    }
                    for (int e = K * B + lane; e < rows * B; e += 64) xs[e] = 0;
                }
            }
            if (lane == 0) flag = ok;
            __syncthreads();  // A
            if (!ok) break;
            __syncthreads();  // B
            if (lane < B * 8) {
#pragma clang fp contract(off)
                float v = red[lane];
#pragma unroll
                for (int w = 1; w < NW; ++w) v += red[w * B * 8 + lane];
                const int i = (lane / 8) * a.H + s * 8 + (lane % 8);
                float* slot = a.slots + (int64_t)j * a.n_ranks * len;
                slot[(int64_t)a.rank * len + i] = v;
                // ring order: chunk c starts at rank c, then c+1, ... (mod N)
                const int c = i / a.chunk;
                float sum = 0.f;
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    if (u < a.n_ranks) {
                        int r = c + u;
                        if (r >= a.n_ranks) r -= a.n_ranks;
                        const float val = r == a.rank ? v : others[u];
                        sum = u == 0 ? val : sum + val;
                    }
                }
                float* hs = h_strip + (t % my_strips) * B * 8 + lane;
                const float h = sum + *hs;
                *hs = h;
                // The strip's hidden state lives in this workgroup's LDS for
                // the whole step (no other workgroup reads it), so the store
                // is for the caller only and the strip can count as done now.
                a.hidden[i] = h;
            }
            // this workgroup's strips of point j are done after its last one
            if (t % my_strips == my_strips - 1) tree_arrive(tb, blockIdx.x, G, j, lane);
            if (t + 1 < n_tasks) fetch_others(t + 1);
        }
    } else {
        // --------------------------------------------------- compute waves
        const int cw = wave - 1;
        // Weight loads go through a buffer descriptor per task: one lane
        // offset VGPR, a uniform scalar offset per load, and the hardware
        // range check returns zeros past the strip's K rows.
        u32x4_t wv[NI];
        const int lane_off = (cw * 64 + lane) * 16;
        auto issue = [&](int t, int dep) {
            const int j = task_point(t), s = task_strip(t), K = task_k(t);
            const uint16_t* base = ((j & 1) ? a.w1 : a.w0) + ((int64_t)(j >> 1) * a.strips + s) * K * 8;
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint16_t*>(base), (short)0, K * 16, kBufferRsrcWord3);
            const int ni_used = (K + NW * 64 - 1) / (NW * 64);  // wave-uniform
#pragma unroll
            for (int i = 0; i < NI; ++i)
                if (i < ni_used)
                    wv[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                            rs, lane_off + dep, i * NW * 1024, kCachePolicyNT));
        };
        if (n_tasks > 0) issue(0, 0);
        for (int t = 0; t < n_tasks; ++t) {
            const int K = task_k(t);
            __syncthreads();  // A
            if (!__builtin_amdgcn_readfirstlane(flag)) break;
            float acc[B][8];
#pragma unroll
            for (int bb = 0; bb < B; ++bb)
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[bb][c] = 0.f;
            const uint16_t* xr = xs + (cw * 64 + lane) * B;
            const int ni_used = (K + NW * 64 - 1) / (NW * 64);  // wave-uniform
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                if (i < ni_used) {
                    const u32x4_t wq = wv[i];
                    const float wf[8] = {bf16_lo(wq.x), bf16_hi(wq.x), bf16_lo(wq.y), bf16_hi(wq.y),
                                         bf16_lo(wq.z), bf16_hi(wq.z), bf16_lo(wq.w), bf16_hi(wq.w)};
#pragma unroll
                    for (int bb = 0; bb < B; ++bb) {
                        const float xv = bf16_to_f32(xr[i * NW * 64 * B + bb]);
#pragma unroll
                        for (int c = 0; c < 8; ++c) acc[bb][c] = __builtin_fmaf(xv, wf[c], acc[bb][c]);
                    }
                }
            }
            // loads that take this opaque zero cannot move above the multiplies
            const int dep = after_all(acc);
            // sum over the wave's 64 rows
#pragma unroll
            for (int bb = 0; bb < B; ++bb)
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[bb][c] = wave_sum(acc[bb][c]);
            if (lane < B * 8) {
                float v = 0.f;
#pragma unroll
                for (int bb = 0; bb < B; ++bb)
#pragma unroll
                    for (int c = 0; c < 8; ++c)
                        if (lane == bb * 8 + c) v = acc[bb][c];
                red[cw * B * 8 + lane] = v;
            }
            __syncthreads();  // B
            // the registers are free: start the next task's weights
            if (t + 1 < n_tasks) issue(t + 1, dep);
        }
    }
    // The last workgroup to leave resets the step's sync words for the next
    // launch (no workgroup reads them any more).
    __syncthreads();
    if (wave == 0) {
        int last = 0;
        if (lane == 0) last = add_dev_u32(a.sync + kSyncExit, 1u) == gridDim.x - 1;
        if (__builtin_amdgcn_readfirstlane(last)) {
            for (int r = lane; r < kTreeGroups; r += 64) {
                st_dev_u32(tb.group_ctr(r), 0u);
                st_dev_u32(tb.release(r), 0u);
            }
            if (lane == 0) {
                st_dev_u32(tb.top(), 0u);
                st_dev_u32(a.sync + kSyncExit, 0u);
            }
        }
    }
}

typedef void (*strip_fn)(StripArgs);

template <int NW, int NI>
strip_fn strip_kernel_for(int b) {
    switch (b) {
        case 1: return decode_strips<1, NW, NI>;
        case 2: return decode_strips<2, NW, NI>;
        case 3: return decode_strips<3, NW, NI>;
        case 4: return decode_strips<4, NW, NI>;
        case 5: return decode_strips<5, NW, NI>;
        case 6: return decode_strips<6, NW, NI>;
        case 7: return decode_strips<7, NW, NI>;
        case 8: return decode_strips<8, NW, NI>;
    }
    return nullptr;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Kernel variants: compute waves per workgroup x 16-byte weight vectors per
// compute lane. A task (one strip of one point) must fit: K <= NI * NW * 64.
// Workgroups are 4 or 8 waves (control + NW): a workgroup's waves are spread
// round-robin over the CU's four SIMDs, so only multiples of 4 let the
// residency that the occupancy query reports actually be reached (the
// cooperative grid relies on it).
struct StripVariant {
    int nw, ni;
    strip_fn (*get)(int);
};
const StripVariant kStripVariants[] = {
    {7, 10, strip_kernel_for<7, 10>},
    {3, 24, strip_kernel_for<3, 24>},
    {7, 20, strip_kernel_for<7, 20>},
};

}  // namespace

// Can the strip step run this plan? (batch, ranks, K alignment, LDS for x)
int tp_strip_loads(const tp_plan_s* p) {
    if (p->batch > kStripMaxBatch || p->n_ranks > 8) return 0;
    const int64_t k0 = p->k_attn / p->n_ranks, k1 = p->inter / p->n_ranks;
    const int64_t kmax = k0 > k1 ? k0 : k1;
    if (k0 % 8 || k1 % 8) return 0;
    if (kmax * p->batch * 2 > kStripMaxXsBytes) return 0;
    for (const StripVariant& v : kStripVariants)
        if (kmax <= (int64_t)v.ni * v.nw * 64) return v.ni;
    return 0;
}

namespace {

// Pick the variant whose resident grid covers the most strips per wave
// (ideally every strip has its own workgroup). Returns false if none fits.
bool pick_strip_variant(const tp_plan_s* p, int64_t kmax, strip_fn* fn, int* block, int* grid,
                        int* xs_out) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return false;
    const int64_t strips = p->hidden / 8;
    int64_t best_per_wg = -1;
    int idx = 0;
    for (const StripVariant& v : kStripVariants) {
        ++idx;
        if (p->strip_variant && idx != p->strip_variant) continue;
        if (kmax > (int64_t)v.ni * v.nw * 64) continue;
        strip_fn k = v.get(p->batch);
        if (!k) continue;
        const int blk = (v.nw + 1) * 64;
        const int64_t rows = (kmax + v.nw * 64 - 1) / (v.nw * 64) * (v.nw * 64);
        const int xs_bytes = (int)(rows * p->batch * 2);
        if (xs_bytes > kStripMaxXsBytes) continue;
        int per_cu = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(k),
                                                         blk, xs_bytes) != hipSuccess)
            continue;
        const int64_t cap = (int64_t)per_cu * cus;
        if (cap < 1) continue;
        const int64_t g = strips < cap ? strips : cap;
        const int64_t per_wg = (strips + g - 1) / g;
        if (per_wg > kStripMaxPerWg) continue;
        if (best_per_wg < 0 || per_wg < best_per_wg) {
            best_per_wg = per_wg;
            *fn = k;
            *block = blk;
            *grid = (int)g;
            *xs_out = xs_bytes;
        }
    }
    return best_per_wg > 0;
}

}  // namespace

extern "C" {

tp_status tp_pack_weights(tp_plan_t p, int32_t point, int32_t n_layers, const void* w,
                          void* w_packed, void* stream) {
    if (!p || !w || !w_packed || n_layers < 0) return TP_ERR_INVALID_ARG;
    if (point != TP_POINT_ATTN_OUT && point != TP_POINT_FFN_DOWN) return TP_ERR_INVALID_ARG;
    if (!aligned16(w) || !aligned16(w_packed)) return TP_ERR_ALIGNMENT;
    if (w == w_packed) return TP_ERR_INVALID_ARG;
    const int64_t K = (point == TP_POINT_ATTN_OUT ? p->k_attn : p->inter) / p->n_ranks;
    const int64_t total = (int64_t)n_layers * K * (p->hidden / 8);
    if (total == 0) return TP_OK;
    const int64_t blocks = (total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536;
    hipLaunchKernelGGL(pack_strips_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       static_cast<const uint16_t*>(w), static_cast<uint16_t*>(w_packed),
                       (int64_t)n_layers, K, p->hidden);
    return hipGetLastError() == hipSuccess ? TP_OK : TP_ERR_DEVICE;
}

tp_status tp_decode_layers_packed(tp_plan_t p, int32_t n_layers, int32_t rank, const void* x_attn,
                                  const void* w_o_packed, const void* x_ffn,
                                  const void* w_down_packed, float* slots, float* hidden,
                                  void* ws, void* stream) {
    if (!p || !x_attn || !w_o_packed || !x_ffn || !w_down_packed || !slots || !hidden || !ws)
        return TP_ERR_INVALID_ARG;
    if (n_layers < 0 || rank < 0 || rank >= p->n_ranks) return TP_ERR_INVALID_ARG;
    if (!aligned16(x_attn) || !aligned16(w_o_packed) || !aligned16(x_ffn) ||
        !aligned16(w_down_packed) || !aligned16(slots) || !aligned16(hidden) || !aligned16(ws))
        return TP_ERR_ALIGNMENT;
    if (!tp_strip_loads(p)) return TP_ERR_UNSUPPORTED;
    const int64_t strips = p->hidden / 8;
    if ((int64_t)n_layers * 2 * strips >= ((int64_t)1 << 31)) return TP_ERR_UNSUPPORTED;
    if ((int64_t)p->batch * p->hidden >= ((int64_t)1 << 31)) return TP_ERR_UNSUPPORTED;
    if (n_layers == 0) return TP_OK;
    StripArgs a;
    a.x0 = static_cast<const uint16_t*>(x_attn);
    a.x1 = static_cast<const uint16_t*>(x_ffn);
    a.w0 = static_cast<const uint16_t*>(w_o_packed);
    a.w1 = static_cast<const uint16_t*>(w_down_packed);
    a.slots = slots;
    a.hidden = hidden;
    a.sync = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + kSyncOffset);
    a.H = (int32_t)p->hidden;
    a.K0 = (int32_t)(p->k_attn / p->n_ranks);
    a.K1 = (int32_t)(p->inter / p->n_ranks);
    a.strips = (int32_t)strips;
    a.layers = n_layers;
    a.n_ranks = p->n_ranks;
    a.rank = rank;
    a.chunk = (int32_t)((int64_t)p->batch * p->hidden / p->n_ranks);
    a.spin_limit = 1u << 21;
    const int64_t kmax = a.K0 > a.K1 ? a.K0 : a.K1;
    strip_fn k = nullptr;
    int block = 0, grid = 0, xs_bytes = 0;
    if (!pick_strip_variant(p, kmax, &k, &block, &grid, &xs_bytes)) return TP_ERR_UNSUPPORTED;
    a.xs_bytes = xs_bytes;
    void* args[] = {&a};
    if (hipLaunchCooperativeKernel(reinterpret_cast<const void*>(k), dim3((unsigned)grid),
                                   dim3((unsigned)block), args, (unsigned)a.xs_bytes,
                                   (hipStream_t)stream) != hipSuccess)
        return TP_ERR_DEVICE;
    return hipGetLastError() == hipSuccess ? TP_OK : TP_ERR_DEVICE;
}

}  // extern "C"
