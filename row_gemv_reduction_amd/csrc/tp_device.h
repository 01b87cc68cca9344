// Device helpers shared by the HIP translation units (internal).
//
// Cross-workgroup visibility without device-wide fences: the per-XCD L2s
// are not coherent with each other, and a device-scope fence writes back a
// whole L2 (tens of microseconds when every workgroup does it). Data that
// another workgroup reads inside the same launch is therefore written and
// read with device-scope atomic stores/loads, which gfx950 performs
// coherently at device scope (sc1); a writer waits for its stores to
// complete (s_waitcnt vmcnt(0)) before it signals through a device-scope
// atomic counter, and a reader reads only after it has observed the counter.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpdev {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// float -> bf16, round to nearest even, NaN kept quiet
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu))
        return (uint16_t)((u >> 16) | 0x40u);
    uint32_t rounding = 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)((u + rounding) >> 16);
}

// Buffer descriptor word 3 for raw (untyped) buffer loads on gfx9-class
// parts, and the nontemporal cache policy for streamed weights.
constexpr int kBufferRsrcWord3 = 0x00020000;
constexpr int kCachePolicyNT = 2;

// Weights are read exactly once per step: stream them past the caches.
__device__ __forceinline__ u32x4_t load_stream16(const uint16_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

// 16-byte device-coherent (sc1) accesses through a raw buffer descriptor
// over [base, base + bytes): four consecutive fp32 values exchanged between
// workgroups in one access instead of four.
constexpr int kCachePolicyDevice = 16;  // sc1: coherent at device scope
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dev_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             kBufferRsrcWord3);
}
__device__ __forceinline__ floatx4_t ld_dev4(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off) {
    return __builtin_bit_cast(floatx4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, byte_off, 0,
                                                                                kCachePolicyDevice));
}
__device__ __forceinline__ void st_dev4(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off, floatx4_t v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), rs, byte_off, 0,
                                           kCachePolicyDevice);
}

// A device-coherent 32-bit load through a buffer descriptor (zero past its
// range), volatile so that a polling loop re-reads it.
constexpr int kCachePolicyVolatile = (int)(1u << 31);
__device__ __forceinline__ uint32_t ld_dev_u32_buf(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, byte_off, 0,
                                                         kCachePolicyDevice | kCachePolicyVolatile);
}

// Device-coherent accesses for data exchanged inside one launch.
__device__ __forceinline__ void st_dev(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev_u32(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev_u32(const uint32_t* p) {
    return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_dev_u32(uint32_t* p, uint32_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until this wave's memory operations have completed (stores acked at
// the scope they were issued with). Also a compiler barrier.
__device__ __forceinline__ void wait_mem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void compiler_barrier() { asm volatile("" ::: "memory"); }

// Ring-order sum of one element: chunk c = i / C is summed over ranks
// c, c+1, ..., c+N-1 (mod N), one binary32 addition at a time, then the
// residual is added. `own` is this rank's value (bit-identical to what is
// stored in its slot; rank < 0: every value comes from `slots`). The loads
// of a group of up to 8 ranks are issued together (one memory round trip),
// then added in ring order. Only additions, so nothing can be contracted.
__device__ __forceinline__ float ring_element(const float* slots, int64_t len, int64_t i,
                                              int64_t chunk, int n_ranks, int rank, float own,
                                              float residual) {
#pragma clang fp contract(off)
    const int c = (int)(i / chunk);
    float s = 0.f;
    for (int j0 = 0; j0 < n_ranks; j0 += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            int j = j0 + u < n_ranks ? j0 + u : n_ranks - 1;
            int r = c + j;
            if (r >= n_ranks) r -= n_ranks;
            v[u] = r == rank ? own : slots[(int64_t)r * len + i];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (j0 + u < n_ranks) s = (j0 + u == 0) ? v[u] : s + v[u];
        }
    }
    return s + residual;
}

// Thread 0 waits until *ctr >= target; bounded. On timeout (or if another
// workgroup already timed out) the error word is set and false returned,
// and every later wait returns at once, so the grid always drains.
__device__ inline bool wait_at_least(uint32_t* ctr, uint32_t target, uint32_t* err, uint32_t limit) {
    if (target == 0) return true;
    for (uint32_t n = 0;; ++n) {
        if (ld_dev_u32(ctr) >= target) return true;
        if ((n & 31) == 31 && ld_dev_u32(err)) return false;
        if (n >= limit) {
            __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return false;
        }
        __builtin_amdgcn_s_sleep(2);
    }
}


// Sum of v over the 64 lanes of a wave; every lane gets the total. Within
// rows of 16 lanes the partners come from DPP lane swizzles (xor 1, xor 2,
// then half-row and row mirrors), across rows from two cross-lane permutes.
// Each step adds two values in a fixed pairing, so every lane ends with the
// same bits and the result does not depend on scheduling.
__device__ __forceinline__ float wave_sum(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));  // quad_perm 2,3,0,1
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false)); // row_half_mirror
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false)); // row_mirror
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}

// LDS word loads/stores that the compiler neither caches nor reorders with
// respect to each other (flags between the waves of one workgroup).
__device__ __forceinline__ int lds_ld(const int* p) {
    return __hip_atomic_load(const_cast<int*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_st(int* p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_add(int* p, int v) {
    __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// This wave's LDS accesses have completed (and a compiler barrier).
__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Wait until the LDS flag reaches `target`. Bounded (far beyond any real
// wait): on timeout bit 1 of the error word is set and the wave goes on, so
// the launch always ends.
constexpr int kWaveSpinLimit = 1 << 22;
__device__ __forceinline__ void wait_flag(const int* f, int target, uint32_t* err) {
    for (int n = 0; lds_ld(f) < target; ++n) {
        if (n >= kWaveSpinLimit) {
            __hip_atomic_fetch_or(err, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
        __builtin_amdgcn_s_sleep(1);
    }
}

}  // namespace tpdev
