// sv_common.h -- device helpers shared by the verification kernels (gfx950).
//
// Row streaming: a logits row is read once from HBM with 16-byte vector loads
// (8 bfloat16 or 4 float32 per lane), fully coalesced across the wave.  A row
// may start at any element-aligned address: the elements before the first
// 16-byte boundary (the head) and after the last full vector (the tail) are
// read one by one.  Each lane visits its elements in increasing index order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "spec_verify.h"
#include "sv_host.h"

namespace sv {

constexpr int kWave = 64;

// A native 16-byte vector (the HIP uint4 struct is not accepted by the
// nontemporal-load builtin).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 2^x on the hardware exp unit (v_exp_f32, about 1 ulp).  Results below the
// smallest normal float32 (x < -126) flush to zero: such weights are below
// 1.2e-38 of the row maximum's.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroup barrier that waits for this wave's LDS accesses only: global
// loads and atomics stay in flight across it (__syncthreads would wait for
// them too).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ---------------------------------------------------------------------------
// Element decoding.  bfloat16 widens to float32 exactly (it is the high half).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

template <int DT> struct Elem;
template <> struct Elem<SV_F32> {
    static constexpr int kBytes = 4;
    static constexpr int kPerVec = 4;
    __device__ __forceinline__ static float load(const void *base, int64_t i) {
        return reinterpret_cast<const float *>(base)[i];
    }
    __device__ __forceinline__ static void unpack(const u32x4 &v, float (&o)[kPerVec]) {
        o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y);
        o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
    }
    // element k of a vector (k a compile-time constant after unrolling)
    __device__ __forceinline__ static float elem(const u32x4 &v, int k) {
        return __uint_as_float(k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w);
    }
};
template <> struct Elem<SV_BF16> {
    static constexpr int kBytes = 2;
    static constexpr int kPerVec = 8;
    __device__ __forceinline__ static float load(const void *base, int64_t i) {
        return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(base)[i] << 16);
    }
    __device__ __forceinline__ static void unpack(const u32x4 &v, float (&o)[kPerVec]) {
        o[0] = bf16_lo(v.x); o[1] = bf16_hi(v.x); o[2] = bf16_lo(v.y); o[3] = bf16_hi(v.y);
        o[4] = bf16_lo(v.z); o[5] = bf16_hi(v.z); o[6] = bf16_lo(v.w); o[7] = bf16_hi(v.w);
    }
    __device__ __forceinline__ static float elem(const u32x4 &v, int k) {
        const uint32_t w = k < 2 ? v.x : k < 4 ? v.y : k < 6 ? v.z : v.w;
        return (k & 1) ? bf16_hi(w) : bf16_lo(w);
    }
};

// Order-preserving unsigned key of a float32 (larger float -> larger key;
// -0 and +0 get different keys, so callers compare VALUES where they must be equal).
__device__ __forceinline__ uint32_t fkey(float f) {
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float fkey_inv(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// ---------------------------------------------------------------------------
// Row geometry: head / 16-byte vector body / tail split of one row.
// ---------------------------------------------------------------------------
struct RowSplit {
    int32_t head;     // scalar elements before the first 16-byte boundary
    int32_t nvec;     // full 16-byte vectors
    int32_t tail;     // scalar elements after the body
};

template <int DT>
__device__ __forceinline__ RowSplit row_split(const void *row, int32_t len) {
    using E = Elem<DT>;
    uintptr_t a = reinterpret_cast<uintptr_t>(row);
    int32_t head = (int32_t)(((16u - (uint32_t)(a & 15u)) & 15u) / E::kBytes);
    if (head > len) head = len;
    int32_t nvec = (len - head) / E::kPerVec;
    RowSplit s;
    s.head = head;
    s.nvec = nvec;
    s.tail = len - head - nvec * E::kPerVec;
    return s;
}

// ---------------------------------------------------------------------------
// Wave / workgroup reductions (wave64).
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
        T w = __shfl_xor(v, o, kWave);
        v = w > v ? w : v;
    }
    return v;
}

// Argmax pair: larger value wins; equal values go to the lower index.
__device__ __forceinline__ ArgMax argmax_merge(ArgMax a, ArgMax b) {
    return (b.v > a.v || (b.v == a.v && b.i < a.i)) ? b : a;
}
__device__ __forceinline__ ArgMax wave_argmax(ArgMax a) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
        ArgMax b;
        b.v = __shfl_xor(a.v, o, kWave);
        b.i = __shfl_xor(a.i, o, kWave);
        a = argmax_merge(a, b);
    }
    return a;
}

// Online softmax partial: s = sum over the elements of 2^((z - m) * c).
__device__ __forceinline__ MaxSum maxsum_merge(MaxSum a, MaxSum b, float c) {
    if (b.m > a.m) { MaxSum t = a; a = b; b = t; }
    if (b.m == -INFINITY) return a;            // also covers a.m == b.m == -inf
    a.s = a.s + b.s * exp2_hw((b.m - a.m) * c);
    return a;
}
__device__ __forceinline__ MaxSum wave_maxsum(MaxSum a, float c) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
        MaxSum b;
        b.m = __shfl_xor(a.m, o, kWave);
        b.s = __shfl_xor(a.s, o, kWave);
        a = maxsum_merge(a, b, c);
    }
    return a;
}

// Inclusive prefix sum of doubles across a wave (lane order).
__device__ __forceinline__ double wave_incl_scan(double v) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        double w = __shfl_up(v, o, kWave);
        if (lane >= o) v += w;
    }
    return v;
}

// ---------------------------------------------------------------------------
// Publishing results between workgroups of one launch.
//
// On gfx942/gfx950 each XCD has its own L2, and a device-scope fence writes
// back and invalidates the whole L2 -- thousands of workgroups doing that
// serialise on it.  Instead, data that another workgroup will read in the
// same launch is written and read with agent-scope atomic stores / loads
// (coherent across XCDs without cache maintenance), and the fences only
// order: every thread waits for its own stores to complete (s_waitcnt
// vmcnt(0)) before the workgroup bumps the counter, and the last workgroup
// issues its loads only after it has seen the counter.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void pub_u64(void *p, uint64_t v) {
    __hip_atomic_store(reinterpret_cast<uint64_t *>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t sub_u64(const void *p) {
    return __hip_atomic_load(reinterpret_cast<const uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Publish / read a trivially copyable struct whose size is a multiple of 8.
template <typename T>
__device__ __forceinline__ void pub(T *dst, const T &v) {
    static_assert(sizeof(T) % 8 == 0, "published structs are whole 64-bit words");
    uint64_t w[sizeof(T) / 8];
    __builtin_memcpy(w, &v, sizeof(T));
#pragma unroll
    for (int k = 0; k < (int)(sizeof(T) / 8); ++k) pub_u64(reinterpret_cast<uint64_t *>(dst) + k, w[k]);
}
template <typename T>
__device__ __forceinline__ T sub(const T *src) {
    static_assert(sizeof(T) % 8 == 0, "published structs are whole 64-bit words");
    uint64_t w[sizeof(T) / 8];
#pragma unroll
    for (int k = 0; k < (int)(sizeof(T) / 8); ++k) w[k] = sub_u64(reinterpret_cast<const uint64_t *>(src) + k);
    T v;
    __builtin_memcpy(&v, w, sizeof(T));
    return v;
}

// Wait until this thread's vector-memory operations have completed
// (s_waitcnt with vmcnt = 0, expcnt and lgkmcnt left at their maxima),
// with a workgroup-scope fence so the compiler keeps the order.
__device__ __forceinline__ void order_release() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xf << 8));
}
__device__ __forceinline__ void order_acquire() {
    __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xf << 8));
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// ---------------------------------------------------------------------------
// Last-arriving workgroup.  Every workgroup of a group publishes its partial
// results (pub*), then bumps the group's counter; the workgroup that brings
// the counter to `total` continues with the group's combine step (reading
// with sub*) and returns the counter to zero for the next call.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool arrive_last(uint32_t *counter, uint32_t total, int *flag_smem) {
    order_release();
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev =
            __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int last = (prev == total - 1u);
        if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *flag_smem = last;
    }
    __syncthreads();
    const bool last = *flag_smem != 0;
    if (last) {
        order_acquire();
        // the combine step is short and on the critical path: issue ahead of
        // the streaming waves of other workgroups on this CU
        __builtin_amdgcn_s_setprio(3);
    }
    return last;
}

}  // namespace sv
