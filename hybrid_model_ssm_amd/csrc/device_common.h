// Device helpers shared by the ReplaySSM kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rssm {

constexpr int kWave = 64;
constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies, each with its own L2

// ---------------------------------------------------------------------------------------
// bf16 <-> f32 (raw 16-bit storage; round to nearest even)
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;  // quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// Input/output element types: float, or bf16 kept as raw uint16_t.
template <typename IO> struct Io;

template <> struct Io<float> {
    using T = float;
    using Raw4 = float4;  // four elements as loaded
    __device__ static __forceinline__ Raw4 ldraw4(const T* p, size_t i) {
        return *reinterpret_cast<const float4*>(p + i);
    }
    __device__ static __forceinline__ void straw4(T* p, size_t i, Raw4 r) {
        *reinterpret_cast<float4*>(p + i) = r;
    }
    __device__ static __forceinline__ float4 cvt4(Raw4 r) { return r; }
    __device__ static __forceinline__ float ld(const T* p, size_t i) { return p[i]; }
    // four consecutive elements (i multiple of 4, 16-byte aligned)
    __device__ static __forceinline__ float4 ld4(const T* p, size_t i) {
        return *reinterpret_cast<const float4*>(p + i);
    }
};

template <> struct Io<uint16_t> {
    using T = uint16_t;
    using Raw4 = uint2;
    __device__ static __forceinline__ Raw4 ldraw4(const T* p, size_t i) {
        return *reinterpret_cast<const uint2*>(p + i);
    }
    __device__ static __forceinline__ void straw4(T* p, size_t i, Raw4 r) {
        *reinterpret_cast<uint2*>(p + i) = r;
    }
    __device__ static __forceinline__ float4 cvt4(Raw4 r) {
        return make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
                           __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u));
    }
    __device__ static __forceinline__ float ld(const T* p, size_t i) { return bf16_bits_to_f32(p[i]); }
    // four consecutive elements (i multiple of 4, 8-byte aligned)
    __device__ static __forceinline__ float4 ld4(const T* p, size_t i) {
        const uint2 r = *reinterpret_cast<const uint2*>(p + i);
        return make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
                           __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u));
    }
};

__device__ __forceinline__ float4 bf16x4_to_f32x4(uint2 r) {
    return make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
                       __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u));
}

__device__ __forceinline__ uint2 f32x4_to_bf16x4(float4 v) {
    return make_uint2(f32_to_bf16_bits(v.x) | (f32_to_bf16_bits(v.y) << 16),
                      f32_to_bf16_bits(v.z) | (f32_to_bf16_bits(v.w) << 16));
}

// ---------------------------------------------------------------------------------------
// Streaming (non-temporal) accesses for data touched once per launch -- the checkpoint
// stream.  They keep the checkpoint from displacing the small, reused vectors (records,
// B/C) in the caches.
// ---------------------------------------------------------------------------------------
typedef float rssm_v4f __attribute__((ext_vector_type(4)));
typedef unsigned int rssm_v2u __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float4 ld_stream(const float* p) {
    const rssm_v4f t = __builtin_nontemporal_load(reinterpret_cast<const rssm_v4f*>(p));
    return make_float4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ uint2 ld_stream(const uint16_t* p) {
    const rssm_v2u t = __builtin_nontemporal_load(reinterpret_cast<const rssm_v2u*>(p));
    return make_uint2(t.x, t.y);
}
__device__ __forceinline__ void st_stream(float* p, float4 v) {
    rssm_v4f t = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(t, reinterpret_cast<rssm_v4f*>(p));
}
__device__ __forceinline__ void st_stream(uint16_t* p, uint2 v) {
    rssm_v2u t = {v.x, v.y};
    __builtin_nontemporal_store(t, reinterpret_cast<rssm_v2u*>(p));
}

// ---------------------------------------------------------------------------------------
// Scalar math
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ float softplus_f32(float u) {
    return u > 20.0f ? u : log1pf(expf(u));
}

__device__ __forceinline__ float silu_gate(float y, float z) {
    return y * z / (1.0f + expf(-z));
}

__device__ __forceinline__ float dot4(float4 a, float4 b) {
    return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}

// ---------------------------------------------------------------------------------------
// Workgroup -> tile mapping for kernels whose neighbouring workgroups share inputs (the
// conventional kernels: the heads of one group read the same B/C).  The hardware hands
// workgroups to the 8 XCDs round robin (id % 8); the remap puts consecutive logical
// tiles on one XCD so they share its L2.  The replay kernels do not use it: a replay
// workgroup owns its whole group, and there the hardware order streams faster.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
    if (nblocks % kNumXcd) return bid;
    return (bid % kNumXcd) * (nblocks / kNumXcd) + bid / kNumXcd;
}

// ---------------------------------------------------------------------------------------
// Row reduction across the LPR consecutive lanes that share R rows.
//
// Each lane holds partial sums v[0..R) for R rows.  At each butterfly level a lane
// keeps one half of its values and sends the other half to its partner, so R values
// take R-1 exchanges in total instead of R*log2(LPR).  On return v[0] is the full
// sum of row index  (lane % LPR) / (LPR / R);  the LPR/R lanes with the same row
// index hold copies.  Requires R <= LPR, both powers of two, LPR <= 64, and the LPR
// lanes aligned to a multiple of LPR.
// ---------------------------------------------------------------------------------------
template <int CNT, int D>
struct RowReduce {
    __device__ static __forceinline__ void run(float* v, int lane) {
        if constexpr (D == 0) {
            static_assert(CNT == 1, "R must not exceed LPR");
        } else if constexpr (CNT == 1) {
            v[0] += __shfl_xor(v[0], D);
            RowReduce<1, D / 2>::run(v, lane);
        } else {
            const bool up = (lane & D) != 0;
#pragma unroll
            for (int i = 0; i < CNT / 2; ++i) {
                const float send = up ? v[i] : v[i + CNT / 2];
                const float keep = up ? v[i + CNT / 2] : v[i];
                v[i] = keep + __shfl_xor(send, D);
            }
            RowReduce<CNT / 2, D / 2>::run(v, lane);
        }
    }
};

template <int R, int LPR>
__device__ __forceinline__ float row_reduce(float (&v)[R], int lane) {
    static_assert(R >= 1 && R <= LPR && (R & (R - 1)) == 0 && (LPR & (LPR - 1)) == 0, "shape");
    RowReduce<R, LPR / 2>::run(v, lane);
    return v[0];
}

}  // namespace rssm

namespace rssm {

// Full sum of each of the R rows, returned to every one of the LPR lanes of the row
// group: transpose-reduce, then gather each row's total from the lane that holds it.
template <int R, int LPR>
__device__ __forceinline__ void row_allreduce(float (&v)[R], int lane) {
    float t[R];
#pragma unroll
    for (int k = 0; k < R; ++k) t[k] = v[k];
    const float mine = row_reduce<R, LPR>(t, lane);
    const int base = lane & ~(LPR - 1);
#pragma unroll
    for (int k = 0; k < R; ++k) v[k] = __shfl(mine, base + k * (LPR / R));
}

// Sum over a power-of-two group of W consecutive lanes, returned to all of them.
template <int W>
__device__ __forceinline__ float group_allreduce(float x) {
#pragma unroll
    for (int d = W / 2; d >= 1; d >>= 1) x += __shfl_xor(x, d);
    return x;
}

}  // namespace rssm
