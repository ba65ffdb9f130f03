// Device helpers shared by the ReplaySSM kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rssm {

constexpr int kWave = 64;
// bits ORed into the caller's err_flags word
constexpr int kDevErrCursor = 1;
constexpr int kDevErrSlot = 2;

// ---------------------------------------------------------------------------------------
// bf16 <-> f32 (raw 16-bit storage; round to nearest even)
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
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

// four floats -> bf16 rounded to nearest even, as two words of pairs (low half first); the
// conversion compiles to the gfx950 packed f32 -> bf16 instruction, two values at a time
typedef __bf16 rssm_bf2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 f32x4_to_bf16x4(float4 v) {
    rssm_bf2 a, b;
    a.x = (__bf16)v.x; a.y = (__bf16)v.y;
    b.x = (__bf16)v.z; b.y = (__bf16)v.w;
    return make_uint2(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b));
}

// ---------------------------------------------------------------------------------------
// Low-precision read copies of the checkpoint ("ReplaySSM" README, benefit "Separate
// state precisions": non-flush steps read a low-precision copy, flushes read and write
// the fp32 checkpoint and refresh the copy).
//   bf16, fp16   round to nearest even from the fp32 checkpoint
//   fp8 e4m3     OCP 8-bit float (1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
//                largest finite 448, code 0x7f/0xff not a number) with one fp32 scale per
//                checkpoint row: scale = amax / 448, code = e4m3(h * (448 / amax)) rounded
//                to nearest even (a zero row has scale 0 and codes 0)
// ---------------------------------------------------------------------------------------
constexpr int kLpNone = 0;
constexpr int kLpBF16 = 1;
constexpr int kLpF16 = 2;
constexpr int kLpFP8 = 3;

typedef _Float16 rssm_h2 __attribute__((ext_vector_type(2)));

// two fp16 values in one 32-bit word -> float2 (low half first)
__device__ __forceinline__ float2 f16x2_bits_to_f32(uint32_t w) {
    const rssm_h2 h = __builtin_bit_cast(rssm_h2, w);
    return make_float2((float)h.x, (float)h.y);
}

__device__ __forceinline__ uint2 f32x4_to_f16x4(float4 v) {
    rssm_h2 a, b;
    a.x = (_Float16)v.x; a.y = (_Float16)v.y;   // round to nearest even
    b.x = (_Float16)v.z; b.y = (_Float16)v.w;
    return make_uint2(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b));
}

typedef float rssm_v2f __attribute__((ext_vector_type(2)));

// four e4m3 codes (little-endian bytes of w) -> their values, by the gfx950 packed
// conversion (OCP E4M3 decoding, subnormals and NaN included): the low 16-bit word
// gives bytes 0 and 1, the high word bytes 2 and 3
__device__ __forceinline__ float4 e4m3x4_to_f32x4(uint32_t w) {
    const rssm_v2f a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    const rssm_v2f b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    return make_float4(a.x, a.y, b.x, b.y);
}

// e4m3 codes of four floats scaled by inv (little-endian bytes), rounded to nearest even
// by the gfx950 packed f32 -> fp8 conversion.  The callers scale rows to at most 448 in
// magnitude; the conversion rounds magnitudes below 464 (the midpoint past the largest
// code) to at most 448, which is the saturation the format's encoding asks for (checked
// against the rounding written out in integer arithmetic at every code value, every
// midpoint and its neighbours, on the device).
__device__ __forceinline__ uint32_t f32x4_to_e4m3x4(float4 v, float inv) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(v.x * inv, v.y * inv, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(v.z * inv, v.w * inv, w, true);
    return (uint32_t)w;
}

// ---------------------------------------------------------------------------------------
// Streaming (non-temporal) accesses for data touched once per launch -- the checkpoint
// stream.  They keep the checkpoint from displacing the small, reused vectors (records,
// B/C) in the caches.
// ---------------------------------------------------------------------------------------
typedef float rssm_v4f __attribute__((ext_vector_type(4)));
typedef unsigned int rssm_v2u __attribute__((ext_vector_type(2)));
typedef unsigned int rssm_v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 ld_stream(const float* p) {
    const rssm_v4f t = __builtin_nontemporal_load(reinterpret_cast<const rssm_v4f*>(p));
    return make_float4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ uint2 ld_stream(const uint16_t* p) {
    const rssm_v2u t = __builtin_nontemporal_load(reinterpret_cast<const rssm_v2u*>(p));
    return make_uint2(t.x, t.y);
}
// eight bf16 values (16 bytes)
__device__ __forceinline__ uint4 ld_stream8(const uint16_t* p) {
    const rssm_v4u t = __builtin_nontemporal_load(reinterpret_cast<const rssm_v4u*>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ void st_stream(float* p, float4 v) {
    rssm_v4f t = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(t, reinterpret_cast<rssm_v4f*>(p));
}
__device__ __forceinline__ void st_stream(uint8_t* p, uint32_t v) {
    __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(p));
}
__device__ __forceinline__ uint4 ld_stream16(const uint8_t* p) {
    const rssm_v4u t = __builtin_nontemporal_load(reinterpret_cast<const rssm_v4u*>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
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

// The same gate with the hardware exponential and reciprocal (relative error ~1e-7):
// used on the per-output path of the replay kernels.  For z -> -inf the reciprocal of
// +inf is 0, so the result goes to 0 like the exact form.
__device__ __forceinline__ float silu_gate_fast(float y, float z) {
    return (y * z) * __frcp_rn(1.0f + __expf(-z));
}

__device__ __forceinline__ float dot4(float4 a, float4 b) {
    return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}

// ---------------------------------------------------------------------------------------
// Order of the sequences of a speculative round.  A round folds the buffer of some
// sequences only (committed + positions > L); their workgroups run much longer than the
// rest and write their checkpoint in place.  Every workgroup computes the same
// permutation of the batch -- the first lead_num/lead_den of the other sequences, then
// the folding ones, then the rest of the others, each part in batch order -- and takes
// the sequence at position `rank`.  The hardware starts workgroups in id order, so the
// folding workgroups start once the reading ones stream and end while the last reading
// ones still keep the memory busy.  Folding first makes their writes share the whole
// launch with reads and, in GDN rounds, their fold preparation coincide with the
// launch's start; folding last leaves them to run alone at the end.
//
// Each thread loads the cursors of one sequence (all loads issued together, so a
// batch of up to NT sequences costs the one global round trip that loading this
// workgroup's own cursors costs anyway); the thread holding the chosen sequence hands
// its cursors to the workgroup through LDS.  Every workgroup reads every sequence's
// cursors, so batches above kRankedMaxBatch keep batch order (the work would grow
// with the square of the batch, and a large grid leaves a short tail anyway).  The
// values are returned unchecked.  Called by all NT threads (it holds barriers); returns
// the same value in all of them.
// ---------------------------------------------------------------------------------------
constexpr int kRankedMaxBatch = 1024;

struct SpecSeq {
    int b, sb, Tb, hd, cm;   // batch row, state row, positions, ring head, committed records
};

template <int NT>
__device__ SpecSeq spec_sequence_ranked(int rank, int batch, int L, int T, const int32_t* slot,
                                        const int32_t* n_pos_seq, const int32_t* head,
                                        const int32_t* committed, int lead_num, int lead_den) {
    constexpr int NW = NT / kWave;
    __shared__ int s_cnt[NW];
    __shared__ SpecSeq s_pick;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    auto load = [&](int i) {
        SpecSeq r;
        r.b = i;
        r.sb = slot ? slot[i] : i;
        r.Tb = n_pos_seq ? n_pos_seq[i] : T;
        r.hd = head[i];
        r.cm = committed[i];
        return r;
    };
    if (batch > kRankedMaxBatch) return load(rank);
    int nheavy = 0;
    if (batch > NT) {   // more than one chunk: count the folding sequences first
        for (int c0 = 0; c0 < batch; c0 += NT) {
            bool h = false;
            if (c0 + tid < batch) {
                const SpecSeq r = load(c0 + tid);
                h = r.cm + r.Tb > L;
            }
            nheavy += __syncthreads_count(h);
        }
    }
    int before_h = 0, before_l = 0;   // folding and other sequences of earlier chunks
    for (int c0 = 0; c0 < batch; c0 += NT) {
        const int i = c0 + tid;
        const bool in = i < batch;    // the in-range threads are a prefix of the chunk
        SpecSeq mine{};
        if (in) mine = load(i);
        const bool h = in && mine.cm + mine.Tb > L;
        const uint64_t m = __ballot(h);
        if (lane == 0) s_cnt[wave] = __popcll(m);
        __syncthreads();
        int hw = 0, hc = 0;           // folding ones in earlier waves, in the whole chunk
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            hw += (w < wave) ? s_cnt[w] : 0;
            hc += s_cnt[w];
        }
        if (batch <= NT) nheavy = hc;
        const int hb = hw + __popcll(m & __lanemask_lt());   // folding ones before i in the chunk
        const int lead = ((batch - nheavy) * lead_num) / lead_den;   // others ranked first
        const int li = before_l + (tid - hb);                         // index among the others
        const int pos = h ? lead + before_h + hb : (li < lead ? li : nheavy + li);
        if (in && pos == rank) s_pick = mine;
        before_h += hc;
        before_l += min(NT, batch - c0) - hc;
        __syncthreads();
    }
    return s_pick;
}

// ---------------------------------------------------------------------------------------
// Cross-lane exchange without LDS.  exchange<D>(a, b) pairs every lane with a partner
// whose lane-id bit log2(D) is the opposite of its own (lanes stay within aligned groups
// of 2D) and returns, in every lane, its own value of one operand plus the partner's
// value of the same operand: lanes with the bit clear get a_own + a_partner, lanes with
// the bit set get b_own + b_partner.  Distances 1..8 use DPP inside a 16-lane row
// (quad_perm for 1 and 2, the half-row mirror for 4, a row rotation by 8 for 8);
// 16 and 32 use the gfx950 permlane swaps, which exchange both operands at once.
// ---------------------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

template <int D>
__device__ __forceinline__ float exchange(float a, float b, int lane) {
    if constexpr (D == 16 || D == 32) {
        const auto r = (D == 16)
            ? __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false)
            : __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
        // lanes with the bit clear now hold (a_own, a_partner), the others (b_partner, b_own)
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    } else {
        const bool up = (lane & D) != 0;
        const float send = up ? a : b;      // the partner keeps the operand this lane drops
        const float keep = up ? b : a;
        constexpr int CTRL = (D == 1) ? 0xB1 : (D == 2) ? 0x4E : (D == 4) ? 0x141 : 0x128;
        return keep + dpp_mov<CTRL>(send);
    }
}

// Sum over an aligned group of W lanes (W a power of two <= 64), returned to all of them.
template <int W>
__device__ __forceinline__ float group_allreduce(float x, int lane) {
    if constexpr (W >= 64) x = exchange<32>(x, x, lane);
    if constexpr (W >= 32) x = exchange<16>(x, x, lane);
    if constexpr (W >= 16) x = exchange<8>(x, x, lane);
    if constexpr (W >= 8) x = exchange<4>(x, x, lane);
    if constexpr (W >= 4) x = exchange<2>(x, x, lane);
    if constexpr (W >= 2) x = exchange<1>(x, x, lane);
    return x;
}

// Maximum over an aligned group of W lanes, returned to all of them (same partners as
// group_allreduce).
template <int W>
__device__ __forceinline__ float group_allmax(float x) {
    if constexpr (W >= 64) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    if constexpr (W >= 32) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    if constexpr (W >= 16) x = fmaxf(x, dpp_mov<0x128>(x));
    if constexpr (W >= 8) x = fmaxf(x, dpp_mov<0x141>(x));
    if constexpr (W >= 4) x = fmaxf(x, dpp_mov<0x4E>(x));
    if constexpr (W >= 2) x = fmaxf(x, dpp_mov<0xB1>(x));
    return x;
}

// ---------------------------------------------------------------------------------------
// Row reduction across the LPR consecutive lanes that share R rows.
//
// Each lane holds partial sums v[0..R) for R rows.  At each level a lane keeps one half
// of its values (the upper half when its level bit is set) and adds the partner's copy
// of that half, so R values take R-1 exchanges in total instead of R*log2(LPR).  On
// return v[0] is the full sum of row index  (lane % LPR) / (LPR / R);  the LPR/R lanes
// with the same row index hold copies.  Requires R <= LPR, both powers of two,
// LPR <= 64, and the LPR lanes aligned to a multiple of LPR.
// ---------------------------------------------------------------------------------------
template <int CNT, int D>
struct RowReduce {
    __device__ static __forceinline__ void run(float* v, int lane) {
        if constexpr (D == 0) {
            static_assert(CNT == 1, "R must not exceed LPR");
        } else {
#pragma unroll
            for (int i = 0; i < (CNT > 1 ? CNT / 2 : 1); ++i)
                v[i] = exchange<D>(v[i], CNT > 1 ? v[i + CNT / 2] : v[i], lane);
            RowReduce<(CNT > 1 ? CNT / 2 : 1), D / 2>::run(v, lane);
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

}  // namespace rssm
