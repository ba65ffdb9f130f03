// Streaming-bandwidth probes: the device ceilings the decode kernels are measured against.
//
// Built as its own library (libreplayssm_probes.so) for the benchmark only; it is not part
// of the decode library's C ABI.  The probes move fp32 tiles of 128-float rows the way the
// decode kernels stream the checkpoint: 256 threads, 32 consecutive lanes per row with
// 16-byte accesses, R rows per thread, so a tile is [8R rows, 128] (R = 8: one 64 x 128
// head of the Mamba2 checkpoint, 32 KiB; R = 1: 4 KiB, one 16-byte access per thread).  A
// workgroup owns TPW consecutive tiles and loads tile t+1 while it finishes tile t, as the
// replay kernels do; TPW = 16 with R = 8 is the replay kernel's 16 heads per workgroup,
// TPW = 1 with R = 8 the conventional kernel's one head per workgroup.
//
//   mode 0 (read):        sum each tile's values; one float per workgroup to `sink`
//   mode 1 (read+write):  dst[tile] = scale * src[tile]; dst == src is the in-place
//                         update of the flush and conventional steps, dst != src a copy
//   mode 2 (read+write):  as mode 1, with the next tile's loads and the current tile's
//                         stores alternating (load row k of tile t+1, store row k of tile
//                         t) instead of all loads of tile t+1, then all stores of tile t
//
// Loads and stores are plain or non-temporal (the decode kernels stream the checkpoint
// with non-temporal accesses).  ORDER places a workgroup's tiles:
//   0 blocked:     workgroup w owns tiles [w TPW, (w + 1) TPW), walked in order
//   1 skewed:      the same tiles, walked from tile w % TPW (and wrapping), so that the
//                  workgroups in flight sit at different offsets of their regions
//   2 interleaved: workgroup w's tile t is tile t G + w (G workgroups), so that the
//                  workgroups in flight together touch one compact stretch of memory
//
// A second probe reads in the replay kernels' shape (16 tiles of [64, 128] per workgroup,
// non-temporal) and then stores a block of its own, as the decode kernels store their
// outputs and records after streaming the checkpoint; timed at several block sizes against
// the same stream with no block, it prices a byte written inside a read stream.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rssm_probe {

constexpr int kThreads = 256;
constexpr int kCols = 128;                   // floats per row
constexpr int kLpr = kCols / 4;              // lanes per row (16-byte accesses)
constexpr int kRpp = kThreads / kLpr;        // rows per pass of the workgroup
constexpr int64_t kPassFloats = (int64_t)kRpp * kCols;   // one 16-byte access per thread

typedef float v4f __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ v4f load4(const float* p) {
    if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p));
    else return *reinterpret_cast<const v4f*>(p);
}

template <bool NT>
__device__ __forceinline__ void store4(float* p, v4f v) {
    if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<v4f*>(p));
    else *reinterpret_cast<v4f*>(p) = v;
}

template <int R, int TPW, bool NTL, bool NTS, int MODE, int ORDER>
__global__ void __launch_bounds__(kThreads) stream_probe_kernel(const float* src, float* dst,
                                                                 float* sink, float scale) {
    constexpr int kR = R;
    constexpr int64_t kTileFloats = kR * kPassFloats;
    const int tid = threadIdx.x;
    const int row0 = tid / kLpr;
    const int col4 = tid % kLpr;
    const int64_t first = (int64_t)blockIdx.x * TPW;   // this workgroup's first tile (blocked)
    const int64_t lane_off = (int64_t)row0 * kCols + 4 * col4;
    v4f va[kR], vb[kR];
    const int rot = ORDER == 1 ? (int)(blockIdx.x % TPW) : 0;
    auto tile = [&](int t) -> int64_t {
        if constexpr (ORDER == 2) return (int64_t)t * gridDim.x + blockIdx.x;
        return first + (t + rot < TPW ? t + rot : t + rot - TPW);
    };
    auto issue = [&](int t, v4f (&v)[kR]) {
        const float* p = src + tile(t) * kTileFloats + lane_off;
#pragma unroll
        for (int k = 0; k < kR; ++k) v[k] = load4<NTL>(p + (int64_t)k * kRpp * kCols);
    };
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    auto finish = [&](int t, const v4f (&v)[kR]) {
        if constexpr (MODE == 0) {
#pragma unroll
            for (int k = 0; k < kR; ++k) acc += v[k];
        } else {
            float* p = dst + tile(t) * kTileFloats + lane_off;
#pragma unroll
            for (int k = 0; k < kR; ++k) store4<NTS>(p + (int64_t)k * kRpp * kCols, v[k] * scale);
        }
    };
    issue(0, va);
    for (int t = 0; t + 1 < TPW; ++t) {
        if constexpr (MODE == 2) {
            const float* ps = src + tile(t + 1) * kTileFloats + lane_off;
            float* pd = dst + tile(t) * kTileFloats + lane_off;
#pragma unroll
            for (int k = 0; k < kR; ++k) {
                vb[k] = load4<NTL>(ps + (int64_t)k * kRpp * kCols);
                store4<NTS>(pd + (int64_t)k * kRpp * kCols, va[k] * scale);
            }
        } else {
            issue(t + 1, vb);
            finish(t, va);
        }
#pragma unroll
        for (int k = 0; k < kR; ++k) va[k] = vb[k];
    }
    finish(TPW - 1, va);
    if constexpr (MODE == 0) {
        // one value per workgroup keeps the loads live; the order of the sum is irrelevant
        __shared__ float part[kThreads / 64];
        float s = acc.x + acc.y + acc.z + acc.w;
        for (int d = 32; d >= 1; d >>= 1) s += __shfl_xor(s, d);
        if ((tid & 63) == 0) part[tid / 64] = s;
        __syncthreads();
        if (tid == 0) sink[blockIdx.x] = part[0] + part[1] + part[2] + part[3];
    }
}

template <int R, int TPW, int MODE, int ORDER>
static const void* pick_nt(bool ntl, bool nts) {
    if (ntl) return nts ? (const void*)&stream_probe_kernel<R, TPW, true, true, MODE, ORDER>
                        : (const void*)&stream_probe_kernel<R, TPW, true, false, MODE, ORDER>;
    return nts ? (const void*)&stream_probe_kernel<R, TPW, false, true, MODE, ORDER>
               : (const void*)&stream_probe_kernel<R, TPW, false, false, MODE, ORDER>;
}

template <int R, int TPW, int ORDER>
static const void* pick_mode(int mode, bool ntl, bool nts) {
    return mode == 0 ? pick_nt<R, TPW, 0, ORDER>(ntl, false)
         : mode == 1 ? pick_nt<R, TPW, 1, ORDER>(ntl, nts) : pick_nt<R, TPW, 2, ORDER>(ntl, nts);
}

template <int R, int ORDER>
static const void* pick_tpw(int tpw, int mode, bool ntl, bool nts) {
    return tpw == 4 ? pick_mode<R, 4, ORDER>(mode, ntl, nts) : pick_mode<R, 16, ORDER>(mode, ntl, nts);
}

template <int R>
static const void* pick(int tpw, int mode, bool ntl, bool nts, int order) {
    if (order == 1) return pick_tpw<R, 1>(tpw, mode, ntl, nts);
    if (order == 2) return pick_tpw<R, 2>(tpw, mode, ntl, nts);
    return tpw == 1 ? pick_mode<R, 1, 0>(mode, ntl, nts) : pick_tpw<R, 0>(tpw, mode, ntl, nts);
}

__global__ void __launch_bounds__(kThreads) read_then_write_kernel(const float* src, float* dst, float* sink,
                                                                    int64_t write_floats) {
    constexpr int kR = 8, kTpw = 16;
    constexpr int64_t kTileFloats = kR * kPassFloats;
    const int tid = threadIdx.x;
    const int64_t lane_off = (int64_t)(tid / kLpr) * kCols + 4 * (tid % kLpr);
    const float* base = src + (int64_t)blockIdx.x * kTpw * kTileFloats + lane_off;
    v4f va[kR], vb[kR];
    v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < kR; ++k) va[k] = load4<true>(base + (int64_t)k * kRpp * kCols);
    for (int t = 0; t + 1 < kTpw; ++t) {
#pragma unroll
        for (int k = 0; k < kR; ++k) vb[k] = load4<true>(base + (int64_t)(t + 1) * kTileFloats + (int64_t)k * kRpp * kCols);
#pragma unroll
        for (int k = 0; k < kR; ++k) acc += va[k];
#pragma unroll
        for (int k = 0; k < kR; ++k) va[k] = vb[k];
    }
#pragma unroll
    for (int k = 0; k < kR; ++k) acc += va[k];
    // the block depends on every value read, like the decode kernels' outputs
    float* d = dst + (int64_t)blockIdx.x * write_floats;
    for (int64_t i = 4 * (int64_t)tid; i < write_floats; i += 4 * kThreads) store4<true>(d + i, acc);
    __shared__ float part[kThreads / 64];
    float s = acc.x + acc.y + acc.z + acc.w;
    for (int dd = 32; dd >= 1; dd >>= 1) s += __shfl_xor(s, dd);
    if ((tid & 63) == 0) part[tid / 64] = s;
    __syncthreads();
    if (tid == 0) sink[blockIdx.x] = part[0] + part[1] + part[2] + part[3];
}

}  // namespace rssm_probe

extern "C" {

// Floats one workgroup moves per tile pass (one 16-byte access per thread); a tile with
// R rows per thread is R times that.
int64_t replayssm_probe_pass_floats(void) { return rssm_probe::kPassFloats; }

// One probe launch on `stream`.
//   src       device f32 [n_floats], 16-byte aligned (read by every mode)
//   dst       modes 1, 2: device f32 [n_floats], 16-byte aligned (may equal src); mode 0: ignored
//   sink      mode 0: device f32 [number of workgroups] (one sum each); modes 1, 2: ignored
//   n_floats  > 0 and a multiple of pass_floats * rows_per_thread * tiles_per_wg;
//             the grid is n_floats / that (at most 2^31 - 1 workgroups)
//   rows_per_thread in {1, 2, 8};  tiles_per_wg in {1, 4, 16}
//   mode      0 read, 1 read+write, 2 read+write with alternating loads and stores;
//             nt_load / nt_store: nonzero for non-temporal accesses
//   order     0 blocked, 1 skewed, 2 interleaved (1 and 2 need tiles_per_wg > 1)
// Returns 0 on success, 1 for an invalid argument (nothing launched), 3 when the launch failed.
int replayssm_probe_stream(const float* src, float* dst, float* sink, int64_t n_floats, int32_t rows_per_thread,
                           int32_t tiles_per_wg, int32_t mode, int32_t nt_load, int32_t nt_store, int32_t order,
                           float scale, hipStream_t stream) {
    using namespace rssm_probe;
    if (!src || (reinterpret_cast<uintptr_t>(src) & 15) || n_floats <= 0) return 1;
    if (rows_per_thread != 1 && rows_per_thread != 2 && rows_per_thread != 8) return 1;
    if (tiles_per_wg != 1 && tiles_per_wg != 4 && tiles_per_wg != 16) return 1;
    const int64_t per_wg = kPassFloats * rows_per_thread * tiles_per_wg;
    if (n_floats % per_wg) return 1;
    if (mode == 0 && !sink) return 1;
    if (mode != 0 && (!dst || (reinterpret_cast<uintptr_t>(dst) & 15))) return 1;
    if (mode < 0 || mode > 2) return 1;
    if (order < 0 || order > 2 || (order != 0 && tiles_per_wg == 1)) return 1;
    const int64_t grid = n_floats / per_wg;
    if (grid > INT32_MAX) return 1;
    const bool ntl = nt_load != 0, nts = nt_store != 0;
    const void* fn = rows_per_thread == 1 ? pick<1>(tiles_per_wg, mode, ntl, nts, order)
                   : rows_per_thread == 2 ? pick<2>(tiles_per_wg, mode, ntl, nts, order)
                                          : pick<8>(tiles_per_wg, mode, ntl, nts, order);
    void* args[] = {(void*)&src, (void*)&dst, (void*)&sink, (void*)&scale};
    const hipError_t e = hipLaunchKernel(fn, dim3((unsigned)grid), dim3(kThreads), args, 0, stream);
    return e == hipSuccess ? 0 : 3;
}

// Floats one workgroup of the read-then-write probe reads (16 tiles of [64, 128]).
int64_t replayssm_probe_rtw_read_floats(void) { return rssm_probe::kPassFloats * 8 * 16; }

// One launch of the read-then-write probe on `stream`.
//   src           device f32 [n_floats], 16-byte aligned; n_floats > 0 and a multiple of
//                 replayssm_probe_rtw_read_floats() (the grid is n_floats / that)
//   dst           device f32 [grid * write_floats], 16-byte aligned; may be null when
//                 write_floats is 0
//   sink          device f32 [grid] (one sum per workgroup)
//   write_floats  floats each workgroup stores after its reads: >= 0, a multiple of 4
// Returns 0 on success, 1 for an invalid argument (nothing launched), 3 when the launch failed.
int replayssm_probe_read_then_write(const float* src, float* dst, float* sink, int64_t n_floats,
                                    int64_t write_floats, hipStream_t stream) {
    using namespace rssm_probe;
    const int64_t per_wg = replayssm_probe_rtw_read_floats();
    if (!src || (reinterpret_cast<uintptr_t>(src) & 15) || !sink || n_floats <= 0 || n_floats % per_wg) return 1;
    if (write_floats < 0 || write_floats % 4) return 1;
    if (write_floats > 0 && (!dst || (reinterpret_cast<uintptr_t>(dst) & 15))) return 1;
    const int64_t grid = n_floats / per_wg;
    if (grid > INT32_MAX) return 1;
    void* args[] = {(void*)&src, (void*)&dst, (void*)&sink, (void*)&write_floats};
    const hipError_t e = hipLaunchKernel((const void*)&read_then_write_kernel, dim3((unsigned)grid), dim3(kThreads),
                                         args, 0, stream);
    return e == hipSuccess ? 0 : 3;
}

}  // extern "C"
