// Emulated storage precision of a state ("ReplaySSM" README, the paragraph on its two
// precision folders: the emulation kernels keep the read precision and the recurrence
// precision apart and expose how each rounds).  An fp32 array is
// rounded in place to the values a narrower format holds, so that a recurrence that
// keeps its state in that format can be run on the fp32 kernels: round the checkpoint
// after every flush (replay) or the state after every step (conventional update).
// The formats and their rounding are those of the read copies.
//
// One wave per row (rows are grid-strided); a row is read with 16-byte loads.  The
// row-scaled fp8 format needs the row's amax first, so its rows are read twice (the
// second read hits the caches for the row sizes used here).

#include "device_common.h"
#include "launch.h"

namespace rssm {

constexpr int kEmuThreads = 256;

__device__ __forceinline__ float4 round_bf16x4(float4 v) {
    return bf16x4_to_f32x4(f32x4_to_bf16x4(v));
}

__device__ __forceinline__ float4 round_f16x4(float4 v) {
    const uint2 w = f32x4_to_f16x4(v);
    const float2 a = f16x2_bits_to_f32(w.x), b = f16x2_bits_to_f32(w.y);
    return make_float4(a.x, a.y, b.x, b.y);
}

template <int KIND>
__global__ void __launch_bounds__(kEmuThreads) emulate_precision_kernel(float* data, int64_t rows,
                                                                        int32_t row_len, float* row_scale) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t wave = ((int64_t)blockIdx.x * kEmuThreads + threadIdx.x) / kWave;
    const int64_t nwave = (int64_t)gridDim.x * (kEmuThreads / kWave);
    const int n4 = row_len / 4;
    for (int64_t r = wave; r < rows; r += nwave) {
        float4* row = reinterpret_cast<float4*>(data + r * row_len);
        if constexpr (KIND == kLpFP8) {
            float amax = 0.f;
            for (int i = lane; i < n4; i += kWave) {
                const float4 v = row[i];
                amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
            }
            amax = group_allmax<kWave>(amax);
            const float inv = amax > 0.f ? 448.0f / amax : 0.f;
            const float scale = amax / 448.0f;
            for (int i = lane; i < n4; i += kWave) {
                const float4 d = e4m3x4_to_f32x4(f32x4_to_e4m3x4(row[i], inv));
                row[i] = make_float4(d.x * scale, d.y * scale, d.z * scale, d.w * scale);
            }
            if (row_scale && lane == 0) row_scale[r] = scale;
        } else {
            for (int i = lane; i < n4; i += kWave) {
                const float4 v = row[i];
                row[i] = (KIND == kLpBF16) ? round_bf16x4(v) : round_f16x4(v);
            }
        }
    }
}

hipError_t launch_emulate_precision(float* data, int64_t rows, int32_t row_len, int kind, float* row_scale,
                                    hipStream_t stream) {
    if (rows == 0) return hipSuccess;
    const void* fn = nullptr;
    if (kind == kLpBF16) fn = (const void*)&emulate_precision_kernel<kLpBF16>;
    if (kind == kLpF16) fn = (const void*)&emulate_precision_kernel<kLpF16>;
    if (kind == kLpFP8) fn = (const void*)&emulate_precision_kernel<kLpFP8>;
    if (!fn) return hipErrorInvalidValue;
    constexpr int64_t kRowsPerBlock = kEmuThreads / kWave;
    const int64_t want = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
    const unsigned blocks = (unsigned)(want < 8192 ? want : 8192);
    void* kargs[] = {&data, &rows, &row_len, &row_scale};
    return hipLaunchKernel(fn, dim3(blocks), dim3(kEmuThreads), kargs, 0, stream);
}

}  // namespace rssm
