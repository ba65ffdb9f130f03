// Shape checks, LDS sizing and launches of the Mamba2 kernels.
#include "mamba2_kernels.h"
#include "mamba2_shapes.h"

namespace rssm {

// ---------------------------------------------------------------------------------------
// Dispatch over the compiled (dstate, rows-per-thread) set
// ---------------------------------------------------------------------------------------
bool mamba2_shape_supported(int P, int N) {
#define X(PP, NN) \
    if (P == PP && N == NN) return true;
    RSSM_SHAPES(X)
#undef X
    return false;
}

// Heads of one group per workgroup: all of them up to a cap, else chunks of the cap (the
// last chunk holds the remainder, at least one head).  Speculative rounds use the same
// cap as decode steps: a round folds in some sequences only, and the kernel starts the
// workgroups of those sequences first, so that the long folding workgroups do not run
// alone at the end of the launch (16 heads with that order measured 2.6% faster than 8
// heads in batch order; 16 heads in batch order 6% slower).
constexpr int kMaxHeadsPerWgSpec = 16;

static void chunking(int hpg, int mode, int* nchunk, int* hc) {
    const int cap = (mode == kSpec) ? kMaxHeadsPerWgSpec : kMaxHeadsPerWg;
    *hc = hpg < cap ? hpg : cap;
    *nchunk = (hpg + *hc - 1) / *hc;
}

size_t mamba2_replay_smem_bytes(int P, int N, int hpg, int L, int n_pos, int io_bytes) {
    const int mode = n_pos > 0 ? kSpec : kDecode;
    const int T = n_pos > 0 ? n_pos : 1;
    if (P * L > kFoldXPerThread * 4 * kThreads) return 0;   // fold rows of one head
    int nchunk, hc;
    chunking(hpg, mode, &nchunk, &hc);
    return sizeof(float) * (size_t)GroupSmem(P, N, L, T, hc, mode, io_bytes).total;
}

size_t mamba2_max_smem_bytes() { return 64 * 1024; }

static const void* find_replay(int P, int N, int io, int lp, int mode) {
#define RSSM_PICK(IO, MODE, LP) \
    if (io == IO && mode == MODE && lp == LP) return RSSM_REPLAY_PTR_NAME(IO, MODE, LP)(P, N);
    RSSM_REPLAY_SLICES(RSSM_PICK)
#undef RSSM_PICK
    return nullptr;
}

// rows of the state one conventional workgroup covers
static int conv_rows_per_wg(int P, int N) {
#define X(PP, NN) \
    if (P == PP && N == NN) return ConvShape<PP, NN>::RW;
    RSSM_SHAPES(X)
#undef X
    return 1;
}

static const void* find_conv(int P, int N, int io, bool snap) {
    return io == kIoBF16 ? conv_kernel_ptr_io1(P, N, snap) : conv_kernel_ptr_io0(P, N, snap);
}

hipError_t launch_mamba2_replay(const Mamba2Args& a, int io, int lp, int mode, hipStream_t stream) {
    const void* fn = find_replay(a.headdim, a.dstate, io, a.ckpt_lp != nullptr ? lp : 0, mode);
    if (!fn) return hipErrorInvalidValue;
    Mamba2Args args = a;
    chunking(a.nheads / a.ngroups, mode, &args.nchunk, &args.heads_per_chunk);
    const int T = mode == kSpec ? a.n_pos : (mode == kFold ? 0 : 1);
    const size_t smem = sizeof(float) * (size_t)GroupSmem(a.headdim, a.dstate, a.L, T, args.heads_per_chunk, mode,
                                                          io == kIoBF16 ? 2 : 4).total;
    void* kargs[] = {&args};
    const dim3 grid((unsigned)((size_t)a.batch * a.ngroups * args.nchunk));
    hipError_t e = hipLaunchKernel(fn, grid, dim3(kThreads), kargs, smem, stream);
    if (e != hipSuccess || mode != kSpec || args.nchunk == 1) return e;
    const size_t total = (size_t)a.batch * a.n_pos * a.ngroups * a.dstate;
    const size_t want = (total + kThreads - 1) / kThreads;
    const unsigned blocks = (unsigned)(want < 65536 ? want : 65536);
    const void* app = io == kIoBF16 ? (const void*)&mamba2_spec_append_B_kernel<uint16_t>
                                    : (const void*)&mamba2_spec_append_B_kernel<float>;
    return hipLaunchKernel(app, dim3(blocks), dim3(kThreads), kargs, 0, stream);
}

hipError_t launch_mamba2_conventional(const Mamba2ConvArgs& a, int io, bool snap, hipStream_t stream) {
    const void* fn = find_conv(a.headdim, a.dstate, io, snap);
    if (!fn) return hipErrorInvalidValue;
    Mamba2ConvArgs args = a;
    void* kargs[] = {&args};
    const int64_t rows = (int64_t)a.batch * a.nheads * a.headdim;
    const int64_t rows_per_wg = conv_rows_per_wg(a.headdim, a.dstate);
    const int64_t want = (rows + rows_per_wg - 1) / rows_per_wg;
    const dim3 grid((unsigned)(want < kConvMaxGrid ? want : kConvMaxGrid));
    return hipLaunchKernel(fn, grid, dim3(kThreads), kargs, 0, stream);
}

}  // namespace rssm
