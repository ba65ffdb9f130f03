// Compiled (headdim, dstate) combinations of the Mamba2 kernels, and the names of the
// per-slice lookup functions defined by mamba2_inst.hip.
#pragma once

#define RSSM_SHAPES(X)                                                                   \
    X(16, 16) X(32, 16) X(64, 16) X(128, 16) X(16, 32) X(32, 32) X(64, 32) X(128, 32)    \
    X(16, 64) X(32, 64) X(64, 64) X(128, 64) X(16, 128) X(32, 128) X(64, 128) X(128, 128) \
    X(16, 256) X(32, 256) X(64, 256)

#define RSSM_CAT3(a, b, c) a##b##c
#define RSSM_CAT7(a, b, c, d, e, f, g) a##b##c##d##e##f##g
#define RSSM_REPLAY_PTR_NAME(io, mode, lp) RSSM_CAT7(replay_kernel_ptr_io, io, _mode, mode, _lp, lp, )
#define RSSM_CONV_PTR_NAME(io) RSSM_CAT3(conv_kernel_ptr_io, io, )

// (io, mode, read copy) slices of the replay kernel
#define RSSM_REPLAY_SLICES(X)                                                           \
    X(0, 0, 0) X(0, 0, 1) X(0, 0, 2) X(0, 0, 3) X(0, 1, 0) X(0, 1, 1) X(0, 1, 2) X(0, 1, 3) \
    X(0, 2, 0) X(0, 2, 1) X(0, 2, 2) X(0, 2, 3) X(0, 3, 0) X(0, 3, 1) X(0, 3, 2) X(0, 3, 3) \
    X(1, 0, 0) X(1, 0, 1) X(1, 0, 2) X(1, 0, 3) X(1, 1, 0) X(1, 1, 1) X(1, 1, 2) X(1, 1, 3) \
    X(1, 2, 0) X(1, 2, 1) X(1, 2, 2) X(1, 2, 3) X(1, 3, 0) X(1, 3, 1) X(1, 3, 2) X(1, 3, 3)

namespace rssm {
#define RSSM_DECLARE_SLICE(io, mode, lp) const void* RSSM_REPLAY_PTR_NAME(io, mode, lp)(int P, int N);
RSSM_REPLAY_SLICES(RSSM_DECLARE_SLICE)
#undef RSSM_DECLARE_SLICE
const void* conv_kernel_ptr_io0(int P, int N, bool snap);
const void* conv_kernel_ptr_io1(int P, int N, bool snap);
}  // namespace rssm
