// Compiled (headdim, dstate) combinations of the Mamba2 kernels, and the names of the
// per-slice lookup functions defined by mamba2_inst.hip.
#pragma once

#define RSSM_SHAPES(X)                                                                   \
    X(16, 16) X(32, 16) X(64, 16) X(128, 16) X(16, 32) X(32, 32) X(64, 32) X(128, 32)    \
    X(16, 64) X(32, 64) X(64, 64) X(128, 64) X(16, 128) X(32, 128) X(64, 128) X(128, 128) \
    X(16, 256) X(32, 256) X(64, 256)

#define RSSM_CAT3(a, b, c) a##b##c
#define RSSM_CAT5(a, b, c, d, e) a##b##c##d##e
#define RSSM_REPLAY_PTR_NAME(io, part) RSSM_CAT5(replay_kernel_ptr_io, io, _mode, part, )
#define RSSM_CONV_PTR_NAME(io) RSSM_CAT3(conv_kernel_ptr_io, io, )

namespace rssm {
const void* replay_kernel_ptr_io0_mode0(int P, int N, bool lowp);
const void* replay_kernel_ptr_io0_mode1(int P, int N, bool lowp);
const void* replay_kernel_ptr_io0_mode2(int P, int N, bool lowp);
const void* replay_kernel_ptr_io0_mode3(int P, int N, bool lowp);
const void* replay_kernel_ptr_io1_mode0(int P, int N, bool lowp);
const void* replay_kernel_ptr_io1_mode1(int P, int N, bool lowp);
const void* replay_kernel_ptr_io1_mode2(int P, int N, bool lowp);
const void* replay_kernel_ptr_io1_mode3(int P, int N, bool lowp);
const void* conv_kernel_ptr_io0(int P, int N, bool snap);
const void* conv_kernel_ptr_io1(int P, int N, bool snap);
}  // namespace rssm
