// Instantiates one slice of the Mamba2 kernel templates so that the slices compile in
// parallel.  Built several times with RSSM_IO (0: f32 io, 1: bf16 io), RSSM_PART
// (0..3: replay kernel mode, 4: conventional kernels) and, for the replay kernel,
// RSSM_LP (kind of low-precision read copy, 0..3).
#include "mamba2_kernels.h"
#include "mamba2_shapes.h"

#ifndef RSSM_IO
#error "RSSM_IO must be defined"
#endif
#ifndef RSSM_PART
#error "RSSM_PART must be defined"
#endif

namespace rssm {

#if RSSM_IO == 1
using InstIo = uint16_t;
#else
using InstIo = float;
#endif

#if RSSM_PART < 4
#ifndef RSSM_LP
#error "RSSM_LP must be defined"
#endif
const void* RSSM_REPLAY_PTR_NAME(RSSM_IO, RSSM_PART, RSSM_LP)(int P, int N) {
#define X(PP, NN) \
    if (P == PP && N == NN) return (const void*)&mamba2_replay_kernel<PP, NN, InstIo, RSSM_LP, RSSM_PART>;
    RSSM_SHAPES(X)
#undef X
    return nullptr;
}
#else
const void* RSSM_CONV_PTR_NAME(RSSM_IO)(int P, int N, bool snap) {
#define X(PP, NN)                                                                          \
    if (P == PP && N == NN)                                                                \
        return snap ? (const void*)&mamba2_conventional_kernel<PP, NN, InstIo, true>      \
                    : (const void*)&mamba2_conventional_kernel<PP, NN, InstIo, false>;
    RSSM_SHAPES(X)
#undef X
    return nullptr;
}

#endif

}  // namespace rssm
