// Cursor bookkeeping for speculative decoding on the circular record buffer
// ("ReplaySSM" README, benefit "Cheap rollback": rejected inputs are discarded by
// moving a buffer pointer; the checkpoint is never touched here).

#include "device_common.h"
#include "launch.h"

namespace rssm {

// A sequence with no positions this round (n_pos_seq[b] == 0: a pad row) is left as
// it is; otherwise 1 <= n_keep <= its positions.
__global__ void __launch_bounds__(256) commit_kernel(int32_t batch, int32_t L, int32_t n_pos,
                                                     int32_t* head, int32_t* committed,
                                                     const int32_t* flushed, const int32_t* n_keep,
                                                     const int32_t* n_pos_seq, int32_t* err_flags) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= batch) return;
    const int tb = n_pos_seq ? n_pos_seq[b] : n_pos;
    if (tb == 0) return;
    int hd = head[b], cm = committed[b];
    const int nk = n_keep[b];
    if (flushed[b]) {
        hd = (hd + cm) % L;
        cm = 0;
    }
    if (hd < 0 || hd >= L || cm < 0 || tb < 0 || tb > n_pos || nk < 1 || nk > tb || cm + nk > L) {
        if (err_flags) atomicOr(err_flags, kDevErrCursor);
        return;
    }
    head[b] = hd;
    committed[b] = cm + nk;
}

__global__ void __launch_bounds__(256) reset_kernel(int32_t batch, int32_t* head, int32_t* cursor,
                                                    const int32_t* seq_idx, int32_t n_seq) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n_seq) return;
    const int b = seq_idx ? seq_idx[i] : i;
    if (b < 0 || b >= batch) return;
    if (head) head[b] = 0;
    cursor[b] = 0;
}

hipError_t launch_commit(int32_t batch, int32_t L, int32_t n_pos, int32_t* head, int32_t* committed,
                         const int32_t* flushed, const int32_t* n_keep, const int32_t* n_pos_seq,
                         int32_t* err_flags, hipStream_t stream) {
    const unsigned blocks = (unsigned)((batch + 255) / 256);
    void* kargs[] = {&batch, &L, &n_pos, &head, &committed, (void*)&flushed, (void*)&n_keep,
                     (void*)&n_pos_seq, &err_flags};
    return hipLaunchKernel((const void*)&commit_kernel, dim3(blocks), dim3(256), kargs, 0, stream);
}

hipError_t launch_reset(int32_t batch, int32_t* head, int32_t* cursor, const int32_t* seq_idx,
                        int32_t n_seq, hipStream_t stream) {
    if (n_seq == 0) return hipSuccess;
    const unsigned blocks = (unsigned)((n_seq + 255) / 256);
    void* kargs[] = {&batch, &head, &cursor, (void*)&seq_idx, &n_seq};
    return hipLaunchKernel((const void*)&reset_kernel, dim3(blocks), dim3(256), kargs, 0, stream);
}

}  // namespace rssm
