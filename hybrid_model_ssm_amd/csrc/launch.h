// Internal interface between the C-ABI layer (api.cpp) and the kernel translation units.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace rssm {

enum IoType { kIoF32 = 0, kIoBF16 = 1 };

struct Mamba2Args {
    float* ckpt;          // [B,H,P,N] f32
    void* ckpt_lp;        // [B,H,P,N] low-precision read copy (bf16, fp16 or fp8) or null
    float* lp_scale;      // [B,H,P] row scales of an fp8 copy
    void* rec_x;          // [B,H,L,P] io
    void* rec_B;          // [B,G,L,N] io
    float* rec_dt;        // [B,L,H]
    const int32_t* cursor_in;   // AR cursor, or the speculative head
    int32_t* cursor_out;        // AR only
    const int32_t* committed;   // speculative only
    int32_t* flushed;           // speculative only
    const void* x;        // [B,(T,)H,P]
    const void* z;        // [B,(T,)H,P]
    const void* B;        // [B,(T,)G,N]
    const void* C;        // [B,(T,)G,N]
    const void* dt_raw;   // [B,(T,)H]
    const float* dt_bias; // [H]
    const float* A;       // [H]
    const float* D;       // [H]
    float* out;           // [B,(T,)H,P]
    int32_t* err_flags;
    int32_t batch, nheads, headdim, dstate, ngroups, L, dt_softplus, n_pos;
    int32_t nchunk;       // workgroups per (sequence, group)
    int32_t heads_per_chunk;
    const int32_t* slot;       // state row of each batch row (-1: pad), or null (identity)
    int32_t num_slots;         // rows of the state arrays when slot is set
    const int32_t* n_pos_seq;  // speculative: positions of each sequence, or null (n_pos)
};

// Conventional read-update-write step (and the per-position snapshot baseline).
struct Mamba2ConvArgs {
    float* state;           // [B,H,P,N], or snapshots [B,T,H,P,N]
    const int32_t* slot_in; // snapshot baseline only
    const void* x;
    const void* z;
    const void* B;
    const void* C;
    const void* dt_raw;
    const float* dt_bias;
    const float* A;
    const float* D;
    float* out;
    int32_t batch, nheads, headdim, dstate, ngroups, dt_softplus, n_pos;
};

struct GdnArgs {
    float* ckpt;          // [B,HV,dv,dk]
    void* rec_k;          // [B,HK,L,dk]
    void* rec_v;          // [B,HV,L,dv]
    float* rec_alpha;     // [B,L,HV]
    float* rec_beta;      // [B,L,HV]
    const int32_t* cursor_in;   // AR cursor, or the speculative head
    int32_t* cursor_out;        // AR only
    const int32_t* committed;   // speculative only
    int32_t* flushed;           // speculative only
    const void* q;        // [B,(T,)HK,dk]
    const void* k;        // [B,(T,)HK,dk]
    const void* v;        // [B,(T,)HV,dv]
    const float* alpha;   // [B,(T,)HV]
    const float* beta;    // [B,(T,)HV]
    float* out;           // [B,(T,)HV,dv]
    int32_t* err_flags;
    int32_t batch, hv, hk, dk, dv, L, n_pos;
    float scale;
    int32_t nchunk;            // workgroups per (sequence, q/k head)
    int32_t vheads_per_chunk;
    const int32_t* slot;       // state row of each batch row (-1: pad), or null (identity)
    int32_t num_slots;
    const int32_t* n_pos_seq;  // speculative: positions of each sequence, or null (n_pos)
};

bool mamba2_shape_supported(int headdim, int dstate);
// 0 when the replay kernel cannot take this (headdim, dstate, nheads/ngroups, L, n_pos)
size_t mamba2_replay_smem_bytes(int headdim, int dstate, int heads_per_group, int L, int n_pos,
                                int io_bytes);
size_t mamba2_max_smem_bytes();

// mode: 0 = AR decode step, 1 = fold stored records only (flush), 2 = speculative verify,
//       3 = AR decode step by the state-and-output route
// lp: kind of read copy (0 none, 1 bf16, 2 fp16, 3 fp8 with row scales)
hipError_t launch_mamba2_replay(const Mamba2Args& a, int io, int lp, int mode, hipStream_t stream);
hipError_t launch_mamba2_conventional(const Mamba2ConvArgs& a, int io, bool snapshots,
                                      hipStream_t stream);

hipError_t launch_commit(int32_t batch, int32_t L, int32_t n_pos, int32_t* head,
                         int32_t* committed, const int32_t* flushed, const int32_t* n_keep,
                         const int32_t* n_pos_seq, int32_t* err_flags, hipStream_t stream);
hipError_t launch_reset(int32_t batch, int32_t* head, int32_t* cursor, const int32_t* seq_idx,
                        int32_t n_seq, hipStream_t stream);

bool gdn_shape_supported(int dk, int dv);
size_t gdn_smem_bytes(int dk, int dv, int L, int heads_ratio, int mode, int n_pos, int io_bytes);
// mode: 0 = AR decode, 1 = fold stored records only, 2 = speculative verify
hipError_t launch_gdn_replay(const GdnArgs& a, int io, int mode, hipStream_t stream);
// snapshots: per-position snapshot baseline (ckpt = snapshots, cursor_in = slot_in)
hipError_t launch_gdn_conventional(const GdnArgs& a, int io, bool snapshots, hipStream_t stream);

// round rows of an fp32 array in place to the values of a narrower format
// (kind as lp: 1 bf16, 2 fp16, 3 fp8 with row scales, written to row_scale if set)
hipError_t launch_emulate_precision(float* data, int64_t rows, int32_t row_len, int kind, float* row_scale,
                                    hipStream_t stream);

}  // namespace rssm
