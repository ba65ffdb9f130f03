// C ABI of libreplayssm: host-side validation and kernel dispatch.
// Every check runs before the first HIP call; a failed check launches nothing.

#include <stdint.h>

#include <climits>

#include "../../include/replayssm.h"
#include "launch.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

#define REQ(cond)                                          \
    do {                                                   \
        if (!(cond)) return REPLAYSSM_ERR_INVALID_ARGUMENT; \
    } while (0)

replayssm_status hip_status(hipError_t e) { return e == hipSuccess ? REPLAYSSM_OK : REPLAYSSM_ERR_HIP; }

size_t io_size(replayssm_dtype t) { return t == REPLAYSSM_BF16 ? 2 : 4; }

replayssm_status check_mamba2_desc(const replayssm_mamba2_desc* d, bool need_L) {
    REQ(d != nullptr);
    REQ(d->batch >= 1 && d->nheads >= 1 && d->ngroups >= 1 && d->headdim >= 1 && d->dstate >= 1);
    REQ(d->nheads % d->ngroups == 0);
    REQ(d->io_dtype == REPLAYSSM_F32 || d->io_dtype == REPLAYSSM_BF16);
    if (need_L) REQ(d->buffer_len >= 1 && d->buffer_len <= REPLAYSSM_MAX_BUFFER_LEN);
    REQ((int64_t)d->batch * d->nheads <= INT_MAX / REPLAYSSM_MAX_BUFFER_LEN);
    if (!rssm::mamba2_shape_supported(d->headdim, d->dstate)) return REPLAYSSM_ERR_UNSUPPORTED;
    return REPLAYSSM_OK;
}

replayssm_status check_mamba2_state(const replayssm_mamba2_desc* d, const replayssm_mamba2_state* s) {
    REQ(s != nullptr);
    REQ(s->ckpt && s->rec_x && s->rec_B && s->rec_dt);
    REQ(aligned(s->ckpt, 16) && aligned(s->rec_x, 16) && aligned(s->rec_B, 16) && aligned(s->rec_dt, 4));
    REQ(s->ckpt_lp == nullptr || aligned(s->ckpt_lp, 16));
    REQ(s->ckpt_lp != (void*)s->ckpt);
    if (s->slot != nullptr) {
        REQ(aligned(s->slot, 4) && s->num_slots >= 1);
        REQ((int64_t)s->num_slots * d->nheads <= INT_MAX / REPLAYSSM_MAX_BUFFER_LEN);
    }
    if (s->ckpt_lp != nullptr) {
        REQ(s->lp_dtype == REPLAYSSM_BF16 || s->lp_dtype == REPLAYSSM_F16 || s->lp_dtype == REPLAYSSM_FP8_E4M3);
        if (s->lp_dtype == REPLAYSSM_FP8_E4M3) {
            REQ(s->lp_scale != nullptr && aligned(s->lp_scale, 4));
            if (d->dstate % 16 != 0) return REPLAYSSM_ERR_UNSUPPORTED;
        }
    }
    return REPLAYSSM_OK;
}

replayssm_status check_mamba2_inputs(const replayssm_mamba2_desc* d, const void* x, const void* z,
                                     const void* B, const void* C, const void* dt_raw,
                                     const float* dt_bias, const float* A, const float* D,
                                     const float* out) {
    REQ(x && z && B && C && dt_raw && dt_bias && A && D && out);
    REQ(aligned(x, 16) && aligned(z, 16) && aligned(B, 16) && aligned(C, 16));
    REQ(aligned(dt_raw, io_size(d->io_dtype)) && aligned(dt_bias, 4) && aligned(A, 4) &&
        aligned(D, 4) && aligned(out, 4));
    return REPLAYSSM_OK;
}

// kind of read copy for the kernels: 0 none, 1 bf16, 2 fp16, 3 fp8
int lp_kind(const replayssm_mamba2_state* s) {
    if (s->ckpt_lp == nullptr) return 0;
    return s->lp_dtype == REPLAYSSM_BF16 ? 1 : s->lp_dtype == REPLAYSSM_F16 ? 2 : 3;
}

// The replay kernel stages one head's window and the group's records in LDS.
bool replay_fits(const replayssm_mamba2_desc* d, int n_pos) {
    const size_t bytes = rssm::mamba2_replay_smem_bytes(d->headdim, d->dstate, d->nheads / d->ngroups,
                                                        d->buffer_len, n_pos, d->io_dtype == REPLAYSSM_BF16 ? 2 : 4);
    return bytes > 0 && bytes <= rssm::mamba2_max_smem_bytes();
}

rssm::Mamba2Args mamba2_args(const replayssm_mamba2_desc* d, const replayssm_mamba2_state* s) {
    rssm::Mamba2Args a{};
    a.ckpt = s->ckpt;
    a.ckpt_lp = s->ckpt_lp;
    a.lp_scale = s->lp_scale;
    a.slot = s->slot;
    a.num_slots = s->num_slots;
    a.rec_x = s->rec_x;
    a.rec_B = s->rec_B;
    a.rec_dt = s->rec_dt;
    a.batch = d->batch;
    a.nheads = d->nheads;
    a.headdim = d->headdim;
    a.dstate = d->dstate;
    a.ngroups = d->ngroups;
    a.L = d->buffer_len;
    a.dt_softplus = d->dt_softplus ? 1 : 0;
    return a;
}

replayssm_status check_gdn_desc(const replayssm_gdn_desc* d, bool need_L) {
    REQ(d != nullptr);
    REQ(d->batch >= 1 && d->num_v_heads >= 1 && d->num_k_heads >= 1 && d->dk >= 1 && d->dv >= 1);
    REQ(d->num_v_heads % d->num_k_heads == 0);
    REQ(d->io_dtype == REPLAYSSM_F32 || d->io_dtype == REPLAYSSM_BF16);
    REQ(d->scale >= 0.0f && d->scale < 1e30f);
    if (need_L) REQ(d->buffer_len >= 1 && d->buffer_len <= REPLAYSSM_MAX_BUFFER_LEN);
    REQ((int64_t)d->batch * d->num_v_heads * 2 <= INT_MAX / REPLAYSSM_MAX_BUFFER_LEN);
    if (!rssm::gdn_shape_supported(d->dk, d->dv)) return REPLAYSSM_ERR_UNSUPPORTED;
    return REPLAYSSM_OK;
}

replayssm_status check_gdn_state(const replayssm_gdn_desc* d, const replayssm_gdn_state* s) {
    REQ(s && s->ckpt && s->rec_k && s->rec_v && s->rec_alpha && s->rec_beta);
    REQ(aligned(s->ckpt, 16) && aligned(s->rec_k, 16) && aligned(s->rec_v, 16) &&
        aligned(s->rec_alpha, 4) && aligned(s->rec_beta, 4));
    if (s->slot != nullptr) {
        REQ(aligned(s->slot, 4) && s->num_slots >= 1);
        REQ((int64_t)s->num_slots * d->num_v_heads * 2 <= INT_MAX / REPLAYSSM_MAX_BUFFER_LEN);
    }
    return REPLAYSSM_OK;
}

replayssm_status check_gdn_inputs(const void* q, const void* k, const void* v, const float* alpha,
                                  const float* beta, const float* out) {
    REQ(q && k && v && alpha && beta && out);
    REQ(aligned(q, 16) && aligned(k, 16) && aligned(v, 16) && aligned(alpha, 4) && aligned(beta, 4) &&
        aligned(out, 4));
    return REPLAYSSM_OK;
}

// whether the replay kernel's LDS staging of one workgroup fits
bool gdn_fits(const replayssm_gdn_desc* d, int mode, int n_pos) {
    return rssm::gdn_smem_bytes(d->dk, d->dv, d->buffer_len, d->num_v_heads / d->num_k_heads, mode, n_pos,
                                d->io_dtype == REPLAYSSM_BF16 ? 2 : 4) <= rssm::mamba2_max_smem_bytes();
}

rssm::GdnArgs gdn_args(const replayssm_gdn_desc* d, const replayssm_gdn_state* s) {
    rssm::GdnArgs a{};
    if (s) {
        a.ckpt = s->ckpt; a.rec_k = s->rec_k; a.rec_v = s->rec_v;
        a.rec_alpha = s->rec_alpha; a.rec_beta = s->rec_beta;
        a.slot = s->slot; a.num_slots = s->num_slots;
    }
    a.batch = d->batch;
    a.hv = d->num_v_heads;
    a.hk = d->num_k_heads;
    a.dk = d->dk;
    a.dv = d->dv;
    a.L = d->buffer_len;
    a.scale = d->scale > 0.0f ? d->scale : 1.0f / __builtin_sqrtf((float)d->dk);
    return a;
}

}  // namespace

// One autoregressive decode step; mode 0 is the output-only route, mode 3 the
// state-and-output route (same arguments, same cursor and record rules).
static replayssm_status mamba2_decode_route(int mode, const replayssm_mamba2_desc* desc,
                                            const replayssm_mamba2_state* state,
                                            const int32_t* cursor_in, int32_t* cursor_out,
                                            const void* x, const void* z, const void* B,
                                            const void* C, const void* dt_raw, const float* dt_bias,
                                            const float* A, const float* D, float* out,
                                            int32_t* err_flags, hipStream_t stream) {
    replayssm_status st = check_mamba2_desc(desc, true);
    if (st != REPLAYSSM_OK) return st;
    if ((st = check_mamba2_state(desc, state)) != REPLAYSSM_OK) return st;
    if ((st = check_mamba2_inputs(desc, x, z, B, C, dt_raw, dt_bias, A, D, out)) != REPLAYSSM_OK) return st;
    REQ(cursor_in && cursor_out && cursor_in != cursor_out);
    REQ(aligned(cursor_in, 4) && aligned(cursor_out, 4) && aligned(err_flags, 4));
    if (!replay_fits(desc, 0)) return REPLAYSSM_ERR_UNSUPPORTED;
    rssm::Mamba2Args a = mamba2_args(desc, state);
    a.cursor_in = cursor_in;
    a.cursor_out = cursor_out;
    a.x = x; a.z = z; a.B = B; a.C = C; a.dt_raw = dt_raw;
    a.dt_bias = dt_bias; a.A = A; a.D = D; a.out = out; a.err_flags = err_flags;
    a.n_pos = 1;
    return hip_status(rssm::launch_mamba2_replay(a, desc->io_dtype, lp_kind(state), mode, stream));
}

extern "C" {

const char* replayssm_status_string(replayssm_status status) {
    switch (status) {
        case REPLAYSSM_OK: return "ok";
        case REPLAYSSM_ERR_INVALID_ARGUMENT: return "invalid argument";
        case REPLAYSSM_ERR_UNSUPPORTED: return "unsupported shape";
        case REPLAYSSM_ERR_HIP: return "HIP launch failure";
    }
    return "unknown status";
}

int32_t replayssm_version(void) { return 300; }

replayssm_status replayssm_mamba2_decode(const replayssm_mamba2_desc* desc,
                                         const replayssm_mamba2_state* state,
                                         const int32_t* cursor_in, int32_t* cursor_out,
                                         const void* x, const void* z, const void* B,
                                         const void* C, const void* dt_raw, const float* dt_bias,
                                         const float* A, const float* D, float* out,
                                         int32_t* err_flags, hipStream_t stream) {
    return mamba2_decode_route(0, desc, state, cursor_in, cursor_out, x, z, B, C, dt_raw, dt_bias, A, D, out,
                               err_flags, stream);
}

replayssm_status replayssm_mamba2_decode_state_and_output(const replayssm_mamba2_desc* desc,
                                                          const replayssm_mamba2_state* state,
                                                          const int32_t* cursor_in, int32_t* cursor_out,
                                                          const void* x, const void* z, const void* B,
                                                          const void* C, const void* dt_raw,
                                                          const float* dt_bias, const float* A,
                                                          const float* D, float* out, int32_t* err_flags,
                                                          hipStream_t stream) {
    return mamba2_decode_route(3, desc, state, cursor_in, cursor_out, x, z, B, C, dt_raw, dt_bias, A, D, out,
                               err_flags, stream);
}

replayssm_status replayssm_mamba2_flush(const replayssm_mamba2_desc* desc,
                                        const replayssm_mamba2_state* state,
                                        const int32_t* cursor_in, int32_t* cursor_out,
                                        const float* A, int32_t* err_flags, hipStream_t stream) {
    replayssm_status st = check_mamba2_desc(desc, true);
    if (st != REPLAYSSM_OK) return st;
    if ((st = check_mamba2_state(desc, state)) != REPLAYSSM_OK) return st;
    REQ(A && aligned(A, 4));
    REQ(cursor_in && cursor_out && cursor_in != cursor_out);
    REQ(aligned(cursor_in, 4) && aligned(cursor_out, 4) && aligned(err_flags, 4));
    if (!replay_fits(desc, 0)) return REPLAYSSM_ERR_UNSUPPORTED;
    rssm::Mamba2Args a = mamba2_args(desc, state);
    a.cursor_in = cursor_in;
    a.cursor_out = cursor_out;
    a.A = A;
    a.err_flags = err_flags;
    a.n_pos = 0;
    return hip_status(rssm::launch_mamba2_replay(a, desc->io_dtype, lp_kind(state), 1, stream));
}

replayssm_status replayssm_mamba2_spec_verify(const replayssm_mamba2_desc* desc,
                                              const replayssm_mamba2_state* state,
                                              const int32_t* head, const int32_t* committed,
                                              int32_t n_pos, const int32_t* n_pos_seq, const void* x,
                                              const void* z,
                                              const void* B, const void* C, const void* dt_raw,
                                              const float* dt_bias, const float* A, const float* D,
                                              float* out, int32_t* flushed, int32_t* err_flags,
                                              hipStream_t stream) {
    replayssm_status st = check_mamba2_desc(desc, true);
    if (st != REPLAYSSM_OK) return st;
    if ((st = check_mamba2_state(desc, state)) != REPLAYSSM_OK) return st;
    if ((st = check_mamba2_inputs(desc, x, z, B, C, dt_raw, dt_bias, A, D, out)) != REPLAYSSM_OK) return st;
    REQ(n_pos >= 1 && n_pos <= desc->buffer_len);
    REQ((int64_t)desc->batch * n_pos * desc->nheads <= INT_MAX / 2);
    REQ(head && committed && flushed && head != committed);
    REQ((const int32_t*)flushed != head && (const int32_t*)flushed != committed);
    REQ(aligned(head, 4) && aligned(committed, 4) && aligned(flushed, 4) && aligned(err_flags, 4));
    REQ(aligned(n_pos_seq, 4));
    if (!replay_fits(desc, n_pos)) return REPLAYSSM_ERR_UNSUPPORTED;
    rssm::Mamba2Args a = mamba2_args(desc, state);
    a.cursor_in = head;
    a.committed = committed;
    a.flushed = flushed;
    a.n_pos_seq = n_pos_seq;
    a.x = x; a.z = z; a.B = B; a.C = C; a.dt_raw = dt_raw;
    a.dt_bias = dt_bias; a.A = A; a.D = D; a.out = out; a.err_flags = err_flags;
    a.n_pos = n_pos;
    return hip_status(rssm::launch_mamba2_replay(a, desc->io_dtype, lp_kind(state), 2, stream));
}

replayssm_status replayssm_commit(int32_t batch, int32_t buffer_len, int32_t n_pos, int32_t* head,
                                  int32_t* committed, const int32_t* flushed, const int32_t* n_keep,
                                  const int32_t* n_pos_seq, int32_t* err_flags, hipStream_t stream) {
    REQ(batch >= 1 && buffer_len >= 1 && buffer_len <= REPLAYSSM_MAX_BUFFER_LEN);
    REQ(n_pos >= 1 && n_pos <= buffer_len);
    REQ(head && committed && flushed && n_keep && head != committed);
    REQ(aligned(head, 4) && aligned(committed, 4) && aligned(flushed, 4) && aligned(n_keep, 4) &&
        aligned(err_flags, 4) && aligned(n_pos_seq, 4));
    return hip_status(rssm::launch_commit(batch, buffer_len, n_pos, head, committed, flushed, n_keep,
                                          n_pos_seq, err_flags, stream));
}

replayssm_status replayssm_reset_cursors(int32_t batch, int32_t* head, int32_t* cursor,
                                         const int32_t* seq_idx, int32_t n_seq, hipStream_t stream) {
    REQ(batch >= 1 && cursor && head != cursor);
    REQ(aligned(head, 4) && aligned(cursor, 4) && aligned(seq_idx, 4));
    if (seq_idx == nullptr) n_seq = batch;
    REQ(n_seq >= 0);
    return hip_status(rssm::launch_reset(batch, head, cursor, seq_idx, n_seq, stream));
}

replayssm_status replayssm_selective_state_update(const replayssm_mamba2_desc* desc, float* state,
                                                  const void* x, const void* z, const void* B,
                                                  const void* C, const void* dt_raw,
                                                  const float* dt_bias, const float* A,
                                                  const float* D, float* out, hipStream_t stream) {
    replayssm_status st = check_mamba2_desc(desc, false);
    if (st != REPLAYSSM_OK) return st;
    if ((st = check_mamba2_inputs(desc, x, z, B, C, dt_raw, dt_bias, A, D, out)) != REPLAYSSM_OK) return st;
    REQ(state && aligned(state, 16));
    rssm::Mamba2ConvArgs a{};
    a.state = state;
    a.x = x; a.z = z; a.B = B; a.C = C; a.dt_raw = dt_raw;
    a.dt_bias = dt_bias; a.A = A; a.D = D; a.out = out;
    a.batch = desc->batch; a.nheads = desc->nheads; a.headdim = desc->headdim;
    a.dstate = desc->dstate; a.ngroups = desc->ngroups; a.dt_softplus = desc->dt_softplus ? 1 : 0;
    a.n_pos = 1;
    return hip_status(rssm::launch_mamba2_conventional(a, desc->io_dtype, false, stream));
}

replayssm_status replayssm_mamba2_spec_baseline(const replayssm_mamba2_desc* desc, float* snapshots,
                                                const int32_t* slot_in, int32_t n_pos,
                                                const void* x, const void* z, const void* B,
                                                const void* C, const void* dt_raw,
                                                const float* dt_bias, const float* A,
                                                const float* D, float* out, hipStream_t stream) {
    replayssm_status st = check_mamba2_desc(desc, false);
    if (st != REPLAYSSM_OK) return st;
    if ((st = check_mamba2_inputs(desc, x, z, B, C, dt_raw, dt_bias, A, D, out)) != REPLAYSSM_OK) return st;
    REQ(snapshots && aligned(snapshots, 16) && slot_in && aligned(slot_in, 4));
    REQ(n_pos >= 1 && n_pos <= REPLAYSSM_MAX_BUFFER_LEN);
    REQ((int64_t)desc->batch * n_pos * desc->nheads <= INT_MAX / 2);
    rssm::Mamba2ConvArgs a{};
    a.state = snapshots;
    a.slot_in = slot_in;
    a.x = x; a.z = z; a.B = B; a.C = C; a.dt_raw = dt_raw;
    a.dt_bias = dt_bias; a.A = A; a.D = D; a.out = out;
    a.batch = desc->batch; a.nheads = desc->nheads; a.headdim = desc->headdim;
    a.dstate = desc->dstate; a.ngroups = desc->ngroups; a.dt_softplus = desc->dt_softplus ? 1 : 0;
    a.n_pos = n_pos;
    return hip_status(rssm::launch_mamba2_conventional(a, desc->io_dtype, true, stream));
}

replayssm_status replayssm_gdn_decode(const replayssm_gdn_desc* desc, const replayssm_gdn_state* state,
                                      const int32_t* cursor_in, int32_t* cursor_out, const void* q,
                                      const void* k, const void* v, const float* alpha,
                                      const float* beta, float* out, int32_t* err_flags,
                                      hipStream_t stream) {
    replayssm_status st = check_gdn_desc(desc, true);
    if (st != REPLAYSSM_OK) return st;
    if ((st = check_gdn_state(desc, state)) != REPLAYSSM_OK) return st;
    if ((st = check_gdn_inputs(q, k, v, alpha, beta, out)) != REPLAYSSM_OK) return st;
    REQ(cursor_in && cursor_out && cursor_in != cursor_out);
    REQ(aligned(cursor_in, 4) && aligned(cursor_out, 4) && aligned(err_flags, 4));
    if (!gdn_fits(desc, 0, 1)) return REPLAYSSM_ERR_UNSUPPORTED;
    rssm::GdnArgs a = gdn_args(desc, state);
    a.cursor_in = cursor_in; a.cursor_out = cursor_out;
    a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta; a.out = out; a.err_flags = err_flags;
    return hip_status(rssm::launch_gdn_replay(a, desc->io_dtype, 0, stream));
}

replayssm_status replayssm_gdn_flush(const replayssm_gdn_desc* desc, const replayssm_gdn_state* state,
                                     const int32_t* cursor_in, int32_t* cursor_out, int32_t* err_flags,
                                     hipStream_t stream) {
    replayssm_status st = check_gdn_desc(desc, true);
    if (st != REPLAYSSM_OK) return st;
    if ((st = check_gdn_state(desc, state)) != REPLAYSSM_OK) return st;
    REQ(cursor_in && cursor_out && cursor_in != cursor_out);
    REQ(aligned(cursor_in, 4) && aligned(cursor_out, 4) && aligned(err_flags, 4));
    if (!gdn_fits(desc, 1, 0)) return REPLAYSSM_ERR_UNSUPPORTED;
    rssm::GdnArgs a = gdn_args(desc, state);
    a.cursor_in = cursor_in; a.cursor_out = cursor_out; a.err_flags = err_flags;
    return hip_status(rssm::launch_gdn_replay(a, desc->io_dtype, 1, stream));
}

replayssm_status replayssm_gdn_spec_verify(const replayssm_gdn_desc* desc, const replayssm_gdn_state* state,
                                           const int32_t* head, const int32_t* committed, int32_t n_pos,
                                           const int32_t* n_pos_seq, const void* q, const void* k,
                                           const void* v, const float* alpha, const float* beta, float* out,
                                           int32_t* flushed, int32_t* err_flags, hipStream_t stream) {
    replayssm_status st = check_gdn_desc(desc, true);
    if (st != REPLAYSSM_OK) return st;
    if ((st = check_gdn_state(desc, state)) != REPLAYSSM_OK) return st;
    if ((st = check_gdn_inputs(q, k, v, alpha, beta, out)) != REPLAYSSM_OK) return st;
    REQ(n_pos >= 1 && n_pos <= desc->buffer_len);
    REQ((int64_t)desc->batch * n_pos * desc->num_v_heads <= INT_MAX / 2);
    REQ(head && committed && flushed && head != committed);
    REQ((const int32_t*)flushed != head && (const int32_t*)flushed != committed);
    REQ(aligned(head, 4) && aligned(committed, 4) && aligned(flushed, 4) && aligned(err_flags, 4));
    REQ(aligned(n_pos_seq, 4));
    if (!gdn_fits(desc, 2, n_pos)) return REPLAYSSM_ERR_UNSUPPORTED;
    rssm::GdnArgs a = gdn_args(desc, state);
    a.cursor_in = head;
    a.committed = committed;
    a.flushed = flushed;
    a.n_pos_seq = n_pos_seq;
    a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta; a.out = out; a.err_flags = err_flags;
    a.n_pos = n_pos;
    return hip_status(rssm::launch_gdn_replay(a, desc->io_dtype, 2, stream));
}

replayssm_status replayssm_gdn_conventional_decode(const replayssm_gdn_desc* desc, float* state,
                                                   const void* q, const void* k, const void* v,
                                                   const float* alpha, const float* beta,
                                                   float* out, hipStream_t stream) {
    replayssm_status st = check_gdn_desc(desc, false);
    if (st != REPLAYSSM_OK) return st;
    REQ(state && aligned(state, 16));
    if ((st = check_gdn_inputs(q, k, v, alpha, beta, out)) != REPLAYSSM_OK) return st;
    rssm::GdnArgs a = gdn_args(desc, nullptr);
    a.ckpt = state;
    a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta; a.out = out;
    return hip_status(rssm::launch_gdn_conventional(a, desc->io_dtype, false, stream));
}

replayssm_status replayssm_gdn_spec_baseline(const replayssm_gdn_desc* desc, float* snapshots,
                                             const int32_t* slot_in, int32_t n_pos, const void* q,
                                             const void* k, const void* v, const float* alpha,
                                             const float* beta, float* out, hipStream_t stream) {
    replayssm_status st = check_gdn_desc(desc, false);
    if (st != REPLAYSSM_OK) return st;
    REQ(snapshots && aligned(snapshots, 16) && slot_in && aligned(slot_in, 4));
    if ((st = check_gdn_inputs(q, k, v, alpha, beta, out)) != REPLAYSSM_OK) return st;
    REQ(n_pos >= 1 && n_pos <= REPLAYSSM_MAX_BUFFER_LEN);
    REQ((int64_t)desc->batch * n_pos * desc->num_v_heads <= INT_MAX / 2);
    rssm::GdnArgs a = gdn_args(desc, nullptr);
    a.ckpt = snapshots;
    a.cursor_in = slot_in;
    a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta; a.out = out;
    a.n_pos = n_pos;
    return hip_status(rssm::launch_gdn_conventional(a, desc->io_dtype, true, stream));
}

replayssm_status replayssm_emulate_precision(float* data, int64_t rows, int32_t row_len,
                                             replayssm_dtype dtype, float* row_scale, hipStream_t stream) {
    REQ(rows >= 0 && row_len >= 4 && row_len % 4 == 0);
    REQ(dtype == REPLAYSSM_F32 || dtype == REPLAYSSM_BF16 || dtype == REPLAYSSM_F16 ||
        dtype == REPLAYSSM_FP8_E4M3);
    REQ(aligned(data, 16) && aligned(row_scale, 4));
    REQ(data || rows == 0);
    if (dtype == REPLAYSSM_F32 || rows == 0) return REPLAYSSM_OK;
    const int kind = dtype == REPLAYSSM_BF16 ? 1 : dtype == REPLAYSSM_F16 ? 2 : 3;
    return hip_status(rssm::launch_emulate_precision(data, rows, row_len, kind, row_scale, stream));
}

}  // extern "C"
