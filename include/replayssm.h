/*
 * replayssm.h -- C ABI of the ReplaySSM decode library for AMD Instinct MI355X (gfx950).
 *
 * ReplaySSM keeps the recurrent state of a state-space (SSM) layer as a checkpoint
 * plus a bounded buffer of recent input records ("ReplaySSM Caches Inputs Instead of
 * State to Speed Up Hybrid-Model Decoding", section "How ReplaySSM works").  On a
 * non-flush step the kernel appends the step's record and evaluates the output from
 * the checkpoint plus the stored records, writing no state back; the step that brings
 * the buffer to L records merges them into the checkpoint, which it writes back
 * once.  Speculative verification appends draft records and is output-only; rollback
 * moves a cursor ("ReplaySSM" README, benefit "Cheap rollback").  An optional
 * low-precision read copy of the checkpoint (bf16, fp16 or fp8) serves non-flush reads
 * while the fp32 checkpoint carries the recurrence (same README, benefit "Separate
 * state precisions").  The
 * entry points follow the kernels listed in "ReplaySSM (a vLLM research fork)",
 * section "Core implementation files".
 *
 * Conventions (all entry points)
 * ------------------------------
 * - Every pointer argument is a DEVICE pointer owned by the caller, except the
 *   descriptor and state structs themselves, which are host memory read during the
 *   call only.  The library never allocates or frees memory, keeps no mutable
 *   global state and never synchronises: each call enqueues its kernels on `stream`
 *   and returns.  Buffers must stay alive until that stream work has finished.
 * - Arrays are dense and row-major with the last dimension contiguous, in the
 *   shapes written next to each argument ([batch, nheads, headdim] and so on).
 * - Alignment: the checkpoint and its read copy must be 16-byte aligned; every
 *   other array must be aligned to its element size.
 * - Errors: every entry point validates its arguments on the host before it touches
 *   the GPU.  On REPLAYSSM_ERR_INVALID_ARGUMENT or REPLAYSSM_ERR_UNSUPPORTED nothing
 *   is launched and nothing is written.  REPLAYSSM_ERR_HIP reports a launch failure
 *   (hipGetLastError) after the enqueue.
 * - Device-side errors: `err_flags` (may be NULL) points to one int32 word.  A
 *   kernel that meets a cursor or position count outside its documented range ORs
 *   REPLAYSSM_DEVERR_CURSOR into it (a state slot out of range: REPLAYSSM_DEVERR_SLOT),
 *   skips that sequence (its outputs, records and checkpoint are left untouched,
 *   flushed[b] = 0) and copies the cursor to the output cursor unchanged.  The
 *   caller clears the word.
 * - State slots (serving): a state struct may carry `slot`, a device array [batch]
 *   mapping each batch row to a row of the state arrays, which then have num_slots
 *   rows (a pool).  slot[b] == -1 marks a pad row: it is skipped like a bad one but
 *   without an error.  Inputs, outputs and cursors stay indexed by batch row.  Two
 *   batch rows must not name the same slot in one call.  slot == NULL is the
 *   identity (the state arrays have batch rows).
 * - Reentrancy: functions are reentrant and thread-safe; calls on one stream are
 *   ordered by the stream.
 * - Determinism: reductions use no atomics; the same inputs give bit-identical
 *   outputs.
 */
#ifndef REPLAYSSM_H
#define REPLAYSSM_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    REPLAYSSM_OK = 0,
    REPLAYSSM_ERR_INVALID_ARGUMENT = 1, /* null required pointer, bad size, misalignment, aliasing */
    REPLAYSSM_ERR_UNSUPPORTED = 2,      /* a shape outside the compiled set (see each call) */
    REPLAYSSM_ERR_HIP = 3               /* the HIP runtime rejected the launch */
} replayssm_status;

typedef enum {
    REPLAYSSM_F32 = 0,
    REPLAYSSM_BF16 = 1,
    REPLAYSSM_F16 = 2,      /* read copies and precision emulation only */
    REPLAYSSM_FP8_E4M3 = 3  /* read copies and precision emulation only: OCP 8-bit float
                               with a scale per row */
} replayssm_dtype;

enum { REPLAYSSM_DEVERR_CURSOR = 1, REPLAYSSM_DEVERR_SLOT = 2 };

/* Largest buffer length (window L) the kernels accept. */
#define REPLAYSSM_MAX_BUFFER_LEN 64

/* Human-readable name of a status code (static storage; never NULL). */
const char* replayssm_status_string(replayssm_status status);

/* Library version as major*10000 + minor*100 + patch. */
int32_t replayssm_version(void);

/* ======================================================================================
 * Mamba2
 * ====================================================================================== */

/*
 * Shapes of one Mamba2 SSM layer.  Head h reads the B/C vectors of group
 * g = h / (nheads / ngroups) (consecutive heads share a group).
 *
 *   batch        >= 1
 *   nheads       >= 1, a multiple of ngroups
 *   headdim (P)  in {16, 32, 64, 128};  dstate (N) in {16, 32, 64, 128, 256};
 *                headdim*dstate <= 16384                       (else UNSUPPORTED)
 *   buffer_len   window L, 1 <= L <= REPLAYSSM_MAX_BUFFER_LEN
 *   io_dtype     dtype of x, z, B, C, dt_raw and of the x/B records
 *   dt_softplus  nonzero: dt = softplus(dt_raw + dt_bias); zero: dt = dt_raw + dt_bias
 */
typedef struct {
    int32_t batch, nheads, headdim, dstate, ngroups, buffer_len;
    replayssm_dtype io_dtype;
    int32_t dt_softplus;
} replayssm_mamba2_desc;

/*
 * Per-layer decode state.  The record buffer ("ring") has buffer_len slots per
 * sequence.  Autoregressive decode keeps records in slots 0..cursor-1; speculative
 * decode uses the slots circularly from `head`.
 *
 *   ckpt     f32  [batch, nheads, headdim, dstate]   fp32 checkpoint (required)
 *   ckpt_lp  lp   [batch, nheads, headdim, dstate]   optional read copy, or NULL.
 *            When set, non-flush steps of the output-only route and of speculative
 *            verification read it instead of ckpt; every flush reads ckpt, writes
 *            ckpt and refreshes ckpt_lp ("ReplaySSM" README, benefit "Separate state
 *            precisions": rounding of the copy never enters the recurrence).
 *   rec_x    io   [batch, nheads, buffer_len, headdim]   x records (exact copies)
 *   rec_B    io   [batch, ngroups, buffer_len, dstate]   B records (exact copies)
 *   rec_dt   f32  [batch, buffer_len, nheads]            dt after softplus (slot-major: the
 *            dt of one step is a contiguous row)
 *   lp_dtype dtype of ckpt_lp (ignored when ckpt_lp is NULL):
 *            REPLAYSSM_BF16, REPLAYSSM_F16  round to nearest even from ckpt;
 *            REPLAYSSM_FP8_E4M3  OCP e4m3 (bias 7, 3 mantissa bits, largest 448, no
 *            infinities) with one scale per row: lp_scale[b,h,p] = amax / 448 where
 *            amax = max_n |ckpt[b,h,p,n]|, code = e4m3(ckpt * (448 / amax)) rounded
 *            to nearest even; a zero row has scale 0 and zero codes.  The value read
 *            is code * lp_scale.  dstate must be a multiple of 16.
 *   lp_scale f32  [batch, nheads, headdim]   row scales of an fp8 copy (else NULL)
 */
typedef struct {
    float* ckpt;
    void* ckpt_lp;
    void* rec_x;
    void* rec_B;
    float* rec_dt;
    replayssm_dtype lp_dtype;
    float* lp_scale;
    const int32_t* slot;   /* [batch] state row of each batch row, -1 = pad; or NULL */
    int32_t num_slots;     /* rows of the state arrays when slot is set */
} replayssm_mamba2_state;

/*
 * One autoregressive decode step, output-only route ("How ReplaySSM works":
 * non-flush steps append their inputs and evaluate the output from the checkpoint
 * plus the records, with no state written; the step that fills the buffer merges
 * the records into the checkpoint and writes it back once).
 *
 * For every sequence b with c = cursor_in[b] (0 <= c < L):
 *   window = the c stored records followed by this step's record (x_t, B_t, dt_t);
 *   lam_s  = sum of dt over the window records after s;  decay = exp(A[h] * sum dt);
 *   w_s    = dt_s * exp(A[h] * lam_s);
 *   y      = decay * (ckpt . C_t) + sum_s w_s (B_s . C_t) x_s + D[h] x_t;
 *   out    = y * z * sigmoid(z).
 *   If c + 1 < L: the record is stored in slot c; cursor_out[b] = c + 1; the
 *   checkpoint is not written.
 *   If c + 1 == L (flush): ckpt <- decay * ckpt + sum_s w_s outer(x_s, B_s) is
 *   stored (and ckpt_lp refreshed); y is read from the new checkpoint
 *   (y = ckpt_new . C_t + D[h] x_t); cursor_out[b] = 0.
 * Sequences flush independently, so one call may mix flush and non-flush
 * sequences.
 *
 *   cursor_in  int32 [batch]  read only;  cursor_out int32 [batch]  written.
 *              They must be distinct arrays (ping-pong between steps).
 *   x, z       io [batch, nheads, headdim];  B, C io [batch, ngroups, dstate];
 *   dt_raw     io [batch, nheads];  dt_bias, A, D f32 [nheads];
 *   out        f32 [batch, nheads, headdim];  err_flags int32 [1] or NULL.
 */
replayssm_status replayssm_mamba2_decode(const replayssm_mamba2_desc* desc,
                                         const replayssm_mamba2_state* state,
                                         const int32_t* cursor_in, int32_t* cursor_out,
                                         const void* x, const void* z, const void* B,
                                         const void* C, const void* dt_raw,
                                         const float* dt_bias, const float* A, const float* D,
                                         float* out, int32_t* err_flags, hipStream_t stream);

/*
 * The same decode step by the state-and-output route (named beside the default
 * output-only route in "Core implementation files"; the pages give no formula for it).
 * Every step rebuilds the current state in registers,
 *   h = decay * ckpt + sum_s w_s outer(x_s, B_s)   over the window of c + 1 records,
 * and reads the output from it: y = h . C_t + D[h] x_t, out = y * z * sigmoid(z).  Only
 * the step that fills the buffer (c + 1 == L) stores h as the new checkpoint (and
 * refreshes ckpt_lp); other steps append their record and store no state.  Cursor,
 * record and error rules, arguments and shapes are those of replayssm_mamba2_decode;
 * it reads the fp32 checkpoint on every step (ckpt_lp is only refreshed).  The two
 * routes give the same outputs up to rounding and may be mixed from step to step.
 */
replayssm_status replayssm_mamba2_decode_state_and_output(const replayssm_mamba2_desc* desc,
                                                          const replayssm_mamba2_state* state,
                                                          const int32_t* cursor_in, int32_t* cursor_out,
                                                          const void* x, const void* z, const void* B,
                                                          const void* C, const void* dt_raw,
                                                          const float* dt_bias, const float* A,
                                                          const float* D, float* out, int32_t* err_flags,
                                                          hipStream_t stream);

/*
 * Fold the 0..L-1 records each sequence holds into its checkpoint (same fold as
 * the flush step, over the stored records only), refresh ckpt_lp when it is set,
 * and set cursor_out[b] = 0.  With c = 0 the checkpoint is left bit-unchanged and
 * only ckpt_lp is (re)created, which is how a read copy is initialised.  Used to
 * hand a sequence's whole state over (checkpoint save, migration).
 *   cursor_in, cursor_out  int32 [batch], distinct;  A f32 [nheads].
 */
replayssm_status replayssm_mamba2_flush(const replayssm_mamba2_desc* desc,
                                        const replayssm_mamba2_state* state,
                                        const int32_t* cursor_in, int32_t* cursor_out,
                                        const float* A, int32_t* err_flags, hipStream_t stream);

/*
 * Speculative verification over n_pos positions (the last accepted token and the
 * drafts) on the circular buffer ("ReplaySSM" README, benefit "Cheap rollback";
 * "How ReplaySSM works": draft inputs are appended to the buffer instead of
 * snapshotting the state).
 *
 * Per sequence b, with hd = head[b] (0 <= hd < L), cm = committed[b]
 * (0 <= cm <= L) and 1 <= n_pos <= L:
 *   if cm + n_pos > L the cm committed records (slots (hd + i) % L) are folded into
 *   the checkpoint, which is stored (and ckpt_lp refreshed), flushed[b] = 1 and the
 *   window starts empty; otherwise flushed[b] = 0 and the checkpoint is not written.
 *   Position j's record is written to slot (hd + cm + j) % L and its output is the
 *   replay output over the committed records (none after a flush) followed by
 *   positions 0..j.  One checkpoint read serves all n_pos outputs.
 * head and committed are NOT changed here; replayssm_commit applies the round.
 *
 *   x, z   io [batch, n_pos, nheads, headdim];  B, C io [batch, n_pos, ngroups, dstate];
 *   dt_raw io [batch, n_pos, nheads];  out f32 [batch, n_pos, nheads, headdim];
 *   flushed int32 [batch] written;  head, committed int32 [batch] read only.
 *   n_pos_seq int32 [batch] or NULL: positions of each sequence this round
 *   (0 <= n_pos_seq[b] <= n_pos; the fold rule uses it in place of n_pos).  Inputs
 *   past a sequence's count are ignored and its outputs there are not written; a
 *   sequence with 0 positions is a pad row (skipped, flushed[b] = 0).
 */
replayssm_status replayssm_mamba2_spec_verify(const replayssm_mamba2_desc* desc,
                                              const replayssm_mamba2_state* state,
                                              const int32_t* head, const int32_t* committed,
                                              int32_t n_pos, const int32_t* n_pos_seq,
                                              const void* x, const void* z, const void* B,
                                              const void* C, const void* dt_raw,
                                              const float* dt_bias, const float* A,
                                              const float* D, float* out, int32_t* flushed,
                                              int32_t* err_flags, hipStream_t stream);

/*
 * Apply a verified round: for each b, if flushed[b] then head[b] = (head[b] +
 * committed[b]) % buffer_len and committed[b] = 0; then committed[b] += n_keep[b].
 * n_keep[b] (1 <= n_keep <= n_pos, or <= n_pos_seq[b] when given) is the kept prefix
 * (last accepted token plus the accepted drafts).  Rejected records are dropped by
 * not counting them; no state is touched.  A sequence with n_pos_seq[b] == 0 (a pad
 * row) is left unchanged; rows that a state-slot map marks as pads should pass 0
 * here too, since this call sees no slot map.  A sequence whose n_keep is out of range or whose result
 * would exceed buffer_len is left unchanged and REPLAYSSM_DEVERR_CURSOR is ORed into
 * err_flags.
 *   head, committed int32 [batch] read-write;  flushed, n_keep int32 [batch];
 *   n_pos_seq int32 [batch] or NULL, as passed to the verify call.
 */
replayssm_status replayssm_commit(int32_t batch, int32_t buffer_len, int32_t n_pos,
                                  int32_t* head, int32_t* committed, const int32_t* flushed,
                                  const int32_t* n_keep, const int32_t* n_pos_seq, int32_t* err_flags,
                                  hipStream_t stream);

/*
 * Reset cursors for new sequences: head[b] = 0 (when head is not NULL) and
 * cursor[b] = 0, for b in seq_idx[0..n_seq-1] (seq_idx NULL: every b < batch).
 * `cursor` is the committed count (speculative) or the AR cursor.  Indices outside
 * [0, batch) are ignored.  The caller supplies the new sequence's checkpoint.
 */
replayssm_status replayssm_reset_cursors(int32_t batch, int32_t* head, int32_t* cursor,
                                         const int32_t* seq_idx, int32_t n_seq,
                                         hipStream_t stream);

/*
 * Conventional read-update-write decode step, the baseline the method is measured
 * against ("Why SSM layers slow down hybrid models": every step reads the whole state
 * from HBM and writes it back).  state f32 [batch, nheads, headdim, dstate] is updated in place:
 *   h = exp(dt*A) h + dt outer(x, B);  y = h . C + D x;  out = y * z * sigmoid(z).
 * desc->buffer_len is ignored.  Other arguments as in replayssm_mamba2_decode.
 */
replayssm_status replayssm_selective_state_update(const replayssm_mamba2_desc* desc, float* state,
                                                  const void* x, const void* z, const void* B,
                                                  const void* C, const void* dt_raw,
                                                  const float* dt_bias, const float* A,
                                                  const float* D, float* out, hipStream_t stream);

/*
 * Conventional speculative baseline: one state snapshot per position ("Why SSM
 * layers slow down hybrid models": engines keep the state after every draft token,
 * so a verify step reads one state and writes T of them).  Reads snapshot slot_in[b] of
 * snapshots f32 [batch, n_pos, nheads, headdim, dstate], runs the n_pos updates in
 * order and writes the state after position j into slot j; outputs as
 * replayssm_mamba2_spec_verify.  The next round passes slot_in[b] = n_keep[b] - 1.
 */
replayssm_status replayssm_mamba2_spec_baseline(const replayssm_mamba2_desc* desc, float* snapshots,
                                                const int32_t* slot_in, int32_t n_pos,
                                                const void* x, const void* z, const void* B,
                                                const void* C, const void* dt_raw,
                                                const float* dt_bias, const float* A,
                                                const float* D, float* out, hipStream_t stream);

/* ======================================================================================
 * Gated DeltaNet
 * ====================================================================================== */

/*
 * Shapes of one Gated DeltaNet layer.  Value head hv reads q/k head
 * hv / (num_v_heads / num_k_heads).
 *   dk, dv in {64, 128} (else UNSUPPORTED);  1 <= buffer_len <= REPLAYSSM_MAX_BUFFER_LEN;
 *   io_dtype: dtype of q, k, v and of the k/v records;
 *   scale: output scale; 0 means 1/sqrt(dk).
 */
typedef struct {
    int32_t batch, num_v_heads, num_k_heads, dk, dv, buffer_len;
    replayssm_dtype io_dtype;
    float scale;
} replayssm_gdn_desc;

/*
 *   ckpt       f32 [batch, num_v_heads, dv, dk]
 *   rec_k      io  [batch, num_k_heads, buffer_len, dk]
 *   rec_v      io  [batch, num_v_heads, buffer_len, dv]
 *   rec_alpha  f32 [batch, buffer_len, num_v_heads]   (slot-major, as rec_dt)
 *   rec_beta   f32 [batch, buffer_len, num_v_heads]
 *   slot, num_slots  state-slot map as for Mamba2 (NULL: identity)
 */
typedef struct {
    float* ckpt;
    void* rec_k;
    void* rec_v;
    float* rec_alpha;
    float* rec_beta;
    const int32_t* slot;
    int32_t num_slots;
} replayssm_gdn_state;

/*
 * One autoregressive Gated DeltaNet decode step in replay form (the GDN
 * autoregressive kernel of "Core implementation files"; mechanism of "How
 * ReplaySSM works").  The gated delta rule is
 *   S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,  o_t = scale S_t q_t.
 * Without storing S_t the output is o = scale (ckpt u + acc), where q is carried
 * back through the window (newest record first):
 *   kappa = k_s . u;  acc += beta_s kappa v_s;  u = alpha_s (u - beta_s kappa k_s).
 * Flush (c + 1 == L): the window's updates are applied to the checkpoint row by row
 * in order and the checkpoint is stored once; o is read from the new checkpoint.
 *
 *   cursor_in/out int32 [batch] (distinct);  q, k io [batch, num_k_heads, dk];
 *   v io [batch, num_v_heads, dv];  alpha, beta f32 [batch, num_v_heads];
 *   out f32 [batch, num_v_heads, dv].
 */
replayssm_status replayssm_gdn_decode(const replayssm_gdn_desc* desc, const replayssm_gdn_state* state,
                                      const int32_t* cursor_in, int32_t* cursor_out,
                                      const void* q, const void* k, const void* v,
                                      const float* alpha, const float* beta, float* out,
                                      int32_t* err_flags, hipStream_t stream);

/* Fold the 0..L-1 stored GDN records into the checkpoint; cursor_out[b] = 0. */
replayssm_status replayssm_gdn_flush(const replayssm_gdn_desc* desc, const replayssm_gdn_state* state,
                                     const int32_t* cursor_in, int32_t* cursor_out,
                                     int32_t* err_flags, hipStream_t stream);

/*
 * Gated DeltaNet speculative verification over n_pos positions on the circular
 * buffer (the GDN speculative decode kernel of "Core implementation files", with
 * its own commit and reset calls; rollback as in "ReplaySSM" README, "Cheap
 * rollback").  Cursor rules as replayssm_mamba2_spec_verify: with hd = head[b]
 * (0 <= hd < L) and cm = committed[b] (0 <= cm <= L), if cm + n_pos > L the cm
 * committed records (slots (hd + i) % L) are folded into the checkpoint, which is
 * stored, and flushed[b] = 1; otherwise flushed[b] = 0 and the checkpoint is not
 * written.  Position j's record goes to slot (hd + cm + j) % L, and its output
 * carries q_j back through positions j..0 and then the committed records (none
 * after a fold):  o_j = scale (ckpt u_j + acc_j).  head and committed are NOT
 * changed here; replayssm_commit applies the round and replayssm_reset_cursors
 * starts new sequences.
 *
 *   q, k io [batch, n_pos, num_k_heads, dk];  v io [batch, n_pos, num_v_heads, dv];
 *   alpha, beta f32 [batch, n_pos, num_v_heads];
 *   out f32 [batch, n_pos, num_v_heads, dv];  flushed int32 [batch] written;
 *   head, committed int32 [batch] read only.  1 <= n_pos <= buffer_len; shapes
 *   whose staging exceeds one workgroup's LDS give REPLAYSSM_ERR_UNSUPPORTED.
 *   n_pos_seq int32 [batch] or NULL: positions of each sequence, as for Mamba2.
 *   Invalid cursors: REPLAYSSM_DEVERR_CURSOR is ORed into err_flags and that
 *   sequence's outputs, records, checkpoint and flushed[b] are left untouched.
 */
replayssm_status replayssm_gdn_spec_verify(const replayssm_gdn_desc* desc, const replayssm_gdn_state* state,
                                           const int32_t* head, const int32_t* committed, int32_t n_pos,
                                           const int32_t* n_pos_seq,
                                           const void* q, const void* k, const void* v,
                                           const float* alpha, const float* beta, float* out,
                                           int32_t* flushed, int32_t* err_flags, hipStream_t stream);

/* Conventional GDN step: state f32 [batch, num_v_heads, dv, dk] updated in place. */
replayssm_status replayssm_gdn_conventional_decode(const replayssm_gdn_desc* desc, float* state,
                                                   const void* q, const void* k, const void* v,
                                                   const float* alpha, const float* beta,
                                                   float* out, hipStream_t stream);

/*
 * Conventional Gated DeltaNet speculative baseline: one state snapshot per position
 * ("Why SSM layers slow down hybrid models": a snapshot is stored after every draft
 * token).  Reads snapshot slot_in[b] (clamped to [0, n_pos)) of snapshots f32
 * [batch, n_pos, num_v_heads, dv, dk], runs the n_pos gated delta updates in order
 * and writes the state after position j into slot j; outputs as
 * replayssm_gdn_spec_verify.  The next round passes slot_in[b] = n_keep[b] - 1.
 */
replayssm_status replayssm_gdn_spec_baseline(const replayssm_gdn_desc* desc, float* snapshots,
                                             const int32_t* slot_in, int32_t n_pos, const void* q,
                                             const void* k, const void* v, const float* alpha,
                                             const float* beta, float* out, hipStream_t stream);

/* ======================================================================================
 * Precision emulation
 * ====================================================================================== */

/*
 * Emulated storage precision ("ReplaySSM" README, the paragraph on its two precision
 * folders: emulation kernels that keep the read precision apart from
 * the recurrence precision and expose their rounding).  Rounds each of `rows` rows of
 * `row_len` fp32 values in `data` (device, 16-byte aligned, row-major) in place to
 * the value the format holds, so that a state kept in that format can be run through
 * the fp32 entry points: round a checkpoint after every flush for a low-precision
 * recurrence in replay form, or a conventional state after every update.
 *
 *   dtype = BF16, F16   round to nearest even (F16 overflows to +-inf)
 *   dtype = FP8_E4M3    per row: scale = amax / 448, value = e4m3(h * (448 / amax)) *
 *                       scale, the code rounded to nearest even and saturated to +-448
 *                       (the read-copy format); a zero row stays zero.  If row_scale
 *                       (device f32 [rows], 4-byte aligned) is set, the scales are
 *                       written there.
 *   dtype = F32         nothing to do; OK
 *
 * row_len >= 4 and a multiple of 4; rows >= 0.  INVALID_ARGUMENT otherwise, and then
 * nothing is launched.  Asynchronous on `stream`.
 */
replayssm_status replayssm_emulate_precision(float* data, int64_t rows, int32_t row_len,
                                             replayssm_dtype dtype, float* row_scale, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* REPLAYSSM_H */
