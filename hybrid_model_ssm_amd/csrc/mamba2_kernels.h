// Mamba2 ReplaySSM kernels for gfx950.
//
// The method ("ReplaySSM Caches Inputs Instead of State to Speed Up Hybrid-Model
// Decoding", section "How ReplaySSM works"): the state is held as a checkpoint and a
// ring of the latest input records.  On a non-flush step the record is appended and y
// is evaluated from the checkpoint plus the records, with no state written back; the
// step that fills the buffer merges the records into the checkpoint, written once per
// window.  Unrolling the Mamba2 recurrence h = exp(dt A) h + dt x B^T over a window of
// records s (oldest first) gives, with lam_s = sum of dt over the window records after s:
//
//     decay = exp(A * sum_s dt_s),   w_s = dt_s * exp(A * lam_s)
//     y     = decay * (Hc . C_t) + sum_s w_s (B_s . C_t) x_s + D x_t
//     fold:   Hc <- decay * Hc + sum_s w_s x_s B_s^T
//
// Work decomposition: one 256-thread workgroup per (sequence, group of heads that share
// B and C).  The group's B records, C vectors, the B_s . C_t dots and every head's
// decay coefficients are staged once in LDS; the workgroup then streams its heads'
// [headdim, dstate] fp32 checkpoint tiles, loading head i+1's tile into a second set
// of registers while it reduces head i, so the HBM stream never waits on the per-head
// work.  Within a tile, LPR = dstate/4 consecutive lanes cover one row with 16-byte
// loads (a wave load instruction reads whole contiguous rows) and each thread holds
// R rows.  Row dot products  Hc[p,:] . C  are finished with a transpose-reduce across
// the LPR lanes, and the window's record terms  sum_s coef_s x_s[p]  ride in the same
// reduction: lane q of a row adds the term of record s = q.  The flush fold is a
// rank-|window| update applied to the tile in registers.
//
// Modes share one kernel body:
//   kDecode  one autoregressive step (flushes in place when the buffer fills)
//   kFold    fold the stored records only (explicit flush / read-copy refresh)
//   kSpec    speculative verification over n_pos positions on the circular buffer
//            ("ReplaySSM" README, benefit "Cheap rollback": output-only verification,
//            rejected inputs dropped by moving a pointer)
//   kDecodeSO  one autoregressive step by the state-and-output route ("ReplaySSM (a
//            vLLM research fork)", "Core implementation files", names it beside the
//            default output-only route): every step rebuilds the current state
//            decay * Hc + sum_s w_s x_s B_s^T of the whole window in registers and reads
//            the output from it; only the step that fills the buffer stores it.

#pragma once

#include "device_common.h"
#include "launch.h"

namespace rssm {

constexpr int kDecode = 0;
constexpr int kFold = 1;
constexpr int kSpec = 2;
constexpr int kDecodeSO = 3;
constexpr int kThreads = 256;
constexpr int kMaxHeadsPerWg = 16;
constexpr int kFoldXPerThread = 4;  // 4-element loads per thread for one head's fold rows
constexpr int kRecBatch = 8;        // record rows loaded together when forming the record terms

template <int P, int N>
struct Mamba2Tile {
    static constexpr int LPR = N / 4;                  // lanes per checkpoint row
    static constexpr int RPP = kThreads / LPR;         // rows per pass of the workgroup
    static constexpr int R = (P + RPP - 1) / RPP;      // rows per thread
    static constexpr bool MASK = (P % RPP) != 0;       // some threads hold no row
    static_assert(R >= 1 && R <= LPR && (R & (R - 1)) == 0, "tile shape");
};

// Mapping of a tile read from a low-precision copy: 16-byte loads of EPL elements
// (8 for bf16/fp16, 16 for fp8), N/EPL lanes per row.
template <int P, int N, int EPL>
struct Mamba2TileLp {
    static constexpr int LPR = N / EPL;
    static constexpr int RPP = kThreads / LPR;
    static constexpr int R = (P + RPP - 1) / RPP;
    static constexpr bool MASK = (P % RPP) != 0;
    static_assert(R >= 1 && R <= LPR && (R & (R - 1)) == 0, "low-precision tile shape");
};

// LDS layout of the replay kernel (in 4-byte words).
struct GroupSmem {
    int NR, T1, US;
    int oB, oC, oDt, oBeta, oCf, oDec, oW, oDecf, oY, oZ, oU, oA, oD, total;
    __host__ __device__ GroupSmem(int P, int N, int L, int T, int HC, int mode, int io_bytes) {
        NR = (mode == kSpec) ? L + T : L;   // most window rows
        T1 = T > 0 ? T : 1;
        US = NR + 1;                        // row stride of the fold factors
        oB = 0;                             // [NR][N] io    B rows of the window
        oC = oB + (NR * N * io_bytes + 3) / 4;  // [T1][N]  C of each position
        oDt = oC + T1 * N;                  // [HC][NR]      dt of each head and row
        oBeta = oDt + HC * NR;              // [T1][NR]      B_s . C_j
        oCf = oBeta + T1 * NR;              // [HC][T1][NR]  output coefficients w*beta
        oDec = oCf + HC * T1 * NR;          // [HC][T1]      output decays
        oW = oDec + HC * T1;                // [HC][NR]      fold weights
        oDecf = oW + HC * NR;               // [HC]          fold decays
        oY = oDecf + HC;                    // [HC][T1][P]   record terms + D x of each output
        oZ = oY + HC * T1 * P;              // [HC][T1][P] io  z of each output
        oU = oZ + (HC * T1 * P * io_bytes + 3) / 4;  // [P][US]  fold factors w_s x_s[p] of one head
        oA = oU + P * US;                   // [HC]
        oD = oA + HC;                       // [HC]
        total = oD + HC;
    }
};

// LP: kind of low-precision read copy (kLpNone, kLpBF16, kLpF16, kLpFP8).  Decode steps
// that read a copy stream half or a quarter of the fp32 bytes per tile, keep two (bf16,
// fp16) or three (fp8) copy tiles in flight, request the first tiles before the prologue,
// and are held to three waves per SIMD (the register budget of those buffers without
// spills); the other instances keep the budget the compiler picks.
template <int P, int N, typename IO, int LP, int MODE>
__global__ void __launch_bounds__(kThreads, (LP != kLpNone && MODE == kDecode) ? 3 : 1)
mamba2_replay_kernel(Mamba2Args a) {
    constexpr bool LOWP = LP != kLpNone;
    using io = Io<IO>;
    using Raw4 = typename io::Raw4;
    using Tl = Mamba2Tile<P, N>;
    constexpr int LPR = Tl::LPR, RPP = Tl::RPP, R = Tl::R;
    constexpr bool MASK = Tl::MASK;
    constexpr int P4 = P / 4, N4 = N / 4;
    extern __shared__ float smem[];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int H = a.nheads, G = a.ngroups, L = a.L;
    const int hpg = H / G;
    const int nchunk = a.nchunk;
    const int wid = blockIdx.x;
    const int chunk = wid % nchunk;
    const int bg = wid / nchunk;
    const int g = bg % G;
    const int h0 = g * hpg + chunk * a.heads_per_chunk;
    const int nh = min(a.heads_per_chunk, hpg - chunk * a.heads_per_chunk);
    const bool lead = (g == 0 && chunk == 0);  // writes the per-sequence cursor outputs
    // T: position stride of this call's inputs; Tb: positions of this sequence
    const int T = (MODE == kSpec) ? a.n_pos : (MODE == kFold ? 0 : 1);

    // ---- state row, positions and cursors of this sequence ------------------------------
    // A pad row (state slot -1, or no positions) is skipped; a slot or position count
    // out of range, or a bad cursor, is flagged and skipped.  Skipped rows keep their
    // cursors (cursor_out = cursor_in) and report no flush.
    // Speculative rounds rank the folding sequences after two thirds of the others
    // (measured best between first and last); the ordering hands over the chosen
    // sequence's cursors.
    int b, sb, Tb, c = 0, hd = 0, cm = 0;
    if constexpr (MODE == kSpec) {
        const SpecSeq q = spec_sequence_ranked<kThreads>(bg / G, a.batch, L, T, a.slot, a.n_pos_seq,
                                                         a.cursor_in, a.committed, 2, 3);
        // the pick is the same in every lane (it comes through LDS): keep it in scalar
        // registers, with everything derived from it
        b = __builtin_amdgcn_readfirstlane(q.b);
        sb = __builtin_amdgcn_readfirstlane(q.sb);
        Tb = __builtin_amdgcn_readfirstlane(q.Tb);
        hd = __builtin_amdgcn_readfirstlane(q.hd);
        cm = __builtin_amdgcn_readfirstlane(q.cm);
    } else {
        b = bg / G;
        sb = a.slot ? a.slot[b] : b;
        Tb = T;
        c = a.cursor_in[b];
    }
    int err = 0;
    if (sb < -1 || sb >= (a.slot ? a.num_slots : a.batch)) err |= kDevErrSlot;
    if (Tb < 0 || Tb > T) err |= kDevErrCursor;
    if constexpr (MODE == kSpec) {
        if (hd < 0 || hd >= L || cm < 0 || cm > L) err |= kDevErrCursor;
    } else {
        if (c < 0 || c >= L) err |= kDevErrCursor;
    }
    if (err || sb < 0 || (MODE == kSpec && Tb == 0)) {
        if (tid == 0) {
            if (err && a.err_flags) atomicOr(a.err_flags, err);
            if (lead) {
                if (MODE == kSpec) a.flushed[b] = 0;
                else a.cursor_out[b] = c;
            }
        }
        return;
    }
    const int nstored = (MODE == kSpec) ? cm : c;   // window rows taken from the ring
    const int nrec = nstored + Tb;                   // window rows
    // flush: the checkpoint is rewritten; fold: the window is applied to the tile in
    // registers (every step of the state-and-output route)
    const bool flush = (MODE == kFold) || ((MODE == kDecode || MODE == kDecodeSO) && c + 1 == L) ||
                       (MODE == kSpec && cm + Tb > L);
    const bool fold = flush || MODE == kDecodeSO;
    const int nf = (MODE == kSpec) ? cm : nrec;      // the fold covers rows [0, nf)
    const int st = fold ? nf : 0;                    // first row of every output window
    const bool use_lp = LOWP && !fold;
    // explicit flush of an empty buffer: the fp32 checkpoint stays as it is
    const bool keep_ckpt = ((MODE == kFold) && c == 0) || !flush;
    const bool store_lp = LOWP && flush;
    const bool idle = (MODE == kFold) && c == 0 && !LOWP;

    const GroupSmem lay(P, N, L, T, a.heads_per_chunk, MODE, (int)sizeof(IO));
    const int NR = lay.NR, T1 = lay.T1, US = lay.US;
    IO* sB = reinterpret_cast<IO*>(smem + lay.oB);
    float* sC = smem + lay.oC;
    float* sdt = smem + lay.oDt;
    float* sbeta = smem + lay.oBeta;
    float* scf = smem + lay.oCf;
    float* sdec = smem + lay.oDec;
    float* sw = smem + lay.oW;
    float* sdecf = smem + lay.oDecf;
    float* sY = smem + lay.oY;
    IO* sZ = reinterpret_cast<IO*>(smem + lay.oZ);
    float* sU = smem + lay.oU;
    float* sA = smem + lay.oA;
    float* sD = smem + lay.oD;

    const int row0 = tid / LPR;
    const int col4 = tid % LPR;
    const IO* xin = reinterpret_cast<const IO*>(a.x);
    const IO* zin = reinterpret_cast<const IO*>(a.z);
    const IO* Bin = reinterpret_cast<const IO*>(a.B);
    const IO* Cin = reinterpret_cast<const IO*>(a.C);
    const IO* dtin = reinterpret_cast<const IO*>(a.dt_raw);
    const IO* recX = reinterpret_cast<const IO*>(a.rec_x);
    const IO* recB = reinterpret_cast<const IO*>(a.rec_B) + (size_t)(sb * G + g) * L * N;
    const size_t bH = (size_t)b * H;    // inputs and outputs: batch row
    const size_t sH = (size_t)sb * H;   // checkpoint, copy and records: state row

    auto slot_of = [&](int s) {
        if constexpr (MODE == kSpec) {
            const int t = hd + s;
            return t < L ? t : t - L;
        } else {
            return s;
        }
    };
    // row s of head h's x window: a ring record or one of this call's positions
    auto xrow = [&](int h, int s) -> const IO* {
        if (s < nstored) return recX + ((sH + h) * L + slot_of(s)) * P;
        const int j = s - nstored;
        return xin + ((MODE == kSpec) ? ((size_t)(b * T + j) * H + h) * P : (bH + h) * P);
    };
    auto pos_x = [&](int h, int j) -> size_t {   // x/z/out offset of head h, position j
        return (MODE == kSpec) ? ((size_t)(b * T + j) * H + h) * P : (bH + h) * P;
    };
    auto pos_g = [&](int j) -> size_t {
        return (MODE == kSpec) ? ((size_t)(b * T + j) * G + g) * N : (size_t)(b * G + g) * N;
    };
    auto pos_h = [&](int h, int j) -> size_t {
        return (MODE == kSpec) ? (size_t)(b * T + j) * H + h : bH + h;
    };

    // ---- checkpoint tile loads (head hl into v / vl) -------------------------------------
    auto issue_tile = [&](int hl, float4 (&v)[R]) {
        if (!idle) {
            const size_t t = (sH + h0 + hl) * (size_t)(P * N) + (size_t)row0 * N + 4 * col4;
#pragma unroll
            for (int k = 0; k < R; ++k)
                if (!MASK || row0 + k * RPP < P) v[k] = ld_stream(a.ckpt + t + (size_t)k * RPP * N);
        }
    };
    // tiles of the low-precision read copy (non-flush steps with LOWP), in their own
    // mapping; with fp8, also the scale of the row each lane writes
    constexpr int EPL = (LP == kLpFP8) ? 16 : 8;
    using Tq = Mamba2TileLp<P, N, EPL>;
    constexpr int RQ = Tq::R;
    constexpr int TBQ = (MODE == kSpec) ? Tq::LPR / RQ : 1;   // positions per reduce
    const int rowq0 = tid / Tq::LPR;
    const int colq = tid % Tq::LPR;
    // the row this lane writes after the transpose-reduce (fixed for the whole call)
    const int pq = rowq0 + ((colq / (Tq::LPR / (RQ * TBQ))) % RQ) * Tq::RPP;
    auto issue_tile_lp = [&](int hl, uint4 (&v)[RQ], float& sc) {
        const size_t t = (sH + h0 + hl) * (size_t)(P * N) + (size_t)rowq0 * N + EPL * colq;
#pragma unroll
        for (int k = 0; k < RQ; ++k) {
            if (!Tq::MASK || rowq0 + k * Tq::RPP < P) {
                if constexpr (LP == kLpFP8)
                    v[k] = ld_stream16(reinterpret_cast<const uint8_t*>(a.ckpt_lp) + t + (size_t)k * Tq::RPP * N);
                else
                    v[k] = ld_stream8(reinterpret_cast<const uint16_t*>(a.ckpt_lp) + t + (size_t)k * Tq::RPP * N);
            }
        }
        if constexpr (LP == kLpFP8) sc = a.lp_scale[(sH + h0 + hl) * P + min(pq, P - 1)];
    };
    // fold rows of head hl: x_s[p] for s < nf, as 4-element chunks
    Raw4 xf[kFoldXPerThread];
    auto issue_foldx = [&](int hl) {
#pragma unroll
        for (int i = 0; i < kFoldXPerThread; ++i) {
            const int task = tid + i * kThreads;
            if (task < nf * P4) {
                const int s = task / P4, p4 = task % P4;
                xf[i] = io::ldraw4(xrow(h0 + hl, s), 4 * p4);
            }
        }
    };

    // ---- prologue 1 requests ----------------------------------------------------------
    // The values the staging below needs (up to kPre1 tasks of each kind per thread; a
    // longer window takes the rest in a loop) are requested before the first checkpoint
    // tile, with clamped indices and no branch between the loads: the loads retire in
    // order, so staging then waits on these alone and not on the tile requested after them.
    constexpr int kPre1 = 2;
    const int nBt = nrec * N4;          // staging tasks of the window's B rows
    const int nDt = nh * nrec;          // staging tasks of the window's dt values
    Raw4 preB[kPre1];
    float preRec[kPre1], preIn[kPre1], preBias[kPre1];
#pragma unroll
    for (int i = 0; i < kPre1; ++i) {
        const int task = min(tid + i * kThreads, max(nBt - 1, 0));
        const int s = task / N4, n4 = task - (task / N4) * N4;
        // the explicit flush has no inputs: its rows (none, for an empty buffer) are records
        const IO* src = (MODE == kFold || s < nstored) ? recB + (size_t)slot_of(min(s, L - 1)) * N
                                                       : Bin + pos_g(s - nstored);
        preB[i] = io::ldraw4(src, 4 * n4);
    }
    Raw4 preC{};
    if constexpr (MODE != kFold) preC = io::ldraw4(Cin, pos_g(min(tid / N4, max(Tb - 1, 0))) + 4 * (tid % N4));
#pragma unroll
    for (int i = 0; i < kPre1; ++i) {
        const int task = min(tid + i * kThreads, max(nDt - 1, 0));
        const int s = task / nh, h = h0 + (task - (task / nh) * nh);
        preRec[i] = a.rec_dt[((size_t)sb * L + slot_of(min(s, L - 1))) * H + h];
        preIn[i] = preBias[i] = 0.f;
        if constexpr (MODE != kFold) {
            preIn[i] = io::ld(dtin, pos_h(h, min(max(s - nstored, 0), max(Tb - 1, 0))));
            preBias[i] = a.dt_bias[h];
        }
    }
    const float preA = a.A[h0 + min(tid, nh - 1)];
    const float preD = (MODE != kFold) ? a.D[h0 + min(tid, nh - 1)] : 0.f;

    float4 va[R], vb[R];
    // copy tiles: NQ buffers in fixed roles; in decode steps the first NQ heads are
    // requested before the prologue so that they stream while the window is staged (the
    // speculative instance would lose a wave per SIMD holding them)
    constexpr int NQ = (LP == kLpFP8 && MODE == kDecode) ? 4 : 3;
    constexpr int NQE = (MODE == kDecode) ? NQ : 1;
    uint4 qr[NQ][RQ];
    float sqr[NQ];
    if (use_lp) {
#pragma unroll
        for (int u = 0; u < NQE; ++u) issue_tile_lp(min(u, nh - 1), qr[u], sqr[u]);
    } else {
        issue_tile(0, va);
    }
    if (fold && !idle) issue_foldx(0);

    // this call's records, loaded now and stored after every head has read the ring
    // (autoregressive decode only: in speculative mode they would stay live across the
    // head loop and cost occupancy)
    constexpr int kAppendPerThread = (MODE == kDecode) ? 2 : 0;
    const int napp = (MODE == kFold || (MODE != kSpec && flush)) ? 0 : nh * Tb * P4;
    Raw4 app[kAppendPerThread > 0 ? kAppendPerThread : 1];
#pragma unroll
    for (int i = 0; i < kAppendPerThread; ++i) {
        const int task = tid + i * kThreads;
        if (task < napp) {
            const int p4 = task % P4, hj = task / P4;
            const int hl = hj / Tb, j = hj - hl * Tb;
            app[i] = io::ldraw4(xin, pos_x(h0 + hl, j) + 4 * p4);
        }
    }

    // ---- prologue 1: stage the group's window -------------------------------------------
    auto dt_of = [&](float rec, float in, float bias, bool stored) {
        if (stored) return rec;                         // records keep the prepared dt
        const float dt = in + bias;
        return a.dt_softplus ? softplus_f32(dt) : dt;
    };
#pragma unroll
    for (int i = 0; i < kPre1; ++i) {
        const int task = tid + i * kThreads;
        if (task < nBt) *reinterpret_cast<Raw4*>(sB + task * 4) = preB[i];   // row task / N4, column 4 (task % N4)
    }
    for (int task = tid + kPre1 * kThreads; task < nBt; task += kThreads) {
        const int s = task / N4, n4 = task % N4;
        const Raw4 r = (s < nstored) ? io::ldraw4(recB, (size_t)slot_of(s) * N + 4 * n4)
                                     : io::ldraw4(Bin, pos_g(s - nstored) + 4 * n4);
        *reinterpret_cast<Raw4*>(sB + s * N + 4 * n4) = r;
    }
    if (tid < Tb * N4) *reinterpret_cast<float4*>(sC + tid * 4) = io::cvt4(preC);
    for (int task = tid + kThreads; task < Tb * N4; task += kThreads) {
        const int j = task / N4, n4 = task % N4;
        *reinterpret_cast<float4*>(sC + j * N + 4 * n4) = io::cvt4(io::ldraw4(Cin, pos_g(j) + 4 * n4));
    }
    // a slot's heads are contiguous in rec_dt: task = s * nh + head
#pragma unroll
    for (int i = 0; i < kPre1; ++i) {
        const int task = tid + i * kThreads;
        if (task < nDt) {
            const int s = task / nh, hl = task - s * nh;
            sdt[hl * NR + s] = dt_of(preRec[i], preIn[i], preBias[i], s < nstored);
        }
    }
    for (int task = tid + kPre1 * kThreads; task < nDt; task += kThreads) {
        const int s = task / nh, hl = task - s * nh;
        const int h = h0 + hl;
        sdt[hl * NR + s] = dt_of(s < nstored ? a.rec_dt[((size_t)sb * L + slot_of(s)) * H + h] : 0.f,
                                 s < nstored ? 0.f : io::ld(dtin, pos_h(h, s - nstored)), a.dt_bias[h], s < nstored);
    }
    if (tid < nh) {
        sA[tid] = preA;
        if (MODE != kFold) sD[tid] = preD;
    }
    for (int hl = tid + kThreads; hl < nh; hl += kThreads) {
        sA[hl] = a.A[h0 + hl];
        if (MODE != kFold) sD[hl] = a.D[h0 + hl];
    }
    __syncthreads();

    if constexpr (MODE != kFold) {
        // ---- prologue 2: beta[j][s] = B_s . C_j, 16 lanes a pair -----------------------
        for (int base = 0; base < Tb * nrec; base += kThreads / 16) {
            const int pr = base + tid / 16;
            const int part = tid & 15;
            if (pr < Tb * nrec) {
                const int j = pr / nrec, s = pr - j * nrec;
                float beta = 0.f;
                for (int n = part; n < N; n += 16) beta += io::ld(sB, s * N + n) * sC[j * N + n];
                beta = group_allreduce<16>(beta, lane);
                if (part == 0) sbeta[j * NR + s] = beta;
            }
        }
        __syncthreads();
    }

    // ---- prologue 3: per-head coefficients (log-space decay sums, newest row first) -------
    for (int pr = tid; pr < nh * Tb; pr += kThreads) {
        const int hl = pr / Tb, j = pr - hl * Tb;
        const int e = nstored + j;          // position j's own row
        const float Ah = sA[hl];
        float lam = 0.f;
        for (int s = e; s >= st; --s) {
            const float dt = sdt[hl * NR + s];
            scf[(hl * T1 + j) * NR + s] = dt * expf(Ah * lam) * sbeta[j * NR + s];
            lam += dt;
        }
        sdec[hl * T1 + j] = expf(Ah * lam);   // 1 for an empty window
    }
    if (fold) {
        for (int hl = tid; hl < nh; hl += kThreads) {
            const float Ah = sA[hl];
            float lam = 0.f;
            for (int s = nf - 1; s >= 0; --s) {
                const float dt = sdt[hl * NR + s];
                sw[hl * NR + s] = dt * expf(Ah * lam);
                lam += dt;
            }
            sdecf[hl] = expf(Ah * lam);
        }
    }
    __syncthreads();

    if constexpr (MODE != kFold) {
        // ---- prologue 4: record terms of every output, and z ---------------------------
        //   Y[h][j][p] = sum_{s in window j} coef_s x_s[p] + D x_j[p]
        // One task per (head, 4 columns, up to kPosBatch positions): each window row is
        // loaded once and feeds every position whose window holds it.
        constexpr int kPosBatch = 4;
        const int njb = (Tb + kPosBatch - 1) / kPosBatch;
        for (int task = tid; task < nh * njb * P4; task += kThreads) {
            const int p4 = task % P4;
            const int hb = task / P4;
            const int hl = hb / njb, j0 = (hb - hl * njb) * kPosBatch;
            const int h = h0 + hl;
            const int jn = min(kPosBatch, Tb - j0);
            const int elast = nstored + j0 + jn - 1;        // last row any of these windows uses
            const float Dh = sD[hl];
            // z of these outputs and the window rows are requested before any of them is
            // used, with no branch between the loads (rows past the window repeat its last
            // row), so that their round trips overlap
            Raw4 zr[kPosBatch];
#pragma unroll
            for (int jj = 0; jj < kPosBatch; ++jj) zr[jj] = io::ldraw4(zin, pos_x(h, j0 + min(jj, jn - 1)) + 4 * p4);
            float4 y[kPosBatch];
#pragma unroll
            for (int jj = 0; jj < kPosBatch; ++jj) y[jj] = make_float4(0.f, 0.f, 0.f, 0.f);
            for (int s0 = st; s0 <= elast; s0 += kRecBatch) {
                Raw4 xr[kRecBatch];
#pragma unroll
                for (int i = 0; i < kRecBatch; ++i) xr[i] = io::ldraw4(xrow(h, min(s0 + i, elast)), 4 * p4);
#pragma unroll
                for (int i = 0; i < kRecBatch; ++i) {
                    const int sr = s0 + i;
                    if (sr <= elast) {
                        const float4 xv = io::cvt4(xr[i]);
#pragma unroll
                        for (int jj = 0; jj < kPosBatch; ++jj) {
                            const int j = j0 + jj;
                            if (jj < jn && sr <= nstored + j) {
                                float w = scf[(hl * T1 + j) * NR + sr];
                                if (sr == nstored + j) w += Dh;     // position j's own row: + D x_j
                                y[jj].x += w * xv.x; y[jj].y += w * xv.y; y[jj].z += w * xv.z; y[jj].w += w * xv.w;
                            }
                        }
                    }
                }
            }
            // rows before st (flushed windows) still need D x_j for position j's own row;
            // a constant trip count keeps y[] in registers
#pragma unroll
            for (int jj = 0; jj < kPosBatch; ++jj) {
                if (jj < jn) {
                    const int j = j0 + jj;
                    const int o = (hl * T1 + j) * P + 4 * p4;
                    float4 yv = y[jj];
                    if (nstored + j < st) {     // empty window (AR flush step): only D x_j
                        const float4 xj = io::cvt4(io::ldraw4(xrow(h, nstored + j), 4 * p4));
                        yv = make_float4(Dh * xj.x, Dh * xj.y, Dh * xj.z, Dh * xj.w);
                    }
                    *reinterpret_cast<float4*>(sY + o) = yv;
                    *reinterpret_cast<Raw4*>(sZ + o) = zr[jj];
                }
            }
        }
        __syncthreads();
    }

    // ---- stream the heads' checkpoint tiles ---------------------------------------------
    // Each loop issues head hl+1's loads before working on head hl and peels the last
    // head, so that every load is unconditional and the wait before head hl's work
    // covers only loads issued before head hl+1's.
    const int q = tid % LPR;
    const int ridx = q / (LPR / R);
    const int pw = row0 + ridx * RPP;                // row this lane writes
    const bool writer = (q % (LPR / R)) == 0 && (!MASK || pw < P);

    // Speculative verify reduces TB positions of a head in one transpose-reduce (R*TB
    // values over LPR lanes; two positions keep the register budget of three waves per
    // SIMD).
    constexpr int TB = (MODE == kSpec) ? (LPR / R >= 2 ? 2 : 1) : 1;
    auto outputs = [&](int hl, const float4 (&v)[R]) {
        if constexpr (MODE == kDecode || MODE == kDecodeSO) {
            const float4 Cv = *reinterpret_cast<const float4*>(sC + 4 * col4);
            float acc[R];
#pragma unroll
            for (int k = 0; k < R; ++k) acc[k] = dot4(v[k], Cv);
            const float r = row_reduce<R, LPR>(acc, lane);
            if (writer) {
                const int o = hl * T1 * P + pw;
                sY[o] = silu_gate_fast(sdec[hl * T1] * r + sY[o], io::ld(sZ, o));
            }
        } else if constexpr (MODE == kSpec) {
            for (int j0 = 0; j0 < Tb; j0 += TB) {
                float acc[R * TB];
#pragma unroll
                for (int jj = 0; jj < TB; ++jj) {
                    const int j = min(j0 + jj, Tb - 1);
                    const float4 Cv = *reinterpret_cast<const float4*>(sC + j * N + 4 * col4);
#pragma unroll
                    for (int k = 0; k < R; ++k) acc[jj * R + k] = dot4(v[k], Cv);
                }
                const float r = row_reduce<R * TB, LPR>(acc, lane);
                const int vi = q / (LPR / (R * TB));          // value index this lane holds
                const int j = j0 + vi / R;
                const int p = row0 + (vi % R) * RPP;
                if ((q % (LPR / (R * TB))) == 0 && j < Tb && (!MASK || p < P)) {
                    const int o = (hl * T1 + j) * P + p;
                    sY[o] = silu_gate_fast(sdec[hl * T1 + j] * r + sY[o], io::ld(sZ, o));
                }
            }
        }
    };
    auto rotate = [&]() {
#pragma unroll
        for (int k = 0; k < R; ++k) va[k] = vb[k];
    };

    // outputs of head hl from a low-precision tile: same arithmetic as `outputs`, in the
    // EPL-elements-per-lane mapping.  fp8 tiles decode to the code values; the row scale
    // multiplies the reduced row.
    auto lp_dot = [&](const uint4& v, int j) -> float {
        const float* c = sC + j * N + EPL * colq;
        const float4 C0 = *reinterpret_cast<const float4*>(c);
        const float4 C1 = *reinterpret_cast<const float4*>(c + 4);
        if constexpr (LP == kLpBF16) {
            return dot4(bf16x4_to_f32x4(make_uint2(v.x, v.y)), C0) + dot4(bf16x4_to_f32x4(make_uint2(v.z, v.w)), C1);
        } else if constexpr (LP == kLpF16) {
            const float2 e0 = f16x2_bits_to_f32(v.x), e1 = f16x2_bits_to_f32(v.y);
            const float2 e2 = f16x2_bits_to_f32(v.z), e3 = f16x2_bits_to_f32(v.w);
            return dot4(make_float4(e0.x, e0.y, e1.x, e1.y), C0) + dot4(make_float4(e2.x, e2.y, e3.x, e3.y), C1);
        } else {
            const float4 C2 = *reinterpret_cast<const float4*>(c + 8);
            const float4 C3 = *reinterpret_cast<const float4*>(c + 12);
            return dot4(e4m3x4_to_f32x4(v.x), C0) + dot4(e4m3x4_to_f32x4(v.y), C1) +
                   dot4(e4m3x4_to_f32x4(v.z), C2) + dot4(e4m3x4_to_f32x4(v.w), C3);
        }
    };
    auto outputs_lp = [&](int hl, const uint4 (&v)[RQ], float sc) {
        if constexpr (MODE != kFold && LOWP) {
            constexpr int LQ = Tq::LPR;
            const int qq = tid % LQ;
            const float rs = (LP == kLpFP8) ? sc : 1.0f;
            for (int j0 = 0; j0 < Tb; j0 += TBQ) {
                float acc[RQ * TBQ];
#pragma unroll
                for (int jj = 0; jj < TBQ; ++jj) {
                    const int j = min(j0 + jj, Tb - 1);
#pragma unroll
                    for (int k = 0; k < RQ; ++k) acc[jj * RQ + k] = lp_dot(v[k], j);
                }
                const float r = row_reduce<RQ * TBQ, LQ>(acc, lane);
                const int vi = qq / (LQ / (RQ * TBQ));
                const int j = j0 + vi / RQ;
                const int p = rowq0 + (vi % RQ) * Tq::RPP;
                if ((qq % (LQ / (RQ * TBQ))) == 0 && j < Tb && (!Tq::MASK || p < P)) {
                    const int o = (hl * T1 + j) * P + p;
                    sY[o] = silu_gate_fast(sdec[hl * T1 + j] * (rs * r) + sY[o], io::ld(sZ, o));
                }
            }
        }
    };

    if (!fold && use_lp && nh >= NQ) {
        // copy tiles are small: heads hl+1 .. hl+NQ-1 stream while head hl is reduced.
        // The buffers keep fixed roles (the loop is unrolled by NQ): a register copy of a
        // tile still in flight would wait for it.
#pragma unroll
        for (int u = NQE; u < NQ; ++u) issue_tile_lp(u, qr[u], sqr[u]);
        int hl = 0;
        for (; hl + 2 * NQ - 1 < nh; hl += NQ) {
#pragma unroll
            for (int u = 0; u < NQ; ++u) {
                outputs_lp(hl + u, qr[u], sqr[u]);
                issue_tile_lp(hl + u + NQ, qr[u], sqr[u]);
            }
        }
        const int rest = nh - hl;       // NQ .. 2 NQ - 1 heads remain
#pragma unroll
        for (int u = 0; u < NQ; ++u) {
            outputs_lp(hl + u, qr[u], sqr[u]);
            if (u + NQ < rest) issue_tile_lp(hl + u + NQ, qr[u], sqr[u]);
        }
#pragma unroll
        for (int u = 0; u < NQ - 1; ++u)
            if (u + NQ < rest) outputs_lp(hl + NQ + u, qr[u], sqr[u]);
    } else if (!fold && use_lp) {
        // fewer heads than buffers: tile hl+1 is loaded while head hl is reduced
        for (int hl = 0; hl + 1 < nh; ++hl) {
            issue_tile_lp(hl + 1, qr[1], sqr[1]);
            outputs_lp(hl, qr[0], sqr[0]);
#pragma unroll
            for (int k = 0; k < RQ; ++k) qr[0][k] = qr[1][k];
            sqr[0] = sqr[1];
        }
        outputs_lp(nh - 1, qr[0], sqr[0]);
    } else if (!fold) {
        // tile hl+1 is loaded while head hl is reduced
        for (int hl = 0; hl + 1 < nh; ++hl) {
            issue_tile(hl + 1, vb);
            outputs(hl, va);
            rotate();
        }
        outputs(nh - 1, va);
    } else if (!idle) {
        auto stage_u = [&](int hl) {     // fold factors u_s[p] = w_s x_s[p] of head hl
            __syncthreads();
#pragma unroll
            for (int i = 0; i < kFoldXPerThread; ++i) {
                const int task = tid + i * kThreads;
                if (task < nf * P4) {
                    const int s = task / P4, p4 = task % P4;
                    const float w = sw[hl * NR + s];
                    const float4 xv = io::cvt4(xf[i]);
                    float* d = sU + (4 * p4) * US + s;
                    d[0] = w * xv.x; d[US] = w * xv.y; d[2 * US] = w * xv.z; d[3 * US] = w * xv.w;
                }
            }
        };
        auto body = [&](int hl) {
            __syncthreads();
            const float decf = sdecf[hl];
#pragma unroll
            for (int k = 0; k < R; ++k) {
                va[k].x *= decf; va[k].y *= decf; va[k].z *= decf; va[k].w *= decf;
            }
            for (int s = 0; s < nf; ++s) {
                const float4 Bv = io::cvt4(*reinterpret_cast<const Raw4*>(sB + s * N + 4 * col4));
#pragma unroll
                for (int k = 0; k < R; ++k) {
                    if (!MASK || row0 + k * RPP < P) {
                        const float u = sU[(row0 + k * RPP) * US + s];
                        va[k].x += u * Bv.x; va[k].y += u * Bv.y; va[k].z += u * Bv.z; va[k].w += u * Bv.w;
                    }
                }
            }
            const size_t t = (sH + h0 + hl) * (size_t)(P * N) + (size_t)row0 * N + 4 * col4;
#pragma unroll
            for (int k = 0; k < R; ++k) {
                // fp8 copy: the row's largest magnitude over its LPR lanes (every lane
                // takes part; rows past P are never stored)
                float amax = 0.f;
                if constexpr (LP == kLpFP8) {
                    if (store_lp) {
                        amax = fmaxf(fmaxf(fabsf(va[k].x), fabsf(va[k].y)), fmaxf(fabsf(va[k].z), fabsf(va[k].w)));
                        amax = group_allmax<LPR>(amax);
                    }
                }
                if (!MASK || row0 + k * RPP < P) {
                    const size_t off = t + (size_t)k * RPP * N;
                    if (!keep_ckpt) st_stream(a.ckpt + off, va[k]);
                    if (store_lp) {
                        if constexpr (LP == kLpBF16) {
                            st_stream(reinterpret_cast<uint16_t*>(a.ckpt_lp) + off, f32x4_to_bf16x4(va[k]));
                        } else if constexpr (LP == kLpF16) {
                            st_stream(reinterpret_cast<uint16_t*>(a.ckpt_lp) + off, f32x4_to_f16x4(va[k]));
                        } else if constexpr (LP == kLpFP8) {
                            const float inv = amax > 0.f ? 448.0f / amax : 0.f;
                            st_stream(reinterpret_cast<uint8_t*>(a.ckpt_lp) + off, f32x4_to_e4m3x4(va[k], inv));
                            if (col4 == 0) a.lp_scale[(sH + h0 + hl) * P + row0 + k * RPP] = amax / 448.0f;
                        }
                    }
                }
            }
            outputs(hl, va);
        };
        for (int hl = 0; hl + 1 < nh; ++hl) {
            stage_u(hl);
            issue_foldx(hl + 1);
            issue_tile(hl + 1, vb);
            body(hl);
            rotate();
        }
        stage_u(nh - 1);
        body(nh - 1);
    }

    // ---- store the outputs ----------------------------------------------------------------
    // Each output replaced its record term in sY (the lane that reads an entry writes it);
    // the workgroup's outputs of one position are one contiguous block of nh * P floats,
    // stored here in one coalesced pass rather than as scattered words between the
    // checkpoint loads (scattered writes in the read stream cost far more than their bytes).
    if constexpr (MODE != kFold) {
        __syncthreads();
        for (int task = tid; task < Tb * nh * P4; task += kThreads) {
            const int p4 = task % P4, jh = task / P4;
            const int j = jh / nh, hl = jh - j * nh;
            *reinterpret_cast<float4*>(a.out + pos_x(h0 + hl, j) + 4 * p4) =
                *reinterpret_cast<const float4*>(sY + (hl * T1 + j) * P + 4 * p4);
        }
    }

    // ---- append this step's records --------------------------------------------------
    if constexpr (MODE != kFold) {
        if (MODE == kSpec || !flush) {
            // speculative rounds may overwrite ring slots that other heads read above (the
            // barrier before the output stores orders them)
            const int slot0 = (MODE == kSpec) ? hd + cm : c;
#pragma unroll
            for (int i = 0; i < kAppendPerThread; ++i) {
                const int task = tid + i * kThreads;
                if (task < napp) {
                    const int p4 = task % P4, hj = task / P4;
                    const int hl = hj / Tb, j = hj - hl * Tb;
                    const int slot = (slot0 + j) % L;
                    io::straw4(reinterpret_cast<IO*>(a.rec_x), ((sH + h0 + hl) * L + slot) * P + 4 * p4, app[i]);
                }
            }
            for (int task = tid + kAppendPerThread * kThreads; task < napp; task += kThreads) {
                const int p4 = task % P4, hj = task / P4;
                const int hl = hj / Tb, j = hj - hl * Tb;
                const int slot = (slot0 + j) % L;
                io::straw4(reinterpret_cast<IO*>(a.rec_x), ((sH + h0 + hl) * L + slot) * P + 4 * p4,
                           io::ldraw4(xin, pos_x(h0 + hl, j) + 4 * p4));
            }
            // one slot's dt of the workgroup's heads: one contiguous block (scattered 4-byte
            // stores into the read stream are costly)
            for (int task = tid; task < nh * Tb; task += kThreads) {
                const int j = task / nh, hl = task - j * nh;
                a.rec_dt[((size_t)sb * L + (slot0 + j) % L) * H + h0 + hl] = sdt[hl * NR + nstored + j];
            }
            // the group's B records: with several workgroups per group the host appends
            // them in a separate launch (speculative rounds only)
            if (nchunk == 1 || (MODE != kSpec && chunk == 0)) {
                for (int task = tid; task < Tb * N4; task += kThreads) {
                    const int j = task / N4, n4 = task % N4;
                    io::straw4(reinterpret_cast<IO*>(a.rec_B), ((size_t)(sb * G + g) * L + (slot0 + j) % L) * N + 4 * n4,
                               *reinterpret_cast<const Raw4*>(sB + (nstored + j) * N + 4 * n4));
                }
            }
        }
    }

    if (tid == 0 && lead) {
        if (MODE == kSpec) a.flushed[b] = flush ? 1 : 0;
        else a.cursor_out[b] = flush ? 0 : c + 1;
    }
}

// Appends the speculative round's B vectors to each group's ring (slots
// (head + committed + j) % L) when a group's heads are split over several
// workgroups.  Runs after the verify kernel on the same stream, so every head has
// finished reading the slots it replaces.
template <typename IO>
__global__ void __launch_bounds__(kThreads) mamba2_spec_append_B_kernel(Mamba2Args a) {
    const int G = a.ngroups, N = a.dstate, L = a.L, T = a.n_pos;
    const size_t total = (size_t)a.batch * T * G * N;
    for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < total;
         i += (size_t)gridDim.x * kThreads) {
        const int n = (int)(i % N);
        size_t r = i / N;
        const int g = (int)(r % G);
        r /= G;
        const int j = (int)(r % T);
        const int b = (int)(r / T);
        const int sb = a.slot ? a.slot[b] : b;
        const int Tb = a.n_pos_seq ? a.n_pos_seq[b] : T;
        const int hd = a.cursor_in[b], cm = a.committed[b];
        if (hd < 0 || hd >= L || cm < 0 || cm > L) continue;
        if (sb < 0 || sb >= (a.slot ? a.num_slots : a.batch) || Tb < 0 || Tb > T || j >= Tb) continue;
        const int slot = (hd + cm + j) % L;
        reinterpret_cast<IO*>(a.rec_B)[((size_t)(sb * G + g) * L + slot) * N + n] =
            reinterpret_cast<const IO*>(a.B)[i];
    }
}

// ---------------------------------------------------------------------------------------
// Conventional read-update-write step ("Why SSM layers slow down hybrid models": load
// the state, update it, read the output, store it -- every step).  SNAP: per-position
// snapshot baseline for speculative decoding -- read snapshot slot_in[b], run the n_pos
// updates, store all n_pos states.
//
// Every state row (b, h, p) is updated and reduced on its own (y[p] = h[p,:] . C), so
// the kernel is cut finely: LPR = N/4 lanes per row with one 16-byte access each, RPT
// rows per thread, one workgroup per RW = (256/LPR) * RPT consecutive rows.  Small
// chunks per workgroup keep the memory touched by the workgroups in flight within a
// narrow window, which an in-place read-modify-write stream needs to approach the
// device's read+write limit (whole 32 KiB heads per workgroup stream 15% slower); a few
// rows per thread share the per-head work (dt, its softplus and decay, B and C) so that
// the vector ALU, which one 16-byte access per lane would keep busy, stays off the
// critical path.  When RW divides P a workgroup stays inside one head and its (b, h)
// is computed once in scalar registers; otherwise each lane finds its own row's head.
// ---------------------------------------------------------------------------------------
#ifndef RSSM_CONV_RPT
#define RSSM_CONV_RPT 2
#endif
constexpr int kConvMaxGrid = 1 << 24;   // workgroups per launch; larger problems loop
constexpr int kConvPosGroup = 4;        // snapshot baseline: positions whose inputs load together

template <int P, int N>
struct ConvShape {
    static constexpr int LPR = N / 4;                   // lanes per state row
    static constexpr int RPP = kThreads / LPR;          // rows per pass of the workgroup
    static constexpr int RPT = (P / RPP >= RSSM_CONV_RPT) ? RSSM_CONV_RPT : 1;   // rows per thread
    static constexpr int RW = RPP * RPT;                // rows per workgroup
    static constexpr bool ONE_HEAD = (P % RW) == 0;     // a workgroup stays inside one head
};

// One position's small inputs of a conventional Mamba2 step, as loaded (no arithmetic, so
// the compiler issues every load of a position together).
template <int RPT>
struct ConvInputs {
    float dt_raw;
    float x[RPT], z[RPT];
    float4 B, C;
};

template <int P, int N, typename IO, bool SNAP>
__global__ void __launch_bounds__(kThreads) mamba2_conventional_kernel(Mamba2ConvArgs a) {
    using io = Io<IO>;
    using Sh = ConvShape<P, N>;
    constexpr int LPR = Sh::LPR, RPP = Sh::RPP, RPT = Sh::RPT, RW = Sh::RW;
    constexpr bool ONE_HEAD = Sh::ONE_HEAD;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int row0 = tid / LPR;
    const int col4 = tid % LPR;
    const int H = a.nheads, G = a.ngroups;
    const int hpg = H / G;
    const int T = SNAP ? a.n_pos : 1;
    const int64_t rows = (int64_t)a.batch * H * P;
    const int64_t nchunks = (rows + RW - 1) / RW;
    const IO* xin = reinterpret_cast<const IO*>(a.x);
    const IO* zin = reinterpret_cast<const IO*>(a.z);
    const IO* Bin = reinterpret_cast<const IO*>(a.B);
    const IO* Cin = reinterpret_cast<const IO*>(a.C);
    const IO* dtin = reinterpret_cast<const IO*>(a.dt_raw);
    constexpr size_t PN = (size_t)P * N;
    const int q = tid % LPR;
    const int ridx = q / (LPR / RPT);                   // row this lane writes after the reduce
    const bool writer = (q % (LPR / RPT)) == 0;

    for (int64_t chunk = blockIdx.x; chunk < nchunks; chunk += gridDim.x) {
        int64_t bh;   // b * H + h of this lane's rows
        int p;        // this lane's first row within the head (the others follow RPP apart)
        if constexpr (ONE_HEAD) {
            bh = chunk / (P / RW);
            p = (int)(chunk % (P / RW)) * RW + row0;
        } else {
            const int64_t r = chunk * RW + row0;
            if (r >= rows) continue;                    // whole rows drop out together
            bh = r / P;
            p = (int)(r % P);
        }
        const int b = (int)(bh / H), h = (int)(bh - (int64_t)(bh / H) * H);
        const int g = h / hpg;
        size_t src;
        if constexpr (SNAP) {
            int sl = a.slot_in[b];
            sl = sl < 0 ? 0 : (sl >= T ? T - 1 : sl);
            src = ((size_t)(b * T + sl) * H + h) * PN + (size_t)p * N + 4 * col4;
        } else {
            src = (size_t)bh * PN + (size_t)p * N + 4 * col4;
        }
        float4 v[RPT];
#pragma unroll
        for (int k = 0; k < RPT; ++k) v[k] = ld_stream(a.state + src + (size_t)k * RPP * N);
        auto load_in = [&](int j) {
            const size_t xo = (SNAP ? ((size_t)(b * T + j) * H + h) * P : (size_t)bh * P) + p;
            const size_t go = SNAP ? ((size_t)(b * T + j) * G + g) * N : (size_t)(b * G + g) * N;
            const size_t ho = SNAP ? (size_t)(b * T + j) * H + h : (size_t)bh;
            ConvInputs<RPT> in;
            in.dt_raw = io::ld(dtin, ho);
#pragma unroll
            for (int k = 0; k < RPT; ++k) {
                in.x[k] = io::ld(xin, xo + k * RPP);
                in.z[k] = io::ld(zin, xo + k * RPP);
            }
            in.B = io::ld4(Bin, go + 4 * col4);
            in.C = io::ld4(Cin, go + 4 * col4);
            return in;
        };
        const float Ah = a.A[h], Dh = a.D[h], bias = a.dt_bias[h];
        // positions in unrolled groups of kConvPosGroup, each group's inputs loaded together
        // (a loop-carried wait would hold every position until the previous store landed)
        constexpr int GRP = SNAP ? kConvPosGroup : 1;
        for (int j0 = 0; j0 < T; j0 += GRP) {
            ConvInputs<RPT> in[GRP];
#pragma unroll
            for (int jj = 0; jj < GRP; ++jj) in[jj] = load_in(min(j0 + jj, T - 1));   // no branch between loads
#pragma unroll
            for (int jj = 0; jj < GRP; ++jj) {
                const int j = j0 + jj;
                if (j < T) {
                    const float u = in[jj].dt_raw + bias;
                    const float dt = a.dt_softplus ? softplus_f32(u) : u;
                    const float dA = expf(dt * Ah);
                    float acc[RPT];
                    const size_t dst = SNAP ? ((size_t)(b * T + j) * H + h) * PN + (size_t)p * N + 4 * col4 : src;
#pragma unroll
                    for (int k = 0; k < RPT; ++k) {
                        const float xd = dt * in[jj].x[k];
                        v[k].x = dA * v[k].x + xd * in[jj].B.x;
                        v[k].y = dA * v[k].y + xd * in[jj].B.y;
                        v[k].z = dA * v[k].z + xd * in[jj].B.z;
                        v[k].w = dA * v[k].w + xd * in[jj].B.w;
                        st_stream(a.state + dst + (size_t)k * RPP * N, v[k]);
                        acc[k] = dot4(v[k], in[jj].C);
                    }
                    const float y = row_reduce<RPT, LPR>(acc, lane);
                    if (writer) {
                        float xw = in[jj].x[0], zw = in[jj].z[0];
#pragma unroll
                        for (int k = 1; k < RPT; ++k) {
                            xw = (k == ridx) ? in[jj].x[k] : xw;
                            zw = (k == ridx) ? in[jj].z[k] : zw;
                        }
                        const size_t xo = (SNAP ? ((size_t)(b * T + j) * H + h) * P : (size_t)bh * P) + p + ridx * RPP;
                        a.out[xo] = silu_gate_fast(y + Dh * xw, zw);
                    }
                }
            }
        }
    }
}

}  // namespace rssm
