// Gated DeltaNet ReplaySSM kernels for gfx950.
//
// Gated delta rule with a [dv, dk] state per value head:
//     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = scale S_t q_t.
// Replay form ("ReplaySSM Caches Inputs Instead of State to Speed Up Hybrid-Model
// Decoding", section "How ReplaySSM works", applied to the Gated DeltaNet layer that
// "ReplaySSM (a vLLM research fork)", section "Core implementation files", lists):
// the checkpoint S_c and a buffer of (k, v, alpha, beta) records.  Without forming
// S_t, carry q back through the window, newest record first,
//     kappa = k_s . u;   acc += beta_s kappa v_s;   u = alpha_s (u - beta_s kappa k_s),
// so that S_t q = S_c u + acc.  The chain is sequential in s but only dk long; the
// chains run on the workgroup's waves while the first checkpoint tile is in flight.
// The flush applies the window's updates to the checkpoint (rows are independent; the
// updates of up to 16 records are applied together in matrix form, see the fold
// branch) and stores it once.  Speculative verification runs one chain per position.
//
// Decomposition: the replay kernel runs one 256-thread workgroup per (sequence, q/k
// head, up to four of its value heads) and streams the [64, dk] tiles of those value
// heads (k records and q are shared by them); the conventional kernel runs one
// workgroup per (sequence, value head, 64-row tile).  dk/4 consecutive lanes cover one
// row of a tile with 16-byte loads.

#include "device_common.h"
#include "launch.h"

namespace rssm {

constexpr int kGdnThreads = 256;
constexpr int kGdnDecode = 0;
constexpr int kGdnFold = 1;
constexpr int kGdnSpec = 2;
constexpr int kGdnMaxVHeads = 4;   // value heads per workgroup
constexpr int kGdnFoldChunk = 16;  // records folded together in matrix form
constexpr int kGdnXStride = 36;     // floats per row of a wave's exchange buffer (32 + 4 against bank conflicts)
constexpr size_t kGdnMaxSmemBytes = 64 * 1024;

template <int DK>
struct GdnShape {
    static constexpr int LPR = DK / 4;                 // lanes per state row
    static constexpr int RPP = kGdnThreads / LPR;      // rows per pass
    static constexpr int R = 64 / RPP;                 // rows per thread: tiles of 64 rows
    static constexpr int DVT = RPP * R;
};

// LDS layout (4-byte words) of the replay kernel.  NR bounds the window rows (stored
// records plus this call's positions), T1 the positions.
struct GdnSmem {
    int NR, T1, oK, oV, oAl, oBe, oQ, oU, oAcc;
    int oGr, oNm, oGW, oDd, oDc, oX, total;
    __host__ __device__ GdnSmem(int DK, int DV, int L, int T, int mode, int NV, int io_bytes) {
        NR = (mode == kGdnSpec) ? L + T : L;
        T1 = T > 1 ? T : 1;
        oK = 0;                                    // [NR][DK]      k rows of the window (io dtype)
        oV = oK + (NR * DK * io_bytes + 3) / 4;    // [NV][NR][DV]  v rows (io dtype)
        oAl = oV + (NV * NR * DV * io_bytes + 3) / 4;   // [NV][NR]
        oBe = oAl + NV * NR;                       // [NV][NR]
        oQ = oBe + NV * NR;                        // [T1][DK]
        oU = oQ + T1 * DK;                         // [NV][T1][DK]  carried-back q
        oAcc = oU + NV * T1 * DK;                  // [NV][T1][DV]  sum_s beta_s kappa_s v_s
        // fold in matrix form over chunks of CH records (see the fold branch)
        constexpr int CH = kGdnFoldChunk;
        oGr = oAcc + NV * T1 * DV;                 // [L][CH]       k_s . k_t within each chunk
        oNm = oGr + L * CH;                        // [NV][L][CH]   coupling of records within a chunk
        oGW = oNm + NV * L * CH;                   // [NV][L][CH]   G (I + Nm)^-1 of each chunk
        oDd = oGW + NV * L * CH;                   // [NV][L]       a_s beta_s prod_{u<s} a_u
        oDc = oDd + NV * L;                        // [NV][L/CH+1]  decay of each chunk
        oX = (oDc + NV * (L / CH + 1) + 3) & ~3;   // [4 waves][16][36]  fold tiles' re-layout (16-byte aligned)
        total = oX + 4 * 16 * kGdnXStride;
    }
};

// One workgroup per (sequence, q/k head, chunk of its value heads).  The k records and
// q are shared by the value heads of one q/k head and staged once.  The carry-back
// chains run on the workgroup's waves (several chains of a wave in lockstep) while the
// first checkpoint tile is in flight; the workgroup then streams the value heads'
// [64, dk] checkpoint tiles, loading the next tile while it reduces the current one.
//
// Modes:
//   kGdnDecode  one autoregressive step; the record is stored at the cursor, and the
//               step that fills the buffer folds it into the checkpoint
//   kGdnFold    fold the stored records only (no outputs)
//   kGdnSpec    speculative verification of n_pos positions on the circular buffer:
//               window row s < committed is ring slot (head + s) % L, row committed + j
//               is position j; if committed + n_pos > L the committed rows are folded
//               first and every position's chain starts after them.
//
// Waves per SIMD: decode steps hold three (a flush step's fold re-lays its tiles through
// LDS, which fits in registers only at that occupancy, and the flush steps gain more than
// the others lose), speculative rounds four (their workgroups are shorter and need the
// occupancy), the explicit fold is unbounded.
template <int DK, int DV, typename IO, int MODE>
__global__ void __launch_bounds__(kGdnThreads, MODE == kGdnFold ? 1 : (MODE == kGdnDecode ? 3 : 4))
gdn_replay_kernel(GdnArgs a) {
    using io = Io<IO>;
    using Raw4 = typename io::Raw4;
    using S = GdnShape<DK>;
    constexpr int LPR = S::LPR, RPP = S::RPP, R = S::R, DVT = S::DVT;
    constexpr int NTILE = DV / DVT;
    constexpr int UPL = DK / kWave;  // u elements per lane in a carry-back wave
    constexpr int DK4 = DK / 4, DV4 = DV / 4;
    constexpr int NWAVE = kGdnThreads / kWave;
    // chains a wave runs in lockstep, and positions reduced together per tile (one: two
    // at a time spill registers in speculative rounds, which costs more than the extra
    // reductions)
    constexpr int TC = (MODE == kGdnSpec) ? 2 : 1;
    constexpr int TB = 1;
    extern __shared__ float smem[];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int HV = a.hv, HK = a.hk, L = a.L;
    const int rv = HV / HK;
    const int nchunk = a.nchunk;
    const int wid = blockIdx.x;
    const int chunk = wid % nchunk;
    const int bk = wid / nchunk;
    const int hk = bk % HK;
    const int hv0 = hk * rv + chunk * a.vheads_per_chunk;
    const int nv = min(a.vheads_per_chunk, rv - chunk * a.vheads_per_chunk);
    const bool lead = (hk == 0 && chunk == 0);
    // T: position stride of this call's inputs; Tb: positions of this sequence
    const int T = (MODE == kGdnSpec) ? a.n_pos : (MODE == kGdnDecode ? 1 : 0);

    // ---- state row, positions and cursors of this sequence ------------------------------
    // A pad row (state slot -1, or no positions) is skipped; a slot or position count
    // out of range, or a bad cursor, is flagged and skipped.  Skipped rows keep their
    // cursors (cursor_out = cursor_in) and report no flush.
    // Speculative rounds rank the folding sequences after three quarters of the others
    // (measured best between first and last); the ordering hands over the chosen
    // sequence's cursors.
    int b, sb, Tb, c = 0, hd = 0, cm = 0;
    if constexpr (MODE == kGdnSpec) {
        const SpecSeq q = spec_sequence_ranked<kGdnThreads>(bk / HK, a.batch, L, T, a.slot, a.n_pos_seq,
                                                            a.cursor_in, a.committed, 3, 4);
        // the pick is the same in every lane (it comes through LDS): keep it in scalar
        // registers, with everything derived from it
        b = __builtin_amdgcn_readfirstlane(q.b);
        sb = __builtin_amdgcn_readfirstlane(q.sb);
        Tb = __builtin_amdgcn_readfirstlane(q.Tb);
        hd = __builtin_amdgcn_readfirstlane(q.hd);
        cm = __builtin_amdgcn_readfirstlane(q.cm);
    } else {
        b = bk / HK;
        sb = a.slot ? a.slot[b] : b;
        Tb = T;
        c = a.cursor_in[b];
    }
    int err = 0;
    if (sb < -1 || sb >= (a.slot ? a.num_slots : a.batch)) err |= kDevErrSlot;
    if (Tb < 0 || Tb > T) err |= kDevErrCursor;
    if constexpr (MODE == kGdnSpec) {
        if (hd < 0 || hd >= L || cm < 0 || cm > L) err |= kDevErrCursor;
    } else {
        if (c < 0 || c >= L) err |= kDevErrCursor;
    }
    if (err || sb < 0 || (MODE == kGdnSpec && Tb == 0)) {
        if (tid == 0) {
            if (err && a.err_flags) atomicOr(a.err_flags, err);
            if (lead) {
                if (MODE == kGdnSpec) a.flushed[b] = 0;
                else a.cursor_out[b] = c;
            }
        }
        return;
    }
    const int nstored = (MODE == kGdnSpec) ? cm : c;   // window rows taken from the ring
    const int nrec = nstored + Tb;                      // window rows
    const bool fold = (MODE == kGdnFold) || (MODE == kGdnDecode && c + 1 == L) ||
                      (MODE == kGdnSpec && cm + Tb > L);
    const int nf = (MODE == kGdnSpec) ? cm : nrec;      // the fold covers rows [0, nf)
    const int st = fold ? nf : 0;                       // first row of every chain
    const bool idle = (MODE == kGdnFold) && c == 0;
    const size_t bHV = (size_t)b * HV;    // inputs and outputs: batch row
    const size_t sHV = (size_t)sb * HV;   // checkpoint and records: state row

    const GdnSmem lay(DK, DV, L, T, MODE, a.vheads_per_chunk, (int)sizeof(IO));
    const int NR = lay.NR, T1 = lay.T1;
    IO* sK = reinterpret_cast<IO*>(smem + lay.oK);   // exact copies of the k rows
    IO* sV = reinterpret_cast<IO*>(smem + lay.oV);
    float* sAl = smem + lay.oAl;
    float* sBe = smem + lay.oBe;
    float* sQ = smem + lay.oQ;
    float* sU = smem + lay.oU;
    float* sAcc = smem + lay.oAcc;

    const int row0 = tid / LPR;
    const int col4 = tid % LPR;
    auto tile_base = [&](int u) -> size_t {   // unit u = (value head u / NTILE, tile u % NTILE)
        const int vl = u / NTILE, tl = u % NTILE;
        return ((sHV + hv0 + vl) * DV + tl * DVT + row0) * (size_t)DK + 4 * col4;
    };
    auto issue_tile = [&](int u, float4 (&v)[R]) {
        const size_t t = tile_base(u);
#pragma unroll
        for (int k = 0; k < R; ++k) v[k] = ld_stream(a.ckpt + t + (size_t)k * RPP * DK);
    };
    // Fold steps compute on a tile in the lane mapping of the 16x16x4 matrix
    // instructions: wave w takes rows 16w..16w+15 of the 64, lane l row 16w + (l & 15)
    // and, in each 16-column block cb, columns 16cb + 4(l >> 4) .. +3 (R = DK/16 blocks).
    // That mapping touches 64 bytes of 16 rows per access, which streams 10-12% slower
    // than whole 128-byte lines, so fold tiles move in a chunk mapping instead -- registers
    // 2cc and 2cc+1 hold 32-column chunk cc of the wave's rows 0-7 and 8-15, lane l row
    // (l >> 3) of the eight and columns 32cc + 4(l & 7) .. +3, eight lanes a line -- and are
    // re-laid between the two through a buffer of the wave's own in LDS, one chunk (the
    // same two registers in both mappings) at a time.
    const int fr = lane & 15, fg = lane >> 4;
    static_assert(R * 16 == DK, "fold mapping: one 16-column block per tile register");
    constexpr int NCC = DK / 32;                      // 32-column chunks
    float* sX = smem + lay.oX + wave * 16 * kGdnXStride;
    // a lane's accesses to a fold tile, from one address between its two row halves (row
    // 16w + 4 + (l >> 3), column 4 (l & 7)): every access is then that address plus a
    // constant that fits the instructions' offset field
    auto tile_mid_c = [&](int u) -> const float* {
        const int vl = u / NTILE, tl = u % NTILE;
        return a.ckpt + ((sHV + hv0 + vl) * DV + tl * DVT + 16 * wave + 4 + (lane >> 3)) * (size_t)DK + 4 * (lane & 7);
    };
    auto issue_tile_f = [&](int u, float4 (&v)[R]) {
        const float* m = tile_mid_c(u);
#pragma unroll
        for (int cc = 0; cc < NCC; ++cc) {
            v[2 * cc] = ld_stream(m - 4 * DK + 32 * cc);
            v[2 * cc + 1] = ld_stream(m + 4 * DK + 32 * cc);
        }
    };
    // chunk mapping -> matrix mapping, in place (the wave's LDS accesses run in order, so
    // a chunk's reads come back before the next chunk's writes land)
    auto to_matrix = [&](float4 (&v)[R]) {
#pragma unroll
        for (int cc = 0; cc < NCC; ++cc) {
            *reinterpret_cast<float4*>(sX + (lane >> 3) * kGdnXStride + 4 * (lane & 7)) = v[2 * cc];
            *reinterpret_cast<float4*>(sX + (8 + (lane >> 3)) * kGdnXStride + 4 * (lane & 7)) = v[2 * cc + 1];
            v[2 * cc] = *reinterpret_cast<const float4*>(sX + fr * kGdnXStride + 4 * fg);
            v[2 * cc + 1] = *reinterpret_cast<const float4*>(sX + fr * kGdnXStride + 16 + 4 * fg);
        }
    };
    // matrix mapping -> chunk mapping, in place, each chunk then stored as whole lines
    auto store_tile_f = [&](int u, float4 (&v)[R]) {
        float* m = const_cast<float*>(tile_mid_c(u));
#pragma unroll
        for (int cc = 0; cc < NCC; ++cc) {
            *reinterpret_cast<float4*>(sX + fr * kGdnXStride + 4 * fg) = v[2 * cc];
            *reinterpret_cast<float4*>(sX + fr * kGdnXStride + 16 + 4 * fg) = v[2 * cc + 1];
            v[2 * cc] = *reinterpret_cast<const float4*>(sX + (lane >> 3) * kGdnXStride + 4 * (lane & 7));
            v[2 * cc + 1] = *reinterpret_cast<const float4*>(sX + (8 + (lane >> 3)) * kGdnXStride + 4 * (lane & 7));
            st_stream(m - 4 * DK + 32 * cc, v[2 * cc]);
            st_stream(m + 4 * DK + 32 * cc, v[2 * cc + 1]);
        }
    };
    const int nunit = nv * NTILE;
    float4 va[R], vb[R];

    // ---- window sources ----------------------------------------------------------------
    auto slot_of = [&](int s) {
        if constexpr (MODE == kGdnSpec) {
            const int t = hd + s;
            return t < L ? t : t - L;
        } else {
            return s;
        }
    };
    auto pos_qk = [&](int j) -> size_t {      // q/k offset of position j
        return (MODE == kGdnSpec) ? ((size_t)(b * T + j) * HK + hk) * DK : ((size_t)b * HK + hk) * DK;
    };
    auto pos_h = [&](int vl, int j) -> size_t {   // alpha/beta index of value head vl, position j
        return (MODE == kGdnSpec) ? (size_t)(b * T + j) * HV + hv0 + vl : bHV + hv0 + vl;
    };
    const IO* recK = reinterpret_cast<const IO*>(a.rec_k) + ((size_t)sb * HK + hk) * L * DK;
    const IO* kin = reinterpret_cast<const IO*>(a.k);
    const IO* qin = reinterpret_cast<const IO*>(a.q);
    const IO* vin = reinterpret_cast<const IO*>(a.v);
    const IO* recV = reinterpret_cast<const IO*>(a.rec_v);
    // window row s of each kind: a ring record (the explicit fold has no inputs, so its rows
    // -- none, for an empty buffer -- are records) or one of this call's positions
    auto rec_row = [&](int s) { return MODE == kGdnFold || s < nstored; };
    auto k_src = [&](int s) -> const IO* {
        return rec_row(s) ? recK + (size_t)slot_of(min(s, L - 1)) * DK : kin + pos_qk(s - nstored);
    };
    auto v_src = [&](int vl, int s) -> const IO* {
        return rec_row(s) ? recV + ((sHV + hv0 + vl) * L + slot_of(min(s, L - 1))) * DV
                          : vin + pos_h(vl, s - nstored) * DV;
    };
    auto ab_src = [&](const float* rec, const float* in, int vl, int s) -> const float* {
        return rec_row(s) ? rec + ((size_t)sb * L + slot_of(min(s, L - 1))) * HV + hv0 + vl : in + pos_h(vl, s - nstored);
    };

    // ---- staging requests ----------------------------------------------------------------
    // Up to a fixed number of staging tasks of each kind per thread (a longer window takes
    // the rest in loops below) are requested before the first checkpoint tile, with
    // clamped indices and no branch between the loads: loads retire in order, so staging
    // then waits on these alone and not on the tile requested after them.
    // Speculative rounds request one of each up front: their windows are longer, and
    // registers held for more spill in the fold (measured slower).
    constexpr int kPreK = (MODE == kGdnSpec) ? 1 : 2;   // k rows: nrec * DK / 4 tasks
    constexpr int kPreV = (MODE == kGdnSpec) ? 1 : 4;   // v rows: nv * nrec * DV / 4 tasks
    const int nKt = nrec * DK4, nVt = nv * nrec * DV4, nAt = nv * nrec;
    Raw4 preK[kPreK], preV[kPreV], preQ{};
    float preAl, preBe;
#pragma unroll
    for (int i = 0; i < kPreK; ++i) {
        const int task = min(tid + i * kGdnThreads, max(nKt - 1, 0));
        preK[i] = io::ldraw4(k_src(task / DK4), 4 * (task % DK4));
    }
#pragma unroll
    for (int i = 0; i < kPreV; ++i) {
        const int task = min(tid + i * kGdnThreads, max(nVt - 1, 0));
        const int vs = task / DV4, vl = vs / max(nrec, 1);
        preV[i] = io::ldraw4(v_src(vl, vs - vl * max(nrec, 1)), 4 * (task % DV4));
    }
    {
        const int task = min(tid, max(nAt - 1, 0));
        const int s = task / nv, vl = task - s * nv;   // a slot's value heads are contiguous
        preAl = *ab_src(a.rec_alpha, a.alpha, vl, s);
        preBe = *ab_src(a.rec_beta, a.beta, vl, s);
    }
    if constexpr (MODE != kGdnFold) {
        const int task = min(tid, max(Tb * DK4 - 1, 0));
        preQ = io::ldraw4(qin, pos_qk(task / DK4) + 4 * (task % DK4));
    }
    if (!idle) {
        if (fold) issue_tile_f(0, va);
        else issue_tile(0, va);
    }

    // ---- stage the window -------------------------------------------------------------
#pragma unroll
    for (int i = 0; i < kPreK; ++i) {
        const int task = tid + i * kGdnThreads;
        if (task < nKt) *reinterpret_cast<Raw4*>(sK + 4 * task) = preK[i];   // row task / DK4
    }
    for (int task = tid + kPreK * kGdnThreads; task < nKt; task += kGdnThreads)
        *reinterpret_cast<Raw4*>(sK + 4 * task) = io::ldraw4(k_src(task / DK4), 4 * (task % DK4));
    auto stage_v = [&](int task, Raw4 r) {
        const int vs = task / DV4, vl = vs / nrec, s = vs - vl * nrec;
        *reinterpret_cast<Raw4*>(sV + (vl * NR + s) * DV + 4 * (task % DV4)) = r;
    };
#pragma unroll
    for (int i = 0; i < kPreV; ++i) {
        const int task = tid + i * kGdnThreads;
        if (task < nVt) stage_v(task, preV[i]);
    }
    for (int task = tid + kPreV * kGdnThreads; task < nVt; task += kGdnThreads) {
        const int vs = task / DV4, vl = vs / nrec;
        stage_v(task, io::ldraw4(v_src(vl, vs - vl * nrec), 4 * (task % DV4)));
    }
    for (int task = tid; task < nAt; task += kGdnThreads) {
        const int s = task / nv, vl = task - s * nv;
        sAl[vl * NR + s] = task == tid ? preAl : *ab_src(a.rec_alpha, a.alpha, vl, s);
        sBe[vl * NR + s] = task == tid ? preBe : *ab_src(a.rec_beta, a.beta, vl, s);
    }
    if (tid < Tb * DK4) *reinterpret_cast<float4*>(sQ + 4 * tid) = io::cvt4(preQ);   // row tid / DK4
    for (int task = tid + kGdnThreads; task < Tb * DK4; task += kGdnThreads)
        *reinterpret_cast<float4*>(sQ + 4 * task) = io::cvt4(io::ldraw4(qin, pos_qk(task / DK4) + 4 * (task % DK4)));
    __syncthreads();

    const int q = tid % LPR;
    const int ridx = q / (LPR / R);
    const int iw = row0 + ridx * RPP;               // row (within a tile) this lane writes
    const bool writer = (q % (LPR / R)) == 0;
    const float scale = a.scale;

    // ---- carry each position's q back through its window --------------------------------
    // Position j's chain covers rows nstored + j down to st.  A wave runs TC chains of
    // one value head in lockstep over the rows (they share k_s, alpha_s and beta_s).
    // The record terms sum_s beta_s kappa_s v_s[i] ride along: beta_s kappa_s is the
    // same in every lane after the all-reduce, and each lane adds its own columns i.
    constexpr int VPL = DV / kWave;  // record-term columns per lane
    if (Tb > 0) {
        const int ngrp = (Tb + TC - 1) / TC;
        for (int task = wave; task < nv * ngrp; task += NWAVE) {
            const int vl = task / ngrp, j0 = (task - vl * ngrp) * TC;
            float u[TC][UPL];
#pragma unroll
            for (int cc = 0; cc < TC; ++cc) {
                const int j = min(j0 + cc, Tb - 1);
#pragma unroll
                for (int m = 0; m < UPL; ++m) u[cc][m] = sQ[j * DK + lane + m * kWave];
            }
            const float* al = sAl + vl * NR;
            const float* be = sBe + vl * NR;
            const int jtop = min(j0 + TC, Tb) - 1;
            float acc[TC][VPL];
#pragma unroll
            for (int cc = 0; cc < TC; ++cc)
#pragma unroll
                for (int m = 0; m < VPL; ++m) acc[cc][m] = 0.f;
            for (int s = nstored + jtop; s >= st; --s) {
                float kap[TC];
#pragma unroll
                for (int cc = 0; cc < TC; ++cc) {
                    kap[cc] = 0.f;
#pragma unroll
                    for (int m = 0; m < UPL; ++m) kap[cc] += io::ld(sK, s * DK + lane + m * kWave) * u[cc][m];
                }
#pragma unroll
                for (int cc = 0; cc < TC; ++cc) kap[cc] = group_allreduce<kWave>(kap[cc], lane);
                const float as = al[s], bs = be[s];
                float vs[VPL];
#pragma unroll
                for (int m = 0; m < VPL; ++m) vs[m] = io::ld(sV, (vl * NR + s) * DV + lane + m * kWave);
#pragma unroll
                for (int cc = 0; cc < TC; ++cc) {
                    const int j = min(j0 + cc, Tb - 1);
                    const bool on = s <= nstored + j;     // row s lies in position j's window
                    const float bk = on ? bs * kap[cc] : 0.f;
#pragma unroll
                    for (int m = 0; m < VPL; ++m) acc[cc][m] += bk * vs[m];
                    if (on) {
#pragma unroll
                        for (int m = 0; m < UPL; ++m) u[cc][m] = as * (u[cc][m] - bk * io::ld(sK, s * DK + lane + m * kWave));
                    }
                }
            }
#pragma unroll
            for (int cc = 0; cc < TC; ++cc) {
                if (j0 + cc < Tb) {
#pragma unroll
                    for (int m = 0; m < UPL; ++m) sU[(vl * T1 + j0 + cc) * DK + lane + m * kWave] = u[cc][m];
#pragma unroll
                    for (int m = 0; m < VPL; ++m) sAcc[(vl * T1 + j0 + cc) * DV + lane + m * kWave] = acc[cc][m];
                }
            }
        }
        __syncthreads();
    }

    // outputs of unit u from its tile: scale * (ckpt u_j + acc_j) for every position j
    auto out_index = [&](int vl, int j, int i) -> size_t {
        return (MODE == kGdnSpec) ? ((size_t)(b * T + j) * HV + hv0 + vl) * DV + i
                                  : (bHV + hv0 + vl) * DV + i;
    };
    auto outputs = [&](int u, const float4 (&v)[R]) {
        const int vl = u / NTILE, tl = u % NTILE;
        if constexpr (MODE == kGdnDecode) {
            const float4 Uv = *reinterpret_cast<const float4*>(sU + vl * DK + 4 * col4);
            float acc[R];
#pragma unroll
            for (int k = 0; k < R; ++k) acc[k] = dot4(v[k], Uv);
            const float r = row_reduce<R, LPR>(acc, lane);
            if (writer) {
                const int i = tl * DVT + iw;
                sAcc[vl * DV + i] = scale * (r + sAcc[vl * DV + i]);
            }
        } else if constexpr (MODE == kGdnSpec) {
            for (int j0 = 0; j0 < Tb; j0 += TB) {
                float acc[R * TB];
#pragma unroll
                for (int jj = 0; jj < TB; ++jj) {
                    const int j = min(j0 + jj, Tb - 1);
                    const float4 Uv = *reinterpret_cast<const float4*>(sU + (vl * T1 + j) * DK + 4 * col4);
#pragma unroll
                    for (int k = 0; k < R; ++k) acc[jj * R + k] = dot4(v[k], Uv);
                }
                const float r = row_reduce<R * TB, LPR>(acc, lane);
                const int vi = q / (LPR / (R * TB));          // value index this lane holds
                const int j = j0 + vi / R;
                const int i = tl * DVT + row0 + (vi % R) * RPP;
                if ((q % (LPR / (R * TB))) == 0 && j < Tb)
                    sAcc[(vl * T1 + j) * DV + i] = scale * (r + sAcc[(vl * T1 + j) * DV + i]);
            }
        }
    };
    auto rotate = [&]() {
#pragma unroll
        for (int k = 0; k < R; ++k) va[k] = vb[k];
    };

    if (!fold) {
        for (int u = 0; u + 1 < nunit; ++u) {
            issue_tile(u + 1, vb);
            outputs(u, va);
            rotate();
        }
        outputs(nunit - 1, va);
    } else if (!idle) {
        // ---- fold rows [0, nf) into the checkpoint -----------------------------------------
        // Matrix form over chunks of up to CH records (s = 0..nc-1 within a chunk, oldest
        // first).  Each record updates every row r of the tile as
        //     r <- a_s r + e_s k_s,   e_s = beta_s v_s[i] - a_s beta_s (r . k_s)
        // with a_s = alpha_s.  Unrolling the chunk, e solves (I + Nm) e = beta o v_i - D K r0
        // with Nm[s][t] = a_s beta_s (prod_{t<u<s} a_u) (k_t . k_s) for t < s and D =
        // diag(a_s beta_s prod_{u<s} a_u), so after the chunk
        //     r <- P r0 + K^T c,   c = GW (beta o v_i - D (K r0)),   GW = G (I + Nm)^-1,
        // P the chunk's decay and G = diag(prod_{u>t} a_u).  GW is a CH x CH matrix per
        // value head and chunk, formed before the tile loop by forward substitution (one
        // column per thread); each tile row then needs the nc dots K r0, one CH x CH
        // product and the rank-nc update, all on the matrix cores.
        constexpr int CH = kGdnFoldChunk;
        const int nch = (nf + CH - 1) / CH;
        // the second tile streams while the fold is prepared; afterwards tile u+1 is in
        // flight while tile u is folded and tile u+2 is requested once u is done (the last
        // two units are peeled so that every request is unconditional)
        if (nunit > 1) issue_tile_f(1, vb);
        float* sGr = smem + lay.oGr;
        float* sNm = smem + lay.oNm;
        float* sGW = smem + lay.oGW;
        float* sDd = smem + lay.oDd;
        float* sDc = smem + lay.oDc;
        const int NDC = L / CH + 1;
        // Gram matrix of the k rows within each chunk, shared by the value heads:
        // sGr[s][y] = k_s . k_t for the chunk's earlier row t = s - (s % CH) + y
        for (int pr = tid; pr < nf * CH; pr += kGdnThreads) {
            const int s = pr / CH, y = pr % CH, x = s % CH;
            if (y < x) {
                const int t = s - x + y;
                float m = 0.f;
                for (int jj = 0; jj < DK4; ++jj) {
                    const int j4 = (jj + pr) % DK4;     // rotated start: fewer bank conflicts
                    m += dot4(io::ld4(sK, s * DK + 4 * j4), io::ld4(sK, t * DK + 4 * j4));
                }
                sGr[pr] = m;
            }
        }
        // per value head and record: d_s = a_s beta_s prod_{u<s} a_u (products over the
        // chunk's records), and each chunk's decay
        for (int pr = tid; pr < nv * nch; pr += kGdnThreads) {
            const int vl = pr / nch, ch = pr - vl * nch;
            const float* al = sAl + vl * NR;
            const float* be = sBe + vl * NR;
            const int s0 = ch * CH, nc = min(CH, nf - s0);
            float pf = 1.f;
            for (int x = 0; x < nc; ++x) {
                sDd[vl * L + s0 + x] = al[s0 + x] * be[s0 + x] * pf;
                pf *= al[s0 + x];
            }
            sDc[vl * NDC + ch] = pf;
        }
        __syncthreads();
        // Nm[s][t] = a_s beta_s (prod_{t<u<s} a_u) (k_t . k_s), per value head.  The decay
        // between two records is a product of the gates in between, never a ratio of
        // running products: those reach zero in fp32 when gates are small, and 0/0 is NaN.
        for (int pr = tid; pr < nv * nf * CH; pr += kGdnThreads) {
            const int vl = pr / (nf * CH), sy = pr - vl * nf * CH;
            const int s = sy / CH, y = sy % CH, x = s % CH;
            if (y < x) {
                const float* al = sAl + vl * NR;
                const int t = s - x + y;
                float g = al[s] * sBe[vl * NR + s];
#pragma unroll
                for (int w = 1; w < CH - 1; ++w) {
                    const int uu = t + w;
                    const float f = al[min(uu, s)];
                    g *= (uu < s) ? f : 1.f;
                }
                sNm[vl * L * CH + sy] = g * sGr[sy];
            }
        }
        __syncthreads();
        // GW = G (I + Nm)^-1 per value head and chunk: column j of W by forward
        // substitution, W[x][j] = [x == j] - sum_{y<x} Nm[x][y] W[y][j] (the terms y < j
        // vanish: W is lower triangular), then row t scaled by g_t = prod_{u>t} a_u.  One
        // wave per (value head, chunk), 16 of its lanes; rows and columns past the chunk's
        // records are zero (the rows of Nm there are never written, and only feed rows
        // that are masked).
        for (int vc = wave; vc < nv * nch; vc += NWAVE) {
            const int j = lane;
            const int vl = vc / nch, ch = vc - vl * nch;
            const int s0 = ch * CH, nc = min(CH, nf - s0);
            if (j < CH) {
                const float* al = sAl + vl * NR;
                const float* nm = sNm + vl * L * CH + s0 * CH;
                float wc[CH];
#pragma unroll
                for (int x = 0; x < CH; ++x) {
                    float acc = (x == j) ? 1.f : 0.f;
#pragma unroll
                    for (int y = 0; y < x; ++y) acc -= nm[x * CH + y] * wc[y];
                    wc[x] = (x < nc) ? acc : 0.f;
                }
                float gs = 1.f;
#pragma unroll
                for (int x = CH - 1; x >= 0; --x) {
                    if (s0 + x < L) sGW[vl * L * CH + (s0 + x) * CH + j] = (j < nc) ? gs * wc[x] : 0.f;
                    if (x < nc) gs *= al[s0 + x];
                }
            }
        }
        __syncthreads();
        auto body = [&](int u) {
            const int vl = u / NTILE, tl = u % NTILE;
            const int i = tl * DVT + 16 * wave + fr;          // this lane's row of the value head
            const float* be = sBe + vl * NR;
            to_matrix(va);
            for (int ch = 0; ch < nch; ++ch) {
                const int s0 = ch * CH, nc = min(CH, nf - s0);
                // w[s][row] = k_s . row for the chunk's records s < 16 (rows past nc read as
                // zero); lane l ends with s = 4(l >> 4) + j, j < 4, of its row
                rssm_v4f w = {0.f, 0.f, 0.f, 0.f};
                const bool srow = fr < nc;
#pragma unroll
                for (int cb = 0; cb < R; ++cb) {
                    const float4 kr = srow ? io::ld4(sK, (s0 + fr) * DK + 16 * cb + 4 * fg)
                                          : make_float4(0.f, 0.f, 0.f, 0.f);
                    w = __builtin_amdgcn_mfma_f32_16x16x4f32(kr.x, va[cb].x, w, 0, 0, 0);
                    w = __builtin_amdgcn_mfma_f32_16x16x4f32(kr.y, va[cb].y, w, 0, 0, 0);
                    w = __builtin_amdgcn_mfma_f32_16x16x4f32(kr.z, va[cb].z, w, 0, 0, 0);
                    w = __builtin_amdgcn_mfma_f32_16x16x4f32(kr.w, va[cb].w, w, 0, 0, 0);
                }
                // c = GW y with y_s = beta_s v_s[i] - d_s w_s: the k index of matrix
                // instruction j is record 4(l >> 4) + j on both operands, so each lane's y
                // values feed the instructions as they are; lane l ends with c_t, t = 4(l >> 4)
                // + j, of its row
                rssm_v4f cm = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int sj = 4 * fg + j;
                    const float y = (sj < nc) ? be[s0 + sj] * io::ld(sV, (vl * NR + s0 + sj) * DV + i) -
                                                    sDd[vl * L + s0 + sj] * w[j]
                                              : 0.f;
                    const float gw = srow ? sGW[vl * L * CH + (s0 + fr) * CH + sj] : 0.f;   // rows past nc: zero
                    cm = __builtin_amdgcn_mfma_f32_16x16x4f32(gw, y, cm, 0, 0, 0);
                }
                const float dc = sDc[vl * NDC + ch];
                // row += sum_t c_t k_t, as (block of 16 columns)^T += K^T c^T: the k index of
                // matrix instruction j is record 4(l >> 4) + j on both operands
#pragma unroll
                for (int cb = 0; cb < R; ++cb) {
                    rssm_v4f acc = {dc * va[cb].x, dc * va[cb].y, dc * va[cb].z, dc * va[cb].w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int t = 4 * fg + j;
                        const float kv = (t < nc) ? io::ld(sK, (s0 + t) * DK + 16 * cb + fr) : 0.f;
                        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kv, cm[j], acc, 0, 0, 0);
                    }
                    va[cb] = make_float4(acc[0], acc[1], acc[2], acc[3]);
                }
            }
            // outputs from the new rows (each row is spread over the 4 lanes l, l^16, l^32,
            // l^48), then the rows go back to the chunk mapping and are stored
            if constexpr (MODE != kGdnFold) {
                for (int j = 0; j < Tb; ++j) {
                    float part = 0.f;
#pragma unroll
                    for (int cb = 0; cb < R; ++cb)
                        part += dot4(va[cb], *reinterpret_cast<const float4*>(sU + (vl * T1 + j) * DK + 16 * cb + 4 * fg));
                    part = exchange<16>(part, part, lane);
                    part = exchange<32>(part, part, lane);
                    if (fg == 0) sAcc[(vl * T1 + j) * DV + i] = scale * (part + sAcc[(vl * T1 + j) * DV + i]);
                }
            }
            store_tile_f(u, va);
        };
        for (int u = 0; u + 2 < nunit; ++u) {
            body(u);
            rotate();
            issue_tile_f(u + 2, vb);
        }
        if (nunit > 1) {
            body(nunit - 2);
            rotate();
        }
        body(nunit - 1);
    }

    // ---- store the outputs ----------------------------------------------------------------
    // Each output replaced its record term in sAcc (the lane that reads an entry writes it);
    // the workgroup's outputs of one position are one contiguous block of nv * DV floats,
    // stored in one coalesced pass rather than as scattered words between the checkpoint
    // loads.
    if constexpr (MODE != kGdnFold) {
        __syncthreads();
        for (int task = tid; task < Tb * nv * DV4; task += kGdnThreads) {
            const int i4 = task % DV4, jv = task / DV4;
            const int j = jv / nv, vl = jv - j * nv;
            *reinterpret_cast<float4*>(a.out + out_index(vl, j, 4 * i4)) =
                *reinterpret_cast<const float4*>(sAcc + (vl * T1 + j) * DV + 4 * i4);
        }
    }

    // ---- append this call's records ---------------------------------------------------
    if constexpr (MODE == kGdnDecode) {
        if (!fold) {
            // the step's record is staged in LDS as an exact copy (row c of the window)
            for (int task = tid; task < nv * DV4; task += kGdnThreads) {
                const int vl = task / DV4, i4 = task % DV4;
                const size_t sv = sHV + hv0 + vl;
                io::straw4(reinterpret_cast<IO*>(a.rec_v), (sv * L + c) * DV + 4 * i4,
                           *reinterpret_cast<const Raw4*>(sV + (vl * NR + c) * DV + 4 * i4));
            }
            for (int vl = tid; vl < nv; vl += kGdnThreads) {
                const size_t g = ((size_t)sb * L + c) * HV + hv0 + vl;
                a.rec_alpha[g] = sAl[vl * NR + c];
                a.rec_beta[g] = sBe[vl * NR + c];
            }
            if (chunk == 0) {
                for (int j4 = tid; j4 < DK4; j4 += kGdnThreads)
                    io::straw4(reinterpret_cast<IO*>(a.rec_k), (((size_t)sb * HK + hk) * L + c) * DK + 4 * j4,
                               *reinterpret_cast<const Raw4*>(sK + c * DK + 4 * j4));
            }
        }
    } else if constexpr (MODE == kGdnSpec) {
        // Every ring row this workgroup reads was staged before the first barrier, so
        // position slots may replace committed ones here (rounds that fold).
        const int slot0 = hd + cm;
        for (int task = tid; task < nv * Tb * DV4; task += kGdnThreads) {
            const int i4 = task % DV4, vj = task / DV4;
            const int vl = vj / Tb, j = vj - vl * Tb;
            const size_t hv = sHV + hv0 + vl;
            io::straw4(reinterpret_cast<IO*>(a.rec_v), (hv * L + (slot0 + j) % L) * DV + 4 * i4,
                       *reinterpret_cast<const Raw4*>(sV + (vl * NR + nstored + j) * DV + 4 * i4));
        }
        for (int task = tid; task < nv * Tb; task += kGdnThreads) {
            const int j = task / nv, vl = task - j * nv;
            const size_t g = ((size_t)sb * L + (slot0 + j) % L) * HV + hv0 + vl;
            a.rec_alpha[g] = sAl[vl * NR + nstored + j];
            a.rec_beta[g] = sBe[vl * NR + nstored + j];
        }
        // the q/k head's k records: with several workgroups per q/k head the host
        // appends them in a separate launch
        if (nchunk == 1) {
            for (int task = tid; task < Tb * DK4; task += kGdnThreads) {
                const int j = task / DK4, j4 = task % DK4;
                io::straw4(reinterpret_cast<IO*>(a.rec_k), (((size_t)sb * HK + hk) * L + (slot0 + j) % L) * DK + 4 * j4,
                           io::ldraw4(kin, pos_qk(j) + 4 * j4));
            }
        }
    }

    if (tid == 0 && lead) {
        if (MODE == kGdnSpec) a.flushed[b] = fold ? 1 : 0;
        else a.cursor_out[b] = fold ? 0 : c + 1;
    }
}

// Appends a speculative round's k vectors to each q/k head's ring (slots
// (head + committed + j) % L) when a q/k head's value heads are split over several
// workgroups.  Runs after the verify kernel on the same stream, so every workgroup has
// finished reading the slots it replaces.
template <int DK, typename IO>
__global__ void __launch_bounds__(kGdnThreads) gdn_spec_append_k_kernel(GdnArgs a) {
    using io = Io<IO>;
    constexpr int DK4 = DK / 4;
    const int HK = a.hk, L = a.L, T = a.n_pos;
    const size_t total = (size_t)a.batch * T * HK * DK4;
    for (size_t i = (size_t)blockIdx.x * kGdnThreads + threadIdx.x; i < total;
         i += (size_t)gridDim.x * kGdnThreads) {
        const int j4 = (int)(i % DK4);
        size_t r = i / DK4;
        const int hk = (int)(r % HK);
        r /= HK;
        const int j = (int)(r % T);
        const int b = (int)(r / T);
        const int sb = a.slot ? a.slot[b] : b;
        const int Tb = a.n_pos_seq ? a.n_pos_seq[b] : T;
        const int hd = a.cursor_in[b], cm = a.committed[b];
        if (hd < 0 || hd >= L || cm < 0 || cm > L) continue;
        if (sb < 0 || sb >= (a.slot ? a.num_slots : a.batch) || Tb < 0 || Tb > T || j >= Tb) continue;
        const int slot = (hd + cm + j) % L;
        io::straw4(reinterpret_cast<IO*>(a.rec_k), (((size_t)sb * HK + hk) * L + slot) * DK + 4 * j4,
                   io::ldraw4(reinterpret_cast<const IO*>(a.k), (((size_t)b * T + j) * HK + hk) * DK + 4 * j4));
    }
}

// Conventional step: S <- alpha (S - beta (S k) k^T) + beta v k^T, o = scale S q, with
// one read and one write of the state.  Uses S_new q = alpha (S q - beta (S k)(k.q)) +
// beta v (k.q), so both row dots come from the state as loaded.  SNAP: per-position
// snapshot baseline for speculative decoding -- read snapshot slot_in[b] of
// [B, n_pos, HV, dv, dk], run the n_pos updates and store the state after each.
//
// Every state row i of a value head is updated and reduced on its own, so the kernel is
// cut as the Mamba2 conventional kernel is: dk/4 lanes per row with one 16-byte access
// each, RPT rows per thread, one workgroup per (256 / (dk/4)) * RPT consecutive rows of
// one value head, whose (b, hv) is computed once per workgroup.
#ifndef RSSM_CONV_RPT
#define RSSM_CONV_RPT 2
#endif
constexpr int kGdnConvMaxGrid = 1 << 24;   // workgroups per launch; larger problems loop
constexpr int kGdnConvPosGroup = 4;        // snapshot baseline: positions whose inputs load together

template <int DK, int DV>
struct GdnConvShape {
    static constexpr int LPR = DK / 4;                  // lanes per state row
    static constexpr int RPP = kGdnThreads / LPR;       // rows per pass of the workgroup
    static constexpr int RPT = (DV / RPP >= RSSM_CONV_RPT) ? RSSM_CONV_RPT : 1;
    static constexpr int RW = RPP * RPT;                // rows per workgroup (divides DV)
    static_assert(DV % RW == 0, "a workgroup stays inside one value head");
};

// One position's small inputs of a conventional GDN step, as loaded.
template <int RPT>
struct GdnConvInputs {
    float4 K, Q;
    float al, be;
    float vi[RPT];
};

template <int DK, int DV, typename IO, bool SNAP>
__global__ void __launch_bounds__(kGdnThreads) gdn_conventional_kernel(GdnArgs a) {
    using io = Io<IO>;
    using Sh = GdnConvShape<DK, DV>;
    constexpr int LPR = Sh::LPR, RPP = Sh::RPP, RPT = Sh::RPT, RW = Sh::RW;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int row0 = tid / LPR;
    const int col4 = tid % LPR;
    const int HV = a.hv, HK = a.hk;
    const int rv = HV / HK;
    const int T = SNAP ? a.n_pos : 1;
    const int64_t nchunks = (int64_t)a.batch * HV * (DV / RW);
    constexpr size_t SS = (size_t)DV * DK;   // one value head's state
    const IO* kin = reinterpret_cast<const IO*>(a.k);
    const IO* qin = reinterpret_cast<const IO*>(a.q);
    const IO* vin = reinterpret_cast<const IO*>(a.v);
    const int q = tid % LPR;
    const int ridx = q / (LPR / RPT);                   // row this lane writes after the reduce
    const bool writer = (q % (LPR / RPT)) == 0;

    for (int64_t chunk = blockIdx.x; chunk < nchunks; chunk += gridDim.x) {
        const int64_t bhv = chunk / (DV / RW);
        const int i = (int)(chunk % (DV / RW)) * RW + row0;   // this lane's first row
        const int b = (int)(bhv / HV), hv = (int)(bhv - (int64_t)(bhv / HV) * HV);
        const int hk = hv / rv;
        size_t src;
        if constexpr (SNAP) {
            int sl = a.cursor_in[b];
            sl = sl < 0 ? 0 : (sl >= T ? T - 1 : sl);
            src = ((size_t)(b * T + sl) * HV + hv) * SS + (size_t)i * DK + 4 * col4;
        } else {
            src = (size_t)bhv * SS + (size_t)i * DK + 4 * col4;
        }
        float4 v[RPT];
#pragma unroll
        for (int k = 0; k < RPT; ++k) v[k] = ld_stream(a.ckpt + src + (size_t)k * RPP * DK);
        auto load_in = [&](int j) {
            const size_t ph = SNAP ? (size_t)(b * T + j) * HV + hv : (size_t)bhv;
            const size_t qk_off = (SNAP ? (size_t)(b * T + j) * HK + hk : (size_t)b * HK + hk) * DK;
            GdnConvInputs<RPT> in;
            in.K = io::ld4(kin, qk_off + 4 * col4);
            in.Q = io::ld4(qin, qk_off + 4 * col4);
            in.al = a.alpha[ph];
            in.be = a.beta[ph];
#pragma unroll
            for (int k = 0; k < RPT; ++k) in.vi[k] = io::ld(vin, ph * DV + i + k * RPP);
            return in;
        };
        // positions in unrolled groups of kGdnConvPosGroup, each group's inputs loaded
        // together (a loop-carried wait would hold every position until the previous
        // store landed)
        constexpr int GRP = SNAP ? kGdnConvPosGroup : 1;
        for (int j0 = 0; j0 < T; j0 += GRP) {
            GdnConvInputs<RPT> in[GRP];
#pragma unroll
            for (int jj = 0; jj < GRP; ++jj) in[jj] = load_in(min(j0 + jj, T - 1));   // no branch between loads
#pragma unroll
            for (int jj = 0; jj < GRP; ++jj) {
                const int j = j0 + jj;
                if (j < T) {
                    const float4 Kv = in[jj].K, Qv = in[jj].Q;
                    const float al = in[jj].al, be = in[jj].be;
                    const float kq = group_allreduce<LPR>(dot4(Kv, Qv), lane);
                    float d[RPT], e[RPT];
#pragma unroll
                    for (int k = 0; k < RPT; ++k) {
                        d[k] = dot4(v[k], Kv);
                        e[k] = dot4(v[k], Qv);
                    }
                    row_allreduce<RPT, LPR>(d, lane);     // every lane needs its rows' S k
                    const float er = row_reduce<RPT, LPR>(e, lane);
                    const size_t dst = SNAP ? ((size_t)(b * T + j) * HV + hv) * SS + (size_t)i * DK + 4 * col4 : src;
                    float dw = d[0], vw = in[jj].vi[0];
#pragma unroll
                    for (int k = 0; k < RPT; ++k) {
                        const float bd = be * d[k];
                        const float bv = be * in[jj].vi[k];
                        v[k].x = al * (v[k].x - bd * Kv.x) + bv * Kv.x;
                        v[k].y = al * (v[k].y - bd * Kv.y) + bv * Kv.y;
                        v[k].z = al * (v[k].z - bd * Kv.z) + bv * Kv.z;
                        v[k].w = al * (v[k].w - bd * Kv.w) + bv * Kv.w;
                        st_stream(a.ckpt + dst + (size_t)k * RPP * DK, v[k]);
                        dw = (k == ridx) ? d[k] : dw;
                        vw = (k == ridx) ? in[jj].vi[k] : vw;
                    }
                    if (writer) {
                        const size_t ph = SNAP ? (size_t)(b * T + j) * HV + hv : (size_t)bhv;
                        a.out[ph * DV + i + ridx * RPP] = a.scale * (al * (er - be * dw * kq) + be * vw * kq);
                    }
                }
            }
        }
    }
}

bool gdn_shape_supported(int dk, int dv) {
    return (dk == 64 || dk == 128) && (dv == 64 || dv == 128);
}

static int gdn_positions(int mode, int n_pos) {
    return (mode == kGdnSpec) ? n_pos : (mode == kGdnDecode ? 1 : 0);
}

// Value heads per workgroup: up to kGdnMaxVHeads, fewer when one workgroup's LDS
// staging would not fit; the last chunk of a q/k head takes the remainder.
static void gdn_chunking(int dk, int dv, int L, int rv, int mode, int n_pos, int io_bytes, int* nchunk,
                         int* per) {
    const int T = gdn_positions(mode, n_pos);
    int p = rv < kGdnMaxVHeads ? rv : kGdnMaxVHeads;
    while (p > 1 && sizeof(float) * (size_t)GdnSmem(dk, dv, L, T, mode, p, io_bytes).total > kGdnMaxSmemBytes) --p;
    *per = p;
    *nchunk = (rv + p - 1) / p;
}

size_t gdn_smem_bytes(int dk, int dv, int L, int rv, int mode, int n_pos, int io_bytes) {
    int nchunk, per;
    gdn_chunking(dk, dv, L, rv, mode, n_pos, io_bytes, &nchunk, &per);
    return sizeof(float) * (size_t)GdnSmem(dk, dv, L, gdn_positions(mode, n_pos), mode, per, io_bytes).total;
}

template <int DK, int DV, typename IO>
static const void* gdn_pick_mode(int mode) {
    if (mode == kGdnFold) return (const void*)&gdn_replay_kernel<DK, DV, IO, kGdnFold>;
    if (mode == kGdnSpec) return (const void*)&gdn_replay_kernel<DK, DV, IO, kGdnSpec>;
    return (const void*)&gdn_replay_kernel<DK, DV, IO, kGdnDecode>;
}

template <int DK, int DV>
static const void* gdn_pick(int io, int mode) {
    return io == kIoBF16 ? gdn_pick_mode<DK, DV, uint16_t>(mode) : gdn_pick_mode<DK, DV, float>(mode);
}

hipError_t launch_gdn_replay(const GdnArgs& a, int io, int mode, hipStream_t stream) {
    const void* fn = nullptr;
    if (a.dk == 64 && a.dv == 64) fn = gdn_pick<64, 64>(io, mode);
    if (a.dk == 64 && a.dv == 128) fn = gdn_pick<64, 128>(io, mode);
    if (a.dk == 128 && a.dv == 64) fn = gdn_pick<128, 64>(io, mode);
    if (a.dk == 128 && a.dv == 128) fn = gdn_pick<128, 128>(io, mode);
    if (!fn) return hipErrorInvalidValue;
    GdnArgs args = a;
    if (mode != kGdnSpec) args.n_pos = (mode == kGdnDecode) ? 1 : 0;
    const int io_bytes = io == kIoBF16 ? 2 : 4;
    gdn_chunking(a.dk, a.dv, a.L, a.hv / a.hk, mode, args.n_pos, io_bytes, &args.nchunk, &args.vheads_per_chunk);
    const size_t smem = gdn_smem_bytes(a.dk, a.dv, a.L, a.hv / a.hk, mode, args.n_pos, io_bytes);
    void* kargs[] = {&args};
    const dim3 grid((unsigned)((size_t)a.batch * a.hk * args.nchunk));
    hipError_t e = hipLaunchKernel(fn, grid, dim3(kGdnThreads), kargs, smem, stream);
    if (e != hipSuccess || mode != kGdnSpec || args.nchunk == 1) return e;
    const void* app = nullptr;
    if (a.dk == 64)
        app = io == kIoBF16 ? (const void*)&gdn_spec_append_k_kernel<64, uint16_t>
                            : (const void*)&gdn_spec_append_k_kernel<64, float>;
    else
        app = io == kIoBF16 ? (const void*)&gdn_spec_append_k_kernel<128, uint16_t>
                            : (const void*)&gdn_spec_append_k_kernel<128, float>;
    const size_t total = (size_t)a.batch * args.n_pos * a.hk * (a.dk / 4);
    const size_t want = (total + kGdnThreads - 1) / kGdnThreads;
    const unsigned blocks = (unsigned)(want < 65536 ? want : 65536);
    return hipLaunchKernel(app, dim3(blocks), dim3(kGdnThreads), kargs, 0, stream);
}

template <int DK, int DV, typename IO>
static const void* gdn_conv_pick(bool snapshots) {
    return snapshots ? (const void*)&gdn_conventional_kernel<DK, DV, IO, true>
                     : (const void*)&gdn_conventional_kernel<DK, DV, IO, false>;
}

template <int DK, int DV>
static const void* gdn_conv_pick_io(int io, bool snapshots, int* rows_per_wg) {
    *rows_per_wg = GdnConvShape<DK, DV>::RW;
    return io == kIoBF16 ? gdn_conv_pick<DK, DV, uint16_t>(snapshots) : gdn_conv_pick<DK, DV, float>(snapshots);
}

hipError_t launch_gdn_conventional(const GdnArgs& a, int io, bool snapshots, hipStream_t stream) {
    const void* fn = nullptr;
    int rows_per_wg = 1;
    if (a.dk == 64 && a.dv == 64) fn = gdn_conv_pick_io<64, 64>(io, snapshots, &rows_per_wg);
    if (a.dk == 64 && a.dv == 128) fn = gdn_conv_pick_io<64, 128>(io, snapshots, &rows_per_wg);
    if (a.dk == 128 && a.dv == 64) fn = gdn_conv_pick_io<128, 64>(io, snapshots, &rows_per_wg);
    if (a.dk == 128 && a.dv == 128) fn = gdn_conv_pick_io<128, 128>(io, snapshots, &rows_per_wg);
    if (!fn) return hipErrorInvalidValue;
    GdnArgs args = a;
    if (!snapshots) args.n_pos = 1;
    void* kargs[] = {&args};
    const int64_t want = (int64_t)a.batch * a.hv * (a.dv / rows_per_wg);
    const dim3 grid((unsigned)(want < kGdnConvMaxGrid ? want : kGdnConvMaxGrid));
    return hipLaunchKernel(fn, grid, dim3(kGdnThreads), kargs, 0, stream);
}

}  // namespace rssm
