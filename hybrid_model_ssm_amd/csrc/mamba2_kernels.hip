// Mamba2 ReplaySSM kernels for gfx950.
//
// The method ("ReplaySSM Caches Inputs Instead of State to Speed Up Hybrid-Model
// Decoding", section "How ReplaySSM works"): the state is a checkpoint plus a buffer of
// recent input records.  A non-flush step appends its record and computes the output
// from the checkpoint and the buffer without storing a state; the step that fills the
// buffer folds the records into the checkpoint and stores it once.  Unrolling the
// Mamba2 recurrence h = exp(dt A) h + dt x B^T over a window of records s (oldest
// first) gives, with lam_s = sum of dt over the window records after s:
//
//     decay = exp(A * sum_s dt_s),   w_s = dt_s * exp(A * lam_s)
//     y     = decay * (Hc . C_t) + sum_s w_s (B_s . C_t) x_s + D x_t
//     fold:   Hc <- decay * Hc + sum_s w_s x_s B_s^T
//
// Work decomposition: one 256-thread workgroup per (sequence, head) tile of the
// checkpoint ([headdim, dstate] fp32).  The tile is streamed once with 16-byte loads:
// LPR = dstate/4 consecutive lanes cover one row (one float4 each), so a wave load
// instruction reads whole contiguous rows, and each thread holds R rows of the tile.
// All loads are issued before the small per-window work (record staging in LDS,
// B_s . C_t dots, log-space decay sums), which hides that work under the HBM latency.
// Row dot products  Hc[p,:] . C  are finished with a transpose-reduce across the LPR
// lanes.  The flush fold is a rank-|window| update applied to the tile in registers.
//
// Modes share one kernel body:
//   kDecode  one autoregressive step (flushes in place when the buffer fills)
//   kFold    fold the stored records only (explicit flush / bf16 copy refresh)
//   kSpec    speculative verification over n_pos positions on the circular buffer
//            ("ReplaySSM" README, benefit "Cheap rollback": output-only verification,
//            rejected inputs dropped by moving a pointer)

#include "device_common.h"
#include "launch.h"

namespace rssm {

constexpr int kDecode = 0;
constexpr int kFold = 1;
constexpr int kSpec = 2;
constexpr int kThreads = 256;

struct SmemLayout {
    int nrec_max, T;
    int oB, oX, oC, oDt, oW, oCoef, oDec, total;
    __host__ __device__ SmemLayout(int P, int N, int L, int T_, int mode) {
        T = T_;
        nrec_max = (mode == kSpec) ? L + T_ : L;
        oB = 0;
        oX = oB + nrec_max * N;
        oC = oX + nrec_max * P;
        oDt = oC + (T > 0 ? T : 1) * N;
        oW = oDt + nrec_max;
        oCoef = oW + nrec_max;
        oDec = oCoef + (T > 0 ? T : 1) * nrec_max;
        total = oDec + (T > 0 ? T : 1) + 1;
    }
};

template <int N, int R, typename IO, bool LOWP, int MODE>
__global__ void __launch_bounds__(kThreads) mamba2_replay_kernel(Mamba2Args a) {
    using io = Io<IO>;
    constexpr int LPR = N / 4;            // lanes per checkpoint row
    constexpr int RPP = kThreads / LPR;   // rows per pass of the workgroup
    extern __shared__ float smem[];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int H = a.nheads, P = a.headdim, G = a.ngroups, L = a.L;
    const int hpg = H / G;
    const int bh = xcd_remap(blockIdx.x, gridDim.x);
    const int b = bh / H;
    const int h = bh - b * H;
    const int g = h / hpg;
    const int T = (MODE == kSpec) ? a.n_pos : (MODE == kDecode ? 1 : 0);

    // ---- cursors -------------------------------------------------------------------
    int c = 0, hd = 0, cm = 0;
    bool bad;
    if constexpr (MODE == kSpec) {
        hd = a.cursor_in[b];
        cm = a.committed[b];
        bad = hd < 0 || hd >= L || cm < 0 || cm > L;
    } else {
        c = a.cursor_in[b];
        bad = c < 0 || c >= L;
    }
    if (bad) {
        if (tid == 0) {
            if (a.err_flags) atomicOr(a.err_flags, 1);
            if (h == 0 && MODE != kSpec) a.cursor_out[b] = c;
        }
        return;
    }
    // window rows staged in LDS: [0, nrec); the fold covers rows [0, nf)
    const int nrec = (MODE == kSpec) ? cm + T : (MODE == kDecode ? c + 1 : c);
    const bool fold = (MODE == kFold) || (MODE == kDecode && c + 1 == L) ||
                      (MODE == kSpec && cm + T > L);
    const int nf = (MODE == kSpec) ? cm : nrec;
    const int st = fold ? nf : 0;  // first row of every output window
    const bool use_lp = LOWP && !fold;

    const SmemLayout lay(P, N, L, T, MODE);
    float* sB = smem + lay.oB;      // [nrec][N]  B records (+ positions)
    float* sX = smem + lay.oX;      // [nrec][P]  x records (+ positions)
    float* sC = smem + lay.oC;      // [T][N]
    float* sdt = smem + lay.oDt;    // [nrec]
    float* sw = smem + lay.oW;      // [nf]       fold weights
    float* scf = smem + lay.oCoef;  // [T][nrec]  output coefficients w*beta
    float* sdec = smem + lay.oDec;  // [T] output decays, [T] fold decay

    const int row0 = tid / LPR;
    const int col4 = tid - row0 * LPR;
    const size_t tile = (size_t)bh * P * N;

    // ---- 1. issue the checkpoint loads -------------------------------------------------
    float4 v[R];
    uint2 vl[R];
    if (MODE == kFold && c == 0 && !LOWP) {
        // nothing stored and no read copy to refresh
    } else if (use_lp) {
#pragma unroll
        for (int k = 0; k < R; ++k) {
            const int p = row0 + k * RPP;
            vl[k] = (p < P) ? *reinterpret_cast<const uint2*>(a.ckpt_lp + tile + (size_t)p * N + 4 * col4)
                            : make_uint2(0u, 0u);
        }
    } else {
#pragma unroll
        for (int k = 0; k < R; ++k) {
            const int p = row0 + k * RPP;
            v[k] = (p < P) ? *reinterpret_cast<const float4*>(a.ckpt + tile + (size_t)p * N + 4 * col4)
                           : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }

    // ---- 2. stage the window in LDS ---------------------------------------------------
    const float Ah = a.A[h];
    const IO* recB = reinterpret_cast<const IO*>(a.rec_B) + (size_t)(b * G + g) * L * N;
    const IO* recX = reinterpret_cast<const IO*>(a.rec_x) + (size_t)bh * L * P;
    const float* recdt = a.rec_dt + (size_t)bh * L;
    const IO* xin = reinterpret_cast<const IO*>(a.x);
    const IO* Bin = reinterpret_cast<const IO*>(a.B);
    const IO* Cin = reinterpret_cast<const IO*>(a.C);
    const IO* dtin = reinterpret_cast<const IO*>(a.dt_raw);
    const int nstored = (MODE == kSpec) ? cm : c;   // rows taken from the ring

    // ring slot of stored row s
    auto slot_of = [&](int s) { return (MODE == kSpec) ? (hd + s) % L : s; };
    // global offsets of position j's inputs
    auto pos_x = [&](int j) -> size_t {
        return (MODE == kSpec) ? ((size_t)(b * T + j) * H + h) * P : (size_t)bh * P;
    };
    auto pos_g = [&](int j) -> size_t {
        return (MODE == kSpec) ? ((size_t)(b * T + j) * G + g) * N : (size_t)(b * G + g) * N;
    };
    auto pos_h = [&](int j) -> size_t {
        return (MODE == kSpec) ? (size_t)(b * T + j) * H + h : (size_t)bh;
    };

    for (int i = tid; i < nrec * N; i += kThreads) {
        const int s = i / N, n = i - s * N;
        sB[i] = (s < nstored) ? io::ld(recB, (size_t)slot_of(s) * N + n)
                              : io::ld(Bin, pos_g(s - nstored) + n);
    }
    for (int i = tid; i < nrec * P; i += kThreads) {
        const int s = i / P, p = i - s * P;
        sX[i] = (s < nstored) ? io::ld(recX, (size_t)slot_of(s) * P + p)
                              : io::ld(xin, pos_x(s - nstored) + p);
    }
    for (int i = tid; i < T * N; i += kThreads) {
        const int j = i / N, n = i - j * N;
        sC[i] = io::ld(Cin, pos_g(j) + n);
    }
    for (int s = tid; s < nrec; s += kThreads) {
        float dt;
        if (s < nstored) {
            dt = recdt[slot_of(s)];
        } else {
            dt = io::ld(dtin, pos_h(s - nstored)) + a.dt_bias[h];
            if (a.dt_softplus) dt = softplus_f32(dt);
        }
        sdt[s] = dt;
    }
    __syncthreads();

    // ---- 3. window coefficients ------------------------------------------------------
    // fold: w_s = dt_s exp(A lam_s) over rows [0, nf); decay over all of them
    if (fold) {
        for (int s = tid; s < nf; s += kThreads) {
            float lam = 0.f;
            for (int r = s + 1; r < nf; ++r) lam += sdt[r];
            sw[s] = sdt[s] * expf(Ah * lam);
            if (s == 0) sdec[T] = expf(Ah * (lam + sdt[0]));
        }
        if (tid == 0 && nf == 0) sdec[T] = 1.f;
    }
    // outputs: position j's window is rows [st, e_j], e_j = nstored + j (decode: c)
    // beta = B_s . C_j over 16 lanes per (j, s) pair
    const int npairs = T * nrec;
    for (int base = 0; base < npairs; base += kThreads / 16) {
        const int pr = base + tid / 16;
        const int part = tid & 15;
        if (pr < npairs) {
            const int j = pr / nrec, s = pr - j * nrec;
            const int e = nstored + j;
            float beta = 0.f;
            for (int n = part; n < N; n += 16) beta += sB[s * N + n] * sC[j * N + n];
            beta += __shfl_xor(beta, 8);
            beta += __shfl_xor(beta, 4);
            beta += __shfl_xor(beta, 2);
            beta += __shfl_xor(beta, 1);
            if (part == 0 && s >= st && s <= e) {
                float lam = 0.f;
                for (int r = s + 1; r <= e; ++r) lam += sdt[r];
                scf[j * nrec + s] = sdt[s] * expf(Ah * lam) * beta;
                if (s == st) sdec[j] = expf(Ah * (lam + sdt[s]));
            }
        }
    }
    for (int j = tid; j < T; j += kThreads)
        if (st > nstored + j) sdec[j] = 1.f;  // empty window: output straight from the new checkpoint
    __syncthreads();

    // ---- 4. consume the checkpoint tile ---------------------------------------------
    if (MODE == kFold && c == 0 && !LOWP) {
        // nothing to fold and nothing to refresh
    } else if (fold) {
        const float decf = sdec[T];
#pragma unroll
        for (int k = 0; k < R; ++k) {
            v[k].x *= decf; v[k].y *= decf; v[k].z *= decf; v[k].w *= decf;
        }
        for (int s = 0; s < nf; ++s) {
            const float4 Bv = *reinterpret_cast<const float4*>(sB + s * N + 4 * col4);
            const float ws = sw[s];
#pragma unroll
            for (int k = 0; k < R; ++k) {
                const int p = row0 + k * RPP;
                const float u = (p < P) ? ws * sX[s * P + p] : 0.f;
                v[k].x += u * Bv.x; v[k].y += u * Bv.y; v[k].z += u * Bv.z; v[k].w += u * Bv.w;
            }
        }
#pragma unroll
        for (int k = 0; k < R; ++k) {
            const int p = row0 + k * RPP;
            if (p < P) {
                const size_t off = tile + (size_t)p * N + 4 * col4;
                if (!(MODE == kFold && c == 0))
                    *reinterpret_cast<float4*>(a.ckpt + off) = v[k];
                if (LOWP) *reinterpret_cast<uint2*>(a.ckpt_lp + off) = f32x4_to_bf16x4(v[k]);
            }
        }
    } else if (use_lp) {
#pragma unroll
        for (int k = 0; k < R; ++k) v[k] = bf16x4_to_f32x4(vl[k]);
    }

    if constexpr (MODE != kFold) {
        const int q = tid % LPR;
        const int ridx = q / (LPR / R);
        const int p = row0 + ridx * RPP;
        const bool writer = (q % (LPR / R)) == 0 && p < P;
        const IO* zin = reinterpret_cast<const IO*>(a.z);
        const float Dh = a.D[h];
        for (int j = 0; j < T; ++j) {
            const float4 Cv = *reinterpret_cast<const float4*>(sC + j * N + 4 * col4);
            float acc[R];
#pragma unroll
            for (int k = 0; k < R; ++k) acc[k] = dot4(v[k], Cv);
            const float r = row_reduce<R, LPR>(acc, lane);
            if (writer) {
                const int e = nstored + j;
                float y = sdec[j] * r;
                for (int s = st; s <= e; ++s) y += scf[j * nrec + s] * sX[s * P + p];
                y += Dh * sX[e * P + p];
                const size_t o = pos_x(j) + p;
                a.out[o] = silu_gate(y, io::ld(zin, o));
            }
        }

        // ---- 5. append this step's records ----------------------------------------------
        if (MODE == kDecode && !fold) {
            IO* wx = reinterpret_cast<IO*>(a.rec_x) + ((size_t)bh * L + c) * P;
            for (int i = tid; i < P; i += kThreads) wx[i] = xin[(size_t)bh * P + i];
            if (tid == 0) a.rec_dt[(size_t)bh * L + c] = sdt[c];
            if (h % hpg == 0) {
                IO* wb = reinterpret_cast<IO*>(a.rec_B) + ((size_t)(b * G + g) * L + c) * N;
                for (int i = tid; i < N; i += kThreads) wb[i] = Bin[(size_t)(b * G + g) * N + i];
            }
        }
        if (MODE == kSpec) {
            // x and dt records of this head; the group's B records are appended by a
            // separate launch, since other heads may still read the slots being replaced
            for (int i = tid; i < T * P; i += kThreads) {
                const int j = i / P, p2 = i - j * P;
                const int slot = (hd + cm + j) % L;
                reinterpret_cast<IO*>(a.rec_x)[((size_t)bh * L + slot) * P + p2] = xin[pos_x(j) + p2];
            }
            for (int j = tid; j < T; j += kThreads)
                a.rec_dt[(size_t)bh * L + (hd + cm + j) % L] = sdt[cm + j];
        }
    }

    if (tid == 0 && h == 0) {
        if (MODE == kSpec) a.flushed[b] = fold ? 1 : 0;
        else a.cursor_out[b] = (MODE == kFold || fold) ? 0 : c + 1;
    }
}

// Appends the speculative round's B vectors to each group's ring (slots
// (head + committed + j) % L).  Runs after mamba2_replay_kernel<kSpec> on the same
// stream, so every head has finished reading the slots it replaces.
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
        const int hd = a.cursor_in[b], cm = a.committed[b];
        if (hd < 0 || hd >= L || cm < 0 || cm > L) continue;
        const int slot = (hd + cm + j) % L;
        reinterpret_cast<IO*>(a.rec_B)[((size_t)(b * G + g) * L + slot) * N + n] =
            reinterpret_cast<const IO*>(a.B)[i];
    }
}

// ---------------------------------------------------------------------------------------
// Conventional read-update-write step ("Why SSM layers slow down hybrid models": load
// the state, update it, read the output, store it -- every step), with the same tiling
// so that it is a fair baseline.  SNAP: per-position snapshot baseline for speculative
// decoding -- read snapshot slot_in[b], run the n_pos updates, store all n_pos states.
// ---------------------------------------------------------------------------------------
template <int N, int R, typename IO, bool SNAP>
__global__ void __launch_bounds__(kThreads) mamba2_conventional_kernel(Mamba2ConvArgs a) {
    using io = Io<IO>;
    constexpr int LPR = N / 4;
    constexpr int RPP = kThreads / LPR;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int H = a.nheads, P = a.headdim, G = a.ngroups;
    const int hpg = H / G;
    const int bh = xcd_remap(blockIdx.x, gridDim.x);
    const int b = bh / H;
    const int h = bh - b * H;
    const int g = h / hpg;
    const int T = SNAP ? a.n_pos : 1;
    const int row0 = tid / LPR;
    const int col4 = tid - row0 * LPR;
    const size_t PN = (size_t)P * N;

    size_t src;
    if constexpr (SNAP) {
        int sl = a.slot_in[b];
        sl = sl < 0 ? 0 : (sl >= T ? T - 1 : sl);
        src = ((size_t)(b * T + sl) * H + h) * PN;
    } else {
        src = (size_t)bh * PN;
    }
    float4 v[R];
#pragma unroll
    for (int k = 0; k < R; ++k) {
        const int p = row0 + k * RPP;
        v[k] = (p < P) ? *reinterpret_cast<const float4*>(a.state + src + (size_t)p * N + 4 * col4)
                       : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const float Ah = a.A[h], Dh = a.D[h], bias = a.dt_bias[h];
    const IO* xin = reinterpret_cast<const IO*>(a.x);
    const IO* zin = reinterpret_cast<const IO*>(a.z);
    const IO* Bin = reinterpret_cast<const IO*>(a.B);
    const IO* Cin = reinterpret_cast<const IO*>(a.C);
    const IO* dtin = reinterpret_cast<const IO*>(a.dt_raw);
    const int q = tid % LPR;
    const int ridx = q / (LPR / R);
    const int pw = row0 + ridx * RPP;
    const bool writer = (q % (LPR / R)) == 0 && pw < P;

    for (int j = 0; j < T; ++j) {
        const size_t xo = SNAP ? ((size_t)(b * T + j) * H + h) * P : (size_t)bh * P;
        const size_t go = SNAP ? ((size_t)(b * T + j) * G + g) * N : (size_t)(b * G + g) * N;
        const size_t ho = SNAP ? (size_t)(b * T + j) * H + h : (size_t)bh;
        float dt = io::ld(dtin, ho) + bias;
        if (a.dt_softplus) dt = softplus_f32(dt);
        const float dA = expf(dt * Ah);
        const float4 Bv = io::ld4(Bin, go + 4 * col4);
        const float4 Cv = io::ld4(Cin, go + 4 * col4);
        float acc[R];
        const size_t dst = SNAP ? ((size_t)(b * T + j) * H + h) * PN : (size_t)bh * PN;
#pragma unroll
        for (int k = 0; k < R; ++k) {
            const int p = row0 + k * RPP;
            const float xd = (p < P) ? dt * io::ld(xin, xo + p) : 0.f;
            v[k].x = dA * v[k].x + xd * Bv.x;
            v[k].y = dA * v[k].y + xd * Bv.y;
            v[k].z = dA * v[k].z + xd * Bv.z;
            v[k].w = dA * v[k].w + xd * Bv.w;
            if (p < P) *reinterpret_cast<float4*>(a.state + dst + (size_t)p * N + 4 * col4) = v[k];
            acc[k] = dot4(v[k], Cv);
        }
        const float r = row_reduce<R, LPR>(acc, lane);
        if (writer) {
            const float y = r + Dh * io::ld(xin, xo + pw);
            a.out[xo + pw] = silu_gate(y, io::ld(zin, xo + pw));
        }
    }
}

// ---------------------------------------------------------------------------------------
// Dispatch over the compiled (dstate, rows-per-thread) set
// ---------------------------------------------------------------------------------------
static int rows_per_thread(int P, int N) {
    const int rpp = kThreads / (N / 4);
    return P <= rpp ? 1 : P / rpp;
}

bool mamba2_shape_supported(int P, int N) {
    if (!(P == 16 || P == 32 || P == 64 || P == 128)) return false;
    if (!(N == 16 || N == 32 || N == 64 || N == 128 || N == 256)) return false;
    const int R = rows_per_thread(P, N);
    return R <= 16 && R <= N / 4;
}

size_t mamba2_replay_smem_bytes(int P, int N, int L, int n_pos) {
    const int mode = n_pos > 0 ? kSpec : kDecode;
    return sizeof(float) * (size_t)SmemLayout(P, N, L, n_pos > 0 ? n_pos : 1, mode).total;
}

size_t mamba2_max_smem_bytes() { return 64 * 1024; }

template <int N, int R>
static const void* pick_replay(int io, bool lowp, int mode) {
#define RSSM_PICK(IO_T)                                                                   \
    if (mode == kDecode)                                                                  \
        return lowp ? (const void*)&mamba2_replay_kernel<N, R, IO_T, true, kDecode>       \
                    : (const void*)&mamba2_replay_kernel<N, R, IO_T, false, kDecode>;     \
    if (mode == kFold)                                                                    \
        return lowp ? (const void*)&mamba2_replay_kernel<N, R, IO_T, true, kFold>         \
                    : (const void*)&mamba2_replay_kernel<N, R, IO_T, false, kFold>;       \
    return lowp ? (const void*)&mamba2_replay_kernel<N, R, IO_T, true, kSpec>             \
                : (const void*)&mamba2_replay_kernel<N, R, IO_T, false, kSpec>;
    if (io == kIoBF16) { RSSM_PICK(uint16_t) }
    RSSM_PICK(float)
#undef RSSM_PICK
}

template <int N, int R>
static const void* pick_conv(int io, bool snap) {
    if (io == kIoBF16)
        return snap ? (const void*)&mamba2_conventional_kernel<N, R, uint16_t, true>
                    : (const void*)&mamba2_conventional_kernel<N, R, uint16_t, false>;
    return snap ? (const void*)&mamba2_conventional_kernel<N, R, float, true>
                : (const void*)&mamba2_conventional_kernel<N, R, float, false>;
}

#define RSSM_SHAPES(X) \
    X(16, 1) X(16, 2) X(32, 1) X(32, 2) X(32, 4) X(64, 1) X(64, 2) X(64, 4) X(64, 8) \
    X(128, 2) X(128, 4) X(128, 8) X(128, 16) X(256, 4) X(256, 8) X(256, 16)

static const void* find_replay(int P, int N, int io, bool lowp, int mode) {
    const int R = rows_per_thread(P, N);
#define X(NN, RR) \
    if (N == NN && R == RR) return pick_replay<NN, RR>(io, lowp, mode);
    RSSM_SHAPES(X)
#undef X
    return nullptr;
}

static const void* find_conv(int P, int N, int io, bool snap) {
    const int R = rows_per_thread(P, N);
#define X(NN, RR) \
    if (N == NN && R == RR) return pick_conv<NN, RR>(io, snap);
    RSSM_SHAPES(X)
#undef X
    return nullptr;
}

hipError_t launch_mamba2_replay(const Mamba2Args& a, int io, int mode, hipStream_t stream) {
    const void* fn = find_replay(a.headdim, a.dstate, io, a.ckpt_lp != nullptr, mode);
    if (!fn) return hipErrorInvalidValue;
    const int T = mode == kSpec ? a.n_pos : 1;
    const size_t smem = sizeof(float) * (size_t)SmemLayout(a.headdim, a.dstate, a.L, T, mode).total;
    Mamba2Args args = a;
    void* kargs[] = {&args};
    const dim3 grid((unsigned)((size_t)a.batch * a.nheads));
    return hipLaunchKernel(fn, grid, dim3(kThreads), kargs, smem, stream);
}

hipError_t launch_mamba2_spec_append_B(const Mamba2Args& a, int io, hipStream_t stream) {
    const size_t total = (size_t)a.batch * a.n_pos * a.ngroups * a.dstate;
    const unsigned blocks = (unsigned)((total + kThreads - 1) / kThreads < 65536 ? (total + kThreads - 1) / kThreads : 65536);
    Mamba2Args args = a;
    void* kargs[] = {&args};
    const void* fn = io == kIoBF16 ? (const void*)&mamba2_spec_append_B_kernel<uint16_t>
                                   : (const void*)&mamba2_spec_append_B_kernel<float>;
    return hipLaunchKernel(fn, dim3(blocks), dim3(kThreads), kargs, 0, stream);
}

hipError_t launch_mamba2_conventional(const Mamba2ConvArgs& a, int io, bool snap, hipStream_t stream) {
    const void* fn = find_conv(a.headdim, a.dstate, io, snap);
    if (!fn) return hipErrorInvalidValue;
    Mamba2ConvArgs args = a;
    void* kargs[] = {&args};
    const dim3 grid((unsigned)((size_t)a.batch * a.nheads));
    return hipLaunchKernel(fn, grid, dim3(kThreads), kargs, 0, stream);
}

}  // namespace rssm
