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
// so that S_t q = S_c u + acc.  The chain is sequential in s but only dk long; each
// value head's chain runs on its own wave while the first checkpoint tile is in
// flight.  The flush applies the window's updates to the checkpoint row by row (rows
// are independent) and stores it once.
//
// Decomposition: the replay kernel runs one 256-thread workgroup per (sequence, q/k
// head) and streams the [64, dk] tiles of that head's value heads (k records and q
// are shared by them); the conventional kernel runs one workgroup per (sequence, value
// head, 64-row tile).  dk/4 consecutive lanes cover one row of a tile with 16-byte
// loads.

#include "device_common.h"
#include "launch.h"

namespace rssm {

constexpr int kGdnThreads = 256;
constexpr int kGdnDecode = 0;
constexpr int kGdnFold = 1;
constexpr int kGdnMaxVHeads = 4;   // value heads per workgroup (one carry-back wave each)

template <int DK>
struct GdnShape {
    static constexpr int LPR = DK / 4;                 // lanes per state row
    static constexpr int RPP = kGdnThreads / LPR;      // rows per pass
    static constexpr int R = 64 / RPP;                 // rows per thread: tiles of 64 rows
    static constexpr int DVT = RPP * R;
};

// LDS layout (4-byte words) of the replay kernel.
struct GdnSmem {
    int oK, oV, oAl, oBe, oQ, oU, oCoef, oAcc, total;
    __host__ __device__ GdnSmem(int DK, int DV, int L, int NV, int io_bytes) {
        oK = 0;                                    // [L][DK]      k rows of the window
        oV = oK + L * DK;                          // [NV][L][DV]  v rows (io dtype)
        oAl = oV + (NV * L * DV * io_bytes + 3) / 4;   // [NV][L]
        oBe = oAl + NV * L;                        // [NV][L]
        oQ = oBe + NV * L;                         // [DK]
        oU = oQ + DK;                              // [NV][DK]     carried-back q
        oCoef = oU + NV * DK;                      // [NV][L]      beta_s kappa_s
        oAcc = oCoef + NV * L;                     // [NV][DV]     sum_s beta_s kappa_s v_s
        total = oAcc + NV * DV;
    }
};

// One workgroup per (sequence, q/k head, chunk of its value heads).  The k records and
// q are shared by the value heads of one q/k head and staged once; each value head's
// carry-back chain runs on its own wave; the workgroup then streams the value heads'
// [64, dk] checkpoint tiles, loading the next tile while it reduces the current one.
template <int DK, int DV, typename IO, int MODE>
__global__ void __launch_bounds__(kGdnThreads) gdn_replay_kernel(GdnArgs a) {
    using io = Io<IO>;
    using Raw4 = typename io::Raw4;
    using S = GdnShape<DK>;
    constexpr int LPR = S::LPR, RPP = S::RPP, R = S::R, DVT = S::DVT;
    constexpr int NTILE = DV / DVT;
    constexpr int UPL = DK / kWave;  // u elements per lane in a carry-back wave
    constexpr int DK4 = DK / 4, DV4 = DV / 4;
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
    const int b = bk / HK;
    const int hk = bk - b * HK;
    const int hv0 = hk * rv + chunk * a.vheads_per_chunk;
    const int nv = min(a.vheads_per_chunk, rv - chunk * a.vheads_per_chunk);
    const bool lead = (hk == 0 && chunk == 0);

    const int c = a.cursor_in[b];
    if (c < 0 || c >= L) {
        if (tid == 0) {
            if (a.err_flags) atomicOr(a.err_flags, 1);
            if (lead) a.cursor_out[b] = c;
        }
        return;
    }
    const int nrec = (MODE == kGdnDecode) ? c + 1 : c;
    const bool fold = (MODE == kGdnFold) || (c + 1 == L);
    const bool idle = (MODE == kGdnFold) && c == 0;
    const size_t bHV = (size_t)b * HV;

    const GdnSmem lay(DK, DV, L, a.vheads_per_chunk, (int)sizeof(IO));
    float* sK = smem + lay.oK;
    IO* sV = reinterpret_cast<IO*>(smem + lay.oV);
    float* sAl = smem + lay.oAl;
    float* sBe = smem + lay.oBe;
    float* sQ = smem + lay.oQ;
    float* sU = smem + lay.oU;
    float* sCoef = smem + lay.oCoef;
    float* sAcc = smem + lay.oAcc;

    const int row0 = tid / LPR;
    const int col4 = tid % LPR;
    auto tile_base = [&](int u) -> size_t {   // unit u = (value head u / NTILE, tile u % NTILE)
        const int vl = u / NTILE, tl = u % NTILE;
        return ((bHV + hv0 + vl) * DV + tl * DVT + row0) * (size_t)DK + 4 * col4;
    };
    auto issue_tile = [&](int u, float4 (&v)[R]) {
        const size_t t = tile_base(u);
#pragma unroll
        for (int k = 0; k < R; ++k) v[k] = ld_stream(a.ckpt + t + (size_t)k * RPP * DK);
    };
    const int nunit = nv * NTILE;
    float4 va[R], vb[R];
    if (!idle) issue_tile(0, va);

    // ---- stage the window -------------------------------------------------------------
    const IO* recK = reinterpret_cast<const IO*>(a.rec_k) + ((size_t)b * HK + hk) * L * DK;
    const IO* kin = reinterpret_cast<const IO*>(a.k) + ((size_t)b * HK + hk) * DK;
    const IO* qin = reinterpret_cast<const IO*>(a.q) + ((size_t)b * HK + hk) * DK;
    const IO* vin = reinterpret_cast<const IO*>(a.v);
    const IO* recV = reinterpret_cast<const IO*>(a.rec_v);
    for (int task = tid; task < nrec * DK4; task += kGdnThreads) {
        const int s = task / DK4, j4 = task % DK4;
        const Raw4 r = (s < c) ? io::ldraw4(recK, (size_t)s * DK + 4 * j4) : io::ldraw4(kin, 4 * j4);
        *reinterpret_cast<float4*>(sK + s * DK + 4 * j4) = io::cvt4(r);
    }
    for (int task = tid; task < nv * nrec * DV4; task += kGdnThreads) {
        const int i4 = task % DV4;
        const int vs = task / DV4;
        const int vl = vs / nrec, s = vs - vl * nrec;
        const size_t hv = bHV + hv0 + vl;
        const Raw4 r = (s < c) ? io::ldraw4(recV, (hv * L + s) * DV + 4 * i4) : io::ldraw4(vin, hv * DV + 4 * i4);
        *reinterpret_cast<Raw4*>(sV + (vl * L + s) * DV + 4 * i4) = r;
    }
    for (int task = tid; task < nv * nrec; task += kGdnThreads) {
        const int vl = task / nrec, s = task - vl * nrec;
        const size_t hv = bHV + hv0 + vl;
        sAl[vl * L + s] = (s < c) ? a.rec_alpha[hv * L + s] : a.alpha[hv];
        sBe[vl * L + s] = (s < c) ? a.rec_beta[hv * L + s] : a.beta[hv];
    }
    if (MODE == kGdnDecode)
        for (int j4 = tid; j4 < DK4; j4 += kGdnThreads)
            *reinterpret_cast<float4*>(sQ + 4 * j4) = io::cvt4(io::ldraw4(qin, 4 * j4));
    __syncthreads();

    const int q = tid % LPR;
    const int ridx = q / (LPR / R);
    const int iw = row0 + ridx * RPP;               // row (within a tile) this lane writes
    const bool writer = (q % (LPR / R)) == 0;
    const float scale = a.scale;

    auto rotate = [&]() {
#pragma unroll
        for (int k = 0; k < R; ++k) va[k] = vb[k];
    };

    if (!fold) {
        // ---- carry q back through each value head's window (one wave per value head) --
        if (wave < nv) {
            float u[UPL];
#pragma unroll
            for (int m = 0; m < UPL; ++m) u[m] = sQ[lane + m * kWave];
            const float* al = sAl + wave * L;
            const float* be = sBe + wave * L;
            for (int s = nrec - 1; s >= 0; --s) {
                float kap = 0.f;
#pragma unroll
                for (int m = 0; m < UPL; ++m) kap += sK[s * DK + lane + m * kWave] * u[m];
                kap = group_allreduce<kWave>(kap, lane);
                const float bk = be[s] * kap;
                if (lane == 0) sCoef[wave * L + s] = bk;
                const float as = al[s];
#pragma unroll
                for (int m = 0; m < UPL; ++m) u[m] = as * (u[m] - bk * sK[s * DK + lane + m * kWave]);
            }
#pragma unroll
            for (int m = 0; m < UPL; ++m) sU[wave * DK + lane + m * kWave] = u[m];
        }
        __syncthreads();
        // ---- record terms sum_s beta_s kappa_s v_s[i] of every value head --------------
        for (int task = tid; task < nv * DV; task += kGdnThreads) {
            const int vl = task / DV, i = task % DV;
            float acc = 0.f;
            for (int s = 0; s < nrec; ++s) acc += sCoef[vl * L + s] * io::ld(sV, (vl * L + s) * DV + i);
            sAcc[vl * DV + i] = acc;
        }
        __syncthreads();

        auto body = [&](int u) {
            const int vl = u / NTILE, tl = u % NTILE;
            const float4 Uv = *reinterpret_cast<const float4*>(sU + vl * DK + 4 * col4);
            float acc[R];
#pragma unroll
            for (int k = 0; k < R; ++k) acc[k] = dot4(va[k], Uv);
            const float r = row_reduce<R, LPR>(acc, lane);
            if (writer) {
                const int i = tl * DVT + iw;
                a.out[(bHV + hv0 + vl) * DV + i] = scale * (r + sAcc[vl * DV + i]);
            }
        };
        for (int u = 0; u + 1 < nunit; ++u) {
            issue_tile(u + 1, vb);
            body(u);
            rotate();
        }
        body(nunit - 1);

        // ---- append the step's record -----------------------------------------------
        for (int task = tid; task < nv * DV4; task += kGdnThreads) {
            const int vl = task / DV4, i4 = task % DV4;
            const size_t hv = bHV + hv0 + vl;
            io::straw4(reinterpret_cast<IO*>(a.rec_v), (hv * L + c) * DV + 4 * i4, io::ldraw4(vin, hv * DV + 4 * i4));
        }
        for (int vl = tid; vl < nv; vl += kGdnThreads) {
            const size_t hv = bHV + hv0 + vl;
            a.rec_alpha[hv * L + c] = a.alpha[hv];
            a.rec_beta[hv * L + c] = a.beta[hv];
        }
        if (chunk == 0) {
            for (int j4 = tid; j4 < DK4; j4 += kGdnThreads)
                io::straw4(reinterpret_cast<IO*>(a.rec_k), (((size_t)b * HK + hk) * L + c) * DK + 4 * j4,
                           io::ldraw4(kin, 4 * j4));
        }
    } else if (!idle) {
        // ---- flush: apply the window's updates row by row, oldest first ------------------
        auto body = [&](int u) {
            const int vl = u / NTILE, tl = u % NTILE;
            const float* al = sAl + vl * L;
            const float* be = sBe + vl * L;
            for (int s = 0; s < nrec; ++s) {
                const float4 Kv = *reinterpret_cast<const float4*>(sK + s * DK + 4 * col4);
                float d[R];
#pragma unroll
                for (int k = 0; k < R; ++k) d[k] = dot4(va[k], Kv);
                row_allreduce<R, LPR>(d, lane);
                const float as = al[s], bs = be[s];
#pragma unroll
                for (int k = 0; k < R; ++k) {
                    const float bd = bs * d[k];
                    const float bv = bs * io::ld(sV, (vl * L + s) * DV + tl * DVT + row0 + k * RPP);
                    va[k].x = as * (va[k].x - bd * Kv.x) + bv * Kv.x;
                    va[k].y = as * (va[k].y - bd * Kv.y) + bv * Kv.y;
                    va[k].z = as * (va[k].z - bd * Kv.z) + bv * Kv.z;
                    va[k].w = as * (va[k].w - bd * Kv.w) + bv * Kv.w;
                }
            }
            const size_t t = tile_base(u);
#pragma unroll
            for (int k = 0; k < R; ++k) st_stream(a.ckpt + t + (size_t)k * RPP * DK, va[k]);
            if (MODE == kGdnDecode) {
                const float4 Qv = *reinterpret_cast<const float4*>(sQ + 4 * col4);
                float acc[R];
#pragma unroll
                for (int k = 0; k < R; ++k) acc[k] = dot4(va[k], Qv);
                const float r = row_reduce<R, LPR>(acc, lane);
                if (writer) a.out[(bHV + hv0 + vl) * DV + tl * DVT + iw] = scale * r;
            }
        };
        for (int u = 0; u + 1 < nunit; ++u) {
            issue_tile(u + 1, vb);
            body(u);
            rotate();
        }
        body(nunit - 1);
    }

    if (tid == 0 && lead) a.cursor_out[b] = fold ? 0 : c + 1;
}

// Conventional step: S <- alpha (S - beta (S k) k^T) + beta v k^T, o = scale S q, with
// one read and one write of the state.  Uses S_new q = alpha (S q - beta (S k)(k.q)) +
// beta v (k.q), so both row dots come from the state as loaded.
template <int DK, typename IO>
__global__ void __launch_bounds__(kGdnThreads) gdn_conventional_kernel(GdnArgs a) {
    using io = Io<IO>;
    using S = GdnShape<DK>;
    constexpr int LPR = S::LPR, RPP = S::RPP, R = S::R, DVT = S::DVT;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int HV = a.hv, HK = a.hk, dv = a.dv;
    const int ntile = dv / DVT;
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int tile = bid % ntile;
    const int bhv = bid / ntile;
    const int b = bhv / HV;
    const int hv = bhv - b * HV;
    const int hk = hv / (HV / HK);
    const int i0 = tile * DVT;
    const int row0 = tid / LPR;
    const int col4 = tid - row0 * LPR;
    const size_t tbase = ((size_t)bhv * dv + i0) * DK;

    float4 v[R];
#pragma unroll
    for (int k = 0; k < R; ++k)
        v[k] = *reinterpret_cast<const float4*>(a.ckpt + tbase + (size_t)(row0 + k * RPP) * DK + 4 * col4);
    const size_t qk_off = (size_t)(b * HK + hk) * DK;
    const float4 Kv = io::ld4(reinterpret_cast<const IO*>(a.k), qk_off + 4 * col4);
    const float4 Qv = io::ld4(reinterpret_cast<const IO*>(a.q), qk_off + 4 * col4);
    const IO* vin = reinterpret_cast<const IO*>(a.v);
    const float al = a.alpha[bhv], be = a.beta[bhv];
    const float kq = group_allreduce<LPR>(dot4(Kv, Qv), lane);

    float d[R], e[R];
#pragma unroll
    for (int k = 0; k < R; ++k) {
        d[k] = dot4(v[k], Kv);
        e[k] = dot4(v[k], Qv);
    }
    row_allreduce<R, LPR>(d, lane);
#pragma unroll
    for (int k = 0; k < R; ++k) {
        const float bd = be * d[k];
        const float bv = be * io::ld(vin, (size_t)bhv * dv + i0 + row0 + k * RPP);
        v[k].x = al * (v[k].x - bd * Kv.x) + bv * Kv.x;
        v[k].y = al * (v[k].y - bd * Kv.y) + bv * Kv.y;
        v[k].z = al * (v[k].z - bd * Kv.z) + bv * Kv.z;
        v[k].w = al * (v[k].w - bd * Kv.w) + bv * Kv.w;
        *reinterpret_cast<float4*>(a.ckpt + tbase + (size_t)(row0 + k * RPP) * DK + 4 * col4) = v[k];
    }
    const int q = tid % LPR;
    const int ridx = q / (LPR / R);
    const int iw = row0 + ridx * RPP;
    float dsel = d[0];
#pragma unroll
    for (int k = 1; k < R; ++k) dsel = (k == ridx) ? d[k] : dsel;
    const float r = row_reduce<R, LPR>(e, lane);
    if ((q % (LPR / R)) == 0) {
        const float vi = io::ld(vin, (size_t)bhv * dv + i0 + iw);
        a.out[(size_t)bhv * dv + i0 + iw] = a.scale * (al * (r - be * dsel * kq) + be * vi * kq);
    }
}

bool gdn_shape_supported(int dk, int dv) {
    return (dk == 64 || dk == 128) && (dv == 64 || dv == 128);
}

static void gdn_chunking(int rv, int* nchunk, int* per) {
    *per = rv < kGdnMaxVHeads ? rv : kGdnMaxVHeads;
    *nchunk = (rv + *per - 1) / *per;
}

size_t gdn_smem_bytes(int dk, int dv, int L, int rv, int io_bytes) {
    int nchunk, per;
    gdn_chunking(rv, &nchunk, &per);
    return sizeof(float) * (size_t)GdnSmem(dk, dv, L, per, io_bytes).total;
}

template <int DK, int DV>
static const void* gdn_pick(int io, int mode) {
    if (io == kIoBF16)
        return mode == kGdnFold ? (const void*)&gdn_replay_kernel<DK, DV, uint16_t, kGdnFold>
                                : (const void*)&gdn_replay_kernel<DK, DV, uint16_t, kGdnDecode>;
    return mode == kGdnFold ? (const void*)&gdn_replay_kernel<DK, DV, float, kGdnFold>
                            : (const void*)&gdn_replay_kernel<DK, DV, float, kGdnDecode>;
}

hipError_t launch_gdn_replay(const GdnArgs& a, int io, int mode, hipStream_t stream) {
    const void* fn = nullptr;
    if (a.dk == 64 && a.dv == 64) fn = gdn_pick<64, 64>(io, mode);
    if (a.dk == 64 && a.dv == 128) fn = gdn_pick<64, 128>(io, mode);
    if (a.dk == 128 && a.dv == 64) fn = gdn_pick<128, 64>(io, mode);
    if (a.dk == 128 && a.dv == 128) fn = gdn_pick<128, 128>(io, mode);
    if (!fn) return hipErrorInvalidValue;
    GdnArgs args = a;
    gdn_chunking(a.hv / a.hk, &args.nchunk, &args.vheads_per_chunk);
    const size_t smem = gdn_smem_bytes(a.dk, a.dv, a.L, a.hv / a.hk, io == kIoBF16 ? 2 : 4);
    void* kargs[] = {&args};
    const dim3 grid((unsigned)((size_t)a.batch * a.hk * args.nchunk));
    return hipLaunchKernel(fn, grid, dim3(kGdnThreads), kargs, smem, stream);
}

hipError_t launch_gdn_conventional(const GdnArgs& a, int io, hipStream_t stream) {
    const void* fn = nullptr;
    if (a.dk == 64)
        fn = io == kIoBF16 ? (const void*)&gdn_conventional_kernel<64, uint16_t>
                           : (const void*)&gdn_conventional_kernel<64, float>;
    else if (a.dk == 128)
        fn = io == kIoBF16 ? (const void*)&gdn_conventional_kernel<128, uint16_t>
                           : (const void*)&gdn_conventional_kernel<128, float>;
    if (!fn) return hipErrorInvalidValue;
    GdnArgs args = a;
    void* kargs[] = {&args};
    const dim3 grid((unsigned)((size_t)a.batch * a.hv * (a.dv / 64)));
    return hipLaunchKernel(fn, grid, dim3(kGdnThreads), kargs, 0, stream);
}

}  // namespace rssm
