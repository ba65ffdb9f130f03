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
// so that S_t q = S_c u + acc.  The chain is sequential in s but only dk long; one
// wave runs it while the other waves' checkpoint loads are in flight.  The flush
// applies the window's updates to the checkpoint row by row (rows are independent)
// and stores it once.
//
// Decomposition: one 256-thread workgroup per (sequence, value head, 64-row tile of
// dv).  dk/4 consecutive lanes cover one row of the tile with 16-byte loads.

#include "device_common.h"
#include "launch.h"

namespace rssm {

constexpr int kGdnThreads = 256;
constexpr int kGdnDecode = 0;
constexpr int kGdnFold = 1;

struct GdnSmem {
    int oK, oV, oAl, oBe, oU, oCoef, total;
    __host__ __device__ GdnSmem(int DK, int DVT, int L) {
        oK = 0;
        oV = oK + L * DK;
        oAl = oV + L * DVT;
        oBe = oAl + L;
        oU = oBe + L;
        oCoef = oU + DK;
        total = oCoef + L;
    }
};

template <int DK>
struct GdnShape {
    static constexpr int LPR = DK / 4;
    static constexpr int RPP = kGdnThreads / LPR;
    static constexpr int R = 64 / RPP;           // rows per thread: tiles of 64 rows
    static constexpr int DVT = RPP * R;
};

template <int DK, typename IO, int MODE>
__global__ void __launch_bounds__(kGdnThreads) gdn_replay_kernel(GdnArgs a) {
    using io = Io<IO>;
    using S = GdnShape<DK>;
    constexpr int LPR = S::LPR, RPP = S::RPP, R = S::R, DVT = S::DVT;
    constexpr int UPL = DK / kWave;  // u elements per lane in the carry-back wave
    extern __shared__ float smem[];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int HV = a.hv, HK = a.hk, dv = a.dv, L = a.L;
    const int ntile = dv / DVT;
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int tile = bid % ntile;
    const int bhv = bid / ntile;
    const int b = bhv / HV;
    const int hv = bhv - b * HV;
    const int hk = hv / (HV / HK);
    const int i0 = tile * DVT;

    const int c = a.cursor_in[b];
    if (c < 0 || c >= L) {
        if (tid == 0) {
            if (a.err_flags) atomicOr(a.err_flags, 1);
            if (hv == 0 && tile == 0) a.cursor_out[b] = c;
        }
        return;
    }
    const int nrec = (MODE == kGdnDecode) ? c + 1 : c;
    const bool fold = (MODE == kGdnFold) || (c + 1 == L);

    const int row0 = tid / LPR;
    const int col4 = tid - row0 * LPR;
    const size_t tbase = ((size_t)bhv * dv + i0) * DK;

    // ---- 1. checkpoint loads ------------------------------------------------------------
    float4 v[R];
    if (!(MODE == kGdnFold && c == 0)) {
#pragma unroll
        for (int k = 0; k < R; ++k)
            v[k] = *reinterpret_cast<const float4*>(a.ckpt + tbase + (size_t)(row0 + k * RPP) * DK + 4 * col4);
    }

    // ---- 2. stage the window ------------------------------------------------------------
    const GdnSmem lay(DK, DVT, L);
    float* sK = smem + lay.oK;      // [nrec][DK]
    float* sV = smem + lay.oV;      // [nrec][DVT]
    float* sAl = smem + lay.oAl;    // [nrec]
    float* sBe = smem + lay.oBe;    // [nrec]
    float* sU = smem + lay.oU;      // [DK]  q, then the carried-back u
    float* sCoef = smem + lay.oCoef;// [nrec] beta_s * kappa_s

    const IO* recK = reinterpret_cast<const IO*>(a.rec_k) + (size_t)(b * HK + hk) * L * DK;
    const IO* recV = reinterpret_cast<const IO*>(a.rec_v) + (size_t)bhv * L * dv;
    const IO* qin = reinterpret_cast<const IO*>(a.q);
    const IO* kin = reinterpret_cast<const IO*>(a.k);
    const IO* vin = reinterpret_cast<const IO*>(a.v);
    const size_t qk_off = (size_t)(b * HK + hk) * DK;

    for (int i = tid; i < nrec * DK; i += kGdnThreads) {
        const int s = i / DK, j = i - s * DK;
        sK[i] = (s < c) ? io::ld(recK, (size_t)s * DK + j) : io::ld(kin, qk_off + j);
    }
    for (int i = tid; i < nrec * DVT; i += kGdnThreads) {
        const int s = i / DVT, ii = i - s * DVT;
        sV[i] = (s < c) ? io::ld(recV, (size_t)s * dv + i0 + ii) : io::ld(vin, (size_t)bhv * dv + i0 + ii);
    }
    for (int s = tid; s < nrec; s += kGdnThreads) {
        sAl[s] = (s < c) ? a.rec_alpha[(size_t)bhv * L + s] : a.alpha[bhv];
        sBe[s] = (s < c) ? a.rec_beta[(size_t)bhv * L + s] : a.beta[bhv];
    }
    if (MODE == kGdnDecode)
        for (int j = tid; j < DK; j += kGdnThreads) sU[j] = io::ld(qin, qk_off + j);
    __syncthreads();

    if (MODE == kGdnFold && c == 0) {
        if (tid == 0 && hv == 0 && tile == 0) a.cursor_out[b] = 0;
        return;
    }

    const int q = tid % LPR;
    const int ridx = q / (LPR / R);
    const int iw = row0 + ridx * RPP;                 // row (within the tile) this lane writes
    const bool writer = (q % (LPR / R)) == 0;
    const float scale = a.scale;

    if (!fold) {
        // ---- 3. carry q back through the window (wave 0) --------------------------------
        if (tid < kWave) {
            float u[UPL];
#pragma unroll
            for (int m = 0; m < UPL; ++m) u[m] = sU[lane + m * kWave];
            for (int s = nrec - 1; s >= 0; --s) {
                float kap = 0.f;
#pragma unroll
                for (int m = 0; m < UPL; ++m) kap += sK[s * DK + lane + m * kWave] * u[m];
                kap = group_allreduce<kWave>(kap);
                const float bk = sBe[s] * kap;
                if (lane == 0) sCoef[s] = bk;
                const float al = sAl[s];
#pragma unroll
                for (int m = 0; m < UPL; ++m) u[m] = al * (u[m] - bk * sK[s * DK + lane + m * kWave]);
            }
#pragma unroll
            for (int m = 0; m < UPL; ++m) sU[lane + m * kWave] = u[m];
        }
        __syncthreads();

        // ---- 4. o = scale (S_c u + sum_s beta_s kappa_s v_s) ----------------------------
        const float4 Uv = *reinterpret_cast<const float4*>(sU + 4 * col4);
        float acc[R];
#pragma unroll
        for (int k = 0; k < R; ++k) acc[k] = dot4(v[k], Uv);
        const float r = row_reduce<R, LPR>(acc, lane);
        if (writer) {
            float o = r;
            for (int s = 0; s < nrec; ++s) o += sCoef[s] * sV[s * DVT + iw];
            a.out[(size_t)bhv * dv + i0 + iw] = scale * o;
        }

        // ---- 5. append the step's record ------------------------------------------------
        IO* wv = reinterpret_cast<IO*>(a.rec_v) + ((size_t)bhv * L + c) * dv + i0;
        for (int ii = tid; ii < DVT; ii += kGdnThreads) wv[ii] = vin[(size_t)bhv * dv + i0 + ii];
        if (tile == 0 && tid == 0) {
            a.rec_alpha[(size_t)bhv * L + c] = a.alpha[bhv];
            a.rec_beta[(size_t)bhv * L + c] = a.beta[bhv];
        }
        if (tile == 0 && hv % (HV / HK) == 0) {
            IO* wk = reinterpret_cast<IO*>(a.rec_k) + ((size_t)(b * HK + hk) * L + c) * DK;
            for (int j = tid; j < DK; j += kGdnThreads) wk[j] = kin[qk_off + j];
        }
    } else {
        // ---- 3'. flush: apply the window's updates row by row, oldest first -------------
        for (int s = 0; s < nrec; ++s) {
            const float4 Kv = *reinterpret_cast<const float4*>(sK + s * DK + 4 * col4);
            const float al = sAl[s], be = sBe[s];
            float d[R];
#pragma unroll
            for (int k = 0; k < R; ++k) d[k] = dot4(v[k], Kv);
            row_allreduce<R, LPR>(d, lane);
#pragma unroll
            for (int k = 0; k < R; ++k) {
                const float bd = be * d[k];
                const float bv = be * sV[s * DVT + row0 + k * RPP];
                v[k].x = al * (v[k].x - bd * Kv.x) + bv * Kv.x;
                v[k].y = al * (v[k].y - bd * Kv.y) + bv * Kv.y;
                v[k].z = al * (v[k].z - bd * Kv.z) + bv * Kv.z;
                v[k].w = al * (v[k].w - bd * Kv.w) + bv * Kv.w;
            }
        }
#pragma unroll
        for (int k = 0; k < R; ++k)
            *reinterpret_cast<float4*>(a.ckpt + tbase + (size_t)(row0 + k * RPP) * DK + 4 * col4) = v[k];
        if (MODE == kGdnDecode) {
            const float4 Qv = *reinterpret_cast<const float4*>(sU + 4 * col4);
            float acc[R];
#pragma unroll
            for (int k = 0; k < R; ++k) acc[k] = dot4(v[k], Qv);
            const float r = row_reduce<R, LPR>(acc, lane);
            if (writer) a.out[(size_t)bhv * dv + i0 + iw] = scale * r;
        }
    }

    if (tid == 0 && hv == 0 && tile == 0) a.cursor_out[b] = fold ? 0 : c + 1;
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
    const float kq = group_allreduce<LPR>(dot4(Kv, Qv));

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

size_t gdn_smem_bytes(int dk, int dv, int L) {
    (void)dv;
    return sizeof(float) * (size_t)GdnSmem(dk, 64, L).total;
}

hipError_t launch_gdn_replay(const GdnArgs& a, int io, int mode, hipStream_t stream) {
    const void* fn = nullptr;
#define RSSM_GDN(DK)                                                                              \
    if (a.dk == DK) {                                                                             \
        if (io == kIoBF16)                                                                        \
            fn = mode == kGdnFold ? (const void*)&gdn_replay_kernel<DK, uint16_t, kGdnFold>       \
                                  : (const void*)&gdn_replay_kernel<DK, uint16_t, kGdnDecode>;    \
        else                                                                                      \
            fn = mode == kGdnFold ? (const void*)&gdn_replay_kernel<DK, float, kGdnFold>          \
                                  : (const void*)&gdn_replay_kernel<DK, float, kGdnDecode>;       \
    }
    RSSM_GDN(64)
    RSSM_GDN(128)
#undef RSSM_GDN
    if (!fn) return hipErrorInvalidValue;
    GdnArgs args = a;
    void* kargs[] = {&args};
    const dim3 grid((unsigned)((size_t)a.batch * a.hv * (a.dv / 64)));
    return hipLaunchKernel(fn, grid, dim3(kGdnThreads), kargs, gdn_smem_bytes(a.dk, a.dv, a.L), stream);
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
