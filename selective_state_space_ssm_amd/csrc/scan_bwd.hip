// scan_bwd.hip -- backward of the selective scan for gfx950.
//
// The pages state that the selection maps receive gradients (TensorViz
// explorer, "Verified by the local recipe") but give no backward pass; this
// is the reverse-mode adjoint of the forward recurrence.  With
// g_t = dLoss/dh_t and dyv the gradient of the pre-gate output:
//   g_t     = C_t * dyv_t + a_{t+1} * g_{t+1}        (g after the last token = dhT)
//   dC_t   += h_t * dyv_t,   da_t = g_t * h_{t-1}
//   dt*B:   ddt += da*a*A + g*B*u,  du += g*dt*B,  dB += g*dt*u,  dA += da*a*dt
//   ZOH:    c = expm1(dt*A)/A;  ddt += da*a*A + g*a*B*u,  du += g*c*B,  dB += g*c*u,
//           dA += da*a*dt + g*B*u*(dt*a*A - expm1(dt*A))/A^2
//   gate:   dyv = dy*z*s,  dz = dy*yv*s*(1 + z*(1-s)),  s = sigmoid(z)
//   dA_log = A * dA,  d_dt_raw = ddt * sigmoid(dt_raw + dt_bias)
//
// Structure.
//  1. States at every T-token boundary come from the forward's two-level
//     machinery (local chunk scans + carry walk), fully parallel over time.
//  2. scan_bwd_kernel: one 256-thread block per (batch, 64 channels) walks
//     the tiles from last to first.  For each tile it re-runs the forward for
//     T tokens from the boundary state, keeping h and the decays in
//     registers, then sweeps the tile backwards.  Four lanes own a channel
//     exactly as in the forward; per-channel sums over the lane quad use DPP.
//     dB and dC are sums over channels: each 16-lane row first adds its four
//     channels with DPP row shifts, then the block's 16 row partials go to
//     fixed LDS slots and are added in a fixed order, so the result is
//     deterministic; one partial per block lands in the workspace.
//  3. Two small kernels add the per-block partials (dB, dC) and the
//     per-batch partials (dA_log, dDskip, d_dt_bias).
#include <algorithm>

#include "launch.hpp"
#include "ssm_device.hpp"

namespace ssm {
namespace {

constexpr int kLPC = 4;
constexpr int kCPB = 64;        // channels per block (4 wavefronts)
constexpr int kSlots = 16;      // 16-lane rows per block
enum { DISC_DB = 0, DISC_ZOH = 1 };

template <int SPL>
constexpr int tile_for() { return SPL <= 4 ? 16 : (SPL == 8 ? 8 : 4); }

struct BwdParams {
    const void *u, *dt;
    const float *dt_bias, *A_log;
    const void *Bm, *Cm;
    const float *Dskip;
    const void *z;
    const void *dy;
    const float *dhT;
    const float *ckpt;       // [B, K, D, N] states at tile starts
    void *du, *ddt, *dz;
    float *dh0;
    float *pB, *pC;          // [G, B, L, N] per-block channel partials
    float *pA;               // [B, D, N]   dLoss/dA summed over time
    float *pD, *pT;          // [B, D]      dDskip, d_dt_bias summed over time
    int64_t B, L, D, N;
    int K;                   // tiles along time
    int G;                   // channel blocks
};

template <typename IOT, int SPL, int DISC>
__global__ __launch_bounds__(256) void scan_bwd_kernel(BwdParams p) {
    constexpr int T = tile_for<SPL>();
    constexpr int NP = kLPC * SPL;
    __shared__ float redB[kSlots][T][NP];
    __shared__ float redC[kSlots][T][NP];

    const IOT *U = static_cast<const IOT *>(p.u);
    const IOT *DT = static_cast<const IOT *>(p.dt);
    const IOT *Bp = static_cast<const IOT *>(p.Bm);
    const IOT *Cp = static_cast<const IOT *>(p.Cm);
    const IOT *Z = static_cast<const IOT *>(p.z);
    const IOT *DY = static_cast<const IOT *>(p.dy);
    IOT *DU = static_cast<IOT *>(p.du);
    IOT *DDT = static_cast<IOT *>(p.ddt);
    IOT *DZ = static_cast<IOT *>(p.dz);

    const int tid = threadIdx.x;
    const int wv = tid >> 6, lane = tid & 63;
    const int ch = lane / kLPC, q = lane % kLPC;
    const int row = lane >> 4;
    const int64_t gblk = blockIdx.x % p.G;
    const int64_t b = blockIdx.x / p.G;
    const int64_t d = gblk * kCPB + wv * 16 + ch;
    const bool dvalid = d < p.D;
    const int64_t dc = dvalid ? d : (p.D - 1);
    const int64_t N = p.N, D = p.D, L = p.L;
    const int n0 = q * SPL;
    const int nvalid = max(0, min(SPL, (int)(N - n0)));
    const bool vecN = (N % 4) == 0;
    const bool gate = Z != nullptr;
    const float vmask = dvalid ? 1.0f : 0.0f;

    float A2[SPL], An[SPL], Ainv[SPL];
#pragma unroll
    for (int j = 0; j < SPL; ++j) {
        const bool v = j < nvalid;
        const float A = neg_exp_f(v ? p.A_log[dc * N + n0 + j] : 0.0f);
        A2[j] = v ? A * kLog2e : 0.0f;
        An[j] = A;
        Ainv[j] = 1.0f / A;
    }
    const float dtb = p.dt_bias ? p.dt_bias[dc] : 0.0f;
    const float Dd = p.Dskip ? p.Dskip[dc] : 0.0f;

    float gad[SPL], dAt[SPL];
#pragma unroll
    for (int j = 0; j < SPL; ++j) { gad[j] = 0.0f; dAt[j] = 0.0f; }
    if (p.dhT != nullptr && dvalid && nvalid > 0)
        load_k_guard<SPL>(p.dhT + (b * D + d) * N + n0, gad, nvalid, vecN);
    float dDt = 0.0f, dTt = 0.0f;

    for (int c = p.K - 1; c >= 0; --c) {
        const int64_t t0 = (int64_t)c * T;
        const int len = (int)min((int64_t)T, L - t0);
        float hs[T + 1][SPL], as[T][SPL], yv[T];
        load_k_guard<SPL>(p.ckpt + ((b * p.K + c) * D + dc) * N + n0, hs[0], nvalid, vecN);

        // forward re-run of the tile
#pragma unroll
        for (int i = 0; i < T; ++i) {
            if (i < len) {
                const int64_t t = t0 + i;
                const int64_t e = (b * L + t) * D + dc;
                const float uu = to_f32(U[e]);
                const float dl = softplus_f(to_f32(DT[e]) + dtb);
                const float du = dl * uu;
                float Bq[SPL], Cq[SPL];
                load_k_guard<SPL>(Bp + (b * L + t) * N + n0, Bq, nvalid, vecN);
                if (gate) load_k_guard<SPL>(Cp + (b * L + t) * N + n0, Cq, nvalid, vecN);
                float yacc = 0.0f;
#pragma unroll
                for (int j = 0; j < SPL; ++j) {
                    const float a = hw_exp2(dl * A2[j]);
                    float w;
                    if constexpr (DISC == DISC_DB)
                        w = du * Bq[j];
                    else
                        w = expm1f(dl * An[j]) * Ainv[j] * Bq[j] * uu;
                    hs[i + 1][j] = fmaf(a, hs[i][j], w);
                    as[i][j] = a;
                    if (gate) yacc = fmaf(Cq[j], hs[i + 1][j], yacc);
                }
                if (gate) yv[i] = fmaf(Dd, uu, group_sum<kLPC>(yacc));
            }
        }

        float dAc[SPL];
#pragma unroll
        for (int j = 0; j < SPL; ++j) dAc[j] = 0.0f;
        float dDc = 0.0f, dTc = 0.0f;

        // reverse sweep of the tile
#pragma unroll
        for (int i = T - 1; i >= 0; --i) {
            if (i < len) {
                const int64_t t = t0 + i;
                const int64_t e = (b * L + t) * D + dc;
                const float uu = to_f32(U[e]);
                const float r = to_f32(DT[e]) + dtb;
                const float dl = softplus_f(r);
                const float sg = sigmoid_f(r);
                const float dyr = to_f32(DY[e]) * vmask;
                float dyv, dzv = 0.0f;
                if (gate) {
                    const float zz = to_f32(Z[e]);
                    const float s = sigmoid_f(zz);
                    dyv = dyr * zz * s;
                    dzv = dyr * yv[i] * s * (1.0f + zz * (1.0f - s));
                } else {
                    dyv = dyr;
                }
                dDc = fmaf(dyv, uu, dDc);
                float Bq[SPL], Cq[SPL];
                load_k_guard<SPL>(Bp + (b * L + t) * N + n0, Bq, nvalid, vecN);
                load_k_guard<SPL>(Cp + (b * L + t) * N + n0, Cq, nvalid, vecN);
                const float du = dl * uu;
                float ddt_p = 0.0f, du_p = 0.0f;
                float bpart[SPL], cpart[SPL];
#pragma unroll
                for (int j = 0; j < SPL; ++j) {
                    const float gj = fmaf(Cq[j], dyv, gad[j]);
                    cpart[j] = hs[i + 1][j] * dyv;
                    const float a = as[i][j];
                    const float daa = gj * hs[i][j] * a;
                    if constexpr (DISC == DISC_DB) {
                        const float gB = gj * Bq[j];
                        ddt_p = fmaf(daa, An[j], ddt_p);
                        ddt_p = fmaf(gB, uu, ddt_p);
                        du_p += gB;
                        bpart[j] = gj * du;
                        dAc[j] = fmaf(daa, dl, dAc[j]);
                    } else {
                        const float em1 = expm1f(dl * An[j]);
                        const float cz = em1 * Ainv[j];
                        const float gBu = gj * Bq[j] * uu;
                        ddt_p = fmaf(daa, An[j], ddt_p);
                        ddt_p = fmaf(gBu, a, ddt_p);
                        du_p = fmaf(gj * cz, Bq[j], du_p);
                        bpart[j] = gj * cz * uu;
                        dAc[j] = fmaf(daa, dl, dAc[j]);
                        dAc[j] = fmaf(gBu * (dl * a * An[j] - em1), Ainv[j] * Ainv[j], dAc[j]);
                    }
                    gad[j] = a * gj;
                }
                const float ddt = group_sum<kLPC>(ddt_p);
                const float dup = group_sum<kLPC>(du_p);
                float duv;
                if constexpr (DISC == DISC_DB)
                    duv = fmaf(dl, dup, Dd * dyv);
                else
                    duv = fmaf(Dd, dyv, dup);
                const float ddr = ddt * sg;
                dTc += ddr;
                if (q == 0 && dvalid) {
                    const int64_t eo = (b * L + t) * D + d;
                    if (DU) store_io(DU + eo, duv);
                    if (DDT) store_io(DDT + eo, ddr);
                    if (DZ && gate) store_io(DZ + eo, dzv);
                }
                // channel sums for dB, dC: four channels of each 16-lane row
#pragma unroll
                for (int j = 0; j < SPL; ++j) {
                    bpart[j] = row_stride4_sum(bpart[j]);
                    cpart[j] = row_stride4_sum(cpart[j]);
                }
                if ((lane & 15) >= 12) {
                    const int slot = wv * 4 + row;
#pragma unroll
                    for (int j = 0; j < SPL; ++j) {
                        redB[slot][i][n0 + j] = bpart[j];
                        redC[slot][i][n0 + j] = cpart[j];
                    }
                }
            }
        }
        __syncthreads();
        for (int e2 = tid; e2 < T * NP; e2 += 256) {
            const int i = e2 / NP, n = e2 % NP;
            if (i < len && n < N) {
                float sb = 0.0f, sc = 0.0f;
#pragma unroll
                for (int s2 = 0; s2 < kSlots; ++s2) {
                    sb += redB[s2][i][n];
                    sc += redC[s2][i][n];
                }
                const int64_t o = ((gblk * p.B + b) * L + t0 + i) * N + n;
                p.pB[o] = sb;
                p.pC[o] = sc;
            }
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < SPL; ++j) dAt[j] += dAc[j];
        dDt += dDc;
        dTt += dTc;
    }

    if (dvalid) {
        if (nvalid > 0) {
            if (p.dh0 != nullptr) store_k<SPL>(p.dh0 + (b * D + d) * N + n0, gad, nvalid, vecN);
            store_k<SPL>(p.pA + (b * D + d) * N + n0, dAt, nvalid, vecN);
        }
        if (q == 0) {
            p.pD[b * D + d] = dDt;
            p.pT[b * D + d] = dTt;
        }
    }
}

template <typename IOT>
__global__ __launch_bounds__(256) void bwd_reduce_bc(const float *pB, const float *pC, int G, int64_t total,
                                                     IOT *dB, IOT *dC) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    float sb = 0.0f, sc = 0.0f;
    for (int g = 0; g < G; ++g) {
        sb += pB[(int64_t)g * total + i];
        sc += pC[(int64_t)g * total + i];
    }
    if (dB) store_io(dB + i, sb);
    if (dC) store_io(dC + i, sc);
}

__global__ __launch_bounds__(256) void bwd_reduce_params(const float *A_log, const float *pA, const float *pD,
                                                         const float *pT, int64_t B, int64_t D, int64_t N,
                                                         float *dA_log, float *dD, float *ddtb) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < D * N && dA_log) {
        float s = 0.0f;
        for (int64_t b = 0; b < B; ++b) s += pA[b * D * N + i];
        dA_log[i] = s * neg_exp_f(A_log[i]);
    }
    if (i < D) {
        float sD = 0.0f, sT = 0.0f;
        for (int64_t b = 0; b < B; ++b) {
            sD += pD[b * D + i];
            sT += pT[b * D + i];
        }
        if (dD) dD[i] = sD;
        if (ddtb) ddtb[i] = sT;
    }
}

struct BwdWs {
    float *ckpt, *aggs, *pB, *pC, *pA, *pD, *pT;
};

int tile_len(int64_t N) { return N <= 16 ? 16 : (N <= 32 ? 8 : 4); }

BwdWs carve(void *ws, int64_t B, int64_t L, int64_t D, int64_t N, size_t *total) {
    const int T = tile_len(N);
    const int64_t K = std::max<int64_t>(1, (L + T - 1) / T);
    const int64_t G = (D + kCPB - 1) / kCPB;
    char *base = static_cast<char *>(ws);
    size_t off = 0;
    BwdWs r;
    auto take = [&](size_t n) {
        float *ptr = reinterpret_cast<float *>(base ? base + off : nullptr);
        off += ws_align(n * sizeof(float));
        return ptr;
    };
    r.ckpt = take((size_t)(B * K * D * N));
    r.aggs = take((size_t)(B * K * D));
    r.pB = take((size_t)(G * B * L * N));
    r.pC = take((size_t)(G * B * L * N));
    r.pA = take((size_t)(B * D * N));
    r.pD = take((size_t)(B * D));
    r.pT = take((size_t)(B * D));
    if (total) *total = off;
    return r;
}

template <typename IOT, int SPL>
hipError_t launch_bwd_typed(const ScanBwdArgs &a, const BwdWs &w, hipStream_t s) {
    BwdParams p{};
    p.u = a.u; p.dt = a.dt; p.dt_bias = a.dt_bias; p.A_log = a.A_log;
    p.Bm = a.Bm; p.Cm = a.Cm; p.Dskip = a.Dskip; p.z = a.z; p.dy = a.dy; p.dhT = a.dhT;
    p.ckpt = w.ckpt;
    p.du = a.du; p.ddt = a.ddt; p.dz = a.dz; p.dh0 = a.dh0;
    p.pB = w.pB; p.pC = w.pC; p.pA = w.pA; p.pD = w.pD; p.pT = w.pT;
    p.B = a.B; p.L = a.L; p.D = a.D; p.N = a.N;
    constexpr int T = tile_for<SPL>();
    p.K = (int)std::max<int64_t>(1, (a.L + T - 1) / T);
    p.G = (int)((a.D + kCPB - 1) / kCPB);
    const int64_t blocks = (int64_t)p.G * a.B;
    if (a.disc == DISC_ZOH)
        hipLaunchKernelGGL((scan_bwd_kernel<IOT, SPL, DISC_ZOH>), dim3((unsigned)blocks), dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL((scan_bwd_kernel<IOT, SPL, DISC_DB>), dim3((unsigned)blocks), dim3(256), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t total = a.B * a.L * a.N;
    if ((a.dB || a.dC) && total > 0) {
        hipLaunchKernelGGL((bwd_reduce_bc<IOT>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, w.pB,
                           w.pC, p.G, total, static_cast<IOT *>(a.dB), static_cast<IOT *>(a.dC));
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t pn = std::max(a.D * a.N, a.D);
    hipLaunchKernelGGL(bwd_reduce_params, dim3((unsigned)((pn + 255) / 256)), dim3(256), 0, s, a.A_log, w.pA,
                       w.pD, w.pT, a.B, a.D, a.N, a.dA_log, a.dD, a.ddt_bias);
    return hipGetLastError();
}

template <typename IOT>
hipError_t launch_bwd_spl(const ScanBwdArgs &a, const BwdWs &w, hipStream_t s) {
    if (a.N <= 4) return launch_bwd_typed<IOT, 1>(a, w, s);
    if (a.N <= 8) return launch_bwd_typed<IOT, 2>(a, w, s);
    if (a.N <= 16) return launch_bwd_typed<IOT, 4>(a, w, s);
    if (a.N <= 32) return launch_bwd_typed<IOT, 8>(a, w, s);
    return launch_bwd_typed<IOT, 16>(a, w, s);
}

}  // namespace

size_t scan_bwd_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N) {
    size_t total = 0;
    carve(nullptr, B, L, D, N, &total);
    return total;
}

hipError_t launch_scan_bwd(const ScanBwdArgs &a, hipStream_t s) {
    BwdWs w = carve(a.ws, a.B, a.L, a.D, a.N, nullptr);
    ScanFwdArgs f{};
    f.B = a.B; f.L = a.L; f.D = a.D; f.N = a.N; f.W = 0; f.bf16 = a.bf16; f.disc = a.disc;
    f.x = a.u; f.dt = a.dt; f.dt_bias = a.dt_bias; f.A_log = a.A_log; f.Bm = a.Bm; f.Cm = a.Cm;
    f.h0 = a.h0;
    hipError_t e = launch_scan_checkpoints(f, tile_len(a.N), w.ckpt, w.aggs, s);
    if (e != hipSuccess) return e;
    if (a.bf16) return launch_bwd_spl<bf16_t>(a, w, s);
    return launch_bwd_spl<float>(a, w, s);
}

}  // namespace ssm
