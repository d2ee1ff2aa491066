// model.hip -- one streaming token of a whole Mamba-style language model.
//
// "mamba, live" (section "what is actually running") gives the model in its
// streaming form: x = emb[token]; per block LayerNorm, in_proj to [xin, z],
// the causal depthwise conv + SiLU over the carried history, x_proj to
// [dt, B, C], dt_proj and softplus, the selective state update and readout
// gated by SiLU(z), out_proj added to the residual stream; then the final
// LayerNorm and the head tied to the embedding.  LayerNorm is affine with
// eps 1e-5; in_proj, x_proj and out_proj have no bias, the conv and dt_proj
// do (the readings that give the pages' 13.14M parameters for Mamba-mini).
//
// Kernels, in launch order for one token of S streams (4 per block + 1):
//   per block
//     linear<INPROJ>   LayerNorm(x) @ in_proj^T on the matrix cores: the
//                      LayerNorm is folded into the product algebraically
//                      (the raw rows times the weights scaled by the norm's
//                      weight, then the row mean and 1/std applied in the
//                      epilogue with per-column sums of the scaled weights and
//                      of the norm's bias times the weights); block 0 takes
//                      its rows from emb[token] and starts the residual
//                      stream; the epilogue runs the conv step on the xin half
//                      (history shift in place, SiLU) and stores z;
//     linear<XPROJ>    u @ x_proj^T, split into dt (rank R), B and C;
//     step_kernel      dt_proj (rank R, per channel) and the selective state
//                      update of every (stream, channel), gated readout (the
//                      streaming step kernel with a dt_proj prologue);
//     linear<RESID>    y @ out_proj^T added to the residual stream;
//   linear<STORE>      LayerNorm_out(x) @ emb^T, the tied head.
//
// Matrix products: C[M, N] = A[M, K] W[N, K]^T with float32 MFMA
// (v_mfma_f32_16x16x4_f32).  A wavefront owns a 16 x 16 output tile; a
// workgroup holds WN column tiles and splits each tile's reduction over WK
// wavefronts, the shares summed through LDS in a fixed order.  Each lane
// loads 4 consecutive k of one A row and one W row (16 bytes); MFMA call q
// takes element q of every lane, so lane group g supplies k = k0 + 4g + q to
// both operands and the 16 k of a step are all covered.  The reduction runs
// in groups of two 16-k steps held in two register sets: the next group's
// loads are issued before the current group's MFMAs.  At one stream the products are
// matrix-vector: the weights are streamed once, and splitting the reduction
// over up to 16 wavefronts spreads them over many CUs.
#include <math.h>

#include <algorithm>

#include "launch.hpp"
#include "ssm_device.hpp"

namespace ssm {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr float kLnEps = 1e-5f;
constexpr int kMaxConvW = 8;   // widest conv the in_proj epilogue carries

enum { EPI_STORE = 0, EPI_INPROJ = 1, EPI_XPROJ = 2, EPI_RESID = 3 };

struct LinArgs {
    const float *A;      // [M, K], row stride lda
    int64_t lda;
    const float *W;      // [N, K]
    int64_t M, N, K;
    float *C;            // STORE: [M, N] (row stride ldc); RESID: the residual stream, += C
    int64_t ldc;
    // LN prologue: A rows are normalised on the fly, (a - mean) * rstd * lnw + lnb
    // (K = d_model); EMBED: row m of A is emb[tok[m]] (a token outside
    // [0, vocab) gives a NaN row), and the workgroups of column tile 0 write
    // it to the residual stream xres
    const float *lnw, *lnb;
    const int32_t *tok;
    int vocab;
    float *xres;
    // INPROJ (N = 2 Di): xin -> conv + SiLU -> u, z; history [M, Wc-1, Di]
    float *u, *z, *hist;
    const float *cw, *cb;
    int Wc;
    int64_t Di;
    // XPROJ (N = R + 2 Ns): dt [M, R], B [M, Ns], C [M, Ns]
    float *dtl, *Bv, *Cv;
    int R, Ns;
};

// 4 consecutive values of a [K] vector from k (VEC: one 16-byte load), `dflt`
// for a NULL vector and past ke.
template <bool VEC>
__device__ __forceinline__ float4 vec_load(const float *p, int64_t k, int64_t ke, float dflt) {
    if (p == nullptr) return make_float4(dflt, dflt, dflt, dflt);
    if constexpr (VEC) {
        return k < ke ? *reinterpret_cast<const float4 *>(p + k) : make_float4(dflt, dflt, dflt, dflt);
    } else {
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = (k + q < ke) ? p[k + q] : dflt;
        return make_float4(v[0], v[1], v[2], v[3]);
    }
}

// Workgroup = WN x WK wavefronts.  A wavefront owns TN column tiles of 16
// (one A load feeds TN products), the workgroup WN such groups, and each
// reduction is split in WK shares (summed through LDS in a fixed order).
// The reduction runs in groups of U steps held in two register sets: the
// loads of the next group are issued before the products of the current one,
// so each wavefront has 2U steps of loads in flight.
template <int EPI, int WN, int WK, int TN, bool VEC, bool LNA, bool EMBED>
__global__ __launch_bounds__(64 * WN * WK) void linear_kernel(LinArgs a) {
    constexpr int U = 2;
    constexpr int NW = 16 * TN;                        // columns per wavefront
    __shared__ floatx4 red[WK > 1 ? WN * WK : 1][TN][64];
    __shared__ float4 red2[(WK > 1 && LNA) ? WN * WK : 1][TN][64];
    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
    const int wn = wv % WN, wk = wv / WN;
    const int64_t ntn = (a.N + NW * WN - 1) / (NW * WN);
    // XCD-aware order: the hardware deals workgroups round-robin over the 8
    // XCDs; after the remap each XCD holds a contiguous run of logical
    // workgroups, taken column-tile-major, so an XCD streams only its share
    // of the weights through its own L2 (every XCD reads the small A)
    const int64_t mtn = (a.M + 15) / 16;
    const int64_t lb = xcd_remap((int64_t)blockIdx.x, (int64_t)gridDim.x, 8);
    const int64_t ntile = lb / mtn;
    const int64_t m0 = (lb % mtn) * 16;
    const int64_t n0 = ntile * (NW * WN) + wn * NW;
    const int li = lane & 15, g = lane >> 4;
    const int64_t am = m0 + li;
    const bool arow = am < a.M;
    const float *Ap;
    bool bad = false;
    if constexpr (EMBED) {
        const int32_t t = arow ? a.tok[am] : 0;
        bad = t < 0 || t >= a.vocab;
        Ap = a.A + (int64_t)(bad ? 0 : t) * a.lda;
    } else {
        Ap = a.A + (arow ? am : 0) * a.lda;
    }
    const float *Wp[TN];
    bool wrow[TN];
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
        const int64_t wr = n0 + 16 * tn + li;
        wrow[tn] = wr < a.N;
        Wp[tn] = a.W + (wrow[tn] ? wr : 0) * a.K;
    }
    // LayerNorm folded into the product (LNA).  With w, b the norm's weight
    // and bias: sum_k LN(x)_k W_nk = rs (P_n - mu c_n) + d_n, where
    // P_n = sum_k x_k (w_k W_nk) is the MFMA product with W scaled by w,
    // c_n = sum_k w_k W_nk and d_n = sum_k b_k W_nk.  mu and rs come from the
    // sums of x - x_0 over the row (shifting by the row's first value keeps
    // the one-pass variance free of cancellation).  Every sum is accumulated
    // from the loads the product makes anyway, so the norm adds no pass over
    // memory.
    float sh = 0.0f, s1 = 0.0f, s2 = 0.0f, cs[TN], ds[TN];
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) cs[tn] = ds[tn] = 0.0f;
    if constexpr (LNA) {
        sh = arow ? Ap[0] : 0.0f;
        if constexpr (EMBED) {
            // the residual stream starts as the embedding row; the workgroups
            // of one row tile each copy a slice of its 16 rows (column tile ct
            // takes k in [ct*ch, (ct+1)*ch)), wavefront 0, a lane per value
            const int64_t ct = ntile, ch = (a.K + ntn - 1) / ntn;
            const int64_t k0 = ct * ch, k1 = min(a.K, k0 + ch);
            if (wv == 0) {
                for (int64_t e = lane; e < 16 * (k1 - k0); e += 64) {
                    const int64_t rr = e / (k1 - k0), k = k0 + e % (k1 - k0), mm = m0 + rr;
                    if (mm < a.M) {
                        const int32_t t = a.tok[mm];
                        const bool b2 = t < 0 || t >= a.vocab;
                        const float ev = a.A[(int64_t)(b2 ? 0 : t) * a.lda + k];   // row 0 stands in
                        a.xres[mm * a.K + k] = b2 ? NAN : ev;
                    }
                }
            }
        }
    }
    // this wavefront's share of the reduction, in steps of 16
    const int64_t steps = (a.K + 15) / 16;
    const int64_t per = (steps + WK - 1) / WK;
    const int64_t kb = wk * per * 16, ke = min(a.K, (wk + 1) * per * 16);
    floatx4 acc[TN];
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) acc[tn] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    struct Frag {
        float4 xa[U], xw[U][TN], lw[U], lb[U];
    };
    auto load = [&](Frag &f, int64_t k0) {
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const int64_t kk = k0 + 16 * j + 4 * g;
            f.xa[j] = vec_load<VEC>(arow ? Ap : nullptr, kk, ke, 0.0f);
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) f.xw[j][tn] = vec_load<VEC>(wrow[tn] ? Wp[tn] : nullptr, kk, ke, 0.0f);
            if constexpr (LNA) {
                f.lw[j] = vec_load<VEC>(a.lnw, kk, ke, 1.0f);
                f.lb[j] = vec_load<VEC>(a.lnb, kk, ke, 0.0f);
            }
        }
    };
    auto comp = [&](const Frag &f, int64_t k0) {
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const float av[4] = {f.xa[j].x, f.xa[j].y, f.xa[j].z, f.xa[j].w};
            if constexpr (LNA) {
                const int64_t kk = k0 + 16 * j + 4 * g;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (kk + q < ke) {
                        const float t = av[q] - sh;
                        s1 += t;
                        s2 = fmaf(t, t, s2);
                    }
                }
            }
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) {
                float bv[4] = {f.xw[j][tn].x, f.xw[j][tn].y, f.xw[j][tn].z, f.xw[j][tn].w};
                if constexpr (LNA) {
                    const float wq[4] = {f.lw[j].x, f.lw[j].y, f.lw[j].z, f.lw[j].w};
                    const float bq[4] = {f.lb[j].x, f.lb[j].y, f.lb[j].z, f.lb[j].w};
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        ds[tn] = fmaf(bq[q], bv[q], ds[tn]);
                        bv[q] = bv[q] * wq[q];
                        cs[tn] += bv[q];
                    }
                }
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    acc[tn] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[q], bv[q], acc[tn], 0, 0, 0);
            }
        }
    };
    Frag f0, f1;
    int64_t k0 = kb;
    if (k0 < ke) load(f0, k0);
    while (k0 < ke) {
        const int64_t k1 = k0 + 16 * U;
        if (k1 < ke) load(f1, k1);
        comp(f0, k0);
        if (k1 >= ke) break;
        const int64_t k2 = k1 + 16 * U;
        if (k2 < ke) load(f0, k2);
        comp(f1, k1);
        k0 = k2;
    }
    if constexpr (WK > 1) {
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
            red[wv][tn][lane] = acc[tn];
            if constexpr (LNA) red2[wv][tn][lane] = make_float4(s1, s2, cs[tn], ds[tn]);
        }
        __syncthreads();
        if (wk != 0) return;
#pragma unroll
        for (int j = 1; j < WK; ++j) {
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) {
                acc[tn] += red[wn + j * WN][tn][lane];
                if constexpr (LNA) {
                    const float4 o = red2[wn + j * WN][tn][lane];
                    if (tn == 0) { s1 += o.x; s2 += o.y; }
                    cs[tn] += o.z; ds[tn] += o.w;
                }
            }
        }
    }
    // row li's statistics and column li's sums, combined over the lane groups
    float mur[4] = {0.0f, 0.0f, 0.0f, 0.0f}, rsr[4] = {1.0f, 1.0f, 1.0f, 1.0f};
    if constexpr (LNA) {
        s1 += __shfl_xor(s1, 16, 64); s1 += __shfl_xor(s1, 32, 64);
        s2 += __shfl_xor(s2, 16, 64); s2 += __shfl_xor(s2, 32, 64);
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
            cs[tn] += __shfl_xor(cs[tn], 16, 64); cs[tn] += __shfl_xor(cs[tn], 32, 64);
            ds[tn] += __shfl_xor(ds[tn], 16, 64); ds[tn] += __shfl_xor(ds[tn], 32, 64);
        }
        const float mk = s1 / (float)a.K;
        const float mu = bad ? NAN : sh + mk;
        const float rs = 1.0f / sqrtf(fmaxf(s2 / (float)a.K - mk * mk, 0.0f) + kLnEps);
        // this lane's output rows are 4g + r; their statistics sit in lanes 4g + r
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            mur[r] = __shfl(mu, 4 * g + r, 64);
            rsr[r] = __shfl(rs, 4 * g + r, 64);
        }
    }
    // lane holds rows m0 + 4g + r, column n0 + 16 tn + li.  Everything the
    // epilogue reads (the residual, the conv history and taps) is loaded for
    // all of the lane's outputs before the first store: the compiler cannot
    // move a load of one output's column above another output's store.
    float v[TN][4];
    bool ok[TN][4];
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
        const int64_t n = n0 + 16 * tn + li;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            ok[tn][r] = n < a.N && m0 + 4 * g + r < a.M;
            v[tn][r] = acc[tn][r];
            if constexpr (LNA) v[tn][r] = rsr[r] * (v[tn][r] - mur[r] * cs[tn]) + ds[tn];
        }
    }
    if constexpr (EPI == EPI_RESID) {
        float old[TN][4];
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                old[tn][r] = ok[tn][r] ? a.C[(m0 + 4 * g + r) * a.ldc + n0 + 16 * tn + li] : 0.0f;
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (ok[tn][r]) a.C[(m0 + 4 * g + r) * a.ldc + n0 + 16 * tn + li] = old[tn][r] + v[tn][r];
    } else if constexpr (EPI == EPI_INPROJ) {
        // causal conv over [history, xin] for the xin half: bias, then taps
        // oldest to newest; the history shifts by one input (this thread
        // owns the (stream, channel) column); the z half is stored as is
        constexpr int MH = kMaxConvW - 1;
        const int64_t Di = a.Di;
        const int W = a.Wc;
        float hv[TN][4][MH], cwv[TN][kMaxConvW], cbv[TN];
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
            const int64_t n = n0 + 16 * tn + li;
            const bool xin = n < Di && n < a.N;
#pragma unroll
            for (int j = 0; j < kMaxConvW; ++j) cwv[tn][j] = (xin && j < W) ? a.cw[n * W + j] : 0.0f;
            cbv[tn] = (xin && a.cb) ? a.cb[n] : 0.0f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float *hp = a.hist + (m0 + 4 * g + r) * (int64_t)(W - 1) * Di + n;
#pragma unroll
                for (int j = 0; j < MH; ++j) hv[tn][r][j] = (xin && ok[tn][r] && j < W - 1) ? hp[j * Di] : 0.0f;
            }
        }
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
            const int64_t n = n0 + 16 * tn + li;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (!ok[tn][r]) continue;
                const int64_t m = m0 + 4 * g + r;
                if (n < Di) {
                    float cacc = cbv[tn];
#pragma unroll
                    for (int j = 0; j < MH; ++j)
                        if (j < W - 1) cacc = fmaf(cwv[tn][j], hv[tn][r][j], cacc);
                    float cwl = cwv[tn][0];
#pragma unroll
                    for (int j = 1; j < kMaxConvW; ++j)
                        if (j == W - 1) cwl = cwv[tn][j];
                    cacc = fmaf(cwl, v[tn][r], cacc);
                    float *hp = a.hist + m * (int64_t)(W - 1) * Di + n;
#pragma unroll
                    for (int j = 0; j + 1 < MH; ++j)
                        if (j + 1 < W - 1) hp[j * Di] = hv[tn][r][j + 1];
                    if (W > 1) hp[(W - 2) * Di] = v[tn][r];
                    a.u[m * Di + n] = silu_f(cacc);
                } else {
                    a.z[m * Di + (n - Di)] = v[tn][r];
                }
            }
        }
    } else {
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
            const int64_t n = n0 + 16 * tn + li;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (!ok[tn][r]) continue;
                const int64_t m = m0 + 4 * g + r;
                if constexpr (EPI == EPI_STORE) {
                    a.C[m * a.ldc + n] = v[tn][r];
                } else {   // EPI_XPROJ
                    if (n < a.R)
                        a.dtl[m * a.R + n] = v[tn][r];
                    else if (n < a.R + a.Ns)
                        a.Bv[m * a.Ns + (n - a.R)] = v[tn][r];
                    else
                        a.Cv[m * a.Ns + (n - a.R - a.Ns)] = v[tn][r];
                }
            }
        }
    }
}

template <int EPI, int WN, int WK, int TN, bool LNA, bool EMBED>
hipError_t launch_lin_cfg(const LinArgs &a, hipStream_t s) {
    const int64_t blocks = ((a.M + 15) / 16) * ((a.N + 16 * TN * WN - 1) / (16 * TN * WN));
    if (blocks <= 0) return hipSuccess;
    const bool vec = (a.K % 4 == 0) && (a.lda % 4 == 0);
    const dim3 grid((unsigned)blocks), blk(64 * WN * WK);
    if (vec)
        hipLaunchKernelGGL((linear_kernel<EPI, WN, WK, TN, true, LNA, EMBED>), grid, blk, 0, s, a);
    else
        hipLaunchKernelGGL((linear_kernel<EPI, WN, WK, TN, false, LNA, EMBED>), grid, blk, 0, s, a);
    return hipGetLastError();
}

// Launch shape by the number of 16 x 16 output tiles (chosen by a sweep of
// the Mamba-mini products at 1 and 256 streams):
//  - plenty of tiles (in_proj and the head at 256 streams): two column
//    tiles per wavefront, two wavefronts side by side, the reduction split
//    in two;
//  - a few hundred tiles over a long reduction (out_proj at 256 streams):
//    two column tiles per wavefront, the reduction split over 8;
//  - otherwise one column tile per workgroup and the reduction split over up
//    to 16 wavefronts (shares of at least 24), so that few-stream products
//    stream their weights from many CUs with several loads in flight.
template <int EPI, bool LNA = false, bool EMBED = false>
hipError_t launch_lin(const LinArgs &a, hipStream_t s) {
    const int64_t tiles = ((a.M + 15) / 16) * ((a.N + 15) / 16);
    if (tiles >= 2048) return launch_lin_cfg<EPI, 2, 2, 2, LNA, EMBED>(a, s);
    if (tiles >= 1024) return launch_lin_cfg<EPI, 4, 1, 1, LNA, EMBED>(a, s);
    if (tiles >= 256 && a.K >= 768) return launch_lin_cfg<EPI, 1, 8, 2, LNA, EMBED>(a, s);
    const int64_t share = a.K / 24;
    if (share >= 16) return launch_lin_cfg<EPI, 1, 16, 1, LNA, EMBED>(a, s);
    if (share >= 8) return launch_lin_cfg<EPI, 1, 8, 1, LNA, EMBED>(a, s);
    if (share >= 4) return launch_lin_cfg<EPI, 1, 4, 1, LNA, EMBED>(a, s);
    if (share >= 2) return launch_lin_cfg<EPI, 1, 2, 1, LNA, EMBED>(a, s);
    return launch_lin_cfg<EPI, 1, 1, 1, LNA, EMBED>(a, s);
}

struct ModelWs {
    float *x, *u, *z, *dtl, *Bv, *Cv, *y;
};

ModelWs carve_model(void *ws, int64_t S, int64_t dm, int64_t Di, int64_t N, int64_t R, size_t *total) {
    char *base = static_cast<char *>(ws);
    size_t off = 0;
    auto take = [&](int64_t n) {
        float *p = reinterpret_cast<float *>(base ? base + off : nullptr);
        off += ws_align((size_t)n * sizeof(float));
        return p;
    };
    ModelWs w;
    w.x = take(S * dm);
    w.u = take(S * Di);
    w.z = take(S * Di);
    w.dtl = take(S * R);
    w.Bv = take(S * N);
    w.Cv = take(S * N);
    w.y = take(S * Di);
    if (total) *total = off;
    return w;
}

}  // namespace

size_t model_workspace_bytes(int64_t S, int64_t dm, int64_t Di, int64_t N, int64_t R) {
    size_t total = 0;
    carve_model(nullptr, S, dm, Di, N, R, &total);
    return total;
}

hipError_t launch_model_decode(const ModelArgs &a, hipStream_t s) {
    const int64_t S = a.S, dm = a.dm, Di = a.Di, N = a.N, R = a.R;
    const int W = a.W;
    ModelWs w = carve_model(a.ws, S, dm, Di, N, R, nullptr);
    hipError_t e;
    for (int l = 0; l < a.nl; ++l) {
        const ModelLayer &L = a.layers[l];
        // LayerNorm (block 0: of the embedding rows) fused into in_proj, and
        // the conv step with SiLU on the xin half
        LinArgs p{};
        p.lda = dm; p.W = L.in_proj; p.M = S; p.N = 2 * Di; p.K = dm;
        p.lnw = L.norm_w; p.lnb = L.norm_b;
        p.u = w.u; p.z = w.z; p.hist = a.conv + (int64_t)l * S * (W - 1) * Di; p.cw = L.conv_w; p.cb = L.conv_b;
        p.Wc = W; p.Di = Di;
        if (l == 0) {
            p.A = a.emb; p.tok = a.tok; p.vocab = a.V; p.xres = w.x;
            e = launch_lin<EPI_INPROJ, true, true>(p, s);
        } else {
            p.A = w.x;
            e = launch_lin<EPI_INPROJ, true, false>(p, s);
        }
        if (e != hipSuccess) return e;
        // x_proj -> dt (rank R), B, C
        LinArgs q{};
        q.A = w.u; q.lda = Di; q.W = L.x_proj; q.M = S; q.N = R + 2 * N; q.K = Di;
        q.dtl = w.dtl; q.Bv = w.Bv; q.Cv = w.Cv; q.R = (int)R; q.Ns = (int)N;
        if ((e = launch_lin<EPI_XPROJ>(q, s)) != hipSuccess) return e;
        // dt_proj (rank R) fused into the selective step, gated
        StepArgs st{};
        st.nblk = 1; st.S = S; st.D = Di; st.N = N; st.W = 0; st.bf16 = 0; st.disc = 0; st.state_bf16 = 0;
        st.h = a.h + (int64_t)l * S * Di * N; st.conv_state = nullptr;
        st.x = w.u; st.dt = nullptr; st.Bm = w.Bv; st.Cm = w.Cv; st.z = w.z;
        st.conv_w = nullptr; st.conv_b = nullptr; st.dt_bias = L.dt_b; st.A_log = L.A_log; st.Dskip = L.Dskip;
        st.y = w.y;
        st.dt_low = w.dtl; st.dt_w = L.dt_w; st.dt_rank = (int)R;
        if ((e = launch_step_dtproj(st, s)) != hipSuccess) return e;
        // out_proj into the residual stream
        LinArgs o{};
        o.A = w.y; o.lda = Di; o.W = L.out_proj; o.M = S; o.N = dm; o.K = Di; o.C = w.x; o.ldc = dm;
        if ((e = launch_lin<EPI_RESID>(o, s)) != hipSuccess) return e;
    }
    // final LayerNorm fused into the tied head
    LinArgs hd{};
    hd.A = w.x; hd.lda = dm; hd.W = a.emb; hd.M = S; hd.N = a.V; hd.K = dm; hd.C = a.logits; hd.ldc = a.V;
    hd.lnw = a.norm_f_w; hd.lnb = a.norm_f_b;
    return launch_lin<EPI_STORE, true, false>(hd, s);
}

}  // namespace ssm
