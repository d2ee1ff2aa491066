// conv1d.hip -- causal depthwise convolution (+ optional SiLU) for gfx950.
//
// "mamba, live" (section "what is actually running"): xc =
// SiLU(depthwise_conv4(xin)), a 4-tap causal conv per channel; TensorViz
// manifest step "local": left padded, reading the current and W-1 earlier
// inputs.  Cross-correlation with the current token on tap W-1:
//   y[t] = b + sum_{k<W} w[k] * xt[t - (W-1) + k]
//
// Each thread owns one channel and a run of kTL consecutive tokens, keeping
// the last W-1 inputs in registers, so every input is read from HBM once
// (plus W-1 re-reads at the start of each run).  Adjacent threads take
// adjacent channels, so a wavefront reads and writes 64 consecutive values of
// each token row.  The taps sit right-aligned in an 8-slot window, the same
// arithmetic as the conv prologue fused into the scan.
#include <algorithm>

#include "launch.hpp"
#include "ssm_device.hpp"

namespace ssm {
namespace {

constexpr int kTL = 32;

// CW > 0: the width is known to be CW; only the last CW of the 8 tap slots
// (the nonzero ones) enter the sum, and only the CW-1 inputs before a tile
// are loaded.
template <typename IOT, int CW = 0>
__global__ __launch_bounds__(256) void conv1d_kernel(ConvArgs a) {
    constexpr int K0 = CW > 0 ? 8 - CW : 0;   // first nonzero tap slot
    const IOT *X = static_cast<const IOT *>(a.x);
    IOT *Y = static_cast<IOT *>(a.y);
    const int64_t D = a.D, L = a.L;
    const int64_t tiles = std::max<int64_t>(1, (L + kTL - 1) / kTL);
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= a.B * tiles * D) return;
    const int64_t d = gid % D;
    const int64_t tile = (gid / D) % tiles;
    const int64_t b = gid / (D * tiles);
    const int W = a.W;
    const int64_t t0 = tile * kTL;
    const int64_t t1 = std::min(L, t0 + kTL);

    float wk[8], win[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int kk = i - (8 - W);
        wk[i] = (kk >= 0) ? a.w[d * W + kk] : 0.0f;
    }
    const float cb = a.b ? a.b[d] : 0.0f;
#pragma unroll
    for (int i = 0; i < 7; ++i) {
        const int64_t tt = t0 - 7 + i;
        float v = 0.0f;
        if (i >= K0 - 1) {   // slots below are shifted out before any tap reads them
            if (tt >= 0)
                v = to_f32(X[(b * L + tt) * D + d]);
            else if (a.state_in != nullptr && tt >= -(int64_t)(W - 1))
                v = a.state_in[(b * (W - 1) + (W - 1) + tt) * D + d];
        }
        win[i] = v;
    }
    win[7] = 0.0f;
    // eight tokens at a time, their inputs requested before any is used
    // (indices clamped into the sequence, values past it unused)
    for (int64_t tg = t0; tg < t1; tg += 8) {
        float xv[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) xv[q] = to_f32(X[(b * L + std::min(tg + q, t1 - 1)) * D + d]);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            if (tg + q < t1) {
                win[7] = xv[q];
                float acc = cb;
#pragma unroll
                for (int i = K0; i < 8; ++i) acc = fmaf(wk[i], win[i], acc);
#pragma unroll
                for (int i = 0; i < 7; ++i) win[i] = win[i + 1];
                store_io(Y + (b * L + tg + q) * D + d, a.silu ? silu_f(acc) : acc);
            }
        }
    }
    if (a.state_out != nullptr && tile == tiles - 1) {
#pragma unroll
        for (int i = 0; i < 7; ++i) {
            const int j = i - (8 - W);
            if (j >= 0 && j <= W - 2) a.state_out[(b * (W - 1) + j) * D + d] = win[i];
        }
    }
}

// Backward of u = SiLU(conv(x)) given du = dLoss/du.  With xc the conv
// output and s = sigmoid(xc): gx = du s (1 + xc (1 - s)) (the SiLU
// derivative), dx_t = sum_k w_k gx_{t+(W-1)-k} (the transposed conv: input t
// feeds outputs t..t+W-1), dw_k = sum_t gx_t x_{t-(W-1)+k}, db = sum_t gx_t,
// and inputs before t = 0 (the carried history) get the dx of their
// position.  A thread owns one channel and a run of kBL tokens; it walks a
// lead token s from the run start to 7 past its end, recomputing xc_s from
// an 8-input window and keeping the last 8 gx values, and emits dx_{s-7}
// (each output token's 8 gx values then lie in the ring).  Tap and bias sums
// go to per-(batch row, run) partials, added in a fixed order by
// conv1d_bwd_reduce.
constexpr int kBL = 64;

// CW > 0: the width is known to be CW, and only the last CW of the 8 tap slots
// (the nonzero ones) enter the sums.
template <typename IOT, int CW = 0>
__global__ __launch_bounds__(256) void conv1d_bwd_kernel(ConvBwdArgs a) {
    constexpr int K0 = CW > 0 ? 8 - CW : 0;   // first nonzero tap slot
    const IOT *X = static_cast<const IOT *>(a.x);
    const IOT *DU = static_cast<const IOT *>(a.du);
    IOT *DX = static_cast<IOT *>(a.dx);
    const int64_t D = a.D, L = a.L;
    const int64_t runs = std::max<int64_t>(1, (L + kBL - 1) / kBL);
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= a.B * runs * D) return;
    const int64_t d = gid % D;
    const int64_t run = (gid / D) % runs;
    const int64_t b = gid / (D * runs);
    const int W = a.W;
    const int64_t t0 = run * kBL;
    const int64_t t1 = std::min(L, t0 + kBL);

    float wk[8], win[8], gr[8], pw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int kk = i - (8 - W);
        wk[i] = (kk >= 0) ? a.w[d * W + kk] : 0.0f;
        gr[i] = 0.0f;
        pw[i] = 0.0f;
    }
    const float cb = a.b ? a.b[d] : 0.0f;
    float pb = 0.0f;
    // input j sits in window slot j mod 8 and gx_j in ring slot j mod 8 (t0
    // is a multiple of 8): the windows rotate by renaming
    win[0] = 0.0f;
#pragma unroll
    for (int i = 0; i < 7; ++i) {
        const int64_t tt = t0 - 7 + i;
        float v = 0.0f;
        if (tt >= 0)
            v = to_f32(X[(b * L + tt) * D + d]);
        else if (a.state_in != nullptr && tt >= -(int64_t)(W - 1))
            v = a.state_in[(b * (W - 1) + (W - 1) + tt) * D + d];
        win[i + 1] = v;
    }
    // lead tokens s = t0 .. t1 + 6, eight at a time (q = s mod 8); the
    // group's inputs are all requested before any is used (indices clamped
    // into the sequence, values past it unused)
    static_assert(kBL % 8 == 0, "runs start at multiples of 8");
    for (int64_t sg = t0; sg < t1 + 7; sg += 8) {
        float xv[8], dv[8];
        if (L > 0) {
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int64_t o = (b * L + std::min(sg + q, L - 1)) * D + d;
                xv[q] = to_f32(X[o]);
                dv[q] = to_f32(DU[o]);
            }
        }
        static_for<8>([&](auto qc) {
            constexpr int q = decltype(qc)::value;
            const int64_t s = sg + q;
            float gxs = 0.0f;
            if (s < L && s < t1 + 7) {
                win[q] = xv[q];   // x_s, in the slot of x_{s-8}
                float acc = cb;
#pragma unroll
                for (int i = K0; i < 8; ++i) acc = fmaf(wk[i], win[(q + 1 + i) & 7], acc);
                const float sgm = sigmoid_f(acc);
                gxs = dv[q] * (sgm * (1.0f + acc * (1.0f - sgm)));
                if (s < t1) {
                    pb += gxs;
#pragma unroll
                    for (int i = K0; i < 8; ++i) pw[i] = fmaf(gxs, win[(q + 1 + i) & 7], pw[i]);
                }
            }
            gr[q] = gxs;
            const int64_t t = s - 7;
            if (t < t1 && s < t1 + 7 && (t >= t0 || (run == 0 && t >= -(int64_t)(W - 1)))) {
                float acc = 0.0f;
#pragma unroll
                for (int i = K0; i < 8; ++i) acc = fmaf(wk[i], gr[(q - i) & 7], acc);   // gx_{t+7-i}
                if (t >= 0) {
                    store_io(DX + (b * L + t) * D + d, acc);
                } else if (a.dstate != nullptr) {
                    a.dstate[(b * (W - 1) + (W - 1) + t) * D + d] = acc;
                }
            }
        });
    }
    float *pp = a.ws + (b * runs + run) * 9 * D + d;
#pragma unroll
    for (int i = K0; i < 8; ++i) pp[i * D] = pw[i];   // slots below 8 - W are never read
    pp[8 * D] = pb;
}

// dconv_w, dconv_b: the partials of every (batch row, run) in order.
__global__ __launch_bounds__(256) void conv1d_bwd_reduce(const float *ws, int64_t parts, int64_t D, int W, float *dw,
                                                         float *db) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= (int64_t)(W + 1) * D) return;
    const int64_t d = gid % D;
    const int k = (int)(gid / D);                 // tap k < W, or the bias at k == W
    const int slot = k < W ? k + (8 - W) : 8;
    // in order, eight loads in flight
    float acc = 0.0f;
    int64_t p = 0;
    for (; p + 8 <= parts; p += 8) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = ws[((p + j) * 9 + slot) * D + d];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc += v[j];
    }
    for (; p < parts; ++p) acc += ws[(p * 9 + slot) * D + d];
    if (k < W) {
        if (dw) dw[d * W + k] = acc;
    } else if (db) {
        db[d] = acc;
    }
}

}  // namespace

size_t conv1d_bwd_workspace_bytes(int64_t B, int64_t L, int64_t D) {
    const int64_t runs = std::max<int64_t>(1, (L + kBL - 1) / kBL);
    return ws_align((size_t)(B * runs * 9 * D) * sizeof(float));
}

hipError_t launch_conv1d_bwd(const ConvBwdArgs &a, hipStream_t s) {
    const int64_t runs = std::max<int64_t>(1, (a.L + kBL - 1) / kBL);
    const int64_t threads = a.B * runs * a.D;
    if (threads == 0) return hipSuccess;
    const unsigned blocks = (unsigned)((threads + 255) / 256);
    if (a.bf16 && a.W == 4)
        hipLaunchKernelGGL((conv1d_bwd_kernel<bf16_t, 4>), dim3(blocks), dim3(256), 0, s, a);
    else if (a.bf16)
        hipLaunchKernelGGL(conv1d_bwd_kernel<bf16_t>, dim3(blocks), dim3(256), 0, s, a);
    else if (a.W == 4)
        hipLaunchKernelGGL((conv1d_bwd_kernel<float, 4>), dim3(blocks), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(conv1d_bwd_kernel<float>, dim3(blocks), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.dw || a.db) {
        const int64_t n = (int64_t)(a.W + 1) * a.D;
        hipLaunchKernelGGL(conv1d_bwd_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a.ws,
                           a.B * runs, a.D, a.W, a.dw, a.db);
        e = hipGetLastError();
    }
    return e;
}

hipError_t launch_conv1d(const ConvArgs &a, hipStream_t s) {
    const int64_t tiles = std::max<int64_t>(1, (a.L + kTL - 1) / kTL);
    const int64_t threads = a.B * tiles * a.D;
    if (threads == 0) return hipSuccess;
    const unsigned blocks = (unsigned)((threads + 255) / 256);
    if (a.bf16 && a.W == 4)
        hipLaunchKernelGGL((conv1d_kernel<bf16_t, 4>), dim3(blocks), dim3(256), 0, s, a);
    else if (a.bf16)
        hipLaunchKernelGGL(conv1d_kernel<bf16_t>, dim3(blocks), dim3(256), 0, s, a);
    else if (a.W == 4)
        hipLaunchKernelGGL((conv1d_kernel<float, 4>), dim3(blocks), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(conv1d_kernel<float>, dim3(blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace ssm
