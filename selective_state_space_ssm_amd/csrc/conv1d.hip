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

template <typename IOT>
__global__ __launch_bounds__(256) void conv1d_kernel(ConvArgs a) {
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
        if (tt >= 0)
            v = to_f32(X[(b * L + tt) * D + d]);
        else if (a.state_in != nullptr && tt >= -(int64_t)(W - 1))
            v = a.state_in[(b * (W - 1) + (W - 1) + tt) * D + d];
        win[i] = v;
    }
    win[7] = 0.0f;
    for (int64_t t = t0; t < t1; ++t) {
        win[7] = to_f32(X[(b * L + t) * D + d]);
        float acc = cb;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc = fmaf(wk[i], win[i], acc);
#pragma unroll
        for (int i = 0; i < 7; ++i) win[i] = win[i + 1];
        store_io(Y + (b * L + t) * D + d, a.silu ? silu_f(acc) : acc);
    }
    if (a.state_out != nullptr && tile == tiles - 1) {
#pragma unroll
        for (int i = 0; i < 7; ++i) {
            const int j = i - (8 - W);
            if (j >= 0 && j <= W - 2) a.state_out[(b * (W - 1) + j) * D + d] = win[i];
        }
    }
}

}  // namespace

hipError_t launch_conv1d(const ConvArgs &a, hipStream_t s) {
    const int64_t tiles = std::max<int64_t>(1, (a.L + kTL - 1) / kTL);
    const int64_t threads = a.B * tiles * a.D;
    if (threads == 0) return hipSuccess;
    const unsigned blocks = (unsigned)((threads + 255) / 256);
    if (a.bf16)
        hipLaunchKernelGGL(conv1d_kernel<bf16_t>, dim3(blocks), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(conv1d_kernel<float>, dim3(blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace ssm
