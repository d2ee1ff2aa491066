// launch.hpp -- internal interface between the C-ABI layer (abi.cpp) and the
// kernel launchers.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ssm {

struct ConvArgs {
    int64_t B, L, D;
    int W;
    int silu;
    int bf16;
    const void *x;
    const float *w, *b, *state_in;
    float *state_out;
    void *y;
};
hipError_t launch_conv1d(const ConvArgs &a, hipStream_t s);

struct ScanFwdArgs {
    int64_t B, L, D, N;
    int W;          // 0: no fused conv
    int bf16;
    int disc;
    int64_t chunk_len;  // resolved: >= L means a single chunk
    const void *x, *dt;
    const float *dt_bias, *A_log;
    const void *Bm, *Cm;
    const float *Dskip;
    const void *z;
    const float *conv_w, *conv_b, *conv_state_in;
    float *conv_state_out;
    const float *h0;
    float *hT;
    void *y;
    void *ws;
};
// Time-chunk length the library picks for this shape (>= L: no split).
int64_t scan_fwd_auto_chunk(int64_t B, int64_t L, int64_t D, int64_t N);
size_t scan_fwd_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N, int W,
                                int64_t chunk_len);
hipError_t launch_scan_fwd(const ScanFwdArgs &a, hipStream_t s);
struct ScanBwdArgs {
    int64_t B, L, D, N;
    int W;                   // conv width, 0 = no conv prologue
    int bf16;
    int disc;
    const void *x, *dt;      // x is u when W == 0
    const float *dt_bias, *A_log;
    const void *Bm, *Cm;
    const float *Dskip;
    const void *z;
    const float *conv_w, *conv_b, *conv_state_in;
    const float *h0;
    const void *dy;
    const float *dhT;
    void *dx, *ddt;
    float *ddt_bias, *dA_log;
    void *dB, *dC;
    float *dD;
    void *dz;
    float *dh0;
    float *dconv_w, *dconv_b, *dconv_state_in;
    void *ws;
};
size_t scan_bwd_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N);
hipError_t launch_scan_bwd(const ScanBwdArgs &a, hipStream_t s);

struct StepArgs {
    int64_t nblk, S, D, N;
    int W;
    int bf16;
    int disc;
    float *h, *conv_state;
    const void *x, *dt, *Bm, *Cm, *z;
    const float *conv_w, *conv_b, *dt_bias, *A_log, *Dskip;
    void *y;
};
hipError_t launch_step(const StepArgs &a, hipStream_t s);

// Byte offset helper for workspace carving (256-byte aligned regions).
inline size_t ws_align(size_t n) { return (n + 255) & ~(size_t)255; }

}  // namespace ssm
