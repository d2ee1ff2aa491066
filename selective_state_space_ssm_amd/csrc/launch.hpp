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

// Backward of u = SiLU(conv(x)) from du = dLoss/du: dx, the tap and bias
// gradients and the carried history's gradient (each output may be null).
struct ConvBwdArgs {
    int64_t B, L, D;
    int W;
    int bf16;
    const void *x, *du;                  // [B, L, D] io
    const float *w, *b, *state_in;       // [D, W], [D] (null: 0), [B, W-1, D] (null: zeros)
    void *dx;                            // [B, L, D] io
    float *dw, *db, *dstate;             // [D, W], [D], [B, W-1, D]
    float *ws;                           // conv1d_bwd_workspace_bytes
};
size_t conv1d_bwd_workspace_bytes(int64_t B, int64_t L, int64_t D);
hipError_t launch_conv1d_bwd(const ConvBwdArgs &a, hipStream_t s);

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
// Time-chunk length the library picks for this shape (>= L: no split); W is
// the fused conv width (0: none) and disc the decay form.
int64_t scan_fwd_auto_chunk(int64_t B, int64_t L, int64_t D, int64_t N, int W, int disc);
size_t scan_fwd_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N, int W,
                                int64_t chunk_len);
hipError_t launch_scan_fwd(const ScanFwdArgs &a, hipStream_t s);
// The exact state at the start of every time chunk (chunks of `chunk` tokens,
// at least two): local scans of chunks 0..K-2, then the carries.  agg_h
// [B, K, D, N] receives the start states (chunk 0: h0), agg_s [B, K, D] the
// sums of dt of chunks 0..K-2.  Only x, dt, dt_bias, A_log, B, the conv
// inputs and h0 of `a` are read.
hipError_t launch_scan_chunk_starts(const ScanFwdArgs &a, int64_t chunk, float *agg_h, float *agg_s,
                                   hipStream_t s);
struct ScanBwdArgs {
    int64_t B, L, D, N;
    int64_t chunk;           // resolved time-chunk length (>= L: no split)
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
// Time-chunk length of the backward for this shape and request (0: the
// library's choice, -1: never split, > 0: rounded up to a multiple of 64).
int64_t scan_bwd_chunk(int64_t B, int64_t L, int64_t D, int64_t N, int64_t requested);
// W: conv width (0: none), es: bytes per io element
size_t scan_bwd_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N, int64_t chunk, int W, int64_t es);
hipError_t launch_scan_bwd(const ScanBwdArgs &a, hipStream_t s);

struct StepArgs {
    int64_t nblk, S, D, N;
    int W;
    int bf16;
    int disc;
    int state_bf16;          // h stored as bf16 (computed in float32)
    void *h;
    float *conv_state;
    const void *x, *dt, *Bm, *Cm, *z;
    const float *conv_w, *conv_b, *dt_bias, *A_log, *Dskip;
    void *y;
    // launch_step_dtproj only: dt_raw = dt_low[s] . dt_w[d] (rank dt_rank)
    const float *dt_low, *dt_w;
    int dt_rank;
};
hipError_t launch_step(const StepArgs &a, hipStream_t s);
// The step of the whole-model decode: float32, dt*B form, no conv, dt_raw
// formed from the low-rank projection instead of loaded.
hipError_t launch_step_dtproj(const StepArgs &a, hipStream_t s);

// One streaming token of a whole Mamba-style model (model.hip).
struct ModelLayer {
    const float *norm_w, *norm_b;     // [dm] (NULL: 1, 0)
    const float *in_proj;             // [2 Di, dm]
    const float *conv_w, *conv_b;     // [Di, W], [Di]
    const float *x_proj;              // [R + 2N, Di]
    const float *dt_w, *dt_b;         // [Di, R], [Di]
    const float *A_log;               // [Di, N]
    const float *Dskip;               // [Di]
    const float *out_proj;            // [dm, Di]
};
struct ModelArgs {
    int64_t S;
    int V, dm, nl, Di, N, R, W;
    const float *emb;                 // [V, dm], also the head
    const float *norm_f_w, *norm_f_b;
    const ModelLayer *layers;         // host array [nl]
    const int32_t *tok;               // [S]
    float *h;                         // [nl, S, Di, N]
    float *conv;                      // [nl, S, W-1, Di]
    float *logits;                    // [S, V]
    void *ws;
};
size_t model_workspace_bytes(int64_t S, int64_t dm, int64_t Di, int64_t N, int64_t R);
hipError_t launch_model_decode(const ModelArgs &a, hipStream_t s);

// The device address of this device's copy of the library's static scratch
// buffer (SSM_STATIC_SCRATCH_BYTES, scratch.hip), looked up on the first call
// on each device with that device current.
hipError_t static_scratch(void **ptr);

// Byte offset helper for workspace carving (256-byte aligned regions).
inline size_t ws_align(size_t n) { return (n + 255) & ~(size_t)255; }

}  // namespace ssm
