/*
 * ssm.h -- C ABI of the MI355X (gfx950) S6 selective-scan library.
 *
 * The method (pages: "mamba, live", section "what is actually running";
 * "the s6 cell", section "the recurrence"; TensorViz "Carry context through a
 * selective state", explorer page and manifest steps "local", "select",
 * "state", "read"):
 *
 *   u      = SiLU(causal_depthwise_conv_W(x))         (optional, fused)
 *   dt     = softplus(dt_raw + dt_bias)                per (b, t, d)
 *   A      = -exp(A_log)                               per (d, n)
 *   h[n]  <- exp(dt*A[n]) * h[n] + coef(dt, A[n]) * B[t, n] * u
 *            coef = dt                 (SSM_DISC_DELTA_B, the dt*B form)
 *            coef = expm1(dt*A) / A    (SSM_DISC_ZOH, exact zero-order hold)
 *   y      = (sum_n C[t, n] * h[n] + Dskip * u) * SiLU(z)   (C reads the
 *            updated state; the gate only when z is given)
 *
 * The same diagonal cell h <- a*h + b*u with the decay fixed per channel
 * instead of computed per token ("the s6 cell", section "one cell, two
 * architectures"; the fixed-decay side) is selected with
 * disc = SSM_DECAY_CONST:
 *   h[n]  <- exp(A[n]) * h[n] + B[t, n] * u,   A = -exp(A_log)
 * with no step size: dt_raw and dt_bias are not read (they may be NULL) and
 * the backward produces no d_dt_raw / d_dt_bias (those outputs are not
 * written).  State width is dstate (1 for a scalar state per channel).
 *
 * Conventions shared by every call
 *  - Layouts are row-major and channel-last:
 *      x, u, dt_raw, z, y and their gradients       [B, L, D]
 *      B, C and their gradients                     [B, L, N]  (shared by all channels)
 *      A_log, dA_log                                [D, N]
 *      dt_bias, Dskip, conv_b and their gradients   [D]
 *      conv_w                                       [D, W]  (tap W-1 multiplies the current input)
 *      h0, hT, dh0, dhT                             [B, D, N]
 *      conv_state_in / conv_state_out               [B, W-1, D]  (oldest input first)
 *  - Tensors marked "io" hold SSM_F32 or SSM_BF16 values as chosen by the
 *    descriptor's io_dtype; every parameter, state and parameter gradient is
 *    float32.  bf16 results are rounded to nearest, ties to even.
 *  - Every pointer is a DEVICE pointer, except the descriptor pointers, which
 *    are host pointers read before the call returns.  The caller owns all
 *    memory: the library never allocates, frees or keeps a pointer after a
 *    call returns.  Every tensor must start on a 16-byte boundary.
 *  - A NULL optional pointer means "absent": dt_bias, Dskip, conv_b read as 0;
 *    z means "no gate"; h0 and conv_state_in read as zeros; a NULL output is
 *    not written.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *    and is asynchronous: nothing synchronises inside a call.  Calls are
 *    reentrant; concurrent calls on different streams must use different
 *    workspaces and outputs.
 *  - Errors: every call returns an ssm_status.  Argument errors are detected
 *    on the host before any HIP call is made, and then nothing is enqueued.
 *    SSM_ERR_HIP reports a failed launch; a fault inside a kernel surfaces at
 *    the caller's next synchronisation.
 *  - Inputs must be finite.  Outputs may not overlap inputs or each other,
 *    except the exact in-place pairs named below.
 */
#ifndef SSM_AMD_SSM_H
#define SSM_AMD_SSM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_ABI_VERSION 2

typedef int32_t ssm_status;
#define SSM_OK 0
#define SSM_ERR_NULL_ARG 1     /* a required pointer is NULL */
#define SSM_ERR_BAD_SHAPE 2    /* a size is out of range or inconsistent, or needs a launch grid
                                  above 2^31 - 1 workgroups */
#define SSM_ERR_UNSUPPORTED 3  /* a valid request the library does not implement */
#define SSM_ERR_WORKSPACE 4    /* workspace NULL or smaller than the queried size */
#define SSM_ERR_ALIGNMENT 5    /* a tensor does not start on a 16-byte boundary */
#define SSM_ERR_ALIAS 6        /* buffers overlap in a way the call does not allow */
#define SSM_ERR_HIP 7          /* a HIP launch failed */
#define SSM_ERR_SCRATCH_LIMIT 8  /* the request needs more than the static scratch buffer holds */

#define SSM_F32 0
#define SSM_BF16 1

#define SSM_DISC_DELTA_B 0     /* write = dt * B * u ("mamba, live"; "the s6 cell") */
#define SSM_DISC_ZOH 1         /* write = expm1(dt*A)/A * B * u (TensorViz explorer) */
#define SSM_DECAY_CONST 2      /* decay exp(A) fixed per (channel, state), write = B * u,
                                  no step size ("the s6 cell", "one cell, two architectures") */

#define SSM_MAX_DSTATE 64
#define SSM_MAX_CONV_WIDTH 8
#define SSM_MAX_SCAN_DIM ((1 << 24) - 1)   /* channels of a sequence scan: a 64-token tile of one
                                             [B, L, D] float32 tensor, and one backward state
                                             checkpoint (D * N <= 64 * D floats), stay under 2^32
                                             bytes, the reach of the kernels' 32-bit offsets */
#define SSM_STATIC_SCRATCH_BYTES (16u << 20)   /* ssm_scan_fwd_static's device buffer, per GPU */

/* Descriptor of a sequence scan (forward or backward). */
typedef struct ssm_scan_desc {
    int64_t batch;       /* B >= 1 */
    int64_t seqlen;      /* L >= 0 */
    int64_t dim;         /* D in [1, SSM_MAX_SCAN_DIM], inner channels */
    int64_t dstate;      /* N in [1, SSM_MAX_DSTATE] */
    int32_t conv_width;  /* 0: x already is the scan input u; 1..8: fused causal conv + SiLU */
    int32_t io_dtype;    /* SSM_F32 or SSM_BF16 */
    int32_t disc;        /* SSM_DISC_DELTA_B, SSM_DISC_ZOH or SSM_DECAY_CONST */
    int32_t chunk_len;   /* 0: library's choice; > 0: split time into chunks of this
                            length (two-level scan); -1: never split time */
} ssm_scan_desc;

/* Descriptor of one streaming step for a stack of independent blocks. */
typedef struct ssm_step_desc {
    int64_t nblocks;     /* >= 1; every per-block tensor gains a leading [nblocks] axis */
    int64_t nstreams;    /* S >= 1 concurrent sequences */
    int64_t dim;         /* D >= 1 */
    int64_t dstate;      /* N in [1, SSM_MAX_DSTATE] */
    int32_t conv_width;  /* 0: x is u; 1..8: causal conv over the carried history + SiLU */
    int32_t io_dtype;    /* SSM_F32 or SSM_BF16 for x, dt_raw, B, C, z, y */
    int32_t disc;        /* SSM_DISC_DELTA_B, SSM_DISC_ZOH or SSM_DECAY_CONST */
    int32_t state_dtype; /* storage of h: SSM_F32 (0), or SSM_BF16 (updated in float32 and
                            rounded to nearest, ties to even, when stored) */
} ssm_step_desc;

/* Descriptor of a causal depthwise convolution. */
typedef struct ssm_conv_desc {
    int64_t batch;       /* B >= 1 */
    int64_t seqlen;      /* L >= 0 */
    int64_t dim;         /* D >= 1 */
    int32_t width;       /* W in [1, SSM_MAX_CONV_WIDTH] */
    int32_t fuse_silu;   /* 1: y = SiLU(conv), 0: y = conv */
    int32_t io_dtype;    /* SSM_F32 or SSM_BF16 for x and y */
    int32_t reserved;    /* must be 0 */
} ssm_conv_desc;

/* Shape of a whole Mamba-style language model (ssm_model_decode_step). */
typedef struct ssm_model_desc {
    int64_t nstreams;    /* S >= 1 independent token streams decoded together */
    int32_t vocab;       /* V >= 1 tokens; the head is tied to the embedding */
    int32_t d_model;     /* residual width, 1 .. SSM_MAX_D_MODEL */
    int32_t n_layers;    /* blocks, >= 1 */
    int32_t d_inner;     /* inner channels per block, >= 1 */
    int32_t d_state;     /* N in [1, SSM_MAX_DSTATE] */
    int32_t dt_rank;     /* rank of the step-size projection, >= 1 */
    int32_t conv_width;  /* W in [1, SSM_MAX_CONV_WIDTH] */
    int32_t reserved;    /* must be 0 */
} ssm_model_desc;
#define SSM_MAX_D_MODEL 8192

/* One block's weights, all float32 device pointers (PyTorch Linear layout,
 * [out_features, in_features]).  NULL optionals: norm_w 1, norm_b 0,
 * conv_b 0, dt_proj_b 0, Dskip 0. */
typedef struct ssm_layer_weights {
    const float *norm_w, *norm_b;      /* [d_model] LayerNorm (eps 1e-5), optional */
    const float *in_proj;              /* [2*d_inner, d_model]: rows 0..d_inner-1 give xin, the rest z */
    const float *conv_w;               /* [d_inner, W], tap W-1 on the current input */
    const float *conv_b;               /* [d_inner], optional */
    const float *x_proj;               /* [dt_rank + 2*d_state, d_inner]: rows give dt, B, C in that order */
    const float *dt_proj_w;            /* [d_inner, dt_rank] */
    const float *dt_proj_b;            /* [d_inner], optional (the scan's dt_bias) */
    const float *A_log;                /* [d_inner, d_state] */
    const float *Dskip;                /* [d_inner], optional */
    const float *out_proj;             /* [d_model, d_inner] */
} ssm_layer_weights;

/* Library version (SSM_ABI_VERSION * 100 + minor). */
int32_t ssm_version(void);

/* Static English text of a status code (never NULL). */
const char *ssm_status_string(ssm_status status);

/*
 * conv1d_causal -- causal depthwise convolution, optionally followed by SiLU
 * ("mamba, live": xc = SiLU(depthwise_conv4(xin)), 4-tap causal, per channel;
 * TensorViz manifest step "local": left padded, reads the current and W-1
 * earlier inputs).
 *   y[b,t,d] = act(b[d] + sum_{k<W} w[d,k] * xt[b, t-(W-1)+k, d])
 * with xt = x for index >= 0 and the carried history state_in (or 0) before.
 *   x         io  [B, L, D]     input
 *   w         f32 [D, W]        taps (required)
 *   b         f32 [D]           bias, optional
 *   state_in  f32 [B, W-1, D]   history before x, optional (zeros)
 *   state_out f32 [B, W-1, D]   the last W-1 inputs after x, optional; must not
 *                               overlap state_in (SSM_ERR_ALIAS)
 *   y         io  [B, L, D]     output (required when L > 0)
 */
ssm_status conv1d_causal(const ssm_conv_desc *desc, const void *x, const float *w,
                         const float *b, const float *state_in, float *state_out,
                         void *y, void *stream);

/* Bytes of device workspace ssm_scan_fwd needs for this descriptor (0 when
 * time is not split). */
ssm_status ssm_scan_fwd_workspace_size(const ssm_scan_desc *desc, size_t *bytes);

/*
 * ssm_scan_fwd -- the selective scan over a whole sequence (the recurrence
 * above, run for t = 0 .. L-1 from h0).  Long sequences with little batch and
 * channel parallelism are split in time into chunks whose end states are
 * combined by the associative rule (P1, W1) then (P2, W2) = (P1*P2, P2*W1 + W2)
 * and then re-scanned from their exact starting states; the result equals the
 * sequential recurrence up to rounding.
 *   x              io  [B, L, D]   u, or the conv input when conv_width > 0 (required)
 *   dt_raw         io  [B, L, D]   required (not read with SSM_DECAY_CONST)
 *   dt_bias        f32 [D]         optional
 *   A_log          f32 [D, N]      required
 *   B, C           io  [B, L, N]   required
 *   Dskip          f32 [D]         optional
 *   z              io  [B, L, D]   gate input, optional
 *   conv_w         f32 [D, W]      required when conv_width > 0, else ignored
 *   conv_b         f32 [D]         optional
 *   conv_state_in  f32 [B, W-1, D] optional
 *   conv_state_out f32 [B, W-1, D] optional (may be exactly conv_state_in)
 *   h0             f32 [B, D, N]   optional
 *   hT             f32 [B, D, N]   optional (may be exactly h0)
 *   y              io  [B, L, D]   required when L > 0
 *   workspace      device memory of ssm_scan_fwd_workspace_size bytes (may be
 *                  NULL when that size is 0)
 */
ssm_status ssm_scan_fwd(const ssm_scan_desc *desc, const void *x, const void *dt_raw,
                        const float *dt_bias, const float *A_log, const void *B,
                        const void *C, const float *Dskip, const void *z,
                        const float *conv_w, const float *conv_b,
                        const float *conv_state_in, float *conv_state_out,
                        const float *h0, float *hT, void *y,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * ssm_scan_fwd_static -- ssm_scan_fwd without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Arguments,
 * results and errors are those of ssm_scan_fwd; the chunk summaries of a
 * time split go to a buffer of SSM_STATIC_SCRATCH_BYTES that the library
 * holds on every GPU it runs on (a static device array, kept until the
 * process ends).  The call allocates nothing.
 *   Returns SSM_ERR_SCRATCH_LIMIT, before any HIP call, when
 *   ssm_scan_fwd_workspace_size for the same descriptor exceeds
 *   SSM_STATIC_SCRATCH_BYTES (pass a shorter chunk_len, or -1, or use
 *   ssm_scan_fwd with a workspace).
 *   Every call on one GPU shares that GPU's buffer: calls that overlap on a
 *   GPU (on different streams, or from different host threads without
 *   ordering) race on it and must be serialised by the caller.  Calls on one
 *   stream are ordered and safe.  The buffer keeps the last call's contents;
 *   every value a call reads from it is written earlier in the same call.
 *   The first call on a device looks up the buffer's device address (a HIP
 *   call that is not capturable): make one call on each device before any
 *   graph capture.
 */
ssm_status ssm_scan_fwd_static(const ssm_scan_desc *desc, const void *x, const void *dt_raw,
                               const float *dt_bias, const float *A_log, const void *B,
                               const void *C, const float *Dskip, const void *z,
                               const float *conv_w, const float *conv_b,
                               const float *conv_state_in, float *conv_state_out,
                               const float *h0, float *hT, void *y, void *stream);

/* Bytes of device workspace ssm_scan_bwd needs for this descriptor. */
ssm_status ssm_scan_bwd_workspace_size(const ssm_scan_desc *desc, size_t *bytes);

/*
 * ssm_scan_bwd -- gradients of ssm_scan_fwd for the loss
 * sum(y * dy) + sum(hT * dhT).  The pages state that the selection maps
 * receive gradients (TensorViz explorer, numerical checks) but give no
 * backward; this is the reverse-mode adjoint of the recurrence: with
 * g = dLoss/dh_t, g_{t-1} = exp(dt_t*A) * g_t + C_{t-1} * dyv_{t-1}.  With
 * conv_width > 0 the conv + SiLU prologue ("mamba, live": the 4-tap causal
 * conv before the scan; TensorViz manifest step "local") is differentiated
 * in the same pass: u is recomputed from x, and the gradient of u flows on
 * through SiLU and the taps to x, conv_w, conv_b and conv_state_in.
 *   x, dt_raw, B, C, z, dy    io  as in ssm_scan_fwd (dy [B, L, D] required)
 *   dt_bias, A_log, Dskip, h0 f32 as in ssm_scan_fwd
 *   conv_w, conv_b, conv_state_in  f32 as in ssm_scan_fwd (conv_w required
 *                             when conv_width > 0; all ignored when it is 0)
 *   dhT        f32 [B, D, N]  optional upstream gradient of hT
 *   dx, d_dt_raw, dz   io [B, L, D]  optional outputs (dx is dLoss/dx: the
 *                                    scan input u when conv_width is 0; dz
 *                                    needs z)
 *   dB, dC             io [B, L, N]  optional outputs (summed over channels)
 *   d_dt_bias, dDskip  f32 [D]       optional outputs (summed over batch and time)
 *                                    (d_dt_raw and d_dt_bias are not written with
 *                                    SSM_DECAY_CONST, which has no step size)
 *   dA_log             f32 [D, N]    optional output (summed over batch and time)
 *   dh0                f32 [B, D, N] optional output
 *   dconv_w   f32 [D, W]      optional output (summed over batch and time)
 *   dconv_b   f32 [D]         optional output (summed over batch and time)
 *   dconv_state_in f32 [B, W-1, D]  optional output, the gradient of the
 *                             carried history (written whether or not
 *                             conv_state_in was given)
 *   The three conv outputs must be NULL when conv_width is 0.
 *   workspace  device memory of ssm_scan_bwd_workspace_size bytes (required)
 * Time chunks (desc->chunk_len: 0 the library's choice, -1 never, > 0 this
 * length rounded up to a multiple of 64): with few channel workgroups the
 * sequence is split in time.  The forward's chunk scan and carry give every
 * chunk its exact start state; a reverse walk over chunk summaries gives its
 * end adjoint (over a chunk the adjoint is affine, g_start = prod(exp(dt*A))
 * * g_end + R); every chunk then runs the backward sweep independently.  The
 * result equals the unsplit backward up to rounding.
 */
ssm_status ssm_scan_bwd(const ssm_scan_desc *desc, const void *x, const void *dt_raw,
                        const float *dt_bias, const float *A_log, const void *B,
                        const void *C, const float *Dskip, const void *z,
                        const float *conv_w, const float *conv_b, const float *conv_state_in,
                        const float *h0, const void *dy, const float *dhT,
                        void *dx, void *d_dt_raw, float *d_dt_bias, float *dA_log,
                        void *dB, void *dC, float *dDskip, void *dz, float *dh0,
                        float *dconv_w, float *dconv_b, float *dconv_state_in,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * ssm_step -- one token of batched streaming decode ("mamba, live": one token
 * in, one token out, constant work; the whole memory is h plus a (W-1)-token
 * conv history per channel).  For every block k, stream s and channel d:
 *   u = SiLU(conv_b + sum_{j<W-1} conv_w[j] * hist[j] + conv_w[W-1] * x)   (conv_width > 0)
 *   hist <- [hist[1..W-2], x]
 *   then one recurrence step of the scan with u, updating h in place.
 * y reads the updated state; with state_dtype SSM_BF16 what is kept for the
 * next token is its bfloat16 rounding (the pages keep the state in float32;
 * bf16 storage halves the state traffic that bounds a decode step).
 * Tensors (each with a leading [nblocks] axis, block-major):
 *   h          f32 or bf16 [S, D, N]   state (state_dtype), in/out (required)
 *   conv_state f32 [S, W-1, D] history, in/out (required when conv_width > 1)
 *   x, dt_raw  io  [S, D]      required (dt_raw not read with SSM_DECAY_CONST)
 *   B, C       io  [S, N]      required
 *   z          io  [S, D]      optional gate input
 *   conv_w     f32 [D, W]      required when conv_width > 0
 *   conv_b, dt_bias, Dskip  f32 [D]  optional
 *   A_log      f32 [D, N]      required
 *   y          io  [S, D]      output (required)
 */
ssm_status ssm_step(const ssm_step_desc *desc, void *h, float *conv_state, const void *x,
                    const void *dt_raw, const void *B, const void *C, const void *z,
                    const float *conv_w, const float *conv_b, const float *dt_bias,
                    const float *A_log, const float *Dskip, void *y, void *stream);

/*
 * ssm_model_decode_step -- one token of every stream through a whole
 * Mamba-style language model ("mamba, live", section "what is actually
 * running": the streaming form, one token in, one token out):
 *   x = emb[token]
 *   for each block:  hn = LayerNorm(x);  [xin, z] = in_proj(hn)
 *                    u = SiLU(causal conv of xin over the carried history)
 *                    [dt, B, C] = x_proj(u);  dt_raw = dt_proj_w dt
 *                    one ssm_step of the block's state with u, dt_raw,
 *                    dt_bias = dt_proj_b, B, C and the gate z -> y
 *                    x += out_proj(y)
 *   logits = LayerNorm_out(x) emb^T          (head tied to the embedding)
 * The projections run on the matrix cores in float32.  Everything is float32.
 *   desc        host pointer, the model's shape
 *   emb         f32 [V, d_model]   embedding and head (required)
 *   norm_f_w, norm_f_b  f32 [d_model]  final LayerNorm, optional (1, 0)
 *   layers      HOST array of n_layers ssm_layer_weights (device pointers inside),
 *               read before the call returns
 *   tokens      int32 [S]           device; a token outside [0, V) makes that
 *                                   stream's logits and state NaN
 *   h           f32 [n_layers, S, d_inner, d_state]   state, in/out (zeros to start)
 *   conv_state  f32 [n_layers, S, W-1, d_inner]       conv history, in/out (oldest
 *                                   first; may be NULL when W = 1)
 *   logits      f32 [S, V]          output
 *   workspace   ssm_model_decode_workspace_size bytes (required)
 * Every pointer must be 16-byte aligned, except tokens (4-byte aligned);
 * outputs may not overlap the inputs, the workspace or each other.
 */
ssm_status ssm_model_decode_workspace_size(const ssm_model_desc *desc, size_t *bytes);
ssm_status ssm_model_decode_step(const ssm_model_desc *desc, const float *emb, const float *norm_f_w,
                                 const float *norm_f_b, const ssm_layer_weights *layers,
                                 const int32_t *tokens, float *h, float *conv_state, float *logits,
                                 void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SSM_AMD_SSM_H */
