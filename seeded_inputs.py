"""Seeded synthetic inputs for the S6 selective scan (shared by tests and bench).

This module holds only the input recipe -- shapes, distributions and seeds --
and none of the scan's arithmetic.  Both the GPU path and the float64 oracle
are fed the arrays it returns (the oracle widens them exactly to float64).

Recipe (the pages' Mamba-mini shapes; the TinyStories activations and trained
weights they were measured on are not available, so seeded random draws of the
same shapes stand in for them):
  x (conv input) / u, B, C, z, dy   standard normal
  dt_raw                            0.1 * standard normal
  dt_bias[d]                        inverse softplus of delta0[d], with
                                    delta0 log-uniform in [1e-3, 1e-1]
  A_log[d, n]                       log(n + 1)   (perturbed variant: + 0.1*normal;
                                    constant-decay variant: + log(delta0[d]), so a
                                    decay fixed per channel, exp(-exp(A_log)), is
                                    the one the input-driven cell has at delta0)
  Dskip[d]                          1            (perturbed variant: normal)
  conv_w [D, W], conv_b [D]         standard normal
Every tensor has its own numpy Generator seeded with
[seed, workload_id, tensor_id], so adding a tensor never shifts another.
bf16 inputs are float32 draws rounded to the nearest bf16 (ties to even);
the returned float32 arrays then hold exactly the bf16 values.
"""
from __future__ import annotations

import numpy as np

# tensor ids inside one workload
_T = dict(x=1, dt_raw=2, B=3, C=4, z=5, dy=6, dt_bias=7, A_log=8, Dskip=9,
          conv_w=10, conv_b=11, h0=12, conv_state=13, dhT=14,
          emb=20, norm_w=21, norm_b=22, in_proj=23, x_proj=24, dt_proj_w=25, out_proj=26, tokens=27)

WL_TINY = 1
WL_BLOCK = 2
WL_STREAM = 3
WL_LONG = 4
WL_FWDBWD = 5
WL_MODEL = 6

# Model shapes: the pages' Mamba-mini (6 blocks at width 384, expand 4, N 16,
# dt rank 24, conv 4, 4k-token vocabulary with the head tied to the embedding)
# and two small ones for quick parity runs.
MAMBA_MINI = dict(vocab=4096, d_model=384, n_layers=6, d_inner=1536, d_state=16, dt_rank=24, conv_width=4)
TINY_MODEL = dict(vocab=64, d_model=16, n_layers=2, d_inner=32, d_state=4, dt_rank=4, conv_width=4)
RAGGED_MODEL = dict(vocab=50, d_model=24, n_layers=3, d_inner=40, d_state=3, dt_rank=5, conv_width=3)


def rng(seed, workload, tensor, *extra):
    return np.random.default_rng([int(seed), int(workload), _T[tensor]] + [int(e) for e in extra])


def bf16_round(a):
    """Round float32 values to the nearest bfloat16 (ties to even), returned
    as float32 holding exactly those bf16 values.  NaN stays NaN."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16) << 16
    out = rounded.astype(np.uint32).view(np.float32)
    return np.where(np.isnan(a), a, out).astype(np.float32)


def inverse_softplus(delta0):
    """r such that log(1 + e^r) = delta0 (input recipe for dt_bias)."""
    d = np.asarray(delta0, dtype=np.float64)
    return d + np.log(-np.expm1(-d))


def tiny_block(seed=0):
    """The recorded teaching block's size: batch 1, L=6, D_inner=8, N=3,
    causal conv width 3, fp32, seed 0.  x (used both as the scan input u and as
    the pre-conv input), dt_raw, B, C, z and the conv weights are standard
    normal; A_log = log(1..3) in every channel; Dskip = 1; dt_bias = 0."""
    Bn, L, D, N, W = 1, 6, 8, 3, 3
    wl = WL_TINY
    g = lambda t, shape: rng(seed, wl, t).standard_normal(shape).astype(np.float32)
    return dict(
        x=g("x", (Bn, L, D)), dt_raw=g("dt_raw", (Bn, L, D)), B=g("B", (Bn, L, N)),
        C=g("C", (Bn, L, N)), z=g("z", (Bn, L, D)), dy=g("dy", (Bn, L, D)),
        dt_bias=np.zeros(D, np.float32),
        A_log=np.tile(np.log(np.arange(1, N + 1, dtype=np.float64)), (D, 1)).astype(np.float32),
        Dskip=np.ones(D, np.float32),
        conv_w=g("conv_w", (D, W)), conv_b=g("conv_b", (D,)),
    )


def mamba_block(Bn, L, D, N, W=4, workload=WL_BLOCK, seed=0, bf16=False,
                perturbed=False, with_dy=False, with_state=False, const_decay=False):
    """Mamba-mini-shaped block inputs with the recipe in the module docstring.
    Returns float32 numpy arrays (bf16-representable when bf16=True).
    const_decay: A_log for a decay fixed per channel (see the docstring)."""
    def g(t, shape, scale=1.0):
        v = rng(seed, workload, t).standard_normal(shape, dtype=np.float32)
        if scale != 1.0:
            v = (v * np.float32(scale)).astype(np.float32)
        return bf16_round(v) if bf16 else v
    delta0 = np.exp(rng(seed, workload, "dt_bias").uniform(np.log(1e-3), np.log(1e-1), D))
    A_log = np.tile(np.log(np.arange(1, N + 1, dtype=np.float64)), (D, 1))
    Dskip = np.ones(D, np.float64)
    if perturbed:
        A_log = A_log + 0.1 * rng(seed, workload, "A_log").standard_normal((D, N))
        Dskip = rng(seed, workload, "Dskip").standard_normal(D)
    if const_decay:
        A_log = A_log + np.log(delta0)[:, None]
    out = dict(
        x=g("x", (Bn, L, D)), dt_raw=g("dt_raw", (Bn, L, D), 0.1),
        B=g("B", (Bn, L, N)), C=g("C", (Bn, L, N)), z=g("z", (Bn, L, D)),
        dt_bias=inverse_softplus(delta0).astype(np.float32),
        A_log=A_log.astype(np.float32), Dskip=Dskip.astype(np.float32),
        conv_w=rng(seed, workload, "conv_w").standard_normal((D, W)).astype(np.float32),
        conv_b=rng(seed, workload, "conv_b").standard_normal(D).astype(np.float32),
    )
    if with_dy:
        out["dy"] = g("dy", (Bn, L, D))
    if with_state:
        out["h0"] = rng(seed, workload, "h0").standard_normal((Bn, D, N)).astype(np.float32)
        out["conv_state"] = rng(seed, workload, "conv_state").standard_normal(
            (Bn, max(W - 1, 0), D)).astype(np.float32)
        out["dhT"] = rng(seed, workload, "dhT").standard_normal((Bn, D, N)).astype(np.float32)
    return out


def stream_params(nblocks, D, N, W=4, seed=0):
    """Per-block parameters of the batched streaming decode (one set per
    block): dt_bias, A_log, Dskip, conv_w, conv_b, stacked on a leading
    [nblocks] axis."""
    ps = [mamba_block(1, 1, D, N, W, workload=WL_STREAM * 100 + k, seed=seed) for k in range(nblocks)]
    keys = ("dt_bias", "A_log", "Dskip", "conv_w", "conv_b")
    return {k: np.stack([p[k] for p in ps]) for k in keys}


def stream_token_torch(block, step, S, D, N, device, seed=0):
    """Fresh per-step inputs of the streaming decode for one block, drawn on
    `device` with a torch Generator seeded by (seed, block, step):
    x, dt_raw (0.1 scale), z [S, D] and B, C [S, N], float32."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(((int(seed) * 1_000_003 + int(block)) * 1_000_033 + int(step)) & 0x7FFF_FFFF_FFFF)
    kw = dict(generator=gen, device=device, dtype=torch.float32)
    x = torch.randn(S, D, **kw)
    dt_raw = torch.randn(S, D, **kw) * 0.1
    z = torch.randn(S, D, **kw)
    Bm = torch.randn(S, N, **kw)
    Cm = torch.randn(S, N, **kw)
    return dict(x=x, dt_raw=dt_raw, z=z, B=Bm, C=Cm)


def model_params(cfg, seed=0):
    """Random-init weights of a whole Mamba-style language model of shape cfg
    (keys as in MAMBA_MINI), float32:
      emb [vocab, d_model]                    standard normal (also the tied head)
      per layer:
        norm_w, norm_b [d_model]              1 + 0.1*normal, 0.1*normal
        in_proj [2*d_inner, d_model]          uniform(+-1/sqrt(d_model))
        conv_w [d_inner, W], conv_b [d_inner] uniform(+-1/sqrt(W))
        x_proj [dt_rank + 2N, d_inner]        uniform(+-1/sqrt(d_inner))
        dt_proj_w [d_inner, dt_rank]          uniform(+-1/sqrt(dt_rank))
        dt_proj_b [d_inner]                   inverse softplus of delta0, delta0
                                              log-uniform in [1e-3, 1e-1]
        A_log [d_inner, N] = log(n + 1),  Dskip [d_inner] = 1
        out_proj [d_model, d_inner]           uniform(+-1/sqrt(d_inner))
      norm_f_w, norm_f_b [d_model]            as the layers' norms
    (the uniform ranges are PyTorch's default Linear / Conv1d init; the norms
    are perturbed from 1 and 0 so that their parameters matter)."""
    V, dm, nl = cfg["vocab"], cfg["d_model"], cfg["n_layers"]
    Di, N, R, W = cfg["d_inner"], cfg["d_state"], cfg["dt_rank"], cfg["conv_width"]
    wl = WL_MODEL

    def u(t, shape, bound, *ex):
        return rng(seed, wl, t, *ex).uniform(-bound, bound, shape).astype(np.float32)

    def n(t, shape, *ex):
        return rng(seed, wl, t, *ex).standard_normal(shape).astype(np.float32)

    layers = []
    for l in range(nl):
        delta0 = np.exp(rng(seed, wl, "dt_bias", l).uniform(np.log(1e-3), np.log(1e-1), Di))
        layers.append(dict(
            norm_w=(1.0 + 0.1 * n("norm_w", (dm,), l)).astype(np.float32),
            norm_b=(0.1 * n("norm_b", (dm,), l)).astype(np.float32),
            in_proj=u("in_proj", (2 * Di, dm), 1.0 / np.sqrt(dm), l),
            conv_w=u("conv_w", (Di, W), 1.0 / np.sqrt(W), l),
            conv_b=u("conv_b", (Di,), 1.0 / np.sqrt(W), l),
            x_proj=u("x_proj", (R + 2 * N, Di), 1.0 / np.sqrt(Di), l),
            dt_proj_w=u("dt_proj_w", (Di, R), 1.0 / np.sqrt(R), l),
            dt_proj_b=inverse_softplus(delta0).astype(np.float32),
            A_log=np.tile(np.log(np.arange(1, N + 1, dtype=np.float64)), (Di, 1)).astype(np.float32),
            Dskip=np.ones(Di, np.float32),
            out_proj=u("out_proj", (dm, Di), 1.0 / np.sqrt(Di), l),
        ))
    return dict(cfg=dict(cfg), emb=n("emb", (V, dm)), layers=layers,
                norm_f_w=(1.0 + 0.1 * n("norm_w", (dm,), nl)).astype(np.float32),
                norm_f_b=(0.1 * n("norm_b", (dm,), nl)).astype(np.float32))


def model_tokens(cfg, S, T, seed=0):
    """Token ids [S, T], uniform over the vocabulary (int32)."""
    return rng(seed, WL_MODEL, "tokens", S, T).integers(0, cfg["vocab"], (S, T)).astype(np.int32)
