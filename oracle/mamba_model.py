"""Float64 reference of a whole Mamba-style language model's streaming decode
(test infrastructure only: the tests, the smoke check and the benchmark's
CPU-baseline leg may use it; the GPU library never does).

Written from the streaming pseudocode of "mamba, live" (section "what is
actually running"): per token, x = emb[token]; for each block
    h       = LayerNorm(x)
    [xin,z] = in_proj(h)
    xc      = SiLU(causal depthwise conv(xin))      (the carried W-1 inputs)
    [dt,B,C]= x_proj(xc)
    dt      = softplus(dt_proj(dt))
    the selective-state update and readout, gated by SiLU(z)
    x      += out_proj(y)
and logits = head(LayerNorm_out(x)) with the head tied to the embedding.

Readings where that pseudocode is silent (every one is also the one that
gives the pages' 13.14M parameter count for Mamba-mini, "two recurrences",
section "why bother"): LayerNorm has a weight and a bias and eps = 1e-5
(PyTorch's defaults); in_proj, x_proj and out_proj have no bias; dt_proj has
one (it is the scan's dt_bias); the conv has a bias.

The matrix products are numpy float64 matmuls (a library primitive as a
step); the state update is the C oracle's orc_step with the conv disabled
(its input u is xc).  Weights are the float32 values given, widened exactly.
"""
from __future__ import annotations

import numpy as np

import oracle

LN_EPS = 1e-5


def param_count(params) -> int:
    """Number of parameters (the tied head adds none)."""
    n = params["emb"].size + params["norm_f_w"].size + params["norm_f_b"].size
    return int(n + sum(v.size for layer in params["layers"] for v in layer.values()))


def layer_norm(x, w, b, eps=LN_EPS):
    """(x - mean) / sqrt(var + eps) * w + b over the last axis, with the
    biased variance (PyTorch's LayerNorm)."""
    x = np.asarray(x, np.float64)
    mu = x.mean(-1, keepdims=True)
    var = ((x - mu) ** 2).mean(-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * np.asarray(w, np.float64) + np.asarray(b, np.float64)


def _silu(v):
    return v / (1.0 + np.exp(-v))


def new_state(cfg, S):
    """Zero state: h [n_layers, S, d_inner, N] and the conv history
    [n_layers, S, W-1, d_inner] (oldest input first), float64."""
    return (np.zeros((cfg["n_layers"], S, cfg["d_inner"], cfg["d_state"])),
            np.zeros((cfg["n_layers"], S, cfg["conv_width"] - 1, cfg["d_inner"])))


def _f64(a):
    return np.asarray(a, np.float64)


def decode_step(params, tokens, h, conv):
    """One token for each of S streams.  tokens [S] ints; h and conv (from
    new_state, float64) are updated in place.  Returns logits [S, vocab]."""
    cfg = params["cfg"]
    Di, N, R, W = cfg["d_inner"], cfg["d_state"], cfg["dt_rank"], cfg["conv_width"]
    emb = _f64(params["emb"])
    x = emb[np.asarray(tokens)]                              # [S, d_model]
    for l, p in enumerate(params["layers"]):
        hn = layer_norm(x, p["norm_w"], p["norm_b"])
        xz = hn @ _f64(p["in_proj"]).T                       # [S, 2 Di]
        xin, z = xz[:, :Di], xz[:, Di:]
        # causal conv over [history, xin], tap W-1 on the current input
        cw = _f64(p["conv_w"])
        acc = _f64(p["conv_b"])[None, :] + cw[None, :, W - 1] * xin
        for k in range(W - 1):
            acc = acc + cw[None, :, k] * conv[l][:, k, :]
        if W > 1:
            conv[l][:, :-1, :] = conv[l][:, 1:, :].copy()
            conv[l][:, -1, :] = xin
        xc = _silu(acc)
        xp = xc @ _f64(p["x_proj"]).T                        # [S, R + 2N]
        dt_low, Bm, Cm = xp[:, :R], xp[:, R:R + N], xp[:, R + N:]
        dt_raw = dt_low @ _f64(p["dt_proj_w"]).T             # [S, Di]
        hl = np.ascontiguousarray(h[l])
        y = oracle.step(hl, None, xc, dt_raw, Bm, Cm, p["A_log"], z=z, dt_bias=p["dt_proj_b"],
                        Dskip=p["Dskip"])
        h[l] = hl
        x = x + y @ _f64(p["out_proj"]).T
    return layer_norm(x, params["norm_f_w"], params["norm_f_b"]) @ emb.T


def forward_sequence(params, tokens):
    """The same model over whole sequences tokens [S, T] from a zero state,
    built from the sequence-level oracle calls (conv1d_causal over the
    sequence, scan_fwd over the sequence) instead of token steps.  Returns
    logits [S, T, vocab]."""
    cfg = params["cfg"]
    Di, N, R = cfg["d_inner"], cfg["d_state"], cfg["dt_rank"]
    emb = _f64(params["emb"])
    x = emb[np.asarray(tokens)]                              # [S, T, d_model]
    for p in params["layers"]:
        hn = layer_norm(x, p["norm_w"], p["norm_b"])
        xz = hn @ _f64(p["in_proj"]).T
        xin, z = xz[..., :Di], xz[..., Di:]
        xc, _ = oracle.conv1d_causal(xin, p["conv_w"], p["conv_b"])
        xp = xc @ _f64(p["x_proj"]).T
        dt_raw = xp[..., :R] @ _f64(p["dt_proj_w"]).T
        y, _ = oracle.scan_fwd(xc, dt_raw, p["A_log"], xp[..., R:R + N], xp[..., R + N:],
                               dt_bias=p["dt_proj_b"], Dskip=p["Dskip"], z=z)
        x = x + y @ _f64(p["out_proj"]).T
    return layer_norm(x, params["norm_f_w"], params["norm_f_b"]) @ emb.T
