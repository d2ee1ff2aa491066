"""Pins of the whole-model decode oracle (oracle/mamba_model.py) to facts
other than itself: the pages' parameter count, a library LayerNorm, the
sequence-level composition of the same model, causality, and closed forms
that fix the order of the projections' splits ([xin, z] from in_proj,
[dt, B, C] from x_proj) by zeroing one part at a time."""
import numpy as np
import pytest
import torch

import seeded_inputs as si
from oracle import mamba_model as mm


def test_mamba_mini_parameter_count():
    """The Mamba-mini shape with these readings (LayerNorm weight and bias,
    biases on the conv and on dt_proj only, head tied to the embedding) has
    13,144,320 parameters: the pages' 13.14M ("two recurrences", section
    "why bother")."""
    p = si.model_params(si.MAMBA_MINI)
    n = mm.param_count(p)
    assert n == 13_144_320
    assert round(n / 1e6, 2) == 13.14


def test_layer_norm_against_torch():
    r = np.random.default_rng(1)
    x, w, b = r.standard_normal((5, 384)) * 3 + 1, r.standard_normal(384), r.standard_normal(384)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (384,), torch.from_numpy(w), torch.from_numpy(b),
                                         eps=1e-5).numpy()
    np.testing.assert_allclose(mm.layer_norm(x, w, b), ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("cfg", [si.TINY_MODEL, si.RAGGED_MODEL])
def test_streaming_decode_equals_sequence_forward(oracle_lib, cfg):
    """Token-by-token decode with the carried state (h and the conv history
    of every block) gives the logits of the whole-sequence composition built
    from the sequence calls (conv over the sequence, scan over the
    sequence)."""
    p = si.model_params(cfg, seed=3)
    S, T = 3, 9
    tok = si.model_tokens(cfg, S, T, seed=3)
    ref = mm.forward_sequence(p, tok)
    h, conv = mm.new_state(cfg, S)
    for t in range(T):
        lg = mm.decode_step(p, tok[:, t], h, conv)
        np.testing.assert_allclose(lg, ref[:, t], rtol=1e-11, atol=1e-11)


def test_decode_causality(oracle_lib):
    """A different token at step t0 leaves the logits of earlier steps
    unchanged and changes those from t0 on."""
    cfg = si.TINY_MODEL
    p = si.model_params(cfg, seed=4)
    tok = si.model_tokens(cfg, 2, 8, seed=4)
    tok2 = tok.copy()
    tok2[:, 5] = (tok2[:, 5] + 1) % cfg["vocab"]
    a, b = mm.forward_sequence(p, tok), mm.forward_sequence(p, tok2)
    np.testing.assert_array_equal(a[:, :5], b[:, :5])
    assert np.all(np.any(a[:, 5:] != b[:, 5:], axis=-1))


def test_zero_output_projections_leave_the_embedding(oracle_lib):
    """With every out_proj zero the blocks add nothing to the residual
    stream: logits = LayerNorm_out(emb[token]) @ emb^T, whatever the state."""
    cfg = si.RAGGED_MODEL
    p = si.model_params(cfg, seed=5)
    for layer in p["layers"]:
        layer["out_proj"] = np.zeros_like(layer["out_proj"])
    tok = si.model_tokens(cfg, 4, 3, seed=5)
    h, conv = mm.new_state(cfg, 4)
    e = p["emb"].astype(np.float64)
    for t in range(3):
        lg = mm.decode_step(p, tok[:, t], h, conv)
        x = e[tok[:, t]]
        mu = x.mean(-1, keepdims=True)
        sd = np.sqrt(((x - mu) ** 2).mean(-1, keepdims=True) + 1e-5)
        ref = ((x - mu) / sd * p["norm_f_w"] + p["norm_f_b"]) @ e.T
        np.testing.assert_allclose(lg, ref, rtol=1e-12, atol=1e-10)
    assert np.any(h != 0) and np.any(conv != 0)   # the blocks still ran


def test_state_shapes_of_mamba_mini():
    """The decode state of Mamba-mini: 6 blocks x 1536 channels x 16 states =
    147,456 numbers ("mamba, live", section "what is actually running"),
    plus a 3-input conv history per channel."""
    h, conv = mm.new_state(si.MAMBA_MINI, 1)
    assert h.size == 147_456
    assert conv.shape == (6, 1, 3, 1536)


def _zero_write_rows(p, cfg):
    R, N = cfg["dt_rank"], cfg["d_state"]
    for layer in p["layers"]:
        layer["x_proj"] = layer["x_proj"].copy()
        layer["x_proj"][R:R + N] = 0.0        # the rows that produce B


@pytest.mark.parametrize("cfg", [si.TINY_MODEL, si.RAGGED_MODEL])
def test_zero_write_rows_keep_the_state_zero(oracle_lib, cfg):
    """x_proj's output is split as [dt (dt_rank), B (N), C (N)]: with the B rows
    zero nothing is written, so a zero state stays exactly zero."""
    p = si.model_params(cfg, seed=6)
    _zero_write_rows(p, cfg)
    tok = si.model_tokens(cfg, 3, 4, seed=6)
    h, conv = mm.new_state(cfg, 3)
    for t in range(4):
        mm.decode_step(p, tok[:, t], h, conv)
    assert not np.any(h) and np.any(conv)


def test_constant_step_decays_the_state_by_the_bias_step(oracle_lib):
    """dt_proj's weights zero and no writes: every block's step size is
    softplus(dt_proj bias) whatever the input, so one token multiplies each
    block's state by exp(-softplus(b_d) * exp(A_log[d, n])) exactly
    (softplus by np.logaddexp)."""
    cfg = si.RAGGED_MODEL
    p = si.model_params(cfg, seed=7)
    _zero_write_rows(p, cfg)
    for layer in p["layers"]:
        layer["dt_proj_w"] = np.zeros_like(layer["dt_proj_w"])
    S = 2
    h, conv = mm.new_state(cfg, S)
    r = np.random.default_rng(7)
    h[...] = r.standard_normal(h.shape)
    h0 = h.copy()
    mm.decode_step(p, si.model_tokens(cfg, S, 1, seed=7)[:, 0], h, conv)
    for l, layer in enumerate(p["layers"]):
        dt = np.logaddexp(0.0, layer["dt_proj_b"].astype(np.float64))
        a = np.exp(-dt[:, None] * np.exp(layer["A_log"].astype(np.float64)))
        np.testing.assert_allclose(h[l], a[None] * h0[l], rtol=1e-13, atol=0)


def _ln_head(p, x):
    """LayerNorm_out(x) @ emb^T written out (mean, biased variance, eps 1e-5)."""
    e = p["emb"].astype(np.float64)
    mu = x.mean(-1, keepdims=True)
    sd = np.sqrt(((x - mu) ** 2).mean(-1, keepdims=True) + 1e-5)
    return ((x - mu) / sd * p["norm_f_w"] + p["norm_f_b"]) @ e.T


@pytest.mark.parametrize("cfg", [si.TINY_MODEL, si.RAGGED_MODEL])
def test_zero_gate_rows_switch_every_block_off(oracle_lib, cfg):
    """in_proj's output is split as [xin (d_inner), z (d_inner)] ("mamba, live",
    section "what is actually running"): with the z rows zero the gate
    SiLU(0) = 0 closes every block, so the logits are
    LayerNorm_out(emb[token]) @ emb^T while the state still moves."""
    Di = cfg["d_inner"]
    p = si.model_params(cfg, seed=8)
    for layer in p["layers"]:
        layer["in_proj"] = layer["in_proj"].copy()
        layer["in_proj"][Di:] = 0.0
    S, T = 3, 4
    tok = si.model_tokens(cfg, S, T, seed=8)
    h, conv = mm.new_state(cfg, S)
    for t in range(T):
        lg = mm.decode_step(p, tok[:, t], h, conv)
        ref = _ln_head(p, p["emb"].astype(np.float64)[tok[:, t]])
        np.testing.assert_allclose(lg, ref, rtol=1e-12, atol=1e-10)
    assert np.any(h != 0) and np.any(conv != 0)
    lg_seq = mm.forward_sequence(p, tok)
    for t in range(T):
        np.testing.assert_allclose(lg_seq[:, t], _ln_head(p, p["emb"].astype(np.float64)[tok[:, t]]),
                                   rtol=1e-12, atol=1e-10)


@pytest.mark.parametrize("cfg", [si.TINY_MODEL, si.RAGGED_MODEL])
def test_zero_readout_rows_leave_only_the_skip_path(oracle_lib, cfg):
    """x_proj's output is split as [dt (dt_rank), B (N), C (N)]: with the C rows
    zero nothing is read from the state, so every block adds
    out_proj(Dskip * u * SiLU(z)) with u = SiLU(conv(xin)).  The model is
    recomputed here without the scan, the conv by torch's conv1d (left
    padding of W - 1 zeros, float64).  TINY_MODEL has dt_rank == d_state, so
    a dt / C mix-up cannot hide behind a shape error."""
    Di, R, N, W = cfg["d_inner"], cfg["dt_rank"], cfg["d_state"], cfg["conv_width"]
    p = si.model_params(cfg, seed=9)
    r = np.random.default_rng(9)
    for layer in p["layers"]:
        layer["x_proj"] = layer["x_proj"].copy()
        layer["x_proj"][R + N:] = 0.0
        layer["Dskip"] = r.standard_normal(Di).astype(np.float32)
    S, T = 2, 6
    tok = si.model_tokens(cfg, S, T, seed=9)
    x = p["emb"].astype(np.float64)[tok]                              # [S, T, dm]
    for layer in p["layers"]:
        hn = torch.nn.functional.layer_norm(torch.from_numpy(x), (x.shape[-1],),
                                            torch.from_numpy(layer["norm_w"].astype(np.float64)),
                                            torch.from_numpy(layer["norm_b"].astype(np.float64)), eps=1e-5)
        wi = torch.from_numpy(layer["in_proj"].astype(np.float64))
        xin, z = hn @ wi[:Di].T, hn @ wi[Di:].T                       # [S, T, Di]
        xc = torch.nn.functional.conv1d(xin.transpose(1, 2),
                                        torch.from_numpy(layer["conv_w"].astype(np.float64))[:, None, :],
                                        torch.from_numpy(layer["conv_b"].astype(np.float64)),
                                        padding=W - 1, groups=Di)[..., :T].transpose(1, 2)
        u = torch.nn.functional.silu(xc)
        y = torch.from_numpy(layer["Dskip"].astype(np.float64)) * u * torch.nn.functional.silu(z)
        x = x + (y @ torch.from_numpy(layer["out_proj"].astype(np.float64)).T).numpy()
    ref = _ln_head(p, x)
    h, conv = mm.new_state(cfg, S)
    for t in range(T):
        lg = mm.decode_step(p, tok[:, t], h, conv)
        np.testing.assert_allclose(lg, ref[:, t], rtol=1e-11, atol=1e-10)
    assert np.any(h != 0)
    np.testing.assert_allclose(mm.forward_sequence(p, tok), ref, rtol=1e-11, atol=1e-10)
