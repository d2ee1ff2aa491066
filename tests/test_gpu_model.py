"""GPU parity of the whole-model streaming decode (ssm_model_decode_step)
against the float64 model oracle (oracle/mamba_model.py), on seeded
random-init weights.

Tolerance: relative L-inf 1e-5 on logits, state and conv history, the bar
of the float32 scan rows.  The model adds float32 matrix products of length
up to K = 1536; their rounding error grows like sqrt(K)*u = 2.4e-6 for
operands of random sign (the worst case, K*u = 9.2e-5 of sum |a_k b_k|,
needs every rounding to fall the same way), and the measured errors at the
Mamba-mini size stay below 1e-6."""
import numpy as np
import pytest
import torch

import seeded_inputs as si
from oracle import mamba_model as mm
from parity import rel_linf

pytestmark = pytest.mark.gpu

MODEL_TOL = 1e-5


@pytest.fixture(scope="module")
def ssm():
    import selective_state_space_ssm_amd as m
    m.lib()
    assert torch.cuda.is_available(), "no GPU visible"
    return m


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


class _Model:
    def __init__(self, ssm, cfg, seed, S):
        self.ssm, self.cfg, self.S = ssm, cfg, S
        self.p = si.model_params(cfg, seed=seed)
        self.emb = _dev(self.p["emb"])
        self.nfw, self.nfb = _dev(self.p["norm_f_w"]), _dev(self.p["norm_f_b"])
        self.layers = ssm.ModelLayers([{k: _dev(v) for k, v in lay.items()} for lay in self.p["layers"]])
        self.desc = ssm.model_desc(cfg, S)
        L, Di, N, W = cfg["n_layers"], cfg["d_inner"], cfg["d_state"], cfg["conv_width"]
        self.h = torch.zeros(L, S, Di, N, device="cuda")
        self.conv = torch.zeros(L, S, W - 1, Di, device="cuda") if W > 1 else None
        self.ho, self.co = mm.new_state(cfg, S)

    def step_gpu(self, tok, logits=None):
        t = torch.from_numpy(np.ascontiguousarray(tok, np.int32)).cuda()
        return self.ssm.ssm_model_decode_step(self.desc, self.emb, self.layers, t, self.h, self.conv,
                                              logits=logits, norm_f_w=self.nfw, norm_f_b=self.nfb)

    def step_oracle(self, tok):
        return mm.decode_step(self.p, tok, self.ho, self.co)


def _run(ssm, cfg, seed, S, T):
    m = _Model(ssm, cfg, seed, S)
    tok = si.model_tokens(cfg, S, T, seed=seed)
    errs = []
    for t in range(T):
        lg = m.step_gpu(tok[:, t])
        torch.cuda.synchronize()
        ref = m.step_oracle(tok[:, t])
        errs.append(rel_linf(lg, ref))
    eh = rel_linf(m.h, m.ho)
    ec = rel_linf(m.conv, m.co) if m.conv is not None else 0.0
    return errs, eh, ec


@pytest.mark.parametrize("cfg", [si.TINY_MODEL, si.RAGGED_MODEL], ids=["tiny", "ragged"])
@pytest.mark.parametrize("S", [1, 3, 17, 40])
def test_model_decode_small(ssm, cfg, S):
    """Small model shapes (odd widths, N 3 and 4, conv 3 and 4), several
    stream counts (ragged 16-row tiles), six tokens of decode."""
    errs, eh, ec = _run(ssm, cfg, 11, S, 6)
    assert max(errs) <= MODEL_TOL, errs
    assert eh <= MODEL_TOL and ec <= MODEL_TOL, (eh, ec)


EDGE_MODELS = [
    dict(vocab=7, d_model=5, n_layers=2, d_inner=9, d_state=64, dt_rank=1, conv_width=1),   # no conv history
    dict(vocab=300, d_model=130, n_layers=1, d_inner=200, d_state=17, dt_rank=33, conv_width=8),
]


@pytest.mark.parametrize("cfg", EDGE_MODELS, ids=["W1_N64_R1", "W8_N17_R33"])
@pytest.mark.parametrize("S", [1, 33])
def test_model_decode_edge_shapes(ssm, cfg, S):
    """Edge shapes: conv width 1 (no history), 64 states, rank-1 step size,
    widths that are not multiples of 4 (scalar loads), conv width 8."""
    errs, eh, ec = _run(ssm, cfg, 14, S, 5)
    assert max(errs) <= MODEL_TOL, errs
    assert eh <= MODEL_TOL and ec <= MODEL_TOL, (eh, ec)


def test_model_decode_mamba_mini_single_stream(ssm):
    """Mamba-mini (6 blocks, d 384, D_inner 1536, N 16, dt rank 24, conv 4,
    4096-token tied head), one stream, 16 tokens of decode."""
    errs, eh, ec = _run(ssm, si.MAMBA_MINI, 0, 1, 16)
    assert max(errs) <= MODEL_TOL, errs
    assert eh <= MODEL_TOL and ec <= MODEL_TOL, (eh, ec)


def test_model_decode_mamba_mini_256_streams(ssm):
    """Mamba-mini decoding 256 streams at once (the batched streaming shape),
    4 tokens, every stream compared."""
    errs, eh, ec = _run(ssm, si.MAMBA_MINI, 1, 256, 4)
    assert max(errs) <= MODEL_TOL, errs
    assert eh <= MODEL_TOL and ec <= MODEL_TOL, (eh, ec)


def test_model_decode_mamba_mini_96_streams(ssm):
    """Mamba-mini at 96 streams: in_proj (1152 output tiles of 16 x 16) and
    the head (1536) take the launch shape for 1024-2047 tiles, which neither
    the 1-stream nor the 256-stream decode reaches; 3 tokens, every stream
    compared."""
    errs, eh, ec = _run(ssm, si.MAMBA_MINI, 2, 96, 3)
    assert max(errs) <= MODEL_TOL, errs
    assert eh <= MODEL_TOL and ec <= MODEL_TOL, (eh, ec)


def test_model_bad_token_poisons_only_its_stream(ssm):
    """A token outside the vocabulary gives NaN logits and state for its own
    stream; the other streams decode normally."""
    cfg = si.TINY_MODEL
    m = _Model(ssm, cfg, 12, 4)
    tok = np.array([3, cfg["vocab"], 5, -1], np.int32)
    lg = m.step_gpu(tok).cpu().numpy()
    assert np.all(np.isnan(lg[1])) and np.all(np.isnan(lg[3]))
    assert np.all(np.isfinite(lg[[0, 2]]))
    ho, co = mm.new_state(cfg, 2)
    ref = mm.decode_step(m.p, tok[[0, 2]], ho, co)
    assert rel_linf(lg[[0, 2]], ref) <= MODEL_TOL
    h = m.h.cpu().numpy()
    assert np.all(np.isnan(h[:, 1])) and np.all(np.isfinite(h[:, [0, 2]]))


def test_model_decode_graph_replay(ssm):
    """Token steps captured in a HIP graph (as the benchmark runs them):
    every replay, with eager work and synchronisation in between, gives the
    eager steps' logits and state bit for bit."""
    cfg, S, T = si.RAGGED_MODEL, 5, 3
    tok = si.model_tokens(cfg, S, T, seed=13)
    toks = [torch.from_numpy(np.ascontiguousarray(tok[:, t])).cuda() for t in range(T)]
    a = _Model(ssm, cfg, 13, S)
    outs_e = [torch.empty(S, cfg["vocab"], device="cuda") for _ in range(T)]
    for t in range(T):
        ssm.ssm_model_decode_step(a.desc, a.emb, a.layers, toks[t], a.h, a.conv, logits=outs_e[t],
                                  norm_f_w=a.nfw, norm_f_b=a.nfb)
    torch.cuda.synchronize()
    b = _Model(ssm, cfg, 13, S)
    ws = torch.empty(ssm.ssm_model_decode_workspace_size(b.desc), dtype=torch.uint8, device="cuda")
    outs_g = [torch.empty(S, cfg["vocab"], device="cuda") for _ in range(T)]

    def run():
        for t in range(T):
            ssm.ssm_model_decode_step(b.desc, b.emb, b.layers, toks[t], b.h, b.conv, logits=outs_g[t],
                                      norm_f_w=b.nfw, norm_f_b=b.nfb, workspace=ws)

    run()                      # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for _ in range(3):
        b.h.zero_()
        b.conv.zero_()
        for o in outs_g:
            o.fill_(-1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t in range(T):
            assert torch.equal(outs_g[t], outs_e[t]), t
        assert torch.equal(b.h, a.h) and torch.equal(b.conv, a.conv)
