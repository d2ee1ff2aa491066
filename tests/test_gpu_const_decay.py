"""GPU parity of the constant decay source against the float64 oracle.

The diagonal cell h <- a*h + b*u with the decay fixed per (channel, state),
a = exp(-exp(A_log)), and the write B_t*u_t ("the s6 cell", section "one cell,
two architectures": the fixed-decay side of the same primitive).  There is no
step size, so every call here passes dt_raw=None: the kernels must never read
it.  Same tolerances as the other parity tests (relative L-inf 1e-5 for
float32 I/O, 2e-2 for bf16 I/O with a float32 state)."""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from parity import BF16_TOL, FP32_TOL, dev, host, rel_linf, tol

pytestmark = pytest.mark.gpu

CONST = 2


@pytest.fixture(scope="module")
def ssm():
    import selective_state_space_ssm_amd as m
    m.lib()  # raises if the library is not built
    assert torch.cuda.is_available(), "no GPU visible"
    assert m.SSM_DECAY_CONST == CONST
    return m


def _rand(seed, Bn, L, D, N, W=4, bf16=False, slow=False):
    """Seeded normal inputs.  A_log ~ 0.5*normal gives decays exp(-exp(A_log))
    spread over (0.07, 0.9); slow=True puts A_log near -4 (decays near 0.98),
    so the state carries across tens of tokens."""
    r = np.random.default_rng(seed)
    f = lambda *s: r.standard_normal(s).astype(np.float32)
    a_log = (0.2 * f(D, N) - 4.0).astype(np.float32) if slow else (0.5 * f(D, N)).astype(np.float32)
    p = dict(x=f(Bn, L, D), B=f(Bn, L, N), C=f(Bn, L, N), z=f(Bn, L, D), dy=f(Bn, L, D), A_log=a_log,
             Dskip=f(D), h0=f(Bn, D, N), dhT=f(Bn, D, N), conv_w=f(D, W), conv_b=f(D),
             conv_state=f(Bn, max(W - 1, 0), D), dt_raw=f(Bn, L, D), dt_bias=f(D))
    if bf16:
        for k in ("x", "B", "C", "z", "dy"):
            p[k] = si.bf16_round(p[k])
    return p


def _fwd_gpu(ssm, p, dtype, conv=True, gate=True, h0=True, chunk=-1, with_dt=False):
    N = p["A_log"].shape[1]
    W = p["conv_w"].shape[1]
    Bn, L, D = p["x"].shape
    hT = torch.empty(Bn, D, N, device="cuda")
    st = conv and W > 1
    cso = torch.empty(Bn, W - 1, D, device="cuda") if st else None
    y = ssm.ssm_scan_fwd(dev(p["x"], dtype), dev(p["dt_raw"], dtype) if with_dt else None, dev(p["A_log"]),
                         dev(p["B"], dtype), dev(p["C"], dtype), dt_bias=dev(p["dt_bias"]) if with_dt else None,
                         Dskip=dev(p["Dskip"]), z=dev(p["z"], dtype) if gate else None,
                         conv_w=dev(p["conv_w"]) if conv else None, conv_b=dev(p["conv_b"]) if conv else None,
                         conv_state_in=dev(p["conv_state"]) if st else None, conv_state_out=cso,
                         h0=dev(p["h0"]) if h0 else None, hT=hT, disc=CONST, chunk_len=chunk)
    torch.cuda.synchronize()
    return y, hT, cso


def _fwd_oracle(p, conv=True, gate=True, h0=True):
    W = p["conv_w"].shape[1]
    if conv:
        u, cso = oracle.conv1d_causal(p["x"], p["conv_w"], p["conv_b"], p["conv_state"] if W > 1 else None)
    else:
        u, cso = p["x"], None
    y, hT = oracle.scan_fwd(u, None, p["A_log"], p["B"], p["C"], Dskip=p["Dskip"], z=p["z"] if gate else None,
                            h0=p["h0"] if h0 else None, disc=oracle.DECAY_CONST)
    return y, hT, cso


def _check_fwd(ssm, p, dtype=torch.float32, **kw):
    okw = {k: v for k, v in kw.items() if k in ("conv", "gate", "h0")}
    y, hT, cso = _fwd_gpu(ssm, p, dtype, **kw)
    yr, hr, csr = _fwd_oracle(p, **okw)
    assert rel_linf(y, yr) <= tol(dtype)
    assert rel_linf(hT, hr) <= tol(dtype)
    if cso is not None:
        np.testing.assert_array_equal(host(cso), csr)
    return y, hT


# --------------------------------------------------------------------------- forward

@pytest.mark.parametrize("Bn,L,D,N,W", [
    (2, 300, 40, 16, 4),    # ragged D and L
    (2, 130, 24, 1, 4),     # state width 1 (one scalar state per channel)
    (1, 50, 20, 3, 3),
    (2, 41, 48, 8, 2),
    (1, 37, 32, 33, 4),
    (1, 29, 16, 64, 8),
    (1, 64, 1, 16, 4),      # one channel
    (1, 1, 48, 16, 4),      # one token
])
@pytest.mark.parametrize("conv", [False, True])
def test_const_fwd_shapes(ssm, Bn, L, D, N, W, conv):
    _check_fwd(ssm, _rand(41, Bn, L, D, N, W), conv=conv)


@pytest.mark.parametrize("gate,h0", [(False, False), (True, False), (False, True)])
def test_const_fwd_optional_inputs(ssm, gate, h0):
    _check_fwd(ssm, _rand(42, 2, 70, 32, 16), gate=gate, h0=h0)


def test_const_fwd_empty_sequence(ssm):
    p = _rand(43, 2, 0, 32, 16)
    _, hT, cso = _fwd_gpu(ssm, p, torch.float32)
    np.testing.assert_array_equal(host(hT), p["h0"])
    np.testing.assert_array_equal(host(cso), p["conv_state"])


@pytest.mark.parametrize("chunk", [1, 37, 64, 100, 0])
@pytest.mark.parametrize("N", [1, 16])
def test_const_fwd_chunked(ssm, chunk, N):
    """The two-level time split with a constant decay: each chunk's decay
    product is a^(chunk length), composed by the carry walk."""
    _check_fwd(ssm, _rand(44, 2, 333, 40, N, slow=True), chunk=chunk)


def test_const_fwd_bf16(ssm):
    p = _rand(45, 2, 160, 48, 16, bf16=True, slow=True)
    for chunk in (-1, 40):
        y, _ = _check_fwd(ssm, p, torch.bfloat16, chunk=chunk)
        assert y.dtype == torch.bfloat16


def test_const_fwd_reads_no_step_size(ssm):
    """dt_raw and dt_bias, when passed, are ignored: bit-identical outputs."""
    p = _rand(46, 2, 200, 48, 16)
    a = _fwd_gpu(ssm, p, torch.float32, chunk=64)
    b = _fwd_gpu(ssm, p, torch.float32, chunk=64, with_dt=True)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_const_fwd_is_the_live_cell_at_unit_step(ssm):
    """One cell, two parameterisations, on the GPU: the live dt*B path with
    dt_raw chosen so that softplus gives 1.0 in float32 matches the constant
    path to rounding (the live path still evaluates its per-token exp2)."""
    p = _rand(47, 2, 150, 40, 16)
    y, hT, _ = _fwd_gpu(ssm, p, torch.float32)
    r = np.float32(np.log(np.expm1(1.0)))
    q = dict(p, dt_raw=np.full_like(p["x"], r), dt_bias=np.zeros_like(p["dt_bias"]))
    N = p["A_log"].shape[1]
    hl = torch.empty_like(hT)
    yl = ssm.ssm_scan_fwd(dev(q["x"]), dev(q["dt_raw"]), dev(q["A_log"]), dev(q["B"]), dev(q["C"]),
                          dt_bias=dev(q["dt_bias"]), Dskip=dev(q["Dskip"]), z=dev(q["z"]), conv_w=dev(q["conv_w"]),
                          conv_b=dev(q["conv_b"]), conv_state_in=dev(q["conv_state"]), h0=dev(q["h0"]), hT=hl,
                          chunk_len=-1)
    torch.cuda.synchronize()
    assert N == 16
    assert rel_linf(yl, y) <= FP32_TOL
    assert rel_linf(hl, hT) <= FP32_TOL


@pytest.mark.parametrize("N", [16, 1])
def test_const_fwd_workload(ssm, N):
    """The constant-decay forward at batch 8, L=2,048, D_inner=1536, fp32,
    fused 4-tap conv and SiLU(z) gate, state width 16 and 1, with the
    decays the input-driven workload has at its bias step (the benchmark's
    workload and launch configuration)."""
    p = si.mamba_block(8, 2048, 1536, N, 4, workload=si.WL_FWDBWD, const_decay=True)
    hT = torch.empty(8, 1536, N, device="cuda")
    y = ssm.ssm_scan_fwd(dev(p["x"]), None, dev(p["A_log"]), dev(p["B"]), dev(p["C"]), Dskip=dev(p["Dskip"]),
                         z=dev(p["z"]), conv_w=dev(p["conv_w"]), conv_b=dev(p["conv_b"]), hT=hT, disc=CONST)
    torch.cuda.synchronize()
    u, _ = oracle.conv1d_causal(p["x"], p["conv_w"], p["conv_b"])
    yr, hr = oracle.scan_fwd(u, None, p["A_log"], p["B"], p["C"], Dskip=p["Dskip"], z=p["z"],
                             disc=oracle.DECAY_CONST)
    assert rel_linf(y, yr) <= FP32_TOL
    assert rel_linf(hT, hr) <= FP32_TOL


# --------------------------------------------------------------------------- streaming step

def _step_gpu(ssm, p, steps, io=torch.float32, state_dtype=torch.float32, gate=True):
    h = dev(p["h0"], state_dtype)[None].contiguous()
    W = p["conv_w"].shape[1]
    cs = dev(p["conv_state"])[None].contiguous() if W > 1 else None
    ys = []
    for t in range(steps):
        ys.append(ssm.ssm_step(h, dev(p["x"][:, t], io)[None], None, dev(p["A_log"])[None],
                               dev(p["B"][:, t], io)[None], dev(p["C"][:, t], io)[None], conv_state=cs,
                               z=dev(p["z"][:, t], io)[None] if gate else None, conv_w=dev(p["conv_w"])[None],
                               conv_b=dev(p["conv_b"])[None], Dskip=dev(p["Dskip"])[None], disc=CONST)[0])
    torch.cuda.synchronize()
    return torch.stack(ys, 1), h[0], (cs[0] if cs is not None else None)


def _step_oracle(p, steps, state_bf16=False, gate=True):
    h = p["h0"].astype(np.float64).copy()
    if state_bf16:
        h = oracle.round_bf16(h)
    cs = p["conv_state"].astype(np.float64).copy()
    ys = []
    for t in range(steps):
        ys.append(oracle.step(h, cs, p["x"][:, t], None, p["B"][:, t], p["C"][:, t], p["A_log"],
                              z=p["z"][:, t] if gate else None, conv_w=p["conv_w"], conv_b=p["conv_b"],
                              Dskip=p["Dskip"], disc=oracle.DECAY_CONST, state_bf16=state_bf16))
    return np.stack(ys, 1), h, cs


@pytest.mark.parametrize("S,D,N,W", [(4, 40, 16, 4), (3, 8, 1, 3), (2, 16, 33, 2), (5, 24, 64, 1), (4, 128, 16, 4)])
def test_const_step_parity(ssm, S, D, N, W):
    p = _rand(48, S, 12, D, N, W)
    y, h, cs = _step_gpu(ssm, p, 12)
    yr, hr, csr = _step_oracle(p, 12)
    assert rel_linf(y, yr) <= FP32_TOL
    assert rel_linf(h, hr) <= FP32_TOL
    if cs is not None:
        np.testing.assert_array_equal(host(cs), csr)


def test_const_fwd_many_channel_groups(ssm):
    """A grid of over a thousand blocks with a partial last channel group in
    each batch row, two whole tiles and a ragged tail; then the streaming step
    reproduces a 768-block forward bit for bit."""
    p = _rand(52, 6, 130, 3000, 16, 4)
    _check_fwd(ssm, p)
    p = _rand(53, 4, 20, 3072, 16, 4)
    y, hT, cso = _fwd_gpu(ssm, p, torch.float32)
    ys, h, cs = _step_gpu(ssm, p, 20)
    assert torch.equal(ys, y)
    assert torch.equal(h, hT)
    assert torch.equal(cs, cso)


@pytest.mark.parametrize("N,D", [(16, 48), (1, 48), (33, 48), (16, 128)])
def test_const_step_loop_equals_forward(ssm, N, D):
    """Token-by-token decode with the constant source reproduces the
    sequence kernel bit for bit (D = 128 at N = 16 takes the common shape's
    step path)."""
    p = _rand(49, 3, 25, D, N, 4)
    y, hT, cso = _fwd_gpu(ssm, p, torch.float32)
    ys, h, cs = _step_gpu(ssm, p, 25)
    assert torch.equal(ys, y)
    assert torch.equal(h, hT)
    assert torch.equal(cs, cso)


@pytest.mark.parametrize("io,D", [(torch.float32, 32), (torch.bfloat16, 32), (torch.float32, 64)])
def test_const_step_bf16_state(ssm, io, D):
    steps = 40
    p = _rand(50, 4, steps, D, 16, 4, bf16=io == torch.bfloat16, slow=True)
    y, h, _ = _step_gpu(ssm, p, steps, io=io, state_dtype=torch.bfloat16)
    yr, hr, _ = _step_oracle(p, steps, state_bf16=True)
    assert h.dtype == torch.bfloat16
    assert rel_linf(y, yr) <= BF16_TOL
    assert rel_linf(h, hr) <= BF16_TOL


# --------------------------------------------------------------------------- backward

_GRADS = ["dx", "dA_log", "dB", "dC", "dD", "dz", "dh0"]


def _bwd_check(ssm, p, dtype=torch.float32, gate=True, h0=True, dhT=True, conv=False, chunk=0):
    W = p["conv_w"].shape[1]
    st = p["conv_state"] if (conv and W > 1) else None
    g = ssm.ssm_scan_bwd(dev(p["x"], dtype), None, dev(p["A_log"]), dev(p["B"], dtype), dev(p["C"], dtype),
                         dev(p["dy"], dtype), Dskip=dev(p["Dskip"]), z=dev(p["z"], dtype) if gate else None,
                         conv_w=dev(p["conv_w"]) if conv else None, conv_b=dev(p["conv_b"]) if conv else None,
                         conv_state_in=dev(st) if st is not None else None, h0=dev(p["h0"]) if h0 else None,
                         dhT=dev(p["dhT"]) if dhT else None, disc=CONST, chunk_len=chunk)
    torch.cuda.synchronize()
    assert "d_dt_raw" not in g and "d_dt_bias" not in g
    u = oracle.conv1d_causal(p["x"], p["conv_w"], p["conv_b"], st)[0] if conv else p["x"]
    r = oracle.scan_bwd(u, None, p["A_log"], p["B"], p["C"], p["dy"], Dskip=p["Dskip"],
                        z=p["z"] if gate else None, h0=p["h0"] if h0 else None, dhT=p["dhT"] if dhT else None,
                        disc=oracle.DECAY_CONST)
    r["dx"] = r["du"]
    keys = [k for k in _GRADS if gate or k != "dz"]
    if conv:
        rc = oracle.conv1d_causal_bwd(p["x"], p["conv_w"], r["du"], bias=p["conv_b"], state_in=st)
        r.update(dx=rc["dx"], dconv_w=rc["dw"], dconv_b=rc["db"], dconv_state=rc["dstate"])
        keys += ["dconv_w", "dconv_b"] + (["dconv_state"] if W > 1 else [])
    errs = {k: rel_linf(g[k], r[k]) for k in keys}
    bad = {k: v for k, v in errs.items() if not v <= tol(dtype)}
    assert not bad, (bad, errs)
    return g


@pytest.mark.parametrize("Bn,L,D,N", [(2, 100, 40, 16), (1, 37, 24, 1), (1, 50, 70, 33), (1, 9, 16, 64)])
@pytest.mark.parametrize("conv", [False, True])
def test_const_bwd_shapes(ssm, Bn, L, D, N, conv):
    _bwd_check(ssm, _rand(51, Bn, L, D, N), conv=conv)


@pytest.mark.parametrize("gate,h0,dhT", [(False, False, False), (True, False, True)])
def test_const_bwd_optional_inputs(ssm, gate, h0, dhT):
    _bwd_check(ssm, _rand(52, 2, 64, 32, 16), gate=gate, h0=h0, dhT=dhT)


@pytest.mark.parametrize("Bn,L,D,N,chunk,conv", [(1, 600, 40, 16, 128, False), (1, 500, 48, 16, 64, True),
                                                 (2, 300, 24, 1, 64, True)])
def test_const_bwd_chunked(ssm, Bn, L, D, N, chunk, conv):
    """The backward split in time: chunk start states from the forward chunk
    scan, end adjoints from the reverse walk with a^(chunk length)."""
    _bwd_check(ssm, _rand(53, Bn, L, D, N, slow=True), conv=conv, chunk=chunk)


def test_const_bwd_bf16(ssm):
    _bwd_check(ssm, _rand(54, 2, 80, 48, 16, bf16=True), torch.bfloat16, conv=True)


def test_const_bwd_workload(ssm):
    """Backward of the constant-decay workload: batch 8, L=2,048, D_inner=1536,
    N=16, fp32, through the fused conv prologue and the gate."""
    p = si.mamba_block(8, 2048, 1536, 16, 4, workload=si.WL_FWDBWD, with_dy=True, const_decay=True)
    q = dict(p, h0=np.zeros((8, 1536, 16), np.float32), dhT=np.zeros((8, 1536, 16), np.float32),
             conv_state=np.zeros((8, 3, 1536), np.float32))
    _bwd_check(ssm, q, h0=False, dhT=False, conv=True)
