"""GPU parity: every HIP path against the float64 oracle on the same seeded
inputs, element by element, at the tolerances of the workloads (relative
L-inf 1e-5 for float32 I/O, 2e-2 for bf16 I/O with float32 state)."""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from parity import BF16_TOL, FP32_TOL, dev, host, rel_linf, tol

pytestmark = pytest.mark.gpu

DB, ZOH = 0, 1


@pytest.fixture(scope="module")
def ssm():
    import selective_state_space_ssm_amd as m
    m.lib()  # raises if the library is not built
    assert torch.cuda.is_available(), "no GPU visible"
    return m


def _rand(seed, Bn, L, D, N, W=4, bf16=False, scale_dt=1.0, slow=False):
    """Seeded normal inputs.  slow=True draws A_log around -4 (|A| ~ 0.02), so
    the state and the adjoint carry across hundreds of tokens."""
    r = np.random.default_rng(seed)
    f = lambda *s: r.standard_normal(s).astype(np.float32)
    a_log = (0.2 * f(D, N) - 4.0).astype(np.float32) if slow else 0.5 * f(D, N)
    p = dict(x=f(Bn, L, D), dt_raw=(f(Bn, L, D) * np.float32(scale_dt)), B=f(Bn, L, N), C=f(Bn, L, N),
             z=f(Bn, L, D), dy=f(Bn, L, D), dt_bias=(0.3 * f(D)), A_log=a_log,
             Dskip=f(D), h0=f(Bn, D, N), dhT=f(Bn, D, N), conv_w=f(D, W), conv_b=f(D),
             conv_state=f(Bn, max(W - 1, 0), D))
    if bf16:
        for k in ("x", "dt_raw", "B", "C", "z", "dy"):
            p[k] = si.bf16_round(p[k])
    return p


def _fwd_gpu(ssm, p, dtype, disc=DB, conv=True, gate=True, h0=True, chunk=-1, state=True):
    N = p["A_log"].shape[1]
    W = p["conv_w"].shape[1]
    Bn, L, D = p["x"].shape
    hT = torch.empty(Bn, D, N, device="cuda") if state else None
    cso = torch.empty(Bn, W - 1, D, device="cuda") if (conv and state and W > 1) else None
    y = ssm.ssm_scan_fwd(dev(p["x"], dtype), dev(p["dt_raw"], dtype), dev(p["A_log"]), dev(p["B"], dtype),
                         dev(p["C"], dtype), dt_bias=dev(p["dt_bias"]), Dskip=dev(p["Dskip"]),
                         z=dev(p["z"], dtype) if gate else None,
                         conv_w=dev(p["conv_w"]) if conv else None, conv_b=dev(p["conv_b"]) if conv else None,
                         conv_state_in=dev(p["conv_state"]) if (conv and state and W > 1) else None,
                         conv_state_out=cso, h0=dev(p["h0"]) if h0 else None, hT=hT, disc=disc, chunk_len=chunk)
    torch.cuda.synchronize()
    return y, hT, cso


def _fwd_oracle(p, disc=DB, conv=True, gate=True, h0=True, state=True):
    W = p["conv_w"].shape[1]
    if conv:
        u, cso = oracle.conv1d_causal(p["x"], p["conv_w"], p["conv_b"],
                                      p["conv_state"] if (state and W > 1) else None)
    else:
        u, cso = p["x"], None
    y, hT = oracle.scan_fwd(u, p["dt_raw"], p["A_log"], p["B"], p["C"], dt_bias=p["dt_bias"],
                            Dskip=p["Dskip"], z=p["z"] if gate else None, h0=p["h0"] if h0 else None, disc=disc)
    return y, hT, cso, u


# --------------------------------------------------------------------------- conv

@pytest.mark.parametrize("Bn,L,D,W,state,silu,bf16", [
    (1, 6, 8, 3, False, True, False),        # tiny teaching block
    (3, 77, 100, 4, True, True, False),      # ragged: L, D not multiples of the tiles
    (2, 40, 33, 1, False, False, False),
    (2, 5, 17, 8, True, True, False),        # L < W - 1
    (2, 130, 64, 4, True, True, True),       # bf16 I/O
    (1, 0, 16, 4, True, True, False),        # empty sequence: history passes through
])
def test_conv1d_parity(ssm, Bn, L, D, W, state, silu, bf16):
    p = _rand(11, Bn, L, D, 4, W, bf16=bf16)
    dtype = torch.bfloat16 if bf16 else torch.float32
    so = torch.empty(Bn, W - 1, D, device="cuda") if (state and W > 1) else None
    y = ssm.conv1d_causal(dev(p["x"], dtype), dev(p["conv_w"]), dev(p["conv_b"]),
                          state_in=dev(p["conv_state"]) if (state and W > 1) else None, state_out=so, silu=silu)
    torch.cuda.synchronize()
    ref, rso = oracle.conv1d_causal(p["x"], p["conv_w"], p["conv_b"],
                                    p["conv_state"] if (state and W > 1) else None, silu=silu)
    if L > 0:
        assert rel_linf(y, ref) <= tol(dtype)
    if so is not None:
        np.testing.assert_array_equal(host(so), rso)


# --------------------------------------------------------------------------- forward

@pytest.mark.parametrize("disc", [DB, ZOH])
@pytest.mark.parametrize("conv", [False, True])
def test_fwd_tiny_block(ssm, disc, conv):
    """The teaching block's size (B=1, L=6, D=8, N=3, W=3), seed 0, both
    discretisations, with and without the fused conv."""
    t = si.tiny_block()
    p = dict(t, h0=np.zeros((1, 8, 3), np.float32), conv_state=np.zeros((1, 2, 8), np.float32))
    y, hT, cso = _fwd_gpu(ssm, p, torch.float32, disc=disc, conv=conv)
    yr, hr, csr, _ = _fwd_oracle(p, disc=disc, conv=conv)
    assert rel_linf(y, yr) <= FP32_TOL
    assert rel_linf(hT, hr) <= FP32_TOL
    if conv:
        np.testing.assert_array_equal(host(cso), csr)


@pytest.mark.parametrize("Bn,L,D,N,W", [
    (2, 300, 40, 16, 4),    # D not a multiple of 16, L not a multiple of the unroll
    (1, 33, 24, 1, 4),
    (2, 50, 20, 3, 3),
    (1, 64, 16, 5, 2),
    (2, 41, 48, 8, 4),
    (1, 40, 16, 17, 4),
    (1, 37, 32, 33, 4),
    (1, 29, 16, 64, 8),
    (1, 64, 1, 16, 4),      # one channel
    (1, 1, 48, 16, 4),      # one token
])
@pytest.mark.parametrize("disc", [DB, ZOH])
def test_fwd_shapes(ssm, Bn, L, D, N, W, disc):
    p = _rand(5, Bn, L, D, N, W)
    y, hT, cso = _fwd_gpu(ssm, p, torch.float32, disc=disc)
    yr, hr, csr, _ = _fwd_oracle(p, disc=disc)
    assert rel_linf(y, yr) <= FP32_TOL
    assert rel_linf(hT, hr) <= FP32_TOL
    np.testing.assert_array_equal(host(cso), csr)


@pytest.mark.parametrize("gate,h0,conv", [(False, False, False), (True, False, False), (False, True, True)])
def test_fwd_optional_inputs(ssm, gate, h0, conv):
    p = _rand(6, 2, 70, 32, 16)
    y, hT, _ = _fwd_gpu(ssm, p, torch.float32, gate=gate, h0=h0, conv=conv)
    yr, hr, _, _ = _fwd_oracle(p, gate=gate, h0=h0, conv=conv)
    assert rel_linf(y, yr) <= FP32_TOL
    assert rel_linf(hT, hr) <= FP32_TOL


def test_fwd_empty_sequence(ssm):
    """L = 0: no output tokens, hT = h0 and the conv history passes through."""
    p = _rand(7, 2, 0, 32, 16)
    _, hT, cso = _fwd_gpu(ssm, p, torch.float32)
    np.testing.assert_array_equal(host(hT), p["h0"])
    np.testing.assert_array_equal(host(cso), p["conv_state"])


@pytest.mark.parametrize("chunk", [1, 7, 37, 64, 100, 0])
@pytest.mark.parametrize("conv", [False, True])
def test_fwd_chunked_matches_oracle(ssm, chunk, conv):
    """Two-level time split (local chunk scans, carry walk, re-scan) against
    the sequential oracle, for chunk lengths that leave ragged tails."""
    p = _rand(8, 2, 333, 40, 16)
    y, hT, cso = _fwd_gpu(ssm, p, torch.float32, conv=conv, chunk=chunk)
    yr, hr, csr, _ = _fwd_oracle(p, conv=conv)
    assert rel_linf(y, yr) <= FP32_TOL
    assert rel_linf(hT, hr) <= FP32_TOL
    if conv:
        np.testing.assert_array_equal(host(cso), csr)


@pytest.mark.parametrize("L,chunk", [(333, 1), (333, 7), (333, 32), (333, 37), (333, 100), (1500, 0),
                                     (64, 32), (40, 64)])
@pytest.mark.parametrize("disc", [DB, ZOH])
def test_fwd_one_wavefront_chunks(ssm, L, chunk, disc):
    """The time split of N = 16 scans without a fused conv runs one-wavefront
    chunk scans (four states per lane): chunk lengths that leave ragged
    32-token tiles and a partial last chunk, and the library's own choice
    (L 1500 -> chunks of 320), against the sequential oracle."""
    p = _rand(41, 2, L, 48, 16)
    y, hT, _ = _fwd_gpu(ssm, p, torch.float32, conv=False, chunk=chunk, disc=disc)
    yr, hr, _, _ = _fwd_oracle(p, conv=False, disc=disc)
    assert rel_linf(y, yr) <= FP32_TOL
    assert rel_linf(hT, hr) <= FP32_TOL


@pytest.mark.parametrize("gate,h0,bf16", [(False, False, False), (True, False, True), (False, True, True)])
def test_fwd_one_wavefront_chunks_options(ssm, gate, h0, bf16):
    """One-wavefront chunks without the gate, from a zero or given state, in
    bf16 I/O; Dskip zero in the first case."""
    p = _rand(42, 3, 777, 32, 16, bf16=bf16)
    if not gate:
        p["Dskip"] = np.zeros_like(p["Dskip"])
    dt = torch.bfloat16 if bf16 else torch.float32
    y, hT, _ = _fwd_gpu(ssm, p, dt, conv=False, gate=gate, h0=h0, chunk=96)
    yr, hr, _, _ = _fwd_oracle(p, conv=False, gate=gate, h0=h0)
    assert rel_linf(y, yr) <= tol(dt)
    assert rel_linf(hT, hr) <= tol(dt)


def test_fwd_one_wavefront_chunks_match_unsplit(ssm):
    """Split (one-wavefront chunks) and unsplit forwards agree to rounding."""
    p = _rand(43, 1, 2048, 64, 16, slow=True)
    a = _fwd_gpu(ssm, p, torch.float32, conv=False, chunk=-1)
    b = _fwd_gpu(ssm, p, torch.float32, conv=False, chunk=256)
    c = _fwd_gpu(ssm, p, torch.float32, conv=False, chunk=256)
    assert rel_linf(b[0], a[0]) <= FP32_TOL and rel_linf(b[1], a[1]) <= FP32_TOL
    assert torch.equal(b[0], c[0]) and torch.equal(b[1], c[1])


def test_fwd_split_sequence_equals_whole(ssm):
    """fwd(x[:k]) then fwd(x[k:]) from the carried state and conv history
    gives the single call's outputs bit for bit."""
    p = _rand(9, 2, 90, 48, 16)
    y, hT, cso = _fwd_gpu(ssm, p, torch.float32)
    k = 37
    a = {kk: (v[:, :k] if (v.ndim == 3 and v.shape[1] == 90) else v) for kk, v in p.items()}
    b = {kk: (v[:, k:] if (v.ndim == 3 and v.shape[1] == 90) else v) for kk, v in p.items()}
    y1, h1, c1 = _fwd_gpu(ssm, a, torch.float32)
    b["h0"], b["conv_state"] = host(h1).astype(np.float32), host(c1).astype(np.float32)
    y2, h2, c2 = _fwd_gpu(ssm, b, torch.float32)
    assert torch.equal(torch.cat([y1, y2], 1), y)
    assert torch.equal(h2, hT) and torch.equal(c2, cso)


def test_fwd_in_place_state(ssm):
    """hT may be h0 and conv_state_out may be conv_state_in (in-place)."""
    p = _rand(10, 2, 200, 32, 16)
    yr, hr, csr, _ = _fwd_oracle(p)
    for chunk in (-1, 50):
        h = dev(p["h0"])
        cs = dev(p["conv_state"])
        y = ssm.ssm_scan_fwd(dev(p["x"]), dev(p["dt_raw"]), dev(p["A_log"]), dev(p["B"]), dev(p["C"]),
                             dt_bias=dev(p["dt_bias"]), Dskip=dev(p["Dskip"]), z=dev(p["z"]),
                             conv_w=dev(p["conv_w"]), conv_b=dev(p["conv_b"]), conv_state_in=cs,
                             conv_state_out=cs, h0=h, hT=h, chunk_len=chunk)
        torch.cuda.synchronize()
        assert rel_linf(y, yr) <= FP32_TOL
        assert rel_linf(h, hr) <= FP32_TOL
        np.testing.assert_array_equal(host(cs), csr)


def test_fwd_bf16_io(ssm):
    p = _rand(12, 2, 160, 48, 16, bf16=True)
    for chunk in (-1, 40):
        y, hT, _ = _fwd_gpu(ssm, p, torch.bfloat16, chunk=chunk)
        assert y.dtype == torch.bfloat16
        yr, hr, _, _ = _fwd_oracle(p)
        assert rel_linf(y, yr) <= BF16_TOL
        assert rel_linf(hT, hr) <= BF16_TOL


def test_fwd_deterministic(ssm):
    p = _rand(13, 2, 300, 64, 16)
    a = _fwd_gpu(ssm, p, torch.float32, chunk=64)
    b = _fwd_gpu(ssm, p, torch.float32, chunk=64)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("disc,bf16,conv,W", [
    (DB, False, True, 4),
    (ZOH, False, True, 3),
    (DB, True, True, 4),
    (DB, False, False, 4),
])
def test_fwd_many_channel_groups(ssm, disc, bf16, conv, W):
    """A grid of over a thousand blocks: D = 3000 channels (187 whole groups of
    16 and a last group of 8 in each batch row), L = 130 is two whole tiles
    and a ragged tail."""
    p = _rand(70 + disc, 6, 130, 3000, 16, W=W, bf16=bf16)
    dt = torch.bfloat16 if bf16 else torch.float32
    y, hT, cso = _fwd_gpu(ssm, p, dt, disc=disc, conv=conv)
    yr, hr, csr, _ = _fwd_oracle(p, disc=disc, conv=conv)
    assert rel_linf(y, yr) <= tol(dt)
    assert rel_linf(hT, hr) <= tol(dt)
    if conv:
        np.testing.assert_array_equal(host(cso), csr)


def test_step_loop_equals_forward_many_groups(ssm):
    """The streaming step reproduces the forward bit for bit on a grid of 768
    blocks (4 batch rows x 192 channel groups)."""
    p = _rand(75, 4, 20, 3072, 16)
    y, hT, cso = _fwd_gpu(ssm, p, torch.float32)
    h = dev(p["h0"])[None].contiguous()
    cs = dev(p["conv_state"])[None].contiguous()
    ys = []
    for t in range(20):
        ys.append(ssm.ssm_step(h, dev(p["x"][:, t])[None], dev(p["dt_raw"][:, t])[None], dev(p["A_log"])[None],
                               dev(p["B"][:, t])[None], dev(p["C"][:, t])[None], conv_state=cs,
                               z=dev(p["z"][:, t])[None], conv_w=dev(p["conv_w"])[None],
                               conv_b=dev(p["conv_b"])[None], dt_bias=dev(p["dt_bias"])[None],
                               Dskip=dev(p["Dskip"])[None])[0])
    torch.cuda.synchronize()
    assert torch.equal(torch.stack(ys, 1), y)
    assert torch.equal(h[0], hT)
    assert torch.equal(cs[0], cso)


# ------------------------------------------------------------ workloads at full size

def _mamba_fwd(ssm, p, dtype, chunk=0):
    Bn, L, D = p["x"].shape
    N = p["A_log"].shape[1]
    hT = torch.empty(Bn, D, N, device="cuda")
    y = ssm.ssm_scan_fwd(dev(p["x"], dtype), dev(p["dt_raw"], dtype), dev(p["A_log"]), dev(p["B"], dtype),
                         dev(p["C"], dtype), dt_bias=dev(p["dt_bias"]), Dskip=dev(p["Dskip"]),
                         z=dev(p["z"], dtype), conv_w=dev(p["conv_w"]), conv_b=dev(p["conv_b"]), hT=hT,
                         chunk_len=chunk)
    torch.cuda.synchronize()
    return y, hT


@pytest.mark.parametrize("perturbed", [False, True])
def test_mamba_mini_block_L256(ssm, perturbed):
    """Mamba-mini block forward: batch 8, L=256, D_inner=1536, N=16, fp32,
    4-tap causal conv fused before the scan, SiLU(z) gate; the perturbed run
    uses A_log = log(n+1) + 0.1*normal and Dskip = normal."""
    p = si.mamba_block(8, 256, 1536, 16, 4, workload=si.WL_BLOCK, perturbed=perturbed)
    y, hT = _mamba_fwd(ssm, p, torch.float32)
    u, _ = oracle.conv1d_causal(p["x"], p["conv_w"], p["conv_b"])
    yr, hr = oracle.scan_fwd(u, p["dt_raw"], p["A_log"], p["B"], p["C"], dt_bias=p["dt_bias"],
                             Dskip=p["Dskip"], z=p["z"])
    assert rel_linf(y, yr) <= FP32_TOL
    assert rel_linf(hT, hr) <= FP32_TOL


def test_mamba_mini_block_L2048(ssm):
    """The forward at batch 8, L=2048, D_inner=1536, N=16, fp32 (the
    benchmark's workload and launch configuration)."""
    p = si.mamba_block(8, 2048, 1536, 16, 4, workload=si.WL_FWDBWD)
    y, hT = _mamba_fwd(ssm, p, torch.float32)
    u, _ = oracle.conv1d_causal(p["x"], p["conv_w"], p["conv_b"])
    yr, hr = oracle.scan_fwd(u, p["dt_raw"], p["A_log"], p["B"], p["C"], dt_bias=p["dt_bias"],
                             Dskip=p["Dskip"], z=p["z"])
    assert rel_linf(y, yr) <= FP32_TOL
    assert rel_linf(hT, hr) <= FP32_TOL


def test_long_sequence_bf16_chunked(ssm):
    """Long-sequence two-level scan: batch 1, L=65,536, D_inner=1536, N=16,
    bf16 inputs and output, float32 state, fused SiLU(z) gate."""
    p = si.mamba_block(1, 65536, 1536, 16, 4, workload=si.WL_LONG, bf16=True)
    u = p["x"]  # the scan input itself (no conv on this workload)
    Bn, L, D = u.shape
    hT = torch.empty(Bn, D, 16, device="cuda")
    y = ssm.ssm_scan_fwd(dev(u, torch.bfloat16), dev(p["dt_raw"], torch.bfloat16), dev(p["A_log"]),
                         dev(p["B"], torch.bfloat16), dev(p["C"], torch.bfloat16), dt_bias=dev(p["dt_bias"]),
                         Dskip=dev(p["Dskip"]), z=dev(p["z"], torch.bfloat16), hT=hT)
    torch.cuda.synchronize()
    yr, hr = oracle.scan_fwd(u, p["dt_raw"], p["A_log"], p["B"], p["C"], dt_bias=p["dt_bias"],
                             Dskip=p["Dskip"], z=p["z"])
    assert rel_linf(y, yr) <= BF16_TOL
    assert rel_linf(hT, hr) <= BF16_TOL


# --------------------------------------------------------------------------- step

def _step_oracle_loop(p, steps, disc=DB, gate=True, state_bf16=False):
    h = p["h0"].astype(np.float64).copy()
    if state_bf16:
        h = oracle.round_bf16(h)
    cs = p["conv_state"].astype(np.float64).copy()
    ys = []
    for t in range(steps):
        ys.append(oracle.step(h, cs, p["x"][:, t], p["dt_raw"][:, t], p["B"][:, t], p["C"][:, t], p["A_log"],
                              z=p["z"][:, t] if gate else None, conv_w=p["conv_w"], conv_b=p["conv_b"],
                              dt_bias=p["dt_bias"], Dskip=p["Dskip"], disc=disc, state_bf16=state_bf16))
    return np.stack(ys, 1), h, cs


@pytest.mark.parametrize("disc", [DB, ZOH])
@pytest.mark.parametrize("S,D,N,W", [(4, 40, 16, 4), (3, 8, 3, 3), (2, 16, 33, 2), (5, 24, 16, 1), (3, 20, 24, 4)])
def test_step_parity(ssm, disc, S, D, N, W):
    """Token-by-token streaming with one block against the oracle's step."""
    p = _rand(14, S, 12, D, N, W)
    y_ref, h_ref, cs_ref = _step_oracle_loop(p, 12, disc=disc)
    h = dev(p["h0"])[None].contiguous()
    cs = dev(p["conv_state"])[None].contiguous() if W > 1 else None
    ys = []
    for t in range(12):
        ys.append(ssm.ssm_step(h, dev(p["x"][:, t])[None], dev(p["dt_raw"][:, t])[None], dev(p["A_log"])[None],
                               dev(p["B"][:, t])[None], dev(p["C"][:, t])[None], conv_state=cs,
                               z=dev(p["z"][:, t])[None], conv_w=dev(p["conv_w"])[None],
                               conv_b=dev(p["conv_b"])[None], dt_bias=dev(p["dt_bias"])[None],
                               Dskip=dev(p["Dskip"])[None], disc=disc)[0])
    torch.cuda.synchronize()
    assert rel_linf(torch.stack(ys, 1), y_ref) <= FP32_TOL
    assert rel_linf(h[0], h_ref) <= FP32_TOL
    if cs is not None:
        np.testing.assert_array_equal(host(cs[0]), cs_ref)


@pytest.mark.parametrize("disc", [DB, ZOH])
def test_step_loop_equals_forward(ssm, disc):
    """Streaming with the (W-1)*D history and D*N state reproduces the full
    forward on the GPU (the two kernels share one operation order)."""
    p = _rand(15, 3, 25, 48, 16, 4)
    y, hT, cso = _fwd_gpu(ssm, p, torch.float32, disc=disc)
    h = dev(p["h0"])[None].contiguous()
    cs = dev(p["conv_state"])[None].contiguous()
    ys = []
    for t in range(25):
        ys.append(ssm.ssm_step(h, dev(p["x"][:, t])[None], dev(p["dt_raw"][:, t])[None], dev(p["A_log"])[None],
                               dev(p["B"][:, t])[None], dev(p["C"][:, t])[None], conv_state=cs,
                               z=dev(p["z"][:, t])[None], conv_w=dev(p["conv_w"])[None],
                               conv_b=dev(p["conv_b"])[None], dt_bias=dev(p["dt_bias"])[None],
                               Dskip=dev(p["Dskip"])[None], disc=disc)[0])
    torch.cuda.synchronize()
    ys = torch.stack(ys, 1)
    # the step kernel replays the sequence kernel's operation order, readout
    # tree included, so the decode is bit-identical
    assert torch.equal(ys, y)
    assert torch.equal(h[0], hT)
    assert torch.equal(cs[0], cso)


@pytest.mark.parametrize("disc", [DB, ZOH])
@pytest.mark.parametrize("gate", [True, False])
@pytest.mark.parametrize("state_bf16", [False, True])
@pytest.mark.parametrize("params", [True, False])
def test_step_common_shape_parity(ssm, disc, gate, state_bf16, params):
    """The common shape's path (fp32 io, N = 16, a 4-tap conv, D a multiple of
    64; D = 128 is two workgroups per stream) against the oracle's step over
    12 tokens: gated and ungated, float32 and bf16 stored state, with and
    without dt_bias, Dskip and conv_b."""
    S, D, steps = 5, 128, 12
    p = _rand(19, S, steps, D, 16, 4)
    if not params:
        p["dt_bias"] = np.zeros_like(p["dt_bias"])
        p["Dskip"] = np.zeros_like(p["Dskip"])
        p["conv_b"] = np.zeros_like(p["conv_b"])
    y_ref, h_ref, cs_ref = _step_oracle_loop(p, steps, disc=disc, gate=gate, state_bf16=state_bf16)
    h = dev(p["h0"], torch.bfloat16 if state_bf16 else torch.float32)[None].contiguous()
    cs = dev(p["conv_state"])[None].contiguous()
    opt = lambda k: dev(p[k])[None] if params else None
    ys = []
    for t in range(steps):
        ys.append(ssm.ssm_step(h, dev(p["x"][:, t])[None], dev(p["dt_raw"][:, t])[None], dev(p["A_log"])[None],
                               dev(p["B"][:, t])[None], dev(p["C"][:, t])[None], conv_state=cs,
                               z=dev(p["z"][:, t])[None] if gate else None, conv_w=dev(p["conv_w"])[None],
                               conv_b=opt("conv_b"), dt_bias=opt("dt_bias"), Dskip=opt("Dskip"), disc=disc)[0])
    torch.cuda.synchronize()
    tol = BF16_TOL if state_bf16 else FP32_TOL
    assert rel_linf(torch.stack(ys, 1), y_ref) <= tol
    assert rel_linf(h[0], h_ref) <= tol
    np.testing.assert_array_equal(host(cs[0]), cs_ref)


@pytest.mark.parametrize("disc", [DB, ZOH])
def test_step_common_shape_loop_equals_forward(ssm, disc):
    """At the common shape (D = 192, three workgroups per stream) the
    token-by-token decode still reproduces the full forward bit for bit."""
    p = _rand(21, 3, 25, 192, 16, 4)
    y, hT, cso = _fwd_gpu(ssm, p, torch.float32, disc=disc)
    h = dev(p["h0"])[None].contiguous()
    cs = dev(p["conv_state"])[None].contiguous()
    ys = []
    for t in range(25):
        ys.append(ssm.ssm_step(h, dev(p["x"][:, t])[None], dev(p["dt_raw"][:, t])[None], dev(p["A_log"])[None],
                               dev(p["B"][:, t])[None], dev(p["C"][:, t])[None], conv_state=cs,
                               z=dev(p["z"][:, t])[None], conv_w=dev(p["conv_w"])[None],
                               conv_b=dev(p["conv_b"])[None], dt_bias=dev(p["dt_bias"])[None],
                               Dskip=dev(p["Dskip"])[None], disc=disc)[0])
    torch.cuda.synchronize()
    assert torch.equal(torch.stack(ys, 1), y)
    assert torch.equal(h[0], hT)
    assert torch.equal(cs[0], cso)


def test_step_widest_rows_sampled(ssm):
    """D = 2^26 channels per stream (16 * D state words = 4 GiB per row, past
    the common-shape path's 32-bit offsets, so the general path runs): two
    tokens, then sampled channels at the ends of the row and around the
    powers of two compared with the oracle's step on those channels alone.
    Inputs are drawn on the device from a seeded generator."""
    S, D, N, W = 2, 1 << 26, 16, 4
    g = torch.Generator(device="cuda").manual_seed(23)
    rn = lambda *s: torch.randn(*s, generator=g, device="cuda")
    h = rn(1, S, D, N)
    cs = rn(1, S, W - 1, D)
    prm = dict(A_log=0.5 * rn(1, D, N), conv_w=rn(1, D, W), conv_b=rn(1, D), dt_bias=0.3 * rn(1, D),
               Dskip=rn(1, D))
    tok = [dict(x=rn(1, S, D), dt_raw=rn(1, S, D), B=rn(1, S, N), C=rn(1, S, N), z=rn(1, S, D)) for _ in range(2)]
    idx = torch.tensor([0, 1, 63, 64, (1 << 24) - 1, 1 << 24, (1 << 25) + 7, D - 65, D - 2, D - 1], device="cuda")
    pick = lambda t, dim: np.ascontiguousarray(host(t.index_select(dim, idx)), dtype=np.float64)
    ho, co = pick(h[0], 1), pick(cs[0], 2)
    po = {k: pick(v[0], 0) for k, v in prm.items()}
    ys = []
    for tk in tok:
        ys.append(ssm.ssm_step(h, tk["x"], tk["dt_raw"], prm["A_log"], tk["B"], tk["C"], conv_state=cs, z=tk["z"],
                               conv_w=prm["conv_w"], conv_b=prm["conv_b"], dt_bias=prm["dt_bias"],
                               Dskip=prm["Dskip"])[0].index_select(1, idx))
    torch.cuda.synchronize()
    for t, tk in enumerate(tok):
        yr = oracle.step(ho, co, pick(tk["x"][0], 1), pick(tk["dt_raw"][0], 1), host(tk["B"][0]), host(tk["C"][0]),
                         po["A_log"], z=pick(tk["z"][0], 1), conv_w=po["conv_w"], conv_b=po["conv_b"],
                         dt_bias=po["dt_bias"], Dskip=po["Dskip"])
        assert rel_linf(ys[t], yr) <= FP32_TOL, t
    assert rel_linf(h[0].index_select(1, idx), ho) <= FP32_TOL
    np.testing.assert_array_equal(host(cs[0].index_select(2, idx)), co)


def test_step_graph_replay(ssm):
    """Streaming steps captured in a HIP graph (as the decode benchmark runs
    them): every replay, with eager work and synchronisation in between,
    reproduces the same steps run eagerly, bit for bit."""
    S, D, N, W, steps = 8, 128, 16, 4, 4
    p = _rand(17, S, steps, D, N, W)
    tok = {k: dev(np.ascontiguousarray(p[k].transpose(1, 0, 2))) for k in ("x", "dt_raw", "B", "C", "z")}
    prm = {k: dev(p[k])[None].contiguous() for k in ("A_log", "conv_w", "conv_b", "dt_bias", "Dskip")}
    h0 = dev(p["h0"])[None].contiguous()
    cs0 = dev(p["conv_state"])[None].contiguous()

    def run(h, cs, ys):
        for t in range(steps):
            ssm.ssm_step(h, tok["x"][t][None], tok["dt_raw"][t][None], prm["A_log"], tok["B"][t][None],
                         tok["C"][t][None], conv_state=cs, z=tok["z"][t][None], conv_w=prm["conv_w"],
                         conv_b=prm["conv_b"], dt_bias=prm["dt_bias"], Dskip=prm["Dskip"], y=ys[t])

    h_e, cs_e = h0.clone(), cs0.clone()
    ys_e = torch.empty(steps, 1, S, D, device="cuda")
    run(h_e, cs_e, ys_e)
    torch.cuda.synchronize()
    h_g, cs_g = h0.clone(), cs0.clone()
    ys_g = torch.empty(steps, 1, S, D, device="cuda")
    run(h_g, cs_g, ys_g)            # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(h_g, cs_g, ys_g)
    for _ in range(3):
        h_g.copy_(h0)
        cs_g.copy_(cs0)
        ys_g.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(ys_g, ys_e)
        assert torch.equal(h_g, h_e)
        assert torch.equal(cs_g, cs_e)


def test_step_bf16(ssm):
    p = _rand(16, 4, 6, 32, 16, 4, bf16=True)
    y_ref, h_ref, _ = _step_oracle_loop(p, 6)
    h = dev(p["h0"])[None].contiguous()
    cs = dev(p["conv_state"])[None].contiguous()
    bf = torch.bfloat16
    for t in range(6):
        y = ssm.ssm_step(h, dev(p["x"][:, t], bf)[None], dev(p["dt_raw"][:, t], bf)[None], dev(p["A_log"])[None],
                         dev(p["B"][:, t], bf)[None], dev(p["C"][:, t], bf)[None], conv_state=cs,
                         z=dev(p["z"][:, t], bf)[None], conv_w=dev(p["conv_w"])[None],
                         conv_b=dev(p["conv_b"])[None], dt_bias=dev(p["dt_bias"])[None],
                         Dskip=dev(p["Dskip"])[None])[0]
        torch.cuda.synchronize()
        assert y.dtype == bf
        assert rel_linf(y, y_ref[:, t]) <= BF16_TOL
    assert rel_linf(h[0], h_ref) <= BF16_TOL


@pytest.mark.parametrize("S,D,N,W,io", [(4, 40, 16, 4, torch.float32), (2, 16, 33, 2, torch.float32),
                                        (3, 24, 64, 4, torch.float32), (4, 32, 16, 4, torch.bfloat16),
                                        (2, 20, 24, 3, torch.float32)])
@pytest.mark.parametrize("disc", [DB, ZOH])
def test_step_bf16_state(ssm, S, D, N, W, io, disc):
    """Streaming with the state stored in bf16 (updated in float32, rounded
    when stored) against the oracle's step with the same storage rule, over
    48 tokens."""
    steps = 48
    p = _rand(17, S, steps, D, N, W, bf16=io == torch.bfloat16)
    y_ref, h_ref, cs_ref = _step_oracle_loop(p, steps, disc=disc, state_bf16=True)
    h = dev(p["h0"], torch.bfloat16)[None].contiguous()
    cs = dev(p["conv_state"])[None].contiguous() if W > 1 else None
    ys = []
    for t in range(steps):
        ys.append(ssm.ssm_step(h, dev(p["x"][:, t], io)[None], dev(p["dt_raw"][:, t], io)[None],
                               dev(p["A_log"])[None], dev(p["B"][:, t], io)[None], dev(p["C"][:, t], io)[None],
                               conv_state=cs, z=dev(p["z"][:, t], io)[None], conv_w=dev(p["conv_w"])[None],
                               conv_b=dev(p["conv_b"])[None], dt_bias=dev(p["dt_bias"])[None],
                               Dskip=dev(p["Dskip"])[None], disc=disc)[0])
    torch.cuda.synchronize()
    assert h.dtype == torch.bfloat16
    assert rel_linf(torch.stack(ys, 1), y_ref) <= BF16_TOL
    assert rel_linf(h[0], h_ref) <= BF16_TOL
    if cs is not None:
        np.testing.assert_array_equal(host(cs[0]), cs_ref)


def test_step_bf16_state_first_step_exact_rounding(ssm):
    """One step from a bf16 state: the stored state is the bf16 rounding of
    the float32 update, which the float32-state kernel computes (same
    arithmetic), element for element."""
    p = _rand(18, 4, 1, 48, 16, 4)
    h32 = dev(oracle.round_bf16(p["h0"]).astype(np.float32))[None].contiguous()
    h16 = h32.to(torch.bfloat16)
    args = lambda: (dev(p["x"][:, 0])[None], dev(p["dt_raw"][:, 0])[None], dev(p["A_log"])[None],
                    dev(p["B"][:, 0])[None], dev(p["C"][:, 0])[None])
    kw = lambda: dict(conv_state=dev(p["conv_state"])[None].contiguous(), z=dev(p["z"][:, 0])[None],
                      conv_w=dev(p["conv_w"])[None], conv_b=dev(p["conv_b"])[None],
                      dt_bias=dev(p["dt_bias"])[None], Dskip=dev(p["Dskip"])[None])
    y32 = ssm.ssm_step(h32, *args(), **kw())
    y16 = ssm.ssm_step(h16, *args(), **kw())
    torch.cuda.synchronize()
    assert torch.equal(y16, y32)
    assert torch.equal(h16, h32.to(torch.bfloat16))


def test_streaming_decode_six_blocks(ssm):
    """Batched streaming decode: 6 blocks x 256 streams x 1536 channels x 16
    states, 3-token conv history, 1,024 consecutive steps, one launch per
    block and step.  Every stream of every block is stepped on the GPU.
    Block 0 is replayed by the oracle over all 256 streams, and its y is
    compared at every step; the other blocks are replayed for a sample of 6
    streams, y compared at steps 0, 511 and 1023.  The final state and
    history are compared for every replayed stream."""
    nblk, S, D, N, W, steps = 6, 256, 1536, 16, 4, 1024
    sample = [0, 37, 101, 128, 200, 255]
    prm = si.stream_params(nblk, D, N, W)
    P = {k: dev(v) for k, v in prm.items()}
    h = torch.zeros(nblk, S, D, N, device="cuda")
    cs = torch.zeros(nblk, S, W - 1, D, device="cuda")
    rows = [list(range(S))] + [sample] * (nblk - 1)
    ho = [np.zeros((len(r), D, N)) for r in rows]
    co = [np.zeros((len(r), W - 1, D)) for r in rows]
    worst = 0.0
    for t in range(steps):
        for k in range(nblk):
            inp = si.stream_token_torch(k, t, S, D, N, "cuda")
            y = ssm.ssm_step(h[k:k + 1], inp["x"][None], inp["dt_raw"][None], P["A_log"][k:k + 1],
                             inp["B"][None], inp["C"][None], conv_state=cs[k:k + 1], z=inp["z"][None],
                             conv_w=P["conv_w"][k:k + 1], conv_b=P["conv_b"][k:k + 1],
                             dt_bias=P["dt_bias"][k:k + 1], Dskip=P["Dskip"][k:k + 1])
            sl = {kk: host(v[rows[k]]) for kk, v in inp.items()}
            yr = oracle.step(ho[k], co[k], sl["x"], sl["dt_raw"], sl["B"], sl["C"], prm["A_log"][k], z=sl["z"],
                             conv_w=prm["conv_w"][k], conv_b=prm["conv_b"][k], dt_bias=prm["dt_bias"][k],
                             Dskip=prm["Dskip"][k])
            if k == 0 or t in (0, 511, steps - 1):
                e = rel_linf(y[0][rows[k]], yr)
                worst = max(worst, e)
                assert e <= FP32_TOL, (t, k, e)
        if t % 256 == 255:
            print("decode step %d done, worst y error so far %.2e" % (t + 1, worst), flush=True)
    torch.cuda.synchronize()
    for k in range(nblk):
        assert rel_linf(h[k][rows[k]], ho[k]) <= FP32_TOL, k
        np.testing.assert_array_equal(host(cs[k][rows[k]]), co[k])


# --------------------------------------------------------------------------- backward

_GRADS = ["dx", "d_dt_raw", "d_dt_bias", "dA_log", "dB", "dC", "dD", "dz", "dh0"]
_CONV_GRADS = ["dconv_w", "dconv_b", "dconv_state"]


def _bwd_check(ssm, p, dtype, disc, gate=True, h0=True, dhT=True, conv=False, state=False, tolerance=None,
               chunk=0):
    """ssm_scan_bwd against the oracle.  With conv, x is the conv input and
    the expected gradients come from the oracle's conv, its scan backward on
    the conv output, and its conv backward on that dLoss/du."""
    Bn, L, D = p["x"].shape
    W = p["conv_w"].shape[1]
    st = p["conv_state"] if (conv and state and W > 1) else None
    g = ssm.ssm_scan_bwd(dev(p["x"], dtype), dev(p["dt_raw"], dtype), dev(p["A_log"]), dev(p["B"], dtype),
                         dev(p["C"], dtype), dev(p["dy"], dtype), dt_bias=dev(p["dt_bias"]),
                         Dskip=dev(p["Dskip"]), z=dev(p["z"], dtype) if gate else None,
                         conv_w=dev(p["conv_w"]) if conv else None, conv_b=dev(p["conv_b"]) if conv else None,
                         conv_state_in=dev(st) if st is not None else None,
                         h0=dev(p["h0"]) if h0 else None, dhT=dev(p["dhT"]) if dhT else None, disc=disc,
                         chunk_len=chunk)
    torch.cuda.synchronize()
    u = oracle.conv1d_causal(p["x"], p["conv_w"], p["conv_b"], st)[0] if conv else p["x"]
    r = oracle.scan_bwd(u, p["dt_raw"], p["A_log"], p["B"], p["C"], p["dy"], dt_bias=p["dt_bias"],
                        Dskip=p["Dskip"], z=p["z"] if gate else None, h0=p["h0"] if h0 else None,
                        dhT=p["dhT"] if dhT else None, disc=disc)
    r["dx"] = r["du"]
    keys = list(_GRADS)
    if conv:
        rc = oracle.conv1d_causal_bwd(p["x"], p["conv_w"], r["du"], bias=p["conv_b"], state_in=st)
        r.update(dx=rc["dx"], dconv_w=rc["dw"], dconv_b=rc["db"], dconv_state=rc["dstate"])
        keys += ["dconv_w", "dconv_b"] + (["dconv_state"] if W > 1 else [])
    errs = {}
    for k in keys:
        if k == "dz" and not gate:
            continue
        errs[k] = rel_linf(g[k], r[k])
    lim = tolerance if tolerance is not None else tol(dtype)
    bad = {k: v for k, v in errs.items() if not v <= lim}
    assert not bad, (bad, errs)
    return g


@pytest.mark.parametrize("disc", [DB, ZOH])
def test_bwd_tiny_block(ssm, disc):
    t = si.tiny_block()
    p = dict(t, h0=np.zeros((1, 8, 3), np.float32), dhT=np.zeros((1, 8, 3), np.float32))
    _bwd_check(ssm, p, torch.float32, disc)


@pytest.mark.parametrize("Bn,L,D,N", [(2, 100, 40, 16), (1, 37, 24, 3), (2, 21, 16, 8), (1, 50, 70, 33),
                                      (1, 9, 16, 64), (1, 1, 1, 16)])
@pytest.mark.parametrize("disc", [DB, ZOH])
def test_bwd_shapes(ssm, Bn, L, D, N, disc):
    p = _rand(17, Bn, L, D, N)
    _bwd_check(ssm, p, torch.float32, disc)


@pytest.mark.parametrize("gate,h0,dhT", [(False, False, False), (True, False, True), (False, True, False)])
def test_bwd_optional_inputs(ssm, gate, h0, dhT):
    p = _rand(18, 2, 64, 32, 16)
    _bwd_check(ssm, p, torch.float32, DB, gate=gate, h0=h0, dhT=dhT)


def test_bwd_bf16(ssm):
    p = _rand(19, 2, 80, 48, 16, bf16=True)
    _bwd_check(ssm, p, torch.bfloat16, DB)


def test_bwd_deterministic(ssm):
    p = _rand(20, 2, 96, 128, 16)
    a = _bwd_check(ssm, p, torch.float32, DB)
    b = _bwd_check(ssm, p, torch.float32, DB)
    for k in _GRADS:
        assert torch.equal(a[k], b[k]), k


def test_bwd_forward_backward_workload(ssm):
    """Forward plus backward at batch 8, L=2,048, D_inner=1536, N=16, fp32,
    through the fused conv prologue: gradients w.r.t. x, conv_w, conv_b, dt
    (as d_dt_raw and d_dt_bias), A_log, B, C, Dskip and z against the oracle's
    conv, scan backward and conv backward."""
    p = si.mamba_block(8, 2048, 1536, 16, 4, workload=si.WL_FWDBWD, with_dy=True)
    q = dict(p, h0=np.zeros((8, 1536, 16), np.float32), dhT=np.zeros((8, 1536, 16), np.float32))
    _bwd_check(ssm, q, torch.float32, DB, h0=False, dhT=False, conv=True)


def test_bwd_forward_backward_workload_u_in(ssm):
    """The forward + backward workload in its literal form: batch 8,
    L=2,048, D_inner=1536, N=16, fp32, the scan input u = SiLU(conv4(x))
    computed beforehand (by the oracle's conv, rounded to float32) and given
    with conv_width 0, gated.  Gradients w.r.t. u, dt (as d_dt_raw and
    d_dt_bias), A_log, B, C, Dskip and z against the oracle's scan backward
    (TensorViz explorer, verified by the local recipe: the selection maps
    receive gradients)."""
    p = si.mamba_block(8, 2048, 1536, 16, 4, workload=si.WL_FWDBWD, with_dy=True)
    u, _ = oracle.conv1d_causal(p["x"], p["conv_w"], p["conv_b"])
    q = dict(p, x=u.astype(np.float32), h0=np.zeros((8, 1536, 16), np.float32),
             dhT=np.zeros((8, 1536, 16), np.float32))
    _bwd_check(ssm, q, torch.float32, DB, h0=False, dhT=False, conv=False)


# --------------------------------------------------------------------------- backward with the conv prologue

@pytest.mark.parametrize("Bn,L,D,N,W,state", [
    (2, 100, 40, 16, 4, True),     # ragged L and D, carried history
    (1, 37, 24, 3, 3, False),
    (2, 21, 16, 8, 1, False),      # one tap: no history
    (1, 50, 70, 33, 8, True),      # 8 tokens per tile
    (1, 9, 16, 64, 8, True),       # 4 tokens per tile: the 7-token halo spans two tiles
    (2, 5, 16, 16, 8, True),       # L < W - 1: history gradient reaches past the sequence
    (1, 1, 1, 16, 4, True),
])
@pytest.mark.parametrize("disc", [DB, ZOH])
def test_bwd_conv_shapes(ssm, Bn, L, D, N, W, state, disc):
    p = _rand(23, Bn, L, D, N, W)
    _bwd_check(ssm, p, torch.float32, disc, conv=True, state=state)


def test_bwd_conv_empty_sequence(ssm):
    """L = 0: nothing flows; the tap, bias and history gradients are zero and
    dh0 equals dhT."""
    p = _rand(24, 2, 0, 32, 16, 4)
    g = ssm.ssm_scan_bwd(dev(p["x"]), dev(p["dt_raw"]), dev(p["A_log"]), dev(p["B"]), dev(p["C"]),
                         dev(p["dy"]), conv_w=dev(p["conv_w"]), conv_b=dev(p["conv_b"]),
                         conv_state_in=dev(p["conv_state"]), dhT=dev(p["dhT"]))
    torch.cuda.synchronize()
    for k in ("dconv_w", "dconv_b", "dconv_state", "dD", "d_dt_bias", "dA_log"):
        assert not host(g[k]).any(), k
    np.testing.assert_array_equal(host(g["dh0"]), p["dhT"])


def test_bwd_conv_bf16(ssm):
    p = _rand(25, 2, 80, 48, 16, 4, bf16=True)
    _bwd_check(ssm, p, torch.bfloat16, DB, conv=True, state=True)


def test_bwd_conv_no_gate_no_state(ssm):
    p = _rand(26, 2, 64, 32, 16, 4)
    _bwd_check(ssm, p, torch.float32, DB, gate=False, h0=False, dhT=False, conv=True)


def test_bwd_conv_deterministic(ssm):
    p = _rand(27, 2, 96, 128, 16, 4)
    a = _bwd_check(ssm, p, torch.float32, DB, conv=True, state=True)
    b = _bwd_check(ssm, p, torch.float32, DB, conv=True, state=True)
    for k in _GRADS + _CONV_GRADS:
        assert torch.equal(a[k], b[k]), k


# --------------------------------------------------------------------------- backward split in time

@pytest.mark.parametrize("Bn,L,D,N,chunk,W,state", [
    (1, 600, 40, 16, 128, 0, False),     # ragged L and D, last chunk partial
    (2, 1000, 24, 3, 64, 0, False),
    (1, 300, 70, 33, 64, 0, False),      # 8-token tiles
    (1, 200, 16, 64, 64, 0, False),      # 4-token tiles
    (1, 700, 40, 16, 128, 4, True),      # conv: the boundary inputs feed two chunks
    (1, 500, 48, 16, 64, 8, True),
    (1, 130, 16, 16, 64, 2, False),      # a 2-token last chunk
    (1, 64, 16, 16, 64, 4, True),        # chunk == L: no split
])
@pytest.mark.parametrize("disc", [DB, ZOH])
def test_bwd_chunked_shapes(ssm, Bn, L, D, N, chunk, W, state, disc):
    """The backward split into time chunks (start states from the forward
    chunk scan, end adjoints from the reverse walk) against the sequential
    oracle."""
    p = _rand(31, Bn, L, D, N, max(W, 1), slow=True)
    _bwd_check(ssm, p, torch.float32, disc, conv=W > 0, state=state, chunk=chunk)


def test_bwd_chunked_auto_bf16(ssm):
    """Few channel workgroups and a long sequence: the library splits time on
    its own (B 1, L 4096, D 64 -> 4 chunks of 1024)."""
    p = _rand(32, 1, 4096, 64, 16, 4, bf16=True, slow=True)
    d = ssm.ssm_scan_desc(1, 4096, 64, 16, 0, 1, 0, 0)
    assert ssm.ssm_scan_bwd_workspace_size(d) > ssm.ssm_scan_bwd_workspace_size(
        ssm.ssm_scan_desc(1, 4096, 64, 16, 0, 1, 0, -1))
    _bwd_check(ssm, p, torch.bfloat16, DB)


def test_bwd_chunked_matches_unsplit(ssm):
    """Split and unsplit backward agree to rounding on the same inputs."""
    p = _rand(33, 1, 1024, 48, 16, 4, slow=True)
    args = (dev(p["x"]), dev(p["dt_raw"]), dev(p["A_log"]), dev(p["B"]), dev(p["C"]), dev(p["dy"]))
    kw = dict(dt_bias=dev(p["dt_bias"]), Dskip=dev(p["Dskip"]), z=dev(p["z"]), conv_w=dev(p["conv_w"]),
              conv_b=dev(p["conv_b"]), conv_state_in=dev(p["conv_state"]), h0=dev(p["h0"]), dhT=dev(p["dhT"]))
    a = ssm.ssm_scan_bwd(*args, chunk_len=-1, **kw)
    b = ssm.ssm_scan_bwd(*args, chunk_len=192, **kw)
    torch.cuda.synchronize()
    for k in _GRADS + _CONV_GRADS:
        assert rel_linf(b[k], a[k]) <= FP32_TOL, k


def test_bwd_long_sequence_bf16_workload(ssm):
    """Backward of the long-sequence workload: batch 1, L=65,536, D_inner=1536,
    N=16, bf16 inputs and gradients, float32 state, SiLU(z) gate; time split
    by the library (8 chunks of 8192), against the sequential oracle."""
    p = si.mamba_block(1, 65536, 1536, 16, 4, workload=si.WL_LONG, bf16=True, with_dy=True)
    q = dict(p, h0=np.zeros((1, 1536, 16), np.float32), dhT=np.zeros((1, 1536, 16), np.float32))
    _bwd_check(ssm, q, torch.bfloat16, DB, h0=False, dhT=False)
