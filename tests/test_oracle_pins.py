"""Pins of the float64 oracle to facts outside itself.

Each test checks the oracle against the numbers the pages record, a closed
form, a textbook special case that reduces to a library routine, finite
differences, or an independently written autograd loop -- never against a
retyped copy of its own loop.
"""
import json
import os

import numpy as np
import pytest
import scipy.signal
import scipy.special
import torch

import oracle
import seeded_inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tensorviz_tiny_block.json")


@pytest.fixture(scope="module")
def rec(oracle_lib):
    with open(GOLDEN) as f:
        return json.load(f)


def _recorded_A_log(D=8, N=3):
    # the recorded block stores A_log = log(1..N) as float32 parameters
    return np.tile(np.float32(np.log(np.arange(1, N + 1, dtype=np.float64))), (D, 1))


# --------------------------------------------------------------------------
# The TensorViz recorded example (manifest section "experiment")
# --------------------------------------------------------------------------

@pytest.mark.parametrize("case", ["first", "middle", "last", "changed"])
def test_recorded_decay_law(rec, case):
    """Decay a = exp(dt * -exp(A_log)) reproduces the recorded channel-0 decay
    factors from the recorded deltas, to the last bit or so."""
    c = rec["cases"][case]
    D, N = 8, 3
    delta = np.array(c["delta"]).reshape(1, 1, D)
    zeros = np.zeros((1, 1, D))
    _, _, a, _, _ = oracle.scan_core(zeros, delta, _recorded_A_log(D, N), np.zeros((1, 1, N)),
                                     np.zeros((1, 1, N)), disc=oracle.DISC_ZOH, trace=True)
    np.testing.assert_array_max_ulp(a[0, 0, 0], np.array(c["channel0_decay"]), maxulp=2)
    assert np.all((a > 0) & (a < 1))


def _one_step_from_write(h_prev, delta, write, disc=oracle.DISC_ZOH):
    """Run one oracle step on channel 0 from state h_prev with inputs chosen so
    that its write equals `write` (u = 1, B scaled by the discretised input
    coefficient)."""
    N = len(write)
    A = -np.exp(_recorded_A_log(1, N)[0].astype(np.float64))
    coef = np.expm1(delta * A) / A if disc == oracle.DISC_ZOH else np.full(N, delta)
    Bm = (np.array(write) / coef).reshape(1, 1, N)
    u = np.ones((1, 1, 1))
    h0 = None if h_prev is None else np.array(h_prev).reshape(1, 1, N)
    y, hT, a, w, h = oracle.scan_core(u, np.full((1, 1, 1), delta), _recorded_A_log(1, N), Bm,
                                      np.zeros((1, 1, N)), h0=h0, disc=disc, trace=True)
    return hT[0, 0], a[0, 0, 0], w[0, 0, 0]


@pytest.mark.parametrize("case,t", [("middle", 2), ("last", 5), ("changed", 5)])
def test_recorded_recurrence(rec, case, t):
    """h_t = a_t * h_{t-1} + w_t reproduces the recorded channel-0 history."""
    c = rec["cases"][case]
    hist = np.array(c["channel0_state_history"])
    h_t, a, w = _one_step_from_write(hist[t - 1], c["delta"][0], c["channel0_write"])
    np.testing.assert_array_max_ulp(a, np.array(c["channel0_decay"]), maxulp=2)
    np.testing.assert_allclose(w, c["channel0_write"], rtol=1e-14, atol=0)
    np.testing.assert_allclose(h_t, hist[t], rtol=1e-13, atol=1e-18)


def test_recorded_zero_initial_state(rec):
    """The first recorded state equals the first write: the scan starts at 0."""
    c = rec["cases"]["first"]
    h0, _, _ = _one_step_from_write(None, c["delta"][0], c["channel0_write"])
    np.testing.assert_allclose(h0, c["channel0_state_history"][0], rtol=1e-14, atol=0)
    np.testing.assert_array_equal(c["channel0_state_history"][0], c["channel0_write"])


def test_recorded_state_is_exact_zoh(rec):
    """After token 0 every channel's state is coef(dt_c, A_n) * B_n * u_c with one
    B shared by all channels.  Dividing the recorded 8x3 state by the oracle's
    ZOH coefficient must leave a rank-1 matrix; the dt*B coefficient must not."""
    c = rec["cases"]["first"]
    S = np.array(c["full_state"])
    D, N = S.shape
    delta = np.array(c["delta"]).reshape(1, 1, D)
    ones_u = np.ones((1, 1, D))
    ones_B = np.ones((1, 1, N))
    spreads = {}
    for disc in (oracle.DISC_ZOH, oracle.DISC_DELTA_B):
        _, coef = oracle.scan_core(ones_u, delta, _recorded_A_log(D, N), ones_B,
                                   np.zeros((1, 1, N)), disc=disc)
        R = S / coef[0]
        ratio = R / R[:, :1]
        spreads[disc] = np.max(np.abs(ratio - ratio[0]) / np.abs(ratio[0]))
    assert spreads[oracle.DISC_ZOH] < 1e-6
    assert spreads[oracle.DISC_DELTA_B] > 0.1


def test_recorded_causality_of_the_page_data(rec):
    """Changing token 2 leaves states 0-1 and token 5's delta, decay and write
    unchanged (conv reach W-1 = 2): the record itself is causal."""
    base, chg = rec["cases"]["last"], rec["cases"]["changed"]
    hb, hc = np.array(base["channel0_state_history"]), np.array(chg["channel0_state_history"])
    np.testing.assert_array_equal(hb[:2], hc[:2])
    assert not np.array_equal(hb[2:], hc[2:])
    for k in ("delta", "channel0_decay", "channel0_write", "input_token"):
        np.testing.assert_array_equal(base[k], chg[k])


def test_recorded_streaming_state_sizes(rec):
    """24 SSM values and 16 conv-history values per sequence: D*N and (W-1)*D
    for D=8, N=3, W=3."""
    D, N, W = 8, 3, 3
    assert rec["state_values_per_sequence"] == D * N
    assert rec["conv_history_values_per_sequence"] == (W - 1) * D


# --------------------------------------------------------------------------
# Numerical checks the pages name, on seeded inputs
# --------------------------------------------------------------------------

def _rand_block(Bn=2, L=9, D=3, N=4, W=3, seed=7):
    r = np.random.default_rng(seed)
    return dict(
        x=r.standard_normal((Bn, L, D)), dt_raw=r.standard_normal((Bn, L, D)),
        dt_bias=0.3 * r.standard_normal(D), A_log=0.5 * r.standard_normal((D, N)),
        B=r.standard_normal((Bn, L, N)), C=r.standard_normal((Bn, L, N)),
        z=r.standard_normal((Bn, L, D)), Dskip=r.standard_normal(D),
        h0=r.standard_normal((Bn, D, N)), conv_w=r.standard_normal((D, W)),
        conv_b=r.standard_normal(D), conv_state=r.standard_normal((Bn, W - 1, D)),
        dy=r.standard_normal((Bn, L, D)), dhT=r.standard_normal((Bn, D, N)))


def _block_fwd(p, disc):
    u, cs = oracle.conv1d_causal(p["x"], p["conv_w"], p["conv_b"], p["conv_state"])
    y, hT = oracle.scan_fwd(u, p["dt_raw"], p["A_log"], p["B"], p["C"], dt_bias=p["dt_bias"],
                            Dskip=p["Dskip"], z=p["z"], h0=p["h0"], disc=disc)
    return y, hT, cs


@pytest.mark.parametrize("disc", [oracle.DISC_DELTA_B, oracle.DISC_ZOH])
@pytest.mark.parametrize("what", ["x", "dt_raw", "B", "C", "z"])
def test_causality(oracle_lib, disc, what):
    """A change at time t0 leaves every earlier output bit-identical."""
    p = _rand_block(L=11)
    y0, _, _ = _block_fwd(p, disc)
    t0 = 5
    q = {k: v.copy() for k, v in p.items()}
    q[what][:, t0] += 1.0
    y1, _, _ = _block_fwd(q, disc)
    np.testing.assert_array_equal(y0[:, :t0], y1[:, :t0])
    assert not np.array_equal(y0[:, t0:], y1[:, t0:])


def test_conv_reach(oracle_lib):
    """A change of x at t0 moves the conv output only at t0 .. t0+W-1."""
    p = _rand_block(L=12, W=4)
    u0, _ = oracle.conv1d_causal(p["x"], p["conv_w"], p["conv_b"], p["conv_state"])
    q = p["x"].copy()
    q[:, 5] += 1.0
    u1, _ = oracle.conv1d_causal(q, p["conv_w"], p["conv_b"], p["conv_state"])
    changed = np.any(u0 != u1, axis=(0, 2))
    assert list(np.nonzero(changed)[0]) == [5, 6, 7, 8]


@pytest.mark.parametrize("disc", [oracle.DISC_DELTA_B, oracle.DISC_ZOH])
def test_closed_form_sum_of_decayed_writes(oracle_lib, disc):
    """h_t = exp(A * sum_{r<=t} dt_r) h0 + sum_{s<=t} exp(A * sum_{s<r<=t} dt_r) w_s:
    the recurrent state equals an independent O(L^2) sum of decayed past
    writes (the decay built from summed deltas, not from the per-step factors)."""
    p = _rand_block(Bn=2, L=13, D=3, N=4)
    delta = oracle.delta(p["dt_raw"], p["dt_bias"])
    y, hT, a, w, h = oracle.scan_core(p["x"], delta, p["A_log"], p["B"], p["C"],
                                      Dskip=p["Dskip"], h0=p["h0"], disc=disc, trace=True)
    A = -np.exp(p["A_log"])                       # [D, N]
    Bn, L, D = delta.shape
    cums = np.concatenate([np.zeros((Bn, 1, D)), np.cumsum(delta, axis=1)], axis=1)
    for t in range(L):
        ref = np.exp(A[None] * cums[:, t + 1][..., None]) * p["h0"]
        for s in range(t + 1):
            ref = ref + np.exp(A[None] * (cums[:, t + 1] - cums[:, s + 1])[..., None]) * w[:, s]
        np.testing.assert_allclose(h[:, t], ref, rtol=1e-12, atol=1e-14)
        yref = np.einsum("bn,bdn->bd", p["C"][:, t], ref) + p["Dskip"] * p["x"][:, t]
        np.testing.assert_allclose(y[:, t], yref, rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(hT, h[:, -1])


@pytest.mark.parametrize("disc", [oracle.DISC_DELTA_B, oracle.DISC_ZOH])
def test_time_invariant_case_is_a_convolution(oracle_lib, disc):
    """Constant dt, B, C: the scan is the LTI system whose impulse response is
    K_k = sum_n C_n a_n^k wbar_n, i.e. y = K * u + D u (np.convolve)."""
    r = np.random.default_rng(3)
    L, D, N = 40, 2, 5
    u = r.standard_normal((1, L, D))
    dt = np.full((1, L, D), 0.37)
    A_log = r.uniform(-1, 1.5, (D, N))
    b, c = r.standard_normal(N), r.standard_normal(N)
    Dsk = r.standard_normal(D)
    y, _ = oracle.scan_core(u, dt, A_log, np.tile(b, (1, L, 1)), np.tile(c, (1, L, 1)),
                            Dskip=Dsk, disc=disc)
    A = -np.exp(A_log)
    for d in range(D):
        a = np.exp(0.37 * A[d])
        wbar = (0.37 * b) if disc == oracle.DISC_DELTA_B else (a - 1.0) / A[d] * b
        K = np.array([np.sum(c * a ** k * wbar) for k in range(L)])
        ref = np.convolve(u[0, :, d], K)[:L] + Dsk[d] * u[0, :, d]
        np.testing.assert_allclose(y[0, :, d], ref, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("disc", [oracle.DISC_DELTA_B, oracle.DISC_ZOH])
def test_vanishing_A_is_a_running_sum(oracle_lib, disc):
    """A -> 0 (A_log = -40): no decay, and both discretisations reduce to
    h_t = cumsum(dt * B * u) (np.cumsum)."""
    r = np.random.default_rng(4)
    Bn, L, D, N = 2, 30, 3, 4
    u, Bm = r.standard_normal((Bn, L, D)), r.standard_normal((Bn, L, N))
    dt = r.uniform(0.01, 1.0, (Bn, L, D))
    _, _, _, _, h = oracle.scan_core(u, dt, np.full((D, N), -40.0), Bm, np.zeros((Bn, L, N)),
                                     disc=disc, trace=True)
    ref = np.cumsum(dt[..., None] * Bm[:, :, None, :] * u[..., None], axis=1)
    np.testing.assert_allclose(h, ref, rtol=1e-12, atol=1e-12)


def test_single_state_constant_delta_is_lfilter(oracle_lib):
    """N = 1 with constant dt: h is the first-order IIR filter
    h_t = a h_{t-1} + dt B_t u_t (scipy.signal.lfilter)."""
    r = np.random.default_rng(5)
    L = 64
    u, Bm, Cm = r.standard_normal((1, L, 1)), r.standard_normal((1, L, 1)), r.standard_normal((1, L, 1))
    dt, A_log = 0.21, np.array([[0.4]])
    y, hT, _, _, h = oracle.scan_core(u, np.full((1, L, 1), dt), A_log, Bm, Cm, trace=True)
    a = np.exp(-dt * np.exp(0.4))
    ref = scipy.signal.lfilter([1.0], [1.0, -a], dt * Bm[0, :, 0] * u[0, :, 0])
    np.testing.assert_allclose(h[0, :, 0, 0], ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(y[0, :, 0], Cm[0, :, 0] * ref, rtol=1e-12, atol=1e-14)


def test_decay_factors_in_unit_interval(oracle_lib):
    """Negative A and positive dt give decays in (0, 1) for every state of the
    workload recipes (tiny block, Mamba-mini block, perturbed A_log)."""
    for p in (si.tiny_block(), si.mamba_block(2, 64, 64, 16),
              si.mamba_block(2, 64, 64, 16, perturbed=True)):
        delta = oracle.delta(p["dt_raw"], p["dt_bias"])
        assert delta.min() > 0
        Bn, L, D = delta.shape
        N = p["A_log"].shape[1]
        _, _, a, _, _ = oracle.scan_core(p["x"], delta, p["A_log"], p["B"], p["C"], trace=True)
        assert a.min() > 0 and a.max() < 1


def test_mamba_block_delta_range(oracle_lib):
    """dt_bias is chosen so that softplus gives dt in [1e-3, 1e-1] before the
    0.1*normal perturbation of dt_raw."""
    p = si.mamba_block(1, 1, 512, 16)
    d0 = oracle.delta(np.zeros((1, 1, 512)), p["dt_bias"])[0, 0]
    assert d0.min() >= 1e-3 * (1 - 1e-5) and d0.max() <= 1e-1 * (1 + 1e-5)


# --------------------------------------------------------------------------
# Streaming == full forward, split == whole
# --------------------------------------------------------------------------

@pytest.mark.parametrize("disc", [oracle.DISC_DELTA_B, oracle.DISC_ZOH])
def test_streaming_equals_full_forward(oracle_lib, disc):
    """Token-by-token steps with a (W-1)*D conv cache and a D*N state give the
    full forward's outputs and final state, bit for bit."""
    p = _rand_block(Bn=2, L=10, D=8, N=3, W=3)
    y, hT, cs = _block_fwd(p, disc)
    h = p["h0"].copy()
    conv = p["conv_state"].copy()
    assert h[0].size == 24 and conv[0].size == 16
    for t in range(p["x"].shape[1]):
        yt = oracle.step(h, conv, p["x"][:, t], p["dt_raw"][:, t], p["B"][:, t], p["C"][:, t],
                         p["A_log"], z=p["z"][:, t], conv_w=p["conv_w"], conv_b=p["conv_b"],
                         dt_bias=p["dt_bias"], Dskip=p["Dskip"], disc=disc)
        np.testing.assert_array_equal(yt, y[:, t])
    np.testing.assert_array_equal(h, hT)
    np.testing.assert_array_equal(conv, cs)


@pytest.mark.parametrize("k", [1, 2, 5, 9])
def test_split_sequence_equals_whole(oracle_lib, k):
    """fwd(x[:k]) then fwd(x[k:]) from the carried (h, conv history) equals
    fwd(x), bit for bit."""
    p = _rand_block(Bn=2, L=10, D=4, N=3, W=4)
    y, hT, cs = _block_fwd(p, oracle.DISC_DELTA_B)
    first = {kk: (v[:, :k] if (hasattr(v, "ndim") and v.ndim == 3 and v.shape[1] == 10) else v)
             for kk, v in p.items()}
    second = {kk: (v[:, k:] if (hasattr(v, "ndim") and v.ndim == 3 and v.shape[1] == 10) else v)
              for kk, v in p.items()}
    y1, h1, c1 = _block_fwd(first, oracle.DISC_DELTA_B)
    second["h0"], second["conv_state"] = h1, c1
    y2, h2, c2 = _block_fwd(second, oracle.DISC_DELTA_B)
    np.testing.assert_array_equal(np.concatenate([y1, y2], axis=1), y)
    np.testing.assert_array_equal(h2, hT)
    np.testing.assert_array_equal(c2, cs)


# --------------------------------------------------------------------------
# Elementwise pieces against library routines
# --------------------------------------------------------------------------

def test_softplus_against_logaddexp(oracle_lib):
    r = np.concatenate([np.linspace(-40, 40, 801), [-700, -30, 0, 1e-8, 30, 700]])
    got = oracle.delta(r.reshape(1, 1, -1))[0, 0]
    np.testing.assert_allclose(got, np.logaddexp(0.0, r), rtol=1e-15, atol=0)


def test_silu_gate_against_expit(oracle_lib):
    """With C = 0 and Dskip = 1 the output is u * SiLU(z) (scipy expit)."""
    r = np.random.default_rng(1)
    u, z = r.standard_normal((1, 50, 2)), np.linspace(-30, 30, 100).reshape(1, 50, 2)
    y, _ = oracle.scan_core(u, np.ones((1, 50, 2)), np.zeros((2, 1)), np.zeros((1, 50, 1)),
                            np.zeros((1, 50, 1)), Dskip=np.ones(2), z=z)
    np.testing.assert_allclose(y, u * z * scipy.special.expit(z), rtol=1e-14, atol=1e-300)


@pytest.mark.parametrize("with_state", [False, True])
def test_conv_against_torch_conv1d(oracle_lib, with_state):
    p = _rand_block(Bn=3, L=17, D=5, W=4)
    st = p["conv_state"] if with_state else None
    u, so = oracle.conv1d_causal(p["x"], p["conv_w"], p["conv_b"], st, silu=False)
    W = p["conv_w"].shape[1]
    xt = torch.from_numpy(p["x"]).permute(0, 2, 1)          # [B, D, L]
    prefix = torch.from_numpy(st).permute(0, 2, 1) if with_state else torch.zeros(3, 5, W - 1, dtype=torch.float64)
    full = torch.cat([prefix, xt], dim=2)
    ref = torch.nn.functional.conv1d(full, torch.from_numpy(p["conv_w"])[:, None, :],
                                     torch.from_numpy(p["conv_b"]), groups=5)
    np.testing.assert_allclose(u, ref.permute(0, 2, 1).numpy(), rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(so, full[:, :, -(W - 1):].permute(0, 2, 1).numpy())
    us, _ = oracle.conv1d_causal(p["x"], p["conv_w"], p["conv_b"], st, silu=True)
    np.testing.assert_allclose(us, u * scipy.special.expit(u), rtol=1e-14, atol=1e-300)


def test_short_sequence_conv_state(oracle_lib):
    """L < W-1: the outgoing history mixes the incoming history and x."""
    p = _rand_block(Bn=1, L=2, D=3, W=5)
    _, so = oracle.conv1d_causal(p["x"], p["conv_w"], p["conv_b"], p["conv_state"])
    np.testing.assert_array_equal(so[:, :2], p["conv_state"][:, 2:])
    np.testing.assert_array_equal(so[:, 2:], p["x"])


def test_bf16_rounding_matches_torch():
    r = np.random.default_rng(2)
    a = np.concatenate([r.standard_normal(10000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1e-40, 3.0e38, np.inf, -np.inf], np.float32)])
    ref = torch.from_numpy(a).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(si.bf16_round(a), ref)


# --------------------------------------------------------------------------
# Backward
# --------------------------------------------------------------------------

def _loss(p, disc):
    y, hT = oracle.scan_fwd(p["x"], p["dt_raw"], p["A_log"], p["B"], p["C"], dt_bias=p["dt_bias"],
                            Dskip=p["Dskip"], z=p["z"], h0=p["h0"], disc=disc)
    return np.sum(y * p["dy"]) + np.sum(hT * p["dhT"])


_GRAD_OF = dict(x="du", dt_raw="d_dt_raw", dt_bias="d_dt_bias", A_log="dA_log", B="dB",
                C="dC", Dskip="dD", z="dz", h0="dh0")


@pytest.mark.parametrize("disc", [oracle.DISC_DELTA_B, oracle.DISC_ZOH])
def test_backward_against_finite_differences(oracle_lib, disc):
    """Every gradient of the hand-derived backward matches central finite
    differences of the forward (float64, step 1e-6)."""
    p = _rand_block(Bn=2, L=7, D=3, N=4)
    g = oracle.scan_bwd(p["x"], p["dt_raw"], p["A_log"], p["B"], p["C"], p["dy"],
                        dt_bias=p["dt_bias"], Dskip=p["Dskip"], z=p["z"], h0=p["h0"],
                        dhT=p["dhT"], disc=disc)
    eps = 1e-6
    for name, gname in _GRAD_OF.items():
        fd = np.zeros_like(p[name])
        for idx in np.ndindex(p[name].shape):
            q = {k: v.copy() for k, v in p.items()}
            q[name][idx] += eps
            lp = _loss(q, disc)
            q[name][idx] -= 2 * eps
            lm = _loss(q, disc)
            fd[idx] = (lp - lm) / (2 * eps)
        scale = max(np.max(np.abs(fd)), 1e-3)
        err = np.max(np.abs(g[gname] - fd)) / scale
        assert err < 2e-7, (name, err)
        assert np.any(g[gname] != 0), name
    # d_delta is the gradient w.r.t. dt itself: d_dt_raw = d_delta * sigmoid(r)
    sig = scipy.special.expit(p["dt_raw"] + p["dt_bias"])
    np.testing.assert_allclose(g["d_dt_raw"], g["d_delta"] * sig, rtol=1e-14, atol=1e-16)


def _torch_scan(u, dt_raw, dt_bias, A_log, Bm, Cm, Dsk, z, h0, disc):
    """An independently written float64 PyTorch version of the forward
    (vectorised over batch and channels), differentiated by autograd."""
    A = -torch.exp(A_log)
    dt = torch.nn.functional.softplus(dt_raw + dt_bias)
    h = h0
    ys = []
    for t in range(u.shape[1]):
        dA = dt[:, t, :, None] * A[None]
        if disc == oracle.DISC_ZOH:
            bbar = torch.expm1(dA) / A[None] * Bm[:, t, None, :]
        else:
            bbar = dt[:, t, :, None] * Bm[:, t, None, :]
        h = torch.exp(dA) * h + bbar * u[:, t, :, None]
        yv = (h * Cm[:, t, None, :]).sum(-1) + Dsk * u[:, t]
        ys.append(yv * torch.nn.functional.silu(z[:, t]))
    return torch.stack(ys, 1), h


@pytest.mark.parametrize("disc", [oracle.DISC_DELTA_B, oracle.DISC_ZOH])
def test_backward_against_torch_autograd(oracle_lib, disc):
    p = _rand_block(Bn=2, L=12, D=5, N=3)
    names = ["x", "dt_raw", "dt_bias", "A_log", "B", "C", "Dskip", "z", "h0"]
    ts = {k: torch.tensor(p[k], dtype=torch.float64, requires_grad=True) for k in names}
    y, hT = _torch_scan(*[ts[k] for k in names], disc)
    (y * torch.from_numpy(p["dy"])).sum().add((hT * torch.from_numpy(p["dhT"])).sum()).backward()
    g = oracle.scan_bwd(p["x"], p["dt_raw"], p["A_log"], p["B"], p["C"], p["dy"],
                        dt_bias=p["dt_bias"], Dskip=p["Dskip"], z=p["z"], h0=p["h0"],
                        dhT=p["dhT"], disc=disc)
    for k in names:
        np.testing.assert_allclose(g[_GRAD_OF[k]], ts[k].grad.numpy(), rtol=1e-10, atol=1e-12,
                                   err_msg=k)


def test_backward_without_gate_and_state(oracle_lib):
    """No z, no h0, no dhT: dz is absent and the rest still matches autograd."""
    p = _rand_block(Bn=1, L=6, D=2, N=3)
    names = ["x", "dt_raw", "dt_bias", "A_log", "B", "C", "Dskip"]
    ts = {k: torch.tensor(p[k], dtype=torch.float64, requires_grad=True) for k in names}
    A = -torch.exp(ts["A_log"])
    dt = torch.nn.functional.softplus(ts["dt_raw"] + ts["dt_bias"])
    h = torch.zeros(1, 2, 3, dtype=torch.float64)
    ys = []
    for t in range(6):
        h = torch.exp(dt[:, t, :, None] * A) * h + dt[:, t, :, None] * ts["B"][:, t, None, :] * ts["x"][:, t, :, None]
        ys.append((h * ts["C"][:, t, None, :]).sum(-1) + ts["Dskip"] * ts["x"][:, t])
    (torch.stack(ys, 1) * torch.from_numpy(p["dy"])).sum().backward()
    g = oracle.scan_bwd(p["x"], p["dt_raw"], p["A_log"], p["B"], p["C"], p["dy"],
                        dt_bias=p["dt_bias"], Dskip=p["Dskip"])
    assert g["dz"] is None
    for k in names:
        np.testing.assert_allclose(g[_GRAD_OF[k]], ts[k].grad.numpy(), rtol=1e-10, atol=1e-12,
                                   err_msg=k)


# ------------------------------------------------------------ conv backward
def _conv_loss(x, w, b, st, dy, silu):
    y, _ = oracle.conv1d_causal(x, w, b, st, silu=silu, want_state=False)
    return float(np.sum(y * dy))


@pytest.mark.parametrize("silu", [True, False])
def test_conv_backward_against_finite_differences(oracle_lib, silu):
    """dx, dw, dbias and the history gradient of the conv prologue match
    central finite differences of the oracle's own forward (float64)."""
    r = np.random.default_rng(31)
    x, w, b = r.standard_normal((2, 7, 3)), r.standard_normal((3, 4)), r.standard_normal(3)
    st, dy = r.standard_normal((2, 3, 3)), r.standard_normal((2, 7, 3))
    g = oracle.conv1d_causal_bwd(x, w, dy, bias=b, state_in=st, silu=silu)
    args = {"dx": x, "dw": w, "db": b, "dstate": st}
    eps = 1e-6
    for gname, arr in args.items():
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            keep = arr[idx]
            arr[idx] = keep + eps
            lp = _conv_loss(x, w, b, st, dy, silu)
            arr[idx] = keep - eps
            lm = _conv_loss(x, w, b, st, dy, silu)
            arr[idx] = keep
            fd[idx] = (lp - lm) / (2 * eps)
        err = np.max(np.abs(g[gname] - fd)) / max(np.max(np.abs(fd)), 1e-3)
        assert err < 2e-7, (gname, err)
        assert np.any(g[gname] != 0), gname


@pytest.mark.parametrize("silu", [True, False])
@pytest.mark.parametrize("W", [1, 4, 6])
def test_conv_backward_against_torch_autograd(oracle_lib, silu, W):
    """The same gradients from float64 torch autograd of
    torch.nn.functional.conv1d (depthwise, history prepended), then SiLU."""
    r = np.random.default_rng(32 + W)
    Bn, L, D = 2, 9, 5
    x, w, b = r.standard_normal((Bn, L, D)), r.standard_normal((D, W)), r.standard_normal(D)
    st, dy = r.standard_normal((Bn, W - 1, D)), r.standard_normal((Bn, L, D))
    tx, tw, tb, ts = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (x, w, b, st))
    full = torch.cat([ts, tx], dim=1).permute(0, 2, 1)            # [B, D, W-1+L]
    y = torch.nn.functional.conv1d(full, tw[:, None, :], tb, groups=D).permute(0, 2, 1)
    if silu:
        y = torch.nn.functional.silu(y)
    (y * torch.from_numpy(dy)).sum().backward()
    g = oracle.conv1d_causal_bwd(x, w, dy, bias=b, state_in=st if W > 1 else None, silu=silu)
    np.testing.assert_allclose(g["dx"], tx.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(g["dw"], tw.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(g["db"], tb.grad.numpy(), rtol=1e-12, atol=1e-13)
    if W > 1:
        np.testing.assert_allclose(g["dstate"], ts.grad.numpy(), rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------- bf16 streaming state

def test_round_bf16_matches_torch():
    """The oracle's bfloat16 rounding (nearest, ties to even) against torch's
    float32 -> bfloat16 conversion, including exact ties."""
    r = np.random.default_rng(5)
    x = r.standard_normal(20000).astype(np.float32) * np.float32(3.0)
    bits = x.view(np.uint32)
    ties = ((bits & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)   # exactly halfway
    for v in (x, ties):
        got = oracle.round_bf16(v.astype(np.float64))
        want = torch.from_numpy(v).to(torch.bfloat16).double().numpy()
        np.testing.assert_array_equal(got, want)


def test_step_bf16_state_rounds_after_the_readout():
    """A step with a bf16-stored state: y is the float64 step's y (it reads the
    updated state), and the kept state is the bf16 rounding of the float64
    step's state."""
    p = si.mamba_block(1, 1, 24, 16, 4, workload=si.WL_STREAM, seed=3)
    r = np.random.default_rng(6)
    h0 = oracle.round_bf16(r.standard_normal((2, 24, 16)))
    cs0 = r.standard_normal((2, 3, 24))
    x, dt, z = (r.standard_normal((2, 24)) for _ in range(3))
    B, C = (r.standard_normal((2, 16)) for _ in range(2))
    kw = dict(z=z, conv_w=p["conv_w"], conv_b=p["conv_b"], dt_bias=p["dt_bias"], Dskip=p["Dskip"])
    h64, c64 = h0.copy(), cs0.copy()
    y64 = oracle.step(h64, c64, x, dt, B, C, p["A_log"], **kw)
    hb, cb = h0.copy(), cs0.copy()
    yb = oracle.step(hb, cb, x, dt, B, C, p["A_log"], state_bf16=True, **kw)
    np.testing.assert_array_equal(yb, y64)
    np.testing.assert_array_equal(hb, oracle.round_bf16(h64))
    np.testing.assert_array_equal(cb, c64)


# --------------------------------------------------------------------------- constant decay source
# "the s6 cell", section "one cell, two architectures": the same diagonal cell
# h <- a*h + b*u with the decay a constant per (channel, state) (the RWKV side)
# instead of computed from the input at every token.  The oracle's constant
# source takes a = exp(-exp(A_log)) and the write B_t*u_t, with no step size.

def _const_fwd(p, **kw):
    return oracle.scan_fwd(p["x"], None, p["A_log"], p["B"], p["C"], Dskip=p.get("Dskip"),
                           z=p.get("z"), h0=p.get("h0"), disc=oracle.DECAY_CONST, **kw)


def test_const_decay_single_state_is_lfilter(oracle_lib):
    """State width 1 with a constant decay: h is the first-order IIR filter
    h_t = a h_{t-1} + B_t u_t with a = exp(-exp(A_log)) (scipy.signal.lfilter),
    and y = (C_t h_t + D u_t) * SiLU(z_t)."""
    r = np.random.default_rng(21)
    L, D = 80, 3
    u, z = r.standard_normal((1, L, D)), r.standard_normal((1, L, D))
    Bm, Cm = r.standard_normal((1, L, 1)), r.standard_normal((1, L, 1))
    A_log, Dsk = r.uniform(-2.0, 1.0, (D, 1)), r.standard_normal(D)
    y, hT = oracle.scan_fwd(u, None, A_log, Bm, Cm, Dskip=Dsk, z=z, disc=oracle.DECAY_CONST)
    for d in range(D):
        a = np.exp(-np.exp(A_log[d, 0]))
        h = scipy.signal.lfilter([1.0], [1.0, -a], Bm[0, :, 0] * u[0, :, d])
        ref = (Cm[0, :, 0] * h + Dsk[d] * u[0, :, d]) * z[0, :, d] * scipy.special.expit(z[0, :, d])
        np.testing.assert_allclose(y[0, :, d], ref, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(hT[0, d, 0], h[-1], rtol=1e-12, atol=1e-14)


def test_const_decay_time_invariant_is_a_convolution(oracle_lib):
    """Constant decay and constant B, C: impulse response K_k = sum_n C_n a_n^k B_n,
    y = K * u + D u (np.convolve)."""
    r = np.random.default_rng(22)
    L, D, N = 50, 2, 6
    u = r.standard_normal((1, L, D))
    A_log = r.uniform(-3, 1.0, (D, N))
    b, c = r.standard_normal(N), r.standard_normal(N)
    Dsk = r.standard_normal(D)
    y, _ = oracle.scan_fwd(u, None, A_log, np.tile(b, (1, L, 1)), np.tile(c, (1, L, 1)), Dskip=Dsk,
                           disc=oracle.DECAY_CONST)
    for d in range(D):
        a = np.exp(-np.exp(A_log[d]))
        K = np.array([np.sum(c * a ** k * b) for k in range(L)])
        ref = np.convolve(u[0, :, d], K)[:L] + Dsk[d] * u[0, :, d]
        np.testing.assert_allclose(y[0, :, d], ref, rtol=1e-11, atol=1e-12)


def test_const_decay_closed_form(oracle_lib):
    """h_t = a^(t+1) h0 + sum_{s<=t} a^(t-s) B_s u_s: the recurrent state equals
    an O(L^2) sum of powers of the constant decay (np.power), at every t."""
    p = _rand_block(Bn=2, L=12, D=3, N=4)
    Bn, L, D = p["x"].shape
    a = np.exp(-np.exp(p["A_log"]))                  # [D, N]
    w = p["B"][:, :, None, :] * p["x"][..., None]    # [B, L, D, N]
    y, hT = _const_fwd(dict(p, z=None))
    for t in range(L):
        ref = np.power(a, t + 1)[None] * p["h0"]
        for s in range(t + 1):
            ref = ref + np.power(a, t - s)[None] * w[:, s]
        yref = np.einsum("bn,bdn->bd", p["C"][:, t], ref) + p["Dskip"] * p["x"][:, t]
        np.testing.assert_allclose(y[:, t], yref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(hT, ref, rtol=1e-12, atol=1e-14)


def test_const_decay_reads_no_step_size(oracle_lib):
    """With the constant source dt_raw and dt_bias are not read: any values give
    the result of passing none, bit for bit (forward, backward and step)."""
    p = _rand_block(Bn=2, L=9, D=3, N=4)
    y0, h0 = _const_fwd(p)
    y1, h1 = oracle.scan_fwd(p["x"], p["dt_raw"], p["A_log"], p["B"], p["C"], dt_bias=p["dt_bias"],
                             Dskip=p["Dskip"], z=p["z"], h0=p["h0"], disc=oracle.DECAY_CONST)
    np.testing.assert_array_equal(y0, y1)
    np.testing.assert_array_equal(h0, h1)
    kw = dict(Dskip=p["Dskip"], z=p["z"], h0=p["h0"], dhT=p["dhT"], disc=oracle.DECAY_CONST)
    g0 = oracle.scan_bwd(p["x"], None, p["A_log"], p["B"], p["C"], p["dy"], **kw)
    g1 = oracle.scan_bwd(p["x"], p["dt_raw"], p["A_log"], p["B"], p["C"], p["dy"],
                         dt_bias=p["dt_bias"], **kw)
    for k in g0:
        if g0[k] is not None:
            np.testing.assert_array_equal(g0[k], g1[k], err_msg=k)
    for k in ("d_dt_raw", "d_delta", "d_dt_bias"):
        assert not np.any(g0[k]), k
    ha, hb = p["h0"].copy(), p["h0"].copy()
    ya = oracle.step(ha, None, p["x"][:, 0], None, p["B"][:, 0], p["C"][:, 0], p["A_log"],
                     Dskip=p["Dskip"], disc=oracle.DECAY_CONST)
    yb = oracle.step(hb, None, p["x"][:, 0], p["dt_raw"][:, 0], p["B"][:, 0], p["C"][:, 0], p["A_log"],
                     dt_bias=p["dt_bias"], Dskip=p["Dskip"], disc=oracle.DECAY_CONST)
    np.testing.assert_array_equal(ya, yb)
    np.testing.assert_array_equal(ha, hb)


def test_const_decay_is_the_live_cell_at_unit_step(oracle_lib):
    """One cell, two parameterisations: the constant source is the dt*B cell
    with dt fixed at 1 (a = exp(1*A), write 1*B*u), bit for bit."""
    p = _rand_block(Bn=2, L=10, D=3, N=5)
    yc, hc = _const_fwd(p)
    yl, hl = oracle.scan_core(p["x"], np.ones_like(p["x"]), p["A_log"], p["B"], p["C"], Dskip=p["Dskip"],
                              z=p["z"], h0=p["h0"], disc=oracle.DISC_DELTA_B)
    np.testing.assert_array_equal(yc, yl)
    np.testing.assert_array_equal(hc, hl)


def test_const_decay_streaming_equals_full_forward(oracle_lib):
    """Token-by-token steps with the constant source (and the conv prologue)
    reproduce the full forward bit for bit."""
    p = _rand_block(Bn=2, L=10, D=6, N=3, W=4)
    u, cs = oracle.conv1d_causal(p["x"], p["conv_w"], p["conv_b"], p["conv_state"])
    y, hT = oracle.scan_fwd(u, None, p["A_log"], p["B"], p["C"], Dskip=p["Dskip"], z=p["z"],
                            h0=p["h0"], disc=oracle.DECAY_CONST)
    h, conv = p["h0"].copy(), p["conv_state"].copy()
    for t in range(p["x"].shape[1]):
        yt = oracle.step(h, conv, p["x"][:, t], None, p["B"][:, t], p["C"][:, t], p["A_log"],
                         z=p["z"][:, t], conv_w=p["conv_w"], conv_b=p["conv_b"], Dskip=p["Dskip"],
                         disc=oracle.DECAY_CONST)
        np.testing.assert_array_equal(yt, y[:, t])
    np.testing.assert_array_equal(h, hT)
    np.testing.assert_array_equal(conv, cs)


_CONST_GRAD_OF = dict(x="du", A_log="dA_log", B="dB", C="dC", Dskip="dD", z="dz", h0="dh0")


def _const_loss(p):
    y, hT = _const_fwd(p)
    return np.sum(y * p["dy"]) + np.sum(hT * p["dhT"])


def test_const_decay_backward_against_finite_differences(oracle_lib):
    """Every gradient of the constant-source backward matches central finite
    differences of its forward (float64, step 1e-6)."""
    p = _rand_block(Bn=2, L=7, D=3, N=4)
    g = oracle.scan_bwd(p["x"], None, p["A_log"], p["B"], p["C"], p["dy"], Dskip=p["Dskip"], z=p["z"],
                        h0=p["h0"], dhT=p["dhT"], disc=oracle.DECAY_CONST)
    eps = 1e-6
    for name, gname in _CONST_GRAD_OF.items():
        fd = np.zeros_like(p[name])
        for idx in np.ndindex(p[name].shape):
            q = {k: v.copy() for k, v in p.items()}
            q[name][idx] += eps
            lp = _const_loss(q)
            q[name][idx] -= 2 * eps
            lm = _const_loss(q)
            fd[idx] = (lp - lm) / (2 * eps)
        scale = max(np.max(np.abs(fd)), 1e-3)
        err = np.max(np.abs(g[gname] - fd)) / scale
        assert err < 2e-7, (name, err)
        assert np.any(g[gname] != 0), name


def test_const_decay_backward_against_torch_autograd(oracle_lib):
    """The constant-source backward against float64 autograd of an
    independently written torch loop."""
    p = _rand_block(Bn=2, L=11, D=4, N=3)
    names = ["x", "A_log", "B", "C", "Dskip", "z", "h0"]
    ts = {k: torch.tensor(p[k], dtype=torch.float64, requires_grad=True) for k in names}
    a = torch.exp(-torch.exp(ts["A_log"]))
    h = ts["h0"]
    ys = []
    for t in range(p["x"].shape[1]):
        h = a * h + ts["B"][:, t, None, :] * ts["x"][:, t, :, None]
        yv = (h * ts["C"][:, t, None, :]).sum(-1) + ts["Dskip"] * ts["x"][:, t]
        ys.append(yv * torch.nn.functional.silu(ts["z"][:, t]))
    loss = (torch.stack(ys, 1) * torch.from_numpy(p["dy"])).sum() + (h * torch.from_numpy(p["dhT"])).sum()
    loss.backward()
    g = oracle.scan_bwd(p["x"], None, p["A_log"], p["B"], p["C"], p["dy"], Dskip=p["Dskip"], z=p["z"],
                        h0=p["h0"], dhT=p["dhT"], disc=oracle.DECAY_CONST)
    for k in names:
        np.testing.assert_allclose(g[_CONST_GRAD_OF[k]], ts[k].grad.numpy(), rtol=1e-10, atol=1e-12,
                                   err_msg=k)


def test_const_decay_recipe(oracle_lib):
    """The constant-decay workload's decays lie in (0, 1) and equal the decays
    the input-driven cell has at its bias step delta0 (float32 A_log)."""
    p = si.mamba_block(1, 4, 64, 16, const_decay=True)
    q = si.mamba_block(1, 4, 64, 16)
    a = np.exp(-np.exp(p["A_log"].astype(np.float64)))
    assert a.min() > 0 and a.max() < 1
    d0 = oracle.delta(np.zeros((1, 1, 64)), q["dt_bias"])[0, 0]
    np.testing.assert_allclose(a, np.exp(-d0[:, None] * np.exp(q["A_log"].astype(np.float64))), rtol=1e-5)
