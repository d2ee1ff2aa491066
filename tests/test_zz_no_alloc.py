"""ssm_scan_fwd_static, the forward that allocates nothing: through the C
ABI its results equal ssm_scan_fwd's (same kernels, the chunk summaries in
the library's static buffer instead of a workspace), bit for bit, on two
calls in a row, the second with a smaller input; the first is also checked
against the oracle."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from parity import FP32_TOL, dev, rel_linf

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ssm():
    import selective_state_space_ssm_amd as m
    m.lib()
    assert torch.cuda.is_available(), "no GPU visible"
    return m


def _inputs(seed, Bn, L, D, N, W):
    r = np.random.default_rng(seed)
    f = lambda *s: r.standard_normal(s).astype(np.float32)
    return dict(x=f(Bn, L, D), dt_raw=0.3 * f(Bn, L, D), B=f(Bn, L, N), C=f(Bn, L, N), z=f(Bn, L, D),
                dt_bias=(0.2 * f(D) - 2.0).astype(np.float32), A_log=(0.5 * f(D, N)).astype(np.float32),
                Dskip=f(D), h0=f(Bn, D, N), conv_w=f(D, W), conv_b=f(D), conv_state=f(Bn, W - 1, D))


def _call(ssm, fn, p, chunk, **extra):
    Bn, L, D = p["x"].shape
    N, W = p["A_log"].shape[1], p["conv_w"].shape[1]
    P = {k: dev(v) for k, v in p.items()}
    y = torch.full((Bn, L, D), float("nan"), device="cuda")
    hT = torch.full((Bn, D, N), float("nan"), device="cuda")
    cso = torch.full((Bn, W - 1, D), float("nan"), device="cuda")
    fn(P["x"], P["dt_raw"], P["A_log"], P["B"], P["C"], dt_bias=P["dt_bias"], Dskip=P["Dskip"], z=P["z"],
       conv_w=P["conv_w"], conv_b=P["conv_b"], conv_state_in=P["conv_state"], conv_state_out=cso, h0=P["h0"],
       hT=hT, y=y, chunk_len=chunk, **extra)
    torch.cuda.synchronize()
    return y, hT, cso


@pytest.mark.parametrize("first,second", [((2, 4096, 96, 16, 4, 512), (1, 1000, 48, 16, 4, 256))])
def test_static_forward_equals_workspace_forward(ssm, first, second):
    for i, (Bn, L, D, N, W, chunk) in enumerate((first, second)):
        desc = ssm.ssm_scan_desc(Bn, L, D, N, W, 0, 0, chunk)
        need = ssm.ssm_scan_fwd_workspace_size(desc)
        assert 0 < need <= ssm.SSM_STATIC_SCRATCH_BYTES, need     # the time split is taken
        p = _inputs(100 + i, Bn, L, D, N, W)
        got = _call(ssm, ssm.ssm_scan_fwd_static, p, chunk)
        ref = _call(ssm, ssm.ssm_scan_fwd, p, chunk)
        for g, r, name in zip(got, ref, ("y", "hT", "conv_state_out")):
            assert torch.equal(g, r), (i, name, rel_linf(g, r))
        if i == 0:
            u, cso = oracle.conv1d_causal(p["x"], p["conv_w"], p["conv_b"], p["conv_state"])
            yo, ho = oracle.scan_fwd(u, p["dt_raw"], p["A_log"], p["B"], p["C"], dt_bias=p["dt_bias"],
                                     Dskip=p["Dskip"], z=p["z"], h0=p["h0"])
            assert rel_linf(got[0], yo) <= FP32_TOL
            assert rel_linf(got[1], ho) <= FP32_TOL
            np.testing.assert_array_equal(got[2].cpu().numpy(), cso)


def test_static_forward_refuses_oversized_split(ssm):
    """A split whose summaries exceed the buffer is refused before any HIP
    call (the tensors are tiny; the descriptor is what is checked)."""
    desc = ssm.ssm_scan_desc(64, 4096, 1536, 16, 0, 0, 0, 64)
    assert ssm.ssm_scan_fwd_workspace_size(desc) > ssm.SSM_STATIC_SCRATCH_BYTES
    t = torch.zeros(16, device="cuda")
    ptr = ctypes.c_void_p(t.data_ptr())
    rc = ssm.lib().ssm_scan_fwd_static(ctypes.byref(desc), ptr, ptr, None, ptr, ptr, ptr, None, None, None, None,
                                       None, None, None, None, ptr, None)
    assert rc == ssm.SSM_ERR_SCRATCH_LIMIT
