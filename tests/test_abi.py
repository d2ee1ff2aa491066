"""The C ABI on a machine without a GPU: the library loads, exports every
symbol include/ssm.h declares, and rejects bad arguments with the documented
status before any HIP call.  Device pointers here are fake addresses that the
library never dereferences (validation fails first)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def ssm():
    import selective_state_space_ssm_amd as m
    if not os.path.exists(m.LIB_PATH):
        from selective_state_space_ssm_amd import build
        build.build()
    return m


def _header_functions():
    txt = open(os.path.join(ROOT, "include", "ssm.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_0-9]+)\s*\(", txt)) - {"sizeof"})


def test_header_declares_the_four_calls():
    fns = _header_functions()
    for f in ("ssm_scan_fwd", "ssm_scan_bwd", "ssm_step", "conv1d_causal"):
        assert f in fns


def test_library_exports_every_declared_symbol(ssm):
    lib = ctypes.CDLL(ssm.LIB_PATH)
    fns = _header_functions()
    assert set(fns) == set(ssm.EXPORTED_SYMBOLS)
    for f in fns:
        assert hasattr(lib, f), f


def test_version_and_status_strings(ssm):
    assert ssm.ssm_version() // 100 == 2
    for code in range(0, 9):
        s = ssm.ssm_status_string(code)
        assert isinstance(s, str) and len(s) > 3
    assert ssm.ssm_status_string(99) == "unknown status"


A = 0x10000000  # fake, 16-byte aligned device addresses (never dereferenced)


def _addr(k, off=0):
    return ctypes.c_void_p(A + k * 0x1000000 + off)


def _fwd(ssm, desc, **over):
    names = ["x", "dt_raw", "dt_bias", "A_log", "B", "C", "Dskip", "z", "conv_w", "conv_b",
             "conv_state_in", "conv_state_out", "h0", "hT", "y", "workspace"]
    args = {n: _addr(i) for i, n in enumerate(names)}
    for n in ("dt_bias", "Dskip", "z", "conv_w", "conv_b", "conv_state_in", "conv_state_out", "h0", "hT",
              "workspace"):
        args[n] = None
    args.update(over)
    ws_bytes = over.pop("ws_bytes", 0) if "ws_bytes" in over else 0
    return ssm.lib().ssm_scan_fwd(ctypes.byref(desc), *[args[n] for n in names], ctypes.c_size_t(ws_bytes), None)


def _desc(ssm, B=2, L=16, D=32, N=16, W=0, io=0, disc=0, chunk=-1):
    return ssm.ssm_scan_desc(B, L, D, N, W, io, disc, chunk)


@pytest.mark.parametrize("field,value", [("batch", 0), ("seqlen", -1), ("dim", 0), ("dstate", 0),
                                         ("dstate", 65), ("conv_width", 9), ("conv_width", -1),
                                         ("chunk_len", -2)])
def test_scan_fwd_bad_shape(ssm, field, value):
    d = _desc(ssm)
    setattr(d, field, value)
    assert _fwd(ssm, d) == ssm.SSM_ERR_BAD_SHAPE


@pytest.mark.parametrize("field,value", [("io_dtype", 2), ("disc", 3), ("disc", -1)])
def test_scan_fwd_unsupported(ssm, field, value):
    d = _desc(ssm)
    setattr(d, field, value)
    assert _fwd(ssm, d) == ssm.SSM_ERR_UNSUPPORTED


def test_const_decay_needs_no_step_size(ssm):
    """With the constant decay source dt_raw may be NULL (it is never read):
    the call gets past the NULL checks to the next error planted (a
    misaligned tensor), where the input-driven forms stop at dt_raw."""
    assert ssm.SSM_DECAY_CONST == 2
    d_live, d_const = _desc(ssm), _desc(ssm, disc=ssm.SSM_DECAY_CONST)
    assert _fwd(ssm, d_live, dt_raw=None, y=_addr(40, 4)) == ssm.SSM_ERR_NULL_ARG
    assert _fwd(ssm, d_const, dt_raw=None, y=_addr(40, 4)) == ssm.SSM_ERR_ALIGNMENT
    n = ssm.ssm_scan_bwd_workspace_size(d_const)
    assert _bwd(ssm, d_live, _addr(50), n, dt_raw=None, dx=_addr(40, 4)) == ssm.SSM_ERR_NULL_ARG
    assert _bwd(ssm, d_const, _addr(50), n, dt_raw=None, dx=_addr(40, 4)) == ssm.SSM_ERR_ALIGNMENT
    L = ssm.lib()
    ptrs = [_addr(i) for i in range(13)]
    ptrs[3] = None        # dt_raw
    ptrs[12] = _addr(40, 4)   # misaligned y
    live = ssm.ssm_step_desc(2, 8, 32, 16, 4, 0, 0, 0)
    const = ssm.ssm_step_desc(2, 8, 32, 16, 4, 0, ssm.SSM_DECAY_CONST, 0)
    assert L.ssm_step(ctypes.byref(live), *ptrs, None) == ssm.SSM_ERR_NULL_ARG
    assert L.ssm_step(ctypes.byref(const), *ptrs, None) == ssm.SSM_ERR_ALIGNMENT
    bad = ssm.ssm_step_desc(2, 8, 32, 16, 4, 0, 3, 0)
    assert L.ssm_step(ctypes.byref(bad), *ptrs, None) == ssm.SSM_ERR_UNSUPPORTED


def test_scan_fwd_null_desc(ssm):
    assert ssm.lib().ssm_scan_fwd(None, *([None] * 16), ctypes.c_size_t(0), None) == ssm.SSM_ERR_NULL_ARG


@pytest.mark.parametrize("name", ["x", "dt_raw", "A_log", "B", "C", "y"])
def test_scan_fwd_required_pointers(ssm, name):
    assert _fwd(ssm, _desc(ssm), **{name: None}) == ssm.SSM_ERR_NULL_ARG


def test_scan_fwd_conv_needs_weights(ssm):
    assert _fwd(ssm, _desc(ssm, W=4)) == ssm.SSM_ERR_NULL_ARG


@pytest.mark.parametrize("name", ["x", "B", "A_log", "y", "h0"])
def test_scan_fwd_alignment(ssm, name):
    assert _fwd(ssm, _desc(ssm), **{name: _addr(40, 4)}) == ssm.SSM_ERR_ALIGNMENT


def test_scan_fwd_output_overlapping_input(ssm):
    assert _fwd(ssm, _desc(ssm), y=_addr(0, 64)) == ssm.SSM_ERR_ALIAS


def test_scan_fwd_outputs_overlapping_each_other(ssm):
    assert _fwd(ssm, _desc(ssm), hT=_addr(14, 16)) == ssm.SSM_ERR_ALIAS


def test_scan_fwd_partial_state_alias_rejected(ssm):
    assert _fwd(ssm, _desc(ssm), h0=_addr(20), hT=_addr(20, 16)) == ssm.SSM_ERR_ALIAS


def test_scan_fwd_workspace_required_when_split(ssm):
    d = _desc(ssm, B=1, L=4096, D=32, N=16, chunk=256)
    n = ssm.ssm_scan_fwd_workspace_size(d)
    assert n > 0
    assert _fwd(ssm, d) == ssm.SSM_ERR_WORKSPACE
    assert _fwd(ssm, d, workspace=_addr(30), ws_bytes=n - 1) == ssm.SSM_ERR_WORKSPACE


def test_scan_fwd_workspace_zero_without_split(ssm):
    assert ssm.ssm_scan_fwd_workspace_size(_desc(ssm, chunk=-1)) == 0
    assert ssm.ssm_scan_fwd_workspace_size(_desc(ssm, L=64, chunk=1000)) == 0


_BWD = ["x", "dt_raw", "dt_bias", "A_log", "B", "C", "Dskip", "z", "conv_w", "conv_b", "conv_state_in",
        "h0", "dy", "dhT", "dx", "d_dt_raw", "d_dt_bias", "dA_log", "dB", "dC", "dDskip", "dz", "dh0",
        "dconv_w", "dconv_b", "dconv_state_in"]
_BWD_OPTIONAL_ABSENT = ["dt_bias", "Dskip", "z", "conv_w", "conv_b", "conv_state_in", "h0", "dhT", "dz",
                        "dconv_w", "dconv_b", "dconv_state_in"]


def _bwd(ssm, desc, ws=None, ws_bytes=0, **over):
    args = {k: _addr(i) for i, k in enumerate(_BWD)}
    for k in _BWD_OPTIONAL_ABSENT:
        args[k] = None
    args.update(over)
    return ssm.lib().ssm_scan_bwd(ctypes.byref(desc), *[args[k] for k in _BWD], ws, ctypes.c_size_t(ws_bytes),
                                  None)


def test_scan_bwd_workspace_and_nulls(ssm):
    d = _desc(ssm)
    n = ssm.ssm_scan_bwd_workspace_size(d)
    assert n > 0
    assert _bwd(ssm, d) == ssm.SSM_ERR_WORKSPACE
    assert _bwd(ssm, d, _addr(50), n - 1) == ssm.SSM_ERR_WORKSPACE
    assert _bwd(ssm, d, _addr(50), n, dy=None) == ssm.SSM_ERR_NULL_ARG
    assert _bwd(ssm, d, _addr(50), n, dz=_addr(30)) == ssm.SSM_ERR_NULL_ARG   # dz without z


def test_scan_bwd_conv_arguments(ssm):
    d0, d4 = _desc(ssm), _desc(ssm, W=4)
    n = ssm.ssm_scan_bwd_workspace_size(d4)
    # with the conv prologue the workspace also holds u and dLoss/du
    assert n > ssm.ssm_scan_bwd_workspace_size(d0)
    # conv width 4 needs the taps
    assert _bwd(ssm, d4, _addr(50), n) == ssm.SSM_ERR_NULL_ARG
    # conv gradients without a conv
    for k in ("dconv_w", "dconv_b", "dconv_state_in"):
        assert _bwd(ssm, d0, _addr(50), n, **{k: _addr(40)}) == ssm.SSM_ERR_BAD_SHAPE
    # conv inputs and outputs are alignment- and alias-checked
    assert _bwd(ssm, d4, _addr(50), n, conv_w=_addr(40, 4)) == ssm.SSM_ERR_ALIGNMENT
    assert _bwd(ssm, d4, _addr(50), n, conv_w=_addr(40), dconv_b=_addr(41, 8)) == ssm.SSM_ERR_ALIGNMENT
    assert _bwd(ssm, d4, _addr(50), n, conv_w=_addr(40), dconv_w=_addr(40, 16)) == ssm.SSM_ERR_ALIAS
    assert _bwd(ssm, d4, _addr(50), n, conv_w=_addr(40), conv_state_in=_addr(41),
                dconv_state_in=_addr(41)) == ssm.SSM_ERR_ALIAS


def test_step_validation(ssm):
    L = ssm.lib()
    good = ssm.ssm_step_desc(2, 8, 32, 16, 4, 0, 0, 0)
    ptrs = [_addr(i) for i in range(13)]
    bad = ssm.ssm_step_desc(2, 8, 32, 16, 4, 0, 0, 2)   # no such state dtype
    assert L.ssm_step(ctypes.byref(bad), *ptrs, None) == ssm.SSM_ERR_UNSUPPORTED
    bad = ssm.ssm_step_desc(0, 8, 32, 16, 4, 0, 0, 0)
    assert L.ssm_step(ctypes.byref(bad), *ptrs, None) == ssm.SSM_ERR_BAD_SHAPE
    p2 = list(ptrs)
    p2[1] = None  # conv_state with W = 4
    assert L.ssm_step(ctypes.byref(good), *p2, None) == ssm.SSM_ERR_NULL_ARG
    p3 = list(ptrs)
    p3[12] = _addr(2, 32)  # y inside x
    assert L.ssm_step(ctypes.byref(good), *p3, None) == ssm.SSM_ERR_ALIAS
    p4 = list(ptrs)
    p4[0] = _addr(0, 8)
    assert L.ssm_step(ctypes.byref(good), *p4, None) == ssm.SSM_ERR_ALIGNMENT


def test_launch_grid_limit(ssm):
    """Shapes whose launch grid would pass 2^31 - 1 workgroups are rejected
    before any HIP call: 2^32 streams of one channel and one state (a state of
    16 GB, which fits an MI355X), a conv over 2^40 rows, a forward split into
    one-token chunks over 2^40 tokens."""
    L = ssm.lib()
    ptrs = [_addr(i) for i in range(13)]
    big = ssm.ssm_step_desc(1, 2 ** 32, 1, 1, 0, 0, 0, 0)
    assert L.ssm_step(ctypes.byref(big), *ptrs, None) == ssm.SSM_ERR_BAD_SHAPE
    # an accepted grid must still stop at a later host check: y misaligned
    # (these fake addresses must never reach a kernel on a machine with a GPU)
    ok = ssm.ssm_step_desc(1, 2 ** 20, 1, 1, 0, 0, 0, 0)
    p_ok = list(ptrs)
    p_ok[12] = _addr(12, 4)
    assert L.ssm_step(ctypes.byref(ok), *p_ok, None) == ssm.SSM_ERR_ALIGNMENT
    conv = ssm.ssm_conv_desc(1, 2 ** 40, 1, 4, 1, 0, 0)
    assert L.conv1d_causal(ctypes.byref(conv), *[_addr(i) for i in range(6)], None) == ssm.SSM_ERR_BAD_SHAPE
    assert _fwd(ssm, _desc(ssm, B=1, L=2 ** 40, D=16, N=1, chunk=1)) == ssm.SSM_ERR_BAD_SHAPE
    # accepted: stops at the missing workspace the split needs
    assert _fwd(ssm, _desc(ssm, B=1, L=2 ** 20, D=16, N=1, chunk=1)) == ssm.SSM_ERR_WORKSPACE
    # channels past the sequence kernels' 32-bit tile offsets: a 64-token
    # float32 tile of 2^24 channels is 2^32 bytes
    assert _fwd(ssm, _desc(ssm, B=1, L=4, D=2 ** 24, N=1)) == ssm.SSM_ERR_BAD_SHAPE
    # accepted: stops at y overlapping x
    assert _fwd(ssm, _desc(ssm, B=1, L=4, D=2 ** 24 - 1, N=1), y=_addr(0)) == ssm.SSM_ERR_ALIAS


def test_bwd_checkpoint_offset_limit(ssm):
    """The backward's state checkpoints (D * N floats a tile) take 32-bit byte
    offsets; the channel limit keeps the widest one, N = 64 at the most
    channels, under 2^32 bytes: it passes every shape check and stops at the
    missing workspace, and one channel more is rejected."""
    d = _desc(ssm, B=1, L=4, D=2 ** 24 - 1, N=64)
    assert ssm.ssm_scan_bwd_workspace_size(d) > 0
    assert _bwd(ssm, d) == ssm.SSM_ERR_WORKSPACE
    assert _bwd(ssm, _desc(ssm, B=1, L=4, D=2 ** 24, N=64)) == ssm.SSM_ERR_BAD_SHAPE


def test_bwd_sums_launch_grid_limit(ssm):
    """The backward's cross-workgroup sums are one launch: the dB, dC blocks,
    then the parameter blocks.  A shape whose dB, dC blocks alone fill the
    2^31 - 1 workgroup limit (B*L*N / 256 of them) is rejected before any HIP
    call once the parameter blocks are added; one row of blocks fewer passes
    and stops at the missing workspace."""
    L = 4 * (2 ** 31 - 1)              # L * 64 / 256 = 2^31 - 1 blocks at N = 64
    assert _bwd(ssm, _desc(ssm, B=1, L=L, D=4, N=64)) == ssm.SSM_ERR_BAD_SHAPE
    assert _bwd(ssm, _desc(ssm, B=1, L=L - 4, D=4, N=64)) == ssm.SSM_ERR_WORKSPACE


def test_conv_validation(ssm):
    L = ssm.lib()
    d = ssm.ssm_conv_desc(2, 16, 32, 4, 1, 0, 0)
    ptrs = [_addr(i) for i in range(6)]
    bad = ssm.ssm_conv_desc(2, 16, 32, 9, 1, 0, 0)
    assert L.conv1d_causal(ctypes.byref(bad), *ptrs, None) == ssm.SSM_ERR_BAD_SHAPE
    bad = ssm.ssm_conv_desc(2, 16, 32, 4, 2, 0, 0)
    assert L.conv1d_causal(ctypes.byref(bad), *ptrs, None) == ssm.SSM_ERR_UNSUPPORTED
    p = list(ptrs)
    p[1] = None
    assert L.conv1d_causal(ctypes.byref(d), *p, None) == ssm.SSM_ERR_NULL_ARG
    p = list(ptrs)
    p[4] = p[3]  # state_out == state_in
    assert L.conv1d_causal(ctypes.byref(d), *p, None) == ssm.SSM_ERR_ALIAS


def test_binding_rejects_host_tensors(ssm):
    import torch
    x = torch.zeros(1, 4, 8)
    with pytest.raises(ValueError):
        ssm.conv1d_causal(x, torch.zeros(8, 4))


def _model_call(ssm, desc, ws_bytes=None, layer_over=None, **over):
    """ssm_model_decode_step with fake, aligned, disjoint device addresses."""
    nl = desc.n_layers
    arr = (ssm.ssm_layer_weights * nl)()
    for i in range(nl):
        for j, f in enumerate(ssm.LAYER_FIELDS):
            setattr(arr[i], f, A + (100 + 16 * i + j) * 0x1000000)
        for f, v in (layer_over or {}).items():
            setattr(arr[i], f, v)
    args = dict(emb=_addr(1), norm_f_w=_addr(2), norm_f_b=_addr(3), tokens=_addr(4), h=_addr(5),
                conv_state=_addr(6), logits=_addr(7), workspace=_addr(8))
    args.update(over)
    n = ssm.ssm_model_decode_workspace_size(desc) if ws_bytes is None else ws_bytes
    return ssm.lib().ssm_model_decode_step(
        ctypes.byref(desc), args["emb"], args["norm_f_w"], args["norm_f_b"], arr, args["tokens"], args["h"],
        args["conv_state"], args["logits"], args["workspace"], ctypes.c_size_t(n), None)


def test_model_decode_validation(ssm):
    import seeded_inputs as si
    good = ssm.model_desc(si.TINY_MODEL, 4)
    assert ssm.ssm_model_decode_workspace_size(good) > 0
    for field, value, code in [("d_state", 65, ssm.SSM_ERR_BAD_SHAPE), ("conv_width", 0, ssm.SSM_ERR_BAD_SHAPE),
                               ("conv_width", 9, ssm.SSM_ERR_BAD_SHAPE), ("nstreams", 0, ssm.SSM_ERR_BAD_SHAPE),
                               ("dt_rank", 0, ssm.SSM_ERR_BAD_SHAPE), ("d_model", 8193, ssm.SSM_ERR_BAD_SHAPE),
                               ("reserved", 1, ssm.SSM_ERR_UNSUPPORTED)]:
        d = ssm.model_desc(si.TINY_MODEL, 4)
        setattr(d, field, value)
        assert _model_call(ssm, d, ws_bytes=1 << 20) == code, field
    assert _model_call(ssm, good, emb=None) == ssm.SSM_ERR_NULL_ARG
    assert _model_call(ssm, good, layer_over={"x_proj": None}) == ssm.SSM_ERR_NULL_ARG
    assert _model_call(ssm, good, conv_state=None) == ssm.SSM_ERR_NULL_ARG      # W = 4 needs the history
    n = ssm.ssm_model_decode_workspace_size(good)
    assert _model_call(ssm, good, ws_bytes=n - 1) == ssm.SSM_ERR_WORKSPACE
    assert _model_call(ssm, good, logits=_addr(7, 4)) == ssm.SSM_ERR_ALIGNMENT
    assert _model_call(ssm, good, tokens=_addr(4, 2)) == ssm.SSM_ERR_ALIGNMENT
    assert _model_call(ssm, good, layer_over={"A_log": A + 0x50000004}) == ssm.SSM_ERR_ALIGNMENT
    assert _model_call(ssm, good, logits=_addr(1, 64)) == ssm.SSM_ERR_ALIAS     # logits inside emb
    assert _model_call(ssm, good, h=_addr(8, 256)) == ssm.SSM_ERR_ALIAS         # state inside the workspace


def _fwd_static(ssm, desc, **over):
    names = ["x", "dt_raw", "dt_bias", "A_log", "B", "C", "Dskip", "z", "conv_w", "conv_b",
             "conv_state_in", "conv_state_out", "h0", "hT", "y"]
    args = {n: _addr(i) for i, n in enumerate(names)}
    for n in ("dt_bias", "Dskip", "z", "conv_w", "conv_b", "conv_state_in", "conv_state_out", "h0", "hT"):
        args[n] = None
    args.update(over)
    return ssm.lib().ssm_scan_fwd_static(ctypes.byref(desc), *[args[n] for n in names], None)


def test_scan_fwd_static_rejects_requests_beyond_its_buffer(ssm):
    """The no-allocation forward refuses, before any HIP call, a time split
    whose chunk summaries exceed the static buffer, and validates its other
    arguments as ssm_scan_fwd does (these fake addresses never reach a
    kernel: every case stops at a host check)."""
    assert ssm.SSM_ERR_SCRATCH_LIMIT == 8
    big = _desc(ssm, B=64, L=4096, D=1536, N=16, chunk=64)
    assert ssm.ssm_scan_fwd_workspace_size(big) > ssm.SSM_STATIC_SCRATCH_BYTES
    assert _fwd_static(ssm, big) == ssm.SSM_ERR_SCRATCH_LIMIT
    fits = _desc(ssm, B=1, L=4096, D=64, N=16, chunk=256)
    assert 0 < ssm.ssm_scan_fwd_workspace_size(fits) <= ssm.SSM_STATIC_SCRATCH_BYTES
    assert _fwd_static(ssm, fits, y=_addr(0, 64)) == ssm.SSM_ERR_ALIAS          # y inside x
    assert _fwd_static(ssm, fits, x=None) == ssm.SSM_ERR_NULL_ARG
    assert _fwd_static(ssm, fits, B=_addr(4, 4)) == ssm.SSM_ERR_ALIGNMENT
    assert _fwd_static(ssm, _desc(ssm, N=65)) == ssm.SSM_ERR_BAD_SHAPE
