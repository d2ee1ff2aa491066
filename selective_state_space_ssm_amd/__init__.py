"""Python binding of the gfx950 selective-scan library (libssm_amd.so).

A thin ctypes layer over the C ABI declared in include/ssm.h: every function
here has the name of the C entry point it calls and only marshals arguments
(torch tensors -> device pointers, the current HIP stream, descriptors).
PyTorch supplies device memory and streams; all arithmetic runs in the HIP
kernels.  Outputs that are not passed in are allocated with torch.empty.

The library must have been built (selective_state_space_ssm_amd/build.py);
importing the binding never falls back to any other implementation.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssm_amd.so")

SSM_OK = 0
SSM_ERR_NULL_ARG = 1
SSM_ERR_BAD_SHAPE = 2
SSM_ERR_UNSUPPORTED = 3
SSM_ERR_WORKSPACE = 4
SSM_ERR_ALIGNMENT = 5
SSM_ERR_ALIAS = 6
SSM_ERR_HIP = 7
SSM_ERR_SCRATCH_LIMIT = 8
SSM_STATIC_SCRATCH_BYTES = 16 << 20   # the library's static device buffer (ssm_scan_fwd_static)

SSM_F32 = 0
SSM_BF16 = 1
SSM_DISC_DELTA_B = 0
SSM_DISC_ZOH = 1
SSM_DECAY_CONST = 2   # decay fixed per (channel, state); no step size, dt_raw may be None

EXPORTED_SYMBOLS = (
    "ssm_version", "ssm_status_string", "conv1d_causal", "ssm_scan_fwd_workspace_size",
    "ssm_scan_fwd", "ssm_scan_bwd_workspace_size", "ssm_scan_bwd", "ssm_step",
    "ssm_model_decode_workspace_size", "ssm_model_decode_step", "ssm_scan_fwd_static",
)


class SSMError(RuntimeError):
    def __init__(self, fn, code):
        self.code = int(code)
        super().__init__("%s failed: %s (status %d)" % (fn, ssm_status_string(code), code))


class ssm_scan_desc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("dim", ctypes.c_int64),
                ("dstate", ctypes.c_int64), ("conv_width", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("disc", ctypes.c_int32), ("chunk_len", ctypes.c_int32)]


class ssm_step_desc(ctypes.Structure):
    _fields_ = [("nblocks", ctypes.c_int64), ("nstreams", ctypes.c_int64), ("dim", ctypes.c_int64),
                ("dstate", ctypes.c_int64), ("conv_width", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("disc", ctypes.c_int32), ("state_dtype", ctypes.c_int32)]


class ssm_conv_desc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("dim", ctypes.c_int64),
                ("width", ctypes.c_int32), ("fuse_silu", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class ssm_model_desc(ctypes.Structure):
    _fields_ = [("nstreams", ctypes.c_int64), ("vocab", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("n_layers", ctypes.c_int32), ("d_inner", ctypes.c_int32), ("d_state", ctypes.c_int32),
                ("dt_rank", ctypes.c_int32), ("conv_width", ctypes.c_int32), ("reserved", ctypes.c_int32)]


LAYER_FIELDS = ("norm_w", "norm_b", "in_proj", "conv_w", "conv_b", "x_proj", "dt_proj_w", "dt_proj_b",
                "A_log", "Dskip", "out_proj")


class ssm_layer_weights(ctypes.Structure):
    _fields_ = [(f, ctypes.c_void_p) for f in LAYER_FIELDS]


_lib = None


def lib():
    """The loaded library with argument types set (raises if not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libssm_amd.so is not built; run selective_state_space_ssm_amd/build.py "
                              "(or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        p, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.ssm_version.restype = i32
        L.ssm_version.argtypes = []
        L.ssm_status_string.restype = ctypes.c_char_p
        L.ssm_status_string.argtypes = [i32]
        L.conv1d_causal.restype = i32
        L.conv1d_causal.argtypes = [ctypes.POINTER(ssm_conv_desc)] + [p] * 7
        L.ssm_scan_fwd_workspace_size.restype = i32
        L.ssm_scan_fwd_workspace_size.argtypes = [ctypes.POINTER(ssm_scan_desc), ctypes.POINTER(sz)]
        L.ssm_scan_fwd.restype = i32
        L.ssm_scan_fwd.argtypes = [ctypes.POINTER(ssm_scan_desc)] + [p] * 16 + [sz, p]
        L.ssm_scan_fwd_static.restype = i32
        L.ssm_scan_fwd_static.argtypes = [ctypes.POINTER(ssm_scan_desc)] + [p] * 16
        L.ssm_scan_bwd_workspace_size.restype = i32
        L.ssm_scan_bwd_workspace_size.argtypes = [ctypes.POINTER(ssm_scan_desc), ctypes.POINTER(sz)]
        L.ssm_scan_bwd.restype = i32
        L.ssm_scan_bwd.argtypes = [ctypes.POINTER(ssm_scan_desc)] + [p] * 27 + [sz, p]
        L.ssm_step.restype = i32
        L.ssm_step.argtypes = [ctypes.POINTER(ssm_step_desc)] + [p] * 14
        L.ssm_model_decode_workspace_size.restype = i32
        L.ssm_model_decode_workspace_size.argtypes = [ctypes.POINTER(ssm_model_desc), ctypes.POINTER(sz)]
        L.ssm_model_decode_step.restype = i32
        L.ssm_model_decode_step.argtypes = [ctypes.POINTER(ssm_model_desc), p, p, p,
                                            ctypes.POINTER(ssm_layer_weights), p, p, p, p, p, sz, p]
        _lib = L
    return _lib


def ssm_version() -> int:
    return int(lib().ssm_version())


def ssm_status_string(code: int) -> str:
    return lib().ssm_status_string(int(code)).decode()


# ----------------------------------------------------------------- marshalling
def _io_code(t):
    if t.dtype == torch.float32:
        return SSM_F32
    if t.dtype == torch.bfloat16:
        return SSM_BF16
    raise TypeError("io tensors must be float32 or bfloat16, got %s" % t.dtype)


def _ptr(t, dtype=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _check(fn, rc):
    if rc != SSM_OK:
        raise SSMError(fn, rc)


def _f32(t, name):
    return _ptr(t, torch.float32, name)


# --------------------------------------------------------------------- calls
def conv1d_causal(x, w, b=None, state_in=None, state_out=None, y=None, silu=True, stream=None):
    """y = act(causal depthwise conv(x)) for x [B, L, D] (io dtype), w [D, W].
    Returns y."""
    Bn, L, D = x.shape
    W = w.shape[1]
    io = _io_code(x)
    if y is None:
        y = torch.empty_like(x)
    desc = ssm_conv_desc(Bn, L, D, W, 1 if silu else 0, io, 0)
    _check("conv1d_causal", lib().conv1d_causal(
        ctypes.byref(desc), _ptr(x, x.dtype, "x"), _f32(w, "w"), _f32(b, "b"),
        _f32(state_in, "state_in"), _f32(state_out, "state_out"), _ptr(y, x.dtype, "y"),
        _stream(stream)))
    return y


def _scan_desc(x, N, conv_width, disc, chunk_len):
    Bn, L, D = x.shape
    return ssm_scan_desc(Bn, L, D, N, conv_width, _io_code(x), disc, chunk_len)


def ssm_scan_fwd_workspace_size(desc) -> int:
    n = ctypes.c_size_t(0)
    _check("ssm_scan_fwd_workspace_size", lib().ssm_scan_fwd_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return int(n.value)


def ssm_scan_bwd_workspace_size(desc) -> int:
    n = ctypes.c_size_t(0)
    _check("ssm_scan_bwd_workspace_size", lib().ssm_scan_bwd_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return int(n.value)


def _workspace(nbytes, given, device):
    if nbytes == 0:
        return given
    if given is not None:
        return given
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def ssm_scan_fwd(x, dt_raw, A_log, B, C, dt_bias=None, Dskip=None, z=None, conv_w=None, conv_b=None,
                 conv_state_in=None, conv_state_out=None, h0=None, hT=None, y=None,
                 disc=SSM_DISC_DELTA_B, chunk_len=0, workspace=None, stream=None):
    """Selective scan over x [B, L, D] (u, or the conv input when conv_w is
    given).  Writes hT / conv_state_out when passed; returns y."""
    N = A_log.shape[1]
    W = conv_w.shape[1] if conv_w is not None else 0
    desc = _scan_desc(x, N, W, disc, chunk_len)
    if y is None:
        y = torch.empty_like(x)
    ws = _workspace(ssm_scan_fwd_workspace_size(desc), workspace, x.device)
    t = x.dtype
    _check("ssm_scan_fwd", lib().ssm_scan_fwd(
        ctypes.byref(desc), _ptr(x, t, "x"), _ptr(dt_raw, t, "dt_raw"), _f32(dt_bias, "dt_bias"),
        _f32(A_log, "A_log"), _ptr(B, t, "B"), _ptr(C, t, "C"), _f32(Dskip, "Dskip"), _ptr(z, t, "z"),
        _f32(conv_w, "conv_w"), _f32(conv_b, "conv_b"), _f32(conv_state_in, "conv_state_in"),
        _f32(conv_state_out, "conv_state_out"), _f32(h0, "h0"), _f32(hT, "hT"), _ptr(y, t, "y"),
        _ptr(ws, None, "workspace"), ctypes.c_size_t(ws.numel() if ws is not None else 0),
        _stream(stream)))
    return y


def ssm_scan_fwd_static(x, dt_raw, A_log, B, C, dt_bias=None, Dskip=None, z=None, conv_w=None, conv_b=None,
                        conv_state_in=None, conv_state_out=None, h0=None, hT=None, y=None,
                        disc=SSM_DISC_DELTA_B, chunk_len=0, stream=None):
    """ssm_scan_fwd without a workspace: a time split keeps its chunk summaries
    in the library's static device buffer (SSM_STATIC_SCRATCH_BYTES per GPU).
    Allocates nothing when y is given.  Calls that overlap on one GPU race on
    that buffer.  Returns y."""
    N = A_log.shape[1]
    W = conv_w.shape[1] if conv_w is not None else 0
    desc = _scan_desc(x, N, W, disc, chunk_len)
    if y is None:
        y = torch.empty_like(x)
    t = x.dtype
    _check("ssm_scan_fwd_static", lib().ssm_scan_fwd_static(
        ctypes.byref(desc), _ptr(x, t, "x"), _ptr(dt_raw, t, "dt_raw"), _f32(dt_bias, "dt_bias"),
        _f32(A_log, "A_log"), _ptr(B, t, "B"), _ptr(C, t, "C"), _f32(Dskip, "Dskip"), _ptr(z, t, "z"),
        _f32(conv_w, "conv_w"), _f32(conv_b, "conv_b"), _f32(conv_state_in, "conv_state_in"),
        _f32(conv_state_out, "conv_state_out"), _f32(h0, "h0"), _f32(hT, "hT"), _ptr(y, t, "y"),
        _stream(stream)))
    return y


def ssm_scan_bwd(x, dt_raw, A_log, B, C, dy, dt_bias=None, Dskip=None, z=None, conv_w=None, conv_b=None,
                 conv_state_in=None, h0=None, dhT=None, disc=SSM_DISC_DELTA_B, chunk_len=0,
                 want=("dx", "d_dt_raw", "d_dt_bias", "dA_log", "dB", "dC", "dD", "dz", "dh0",
                       "dconv_w", "dconv_b", "dconv_state"),
                 out=None, workspace=None, stream=None):
    """Gradients of ssm_scan_fwd for the loss sum(y*dy) + sum(hT*dhT).
    x is u, or the conv input when conv_w is given (then dx flows through
    the conv + SiLU prologue).  Returns a dict of the requested gradients
    (allocated unless given in `out`); the conv ones only with conv_w, dz only
    with z, the dt ones not with SSM_DECAY_CONST."""
    Bn, L, D = x.shape
    N = A_log.shape[1]
    W = conv_w.shape[1] if conv_w is not None else 0
    desc = _scan_desc(x, N, W, disc, chunk_len)
    t = x.dtype
    out = dict(out or {})
    f32 = torch.float32
    shapes = dict(dx=((Bn, L, D), t), d_dt_raw=((Bn, L, D), t), d_dt_bias=((D,), f32),
                  dA_log=((D, N), f32), dB=((Bn, L, N), t), dC=((Bn, L, N), t),
                  dD=((D,), f32), dz=((Bn, L, D), t), dh0=((Bn, D, N), f32),
                  dconv_w=((D, W), f32), dconv_b=((D,), f32), dconv_state=((Bn, max(W - 1, 0), D), f32))
    for k in want:
        if k == "dz" and z is None:
            continue
        if k.startswith("dconv") and W == 0:
            continue
        if k in ("d_dt_raw", "d_dt_bias") and disc == SSM_DECAY_CONST:
            continue
        if k not in out:
            shp, dt_ = shapes[k]
            out[k] = torch.empty(shp, dtype=dt_, device=x.device)
    ws = _workspace(ssm_scan_bwd_workspace_size(desc), workspace, x.device)
    g = out.get
    _check("ssm_scan_bwd", lib().ssm_scan_bwd(
        ctypes.byref(desc), _ptr(x, t, "x"), _ptr(dt_raw, t, "dt_raw"), _f32(dt_bias, "dt_bias"),
        _f32(A_log, "A_log"), _ptr(B, t, "B"), _ptr(C, t, "C"), _f32(Dskip, "Dskip"), _ptr(z, t, "z"),
        _f32(conv_w, "conv_w"), _f32(conv_b, "conv_b"), _f32(conv_state_in, "conv_state_in"),
        _f32(h0, "h0"), _ptr(dy, t, "dy"), _f32(dhT, "dhT"), _ptr(g("dx"), t, "dx"),
        _ptr(g("d_dt_raw"), t, "d_dt_raw"), _f32(g("d_dt_bias"), "d_dt_bias"), _f32(g("dA_log"), "dA_log"),
        _ptr(g("dB"), t, "dB"), _ptr(g("dC"), t, "dC"), _f32(g("dD"), "dD"), _ptr(g("dz"), t, "dz"),
        _f32(g("dh0"), "dh0"), _f32(g("dconv_w"), "dconv_w"), _f32(g("dconv_b"), "dconv_b"),
        _f32(g("dconv_state") if W > 1 else None, "dconv_state"),
        _ptr(ws, None, "workspace"), ctypes.c_size_t(ws.numel()), _stream(stream)))
    return out


def ssm_step(h, x, dt_raw, A_log, B, C, conv_state=None, z=None, conv_w=None, conv_b=None, dt_bias=None,
             Dskip=None, y=None, disc=SSM_DISC_DELTA_B, stream=None):
    """One streaming token.  h [nblk, S, D, N] (float32, or bfloat16 for a
    bf16-stored state) and conv_state [nblk, S, W-1, D] (float32) are updated
    in place; x/dt_raw/z [nblk, S, D], B/C [nblk, S, N], per-block parameters
    with a leading [nblk] axis.  Returns y [nblk, S, D]."""
    K, S, D, N = h.shape
    W = conv_w.shape[-1] if conv_w is not None else 0
    t = x.dtype
    if h.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("h must be float32 or bfloat16, got %s" % h.dtype)
    desc = ssm_step_desc(K, S, D, N, W, _io_code(x), disc, _io_code(h))
    if y is None:
        y = torch.empty_like(x)
    _check("ssm_step", lib().ssm_step(
        ctypes.byref(desc), _ptr(h, h.dtype, "h"), _f32(conv_state, "conv_state"), _ptr(x, t, "x"),
        _ptr(dt_raw, t, "dt_raw"), _ptr(B, t, "B"), _ptr(C, t, "C"), _ptr(z, t, "z"), _f32(conv_w, "conv_w"),
        _f32(conv_b, "conv_b"), _f32(dt_bias, "dt_bias"), _f32(A_log, "A_log"), _f32(Dskip, "Dskip"),
        _ptr(y, t, "y"), _stream(stream)))
    return y


def model_desc(cfg, S) -> ssm_model_desc:
    """Descriptor of a model with shape cfg (keys vocab, d_model, n_layers,
    d_inner, d_state, dt_rank, conv_width) decoding S streams."""
    return ssm_model_desc(S, cfg["vocab"], cfg["d_model"], cfg["n_layers"], cfg["d_inner"], cfg["d_state"],
                          cfg["dt_rank"], cfg["conv_width"], 0)


def ssm_model_decode_workspace_size(desc) -> int:
    n = ctypes.c_size_t(0)
    _check("ssm_model_decode_workspace_size",
           lib().ssm_model_decode_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return int(n.value)


class ModelLayers:
    """The host array of per-block weight pointers for ssm_model_decode_step,
    built once from device tensors (keys LAYER_FIELDS) and kept with them."""

    def __init__(self, layers):
        self.tensors = [dict(lay) for lay in layers]
        arr = (ssm_layer_weights * len(layers))()
        for i, lay in enumerate(self.tensors):
            for f in LAYER_FIELDS:
                t = lay.get(f)
                setattr(arr[i], f, None if t is None else _f32(t, f).value)
        self.array = arr


def ssm_model_decode_step(desc, emb, layers, tokens, h, conv_state, logits=None, norm_f_w=None, norm_f_b=None,
                          workspace=None, stream=None):
    """One token for every stream through the whole model.  layers is a
    ModelLayers; tokens int32 [S] on the device; h [n_layers, S, d_inner, N]
    and conv_state [n_layers, S, W-1, d_inner] (float32) are updated in place.
    Returns logits [S, vocab]."""
    S, V = desc.nstreams, desc.vocab
    if logits is None:
        logits = torch.empty(S, V, device=tokens.device, dtype=torch.float32)
    ws = workspace
    if ws is None:
        ws = torch.empty(ssm_model_decode_workspace_size(desc), dtype=torch.uint8, device=tokens.device)
    _check("ssm_model_decode_step", lib().ssm_model_decode_step(
        ctypes.byref(desc), _f32(emb, "emb"), _f32(norm_f_w, "norm_f_w"), _f32(norm_f_b, "norm_f_b"),
        layers.array, _ptr(tokens, torch.int32, "tokens"), _f32(h, "h"), _f32(conv_state, "conv_state"),
        _f32(logits, "logits"), _ptr(ws, None, "workspace"), ctypes.c_size_t(ws.numel()), _stream(stream)))
    return logits
