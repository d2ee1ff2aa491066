"""Float64 CPU oracle of the S6 selective scan (test infrastructure only).

This package is the correctness reference that the GPU library is checked
against.  Only the tests, the smoke check and the benchmark's CPU-baseline leg
may import it; the product path never does, and it shares no code with the HIP
library.  The arithmetic lives in ``ssm_oracle.c`` (plain sequential float64
loops); this module only builds that file with gcc, converts arrays to
contiguous float64 and calls it through ctypes.

Each wrapper names the routine it calls; the routine's header comment in
``ssm_oracle.c`` cites the passage of the pages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssm_oracle.c")
_LIB = os.environ.get("SSM_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

DISC_DELTA_B = 0
DISC_ZOH = 1
# Constant decay source: a = exp(-exp(A_log)) per (channel, state), write B*u,
# no step size (dt_raw and dt_bias are not read and may be None).
DECAY_CONST = 2

_lib = None


def build(force: bool = True) -> str:
    """Compile ssm_oracle.c into liboracle.so with gcc -O2 (no fast-math)."""
    global _lib
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
        _lib = None
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        i64, i32, p = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
        lib.orc_num_threads.restype = ctypes.c_int
        lib.orc_set_num_threads.argtypes = [ctypes.c_int]
        lib.orc_set_num_threads.restype = None
        lib.orc_conv1d_causal.argtypes = [i64, i64, i64, i32, p, p, p, p, p, i32, p]
        lib.orc_conv1d_causal_bwd.argtypes = [i64, i64, i64, i32, p, p, p, p, i32, p, p, p, p, p]
        lib.orc_scan_core.argtypes = [i64, i64, i64, i64, i32] + [p] * 13
        lib.orc_delta.argtypes = [i64, i64, i64, p, p, p]
        lib.orc_scan_fwd.argtypes = [i64, i64, i64, i64, i32] + [p] * 12
        lib.orc_scan_bwd.argtypes = [i64, i64, i64, i64, i32] + [p] * 21
        lib.orc_step.argtypes = [i64, i64, i64, i32, i32] + [p] * 13 + [i32]
        lib.orc_round_bf16_value.argtypes = [ctypes.c_double]
        lib.orc_round_bf16_value.restype = ctypes.c_double
        for f in (lib.orc_conv1d_causal, lib.orc_conv1d_causal_bwd, lib.orc_scan_core, lib.orc_delta,
                  lib.orc_scan_fwd, lib.orc_scan_bwd, lib.orc_step):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().orc_num_threads())


def set_num_threads(n: int) -> None:
    """Threads used by the following oracle calls."""
    _load().orc_set_num_threads(int(n))


def _f64(a):
    """Contiguous float64 copy (exact widening of fp32 / bf16 values)."""
    if a is None:
        return None
    if hasattr(a, "detach"):  # a CPU torch tensor
        a = a.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, name):
    if rc != 0:
        raise RuntimeError("oracle %s failed with code %d" % (name, rc))


def conv1d_causal(x, w, bias=None, state_in=None, silu=True, want_state=True):
    """orc_conv1d_causal: x [B,L,D], w [D,W] -> (y [B,L,D], state_out [B,W-1,D])."""
    x, w, bias, state_in = _f64(x), _f64(w), _f64(bias), _f64(state_in)
    Bn, L, D = x.shape
    W = w.shape[1]
    y = np.empty((Bn, L, D))
    so = np.empty((Bn, W - 1, D)) if want_state else None
    _check(_load().orc_conv1d_causal(Bn, L, D, W, _ptr(x), _ptr(w), _ptr(bias),
                                     _ptr(state_in), _ptr(so), int(bool(silu)),
                                     _ptr(y)), "conv1d_causal")
    return y, so


def conv1d_causal_bwd(x, w, dy, bias=None, state_in=None, silu=True):
    """orc_conv1d_causal_bwd: gradients of conv1d_causal's output (given
    dy [B,L,D]) w.r.t. x, w [D,W], bias [D] and the history [B,W-1,D]."""
    x, w, dy, bias, state_in = _f64(x), _f64(w), _f64(dy), _f64(bias), _f64(state_in)
    Bn, L, D = x.shape
    W = w.shape[1]
    dx = np.empty((Bn, L, D))
    dw = np.empty((D, W))
    db = np.empty(D)
    ds = np.empty((Bn, W - 1, D))
    _check(_load().orc_conv1d_causal_bwd(Bn, L, D, W, _ptr(x), _ptr(w), _ptr(bias), _ptr(state_in),
                                         int(bool(silu)), _ptr(dy), _ptr(dx), _ptr(dw), _ptr(db),
                                         _ptr(ds)), "conv1d_causal_bwd")
    return {"dx": dx, "dw": dw, "db": db, "dstate": ds}


def delta(dt_raw, dt_bias=None):
    """orc_delta: softplus(dt_raw + dt_bias), [B,L,D]."""
    dt_raw, dt_bias = _f64(dt_raw), _f64(dt_bias)
    Bn, L, D = dt_raw.shape
    out = np.empty_like(dt_raw)
    _check(_load().orc_delta(Bn, L, D, _ptr(dt_raw), _ptr(dt_bias), _ptr(out)), "delta")
    return out


def scan_core(u, delta_, A_log, Bm, Cm, Dskip=None, z=None, h0=None,
              disc=DISC_DELTA_B, trace=False):
    """orc_scan_core: the recurrence given dt.  Returns (y, hT) or, with
    trace=True, (y, hT, a, write, h) where the traces are [B,L,D,N]."""
    u, delta_, A_log = _f64(u), _f64(delta_), _f64(A_log)
    Bm, Cm, Dskip, z, h0 = _f64(Bm), _f64(Cm), _f64(Dskip), _f64(z), _f64(h0)
    Bn, L, D = u.shape
    N = A_log.shape[1]
    y = np.empty((Bn, L, D))
    hT = np.empty((Bn, D, N))
    ta = tw = th = None
    if trace:
        ta, tw, th = (np.empty((Bn, L, D, N)) for _ in range(3))
    _check(_load().orc_scan_core(Bn, L, D, N, int(disc), _ptr(u), _ptr(delta_),
                                 _ptr(A_log), _ptr(Bm), _ptr(Cm), _ptr(Dskip),
                                 _ptr(z), _ptr(h0), _ptr(hT), _ptr(y),
                                 _ptr(ta), _ptr(tw), _ptr(th)), "scan_core")
    return (y, hT, ta, tw, th) if trace else (y, hT)


def scan_fwd(u, dt_raw, A_log, Bm, Cm, dt_bias=None, Dskip=None, z=None,
             h0=None, disc=DISC_DELTA_B):
    """orc_scan_fwd: dt = softplus(dt_raw + dt_bias), then the scan (with
    disc=DECAY_CONST there is no dt and dt_raw may be None).
    Returns (y [B,L,D], hT [B,D,N])."""
    u, dt_raw, A_log = _f64(u), _f64(dt_raw), _f64(A_log)
    Bm, Cm, dt_bias, Dskip = _f64(Bm), _f64(Cm), _f64(dt_bias), _f64(Dskip)
    z, h0 = _f64(z), _f64(h0)
    Bn, L, D = u.shape
    N = A_log.shape[1]
    y = np.empty((Bn, L, D))
    hT = np.empty((Bn, D, N))
    _check(_load().orc_scan_fwd(Bn, L, D, N, int(disc), _ptr(u), _ptr(dt_raw),
                                _ptr(dt_bias), _ptr(A_log), _ptr(Bm), _ptr(Cm),
                                _ptr(Dskip), _ptr(z), _ptr(h0), _ptr(hT),
                                _ptr(y), None), "scan_fwd")
    return y, hT


def scan_bwd(u, dt_raw, A_log, Bm, Cm, dy, dt_bias=None, Dskip=None, z=None,
             h0=None, dhT=None, disc=DISC_DELTA_B):
    """orc_scan_bwd: gradients of scan_fwd's y (and hT) w.r.t. its inputs.
    Returns a dict with du, d_dt_raw, d_delta, d_dt_bias, dA_log, dB, dC,
    dD, dz (None without z) and dh0 (the dt gradients are zeros with
    disc=DECAY_CONST, where dt_raw may be None)."""
    u, dt_raw, A_log = _f64(u), _f64(dt_raw), _f64(A_log)
    Bm, Cm, dy = _f64(Bm), _f64(Cm), _f64(dy)
    dt_bias, Dskip, z, h0, dhT = _f64(dt_bias), _f64(Dskip), _f64(z), _f64(h0), _f64(dhT)
    Bn, L, D = u.shape
    N = A_log.shape[1]
    out = dict(du=np.empty((Bn, L, D)), d_dt_raw=np.empty((Bn, L, D)),
               d_delta=np.empty((Bn, L, D)), d_dt_bias=np.empty(D),
               dA_log=np.empty((D, N)), dB=np.empty((Bn, L, N)),
               dC=np.empty((Bn, L, N)), dD=np.empty(D),
               dz=np.empty((Bn, L, D)) if z is not None else None,
               dh0=np.empty((Bn, D, N)))
    _check(_load().orc_scan_bwd(
        Bn, L, D, N, int(disc), _ptr(u), _ptr(dt_raw), _ptr(dt_bias), _ptr(A_log),
        _ptr(Bm), _ptr(Cm), _ptr(Dskip), _ptr(z), _ptr(h0), _ptr(dy), _ptr(dhT),
        _ptr(out["du"]), _ptr(out["d_dt_raw"]), _ptr(out["d_delta"]),
        _ptr(out["d_dt_bias"]), _ptr(out["dA_log"]), _ptr(out["dB"]),
        _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["dz"]), _ptr(out["dh0"])),
        "scan_bwd")
    return out


def round_bf16(x):
    """orc_round_bf16_value: the nearest bfloat16 value of a float64, elementwise."""
    f = _load().orc_round_bf16_value
    a = np.asarray(x, dtype=np.float64)
    return np.vectorize(f, otypes=[np.float64])(a) if a.size else a.copy()


def step(h, conv_state, x, dt_raw, Bm, Cm, A_log, z=None, conv_w=None,
         conv_b=None, dt_bias=None, Dskip=None, disc=DISC_DELTA_B, state_bf16=False):
    """orc_step: one streaming token for S streams.  h [S,D,N] and conv_state
    [S,W-1,D] are float64 numpy arrays updated in place; returns y [S,D].
    With state_bf16 the kept state is rounded to bfloat16 after the update
    (y reads the unrounded update)."""
    assert isinstance(h, np.ndarray) and h.dtype == np.float64 and h.flags.c_contiguous
    if conv_state is not None:
        assert conv_state.dtype == np.float64 and conv_state.flags.c_contiguous
    x, dt_raw, Bm, Cm, A_log = _f64(x), _f64(dt_raw), _f64(Bm), _f64(Cm), _f64(A_log)
    z, conv_w, conv_b = _f64(z), _f64(conv_w), _f64(conv_b)
    dt_bias, Dskip = _f64(dt_bias), _f64(Dskip)
    S, D = x.shape
    N = A_log.shape[1]
    W = conv_w.shape[1] if conv_w is not None else 0
    y = np.empty((S, D))
    _check(_load().orc_step(S, D, N, W, int(disc), _ptr(h), _ptr(conv_state),
                            _ptr(x), _ptr(dt_raw), _ptr(Bm), _ptr(Cm), _ptr(z),
                            _ptr(conv_w), _ptr(conv_b), _ptr(dt_bias),
                            _ptr(A_log), _ptr(Dskip), _ptr(y), int(bool(state_bf16))), "step")
    return y
