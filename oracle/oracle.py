"""ctypes wrapper around the fp64 C oracle (``la_oracle.c``).

Test infrastructure only.  Inputs are converted to float64 exactly (fp32 and
bf16 values are representable in fp64), so the oracle sees the very values the
device sees.  All arrays use the row-major layouts [B, H, N, d] (sequences),
[B, H, d_k, d_v] (state S) and [B, H, d_k] (normaliser z).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "la_oracle.c")
_LIB = os.path.join(_HERE, "liblaoracle.so")
_lib = None


def library_path() -> str:
    return _LIB


def build(force: bool = True) -> str:
    """Compile la_oracle.c with gcc (OpenMP over (batch, head) pairs)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _bind(path: str):
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(ctypes.c_double)
    i = ctypes.c_int
    lib.oracle_fwd_causal_f64.argtypes = [P, P, P, P, P, i, i, i, i, i]
    lib.oracle_fwd_noncausal_f64.argtypes = [P, P, P, P, i, i, i, i, i]
    lib.oracle_decode_step_f64.argtypes = [P, P, P, P, P, P, i, i, i, i]
    lib.oracle_bwd_causal_f64.argtypes = [P, P, P, P, P, P, P, i, i, i, i, i]
    lib.oracle_bwd_noncausal_f64.argtypes = [P, P, P, P, P, P, P, i, i, i, i, i]
    lib.oracle_fwd_causal_decay_f64.argtypes = [P, P, P, P, P, P, i, i, i, i, i]
    lib.oracle_decode_step_decay_f64.argtypes = [P, P, P, P, P, P, P, i, i, i, i]
    lib.oracle_bwd_causal_decay_f64.argtypes = [P, P, P, P, P, P, P, P, i, i, i, i, i]
    lib.oracle_fm_features_f64.argtypes = [P, i, P, i, P, i, i, i, i]
    lib.oracle_fwd_causal_fm_f64.argtypes = [P, P, P, i, P, i, P, P, i, i, i, i, i]
    lib.oracle_fwd_noncausal_fm_f64.argtypes = [P, P, P, i, P, i, P, i, i, i, i, i]
    lib.oracle_decode_step_fm_f64.argtypes = [P, P, P, P, P, i, P, i, P, i, i, i, i]
    lib.oracle_bwd_causal_fm_f64.argtypes = [P, P, P, P, i, P, i, P, P, P, i, i, i, i, i]
    lib.oracle_num_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        _lib = _bind(_LIB)
    return _lib


def _f64(x) -> np.ndarray:
    """Exact conversion to a C-contiguous float64 array (torch or numpy)."""
    if hasattr(x, "detach"):  # torch tensor: go through float64 on the CPU
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def fwd_causal(q, k, v, lib=None):
    """Causal forward.  q, k: [B,H,N,dk]; v: [B,H,N,dv] -> (out [B,H,N,dv], den [B,H,N])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and v.shape[:3] == (B, H, N)
    o = np.empty((B, H, N, dv))
    den = np.empty((B, H, N))
    (lib or _load()).oracle_fwd_causal_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(den), B, H, N, dk, dv)
    return o, den


def fwd_noncausal(q, k, v, lib=None):
    """Non-causal forward.  q, k: [B,H,N,dk]; v: [B,H,N,dv] -> out [B,H,N,dv]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and v.shape[:3] == (B, H, N)
    o = np.empty((B, H, N, dv))
    (lib or _load()).oracle_fwd_noncausal_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, N, dk, dv)
    return o


def decode_step(S, z, q, k, v, lib=None):
    """One decode step.  Returns (S_new, z_new, out); the inputs are not modified.

    S: [B,H,dk,dv], z: [B,H,dk], q, k: [B,H,dk], v: [B,H,dv].
    """
    S = _f64(S).copy()
    z = _f64(z).copy()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, dk, dv = S.shape
    assert z.shape == (B, H, dk) and q.shape == (B, H, dk) and k.shape == (B, H, dk)
    assert v.shape == (B, H, dv)
    o = np.empty((B, H, dv))
    (lib or _load()).oracle_decode_step_f64(_ptr(S), _ptr(z), _ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, dk, dv)
    return S, z, o


def bwd_causal(q, k, v, dout, lib=None):
    """Exact gradient of the causal forward: returns (dq, dk, dv)."""
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    assert g.shape == v.shape
    dq = np.empty_like(q)
    dkk = np.empty_like(k)
    dvv = np.empty_like(v)
    (lib or _load()).oracle_bwd_causal_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(dq), _ptr(dkk), _ptr(dvv),
                                  B, H, N, dk, dv)
    return dq, dkk, dvv


def bwd_noncausal(q, k, v, dout, lib=None):
    """Exact gradient of the non-causal forward: returns (dq, dk, dv)."""
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    assert g.shape == v.shape
    dq = np.empty_like(q)
    dkk = np.empty_like(k)
    dvv = np.empty_like(v)
    (lib or _load()).oracle_bwd_noncausal_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(dq), _ptr(dkk), _ptr(dvv),
                                     B, H, N, dk, dv)
    return dq, dkk, dvv


def fwd_causal_decay(q, k, v, gamma, lib=None):
    """Causal forward with a fixed decay gamma[h] per head.  Returns (out, den)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    g = _f64(np.asarray(gamma, dtype=np.float64).reshape(-1))
    assert k.shape == q.shape and v.shape[:3] == (B, H, N) and g.shape == (H,)
    o = np.empty((B, H, N, dv))
    den = np.empty((B, H, N))
    (lib or _load()).oracle_fwd_causal_decay_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(o), _ptr(den),
                                        B, H, N, dk, dv)
    return o, den


def decode_step_decay(S, z, q, k, v, gamma, lib=None):
    """One decode step with a fixed decay gamma[h] per head.  Returns (S_new, z_new, out)."""
    S = _f64(S).copy()
    z = _f64(z).copy()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, dk, dv = S.shape
    g = _f64(np.asarray(gamma, dtype=np.float64).reshape(-1))
    assert z.shape == (B, H, dk) and q.shape == (B, H, dk) and k.shape == (B, H, dk)
    assert v.shape == (B, H, dv) and g.shape == (H,)
    o = np.empty((B, H, dv))
    (lib or _load()).oracle_decode_step_decay_f64(_ptr(S), _ptr(z), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(o),
                                         B, H, dk, dv)
    return S, z, o


def bwd_causal_decay(q, k, v, dout, gamma, lib=None):
    """Exact gradient of the causal forward with a fixed decay gamma[h] per head: (dq, dk, dv)."""
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    gm = _f64(np.asarray(gamma, dtype=np.float64).reshape(-1))
    assert g.shape == v.shape and gm.shape == (H,)
    dq = np.empty_like(q)
    dkk = np.empty_like(k)
    dvv = np.empty_like(v)
    (lib or _load()).oracle_bwd_causal_decay_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(gm), _ptr(dq), _ptr(dkk),
                                        _ptr(dvv), B, H, N, dk, dv)
    return dq, dkk, dvv


def load_variant(path: str):
    """Bind another build of the oracle source (used by the tests that plant
    mistakes in a copy of la_oracle.c to check that the pins catch them)."""
    return _bind(path)


def source_path() -> str:
    return _SRC


# ---------------------------------------------------------------------------
# Pluggable feature map: "elu1" (phi = elu + 1), "identity" (phi(x) = x) and
# "prf" (positive random features phi(x)_r = exp(w_r . x - |x|^2/2) / sqrt(m),
# W [H, m, d_k], one set of m directions per head).
# ---------------------------------------------------------------------------
FEATURE_MAPS = {"elu1": 0, "identity": 1, "prf": 2}


def _fm(kind, W, H, dk):
    code = FEATURE_MAPS[kind]
    if code == 2:
        W = _f64(W)
        assert W.ndim == 3 and W.shape[0] == H and W.shape[2] == dk, W.shape
        return code, W, W.shape[1]
    return code, np.zeros(1), dk


def features(x, kind, W=None, lib=None):
    """The feature map of every row of x [B,H,N,dk] -> [B,H,N,m]."""
    x = _f64(x)
    B, H, N, dk = x.shape
    code, Wa, m = _fm(kind, W, H, dk)
    out = np.empty((B, H, N, m))
    (lib or _load()).oracle_fm_features_f64(_ptr(x), code, _ptr(Wa), m, _ptr(out), B, H, N, dk)
    return out


def fwd_causal_fm(q, k, v, kind, W=None, lib=None):
    """Causal forward with a feature map: (out [B,H,N,dv], den [B,H,N])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    code, Wa, m = _fm(kind, W, H, dk)
    o = np.empty((B, H, N, dv))
    den = np.empty((B, H, N))
    (lib or _load()).oracle_fwd_causal_fm_f64(_ptr(q), _ptr(k), _ptr(v), code, _ptr(Wa), m, _ptr(o), _ptr(den),
                                             B, H, N, dk, dv)
    return o, den


def fwd_noncausal_fm(q, k, v, kind, W=None, lib=None):
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    code, Wa, m = _fm(kind, W, H, dk)
    o = np.empty((B, H, N, dv))
    (lib or _load()).oracle_fwd_noncausal_fm_f64(_ptr(q), _ptr(k), _ptr(v), code, _ptr(Wa), m, _ptr(o),
                                                B, H, N, dk, dv)
    return o


def decode_step_fm(S, z, q, k, v, kind, W=None, lib=None):
    """One decode step with a feature map.  S: [B,H,m,dv], z: [B,H,m]; returns (S, z, out)."""
    S = _f64(S).copy()
    z = _f64(z).copy()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, dk = q.shape
    dv = v.shape[-1]
    code, Wa, m = _fm(kind, W, H, dk)
    assert S.shape == (B, H, m, dv) and z.shape == (B, H, m)
    o = np.empty((B, H, dv))
    (lib or _load()).oracle_decode_step_fm_f64(_ptr(S), _ptr(z), _ptr(q), _ptr(k), _ptr(v), code, _ptr(Wa), m,
                                              _ptr(o), B, H, dk, dv)
    return S, z, o


def bwd_causal_fm(q, k, v, dout, kind, W=None, lib=None):
    """Exact gradient of the causal forward with a feature map: (dq, dk, dv)."""
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    code, Wa, m = _fm(kind, W, H, dk)
    dq = np.empty_like(q)
    dkk = np.empty_like(k)
    dvv = np.empty_like(v)
    (lib or _load()).oracle_bwd_causal_fm_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(g), code, _ptr(Wa), m, _ptr(dq),
                                             _ptr(dkk), _ptr(dvv), B, H, N, dk, dv)
    return dq, dkk, dvv
