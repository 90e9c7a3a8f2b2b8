"""Python entry points with the names of the C ABI (include/la.h).

Argument marshalling only: tensors are checked (device, dtype, shape,
contiguity), outputs and workspace are allocated with torch when the caller
does not pass them, and the raw pointers plus the current HIP stream go to
liblinattn.so.  Layouts: q, k [B, H, N, d_k]; v, o [B, H, N, d_v]; den
[B, H, N] fp32; S [B, H, d_k, d_v] and z [B, H, d_k] fp32.
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import _lib

_DT = {torch.float32: _lib.LA_F32, torch.bfloat16: _lib.LA_BF16}


def _code(t: torch.Tensor) -> int:
    try:
        return _DT[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16") from None


def _dev(*ts: torch.Tensor) -> torch.device:
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU (there is no CPU path)")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("tensors must be on one device")
    return dev


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(dev: torch.device, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ws(nbytes: int, dev: torch.device, ws: Optional[torch.Tensor]) -> Tuple[Optional[int], int]:
    if nbytes == 0 and ws is None:
        return None, 0
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    return ws.data_ptr(), ws.numel() * ws.element_size()


def la_status_string(code: int) -> str:
    return _lib.status_string(code)


def la_fwd_causal_workspace_bytes(B: int, H: int, N: int, d_k: int, d_v: int, C: int) -> int:
    return int(_lib.load().la_fwd_causal_workspace_bytes(B, H, N, d_k, d_v, C))


def la_fwd_noncausal_workspace_bytes(B: int, H: int, N: int, d_k: int, d_v: int) -> int:
    return int(_lib.load().la_fwd_noncausal_workspace_bytes(B, H, N, d_k, d_v))


def la_bwd_causal_workspace_bytes(B: int, H: int, N: int, d_k: int, d_v: int, C: int) -> int:
    return int(_lib.load().la_bwd_causal_workspace_bytes(B, H, N, d_k, d_v, C))


def la_bwd_noncausal_workspace_bytes(B: int, H: int, N: int, d_k: int, d_v: int) -> int:
    return int(_lib.load().la_bwd_noncausal_workspace_bytes(B, H, N, d_k, d_v))


def _shapes(q, k, v):
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError(f"expected q, k [B,H,N,d_k] and v [B,H,N,d_v]; got {tuple(q.shape)}, "
                         f"{tuple(k.shape)}, {tuple(v.shape)}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share one dtype")
    B, H, N, dk = q.shape
    return B, H, N, dk, v.shape[3]


def la_fwd_causal_state(q, k, v, o=None, den=None, S0=None, z0=None, S_out=None, z_out=None,
                        C: int = 64, out_dtype=None, ws=None, stream=None, want_den: bool = True):
    """Causal forward with an optional carried state.  Returns (o, den)."""
    B, H, N, dk, dv = _shapes(q, k, v)
    dev = _dev(q, k, v, o, den, S0, z0, S_out, z_out, ws)
    if o is None:
        o = torch.empty((B, H, N, dv), dtype=out_dtype or q.dtype, device=dev)
    if den is None and want_den:
        den = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    for t, shp in ((o, (B, H, N, dv)), (den, (B, H, N)), (S0, (B, H, dk, dv)), (z0, (B, H, dk)),
                   (S_out, (B, H, dk, dv)), (z_out, (B, H, dk))):
        if t is not None and tuple(t.shape) != shp:
            raise ValueError(f"expected shape {shp}, got {tuple(t.shape)}")
    for t in (den, S0, z0, S_out, z_out):
        if t is not None and t.dtype != torch.float32:
            raise TypeError("den, S and z are float32")
    _dev(o, den)
    wp, wb = _ws(la_fwd_causal_workspace_bytes(B, H, N, dk, dv, C), dev, ws)
    rc = _lib.load().la_fwd_causal_state(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(den), _ptr(S0), _ptr(z0), _ptr(S_out), _ptr(z_out),
        B, H, N, dk, dv, C, _code(q), _code(o), wp, wb, _stream(dev, stream))
    _lib.check(rc, "la_fwd_causal_state")
    return o, den


def la_fwd_causal_decay(q, k, v, gamma, o=None, den=None, S0=None, z0=None, S_out=None, z_out=None,
                        C: int = 64, out_dtype=None, ws=None, stream=None, want_den: bool = True):
    """Causal forward with a fixed decay gamma[h] per head (float32 [H] on the
    device, values in [0, 1]) and an optional carried state.  Returns (o, den)."""
    B, H, N, dk, dv = _shapes(q, k, v)
    dev = _dev(q, k, v, o, den, S0, z0, S_out, z_out, ws)
    _gamma(gamma, H, dev)
    if o is None:
        o = torch.empty((B, H, N, dv), dtype=out_dtype or q.dtype, device=dev)
    if den is None and want_den:
        den = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    for t, shp in ((o, (B, H, N, dv)), (den, (B, H, N)), (S0, (B, H, dk, dv)), (z0, (B, H, dk)),
                   (S_out, (B, H, dk, dv)), (z_out, (B, H, dk))):
        if t is not None and tuple(t.shape) != shp:
            raise ValueError(f"expected shape {shp}, got {tuple(t.shape)}")
    for t in (den, S0, z0, S_out, z_out):
        if t is not None and t.dtype != torch.float32:
            raise TypeError("den, S and z are float32")
    _dev(o, den)
    wp, wb = _ws(la_fwd_causal_workspace_bytes(B, H, N, dk, dv, C), dev, ws)
    rc = _lib.load().la_fwd_causal_decay(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(den), _ptr(S0), _ptr(z0), _ptr(S_out), _ptr(z_out), _ptr(gamma),
        B, H, N, dk, dv, C, _code(q), _code(o), wp, wb, _stream(dev, stream))
    _lib.check(rc, "la_fwd_causal_decay")
    return o, den


def la_fwd_causal(q, k, v, o=None, den=None, C: int = 64, out_dtype=None, ws=None, stream=None,
                  want_den: bool = True):
    """Causal forward.  Returns (o, den) (den is None when want_den is False and none is given)."""
    B, H, N, dk, dv = _shapes(q, k, v)
    dev = _dev(q, k, v, o, den, ws)
    if o is None:
        o = torch.empty((B, H, N, dv), dtype=out_dtype or q.dtype, device=dev)
    if den is None and want_den:
        den = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    if tuple(o.shape) != (B, H, N, dv) or (den is not None and tuple(den.shape) != (B, H, N)):
        raise ValueError("o must be [B,H,N,d_v] and den [B,H,N]")
    if den is not None and den.dtype != torch.float32:
        raise TypeError("den is float32")
    _dev(o, den)
    wp, wb = _ws(la_fwd_causal_workspace_bytes(B, H, N, dk, dv, C), dev, ws)
    rc = _lib.load().la_fwd_causal(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(den), B, H, N, dk, dv, C,
                                   _code(q), _code(o), wp, wb, _stream(dev, stream))
    _lib.check(rc, "la_fwd_causal")
    return o, den


def la_fwd_causal_noalloc(q, k, v, o, den=None, C: int = 64, stream=None):
    """Causal forward into caller-given o (and den), with no workspace: the
    library's own device array holds the segment states.  Allocates nothing.
    Returns (o, den)."""
    B, H, N, dk, dv = _shapes(q, k, v)
    dev = _dev(q, k, v, o, den)
    if tuple(o.shape) != (B, H, N, dv) or (den is not None and tuple(den.shape) != (B, H, N)):
        raise ValueError("o must be [B,H,N,d_v] and den [B,H,N]")
    if den is not None and den.dtype != torch.float32:
        raise TypeError("den is float32")
    rc = _lib.load().la_fwd_causal_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(den), B, H, N, dk, dv, C,
                                           _code(q), _code(o), _stream(dev, stream))
    _lib.check(rc, "la_fwd_causal_noalloc")
    return o, den


def la_fwd_noncausal(q, k, v, o=None, out_dtype=None, ws=None, stream=None):
    """Non-causal forward.  Returns o."""
    B, H, N, dk, dv = _shapes(q, k, v)
    dev = _dev(q, k, v, o, ws)
    if o is None:
        o = torch.empty((B, H, N, dv), dtype=out_dtype or q.dtype, device=dev)
    if tuple(o.shape) != (B, H, N, dv):
        raise ValueError("o must be [B,H,N,d_v]")
    _dev(o)
    wp, wb = _ws(la_fwd_noncausal_workspace_bytes(B, H, N, dk, dv), dev, ws)
    rc = _lib.load().la_fwd_noncausal(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, N, dk, dv,
                                      _code(q), _code(o), wp, wb, _stream(dev, stream))
    _lib.check(rc, "la_fwd_noncausal")
    return o


def la_bwd_causal(q, k, v, dO, dq=None, dk=None, dv=None, C: int = 64, ws=None, stream=None):
    """Cumulative-sum backward of the causal forward.  Returns (dq, dk, dv) in the dtype of q."""
    B, H, N, d_k, d_v = _shapes(q, k, v)
    dev = _dev(q, k, v, dO, dq, dk, dv, ws)
    if tuple(dO.shape) != (B, H, N, d_v) or dO.dtype != q.dtype:
        raise ValueError("dO must be [B,H,N,d_v] in the dtype of q")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, ref in ((dq, q), (dk, k), (dv, v)):
        if t.shape != ref.shape or t.dtype != ref.dtype:
            raise ValueError("dq, dk, dv must match q, k, v in shape and dtype")
    _dev(dq, dk, dv)
    wp, wb = _ws(la_bwd_causal_workspace_bytes(B, H, N, d_k, d_v, C), dev, ws)
    rc = _lib.load().la_bwd_causal(_ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(dq), _ptr(dk), _ptr(dv),
                                   B, H, N, d_k, d_v, C, _code(q), wp, wb, _stream(dev, stream))
    _lib.check(rc, "la_bwd_causal")
    return dq, dk, dv


def la_bwd_causal_decay(q, k, v, dO, gamma, dq=None, dk=None, dv=None, C: int = 64, ws=None, stream=None):
    """Backward of la_fwd_causal_decay (per-head decay gamma, float32 [H] on the
    device).  Returns (dq, dk, dv) in the dtype of q."""
    B, H, N, d_k, d_v = _shapes(q, k, v)
    dev = _dev(q, k, v, dO, dq, dk, dv, ws)
    _gamma(gamma, H, dev)
    if tuple(dO.shape) != (B, H, N, d_v) or dO.dtype != q.dtype:
        raise ValueError("dO must be [B,H,N,d_v] in the dtype of q")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, ref in ((dq, q), (dk, k), (dv, v)):
        if t.shape != ref.shape or t.dtype != ref.dtype:
            raise ValueError("dq, dk, dv must match q, k, v in shape and dtype")
    _dev(dq, dk, dv)
    wp, wb = _ws(la_bwd_causal_workspace_bytes(B, H, N, d_k, d_v, C), dev, ws)
    rc = _lib.load().la_bwd_causal_decay(_ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(dq), _ptr(dk), _ptr(dv),
                                         _ptr(gamma), B, H, N, d_k, d_v, C, _code(q), wp, wb, _stream(dev, stream))
    _lib.check(rc, "la_bwd_causal_decay")
    return dq, dk, dv


def la_bwd_noncausal(q, k, v, dO, dq=None, dk=None, dv=None, ws=None, stream=None):
    """Backward of the non-causal forward.  Returns (dq, dk, dv) in the dtype of q."""
    B, H, N, d_k, d_v = _shapes(q, k, v)
    dev = _dev(q, k, v, dO, dq, dk, dv, ws)
    if tuple(dO.shape) != (B, H, N, d_v) or dO.dtype != q.dtype:
        raise ValueError("dO must be [B,H,N,d_v] in the dtype of q")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, ref in ((dq, q), (dk, k), (dv, v)):
        if t.shape != ref.shape or t.dtype != ref.dtype:
            raise ValueError("dq, dk, dv must match q, k, v in shape and dtype")
    _dev(dq, dk, dv)
    wp, wb = _ws(la_bwd_noncausal_workspace_bytes(B, H, N, d_k, d_v), dev, ws)
    rc = _lib.load().la_bwd_noncausal(_ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(dq), _ptr(dk), _ptr(dv),
                                      B, H, N, d_k, d_v, _code(q), wp, wb, _stream(dev, stream))
    _lib.check(rc, "la_bwd_noncausal")
    return dq, dk, dv


def la_decode_step(S, z, q, k, v, o=None, stream=None):
    """One decode step, updating S [B,H,d_k,d_v] and z [B,H,d_k] in place.  Returns o [B,H,d_v]."""
    if S.dim() != 4 or z.dim() != 3 or S.dtype != torch.float32 or z.dtype != torch.float32:
        raise ValueError("S must be float32 [B,H,d_k,d_v] and z float32 [B,H,d_k]")
    B, H, dk, dvv = S.shape
    if tuple(z.shape) != (B, H, dk) or tuple(q.shape) != (B, H, dk) or tuple(k.shape) != (B, H, dk) \
            or tuple(v.shape) != (B, H, dvv):
        raise ValueError("q, k must be [B,H,d_k] and v [B,H,d_v]")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share one dtype")
    dev = _dev(S, z, q, k, v, o)
    if o is None:
        o = torch.empty((B, H, dvv), dtype=q.dtype, device=dev)
    if tuple(o.shape) != (B, H, dvv) or o.dtype != q.dtype:
        raise ValueError("o must be [B,H,d_v] in the dtype of q")
    rc = _lib.load().la_decode_step(_ptr(S), _ptr(z), _ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, dk, dvv,
                                    _code(q), _stream(dev, stream))
    _lib.check(rc, "la_decode_step")
    return o


def _gamma(gamma, H, dev):
    if not isinstance(gamma, torch.Tensor) or gamma.dtype != torch.float32 or tuple(gamma.shape) != (H,) \
            or not gamma.is_contiguous():
        raise ValueError(f"gamma must be a contiguous float32 tensor of shape ({H},)")
    _dev(gamma)
    if gamma.device != dev:
        raise ValueError("gamma must be on the device of the other tensors")
    return gamma


def la_decode_step_decay(S, z, q, k, v, gamma, o=None, stream=None):
    """One decode step with a fixed decay gamma[h] per head, updating S and z in
    place.  Returns o [B,H,d_v]."""
    if S.dim() != 4 or z.dim() != 3 or S.dtype != torch.float32 or z.dtype != torch.float32:
        raise ValueError("S must be float32 [B,H,d_k,d_v] and z float32 [B,H,d_k]")
    B, H, dk, dvv = S.shape
    if tuple(z.shape) != (B, H, dk) or tuple(q.shape) != (B, H, dk) or tuple(k.shape) != (B, H, dk) \
            or tuple(v.shape) != (B, H, dvv):
        raise ValueError("q, k must be [B,H,d_k] and v [B,H,d_v]")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share one dtype")
    dev = _dev(S, z, q, k, v, o)
    _gamma(gamma, H, dev)
    if o is None:
        o = torch.empty((B, H, dvv), dtype=q.dtype, device=dev)
    if tuple(o.shape) != (B, H, dvv) or o.dtype != q.dtype:
        raise ValueError("o must be [B,H,d_v] in the dtype of q")
    rc = _lib.load().la_decode_step_decay(_ptr(S), _ptr(z), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(gamma),
                                          B, H, dk, dvv, _code(q), _stream(dev, stream))
    _lib.check(rc, "la_decode_step_decay")
    return o


# ---------------------------------------------------------------------------
# Feature maps: "elu1" (the default of every entry point above), "identity"
# (q and k are the features) and "prf" (positive random features with the
# directions W [H, m, d_k] in the dtype of q).
# ---------------------------------------------------------------------------
_FM = {"elu1": _lib.LA_PHI_ELU1, "identity": _lib.LA_PHI_IDENTITY, "prf": _lib.LA_PHI_PRF}


def _fm_args(feature_map, W, q):
    try:
        code = _FM[feature_map]
    except KeyError:
        raise ValueError(f"feature_map must be one of {sorted(_FM)}") from None
    if code != _lib.LA_PHI_PRF:
        return code, None, q.shape[-1]
    # q is [B, H, N, d_k] or, for a decode step, [B, H, d_k]: H is dim 1 in both
    if W is None or W.dim() != 3 or W.dtype != q.dtype or W.shape[0] != q.shape[1] or W.shape[2] != q.shape[-1]:
        raise ValueError("feature_map='prf' needs W [H, m, d_k] in the dtype of q")
    _dev(q, W)
    return code, W, W.shape[1]


def la_fwd_causal_fm_workspace_bytes(B, H, N, d_k, d_v, C, feature_map, m, dtype) -> int:
    return int(_lib.load().la_fwd_causal_fm_workspace_bytes(B, H, N, d_k, d_v, C, _FM[feature_map], m,
                                                            _DT[dtype]))


def la_fwd_noncausal_fm_workspace_bytes(B, H, N, d_k, d_v, feature_map, m, dtype) -> int:
    return int(_lib.load().la_fwd_noncausal_fm_workspace_bytes(B, H, N, d_k, d_v, _FM[feature_map], m, _DT[dtype]))


def la_bwd_causal_fm_workspace_bytes(B, H, N, d_k, d_v, C, feature_map, m, dtype) -> int:
    return int(_lib.load().la_bwd_causal_fm_workspace_bytes(B, H, N, d_k, d_v, C, _FM[feature_map], m,
                                                            _DT[dtype]))


def la_fwd_causal_fm(q, k, v, feature_map="elu1", W=None, o=None, den=None, C: int = 64, out_dtype=None, ws=None,
                     stream=None, want_den: bool = True):
    """Causal forward with a feature map.  Returns (o, den)."""
    B, H, N, dk, dv = _shapes(q, k, v)
    code, W, m = _fm_args(feature_map, W, q)
    dev = _dev(q, k, v, o, den, ws)
    if o is None:
        o = torch.empty((B, H, N, dv), dtype=out_dtype or q.dtype, device=dev)
    if den is None and want_den:
        den = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    if tuple(o.shape) != (B, H, N, dv) or (den is not None and tuple(den.shape) != (B, H, N)):
        raise ValueError("o must be [B,H,N,d_v] and den [B,H,N]")
    _dev(o, den)
    wp, wb = _ws(la_fwd_causal_fm_workspace_bytes(B, H, N, dk, dv, C, feature_map, m, q.dtype), dev, ws)
    rc = _lib.load().la_fwd_causal_fm(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(den), code, _ptr(W), m,
                                      B, H, N, dk, dv, C, _code(q), _code(o), wp, wb, _stream(dev, stream))
    _lib.check(rc, "la_fwd_causal_fm")
    return o, den


def la_fwd_noncausal_fm(q, k, v, feature_map="elu1", W=None, o=None, out_dtype=None, ws=None, stream=None):
    """Non-causal forward with a feature map.  Returns o."""
    B, H, N, dk, dv = _shapes(q, k, v)
    code, W, m = _fm_args(feature_map, W, q)
    dev = _dev(q, k, v, o, ws)
    if o is None:
        o = torch.empty((B, H, N, dv), dtype=out_dtype or q.dtype, device=dev)
    if tuple(o.shape) != (B, H, N, dv):
        raise ValueError("o must be [B,H,N,d_v]")
    _dev(o)
    wp, wb = _ws(la_fwd_noncausal_fm_workspace_bytes(B, H, N, dk, dv, feature_map, m, q.dtype), dev, ws)
    rc = _lib.load().la_fwd_noncausal_fm(_ptr(q), _ptr(k), _ptr(v), _ptr(o), code, _ptr(W), m, B, H, N, dk, dv,
                                         _code(q), _code(o), wp, wb, _stream(dev, stream))
    _lib.check(rc, "la_fwd_noncausal_fm")
    return o


def la_bwd_causal_fm(q, k, v, dO, feature_map="elu1", W=None, dq=None, dk=None, dv=None, C: int = 64, ws=None,
                     stream=None):
    """Backward of la_fwd_causal_fm.  Returns (dq, dk, dv) in the dtype of q."""
    B, H, N, d_k, d_v = _shapes(q, k, v)
    code, W, m = _fm_args(feature_map, W, q)
    dev = _dev(q, k, v, dO, dq, dk, dv, ws)
    if tuple(dO.shape) != (B, H, N, d_v) or dO.dtype != q.dtype:
        raise ValueError("dO must be [B,H,N,d_v] in the dtype of q")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, ref in ((dq, q), (dk, k), (dv, v)):
        if t.shape != ref.shape or t.dtype != ref.dtype:
            raise ValueError("dq, dk, dv must match q, k, v in shape and dtype")
    _dev(dq, dk, dv)
    wp, wb = _ws(la_bwd_causal_fm_workspace_bytes(B, H, N, d_k, d_v, C, feature_map, m, q.dtype), dev, ws)
    rc = _lib.load().la_bwd_causal_fm(_ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(dq), _ptr(dk), _ptr(dv), code,
                                      _ptr(W), m, B, H, N, d_k, d_v, C, _code(q), wp, wb, _stream(dev, stream))
    _lib.check(rc, "la_bwd_causal_fm")
    return dq, dk, dv


def la_decode_step_fm(S, z, q, k, v, feature_map="elu1", W=None, o=None, stream=None):
    """One decode step with a feature map, updating S [B,H,m',d_v] and z [B,H,m'] in
    place (m' = m for random features, d_k otherwise).  Returns o [B,H,d_v]."""
    if q.dim() != 3 or k.shape != q.shape or v.dim() != 3 or v.shape[:2] != q.shape[:2]:
        raise ValueError("q, k must be [B,H,d_k] and v [B,H,d_v]")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share one dtype")
    B, H, dk = q.shape
    dvv = v.shape[2]
    code, W, m = _fm_args(feature_map, W, q)
    mf = m if code == _lib.LA_PHI_PRF else dk
    if tuple(S.shape) != (B, H, mf, dvv) or tuple(z.shape) != (B, H, mf) or S.dtype != torch.float32 \
            or z.dtype != torch.float32:
        raise ValueError(f"S must be float32 [B,H,{mf},d_v] and z float32 [B,H,{mf}]")
    dev = _dev(S, z, q, k, v, o)
    if o is None:
        o = torch.empty((B, H, dvv), dtype=q.dtype, device=dev)
    if tuple(o.shape) != (B, H, dvv) or o.dtype != q.dtype:
        raise ValueError("o must be [B,H,d_v] in the dtype of q")
    rc = _lib.load().la_decode_step_fm(_ptr(S), _ptr(z), _ptr(q), _ptr(k), _ptr(v), _ptr(o), code, _ptr(W), m,
                                       B, H, dk, dvv, _code(q), _stream(dev, stream))
    _lib.check(rc, "la_decode_step_fm")
    return o
