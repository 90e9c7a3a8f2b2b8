"""ctypes binding of liblinattn.so: argument marshalling only.

Every computation happens in the HIP kernels behind the C ABI declared in
include/la.h; this module only checks tensors, passes raw device pointers and
the current HIP stream, and turns status codes into exceptions.  There is no
fallback: if the library is not built, or a tensor is not on the GPU, the call
raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblinattn.so")

LA_F32 = 0
LA_BF16 = 1

LA_PHI_ELU1 = 0
LA_PHI_IDENTITY = 1
LA_PHI_PRF = 2

# Every symbol include/la.h declares.
EXPORTS = (
    "la_status_string",
    "la_fwd_causal_workspace_bytes",
    "la_fwd_noncausal_workspace_bytes",
    "la_bwd_causal_workspace_bytes",
    "la_bwd_noncausal_workspace_bytes",
    "la_fwd_noncausal",
    "la_fwd_causal",
    "la_fwd_causal_state",
    "la_fwd_causal_decay",
    "la_fwd_causal_noalloc",
    "la_bwd_causal",
    "la_bwd_noncausal",
    "la_bwd_causal_decay",
    "la_decode_step",
    "la_decode_step_decay",
    "la_fwd_causal_fm_workspace_bytes",
    "la_fwd_noncausal_fm_workspace_bytes",
    "la_bwd_causal_fm_workspace_bytes",
    "la_fwd_causal_fm",
    "la_fwd_noncausal_fm",
    "la_bwd_causal_fm",
    "la_decode_step_fm",
)

_lib = None


class LAError(RuntimeError):
    """A non-zero la_status returned by the library."""

    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {status_string(code)}")


def load(path: str | None = None) -> ctypes.CDLL:
    """Load liblinattn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(
            f"{p} is not built: run `python -m linear_attention_elu_amd.build` "
            "(there is no CPU fallback)")
    lib = ctypes.CDLL(p)
    vp, sz, i = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.la_status_string.argtypes = [i]
    lib.la_status_string.restype = ctypes.c_char_p
    lib.la_fwd_causal_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.la_fwd_causal_workspace_bytes.restype = sz
    lib.la_fwd_noncausal_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.la_fwd_noncausal_workspace_bytes.restype = sz
    lib.la_bwd_causal_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.la_bwd_causal_workspace_bytes.restype = sz
    lib.la_fwd_noncausal.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, vp, sz, vp]
    lib.la_fwd_noncausal.restype = i
    lib.la_fwd_causal.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, vp, sz, vp]
    lib.la_fwd_causal.restype = i
    lib.la_fwd_causal_state.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, vp, sz, vp]
    lib.la_fwd_causal_decay.argtypes = [vp] * 10 + [i] * 8 + [vp, sz, vp]
    lib.la_fwd_causal_decay.restype = i
    lib.la_fwd_causal_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, vp]
    lib.la_fwd_causal_noalloc.restype = i
    lib.la_fwd_causal_state.restype = i
    lib.la_bwd_causal.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, vp, sz, vp]
    lib.la_bwd_causal.restype = i
    lib.la_bwd_causal_decay.argtypes = [vp] * 8 + [i] * 7 + [vp, sz, vp]
    lib.la_bwd_causal_decay.restype = i
    lib.la_bwd_noncausal_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.la_bwd_noncausal_workspace_bytes.restype = sz
    lib.la_bwd_noncausal.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, vp, sz, vp]
    lib.la_bwd_noncausal.restype = i
    lib.la_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, vp]
    lib.la_decode_step_decay.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, vp]
    lib.la_decode_step_decay.restype = i
    lib.la_decode_step.restype = i
    lib.la_fwd_causal_fm_workspace_bytes.argtypes = [i] * 9
    lib.la_fwd_causal_fm_workspace_bytes.restype = sz
    lib.la_fwd_noncausal_fm_workspace_bytes.argtypes = [i] * 8
    lib.la_fwd_noncausal_fm_workspace_bytes.restype = sz
    lib.la_bwd_causal_fm_workspace_bytes.argtypes = [i] * 9
    lib.la_bwd_causal_fm_workspace_bytes.restype = sz
    lib.la_fwd_causal_fm.argtypes = [vp] * 5 + [i, vp] + [i] * 9 + [vp, sz, vp]
    lib.la_fwd_causal_fm.restype = i
    lib.la_fwd_noncausal_fm.argtypes = [vp] * 4 + [i, vp] + [i] * 8 + [vp, sz, vp]
    lib.la_fwd_noncausal_fm.restype = i
    lib.la_bwd_causal_fm.argtypes = [vp] * 7 + [i, vp] + [i] * 8 + [vp, sz, vp]
    lib.la_bwd_causal_fm.restype = i
    lib.la_decode_step_fm.argtypes = [vp] * 6 + [i, vp] + [i] * 6 + [vp]
    lib.la_decode_step_fm.restype = i
    if path is None:
        _lib = lib
    return lib


def status_string(code: int) -> str:
    return load().la_status_string(int(code)).decode()


def check(code: int, where: str) -> None:
    if code != 0:
        raise LAError(code, where)
