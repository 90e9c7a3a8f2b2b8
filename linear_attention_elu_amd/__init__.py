"""MI355X (gfx950) linear attention with phi(x) = elu(x) + 1.

The computation lives in liblinattn.so (hand-written HIP kernels behind the C
ABI in include/la.h); the functions here only marshal torch tensors to it.
"""
from ._lib import LAError, LIB_PATH, EXPORTS, load  # noqa: F401
from .binding import (  # noqa: F401
    la_status_string,
    la_fwd_causal_workspace_bytes,
    la_fwd_noncausal_workspace_bytes,
    la_bwd_causal_workspace_bytes,
    la_bwd_noncausal_workspace_bytes,
    la_fwd_causal,
    la_fwd_causal_state,
    la_fwd_causal_decay,
    la_fwd_causal_noalloc,
    la_fwd_noncausal,
    la_bwd_causal,
    la_bwd_noncausal,
    la_bwd_causal_decay,
    la_decode_step,
    la_decode_step_decay,
    la_fwd_causal_fm_workspace_bytes,
    la_fwd_noncausal_fm_workspace_bytes,
    la_bwd_causal_fm_workspace_bytes,
    la_fwd_causal_fm,
    la_fwd_noncausal_fm,
    la_bwd_causal_fm,
    la_decode_step_fm,
)
