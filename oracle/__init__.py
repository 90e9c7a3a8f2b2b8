"""fp64 CPU oracle for linear attention with phi(x) = elu(x) + 1.

Test infrastructure only: the tests, the smoke check and the CPU-baseline leg of
the benchmark import it; the product path never does.  It shares no code with
the HIP library (see ``la_oracle.c`` for the arithmetic and its sources).
"""
from .oracle import (  # noqa: F401
    build,
    fwd_causal,
    fwd_noncausal,
    decode_step,
    bwd_causal,
    bwd_noncausal,
    fwd_causal_decay,
    decode_step_decay,
    bwd_causal_decay,
    FEATURE_MAPS,
    features,
    fwd_causal_fm,
    fwd_noncausal_fm,
    decode_step_fm,
    bwd_causal_fm,
    num_threads,
    library_path,
    load_variant,
    source_path,
)
