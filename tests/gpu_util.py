"""Helpers for the GPU parity tests: seeded inputs on the device, exact fp64
copies of what the device saw, and the error measures the tolerances use.

Tolerances (the same for every parity test):
- fp32 inputs: elementwise max |gpu - oracle| <= 1e-4;
- bf16 inputs: row-wise relative L2, max over rows of
  ||gpu_i - oracle_i||_2 / max(||oracle_i||_2, m) <= 2e-2, where m is the
  median row norm of the compared block.  The floor only matters for rows
  whose exact value cancels to (near) zero -- e.g. dq of the first token is
  exactly zero because out_0 = v_0 -- where a purely relative measure is
  undefined; there the error is measured against the typical row.  When every
  row cancels (a single token: all gradients are exactly zero), an absolute
  floor given by the caller takes over.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from linear_attention_elu_amd import inputs

FP32_MAX_ABS = 1e-4
BF16_ROW_REL = 2e-2

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch.device("cuda:0")


def announce(msg: str) -> None:
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def device_inputs(B, H, N, dk, dv, dtype, seed=0, with_grad=False, device="cuda:0", exact=True):
    """Seeded inputs on the device plus (if `exact`) their exact float64 host copies."""
    host = inputs.attention_inputs(B, H, N, dk, dv, seed=seed, with_grad=with_grad)
    dev = {n: inputs.to_torch(a, DTYPES[dtype], device) for n, a in host.items()}
    del host
    if not exact:
        return dev, None
    return dev, {n: t.detach().to("cpu").double().numpy() for n, t in dev.items()}


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").double().numpy()


def max_abs(a, b) -> float:
    return float(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)).max()) if np.size(a) else 0.0


def row_rel_l2(a, b, abs_floor: float = 1e-300) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    num = np.sqrt(((a - b) ** 2).sum(-1))
    den = np.sqrt((b ** 2).sum(-1))
    if not num.size:
        return 0.0
    floor = max(float(np.median(den)), abs_floor)
    return float((num / np.maximum(den, floor)).max())


def assert_close(got, ref, dtype: str, what: str = "", abs_floor: float = 1e-300) -> None:
    if dtype == "f32":
        err = max_abs(got, ref)
        assert err <= FP32_MAX_ABS, f"{what}: max abs error {err:.3e} > {FP32_MAX_ABS}"
    else:
        err = row_rel_l2(got, ref, abs_floor)
        assert err <= BF16_ROW_REL, f"{what}: row-wise relative L2 {err:.3e} > {BF16_ROW_REL}"
