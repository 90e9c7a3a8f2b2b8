"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle runs.

This module draws random numbers and nothing else: it holds none of the
method's arithmetic.  Inputs are i.i.d. standard normals drawn with
numpy.random.default_rng(seed) in float32, tensor by tensor in the order
q, k, v, dO; bf16 inputs are the round-to-nearest-even casts of those float32
draws (torch's .to(torch.bfloat16)).
"""
from __future__ import annotations

from typing import Dict, Sequence, Tuple

import numpy as np


def normals(shapes: Sequence[Tuple[int, ...]], seed: int = 0) -> Tuple[np.ndarray, ...]:
    """Float32 standard normals of the given shapes, drawn in order from one stream."""
    rng = np.random.default_rng(seed)
    return tuple(rng.standard_normal(tuple(s), dtype=np.float32) for s in shapes)


def attention_inputs(B: int, H: int, N: int, dk: int, dv: int, seed: int = 0,
                     with_grad: bool = False, qk_std: float = 1.0) -> Dict[str, np.ndarray]:
    """q, k [B,H,N,dk], v [B,H,N,dv] (and dO [B,H,N,dv]) as float32.

    q and k are drawn from N(0, qk_std^2) (the unit draws times qk_std, in
    float32); v and dO are unit normals."""
    shapes = [(B, H, N, dk), (B, H, N, dk), (B, H, N, dv)]
    names = ["q", "k", "v"]
    if with_grad:
        shapes.append((B, H, N, dv))
        names.append("dO")
    out = dict(zip(names, normals(shapes, seed)))
    if qk_std != 1.0:
        for n in ("q", "k"):
            out[n] *= np.float32(qk_std)
    return out


def decode_inputs(T: int, B: int, H: int, dk: int, dv: int, seed: int = 0) -> Dict[str, np.ndarray]:
    """Per-step q, k [T,B,H,dk] and v [T,B,H,dv] as float32."""
    q, k, v = normals([(T, B, H, dk), (T, B, H, dk), (T, B, H, dv)], seed)
    return {"q": q, "k": k, "v": v}


def to_torch(x: np.ndarray, dtype, device):
    """float32 array -> torch tensor of `dtype` on `device` (bf16 by RNE cast)."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(x)).to(device).to(dtype).contiguous()


def random_features(H: int, m: int, dk: int, seed: int = 0, orthogonal: bool = True) -> np.ndarray:
    """m random directions of dimension dk per head, [H, m, dk] float32, drawn from
    N(0, I); with `orthogonal`, in blocks of dk mutually orthogonal directions
    (the Q factor of a Gaussian matrix) whose lengths are drawn independently
    like those of N(0, I) vectors, so each direction is still N(0, I) in
    distribution.  Input generation only: the directions are a random input of
    the random-feature map."""
    rng = np.random.default_rng(seed)
    out = np.empty((H, m, dk), np.float64)
    for h in range(H):
        if not orthogonal:
            out[h] = rng.standard_normal((m, dk))
            continue
        rows = []
        while sum(r.shape[0] for r in rows) < m:
            qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
            rows.append(qm.T)
        blk = np.concatenate(rows, 0)[:m]
        lengths = np.linalg.norm(rng.standard_normal((m, dk)), axis=1)
        out[h] = blk * lengths[:, None]
    return out.astype(np.float32)
