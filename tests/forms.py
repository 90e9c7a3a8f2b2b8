"""Independent fp64 forms of linear attention used to pin the oracle.

These are not the oracle: they evaluate the same mathematics by different
algorithms (the masked quadratic form and the chunked form), with the feature
map taken from the library ELU (torch.nn.functional.elu on the CPU in
float64) rather than the oracle's own branch.  Sources, by page and section:

- quadratic causal form: itwiki '선형 어텐션', table 'Comparison of forms'
  (parallel form: the causally masked pair weights);
- non-causal form, phi(Q)(phi(K)^T V) / phi(Q)(phi(K)^T 1): velog review
  section 3.2; blog digest 'Method / key components 2)';
- chunked form (matrix product inside a chunk, state passed between chunks,
  ragged last chunk): itwiki table 'Comparison of forms' (chunked row).  It is
  evaluated here for all chunks at once (chunk sums, then an exclusive prefix
  over chunks), not as a loop over chunks.
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F


def phi(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.asarray(x, dtype=np.float64))
    return (F.elu(t, alpha=1.0) + 1.0).numpy()


def causal_quadratic(q, k, v):
    """[..., N, dk], [..., N, dk], [..., N, dv] -> (out, den).  Every pair
    weight phi(q_i) . phi(k_j), kept where key j does not come after query i."""
    fq, fk = phi(q), phi(k)
    pos = np.arange(q.shape[-2])
    keep = np.greater_equal.outer(pos, pos).astype(np.float64)
    w = np.einsum("...ie,...je->...ij", fq, fk) * keep
    den = w.sum(-1)
    return np.einsum("...ij,...jc->...ic", w, v) / den[..., None], den


def causal_quadratic_decay(q, k, v, gamma):
    """Masked quadratic form with the decay mask gamma^(i - j) (j <= i), one
    gamma per head: q, k [B, H, N, dk], v [B, H, N, dv], gamma [H]."""
    fq, fk = phi(q), phi(k)
    N = q.shape[-2]
    i = np.arange(N)
    expo = (i[:, None] - i[None, :]).astype(np.float64)
    g = np.asarray(gamma, dtype=np.float64).reshape(1, -1, 1, 1)
    mask = np.where(expo >= 0, g ** np.maximum(expo, 0), 0.0)
    a = np.matmul(fq, np.swapaxes(fk, -1, -2)) * mask
    den = a.sum(-1)
    return np.matmul(a, v) / den[..., None], den


def noncausal_quadratic(q, k, v):
    fq, fk = phi(q), phi(k)
    a = np.matmul(fq, np.swapaxes(fk, -1, -2))
    return np.matmul(a, v) / a.sum(-1, keepdims=True)


def noncausal_associative(q, k, v):
    fq, fk = phi(q), phi(k)
    kv = np.matmul(np.swapaxes(fk, -1, -2), v)          # dk x dv
    ks = fk.sum(-2)                                      # dk
    return np.matmul(fq, kv) / np.matmul(fq, ks[..., None])


def causal_chunked(q, k, v, C):
    """The chunked form evaluated for all chunks at once: the sequence is padded
    to whole chunks (padded keys get phi = 0, so they add nothing), every chunk's
    sums phi(K_c)^T [V_c, 1] are formed together, an exclusive prefix over the
    chunk axis gives each chunk's entering state, and the in-chunk part is a
    masked product inside each chunk."""
    lead = q.shape[:-2]
    N, dk = q.shape[-2:]
    nc = -(-N // C)
    pad = [(0, 0)] * len(lead) + [(0, nc * C - N), (0, 0)]
    fq = np.pad(phi(q), pad).reshape(lead + (nc, C, dk))
    fk = np.pad(phi(k), pad).reshape(lead + (nc, C, dk))
    va = np.concatenate([v, np.ones(v.shape[:-1] + (1,))], axis=-1)   # [v, 1]: numerator and normaliser
    va = np.pad(va, pad).reshape(lead + (nc, C, va.shape[-1]))
    sums = np.einsum("...ctd,...ctx->...cdx", fk, va)                    # per chunk phi(K_c)^T [V_c, 1]
    entering = np.cumsum(sums, axis=-3) - sums                         # sum over earlier chunks
    pos = np.arange(C)
    keep = np.greater_equal.outer(pos, pos).astype(np.float64)
    w = np.einsum("...cid,...cjd->...cij", fq, fk) * keep
    both = np.einsum("...cij,...cjx->...cix", w, va) + np.einsum("...cid,...cdx->...cix", fq, entering)
    both = both.reshape(lead + (nc * C, both.shape[-1]))[..., :N, :]
    return both[..., :-1] / both[..., -1:]


def fd_gradient(f, x, h=1e-6):
    """Central finite differences of the scalar function f at x (float64)."""
    g = np.zeros_like(x)
    flat = x.reshape(-1)
    gf = g.reshape(-1)
    for idx in range(flat.size):
        old = flat[idx]
        flat[idx] = old + h
        fp = f(x)
        flat[idx] = old - h
        fm = f(x)
        flat[idx] = old
        gf[idx] = (fp - fm) / (2 * h)
    return g
