"""Independent fp64 forms of linear attention used to pin the oracle.

These are not the oracle: they evaluate the same mathematics by different
algorithms (the masked quadratic form and the chunked form), with the feature
map taken from the library ELU (torch.nn.functional.elu on the CPU in
float64) rather than the oracle's own branch.  Sources, by page and section:

- quadratic causal form: itwiki '선형 어텐션', table 'Comparison of forms'
  (parallel form, masked matrix product) and section 'Implementation';
- non-causal form, phi(Q)(phi(K)^T V) / phi(Q)(phi(K)^T 1): velog review
  section 3.2; blog digest 'Method / key components 2)';
- chunked form (matrix product inside a chunk, state passed between chunks,
  ragged last chunk): itwiki table 'Comparison of forms' (chunked row) and
  section 'Implementation'.
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F


def phi(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.asarray(x, dtype=np.float64))
    return (F.elu(t, alpha=1.0) + 1.0).numpy()


def causal_quadratic(q, k, v):
    """[..., N, dk], [..., N, dk], [..., N, dv] -> (out, den)."""
    fq, fk = phi(q), phi(k)
    N = q.shape[-2]
    a = np.matmul(fq, np.swapaxes(fk, -1, -2)) * np.tril(np.ones((N, N)))
    den = a.sum(-1)
    return np.matmul(a, v) / den[..., None], den


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
    fq, fk = phi(q), phi(k)
    lead = q.shape[:-2]
    N, dk = q.shape[-2:]
    dv = v.shape[-1]
    S = np.zeros(lead + (dk, dv))
    z = np.zeros(lead + (dk,))
    outs = []
    for s in range(0, N, C):
        qc, kc, vc = fq[..., s:s + C, :], fk[..., s:s + C, :], v[..., s:s + C, :]
        n = qc.shape[-2]
        intra = np.matmul(qc, np.swapaxes(kc, -1, -2)) * np.tril(np.ones((n, n)))
        num = np.matmul(qc, S) + np.matmul(intra, vc)
        den = np.matmul(qc, z[..., None])[..., 0] + intra.sum(-1)
        outs.append(num / den[..., None])
        S = S + np.matmul(np.swapaxes(kc, -1, -2), vc)
        z = z + kc.sum(-2)
    return np.concatenate(outs, axis=-2)


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
