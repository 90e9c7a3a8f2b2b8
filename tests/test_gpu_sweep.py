"""A seeded sweep over the shape space against the fp64 oracle.

The other parity tests pick their cases by hand.  Here the cases are drawn
(fixed seed, so every run checks the same ones) from everything the library
accepts: d_k and d_v in {16, 32, 64, 128} independently, C in {16, 32, 64},
N from 1 to 700 (mostly ragged), B, H in 1..3, fp32 or bf16, and one variant per
case -- the plain forms (causal forward with den, non-causal forward, causal
and non-causal backward), a per-head decay (gammas from 0 to 1), the random
feature map (m in {32, 64}, d_k in {32, 64, 128}) or the identity map.
Tolerances are those of every parity test (gpu_util).  When every head of a
decay case has gamma = 0, dq and dk are exactly zero throughout, so the zero-row
rule has no median of its own; its scale is then the median size of the two
terms that cancel in each row (out_i = v_i there): |phi(k_i)| |dO_i . v_i| / den_i
for dq and |phi(q_j)| |dO_j . v_j| / den_j for dk, den_i = phi(q_i) . phi(k_i)."""
import numpy as np
import pytest
import torch

import linear_attention_elu_amd as la
import oracle
from gpu_util import DTYPES, ZERO_SCALE, announce, assert_close, assert_close_scaled, device_inputs, need_gpu, to64
from linear_attention_elu_amd import inputs

pytestmark = pytest.mark.gpu


def _zero_decay_floors(x64):
    """ZERO_SCALE times the median size of the terms that cancel in dq and dk
    rows when gamma = 0 (see the module docstring)."""
    phi = lambda t: np.where(t > 0, t + 1.0, np.exp(np.minimum(t, 0.0)))
    fq, fk = phi(x64["q"]), phi(x64["k"])
    den = (fq * fk).sum(-1)
    gv = np.abs((x64["dO"] * x64["v"]).sum(-1))
    tq = np.linalg.norm(fk, axis=-1) * gv / den
    tk = np.linalg.norm(fq, axis=-1) * gv / den
    return ZERO_SCALE * float(np.median(tq)), ZERO_SCALE * float(np.median(tk))


def _cases(n=96, seed=2024):
    r = np.random.RandomState(seed)
    dims = [16, 32, 64, 128]
    out = []
    for i in range(n):
        kind = ["plain", "plain", "decay", "prf", "identity"][i % 5]
        dk = int(r.choice([32, 64, 128] if kind == "prf" else dims))
        dv = int(r.choice(dims))
        C = int(r.choice([16, 32, 64]))
        N = int(r.choice([1, 2, C - 1, C, C + 1])) if i % 7 == 0 else int(r.randint(1, 701))
        B, H = int(r.randint(1, 4)), int(r.randint(1, 4))
        dtype = ["f32", "bf16"][int(r.randint(0, 2))]
        m = int(r.choice([32, 64])) if kind == "prf" else 0
        out.append((kind, B, H, N, dk, dv, C, m, dtype, seed + i))
    return out


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=lambda c: "{}_B{}_H{}_N{}_dk{}_dv{}_C{}_m{}_{}".format(*c[:9]))
def test_sweep_case(case):
    dev = need_gpu()
    kind, B, H, N, dk, dv, C, m, dtype, seed = case
    announce(f"sweep {case}")
    if kind == "prf":
        x, x64 = device_inputs(B, H, N, dk, dv, dtype, seed=seed, with_grad=True, scale=dk ** -0.25)
        W = inputs.to_torch(inputs.random_features(H, m, dk, seed=seed + 1), DTYPES[dtype], dev)
        W64 = to64(W)
        o, den = la.la_fwd_causal_fm(x["q"], x["k"], x["v"], "prf", W, C=C)
        on = la.la_fwd_noncausal_fm(x["q"], x["k"], x["v"], "prf", W)
        grads = la.la_bwd_causal_fm(x["q"], x["k"], x["v"], x["dO"], "prf", W, C=C)
        torch.cuda.synchronize(dev)
        ref, ref_den = oracle.fwd_causal_fm(x64["q"], x64["k"], x64["v"], "prf", W64)
        assert_close(to64(o), ref, dtype, "causal out")
        assert_close(to64(on), oracle.fwd_noncausal_fm(x64["q"], x64["k"], x64["v"], "prf", W64), dtype, "non-causal")
        for got, want, what in zip(grads, oracle.bwd_causal_fm(x64["q"], x64["k"], x64["v"], x64["dO"], "prf", W64),
                                   ("dq", "dk", "dv")):
            assert_close_scaled(to64(got), want, dtype, what, abs_floor=1e-3)
        return
    x, x64 = device_inputs(B, H, N, dk, dv, dtype, seed=seed, with_grad=True)
    if kind == "identity":  # positive features (exp of normals / 2)
        for n in ("q", "k"):
            x[n] = torch.exp(0.5 * x[n].float()).to(x[n].dtype)
            x64[n] = to64(x[n])
        o, den = la.la_fwd_causal_fm(x["q"], x["k"], x["v"], "identity", C=C)
        grads = la.la_bwd_causal_fm(x["q"], x["k"], x["v"], x["dO"], "identity", C=C)
        torch.cuda.synchronize(dev)
        ref, _ = oracle.fwd_causal_fm(x64["q"], x64["k"], x64["v"], "identity")
        assert_close(to64(o), ref, dtype, "causal out")
        for got, want, what in zip(grads, oracle.bwd_causal_fm(x64["q"], x64["k"], x64["v"], x64["dO"], "identity"),
                                   ("dq", "dk", "dv")):
            assert_close(to64(got), want, dtype, what, abs_floor=1e-3)
        return
    if kind == "decay":
        gam = np.random.RandomState(seed).choice([0.0, 0.05, 0.3, 0.9, 0.99, 1.0], size=H)
        g = torch.tensor(gam, dtype=torch.float32, device=dev)
        o, den = la.la_fwd_causal_decay(x["q"], x["k"], x["v"], g, C=C)
        grads = la.la_bwd_causal_decay(x["q"], x["k"], x["v"], x["dO"], g, C=C)
        torch.cuda.synchronize(dev)
        g64 = g.cpu().double().numpy()
        ref, ref_den = oracle.fwd_causal_decay(x64["q"], x64["k"], x64["v"], g64)
        assert_close(to64(o), ref, dtype, "causal out")
        floors = _zero_decay_floors(x64) + (1e-3,) if not gam.any() else (1e-3, 1e-3, 1e-3)
        for got, want, what, floor in zip(grads, oracle.bwd_causal_decay(x64["q"], x64["k"], x64["v"], x64["dO"], g64),
                                          ("dq", "dk", "dv"), floors):
            assert_close(to64(got), want, dtype, what, abs_floor=max(1e-3, floor))
        return
    o, den = la.la_fwd_causal(x["q"], x["k"], x["v"], C=C)
    on = la.la_fwd_noncausal(x["q"], x["k"], x["v"])
    grads = la.la_bwd_causal(x["q"], x["k"], x["v"], x["dO"], C=C)
    ngrads = la.la_bwd_noncausal(x["q"], x["k"], x["v"], x["dO"])
    torch.cuda.synchronize(dev)
    ref, ref_den = oracle.fwd_causal(x64["q"], x64["k"], x64["v"])
    assert_close(to64(o), ref, dtype, "causal out")
    rel = np.abs(to64(den) - ref_den) / ref_den
    assert rel.max() <= (1e-5 if dtype == "f32" else 2e-2), rel.max()
    assert_close(to64(on), oracle.fwd_noncausal(x64["q"], x64["k"], x64["v"]), dtype, "non-causal")
    for got, want, what in zip(grads, oracle.bwd_causal(x64["q"], x64["k"], x64["v"], x64["dO"]), ("dq", "dk", "dv")):
        assert_close(to64(got), want, dtype, what, abs_floor=1e-3)
    for got, want, what in zip(ngrads, oracle.bwd_noncausal(x64["q"], x64["k"], x64["v"], x64["dO"]),
                               ("ndq", "ndk", "ndv")):
        assert_close(to64(got), want, dtype, what, abs_floor=1e-3)
