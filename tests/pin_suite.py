"""The pins that tie the fp64 oracle to the pages and to mathematics.

Each check takes an oracle library handle (``lib=None`` means the built
oracle) and raises AssertionError on failure.  ``test_oracle.py`` runs them on
the real oracle; ``test_oracle_mutants.py`` runs them on copies of the oracle
with planted mistakes and requires at least one check to fail for each.
"""
from __future__ import annotations

import glob
import json
import os
from fractions import Fraction

import numpy as np

import oracle
import forms

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed=0):
    return np.random.default_rng(seed)


def _qkv(B, H, N, dk, dv, seed=0, scale=1.0):
    r = _rng(seed)
    q = r.standard_normal((B, H, N, dk)) * scale
    k = r.standard_normal((B, H, N, dk)) * scale
    v = r.standard_normal((B, H, N, dv))
    return q, k, v


def _frac_array(m):
    return np.array([[float(Fraction(x)) for x in row] for row in m])[None, None]


def golden_examples():
    return sorted(glob.glob(os.path.join(GOLDEN, "*.json")))


def check_golden(lib=None):
    """Worked examples evaluated exactly from the definition (tests/golden)."""
    files = golden_examples()
    assert files, "no worked examples found"
    for path in files:
        with open(path) as f:
            ex = json.load(f)
        q, k, v, g = (_frac_array(ex[n]) for n in ("q", "k", "v", "dout"))
        o, den = oracle.fwd_causal(q, k, v, lib=lib)
        np.testing.assert_allclose(o, _frac_array(ex["causal_out"]), rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(den[0, 0], [float(Fraction(x)) for x in ex["causal_den"]], rtol=1e-13)
        on = oracle.fwd_noncausal(q, k, v, lib=lib)
        np.testing.assert_allclose(on, _frac_array(ex["noncausal_out"]), rtol=1e-13, atol=1e-14)
        dq, dk, dv = oracle.bwd_causal(q, k, v, g, lib=lib)
        np.testing.assert_allclose(dq, _frac_array(ex["causal_dq"]), rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(dk, _frac_array(ex["causal_dk"]), rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(dv, _frac_array(ex["causal_dv"]), rtol=1e-12, atol=1e-14)
        ndq, ndk, ndv = oracle.bwd_noncausal(q, k, v, g, lib=lib)
        np.testing.assert_allclose(ndq, _frac_array(ex["noncausal_dq"]), rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(ndk, _frac_array(ex["noncausal_dk"]), rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(ndv, _frac_array(ex["noncausal_dv"]), rtol=1e-12, atol=1e-14)


def check_causal_vs_quadratic(lib=None):
    """Recurrent oracle == masked quadratic form (library ELU), N(0,1) inputs."""
    for (B, H, N, dk, dv, seed) in [(2, 2, 1, 16, 32, 1), (1, 3, 7, 4, 5, 2), (2, 1, 50, 16, 32, 3),
                                    (1, 2, 64, 32, 16, 4)]:
        q, k, v = _qkv(B, H, N, dk, dv, seed)
        o, den = oracle.fwd_causal(q, k, v, lib=lib)
        ob, denb = forms.causal_quadratic(q, k, v)
        np.testing.assert_allclose(o, ob, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(den, denb, rtol=1e-12)


def check_causal_vs_chunked(lib=None):
    """Recurrent oracle == chunked form for several chunk sizes and a ragged tail."""
    q, k, v = _qkv(2, 1, 50, 16, 32, seed=5)
    o, _ = oracle.fwd_causal(q, k, v, lib=lib)
    for C in (1, 7, 16, 64):
        np.testing.assert_allclose(o, forms.causal_chunked(q, k, v, C), rtol=1e-11, atol=1e-12)


def check_noncausal(lib=None):
    """Non-causal oracle == quadratic and associative forms; permutation invariance;
    the last causal row equals the last non-causal row (the sums then span all N)."""
    q, k, v = _qkv(2, 2, 33, 8, 12, seed=6)
    on = oracle.fwd_noncausal(q, k, v, lib=lib)
    np.testing.assert_allclose(on, forms.noncausal_quadratic(q, k, v), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(on, forms.noncausal_associative(q, k, v), rtol=1e-11, atol=1e-12)
    perm = _rng(7).permutation(q.shape[2])
    on_p = oracle.fwd_noncausal(q, k[:, :, perm], v[:, :, perm], lib=lib)
    np.testing.assert_allclose(on, on_p, rtol=1e-12, atol=1e-13)
    oc, _ = oracle.fwd_causal(q, k, v, lib=lib)
    np.testing.assert_allclose(oc[:, :, -1], on[:, :, -1], rtol=1e-12, atol=1e-13)


def check_invariants(lib=None):
    """Weighted-mean properties of attention with a positive kernel."""
    q, k, v = _qkv(2, 2, 40, 8, 6, seed=8, scale=2.0)
    o, den = oracle.fwd_causal(q, k, v, lib=lib)
    assert np.all(den > 0), "denominators must be positive (phi > 0)"
    np.testing.assert_allclose(o[:, :, 0], v[:, :, 0], rtol=1e-13, atol=1e-14)  # out_0 = v_0
    # every output lies inside the coordinate range of the values it averages
    lo = np.minimum.accumulate(v, axis=2)
    hi = np.maximum.accumulate(v, axis=2)
    assert np.all(o >= lo - 1e-12) and np.all(o <= hi + 1e-12)
    # equal value rows -> output equals that row, for both forms
    c = _rng(9).standard_normal(6)
    veq = np.broadcast_to(c, v.shape).copy()
    oe, _ = oracle.fwd_causal(q, k, veq, lib=lib)
    np.testing.assert_allclose(oe, veq, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(oracle.fwd_noncausal(q, k, veq, lib=lib), veq, rtol=1e-13, atol=1e-14)
    # linearity in V
    v2 = _rng(10).standard_normal(v.shape)
    o2, _ = oracle.fwd_causal(q, k, v2, lib=lib)
    o3, _ = oracle.fwd_causal(q, k, 2.0 * v - 3.0 * v2, lib=lib)
    np.testing.assert_allclose(o3, 2.0 * o - 3.0 * o2, rtol=1e-11, atol=1e-12)


def check_decode(lib=None):
    """T decode steps from a zero state reproduce the causal forward; the state
    after the steps equals the quadratic-form sums; split and resume is exact."""
    B, H, T, dk, dv = 3, 2, 20, 8, 4
    q, k, v = _qkv(B, H, T, dk, dv, seed=11)
    S = np.zeros((B, H, dk, dv))
    z = np.zeros((B, H, dk))
    outs = []
    for t in range(T):
        S, z, o = oracle.decode_step(S, z, q[:, :, t], k[:, :, t], v[:, :, t], lib=lib)
        outs.append(o)
    outs = np.stack(outs, axis=2)
    ob, _ = forms.causal_quadratic(q, k, v)
    np.testing.assert_allclose(outs, ob, rtol=1e-11, atol=1e-12)
    oc, _ = oracle.fwd_causal(q, k, v, lib=lib)
    assert np.array_equal(outs, oc), "decode must follow the causal forward's own order exactly"
    fk = forms.phi(k)
    np.testing.assert_allclose(S, np.einsum("bhte,bhtc->bhec", fk, v), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(z, fk.sum(2), rtol=1e-13)


def check_backward(lib=None):
    """Oracle gradient == central finite differences of the quadratic form; the
    value gradients sum to the upstream gradients; equal values give zero dq, dk."""
    B, H, N, dk, dv = 1, 2, 9, 3, 4
    q, k, v = _qkv(B, H, N, dk, dv, seed=12)
    g = _rng(13).standard_normal(v.shape)
    dq, dkk, dvv = oracle.bwd_causal(q, k, v, g, lib=lib)

    def loss_q(x):
        return float((forms.causal_quadratic(x, k, v)[0] * g).sum())

    def loss_k(x):
        return float((forms.causal_quadratic(q, x, v)[0] * g).sum())

    def loss_v(x):
        return float((forms.causal_quadratic(q, k, x)[0] * g).sum())

    for got, f, x in ((dq, loss_q, q), (dkk, loss_k, k), (dvv, loss_v, v)):
        ref = forms.fd_gradient(f, x.copy())
        err = np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30)
        assert err < 1e-6, f"finite-difference mismatch {err:.3e}"
    # sum_j dv_j = sum_i g_i because each output's weights sum to one
    np.testing.assert_allclose(dvv.sum(2), g.sum(2), rtol=1e-12, atol=1e-12)
    veq = np.broadcast_to(_rng(14).standard_normal(dv), v.shape).copy()
    dq0, dk0, _ = oracle.bwd_causal(q, k, veq, g, lib=lib)
    assert np.abs(dq0).max() < 1e-12 and np.abs(dk0).max() < 1e-12


def check_backward_noncausal(lib=None):
    """Non-causal oracle gradient == central finite differences of the quadratic
    form; value gradients sum to the upstream gradients; equal values give zero
    dq, dk; a joint permutation of the K and V rows permutes dk and dv and leaves
    dq unchanged; at N = 1 it equals the causal gradient."""
    B, H, N, dk, dv = 1, 2, 8, 3, 4
    q, k, v = _qkv(B, H, N, dk, dv, seed=21)
    g = _rng(22).standard_normal(v.shape)
    dq, dkk, dvv = oracle.bwd_noncausal(q, k, v, g, lib=lib)

    def loss_q(x):
        return float((forms.noncausal_quadratic(x, k, v) * g).sum())

    def loss_k(x):
        return float((forms.noncausal_quadratic(q, x, v) * g).sum())

    def loss_v(x):
        return float((forms.noncausal_quadratic(q, k, x) * g).sum())

    for got, f, x in ((dq, loss_q, q), (dkk, loss_k, k), (dvv, loss_v, v)):
        ref = forms.fd_gradient(f, x.copy())
        err = np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30)
        assert err < 1e-6, f"finite-difference mismatch {err:.3e}"
    np.testing.assert_allclose(dvv.sum(2), g.sum(2), rtol=1e-12, atol=1e-12)
    veq = np.broadcast_to(_rng(23).standard_normal(dv), v.shape).copy()
    dq0, dk0, _ = oracle.bwd_noncausal(q, k, veq, g, lib=lib)
    assert np.abs(dq0).max() < 1e-12 and np.abs(dk0).max() < 1e-12
    perm = _rng(24).permutation(N)
    pq, pk, pv = oracle.bwd_noncausal(q, k[:, :, perm], v[:, :, perm], g, lib=lib)
    np.testing.assert_allclose(pq, dq, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(pk, dkk[:, :, perm], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(pv, dvv[:, :, perm], rtol=1e-12, atol=1e-13)
    q1, k1, v1 = _qkv(2, 1, 1, 5, 3, seed=25)
    g1 = _rng(26).standard_normal(v1.shape)
    for a, b in zip(oracle.bwd_noncausal(q1, k1, v1, g1, lib=lib), oracle.bwd_causal(q1, k1, v1, g1, lib=lib)):
        np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-15)


def check_decay(lib=None):
    """Per-head decay: gamma = 1 is the causal form; the recurrence equals the
    quadratic form with the decay mask gamma^(i-j); gamma = 0 keeps only the
    current token (out = v); equal value rows give that value; T decode steps
    equal the forward; each head uses its own gamma."""
    q, k, v = _qkv(2, 3, 40, 8, 5, seed=31)
    gam = np.array([0.5, 0.9, 0.999])
    o, den = oracle.fwd_causal_decay(q, k, v, gam, lib=lib)
    ob, denb = forms.causal_quadratic_decay(q, k, v, gam)
    np.testing.assert_allclose(o, ob, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(den, denb, rtol=1e-12)
    o1, d1 = oracle.fwd_causal_decay(q, k, v, np.ones(3), lib=lib)
    oc, dc = oracle.fwd_causal(q, k, v, lib=lib)
    np.testing.assert_allclose(o1, oc, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(d1, dc, rtol=1e-14)
    o0, _ = oracle.fwd_causal_decay(q, k, v, np.zeros(3), lib=lib)
    np.testing.assert_allclose(o0, v, rtol=1e-13, atol=1e-14)
    veq = np.broadcast_to(_rng(32).standard_normal(5), v.shape).copy()
    oe, _ = oracle.fwd_causal_decay(q, k, veq, gam, lib=lib)
    np.testing.assert_allclose(oe, veq, rtol=1e-12, atol=1e-12)
    # heads are independent: swapping two heads' gammas swaps their outputs only
    osw, _ = oracle.fwd_causal_decay(q[:, [1, 0, 2]], k[:, [1, 0, 2]], v[:, [1, 0, 2]], gam[[1, 0, 2]], lib=lib)
    np.testing.assert_allclose(osw, o[:, [1, 0, 2]], rtol=1e-14, atol=1e-15)
    S = np.zeros((2, 3, 8, 5))
    z = np.zeros((2, 3, 8))
    outs = []
    for t in range(40):
        S, z, ot = oracle.decode_step_decay(S, z, q[:, :, t], k[:, :, t], v[:, :, t], gam, lib=lib)
        outs.append(ot)
    np.testing.assert_allclose(np.stack(outs, 2), o, rtol=1e-13, atol=1e-14)
    fk = forms.phi(k)
    w = gam.reshape(1, 3, 1) ** np.arange(39, -1, -1).reshape(1, 1, 40)
    np.testing.assert_allclose(z, (fk * w[..., None]).sum(2), rtol=1e-12)


def check_backward_decay(lib=None):
    """Decayed gradient == central finite differences of the decay-masked
    quadratic form; gamma = 1 gives the causal gradient; gamma = 0 makes
    out = v, so dq = dk = 0 and dv = dO; value gradients sum to the upstream ones."""
    B, H, N, dk, dv = 1, 2, 9, 3, 4
    q, k, v = _qkv(B, H, N, dk, dv, seed=41)
    g = _rng(42).standard_normal(v.shape)
    gam = np.array([0.6, 0.95])
    dq, dkk, dvv = oracle.bwd_causal_decay(q, k, v, g, gam, lib=lib)

    def loss_q(x):
        return float((forms.causal_quadratic_decay(x, k, v, gam)[0] * g).sum())

    def loss_k(x):
        return float((forms.causal_quadratic_decay(q, x, v, gam)[0] * g).sum())

    def loss_v(x):
        return float((forms.causal_quadratic_decay(q, k, x, gam)[0] * g).sum())

    for got, f, x in ((dq, loss_q, q), (dkk, loss_k, k), (dvv, loss_v, v)):
        ref = forms.fd_gradient(f, x.copy())
        err = np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30)
        assert err < 1e-6, f"finite-difference mismatch {err:.3e}"
    np.testing.assert_allclose(dvv.sum(2), g.sum(2), rtol=1e-12, atol=1e-12)
    for a, b in zip(oracle.bwd_causal_decay(q, k, v, g, np.ones(2), lib=lib), oracle.bwd_causal(q, k, v, g, lib=lib)):
        np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-15)
    z0 = oracle.bwd_causal_decay(q, k, v, g, np.zeros(2), lib=lib)
    assert np.abs(z0[0]).max() < 1e-13 and np.abs(z0[1]).max() < 1e-13
    np.testing.assert_allclose(z0[2], g, rtol=1e-13, atol=1e-14)


ALL_CHECKS = [check_golden, check_causal_vs_quadratic, check_causal_vs_chunked, check_noncausal,
              check_invariants, check_decode, check_backward, check_backward_noncausal, check_decay,
              check_backward_decay]


def failing_checks(lib):
    """Names of the checks that fail for this oracle build."""
    bad = []
    for chk in ALL_CHECKS:
        try:
            chk(lib)
        except (AssertionError, FloatingPointError, ValueError, ZeroDivisionError):
            bad.append(chk.__name__)
    return bad
