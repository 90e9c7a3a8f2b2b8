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


def check_random_features(lib=None):
    """Positive random features (itwiki '선형 어텐션', section '특징 사상 선택': an
    unbiased estimate of the softmax kernel exp(q . k)).  Closed forms: with all
    directions zero every feature is exp(-|x|^2/2)/sqrt(m), so phi(q).phi(k) =
    exp(-(|q|^2 + |k|^2)/2); with one direction w, phi(q)phi(k) =
    exp(w.(q + k) - (|q|^2 + |k|^2)/2).  The defining property: averaged over
    w ~ N(0, I), phi(q).phi(k) = exp(q . k), with an error that shrinks like
    1/sqrt(m)."""
    r = _rng(51)
    q = r.standard_normal((1, 2, 3, 8)) * 0.4
    k = r.standard_normal((1, 2, 3, 8)) * 0.4
    for m in (16, 64):
        fq = oracle.features(q, "prf", np.zeros((2, m, 8)), lib=lib)
        fk = oracle.features(k, "prf", np.zeros((2, m, 8)), lib=lib)
        want = np.exp(-0.5 * ((q ** 2).sum(-1)[..., :, None] + (k ** 2).sum(-1)[..., None, :]))
        np.testing.assert_allclose(fq @ np.swapaxes(fk, -1, -2), want, rtol=1e-13)
    w = r.standard_normal((2, 1, 8))
    fq = oracle.features(q, "prf", w, lib=lib)[..., 0]
    fk = oracle.features(k, "prf", w, lib=lib)[..., 0]
    wq = np.einsum("bhne,he->bhn", q, w[:, 0])
    wk = np.einsum("bhne,he->bhn", k, w[:, 0])
    np.testing.assert_allclose(fq, np.exp(wq - 0.5 * (q ** 2).sum(-1)), rtol=1e-13)
    np.testing.assert_allclose(fk, np.exp(wk - 0.5 * (k ** 2).sum(-1)), rtol=1e-13)
    # unbiasedness: 24 (q, k) pairs, directions N(0, I); mean relative error at
    # m = 256 and m = 16384 (64x more features -> about 8x smaller error)
    dk = 6
    qs = r.standard_normal((24, dk)) * 0.35
    ks = r.standard_normal((24, dk)) * 0.35
    errs = []
    for m in (256, 16384):
        W = r.standard_normal((1, m, dk))
        fq = oracle.features(qs[None, None], "prf", W, lib=lib)[0, 0]
        fk = oracle.features(ks[None, None], "prf", W, lib=lib)[0, 0]
        est = (fq * fk).sum(-1)
        exact = np.exp((qs * ks).sum(-1))
        terms = m * fq * fk                      # est is the mean of these m samples
        se = terms.std(-1) / np.sqrt(m)
        assert np.all(np.abs(est - exact) <= 5 * se), "estimate outside 5 standard errors"
        errs.append(np.abs(est / exact - 1).mean())
    assert 3.0 < errs[0] / errs[1] < 25.0, errs


def check_feature_map_attention(lib=None):
    """The attention with a feature map: elu + 1 through the map equals the plain
    oracle; the identity map fed with phi(q), phi(k) equals it too; random
    features give the masked quadratic form built on the same features (causal)
    and the associative form (non-causal); T decode steps reproduce the causal
    forward."""
    q, k, v = _qkv(2, 2, 30, 8, 5, seed=52)
    oc, dc = oracle.fwd_causal(q, k, v, lib=lib)
    o1, d1 = oracle.fwd_causal_fm(q, k, v, "elu1", lib=lib)
    np.testing.assert_array_equal(o1, oc)
    np.testing.assert_array_equal(d1, dc)
    o2, _ = oracle.fwd_causal_fm(forms.phi(q), forms.phi(k), v, "identity", lib=lib)
    np.testing.assert_allclose(o2, oc, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(oracle.fwd_noncausal_fm(forms.phi(q), forms.phi(k), v, "identity", lib=lib),
                               oracle.fwd_noncausal(q, k, v, lib=lib), rtol=1e-13, atol=1e-14)
    W = _rng(53).standard_normal((2, 12, 8))
    qs, ks = q * 0.3, k * 0.3
    fq, fk = oracle.features(qs, "prf", W, lib=lib), oracle.features(ks, "prf", W, lib=lib)
    a = (fq @ np.swapaxes(fk, -1, -2)) * np.tril(np.ones((30, 30)))
    o3, d3 = oracle.fwd_causal_fm(qs, ks, v, "prf", W, lib=lib)
    np.testing.assert_allclose(o3, (a @ v) / a.sum(-1, keepdims=True), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(d3, a.sum(-1), rtol=1e-12)
    kv = np.swapaxes(fk, -1, -2) @ v
    np.testing.assert_allclose(oracle.fwd_noncausal_fm(qs, ks, v, "prf", W, lib=lib),
                               (fq @ kv) / (fq @ fk.sum(-2)[..., None]), rtol=1e-11, atol=1e-12)
    S = np.zeros((2, 2, 12, 5))
    z = np.zeros((2, 2, 12))
    outs = []
    for t in range(30):
        S, z, ot = oracle.decode_step_fm(S, z, qs[:, :, t], ks[:, :, t], v[:, :, t], "prf", W, lib=lib)
        outs.append(ot)
    np.testing.assert_array_equal(np.stack(outs, 2), o3)


def check_feature_map_backward(lib=None):
    """Gradient with a feature map == central finite differences of the masked
    quadratic form built on the oracle's features (random features, identity);
    elu + 1 through the map equals the plain gradient; sum_j dv_j = sum_i dO_i."""
    B, H, N, dk, dv, m = 1, 2, 7, 3, 4, 5
    q, k, v = _qkv(B, H, N, dk, dv, seed=54, scale=0.5)
    g = _rng(55).standard_normal(v.shape)
    W = _rng(56).standard_normal((H, m, dk))
    # identity: features with entries of both signs (so that a stray elu' would
    # show), shifted to keep every denominator away from zero (min 0.24 here)
    for kind, Wk, xq, xk in (("prf", W, q, k), ("identity", None, np.exp(q) - 0.6, np.exp(k) - 0.6)):
        dq, dkk, dvv = oracle.bwd_causal_fm(xq, xk, v, g, kind, Wk, lib=lib)

        def out(a, b, c):
            fa, fb = oracle.features(a, kind, Wk, lib=lib), oracle.features(b, kind, Wk, lib=lib)
            w = (fa @ np.swapaxes(fb, -1, -2)) * np.tril(np.ones((N, N)))
            return (w @ c) / w.sum(-1, keepdims=True)

        for got, which in ((dq, 0), (dkk, 1), (dvv, 2)):
            args = [xq, xk, v]

            def loss(x, which=which, args=args):
                a = list(args)
                a[which] = x
                return float((out(*a) * g).sum())

            ref = forms.fd_gradient(loss, args[which].copy())
            err = np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30)
            assert err < 1e-6, f"{kind}: finite-difference mismatch {err:.3e}"
        np.testing.assert_allclose(dvv.sum(2), g.sum(2), rtol=1e-12, atol=1e-12)
    for a, b in zip(oracle.bwd_causal_fm(q, k, v, g, "elu1", lib=lib), oracle.bwd_causal(q, k, v, g, lib=lib)):
        np.testing.assert_array_equal(a, b)


ALL_CHECKS = [check_golden, check_causal_vs_quadratic, check_causal_vs_chunked, check_noncausal,
              check_invariants, check_decode, check_backward, check_backward_noncausal, check_decay,
              check_backward_decay, check_random_features, check_feature_map_attention,
              check_feature_map_backward]


def failing_checks(lib):
    """Names of the checks that fail for this oracle build."""
    bad = []
    for chk in ALL_CHECKS:
        try:
            chk(lib)
        except (AssertionError, FloatingPointError, ValueError, ZeroDivisionError):
            bad.append(chk.__name__)
    return bad
