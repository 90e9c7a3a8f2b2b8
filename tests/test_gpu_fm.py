"""Parity of the feature-map entry points (elu + 1, identity, positive random
features) with the fp64 oracle, through the C ABI.

Random-feature inputs follow the regime the map is used in: q, k ~ N(0, s^2)
with s = d_k^(-1/4) (softmax's 1/sqrt(d) split over q and k), so the
features exp(w.x - |x|^2/2) stay far from the fp32 range limits; the
directions W are N(0, I) in orthogonal blocks (inputs.random_features)."""
import numpy as np
import pytest
import torch

import linear_attention_elu_amd as la
import oracle
from gpu_util import DTYPES, announce, assert_close, assert_close_scaled, check_rows, device_inputs, need_gpu, to64
from linear_attention_elu_amd import inputs

pytestmark = pytest.mark.gpu


def prf_inputs(B, H, N, dk, dv, m, dtype, seed, with_grad=False):
    x, x64 = device_inputs(B, H, N, dk, dv, dtype, seed=seed, with_grad=with_grad, scale=dk ** -0.25)
    W = inputs.to_torch(inputs.random_features(H, m, dk, seed=seed + 1), DTYPES[dtype], "cuda:0")
    return x, x64, W, to64(W)


def id_inputs(B, H, N, d, dv, dtype, seed, with_grad=False):
    """Positive features (exp of normals / 2) for the identity map."""
    x, _ = device_inputs(B, H, N, d, dv, dtype, seed=seed, with_grad=with_grad)
    for n in ("q", "k"):
        x[n] = torch.exp(0.5 * x[n].float()).to(x[n].dtype)
    return x, {n: to64(t) for n, t in x.items()}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_elu1_through_the_seam_is_the_plain_path(dtype):
    dev = need_gpu()
    announce(f"fm elu1 {dtype}")
    x, _ = device_inputs(2, 3, 700, 64, 32, dtype, seed=61, with_grad=True, exact=False)
    o1, d1 = la.la_fwd_causal_fm(x["q"], x["k"], x["v"], "elu1", C=64)
    o2, d2 = la.la_fwd_causal(x["q"], x["k"], x["v"], C=64)
    n1 = la.la_fwd_noncausal_fm(x["q"], x["k"], x["v"], "elu1")
    n2 = la.la_fwd_noncausal(x["q"], x["k"], x["v"])
    g1 = la.la_bwd_causal_fm(x["q"], x["k"], x["v"], x["dO"], "elu1", C=64)
    g2 = la.la_bwd_causal(x["q"], x["k"], x["v"], x["dO"], C=64)
    torch.cuda.synchronize(dev)
    assert torch.equal(o1, o2) and torch.equal(d1, d2) and torch.equal(n1, n2)
    assert all(torch.equal(a, b) for a, b in zip(g1, g2))


PRF_CASES = [  # (B, H, N, d_k, d_v, m, C)
    (2, 2, 64, 32, 32, 32, 16),
    (2, 1, 50, 32, 16, 64, 16),     # ragged last chunk
    (1, 1, 1, 64, 64, 64, 64),      # a single token
    (1, 2, 333, 64, 64, 64, 64),
    (1, 2, 777, 64, 32, 128, 32),
    (2, 1, 300, 128, 64, 64, 64),
    (1, 1, 700, 128, 128, 128, 64),
    (1, 2, 5000, 64, 64, 64, 64),   # several segments per (batch, head)
    (2, 3, 700, 64, 32, 64, 64),    # d_v = 32 and 16 with m = d_k = 64 (the features formed in the chunk kernels)
    (1, 1, 130, 64, 16, 64, 64),
    (1, 2, 300, 32, 32, 32, 64),    # m = d_k = 32 in the chunk kernels
    (2, 1, 77, 32, 64, 32, 64),
    (1, 2, 1024, 64, 64, 64, 64),   # bf16 at d <= 64: 16 chunks run as one segment,
    (1, 2, 1025, 64, 64, 64, 64),   # 17 as several
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", PRF_CASES, ids=lambda c: "B{}_H{}_N{}_dk{}_dv{}_m{}_C{}".format(*c))
def test_random_features_forward(case, dtype):
    dev = need_gpu()
    B, H, N, dk, dv, m, C = case
    announce(f"prf fwd {dtype} {case}")
    x, x64, W, W64 = prf_inputs(B, H, N, dk, dv, m, dtype, seed=sum(case))
    o, den = la.la_fwd_causal_fm(x["q"], x["k"], x["v"], "prf", W, C=C)
    on = la.la_fwd_noncausal_fm(x["q"], x["k"], x["v"], "prf", W)
    torch.cuda.synchronize(dev)
    ref, ref_den = oracle.fwd_causal_fm(x64["q"], x64["k"], x64["v"], "prf", W64)
    assert_close(to64(o), ref, dtype, "causal out")
    rel = np.abs(to64(den) - ref_den) / ref_den
    assert rel.max() <= (1e-5 if dtype == "f32" else 2e-2), rel.max()
    assert_close(to64(on), oracle.fwd_noncausal_fm(x64["q"], x64["k"], x64["v"], "prf", W64), dtype, "non-causal")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", PRF_CASES, ids=lambda c: "B{}_H{}_N{}_dk{}_dv{}_m{}_C{}".format(*c))
def test_random_features_backward(case, dtype):
    dev = need_gpu()
    B, H, N, dk, dv, m, C = case
    announce(f"prf bwd {dtype} {case}")
    x, x64, W, W64 = prf_inputs(B, H, N, dk, dv, m, dtype, seed=sum(case) + 3, with_grad=True)
    dq, dkk, dvv = la.la_bwd_causal_fm(x["q"], x["k"], x["v"], x["dO"], "prf", W, C=C)
    torch.cuda.synchronize(dev)
    rq, rk, rv = oracle.bwd_causal_fm(x64["q"], x64["k"], x64["v"], x64["dO"], "prf", W64)
    # random-feature gradients reach |dk| ~ 100 (directions of length ~ sqrt(d_k))
    assert_close_scaled(to64(dq), rq, dtype, "dq", abs_floor=1e-3)
    assert_close_scaled(to64(dkk), rk, dtype, "dk", abs_floor=1e-3)
    assert_close_scaled(to64(dvv), rv, dtype, "dv", abs_floor=1e-3)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dims", [(32, 32, 32), (64, 16, 128), (128, 64, 64)], ids=lambda d: "dk{}_dv{}_m{}".format(*d))
def test_random_features_decode(dims, dtype):
    """Decode steps with random features equal the oracle's, and a prefill's
    state would be the oracle's sums of phi(k) v^T over the steps."""
    dev = need_gpu()
    dk, dv, m = dims
    B, H, T = 3, 2, 24
    announce(f"prf decode {dtype} {dims}")
    x, x64, W, W64 = prf_inputs(B, H, T, dk, dv, m, dtype, seed=dk + m)
    S = torch.zeros(B, H, m, dv, device=dev)
    z = torch.zeros(B, H, m, device=dev)
    outs = [la.la_decode_step_fm(S, z, *(x[n][:, :, t].contiguous() for n in ("q", "k", "v")), "prf", W)
            for t in range(T)]
    torch.cuda.synchronize(dev)
    ref, _ = oracle.fwd_causal_fm(x64["q"], x64["k"], x64["v"], "prf", W64)
    assert_close(np.stack([to64(o) for o in outs], 2), ref, dtype, "decode")
    fk = oracle.features(x64["k"], "prf", W64)
    np.testing.assert_allclose(to64(z), fk.sum(2), rtol=1e-5 if dtype == "f32" else 1e-2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_identity_map(dtype):
    """The identity map: q and k are the features (positive here)."""
    dev = need_gpu()
    B, H, N, d, dv = 2, 2, 1000, 64, 32
    announce(f"identity map {dtype}")
    x, x64 = id_inputs(B, H, N, d, dv, dtype, seed=62, with_grad=True)
    o, den = la.la_fwd_causal_fm(x["q"], x["k"], x["v"], "identity", C=64)
    on = la.la_fwd_noncausal_fm(x["q"], x["k"], x["v"], "identity")
    dq, dkk, dvv = la.la_bwd_causal_fm(x["q"], x["k"], x["v"], x["dO"], "identity", C=64)
    S = torch.zeros(B, H, d, dv, device=dev)
    z = torch.zeros(B, H, d, device=dev)
    outs = [la.la_decode_step_fm(S, z, *(x[n][:, :, t].contiguous() for n in ("q", "k", "v")), "identity")
            for t in range(40)]
    torch.cuda.synchronize(dev)
    ref, _ = oracle.fwd_causal_fm(x64["q"], x64["k"], x64["v"], "identity")
    assert_close(to64(o), ref, dtype, "causal")
    assert_close(to64(on), oracle.fwd_noncausal_fm(x64["q"], x64["k"], x64["v"], "identity"), dtype, "non-causal")
    assert_close(np.stack([to64(t) for t in outs], 2), ref[:, :, :40], dtype, "decode")
    rq, rk, rv = oracle.bwd_causal_fm(x64["q"], x64["k"], x64["v"], x64["dO"], "identity")
    assert_close(to64(dq), rq, dtype, "dq", abs_floor=1e-3)
    assert_close(to64(dkk), rk, dtype, "dk", abs_floor=1e-3)
    assert_close(to64(dvv), rv, dtype, "dv", abs_floor=1e-3)


def test_random_features_headline_shape_every_head():
    """Random features (m = 64) at B=8, H=8, N=65536, d=64, C=64, bf16, as the
    benchmark times them: every row of every (batch, head) against the oracle."""
    dev = need_gpu()
    B, H, N, d, m = 8, 8, 65536, 64, 64
    announce("prf headline shape")
    x, _ = device_inputs(B, H, N, d, d, "bf16", seed=0, exact=False, scale=d ** -0.25)
    W = inputs.to_torch(inputs.random_features(H, m, d, seed=1), torch.bfloat16, dev)
    o, _ = la.la_fwd_causal_fm(x["q"], x["k"], x["v"], "prf", W, C=64, want_den=False)
    torch.cuda.synchronize(dev)
    W64 = to64(W)
    for b0 in range(0, B, 2):
        sl = slice(b0, b0 + 2)
        ref, _ = oracle.fwd_causal_fm(*(to64(x[n][sl]) for n in ("q", "k", "v")), "prf", W64)
        check_rows(to64(o[sl]), ref, f"batches {b0}..{b0 + 1}")
