"""Parity of the forward kernels with the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import forms
import linear_attention_elu_amd as la
import oracle
from gpu_util import (announce, assert_close, check_rows, device_inputs, max_abs, need_gpu, row_rel_l2,
                      to64)

pytestmark = pytest.mark.gpu

# (B, H, N, d_k, d_v, C): tiles, ragged tails, single- and multi-segment plans,
# every d_k, d_v and C at least once.
CAUSAL_CASES = [
    (2, 1, 64, 16, 32, 16),    # the itwiki demo's widths, N rounded to four chunks of 16
    (2, 1, 50, 16, 32, 16),    # the demo's N = 50: ragged last chunk of 2
    (1, 1, 1, 64, 64, 64),     # a single token
    (1, 2, 50, 32, 16, 32),
    (2, 2, 200, 64, 64, 64),   # several chunks, ragged tail of 8
    (1, 3, 333, 64, 128, 32),
    (2, 1, 129, 128, 32, 16),
    (1, 1, 1000, 128, 128, 64),
    (1, 2, 777, 32, 64, 64),
    (3, 1, 96, 16, 16, 32),
    # bf16 at d <= 64 runs up to 16 chunks per (batch, head) as one segment:
    # both sides of that bound, and a split of several segments at small width
    (1, 2, 1024, 64, 64, 64),
    (1, 2, 1025, 64, 64, 64),
    (2, 1, 2100, 32, 16, 64),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", CAUSAL_CASES, ids=lambda c: "B{}_H{}_N{}_dk{}_dv{}_C{}".format(*c))
def test_causal_forward_matches_oracle(case, dtype):
    dev = need_gpu()
    B, H, N, dk, dv, C = case
    announce(f"causal fwd {dtype} {case}")
    x, x64 = device_inputs(B, H, N, dk, dv, dtype, seed=sum(case))
    o, den = la.la_fwd_causal(x["q"], x["k"], x["v"], C=C)
    torch.cuda.synchronize(dev)
    ref_o, ref_den = oracle.fwd_causal(x64["q"], x64["k"], x64["v"])
    assert_close(to64(o), ref_o, dtype, "out")
    assert np.all(to64(den) > 0)
    np.testing.assert_allclose(to64(den), ref_den, rtol=1e-5 if dtype == "f32" else 2e-2)


def test_causal_fp32_demo_workload():
    """Causal forward, fp32, B=2, H=1, N=64, d_k=16, d_v=32, C=16, seed 0: max abs <= 1e-4."""
    dev = need_gpu()
    announce("causal fwd fp32 demo workload")
    x, x64 = device_inputs(2, 1, 64, 16, 32, "f32", seed=0)
    o, _ = la.la_fwd_causal(x["q"], x["k"], x["v"], C=16)
    torch.cuda.synchronize(dev)
    ref, _ = oracle.fwd_causal(x64["q"], x64["k"], x64["v"])
    err = max_abs(to64(o), ref)
    print(f"max abs error {err:.3e}")
    assert err <= 1e-4


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_causal_output_dtype(out_dtype):
    dev = need_gpu()
    announce(f"causal fwd bf16 in, {out_dtype} out")
    x, x64 = device_inputs(2, 2, 300, 64, 64, "bf16", seed=3)
    o, _ = la.la_fwd_causal(x["q"], x["k"], x["v"], C=64, out_dtype=out_dtype)
    torch.cuda.synchronize(dev)
    assert o.dtype == out_dtype
    ref, _ = oracle.fwd_causal(x64["q"], x64["k"], x64["v"])
    check_rows(to64(o), ref, f"out {out_dtype}")


def check_every_head(x, o, den, ref_fn, what):
    """Every (batch, head) of o (and den) against the oracle, a few batches at a
    time so that the fp64 copies stay small and the oracle's threads stay busy."""
    B, H = o.shape[:2]
    step = max(1, 16 // H)
    worst = 0.0
    for b0 in range(0, B, step):
        sl = slice(b0, min(B, b0 + step))
        ref, ref_den = ref_fn(*(to64(x[n][sl]) for n in ("q", "k", "v")))
        worst = max(worst, check_rows(to64(o[sl]), ref, f"{what} batches {sl.start}..{sl.stop - 1}"))
        if den is not None:
            rel = np.abs(to64(den[sl]) - ref_den) / ref_den
            assert rel.max() <= 2e-2, (what, sl, float(rel.max()))
    return worst


@pytest.mark.parametrize("N", [2 ** e for e in range(9, 17)])
def test_causal_length_sweep_every_head(N):
    """The length sweep 2^9 .. 2^16 at B=8, H=8, d=64, C=64, bf16, seed 0, in the
    launch configuration the benchmark times; every row of every (batch, head)
    against the oracle."""
    dev = need_gpu()
    B, H, d = 8, 8, 64
    announce(f"causal sweep N={N}")
    x, _ = device_inputs(B, H, N, d, d, "bf16", seed=0, exact=False)
    o, den = la.la_fwd_causal(x["q"], x["k"], x["v"], C=64)
    torch.cuda.synchronize(dev)
    check_every_head(x, o, den, oracle.fwd_causal, f"N={N}")


def test_causal_forward_d128_workload_every_head():
    """The forward of the training workload, B=8, H=16, N=8192, d=128, C=64,
    bf16, seed 0, as the benchmark runs it: every row of every (batch, head)."""
    dev = need_gpu()
    B, H, N, d = 8, 16, 8192, 128
    announce("causal fwd d128 workload")
    x, _ = device_inputs(B, H, N, d, d, "bf16", seed=0, with_grad=True, exact=False)
    o, den = la.la_fwd_causal(x["q"], x["k"], x["v"], C=64)
    torch.cuda.synchronize(dev)
    check_every_head(x, o, den, oracle.fwd_causal, "d128 workload")


WIDE_CASES = [(2, 2, 1000, 64, 64, 64), (1, 2, 5000, 64, 64, 64), (1, 2, 700, 128, 128, 64), (2, 1, 333, 32, 16, 32)]


@pytest.mark.parametrize("std", [4.0, 8.0])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", WIDE_CASES, ids=lambda c: "B{}_H{}_N{}_dk{}_dv{}_C{}".format(*c))
def test_wide_range_inputs(case, dtype, std):
    """q, k ~ N(0, std^2): phi spans e^-30 .. 30, where the rounding of phi and
    of the carried state matters most.  Causal and non-causal forward."""
    dev = need_gpu()
    B, H, N, dk, dv, C = case
    announce(f"wide-range fwd {dtype} std={std} {case}")
    x, x64 = device_inputs(B, H, N, dk, dv, dtype, seed=sum(case) + int(std), scale=std)
    o, den = la.la_fwd_causal(x["q"], x["k"], x["v"], C=C)
    on = la.la_fwd_noncausal(x["q"], x["k"], x["v"])
    torch.cuda.synchronize(dev)
    ref, ref_den = oracle.fwd_causal(x64["q"], x64["k"], x64["v"])
    assert_close(to64(o), ref, dtype, "causal out")
    np.testing.assert_allclose(to64(den), ref_den, rtol=1e-5 if dtype == "f32" else 2e-2)
    assert_close(to64(on), oracle.fwd_noncausal(x64["q"], x64["k"], x64["v"]), dtype, "non-causal out")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("bad", [float("nan"), float("inf")], ids=["nan", "inf"])
def test_nonfinite_inputs_propagate(dtype, bad):
    """A NaN or +Inf input is propagated, not reported: in q at token i it makes
    o_i alone non-finite; in k or v at token j it makes every output at and after
    j non-finite, while outputs before the C-token chunk holding j, and every other
    (batch, head), keep their values.  -Inf in k is phi = 0: that token carries no
    weight and every output stays finite."""
    dev = need_gpu()
    B, H, N, d, C = 1, 4, 300, 64, 64
    announce(f"non-finite inputs {dtype} {bad}")
    x, x64 = device_inputs(B, H, N, d, d, dtype, seed=12)
    at = {"q": (0, 100), "k": (1, 130), "v": (2, 170)}
    for name, (h, j) in at.items():
        x[name][0, h, j, 5] = bad
        x64[name][0, h, j, 5] = bad
    x["k"][0, 3, 77, :] = float("-inf")
    x64["k"][0, 3, 77, :] = float("-inf")
    o, den = la.la_fwd_causal(x["q"], x["k"], x["v"], C=C, out_dtype=torch.float32)
    on = la.la_fwd_noncausal(x["q"], x["k"], x["v"], out_dtype=torch.float32)
    torch.cuda.synchronize(dev)
    o, on = to64(o)[0], to64(on)[0]
    with np.errstate(invalid="ignore"):
        ref, _ = oracle.fwd_causal(x64["q"], x64["k"], x64["v"])
    ref = ref[0]
    tol = 1e-4 if dtype == "f32" else 5e-2
    # q at token 100 of head 0: that output alone
    assert not np.isfinite(o[0, 100]).any() and not np.isfinite(on[0, 100]).any()
    keep = np.ones(N, bool)
    keep[100] = False
    assert np.abs(o[0, keep] - ref[0, keep]).max() <= tol
    # k and v at token j: every output from j on; nothing before j's chunk
    for name in ("k", "v"):
        h, j = at[name]
        assert not np.isfinite(o[h, j:]).all(axis=-1).any(), name
        assert not np.isfinite(on[h]).all(axis=-1).any(), name
        start = (j // C) * C
        assert np.abs(o[h, :start] - ref[h, :start]).max() <= tol, name
    # -Inf in k: phi = 0, a token without weight
    assert np.isfinite(o[3]).all() and np.isfinite(on[3]).all()
    assert np.abs(o[3] - ref[3]).max() <= tol
    assert np.isfinite(to64(den)[0, 3]).all()


def test_underflowing_query_gives_zero_denominator():
    """No epsilon is added to the denominator: a query whose entries are all below
    about -87 has phi(q) = 0 in fp32 (exp underflows), so den = 0 and its output is
    not finite, while the fp64 oracle still sees exp(x) > 0.  Every other token is
    unaffected."""
    dev = need_gpu()
    B, H, N, d = 1, 1, 200, 64
    announce("underflowing query")
    x, x64 = device_inputs(B, H, N, d, d, "f32", seed=13)
    x["q"][0, 0, 50, :] = -200.0
    o, den = la.la_fwd_causal(x["q"], x["k"], x["v"], C=64)
    torch.cuda.synchronize(dev)
    o, den = to64(o)[0, 0], to64(den)[0, 0]
    assert den[50] == 0.0 and not np.isfinite(o[50]).any()
    keep = np.arange(N) != 50
    ref, _ = oracle.fwd_causal(x64["q"], x64["k"], x64["v"])
    assert np.abs(o[keep] - ref[0, 0, keep]).max() <= 1e-4


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", [(1, 1, 1, 16, 16), (2, 3, 50, 16, 32), (1, 2, 777, 64, 128),
                                  (2, 1, 300, 128, 64), (1, 1, 5000, 32, 32)],
                         ids=lambda c: "B{}_H{}_N{}_dk{}_dv{}".format(*c))
def test_noncausal_matches_oracle(case, dtype):
    dev = need_gpu()
    B, H, N, dk, dv = case
    announce(f"noncausal {dtype} {case}")
    x, x64 = device_inputs(B, H, N, dk, dv, dtype, seed=11)
    o = la.la_fwd_noncausal(x["q"], x["k"], x["v"])
    torch.cuda.synchronize(dev)
    assert_close(to64(o), oracle.fwd_noncausal(x64["q"], x64["k"], x64["v"]), dtype, "out")


def test_noncausal_workload_full():
    """Non-causal forward, bf16, B=4, H=8, N=4096, d=64: every output checked."""
    dev = need_gpu()
    announce("noncausal full workload")
    x, x64 = device_inputs(4, 8, 4096, 64, 64, "bf16", seed=0)
    o = la.la_fwd_noncausal(x["q"], x["k"], x["v"])
    torch.cuda.synchronize(dev)
    check_rows(to64(o), oracle.fwd_noncausal(x64["q"], x64["k"], x64["v"]), "non-causal workload")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_equal_values_give_that_value(dtype):
    """All value rows equal -> every output equals that row (weighted mean)."""
    dev = need_gpu()
    x, _ = device_inputs(2, 2, 500, 64, 32, dtype, seed=4)
    c = torch.randn(32, generator=torch.Generator().manual_seed(1)).to(x["v"].dtype).to(dev)
    v = c.expand_as(x["v"]).contiguous()
    o, den = la.la_fwd_causal(x["q"], x["k"], v, C=32, out_dtype=torch.float32)
    on = la.la_fwd_noncausal(x["q"], x["k"], v, out_dtype=torch.float32)
    torch.cuda.synchronize(dev)
    tol = 1e-5 if dtype == "f32" else 1e-2
    assert max_abs(to64(o), to64(v)) <= tol
    assert max_abs(to64(on), to64(v)) <= tol
    assert bool((den > 0).all())


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_last_causal_row_equals_noncausal(dtype):
    dev = need_gpu()
    x, _ = device_inputs(2, 2, 640, 64, 64, dtype, seed=5)
    o, _ = la.la_fwd_causal(x["q"], x["k"], x["v"], C=64, out_dtype=torch.float32)
    on = la.la_fwd_noncausal(x["q"], x["k"], x["v"], out_dtype=torch.float32)
    torch.cuda.synchronize(dev)
    a, b = to64(o[:, :, -1]), to64(on[:, :, -1])
    if dtype == "f32":
        assert max_abs(a, b) <= 1e-4
    else:
        assert row_rel_l2(a, b) <= 2e-2


def test_forward_is_deterministic():
    dev = need_gpu()
    x, _ = device_inputs(2, 4, 4096, 64, 64, "bf16", seed=6)
    o1, d1 = la.la_fwd_causal(x["q"], x["k"], x["v"], C=64)
    o2, d2 = la.la_fwd_causal(x["q"], x["k"], x["v"], C=64)
    n1 = la.la_fwd_noncausal(x["q"], x["k"], x["v"])
    n2 = la.la_fwd_noncausal(x["q"], x["k"], x["v"])
    torch.cuda.synchronize(dev)
    assert torch.equal(o1, o2) and torch.equal(d1, d2) and torch.equal(n1, n2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_state_handoff_between_calls(dtype):
    """Two calls over the halves of a sequence, the second seeded with the first's
    final state, match the oracle over the whole sequence; the final state
    matches the oracle's sums."""
    dev = need_gpu()
    B, H, N, dk, dv = 2, 2, 1000, 64, 32
    x, x64 = device_inputs(B, H, N, dk, dv, dtype, seed=7)
    h = 384
    S = torch.empty(B, H, dk, dv, device=dev)
    z = torch.empty(B, H, dk, device=dev)
    first = [t[:, :, :h].contiguous() for t in (x["q"], x["k"], x["v"])]
    second = [t[:, :, h:].contiguous() for t in (x["q"], x["k"], x["v"])]
    o1, _ = la.la_fwd_causal_state(*first, S_out=S, z_out=z, C=64)
    o2, _ = la.la_fwd_causal_state(*second, S0=S, z0=z, S_out=S, z_out=z, C=64)
    torch.cuda.synchronize(dev)
    ref, _ = oracle.fwd_causal(x64["q"], x64["k"], x64["v"])
    assert_close(np.concatenate([to64(o1), to64(o2)], axis=2), ref, dtype, "out")
    fk = forms.phi(x64["k"])
    S_ref = np.einsum("bhne,bhnc->bhec", fk, x64["v"])
    z_ref = fk.sum(2)
    np.testing.assert_allclose(to64(z), z_ref, rtol=1e-5 if dtype == "f32" else 1e-2)
    err = np.abs(to64(S) - S_ref).max() / np.abs(S_ref).max()
    assert err < (1e-5 if dtype == "f32" else 1e-2), err

