"""Parity of the forward kernels with the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import forms
import linear_attention_elu_amd as la
import oracle
from gpu_util import (announce, assert_close, device_inputs, max_abs, need_gpu, row_rel_l2, to64)

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
    assert row_rel_l2(to64(o), ref) <= 2e-2


@pytest.mark.parametrize("N", [2 ** e for e in range(9, 17)])
def test_causal_length_sweep_sampled(N):
    """The length sweep 2^9 .. 2^16 at B=8, H=8, d=64, C=64, bf16, seed 0, in the
    launch configuration the benchmark times; the oracle checks every row of
    three sampled (batch, head) pairs."""
    dev = need_gpu()
    B, H, d = 8, 8, 64
    announce(f"causal sweep N={N}")
    x, _ = device_inputs(B, H, N, d, d, "bf16", seed=0, exact=False)
    o, den = la.la_fwd_causal(x["q"], x["k"], x["v"], C=64)
    torch.cuda.synchronize(dev)
    for (b, h) in [(0, 0), (3, 5), (7, 7)]:
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref, ref_den = oracle.fwd_causal(to64(x["q"][sl]), to64(x["k"][sl]), to64(x["v"][sl]))
        err = row_rel_l2(to64(o[sl]), ref)
        assert err <= 2e-2, f"(b={b}, h={h}) row-wise relative L2 {err:.3e}"
        np.testing.assert_allclose(to64(den[sl]), ref_den, rtol=2e-2)


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
    ref = oracle.fwd_noncausal(x64["q"], x64["k"], x64["v"])
    err = row_rel_l2(to64(o), ref)
    print(f"row-wise relative L2 {err:.3e}")
    assert err <= 2e-2


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

