"""Parity of the non-causal backward with the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import linear_attention_elu_amd as la
import oracle
from gpu_util import announce, assert_close, check_rows, device_inputs, need_gpu, row_rel_l2, to64

pytestmark = pytest.mark.gpu

NC_BWD_CASES = [
    (2, 1, 64, 16, 32),
    (2, 1, 50, 16, 32),     # ragged last chunk
    (1, 1, 1, 64, 64),      # a single token
    (1, 2, 200, 64, 64),
    (1, 3, 333, 64, 128),
    (2, 1, 129, 128, 32),
    (1, 1, 700, 128, 128),
    (1, 2, 777, 32, 64),
    (3, 1, 96, 16, 16),
    (1, 1, 5000, 64, 64),   # several segments per (batch, head)
]


def run(x):
    return la.la_bwd_noncausal(x["q"], x["k"], x["v"], x["dO"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", NC_BWD_CASES, ids=lambda c: "B{}_H{}_N{}_dk{}_dv{}".format(*c))
def test_noncausal_backward_matches_oracle(case, dtype):
    dev = need_gpu()
    B, H, N, dk, dv = case
    announce(f"nc bwd {dtype} {case}")
    x, x64 = device_inputs(B, H, N, dk, dv, dtype, seed=sum(case) + 7, with_grad=True)
    dq, dkk, dvv = run(x)
    torch.cuda.synchronize(dev)
    rq, rk, rv = oracle.bwd_noncausal(x64["q"], x64["k"], x64["v"], x64["dO"])
    # a single token has an exactly zero gradient: 1e-3 is the absolute floor there
    assert_close(to64(dq), rq, dtype, "dq", abs_floor=1e-3)
    assert_close(to64(dkk), rk, dtype, "dk", abs_floor=1e-3)
    assert_close(to64(dvv), rv, dtype, "dv", abs_floor=1e-3)


def test_noncausal_backward_workload_every_head():
    """B=4, H=8, N=4096, d=64, bf16, seed 0 (the non-causal workload shape, as the
    benchmark runs it): every row of every (batch, head) against the oracle."""
    dev = need_gpu()
    B, H, N, d = 4, 8, 4096, 64
    announce("nc bwd workload")
    x, _ = device_inputs(B, H, N, d, d, "bf16", seed=0, with_grad=True, exact=False)
    dq, dkk, dvv = run(x)
    torch.cuda.synchronize(dev)
    rq, rk, rv = oracle.bwd_noncausal(*(to64(x[n]) for n in ("q", "k", "v", "dO")))
    for name, got, ref in (("dq", dq, rq), ("dk", dkk, rk), ("dv", dvv, rv)):
        check_rows(to64(got), ref, name)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_noncausal_backward_invariants(dtype):
    """Value gradients sum to the upstream gradients; equal value rows give zero
    dq and dk; a joint permutation of the K and V rows permutes dk and dv and
    leaves dq unchanged."""
    dev = need_gpu()
    x, _ = device_inputs(2, 2, 300, 64, 32, dtype, seed=31, with_grad=True, exact=False)
    dq, dkk, dvv = run(x)
    torch.cuda.synchronize(dev)
    lhs = to64(dvv).sum(axis=2)
    rhs = to64(x["dO"]).sum(axis=2)
    tol = 1e-3 if dtype == "f32" else 5e-2
    assert np.abs(lhs - rhs).max() <= tol * np.abs(rhs).max()
    perm = torch.randperm(300, generator=torch.Generator().manual_seed(5)).to(dev)
    xp = dict(x)
    xp["k"] = x["k"][:, :, perm].contiguous()
    xp["v"] = x["v"][:, :, perm].contiguous()
    pq, pk, pv = run(xp)
    torch.cuda.synchronize(dev)
    ptol = 1e-4 if dtype == "f32" else 2e-2
    assert row_rel_l2(to64(pq), to64(dq)) <= ptol
    assert row_rel_l2(to64(pk), to64(dkk[:, :, perm])) <= ptol
    assert row_rel_l2(to64(pv), to64(dvv[:, :, perm])) <= ptol
    c = torch.randn(32, generator=torch.Generator().manual_seed(3)).to(x["v"].dtype).to(dev)
    x["v"] = c.expand_as(x["v"]).contiguous()
    dq0, dk0, _ = run(x)
    torch.cuda.synchronize(dev)
    scale = float(np.abs(to64(x["dO"])).max())
    zt = 1e-4 if dtype == "f32" else 2e-2
    assert float(np.abs(to64(dq0)).max()) <= zt * scale and float(np.abs(to64(dk0)).max()) <= zt * scale


def test_noncausal_backward_deterministic():
    """Fixed-order sums: two calls give identical bits."""
    dev = need_gpu()
    x, _ = device_inputs(2, 3, 3000, 64, 64, "bf16", seed=41, with_grad=True, exact=False)
    a = run(x)
    b = run(x)
    torch.cuda.synchronize(dev)
    for u, w in zip(a, b):
        assert torch.equal(u, w)
