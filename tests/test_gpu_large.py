"""Tensors past 2 GiB: byte offsets above 2^31 in every kernel of the causal
forward and backward.

The oracle cannot run 2^25 tokens in a test's time, so these checks use
properties that hold exactly at any size.  With every key row the same, the
score phi(q_i) . phi(k_j) of query i is one value for all keys j <= i and
cancels from output i (itwiki "선형 어텐션", table "Comparison of forms",
parallel row: row-normalised causal weights):
  o_i = (v_0 + ... + v_i) / (i + 1),
and for a loss sum_i dO_i . o_i the value gradient is
  dv_j = sum_{i >= j} dO_i / (i + 1),
while o does not depend on q at all (dq = 0).  The expected values are those
sums in fp64.  Inputs are drawn on the device from a seeded generator (the
host-side generators would take tens of seconds at this size); the key row is
one drawn row repeated.
"""
import pytest
import torch

import linear_attention_elu_amd as la
from gpu_util import announce, check_rows, need_gpu, to64

pytestmark = pytest.mark.gpu

N_BIG = (1 << 25) + 1000  # x 32 features x 2 B: past 2^31 bytes per bf16 tensor, ragged last chunk
D_BIG = 32


def big_inputs(dev, seed):
    g = torch.Generator(device=dev).manual_seed(seed)
    shape = (1, 1, N_BIG, D_BIG)
    q = torch.randn(shape, generator=g, device=dev).to(torch.bfloat16)
    k = torch.randn((1, 1, 1, D_BIG), generator=g, device=dev).to(torch.bfloat16).expand(shape).contiguous()
    v = torch.randn(shape, generator=g, device=dev).to(torch.bfloat16)
    return q, k, v


def sample_rows(n):
    """Every 4099th row, and the last 4096 rows (the end of the largest offsets)."""
    return torch.cat([torch.arange(0, n, 4099), torch.arange(n - 4096, n)]).unique()


def test_causal_forward_past_2_gib():
    dev = need_gpu()
    announce(f"forward past 2 GiB: N={N_BIG} d={D_BIG} bf16")
    q, k, v = big_inputs(dev, 71)
    assert q.numel() * q.element_size() > 2 ** 31
    o, _ = la.la_fwd_causal(q, k, v, C=64, want_den=False)
    torch.cuda.synchronize(dev)
    rows = sample_rows(N_BIG).to(dev)
    count = torch.arange(1, N_BIG + 1, device=dev, dtype=torch.float64)
    ref = (torch.cumsum(v[0, 0].double(), 0) / count[:, None])[rows]
    check_rows(to64(o[0, 0][rows]), ref.cpu().numpy(), "o (running mean)")


def test_causal_backward_past_2_gib():
    dev = need_gpu()
    announce(f"backward past 2 GiB: N={N_BIG} d={D_BIG} bf16")
    q, k, v = big_inputs(dev, 72)
    g = torch.Generator(device=dev).manual_seed(73)
    dO = torch.randn(q.shape, generator=g, device=dev).to(torch.bfloat16)
    dq, dk, dv = la.la_bwd_causal(q, k, v, dO, C=64)
    torch.cuda.synchronize(dev)
    rows = sample_rows(N_BIG).to(dev)
    count = torch.arange(1, N_BIG + 1, device=dev, dtype=torch.float64)
    w = dO[0, 0].double() / count[:, None]
    ref = torch.flip(torch.cumsum(torch.flip(w, [0]), 0), [0])[rows]
    check_rows(to64(dv[0, 0][rows]), ref.cpu().numpy(), "dv (reverse running sum)")
    # dq cancels exactly; what is left is rounding of its two terms, each of size
    # |phi(k)| |o_i . dO_i| / (phi(q_i) . phi(k)) (at most phi'(q) = 1 times that)
    fk = torch.nn.functional.elu(k[0, 0, 0].double()) + 1
    fq = torch.nn.functional.elu(q[0, 0][rows].double()) + 1
    o = torch.cumsum(v[0, 0].double(), 0)[rows] / count[rows][:, None]
    term = fk.norm() * (o * dO[0, 0][rows].double()).sum(1).abs() / (fq @ fk)
    resid = dq[0, 0][rows].double().norm(dim=1)
    assert torch.isfinite(dq).all() and torch.isfinite(dk).all()
    assert (resid <= 2e-2 * term.max()).all(), float((resid / term.max()).max())
