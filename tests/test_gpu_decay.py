"""Parity of the per-head decay variant (forward and decode) with the fp64
oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import linear_attention_elu_amd as la
import oracle
from gpu_util import announce, assert_close, check_rows, device_inputs, need_gpu, to64

pytestmark = pytest.mark.gpu

DECAY_CASES = [
    (2, 2, 64, 16, 32, 16),
    (2, 3, 50, 16, 32, 16),     # ragged last chunk
    (1, 1, 1, 64, 64, 64),      # a single token
    (1, 4, 300, 64, 64, 64),
    (1, 2, 777, 32, 64, 32),
    (1, 2, 129, 128, 32, 16),
    (1, 2, 700, 128, 128, 64),
    (2, 2, 5000, 64, 64, 64),   # several segments per (batch, head): the scan decays too
    (1, 3, 3001, 64, 32, 32),
    (1, 2, 1024, 64, 64, 64),   # bf16 at d <= 64: 16 chunks run as one segment,
    (1, 2, 1025, 64, 64, 64),   # 17 as several
]


def gammas(H, dev):
    """Per-head decays spanning [0, 1]: fast (0.05, 0.2), slow and none."""
    g = np.array([0.2, 0.9, 0.995, 1.0, 0.05, 0.99][:H] if H <= 6 else np.linspace(0.0, 1.0, H))
    return g, torch.tensor(g, dtype=torch.float32, device=dev)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", DECAY_CASES, ids=lambda c: "B{}_H{}_N{}_dk{}_dv{}_C{}".format(*c))
def test_decay_forward_matches_oracle(case, dtype):
    dev = need_gpu()
    B, H, N, dk, dv, C = case
    announce(f"decay fwd {dtype} {case}")
    x, x64 = device_inputs(B, H, N, dk, dv, dtype, seed=sum(case) + 3)
    g64, g = gammas(H, dev)
    o, den = la.la_fwd_causal_decay(x["q"], x["k"], x["v"], g, C=C)
    torch.cuda.synchronize(dev)
    # the oracle takes gamma as the fp32 value the kernel reads
    ref, dref = oracle.fwd_causal_decay(x64["q"], x64["k"], x64["v"], g.cpu().double().numpy())
    assert_close(to64(o), ref, dtype, "out")
    rel = np.abs(to64(den) - dref) / dref
    assert rel.max() <= (1e-5 if dtype == "f32" else 2e-2), rel.max()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("gam", [0.0, 0.05, 0.2], ids=lambda g: f"gamma{g}")
def test_fast_decay(gam, dtype):
    """Fast decays, every head the same: gamma = 0 keeps only the current token
    (out = v exactly), 0.05 and 0.2 let a few tokens through.  Several chunks
    and segments, a ragged tail."""
    dev = need_gpu()
    B, H, N, dk, dv = 2, 2, 3000, 64, 64
    announce(f"fast decay {gam} {dtype}")
    x, x64 = device_inputs(B, H, N, dk, dv, dtype, seed=int(gam * 100) + 40)
    g = torch.full((H,), gam, dtype=torch.float32, device=dev)
    o, den = la.la_fwd_causal_decay(x["q"], x["k"], x["v"], g, C=64)
    torch.cuda.synchronize(dev)
    ref, dref = oracle.fwd_causal_decay(x64["q"], x64["k"], x64["v"], g.cpu().double().numpy())
    assert_close(to64(o), ref, dtype, "out")
    assert np.all(np.isfinite(to64(o)))
    rel = np.abs(to64(den) - dref) / dref
    assert rel.max() <= (1e-5 if dtype == "f32" else 2e-2), rel.max()
    if gam == 0.0:
        assert np.abs(to64(o) - x64["v"]).max() <= (1e-6 if dtype == "f32" else 1e-2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decay_one_is_the_causal_form(dtype):
    """gamma = 1 for every head gives the plain causal forward: the same operands
    and products, summed in another order (the decayed path adds the carried
    state's term first), so fp32 outputs agree to accumulation rounding."""
    dev = need_gpu()
    x, _ = device_inputs(2, 3, 2500, 64, 64, dtype, seed=5, exact=False)
    g = torch.ones(3, dtype=torch.float32, device=dev)
    o1, d1 = la.la_fwd_causal_decay(x["q"], x["k"], x["v"], g, C=64, out_dtype=torch.float32)
    o2, d2 = la.la_fwd_causal(x["q"], x["k"], x["v"], C=64, out_dtype=torch.float32)
    torch.cuda.synchronize(dev)
    assert float((o1 - o2).abs().max()) <= 1e-5 * float(o2.abs().max())
    assert float(((d1 - d2).abs() / d2).max()) <= 1e-6


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decay_state_handoff(dtype):
    """Two decayed calls over the halves of a sequence, the second seeded with
    the first's final state, match the oracle over the whole sequence."""
    dev = need_gpu()
    B, H, N, dk, dv = 2, 2, 1000, 64, 32
    x, x64 = device_inputs(B, H, N, dk, dv, dtype, seed=8)
    g = torch.tensor([0.05, 0.95], dtype=torch.float32, device=dev)
    h = 448
    S = torch.empty(B, H, dk, dv, device=dev)
    z = torch.empty(B, H, dk, device=dev)
    first = [t[:, :, :h].contiguous() for t in (x["q"], x["k"], x["v"])]
    second = [t[:, :, h:].contiguous() for t in (x["q"], x["k"], x["v"])]
    o1, _ = la.la_fwd_causal_decay(*first, g, S_out=S, z_out=z, C=64)
    o2, _ = la.la_fwd_causal_decay(*second, g, S0=S, z0=z, S_out=S, z_out=z, C=64)
    torch.cuda.synchronize(dev)
    ref, _ = oracle.fwd_causal_decay(x64["q"], x64["k"], x64["v"], g.cpu().double().numpy())
    assert_close(np.concatenate([to64(o1), to64(o2)], axis=2), ref, dtype, "out")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decay_decode_steps_match_oracle(dtype):
    dev = need_gpu()
    B, H, T, dk, dv = 3, 4, 40, 32, 64
    x, x64 = device_inputs(B, H, T, dk, dv, dtype, seed=11)
    _, g = gammas(H, dev)
    g64 = g.cpu().double().numpy()
    S = torch.zeros(B, H, dk, dv, device=dev)
    z = torch.zeros(B, H, dk, device=dev)
    So = np.zeros((B, H, dk, dv))
    zo = np.zeros((B, H, dk))
    for t in range(T):
        qt, kt, vt = (x[n][:, :, t].contiguous() for n in ("q", "k", "v"))
        o = la.la_decode_step_decay(S, z, qt, kt, vt, g)
        So, zo, oo = oracle.decode_step_decay(So, zo, x64["q"][:, :, t], x64["k"][:, :, t], x64["v"][:, :, t], g64)
        torch.cuda.synchronize(dev)
        assert_close(to64(o), oo, dtype, f"step {t}")
    assert np.abs(to64(S) - So).max() / np.abs(So).max() < 1e-5
    np.testing.assert_allclose(to64(z), zo, rtol=1e-5)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decay_prefill_then_decode(dtype):
    """A decayed prefill hands its final state to decayed decode steps; the
    outputs of both match the oracle's forward over the whole sequence."""
    dev = need_gpu()
    B, H, N, T, dk, dv = 2, 3, 500, 24, 64, 64
    x, x64 = device_inputs(B, H, N + T, dk, dv, dtype, seed=13)
    _, g = gammas(H, dev)
    S = torch.empty(B, H, dk, dv, device=dev)
    z = torch.empty(B, H, dk, device=dev)
    pre = [t[:, :, :N].contiguous() for t in (x["q"], x["k"], x["v"])]
    o_pre, _ = la.la_fwd_causal_decay(*pre, g, S_out=S, z_out=z, C=64)
    outs = [la.la_decode_step_decay(S, z, *(x[n][:, :, N + t].contiguous() for n in ("q", "k", "v")), g)
            for t in range(T)]
    torch.cuda.synchronize(dev)
    ref, _ = oracle.fwd_causal_decay(x64["q"], x64["k"], x64["v"], g.cpu().double().numpy())
    assert_close(to64(o_pre), ref[:, :, :N], dtype, "prefill")
    assert_close(to64(torch.stack(outs, 2)), ref[:, :, N:], dtype, "decode")


def test_decay_workload_every_head():
    """The headline shape B=8, H=8, N=65536, d=64, C=64, bf16, seed 0, with
    decays 1 - 2^-(3 + h), as the benchmark runs it: every row of every
    (batch, head) against the oracle."""
    dev = need_gpu()
    B, H, N, d = 8, 8, 65536, 64
    announce("decay workload")
    x, _ = device_inputs(B, H, N, d, d, "bf16", seed=0, exact=False)
    g = torch.tensor([1.0 - 2.0 ** -(3 + h) for h in range(H)], dtype=torch.float32, device=dev)
    o, _ = la.la_fwd_causal_decay(x["q"], x["k"], x["v"], g, C=64, want_den=False)
    torch.cuda.synchronize(dev)
    g64 = g.cpu().double().numpy()
    for b0 in range(0, B, 2):
        sl = slice(b0, b0 + 2)
        ref, _ = oracle.fwd_causal_decay(*(to64(x[n][sl]) for n in ("q", "k", "v")), g64)
        check_rows(to64(o[sl]), ref, f"batches {b0}..{b0 + 1}")


@pytest.mark.parametrize("decay", [False, True])
def test_handoff_with_one_segment_per_sequence(decay):
    """With B*H large enough to fill the GPU on its own, each (batch, head) runs
    as one segment and the carried state enters the chunk loop directly (no
    scan): two calls over the halves of a sequence still match the oracle."""
    dev = need_gpu()
    B, H, N, dk, dv = 16, 16, 300, 32, 32
    announce(f"one-segment handoff decay={decay}")
    x, x64 = device_inputs(B, H, N, dk, dv, "f32", seed=17)
    g = torch.tensor(np.linspace(0.6, 1.0, H), dtype=torch.float32, device=dev)
    h = 130
    S = torch.empty(B, H, dk, dv, device=dev)
    z = torch.empty(B, H, dk, device=dev)
    first = [t[:, :, :h].contiguous() for t in (x["q"], x["k"], x["v"])]
    second = [t[:, :, h:].contiguous() for t in (x["q"], x["k"], x["v"])]
    if decay:
        o1, _ = la.la_fwd_causal_decay(*first, g, S_out=S, z_out=z, C=32)
        o2, _ = la.la_fwd_causal_decay(*second, g, S0=S, z0=z, S_out=S, z_out=z, C=32)
        ref, _ = oracle.fwd_causal_decay(x64["q"], x64["k"], x64["v"], g.cpu().double().numpy())
    else:
        o1, _ = la.la_fwd_causal_state(*first, S_out=S, z_out=z, C=32)
        o2, _ = la.la_fwd_causal_state(*second, S0=S, z0=z, S_out=S, z_out=z, C=32)
        ref, _ = oracle.fwd_causal(x64["q"], x64["k"], x64["v"])
    torch.cuda.synchronize(dev)
    assert_close(np.concatenate([to64(o1), to64(o2)], axis=2), ref, "f32", "out")


BWD_DECAY_CASES = [
    (2, 2, 64, 16, 32, 16),
    (2, 3, 50, 16, 32, 16),     # ragged last chunk
    (1, 1, 1, 64, 64, 64),      # a single token
    (1, 4, 300, 64, 64, 64),
    (1, 2, 777, 32, 64, 32),
    (1, 2, 129, 128, 32, 16),
    (1, 2, 700, 128, 128, 64),
    (2, 2, 5000, 64, 64, 64),   # several segments per (batch, head): both scans decay
    (1, 6, 3001, 64, 32, 32),   # all six decays of gammas(), fast ones included
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", BWD_DECAY_CASES, ids=lambda c: "B{}_H{}_N{}_dk{}_dv{}_C{}".format(*c))
def test_decay_backward_matches_oracle(case, dtype):
    dev = need_gpu()
    B, H, N, dk, dv, C = case
    announce(f"decay bwd {dtype} {case}")
    x, x64 = device_inputs(B, H, N, dk, dv, dtype, seed=sum(case) + 9, with_grad=True)
    _, g = gammas(H, dev)
    dq, dkk, dvv = la.la_bwd_causal_decay(x["q"], x["k"], x["v"], x["dO"], g, C=C)
    torch.cuda.synchronize(dev)
    rq, rk, rv = oracle.bwd_causal_decay(x64["q"], x64["k"], x64["v"], x64["dO"], g.cpu().double().numpy())
    assert_close(to64(dq), rq, dtype, "dq", abs_floor=1e-3)
    assert_close(to64(dkk), rk, dtype, "dk", abs_floor=1e-3)
    assert_close(to64(dvv), rv, dtype, "dv", abs_floor=1e-3)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decay_backward_gamma_zero(dtype):
    """gamma = 0 keeps only the current token (out = v): dq and dk vanish and dv = dO."""
    dev = need_gpu()
    B, H, N, d = 2, 2, 1000, 64
    x, x64 = device_inputs(B, H, N, d, d, dtype, seed=71, with_grad=True)
    g = torch.zeros(H, dtype=torch.float32, device=dev)
    dq, dkk, dvv = la.la_bwd_causal_decay(x["q"], x["k"], x["v"], x["dO"], g, C=64)
    torch.cuda.synchronize(dev)
    rq, rk, rv = oracle.bwd_causal_decay(x64["q"], x64["k"], x64["v"], x64["dO"], np.zeros(H))
    assert_close(to64(dq), rq, dtype, "dq", abs_floor=1e-3)
    assert_close(to64(dkk), rk, dtype, "dk", abs_floor=1e-3)
    assert_close(to64(dvv), x64["dO"], dtype, "dv = dO")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decay_backward_gamma_one_is_the_causal_backward(dtype):
    dev = need_gpu()
    x, _ = device_inputs(2, 3, 2500, 64, 64, dtype, seed=72, with_grad=True, exact=False)
    g = torch.ones(3, dtype=torch.float32, device=dev)
    a = la.la_bwd_causal_decay(x["q"], x["k"], x["v"], x["dO"], g, C=64)
    b = la.la_bwd_causal(x["q"], x["k"], x["v"], x["dO"], C=64)
    torch.cuda.synchronize(dev)
    for name, u, w in zip(("dq", "dk", "dv"), a, b):
        u, w = to64(u), to64(w)
        if dtype == "f32":
            assert np.abs(u - w).max() <= 1e-5 * np.abs(w).max(), name
        else:  # the same bf16 operands summed in another order, then rounded to bf16
            assert np.abs(u - w).max() <= 1e-2 * np.abs(w).max(), name


def test_decay_backward_d128_workload_every_head():
    """The training shape B=8, H=16, N=8192, d=128, C=64, bf16, with decays
    1 - 2^-(2 + h/2) per head: every row of dq, dk and dv of every (batch, head)."""
    dev = need_gpu()
    B, H, N, d = 8, 16, 8192, 128
    announce("decay bwd workload")
    x, _ = device_inputs(B, H, N, d, d, "bf16", seed=0, with_grad=True, exact=False)
    g = torch.tensor([1.0 - 2.0 ** -(2 + h / 2) for h in range(H)], dtype=torch.float32, device=dev)
    dq, dkk, dvv = la.la_bwd_causal_decay(x["q"], x["k"], x["v"], x["dO"], g, C=64)
    torch.cuda.synchronize(dev)
    g64 = g.cpu().double().numpy()
    for b in range(B):
        sl = slice(b, b + 1)
        rq, rk, rv = oracle.bwd_causal_decay(*(to64(x[n][sl]) for n in ("q", "k", "v", "dO")), g64)
        for name, got, ref in (("dq", dq, rq), ("dk", dkk, rk), ("dv", dvv, rv)):
            check_rows(to64(got[sl]), ref, f"batch {b} {name}")


NEAR_CANCEL_CASES = [
    (1, 2, 129, 128, 32, 16),
    (1, 4, 257, 64, 64, 32),
    (2, 4, 513, 128, 64, 64),
    (1, 4, 4097, 32, 32, 16),
]


@pytest.mark.parametrize("case", NEAR_CANCEL_CASES, ids=lambda c: "B{}_H{}_N{}_dk{}_dv{}_C{}".format(*c))
def test_decay_backward_near_cancellation(case):
    """Fast decays, last chunk of one token (bf16), at a tighter row bound.

    Under a fast decay out_j is close to v_j, so in the dk of the last tokens
    g_j . v_j and e_j = -(g_j . out_j) den_j cancel to a small part of either,
    and any error of e_j (from the carried state, through out_j) reaches dk
    magnified.  Rounding phi(q) and phi(k) to bf16 alone moves the rows of
    these cases by 4.3e-3 to 5.4e-3 at d_k >= 64 and by 1.0e-2 at d_k = 32 (an
    fp64 evaluation of the same gradient with rounded features; the rounding
    error of a feature dot product falls as 1 / sqrt(d_k)).  The kernels keep
    the carried state to about 16 bits and add about a tenth to that, so the
    bound is 1e-2 sqrt(64 / d_k) up to d_k = 64, half the usual bf16 bound.
    A state whose terms each carry one bf16 rounding (2^-9) moved the last row
    of the first case by 1.9e-2 and dq of the last case by 1.5e-2."""
    dev = need_gpu()
    B, H, N, dk, dv, C = case
    announce(f"decay bwd near cancellation {case}")
    x, x64 = device_inputs(B, H, N, dk, dv, "bf16", seed=sum(case) + 9, with_grad=True)
    gam = np.resize(np.array([0.2, 0.05]), H)
    g = torch.tensor(gam, dtype=torch.float32, device=dev)
    dq, dkk, dvv = la.la_bwd_causal_decay(x["q"], x["k"], x["v"], x["dO"], g, C=C)
    torch.cuda.synchronize(dev)
    rq, rk, rv = oracle.bwd_causal_decay(x64["q"], x64["k"], x64["v"], x64["dO"], gam)
    tol = 1e-2 * np.sqrt(64 / min(dk, 64))
    for got, want, what in ((dq, rq, "dq"), (dkk, rk, "dk"), (dvv, rv, "dv")):
        check_rows(to64(got), want, what, abs_floor=1e-3, tol=tol)
