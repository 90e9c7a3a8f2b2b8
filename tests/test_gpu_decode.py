"""Parity of the decode step with the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import linear_attention_elu_amd as la
import oracle
from gpu_util import announce, assert_close, device_inputs, max_abs, need_gpu, report, to64
from linear_attention_elu_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dims", [(16, 16), (32, 32), (64, 128), (128, 64), (16, 128), (128, 16)],
                         ids=lambda d: f"dk{d[0]}_dv{d[1]}")
def test_decode_steps_match_oracle(dims, dtype):
    dev = need_gpu()
    dk, dv = dims
    B, H, T = 3, 5, 40
    announce(f"decode {dtype} dk={dk} dv={dv}")
    x, x64 = device_inputs(B, H, T, dk, dv, dtype, seed=dk + dv)
    S = torch.zeros(B, H, dk, dv, device=dev)
    z = torch.zeros(B, H, dk, device=dev)
    So = np.zeros((B, H, dk, dv))
    zo = np.zeros((B, H, dk))
    for t in range(T):
        qt, kt, vt = (x[n][:, :, t].contiguous() for n in ("q", "k", "v"))
        o = la.la_decode_step(S, z, qt, kt, vt)
        So, zo, oo = oracle.decode_step(So, zo, x64["q"][:, :, t], x64["k"][:, :, t], x64["v"][:, :, t])
        torch.cuda.synchronize(dev)
        assert_close(to64(o), oo, dtype, f"step {t}")
    rel = np.abs(to64(S) - So).max() / np.abs(So).max()
    assert rel < 1e-5
    np.testing.assert_allclose(to64(z), zo, rtol=1e-5)


def test_decode_workload_every_state():
    """3072 steps at B=256, H=8, d=32, fp32, seed 0 (the 32x32x3 pixel-generation
    shape): every output of every step of all 2048 (batch, head) states, and every
    final state, against the oracle (whose causal forward equals T decode steps
    from zero)."""
    dev = need_gpu()
    T, B, H, d = 3072, 256, 8, 32
    announce("decode workload 3072 steps")
    host = inputs.decode_inputs(T, B, H, d, d, seed=0)
    q, k, v = (torch.from_numpy(host[n]).to(dev) for n in ("q", "k", "v"))
    S = torch.zeros(B, H, d, d, device=dev)
    z = torch.zeros(B, H, d, device=dev)
    outs = torch.empty(T, B, H, d, device=dev)
    for t in range(T):
        la.la_decode_step(S, z, q[t], k[t], v[t], o=outs[t])
    torch.cuda.synchronize(dev)
    got = to64(outs)
    S_got, z_got = to64(S), to64(z)
    worst = 0.0
    for b0 in range(0, B, 32):  # [T, B, H, d] -> [B, H, T, d], 32 batches at a time
        seq = [np.ascontiguousarray(host[n][:, b0:b0 + 32].transpose(1, 2, 0, 3)).astype(np.float64)
               for n in ("q", "k", "v")]
        ref, _ = oracle.fwd_causal(*seq)
        worst = max(worst, max_abs(got[:, b0:b0 + 32].transpose(1, 2, 0, 3), ref))
        fk = np.where(seq[1] > 0, seq[1] + 1, np.exp(np.minimum(seq[1], 0)))
        S_sum = np.einsum("bhte,bhtc->bhec", fk, seq[2])
        assert np.abs(S_got[b0:b0 + 32] - S_sum).max() / np.abs(S_sum).max() < 1e-5
        np.testing.assert_allclose(z_got[b0:b0 + 32], fk.sum(2), rtol=1e-5)
    report(f"decode: max abs error over 3072 steps and 2048 states {worst:.3e}")
    assert worst <= 1e-4


@pytest.mark.parametrize("std", [4.0, 8.0])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_wide_range_inputs(dtype, std):
    dev = need_gpu()
    B, H, T, dk, dv = 2, 3, 64, 64, 32
    announce(f"wide-range decode {dtype} std={std}")
    x, x64 = device_inputs(B, H, T, dk, dv, dtype, seed=int(std), scale=std)
    S = torch.zeros(B, H, dk, dv, device=dev)
    z = torch.zeros(B, H, dk, device=dev)
    outs = [la.la_decode_step(S, z, *(x[n][:, :, t].contiguous() for n in ("q", "k", "v"))) for t in range(T)]
    torch.cuda.synchronize(dev)
    ref, _ = oracle.fwd_causal(x64["q"], x64["k"], x64["v"])
    assert_close(np.stack([to64(o) for o in outs], 2), ref, dtype, "decode")


def test_decode_nonfinite_inputs_propagate():
    """NaN in q at a step makes that step's output alone non-finite; NaN in k or v
    makes the state, and so every later output of that (batch, head), non-finite.
    Other (batch, head) pairs keep their values."""
    dev = need_gpu()
    B, H, T, d = 1, 3, 12, 32
    x, x64 = device_inputs(B, H, T, d, d, "f32", seed=14)
    for h, name in enumerate(("q", "k", "v")):
        x[name][0, h, 5, 3] = float("nan")
    S = torch.zeros(B, H, d, d, device=dev)
    z = torch.zeros(B, H, d, device=dev)
    outs = np.stack([to64(la.la_decode_step(S, z, *(x[n][:, :, t].contiguous() for n in ("q", "k", "v"))))
                     for t in range(T)], 2)[0]
    torch.cuda.synchronize(dev)
    ref, _ = oracle.fwd_causal(x64["q"], x64["k"], x64["v"])
    ref = ref[0]
    assert not np.isfinite(outs[0, 5]).any()
    keep = np.arange(T) != 5
    assert np.abs(outs[0, keep] - ref[0, keep]).max() <= 1e-4
    assert np.isfinite(to64(S)[0, 0]).all()
    for h in (1, 2):
        assert np.abs(outs[h, :5] - ref[h, :5]).max() <= 1e-4
        assert not np.isfinite(outs[h, 5:]).all(axis=-1).any()
        assert not np.isfinite(to64(S)[0, h]).all()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_then_decode(dtype):
    """Chunked prefill hands its final state to the decode step; the decoded
    outputs equal the oracle's causal forward over the whole sequence."""
    dev = need_gpu()
    B, H, N, dk, dv, pre = 2, 3, 300, 64, 64, 250
    x, x64 = device_inputs(B, H, N, dk, dv, dtype, seed=9)
    S = torch.empty(B, H, dk, dv, device=dev)
    z = torch.empty(B, H, dk, device=dev)
    o_pre, _ = la.la_fwd_causal_state(*(x[n][:, :, :pre].contiguous() for n in ("q", "k", "v")),
                                      S_out=S, z_out=z, C=64)
    outs = [to64(o_pre)]
    for t in range(pre, N):
        o = la.la_decode_step(S, z, *(x[n][:, :, t].contiguous() for n in ("q", "k", "v")))
        outs.append(to64(o)[:, :, None])
    torch.cuda.synchronize(dev)
    ref, _ = oracle.fwd_causal(x64["q"], x64["k"], x64["v"])
    assert_close(np.concatenate(outs, axis=2), ref, dtype, "prefill + decode")


def test_decode_split_and_resume_is_exact():
    """Copying (S, z) to the host and back between steps changes nothing."""
    dev = need_gpu()
    B, H, T, d = 4, 2, 64, 32
    x, _ = device_inputs(B, H, T, d, d, "f32", seed=10)
    S1 = torch.zeros(B, H, d, d, device=dev)
    z1 = torch.zeros(B, H, d, device=dev)
    S2, z2 = S1.clone(), z1.clone()
    o1, o2 = [], []
    for t in range(T):
        qt, kt, vt = (x[n][:, :, t].contiguous() for n in ("q", "k", "v"))
        o1.append(la.la_decode_step(S1, z1, qt, kt, vt))
        if t == T // 2:
            S2 = S2.cpu().to(dev)
            z2 = z2.cpu().to(dev)
        o2.append(la.la_decode_step(S2, z2, qt, kt, vt))
    torch.cuda.synchronize(dev)
    assert all(torch.equal(a, b) for a, b in zip(o1, o2))
    assert torch.equal(S1, S2) and torch.equal(z1, z2)
