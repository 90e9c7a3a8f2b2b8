"""The allocation-free causal forward, through the C ABI: two calls in a row
(the second smaller, on the array the first left behind) against
la_fwd_causal's outputs, and a size whose la_fwd_causal workspace (as its
query sizes it) exceeds the array, where the split may be capped."""
import pytest
import torch

import linear_attention_elu_amd as la
from gpu_util import announce, assert_close, device_inputs, need_gpu, to64

pytestmark = pytest.mark.gpu


def run_both(x, C, out_dtype):
    B, H, N, _ = x["q"].shape
    dv = x["v"].shape[-1]
    dev = x["q"].device
    o_ref, d_ref = la.la_fwd_causal(x["q"], x["k"], x["v"], C=C, out_dtype=out_dtype)
    o = torch.full((B, H, N, dv), float("nan"), dtype=out_dtype, device=dev)
    den = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=dev)
    la.la_fwd_causal_noalloc(x["q"], x["k"], x["v"], o, den, C=C)
    torch.cuda.synchronize(dev)
    return o, den, o_ref, d_ref


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_noalloc_matches_causal_forward_twice(dtype):
    dev = need_gpu()
    announce(f"noalloc two calls {dtype}")
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    for case in [(2, 4, 20000, 64, 64, 64), (1, 3, 3001, 32, 64, 32)]:
        B, H, N, dk, dv, C = case
        x, _ = device_inputs(B, H, N, dk, dv, dtype, seed=sum(case), exact=False)
        o, den, o_ref, d_ref = run_both(x, C, tdt)
        # the same segment split as la_fwd_causal here: the same bits
        assert torch.equal(o, o_ref) and torch.equal(den, d_ref), case


def test_noalloc_caps_the_segment_split():
    """d = 128 over a long sequence: la_fwd_causal's workspace query asks for about
    100 MB of states, more than the array holds; the allocation-free call (with
    its split capped when needed) agrees within the bf16 tolerance."""
    dev = need_gpu()
    announce("noalloc capped split")
    B, H, N, d, C = 1, 2, 100000, 128, 64
    assert la.la_fwd_causal_workspace_bytes(B, H, N, d, d, C) > (64 << 20)
    x, _ = device_inputs(B, H, N, d, d, "bf16", seed=3, exact=False)
    o, den, o_ref, d_ref = run_both(x, C, torch.bfloat16)
    assert_close(to64(o), to64(o_ref), "bf16", "capped split vs la_fwd_causal")
    assert float(((den - d_ref).abs() / d_ref).max()) <= 1e-3
    # and a smaller call right after, on what the capped one left in the array
    x, _ = device_inputs(1, 1, 777, d, d, "bf16", seed=4, exact=False)
    o, den, o_ref, d_ref = run_both(x, C, torch.bfloat16)
    assert torch.equal(o, o_ref) and torch.equal(den, d_ref)
