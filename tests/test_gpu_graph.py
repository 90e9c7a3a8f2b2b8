"""The entry points under HIP graph capture, as the benchmark's decode leg runs
them: every replay must equal the eager result bit for bit."""
import pytest
import torch

import linear_attention_elu_amd as la
from gpu_util import announce, device_inputs, need_gpu

pytestmark = pytest.mark.gpu


def test_decode_graph_replays_match_eager():
    dev = need_gpu()
    B, H, T, d = 16, 8, 24, 32
    announce("decode graph")
    x, _ = device_inputs(B, H, T, d, d, "f32", seed=3, exact=False)
    steps = [tuple(x[n][:, :, t].contiguous() for n in ("q", "k", "v")) for t in range(T)]
    S = torch.zeros(B, H, d, d, device=dev)
    z = torch.zeros(B, H, d, device=dev)
    out = torch.empty(T, B, H, d, device=dev)
    for t, (q, k, v) in enumerate(steps):
        la.la_decode_step(S, z, q, k, v, o=out[t])
    torch.cuda.synchronize(dev)
    eager, S_eager = out.clone(), S.clone()

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for t, (q, k, v) in enumerate(steps):
                la.la_decode_step(S, z, q, k, v, o=out[t])
    torch.cuda.synchronize(dev)
    for _ in range(3):
        S.zero_()
        z.zero_()
        out.fill_(float("nan"))
        torch.cuda.synchronize(dev)
        g.replay()
        torch.cuda.synchronize(dev)
        assert torch.equal(out, eager) and torch.equal(S, S_eager)


def test_causal_forward_graph_replays_match_eager():
    dev = need_gpu()
    B, H, N, d = 2, 4, 3000, 64
    announce("forward graph")
    x, _ = device_inputs(B, H, N, d, d, "bf16", seed=4, exact=False)
    ws = torch.empty(max(1, la.la_fwd_causal_workspace_bytes(B, H, N, d, d, 64)), dtype=torch.uint8, device=dev)
    o = torch.empty(B, H, N, d, dtype=torch.bfloat16, device=dev)
    den = torch.empty(B, H, N, dtype=torch.float32, device=dev)
    la.la_fwd_causal(x["q"], x["k"], x["v"], o=o, den=den, C=64, ws=ws)
    torch.cuda.synchronize(dev)
    o_eager, d_eager = o.clone(), den.clone()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            la.la_fwd_causal(x["q"], x["k"], x["v"], o=o, den=den, C=64, ws=ws)
    torch.cuda.synchronize(dev)
    for _ in range(3):
        o.zero_()
        den.zero_()
        ws.zero_()
        torch.cuda.synchronize(dev)
        g.replay()
        torch.cuda.synchronize(dev)
        assert torch.equal(o, o_eager) and torch.equal(den, d_eager)
