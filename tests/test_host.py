"""Host-side logic on the CPU: the benchmark's one-GPU guard and the workspace
queries' documented properties (no GPU call is made)."""
import os
import subprocess
import sys

import pytest

import linear_attention_elu_amd as la
from linear_attention_elu_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from linear_attention_elu_amd import build
        build.build(verbose=False)
    return _lib.load()


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_causal_workspace_is_empty_for_one_segment(lib):
    # B*H large enough to fill the GPU: one segment per sequence, no segment states
    assert la.la_fwd_causal_workspace_bytes(64, 64, 4096, 64, 64, 64) == 0
    # few sequences: segments and their d_k (d_v + 1) fp32 states
    n = la.la_fwd_causal_workspace_bytes(1, 2, 65536, 64, 64, 64)
    assert n > 0 and n % (4 * (64 * 64 + 64)) == 0


def test_workspace_queries_reject_bad_sizes(lib):
    assert la.la_fwd_causal_workspace_bytes(1, 1, 64, 64, 64, 48) == 0
    assert la.la_fwd_noncausal_workspace_bytes(1, 1, 0, 64, 64) == 0
    assert la.la_bwd_causal_workspace_bytes(1, 1, 64, 64, 96, 64) == 0
    assert la.la_bwd_noncausal_workspace_bytes(0, 1, 64, 64, 64) == 0


@pytest.mark.parametrize("N", [1, 50, 4096, 65536])
def test_backward_workspaces_hold_two_floats_per_token(lib, N):
    for q in (la.la_bwd_causal_workspace_bytes(2, 3, N, 64, 32, 64), la.la_bwd_noncausal_workspace_bytes(2, 3, N, 64, 32)):
        assert q >= 2 * 4 * 2 * 3 * N
