"""The C ABI on the CPU: the library loads, exports every declared symbol, and
rejects bad arguments before anything reaches the GPU.

Every call below fails validation (that is what is tested), so no kernel is
ever launched; the pointers passed are placeholders that are never touched.
"""
import ctypes
import os
import re

import pytest

import linear_attention_elu_amd as la
from linear_attention_elu_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "la.h")

# placeholder addresses: non-NULL and 16-byte aligned, never dereferenced
P = 0x1000
MIS = 0x1008  # 8-byte aligned only


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from linear_attention_elu_amd import build
        build.build(verbose=False)
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(la_[a-z_0-9]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(_lib.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in range(8):
        s = la.la_status_string(code)
        assert s and s.startswith("LA_")
    assert la.la_status_string(99) == "unknown la_status"


def test_workspace_queries(lib):
    # the causal path needs no workspace when a sequence is a single segment
    assert la.la_fwd_causal_workspace_bytes(2, 1, 64, 16, 32, 16) >= 0
    big = la.la_fwd_causal_workspace_bytes(8, 8, 65536, 64, 64, 64)
    assert big > 0 and big % 16 == 0
    assert la.la_fwd_noncausal_workspace_bytes(4, 8, 4096, 64, 64) > 0
    # invalid sizes answer 0
    assert la.la_fwd_causal_workspace_bytes(1, 1, 64, 48, 64, 64) == 0
    assert la.la_fwd_causal_workspace_bytes(1, 1, 64, 64, 64, 8) == 0
    assert la.la_fwd_causal_workspace_bytes(0, 1, 64, 64, 64, 64) == 0
    # sequences up to 2^30 tokens
    assert la.la_fwd_causal_workspace_bytes(1, 1, 1 << 30, 64, 64, 64) > 0
    for q in (lib.la_fwd_causal_workspace_bytes, lib.la_bwd_causal_workspace_bytes):
        assert q(1, 1, (1 << 30) + 1, 64, 64, 64) == 0
    assert lib.la_fwd_noncausal_workspace_bytes(1, 1, (1 << 30) + 1, 64, 64) == 0


def _causal(lib, q=P, k=P, v=P, o=P, den=None, B=1, H=1, N=64, dk=64, dv=64, C=64, tin=1, tout=1,
            ws=None, wsb=0):
    return lib.la_fwd_causal(q, k, v, o, den, B, H, N, dk, dv, C, tin, tout, ws, wsb, None)


def test_fwd_causal_rejects(lib):
    assert _causal(lib, q=None) == 1
    assert _causal(lib, o=None) == 1
    assert _causal(lib, B=0) == 2
    assert _causal(lib, N=0) == 2
    assert _causal(lib, N=(1 << 30) + 1) == 2
    assert _causal(lib, H=-3) == 2
    assert _causal(lib, dk=48) == 3
    assert _causal(lib, dv=256) == 3
    assert _causal(lib, C=128) == 3
    assert _causal(lib, C=8) == 3
    assert _causal(lib, tin=2) == 4
    assert _causal(lib, tout=-1) == 4
    assert _causal(lib, q=MIS) == 7
    assert _causal(lib, den=MIS) == 7
    # a multi-segment problem without workspace
    assert _causal(lib, B=8, H=8, N=65536) == 5
    need = la.la_fwd_causal_workspace_bytes(8, 8, 65536, 64, 64, 64)
    assert _causal(lib, B=8, H=8, N=65536, ws=P, wsb=need - 16) == 5


def test_fwd_causal_state_rejects(lib):
    f = lib.la_fwd_causal_state
    # S0 without z0 (and S_out without z_out) are errors
    assert f(P, P, P, P, None, P, None, None, None, 1, 1, 64, 64, 64, 64, 1, 1, None, 0, None) == 1
    assert f(P, P, P, P, None, None, None, None, P, 1, 1, 64, 64, 64, 64, 1, 1, None, 0, None) == 1
    assert f(P, P, P, P, None, MIS, P, None, None, 1, 1, 64, 64, 64, 64, 1, 1, None, 0, None) == 7


def test_fwd_noncausal_rejects(lib):
    f = lib.la_fwd_noncausal
    assert f(None, P, P, P, 1, 1, 64, 64, 64, 1, 1, P, 1 << 20, None) == 1
    assert f(P, P, P, P, 1, 1, 0, 64, 64, 1, 1, P, 1 << 20, None) == 2
    assert f(P, P, P, P, 1, 1, 64, 24, 64, 1, 1, P, 1 << 20, None) == 3
    assert f(P, P, P, P, 1, 1, 64, 64, 64, 5, 1, P, 1 << 20, None) == 4
    assert f(P, P, P, P, 1, 1, 64, 64, 64, 1, 1, None, 0, None) == 5
    assert f(P, P, MIS, P, 1, 1, 64, 64, 64, 1, 1, P, 1 << 20, None) == 7


def test_bwd_causal_rejects(lib):
    f = lib.la_bwd_causal
    need = la.la_bwd_causal_workspace_bytes(1, 1, 64, 64, 64, 64)
    assert need > 0
    args = [P] * 7 + [1, 1, 64, 64, 64, 64, 1, P, need, None]
    bad = list(args)
    bad[3] = None  # dO
    assert f(*bad) == 1
    bad = list(args)
    bad[11] = 96  # d_v
    assert f(*bad) == 3
    bad = list(args)
    bad[13] = 3  # dtype
    assert f(*bad) == 4
    bad = list(args)
    bad[6] = MIS  # dv
    assert f(*bad) == 7
    bad = list(args)
    bad[14] = None  # the workspace is always required
    assert f(*bad) == 5
    bad = list(args)
    bad[15] = need - 1
    assert f(*bad) == 5


def test_bwd_noncausal_rejects(lib):
    f = lib.la_bwd_noncausal
    need = la.la_bwd_noncausal_workspace_bytes(1, 1, 64, 64, 64)
    assert need > 0
    assert la.la_bwd_noncausal_workspace_bytes(1, 1, 64, 48, 64) == 0
    args = [P] * 7 + [1, 1, 64, 64, 64, 1, P, need, None]
    bad = list(args)
    bad[0] = None  # q
    assert f(*bad) == 1
    bad = list(args)
    bad[9] = 0  # N
    assert f(*bad) == 2
    bad = list(args)
    bad[10] = 24  # d_k
    assert f(*bad) == 3
    bad = list(args)
    bad[12] = 9  # dtype
    assert f(*bad) == 4
    bad = list(args)
    bad[4] = MIS  # dq
    assert f(*bad) == 7
    bad = list(args)
    bad[13] = None  # the workspace is always required
    assert f(*bad) == 5
    bad = list(args)
    bad[14] = need - 1
    assert f(*bad) == 5


def test_fwd_causal_decay_rejects(lib):
    f = lib.la_fwd_causal_decay
    need = la.la_fwd_causal_workspace_bytes(1, 1, 64, 64, 64, 64)
    args = [P] * 4 + [None] * 5 + [P] + [1, 1, 64, 64, 64, 64, 1, 1, P, max(need, 16), None]
    bad = list(args)
    bad[5] = P  # S0 without z0
    assert f(*bad) == 1
    bad = list(args)
    bad[13] = 48  # d_k
    assert f(*bad) == 3
    bad = list(args)
    bad[15] = 8  # C
    assert f(*bad) == 3
    bad = list(args)
    bad[17] = 2  # out dtype
    assert f(*bad) == 4
    bad = list(args)
    bad[2] = MIS  # v
    assert f(*bad) == 7


def test_fwd_causal_noalloc_rejects(lib):
    f = lib.la_fwd_causal_noalloc
    args = [P] * 4 + [None] + [1, 1, 64, 64, 64, 64, 1, 1, None]
    bad = list(args)
    bad[0] = None  # q
    assert f(*bad) == 1
    bad = list(args)
    bad[7] = 0  # N
    assert f(*bad) == 2
    bad = list(args)
    bad[8] = 24  # d_k
    assert f(*bad) == 3
    bad = list(args)
    bad[10] = 128  # C
    assert f(*bad) == 3
    bad = list(args)
    bad[12] = 3  # out dtype
    assert f(*bad) == 4
    bad = list(args)
    bad[4] = MIS  # den
    assert f(*bad) == 7


def test_feature_map_entry_points_reject(lib):
    f = lib.la_fwd_causal_fm
    args = [P] * 4 + [None] + [2, P, 64] + [1, 1, 64, 64, 64, 64, 1, 1, P, 1 << 24, None]
    assert f(*args[:5], 7, *args[6:]) == 3           # unknown feature map
    bad = list(args)
    bad[6] = None                                     # random features without W
    assert f(*bad) == 1
    bad = list(args)
    bad[7] = 48                                       # m
    assert f(*bad) == 3
    bad = list(args)
    bad[11] = 16                                      # d_k = 16 with random features
    assert f(*bad) == 3
    bad = list(args)
    bad[6] = MIS                                      # W alignment
    assert f(*bad) == 7
    bad = list(args)
    bad[14] = bad[15] = 0                             # fp32: the features pass through the workspace
    bad[-3] = None                                    # ... which is missing
    bad[-2] = 0
    assert f(*bad) == 5
    assert lib.la_fwd_causal_fm_workspace_bytes(1, 1, 64, 64, 64, 64, 9, 64, 1) == 0
    # bf16 with m = d_k in {32, 64}, d_v <= 64, C = 64: the features are formed in
    # the chunk kernels, so the workspace is the plain forward's; other shapes add
    # phi(q), phi(k) as [B][H][N][m] in the input type
    torch = __import__("torch")
    for B, H, N, dk, dv in ((2, 3, 5000, 64, 64), (1, 2, 300, 32, 16), (8, 8, 65536, 64, 32)):
        plain = lib.la_fwd_causal_workspace_bytes(B, H, N, dk, dv, 64)
        assert la.la_fwd_causal_fm_workspace_bytes(B, H, N, dk, dv, 64, "prf", dk, torch.bfloat16) == plain
        assert lib.la_fwd_noncausal_fm_workspace_bytes(B, H, N, dk, dv, 2, dk, 1) == \
            lib.la_fwd_noncausal_workspace_bytes(B, H, N, dk, dv)
        for C, m, dt in ((32, dk, 1), (64, dk, 0), (64, 2 * dk, 1)):
            inner = lib.la_fwd_causal_workspace_bytes(B, H, N, m, dv, C)
            got = lib.la_fwd_causal_fm_workspace_bytes(B, H, N, dk, dv, C, 2, m, dt)
            assert got >= inner + 2 * B * H * N * m * (2 if dt == 1 else 4), (B, H, N, dk, dv, C, m, dt)
    g = lib.la_decode_step_fm
    assert g(P, P, P, P, P, P, 2, None, 64, 1, 1, 64, 64, 1, None) == 1
    assert g(P, P, P, P, P, P, 2, P, 16, 1, 1, 64, 64, 1, None) == 3
    h = lib.la_bwd_causal_fm
    assert h(*([P] * 7), 5, None, 64, 1, 1, 64, 64, 64, 64, 1, P, 1 << 24, None) == 3
    assert h(*([P] * 7), 2, P, 64, 1, 1, 64, 64, 64, 64, 1, P, 16, None) == 5


def test_bwd_causal_decay_rejects(lib):
    f = lib.la_bwd_causal_decay
    need = la.la_bwd_causal_workspace_bytes(1, 1, 64, 64, 64, 64)
    args = [P] * 8 + [1, 1, 64, 64, 64, 64, 1, P, need, None]
    bad = list(args)
    bad[7] = None  # gamma
    assert f(*bad) == 1
    bad = list(args)
    bad[7] = 0x1002  # gamma not 4-byte aligned
    assert f(*bad) == 7
    bad = list(args)
    bad[13] = 8  # C
    assert f(*bad) == 3
    bad = list(args)
    bad[-2] = need - 1
    assert f(*bad) == 5


def test_decode_decay_rejects(lib):
    f = lib.la_decode_step_decay
    assert f(P, P, P, P, P, P, None, 1, 1, 32, 32, 0, None) == 1
    assert f(P, P, P, P, P, P, P, 0, 1, 32, 32, 0, None) == 2
    assert f(P, P, P, P, P, P, P, 1, 1, 8, 32, 0, None) == 3
    assert f(P, P, P, P, P, P, P, 1, 1, 32, 32, 7, None) == 4
    assert f(P, MIS, P, P, P, P, P, 1, 1, 32, 32, 0, None) == 7


def test_decode_rejects(lib):
    f = lib.la_decode_step
    assert f(None, P, P, P, P, P, 1, 1, 32, 32, 0, None) == 1
    assert f(P, P, P, P, P, P, 0, 1, 32, 32, 0, None) == 2
    assert f(P, P, P, P, P, P, 1, 1, 8, 32, 0, None) == 3
    assert f(P, P, P, P, P, P, 1, 1, 32, 32, 7, None) == 4
    assert f(P, MIS, P, P, P, P, 1, 1, 32, 32, 0, None) == 7


def test_binding_refuses_cpu_tensors(lib):
    import torch
    q = torch.zeros(1, 1, 16, 16)
    with pytest.raises(ValueError):
        la.la_fwd_causal(q, q, q)
    with pytest.raises(ValueError):
        la.la_decode_step(torch.zeros(1, 1, 16, 16), torch.zeros(1, 1, 16), q[0, :, 0], q[0, :, 0], q[0, :, 0])


def test_binding_checks_random_feature_directions(lib):
    """W must be [H, m, d_k] in q's dtype: the kernels index it by head, so a
    W with fewer heads than q would be read past its end.  The shape checks come
    before any device work (CPU tensors suffice)."""
    import torch
    q = torch.zeros(2, 3, 16, 32, dtype=torch.bfloat16)
    for W in (torch.zeros(2, 32, 32, dtype=torch.bfloat16),     # 2 heads for 3
              torch.zeros(3, 32, 16, dtype=torch.bfloat16),     # d_k 16 for 32
              torch.zeros(3, 32, 32, dtype=torch.float32),      # dtype
              torch.zeros(32, 32, dtype=torch.bfloat16),        # rank
              None):
        with pytest.raises(ValueError, match="needs W"):
            la.la_fwd_causal_fm(q, q, q, "prf", W)
        with pytest.raises(ValueError, match="needs W"):
            la.la_fwd_noncausal_fm(q, q, q, "prf", W)
        with pytest.raises(ValueError, match="needs W"):
            la.la_bwd_causal_fm(q, q, q, q, "prf", W)
        with pytest.raises(ValueError, match="needs W"):
            la.la_decode_step_fm(torch.zeros(2, 3, 32, 32), torch.zeros(2, 3, 32), q[:, :, 0], q[:, :, 0],
                                 q[:, :, 0], "prf", W)
