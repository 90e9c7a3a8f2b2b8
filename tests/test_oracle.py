"""Pins of the fp64 oracle (CPU only).  See pin_suite.py for what each checks."""
import numpy as np
import pytest
import torch

import forms
import pin_suite


@pytest.mark.parametrize("check", pin_suite.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(oracle_lib, check):
    check(None)


def test_fp32_forms_agree_with_oracle_at_demo_shapes(oracle_lib):
    """The itwiki 'Implementation' demo runs the parallel, recurrent and chunked
    forms in fp32 on q, k of shape (2, 50, 16) and v of shape (2, 50, 32) and
    reports agreement near 1e-7.  An fp32 evaluation of the parallel form must
    then sit at that level from the fp64 oracle as well."""
    r = np.random.default_rng(0)
    q = r.standard_normal((2, 1, 50, 16)).astype(np.float32)
    k = r.standard_normal((2, 1, 50, 16)).astype(np.float32)
    v = r.standard_normal((2, 1, 50, 32)).astype(np.float32)
    o64, _ = oracle_lib.fwd_causal(q, k, v)
    # fp32 pair weights, each query against the keys up to its own position
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    fq, fk = torch.nn.functional.elu(tq) + 1, torch.nn.functional.elu(tk) + 1
    pos = torch.arange(50)
    w = torch.einsum("bhie,bhje->bhij", fq, fk) * (pos[:, None] >= pos[None, :])
    o32 = (torch.einsum("bhij,bhjc->bhic", w, tv) / w.sum(-1, keepdim=True)).numpy()
    err = np.abs(o32 - o64).max()
    assert err < 2e-6, err
    # and the fp32 chunked form (C = 16, ragged tail of 2) sits at the same level
    oc = forms.causal_chunked(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), 16)
    assert np.abs(oc - o64).max() < 1e-12


def test_oracle_threads_reported(oracle_lib):
    assert oracle_lib.num_threads() >= 1
