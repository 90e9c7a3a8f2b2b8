"""Write the worked examples in this folder.

Every expected value here comes from ``oracle/exact.py``: the attention
definition evaluated as a double sum over token pairs in exact fractions, and
its gradient by exact forward-mode dual numbers.  Nothing else is called.
Run from the repository root:  python tests/golden/make_golden.py
"""
from __future__ import annotations

import json
import os
import sys
from fractions import Fraction as F

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
from oracle import exact  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))

CITATION = (
    "Definition of generalised attention with sim(q,k) = phi(q).phi(k), phi = elu + 1: "
    "'Transformers are RNNs' blog digest (irregular6612), section Methods; velog review "
    "'[논문 리뷰] Transformers are RNNs', sections 3.1, 3.2 and 3.4 (causal range j <= i); "
    "itwiki '선형 어텐션', section Formulas.  Values computed exactly by oracle/exact.py."
)


def s(x):
    return str(F(x))


def mat(m):
    return [[s(x) for x in r] for r in m]


def example(name, q, k, v, g, note):
    out_c = exact.attention(q, k, v, causal=True)
    den_c = exact.denominators(q, k, causal=True)
    out_n = exact.attention(q, k, v, causal=False)
    dq, dk, dv = exact.gradients(q, k, v, g, causal=True)
    ndq, ndk, ndv = exact.gradients(q, k, v, g, causal=False)
    doc = {
        "citation": CITATION,
        "note": note,
        "layout": "one (batch, head) slice; rows are tokens",
        "q": mat(q), "k": mat(k), "v": mat(v), "dout": mat(g),
        "causal_out": mat(out_c), "causal_den": [s(x) for x in den_c],
        "noncausal_out": mat(out_n),
        "causal_dq": mat(dq), "causal_dk": mat(dk), "causal_dv": mat(dv),
        "noncausal_dq": mat(ndq), "noncausal_dk": mat(ndk), "noncausal_dv": mat(ndv),
    }
    with open(os.path.join(HERE, name), "w") as f:
        json.dump(doc, f, indent=1, ensure_ascii=False)
        f.write("\n")


if __name__ == "__main__":
    example(
        "worked_n3_d2.json",
        q=[[F(1, 2), 0], [1, F(1, 4)], [0, 2]],
        k=[[1, 0], [F(1, 2), F(1, 2)], [0, F(1, 3)]],
        v=[[1, -1], [2, 0], [-3, F(1, 2)]],
        g=[[1, 0], [0, 1], [F(1, 2), -1]],
        note="N=3, d_k=2, d_v=2; zeros exercise the x <= 0 branch of phi (phi(0) = 1).",
    )
    example(
        "worked_n5_dk3_dv2.json",
        q=[[0, 0, 0], [F(3, 2), 0, F(1, 5)], [2, 1, 0], [0, F(1, 7), 3], [F(1, 3), F(2, 3), 1]],
        k=[[F(1, 4), 2, 0], [0, 0, 1], [1, 1, 1], [F(5, 2), 0, F(1, 2)], [0, F(3, 4), 0]],
        v=[[2, 3], [-1, F(1, 2)], [0, -4], [F(7, 3), 1], [-2, -F(1, 8)]],
        g=[[0, 1], [1, 1], [-F(1, 2), 0], [2, -3], [F(1, 4), F(3, 4)]],
        note="N=5, d_k=3, d_v=2 (d_k != d_v).  q_0 = 0 gives phi(q_0) = 1 in every feature.",
    )
    print("wrote", sorted(f for f in os.listdir(HERE) if f.endswith(".json")))
