"""Writes ``prefill_4token.json``: a four-token prefill x_0..x_3 (the shape of the
worked example in "Attention is recurrent", section Prefill, whose numbers did not
survive the page) with small rational inputs and key-dimension gates, and the outputs
the fp64 oracle computes for it; and ``delta_4token.json``: the same four-token shape
under the delta rule (the page's Delta attention and the Prefill section after it,
again with its numbers lost), with rational write strengths.  Calls only ``oracle/``.

Run from the repository root:  python -m tests.golden.make_golden
"""
import json
import os
from fractions import Fraction

import numpy as np

from oracle import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def main():
    q = [[1, 0, 2], [-1, 1, 0], [0, 2, 1], [1, 1, -1]]
    k = [[0, 1, 1], [2, -1, 0], [1, 0, -2], [-1, 2, 1]]
    v = [[1, -2], [0, 3], [2, 1], [-1, 1]]
    alpha = [["1/2", "3/4", "1"], ["1/4", "1", "1/2"], ["7/8", "1/2", "3/4"], ["1", "1/8", "5/8"]]
    a = np.array([[float(Fraction(x)) for x in r] for r in alpha])
    o, s = oracle.forward(np.array(q, float).reshape(1, 1, 4, 3), np.array(k, float).reshape(1, 1, 4, 3),
                          np.array(v, float).reshape(1, 1, 4, 2), g=np.log(a).reshape(1, 1, 4, 3),
                          gate="keydim")
    case = dict(source="oracle/gla_oracle.c via tests/golden/make_golden.py",
                q=q, k=k, v=v, alpha=alpha, o=o[0, 0].tolist(), s_final=s[0, 0].tolist())
    with open(os.path.join(HERE, "prefill_4token.json"), "w") as f:
        json.dump(case, f, indent=1)
        f.write("\n")

    # the delta rule: four tokens, d_k = 3, d_v = 2, S_{-1} = 0 as on the page
    kd = [[1, 0, 0], [1, 1, 0], [0, 1, 1], [1, 0, 1]]
    qd = [[0, 1, 1], [1, 0, -1], [2, 1, 0], [1, 1, 1]]
    vd = [[1, 2], [-1, 0], [3, 1], [0, -2]]
    beta = ["1/2", "1/4", "3/4", "1"]
    b = np.array([float(Fraction(x)) for x in beta])
    o, s = oracle.forward_delta(np.array(qd, float).reshape(1, 1, 4, 3), np.array(kd, float).reshape(1, 1, 4, 3),
                                np.array(vd, float).reshape(1, 1, 4, 2), b.reshape(1, 1, 4))
    case = dict(source="oracle/gla_oracle.c via tests/golden/make_golden.py",
                q=qd, k=kd, v=vd, beta=beta, o=o[0, 0].tolist(), s_final=s[0, 0].tolist())
    with open(os.path.join(HERE, "delta_4token.json"), "w") as f:
        json.dump(case, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
