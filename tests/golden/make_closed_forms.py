"""Write closed_forms.json: tiny attention problems whose results have textbook closed forms.

The pages print no worked numeric example, so these fixtures are derived by hand
from the definition softmax(Q K^T * scale) V (page "Agent 帮我写 CUDA：一个 Softmax
Attention 算子的开发全记录", section 二) and evaluated here with ``math`` only
(no oracle code, no GPU):

* logistic: one query, two keys with scores 0 and 1 -> the weight of the second
  key is the logistic sigmoid e/(1+e); LSE = ln(1+e) (softplus of 1).
* uniform: a zero query gives equal scores -> O is the mean of V; LSE = ln 3.
* causal_two_rows: row 0 sees only key 0 (O = v0, LSE = 0); row 1 sees scores
  0 and 1 -> O = (v0 + e v1)/(1+e), LSE = ln(1+e).
* three_scores: scores 1, 2, 3 -> weights e^s / (e + e^2 + e^3).
"""
import json
import math
import os

E = math.e


def main():
    cases = []
    cases.append(dict(name="logistic", scale=1.0, q=[[[1.0]]], k=[[[0.0], [1.0]]], v=[[[0.0], [1.0]]],
                      o=[[[E / (1 + E)]]], lse=[[math.log(1 + E)]]))
    v = [[[1.0, -2.0], [4.0, 0.5], [-3.0, 2.5]]]
    cases.append(dict(name="uniform", scale=0.7, q=[[[0.0, 0.0]]], k=[[[1.0, 2.0], [-1.0, 0.5], [3.0, 3.0]]],
                      v=v, o=[[[(1 + 4 - 3) / 3, (-2 + 0.5 + 2.5) / 3]]], lse=[[math.log(3)]]))
    cases.append(dict(name="causal_two_rows", scale=0.5, causal=True, q=[[[1.0], [1.0]]],
                      k=[[[0.0], [2.0]]], v=[[[1.0], [3.0]]],
                      o=[[[1.0], [(1 + 3 * E) / (1 + E)]]], lse=[[0.0, math.log(1 + E)]]))
    z = E + E ** 2 + E ** 3
    cases.append(dict(name="three_scores", scale=1.0, q=[[[1.0, 2.0]]],
                      k=[[[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]]], v=[[[1.0, 0.0], [0.0, 1.0], [2.0, 2.0]]],
                      o=[[[(E + 2 * E ** 3) / z, (E ** 2 + 2 * E ** 3) / z]]], lse=[[math.log(z)]]))
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "closed_forms.json")
    with open(out, "w") as f:
        json.dump({"source": "hand-derived closed forms of softmax(QK^T*scale)V; see make_closed_forms.py",
                   "cases": cases}, f, indent=1)


if __name__ == "__main__":
    main()
