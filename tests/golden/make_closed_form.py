"""Writes tests/golden/two_keys_closed_form.json from closed forms only.

Case: B=H=1, N=2, d=1, scale=1, q=[1,2], k=[0,1], v=[1,3].
Scores S = q k^T = [[0, 1], [0, 2]]. With the softmax of two scores being a
logistic function, row i has p_i1 = e^{s}/(1+e^{s}) for s = q_i, hence
  o_i = (1 + 3 e^{q_i}) / (1 + e^{q_i}),  lse_i = log(1 + e^{q_i}).
Causal: row 0 sees key 0 only, o_0 = v_0 = 1, lse_0 = 0; row 1 as above.
The formula is the scaled dot-product attention equation of the droidorbit
FlashAttention-3 explainer (introduction), softmax(Q K^T / sqrt(d)) V with the
scale written out. Uses only the math module.
"""
import json
import math
import os

q = [1.0, 2.0]
rows = []
for i, qi in enumerate(q):
    e = math.exp(qi)
    rows.append({"o": (1.0 + 3.0 * e) / (1.0 + e), "lse": math.log(1.0 + e)})
out = {
    "citation": "droidorbit FlashAttention-3 explainer, introduction: softmax(Q K^T / sqrt(d)) V",
    "q": [[1.0], [2.0]], "k": [[0.0], [1.0]], "v": [[1.0], [3.0]], "scale": 1.0,
    "noncausal": {"o": [[r["o"]] for r in rows], "lse": [r["lse"] for r in rows]},
    "causal": {"o": [[1.0], [rows[1]["o"]]], "lse": [0.0, rows[1]["lse"]]},
}
path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "two_keys_closed_form.json")
with open(path, "w") as f:
    json.dump(out, f, indent=1)
    f.write("\n")
