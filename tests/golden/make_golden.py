"""Writes tests/golden/diag_closed_forms.json: closed-form outputs of the Muon
update for small diagonal-like matrices, in exact rational arithmetic.

For G whose only nonzeros are G[i, i] = d_i (rows <= cols), the singular
values are |d_i|, ||G||_F = sqrt(sum d_i^2), and the Newton-Schulz result is
G with each d_i replaced by sign(d_i) p^k(|d_i| / (||G||_F + eps)), where
p(x) = a x + b x^3 + c x^5. The inputs are chosen with integer Pythagorean
norms so every quantity is rational; eps is the binary value of the float
1e-7. This script uses neither the oracle nor the GPU library.

Run: python tests/golden/make_golden.py
"""
import json
import os
from fractions import Fraction as F

EPS = F(1e-7)          # exact binary value of the double nearest 1e-7


def p_iter(x, a, b, c, k):
    for _ in range(k):
        x = a * x + b * x ** 3 + c * x ** 5
    return x


CASES = [
    # (name, rows, cols, diagonal entries, (a, b, c) as decimal strings, k)
    ("diag_3_4_quintic5", 2, 3, [3, 4], ("3.4445", "-4.7750", "2.0315"), 5),
    ("diag_3_neg4_quintic5", 2, 3, [3, -4], ("3.4445", "-4.7750", "2.0315"), 5),
    ("diag_2_3_6_cubic10", 3, 5, [2, 3, 6], ("1.5", "-0.5", "0"), 10),     # norm 7
    ("diag_1_2_2_quintic3", 3, 3, [1, 2, 2], ("3.4445", "-4.7750", "2.0315"), 3),  # norm 3
]


def main():
    out = {"source": "exact rational closed form U p^k(S/(||G||_F+eps)) V^T for diagonal G; "
                     "see make_golden.py", "eps": 1e-7, "cases": []}
    for name, rows, cols, d, abc, k in CASES:
        a, b, c = (F(s) for s in abc)
        norm2 = sum(F(x) ** 2 for x in d)
        norm = F(int(round(float(norm2) ** 0.5)))
        assert norm * norm == norm2, "pick integer-norm cases"
        vals = []
        for x in d:
            s = F(abs(x)) / (norm + EPS)
            v = p_iter(s, a, b, c, k)
            vals.append(float(v if x >= 0 else -v))
        out["cases"].append({"name": name, "rows": rows, "cols": cols, "diag": d,
                             "coeffs": [float(a), float(b), float(c)], "steps": k,
                             "out_diag": vals})
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "diag_closed_forms.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
