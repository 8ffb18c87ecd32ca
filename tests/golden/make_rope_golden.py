"""Writes rope_unit_rotations.json: closed-form RoPE rotations of unit vectors.

For a unit vector e_{2i} the rotary embedding of position t must return
(cos phi, sin phi) in elements (2i, 2i+1) and zero elsewhere, with phi = t * base^(-2i/D)
(the reading of the rotary embedding that "Show HN: NanoEuler", section 2, and
"Tiny Hackable CUDA Language Model Implementation", section 1, apply to queries and keys).
The angles are chosen so that phi is a round number (or sqrt 2), and cos/sin are evaluated
here by their power series in 120-digit decimal arithmetic -- independent of libm and of
both implementations under test.  Run: python tests/golden/make_rope_golden.py
"""
import json
import os
from decimal import Decimal, getcontext

getcontext().prec = 120


def cos_sin(x: Decimal):
    c, s, term, n = Decimal(0), Decimal(0), Decimal(1), 0
    while True:
        r = n % 4
        if r == 0:
            c += term
        elif r == 1:
            s += term
        elif r == 2:
            c -= term
        else:
            s -= term
        n += 1
        term = term * x / n
        if abs(term) < Decimal(10) ** -60 and n > 5:
            return c, s


CASES = [
    # base, D, t, pair i, exact angle (decimal string)
    (10000.0, 8, 100, 0, "100"),
    (10000.0, 8, 100, 1, "10"),
    (10000.0, 8, 100, 2, "1"),
    (10000.0, 8, 100, 3, "0.1"),
    (10000.0, 2, 7, 0, "7"),
    (500000.0, 4, 1000, 1, None),  # angle = 1000 / sqrt(500000) = sqrt(2)
]


def main():
    out = []
    for base, D, t, i, ang in CASES:
        a = Decimal(ang) if ang is not None else Decimal(2).sqrt()
        c, s = cos_sin(a)
        out.append({"base": base, "D": D, "t": t, "pair": i, "angle": str(a)[:40],
                    "cos": float(c), "sin": float(s)})
    doc = {
        "what": "RoPE of unit vectors e_{2i} and e_{2i+1} at position t (pos0 = 0)",
        "source": "closed form of the rotary embedding applied to queries and keys "
                  "(Show HN: NanoEuler, section 2; Tiny Hackable CUDA Language Model "
                  "Implementation, section 1); adjacent pairs, theta_i = base^(-2i/D)",
        "generator": "tests/golden/make_rope_golden.py (decimal power series)",
        "cases": out,
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "rope_unit_rotations.json")
    with open(path, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
