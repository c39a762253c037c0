"""Write epilogue_order.txt: the output rescale y = ((float)acc * s_x) * alpha
in binary32, with expected values from exact rational arithmetic only.

    python tests/golden/make_epilogue_order.py

Reading of the single float rescale after the integer add tree: the exact
int32 sum is converted to fp32 (exact below 2^24), multiplied by the token's
scale and rounded, then multiplied by the row's alpha and rounded.  The cases
are seeded draws kept only where both other orders, (acc * alpha) * s_x and
acc * (s_x * alpha), round to a different binary32 value, so an oracle or
kernel taking either of them fails every case.
"""

from __future__ import annotations

import os
import sys
from fractions import Fraction

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from exact_fp32 import f32_hex, fp32_round  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "epilogue_order.txt")
CASES = 48


def rows():
    rng = np.random.default_rng(20240611)
    out = []
    while len(out) < CASES:
        acc = int(rng.integers(-1_056_768, 1_056_769))       # |acc| <= 384 * K/4 at K <= 11008
        s = np.float32(rng.uniform(1e-3, 0.1))
        a = np.float32(rng.uniform(1e-3, 0.2))
        A, S, Al = Fraction(acc), Fraction(float(s)), Fraction(float(a))
        y = fp32_round(fp32_round(A * S) * Al)
        other1 = fp32_round(fp32_round(A * Al) * S)
        other2 = fp32_round(A * fp32_round(S * Al))
        if acc != 0 and y != other1 and y != other2:
            out.append((acc, s, a, y))
    return out


def render() -> str:
    lines = [
        "# y = ((float)acc * s_x) * alpha in binary32 (written by make_epilogue_order.py",
        "# with exact rational arithmetic; no oracle, no GPU).  Each case is one where",
        "# (acc * alpha) * s_x and acc * (s_x * alpha) both round to another value.",
        "# Columns: acc (int32), s_x, alpha, y (hexadecimal binary32 literals).",
    ]
    for acc, s, a, y in rows():
        lines.append(f"case: {acc} {f32_hex(s)} {f32_hex(a)} {f32_hex(float(y))}")
    return "\n".join(lines) + "\n"


if __name__ == "__main__":
    with open(OUT, "w") as f:
        f.write(render())
    print(OUT)
