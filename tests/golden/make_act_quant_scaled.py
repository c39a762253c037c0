"""Write act_quant_scaled.txt: per-token int8 quantization at scales other
than 1, with expected values from exact rational arithmetic only.

    python tests/golden/make_act_quant_scaled.py

Reading of the activation quantizer (symmetric per token, scale =
max|x|/127): s = fl32(max|x| / 127), then q = clamp(round_half_even(
fl32(x / s)), -127, 127), i.e. one correctly rounded fp32 division followed
by an integer rounding of that fp32 quotient.  The rows are chosen where
that reading gives a different int8 value from two plausible alternatives:
multiplying by the fp32 reciprocal fl32(x * fl32(1/s)), and rounding the
exact quotient x/s to an integer directly (no fp32 step).  An
implementation taking either alternative fails at least one entry of
every row.
"""

from __future__ import annotations

import os
import sys
from fractions import Fraction

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from exact_fp32 import f32_hex, fp32_round, round_half_even  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "act_quant_scaled.txt")
ROW = 64                     # entries per token (K % 16 == 0 for the GPU kernels too)
AMAX = (3.0, 0.7, 1234.5)    # max|x| of the three tokens (signs: +, -, +)


def expected(x: np.ndarray):
    """(s, q) of one token from the definitions above, exactly."""
    amax = max(abs(Fraction(float(v))) for v in x)
    s = fp32_round(amax / 127) if amax != 0 else Fraction(1)
    q = []
    for v in x:
        r = round_half_even(fp32_round(Fraction(float(v)) / s)) if v != 0 else 0
        q.append(max(-127, min(127, r)))
    return s, q


def cases(amax: float, sign: float):
    """Entries of one token: its maximum first, then fp32 values within a
    few ulps of (j + 1/2) * s where the reading differs from both
    alternatives, then zeros."""
    a32 = np.float32(amax)
    s = fp32_round(Fraction(float(a32)) / 127)
    inv = fp32_round(1 / s)
    row = [np.float32(sign) * a32]
    for j in range(0, 127):
        c = np.float32(float((j + Fraction(1, 2)) * s))
        for d in (-2, -1, 0, 1, 2):
            v = c
            for _ in range(abs(d)):
                v = np.nextafter(v, np.float32(np.inf if d > 0 else -np.inf))
            fx = Fraction(float(v))
            q_div = round_half_even(fp32_round(fx / s))
            q_rcp = round_half_even(fp32_round(fx * inv))
            q_exact = round_half_even(fx / s)
            if q_div != q_rcp or q_div != q_exact:
                # alternate signs so negative quotients are covered too
                row.append(v if len(row) % 2 else -v)
            if len(row) == ROW:
                return row
    row += [np.float32(0.0)] * (ROW - len(row))
    return row


def rows():
    out = []
    for amax, sign in zip(AMAX, (1.0, -1.0, 1.0)):
        x = np.array(cases(amax, sign), np.float32)
        s, q = expected(x)
        out.append((x, s, q))
    return out


def render() -> str:
    lines = [
        "# Per-token symmetric int8 quantization at scales other than 1 (written by",
        "# make_act_quant_scaled.py with exact rational arithmetic; no oracle, no GPU).",
        "# s = fl32(max|x|/127); q = clamp(round_half_even(fl32(x / s)), -127, 127).",
        "# Entries sit near (j + 1/2) * s where multiplying by fl32(1/s), or rounding",
        "# the exact x/s without the fp32 step, gives a different q.",
        "# x and s are hexadecimal binary32 literals; one x/s/q triple per token.",
    ]
    for x, s, q in rows():
        lines.append("x: " + " ".join(f32_hex(v) for v in x))
        lines.append("s: " + f32_hex(float(s)))
        lines.append("q: " + " ".join(str(v) for v in q))
    return "\n".join(lines) + "\n"


if __name__ == "__main__":
    with open(OUT, "w") as f:
        f.write(render())
    print(OUT)
