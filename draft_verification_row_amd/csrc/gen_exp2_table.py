#!/usr/bin/env python3
"""Writes exp2_table.inc: the 512 doubles 2^(j/512), j = 0..511, each the
double nearest the exact value (computed with 60 significant decimal digits,
then rounded once to binary64), as C hexadecimal literals.  The fp64 exp of
the kernels scales its reduced polynomial by these.

    python draft_verification_row_amd/csrc/gen_exp2_table.py
"""
import os
from decimal import Decimal, getcontext

N = 512


def entries():
    getcontext().prec = 60
    ln2 = Decimal(2).ln()
    # Decimal -> str -> float rounds the 60-digit value to the nearest double
    return [float(str((ln2 * j / N).exp())) for j in range(N)]


def main():
    vals = entries()
    assert vals[0] == 1.0 and all(1.0 <= v < 2.0 for v in vals)
    lines = [f"// 2^(j/{N}), j = 0..{N - 1}, correctly rounded (written by gen_exp2_table.py)"]
    for i in range(0, N, 4):
        lines.append("    " + ", ".join(v.hex() for v in vals[i:i + 4]) + ",")
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "exp2_table.inc")
    with open(out, "w", encoding="ascii") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
