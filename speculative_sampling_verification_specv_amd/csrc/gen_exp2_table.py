"""Print the table of 2^(j/64), j = 0..63, correctly rounded to fp64, as C++.

The values are computed with 60 significant decimal digits and rounded once
(Python's float() of a decimal string rounds correctly), so each entry is
within half an ulp of 2^(j/64). The output is pasted into specv_math.h.
"""

from decimal import Decimal, getcontext


def table():
    getcontext().prec = 60
    return [float(str(Decimal(2) ** (Decimal(j) / Decimal(64)))) for j in range(64)]


if __name__ == "__main__":
    vals = table()
    print("constexpr double kExp2Table[64] = {")
    for i in range(0, 64, 4):
        print("    " + ", ".join(v.hex() for v in vals[i:i + 4]) + ",")
    print("};")
