"""Print the table of 2^(j/256), j = 0..255, correctly rounded to fp64, as C++.

The values are computed with 60 significant decimal digits and rounded once
(Python's float() of a decimal string rounds correctly), so each entry is
within half an ulp of 2^(j/256). The output is pasted into specv_math.h.
"""

from decimal import Decimal, getcontext

N = 256  # entries: 2^(j/N)


def table():
    getcontext().prec = 60
    return [float(str(Decimal(2) ** (Decimal(j) / Decimal(N)))) for j in range(N)]


if __name__ == "__main__":
    vals = table()
    print(f"constexpr double kExp2Table[{N}] = {{")
    for i in range(0, N, 4):
        print("    " + ", ".join(v.hex() for v in vals[i:i + 4]) + ",")
    print("};")
