"""Constants of softmax_exp.hpp, from exact decimal arithmetic.

exp(x) = 2^(k/64) * exp(r), x = k * ln2/64 + r: ln2/64 is split as LHI + LLO
with LHI holding 36 significant bits (so that k * LHI is exact for |k| <
2^17), and 2^(j/64), j = 0..63, as the double pair hi + lo nearest to it.
Run to print the C++ definitions.
"""
from decimal import Decimal, getcontext
import struct

getcontext().prec = 80


def nearest_double(d: Decimal) -> float:
    # float(Decimal) rounds correctly to the nearest double
    return float(d)


def hexf(x: float) -> str:
    return float.hex(x)


def constants():
    ln2 = Decimal(2).ln()
    L = ln2 / 64
    # LHI: L with its 53-bit significand truncated to 36 bits
    l = nearest_double(L)
    bits = struct.unpack("<Q", struct.pack("<d", l))[0]
    bits &= ~((1 << 17) - 1)
    lhi = struct.unpack("<d", struct.pack("<Q", bits))[0]
    llo = nearest_double(L - Decimal(lhi))
    inv = nearest_double(64 / ln2)
    table = []
    for j in range(64):
        t = (ln2 * j / 64).exp()
        hi = nearest_double(t)
        lo = nearest_double(t - Decimal(hi))
        table.append((hi, lo))
    return inv, lhi, llo, table


def main():
    inv, lhi, llo, table = constants()
    print(f"constexpr double kExpInvL = {hexf(inv)};  // 64 / ln 2")
    print(f"constexpr double kExpLhi = {hexf(lhi)};   // ln 2 / 64, leading 36 bits")
    print(f"constexpr double kExpLlo = {hexf(llo)};   // ln 2 / 64 - kExpLhi")
    print("// 2^(j/64) = hi + lo, j = 0..63")
    print("static __device__ const double kExp2Table[64][2] = {")
    for hi, lo in table:
        print(f"    {{{hexf(hi)}, {hexf(lo)}}},")
    print("};")


if __name__ == "__main__":
    main()
