"""Exact-rational helpers for brute-force pins of the oracle (pure Python,
Fractions; nothing here is shared with the oracle or the HIP path).  Values
come from the bit fields of each format, rounding from explicit integer
arithmetic."""
from fractions import Fraction as Fr


def bf16_value(bits):
    s = (bits >> 15) & 1
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    assert e != 0xFF
    v = Fr(m, 128) * Fr(2) ** -126 if e == 0 else (1 + Fr(m, 128)) * Fr(2) ** (e - 127)
    return (-v if s else v), bool(s)


def e4m3_grid():
    out = []
    for c in range(127):
        e, m = (c >> 3) & 0xF, c & 7
        out.append((c, Fr(m, 8) * Fr(2) ** -6 if e == 0 else (1 + Fr(m, 8)) * Fr(2) ** (e - 7)))
    return out


def e2m1_grid():
    out = []
    for c in range(8):
        e, m = (c >> 1) & 3, c & 1
        out.append((c, Fr(m, 2) if e == 0 else (1 + Fr(m, 2)) * Fr(2) ** (e - 1)))
    return out


E4M3 = e4m3_grid()
E2M1 = e2m1_grid()


def nearest_code(q, grid):
    """Nearest grid code to |q| with ties to the even code, saturating."""
    a = abs(q)
    top = grid[-1][1]
    if a > top:
        a = top
    best = None
    for c, v in grid:
        d = abs(v - a)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


def floor_log2(a):
    """Largest integer e with 2^e <= a (a > 0), found by scanning."""
    e = 200
    while Fr(2) ** e > a:
        e -= 1
    return e


def round_binary(q, sig_bits, min_exp):
    """Round rational q to the binary grid with sig_bits significant bits and
    smallest quantum 2^(min_exp - sig_bits + 1) (IEEE-style subnormals),
    nearest with ties to even.  No overflow handling."""
    if q == 0:
        return Fr(0)
    a = abs(q)
    e = floor_log2(a)
    quantum_exp = max(e, min_exp) - (sig_bits - 1)
    quantum = Fr(2) ** quantum_exp
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fr(1, 2) or (rem == Fr(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * quantum
    return -r if q < 0 else r


def fp32_round(q):
    return round_binary(q, 24, -126)


def bf16_round_value(q):
    return round_binary(q, 8, -126)
