"""Exact-rational NVFP4 micro-oracle -- TEST INFRASTRUCTURE ONLY.

A second, independent formulation of the quantizer for tiny inputs: every
value is a Python Fraction, and each fp32 step is an explicit rounding of an
exact rational to the nearest binary32 (ties to even, subnormals included).
It shares nothing with the C oracle except the recipe, so it pins the C
oracle's use of hardware float operations (operation order, division vs
reciprocal, single rounding per step).

Recipe (two-level microscaling with an FP32 tensor scale and E4M3 block
scales over 16-value blocks of E2M1 values; axbrief.com, "NVFP4: how NVIDIA
pre-trained a 12B model on 10 trillion tokens", section "E2M1 format and
two-level scaling"):
  g  = RN32(amax / 2688);  d6 = RN32(6 g)
  s  = E4M3_RNE_SAT(RN32(bamax / d6))   (0 if d6 == 0)
  d  = RN32(s g);  code = sign | E2M1_RNE_SAT(RN32(|x| / d))  (signed zero if d == 0)
"""
from fractions import Fraction as F

INF = float("inf")
E2M1 = [F(0), F(1, 2), F(1), F(3, 2), F(2), F(3), F(4), F(6)]
E4M3 = [F(m, 512) for m in range(8)] + [
    (1 + F(m, 8)) * F(2) ** (e - 7) for e in range(1, 16) for m in range(8)
][:0x7F - 8]
assert len(E4M3) == 0x7F and E4M3[-1] == 448


def rn32(r: F) -> F:
    """Round a rational to the nearest binary32 value (ties to even).

    Returns a Fraction; overflow beyond the largest finite value rounds to
    infinity per IEEE-754, represented here by float('inf') (it compares and
    divides correctly against Fractions: v / inf == 0)."""
    if r == 0:
        return F(0)
    sign = -1 if r < 0 else 1
    a = abs(r)
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if F(2) ** e > a:
        e -= 1
    while F(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)                       # subnormal range shares the 2^-149 quantum
    quantum = F(2) ** (e - 23)
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > F(1, 2) or (rem == F(1, 2) and fl % 2 == 1):
        fl += 1
    v = fl * quantum
    if v >= F(2) ** 128:                   # overflow -> inf
        return sign * INF
    return sign * v


def _nearest(v: F, grid, sat_code):
    if v > grid[sat_code]:
        return sat_code
    best, bestd = 0, abs(v - grid[0])
    for k in range(1, sat_code + 1):
        d = abs(v - grid[k])
        if d < bestd or (d == bestd and k % 2 == 0):
            best, bestd = k, d
    return best


def e2m1_rne_sat(y: F) -> int:
    return _nearest(y, E2M1, 7)


def e4m3_rne_sat(v: F) -> int:
    if v >= 448:
        return 0x7E
    return _nearest(v, E4M3, 0x7E)


def bf16_to_fraction(bits: int) -> F:
    sign = -1 if bits & 0x8000 else 1
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    if e == 0xFF:
        raise ValueError("non-finite bf16")
    if e == 0:
        return sign * F(m) * F(2) ** -133
    return sign * (1 + F(m, 128)) * F(2) ** (e - 127)


def quantize_rows(x_bits, g=None):
    """x_bits: list of rows (lists of bf16 bit patterns), len(row) % 16 == 0.

    Returns (codes per row, scale bytes per row, g as Fraction)."""
    xs = [[bf16_to_fraction(b) for b in row] for row in x_bits]
    if g is None:
        amax = max((abs(v) for row in xs for v in row), default=F(0))
        g = rn32(amax / 2688)
    d6 = rn32(6 * g)
    codes, scales = [], []
    for row, brow in zip(xs, x_bits):
        rc, rs = [], []
        for b in range(len(row) // 16):
            blk = row[16 * b:16 * b + 16]
            bb = brow[16 * b:16 * b + 16]
            bamax = max(abs(v) for v in blk)
            sbyte = 0 if d6 == 0 else e4m3_rne_sat(rn32(bamax / d6))
            d = rn32(E4M3[sbyte] * g)
            rs.append(sbyte)
            for v, bits in zip(blk, bb):
                sign = (bits >> 15) & 1
                if d == 0:
                    rc.append(sign << 3)
                else:
                    rc.append((sign << 3) | e2m1_rne_sat(rn32(abs(v) / d)))
        codes.append(rc)
        scales.append(rs)
    return codes, scales, g


def dequant_value(code: int, sbyte: int, g: F) -> F:
    """RN32((E2M1(code) * s) * g) with the sign of code bit 3 (exact rational)."""
    v = rn32(E2M1[code & 7] * E4M3[sbyte] * g)
    return -v if code & 8 else v


# ---------------------------------------------------------------- MXFP4
# 32-value blocks with one power-of-two scale 2^X (E8M0 byte X + 127) and no
# tensor scale; X = floor(log2(block amax)) - 2 clamped to [-127, 127] (the
# published Microscaling rule; an all-zero block takes X = -127).
def floor_log2(a: F) -> int:
    """The integer e with 2^e <= a < 2^(e+1), for a > 0, from the bit lengths
    of a's numerator and denominator."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    return e if F(2) ** e <= a else e - 1


def mx_quantize_rows(x_bits):
    """x_bits: list of rows of bf16 bit patterns, len(row) % 32 == 0.
    Returns (codes per row, scale bytes per row)."""
    codes, scales = [], []
    for brow in x_bits:
        row = [bf16_to_fraction(b) for b in brow]
        rc, rs = [], []
        for b in range(len(row) // 32):
            blk, bb = row[32 * b:32 * b + 32], brow[32 * b:32 * b + 32]
            bamax = max(abs(v) for v in blk)
            X = -127 if bamax == 0 else min(127, max(-127, floor_log2(bamax) - 2))
            rs.append(X + 127)
            for v, bits in zip(blk, bb):
                rc.append((((bits >> 15) & 1) << 3) | e2m1_rne_sat(rn32(abs(v) / F(2) ** X)))
        codes.append(rc)
        scales.append(rs)
    return codes, scales


# ---------------------------------------------------------------- variants
def quantize_values(rows, draws=None, tiles=False):
    """The recipe on exact rational inputs (e.g. RHT outputs, which are fp32
    values): rows is a list of rows of Fractions (len % 16 == 0).  draws, if
    given, holds one 16-bit uniform per element (stochastic rounding of the
    element step); tiles=True takes each block's scale from its 16x16 tile.
    Signs come from the values' signs (negative zero is not representable
    here; callers avoid it).  Returns (codes, scales, g)."""
    amax = max((abs(v) for row in rows for v in row), default=F(0))
    g = rn32(amax / 2688)
    d6 = rn32(6 * g)
    codes, scales = [], []
    for r, row in enumerate(rows):
        rc, rs = [], []
        for b in range(len(row) // 16):
            if tiles:
                r0 = r - r % 16
                bamax = max(abs(v) for rr in range(r0, r0 + 16) for v in rows[rr][16 * b:16 * b + 16])
            else:
                bamax = max(abs(v) for v in row[16 * b:16 * b + 16])
            sbyte = 0 if d6 == 0 else e4m3_rne_sat(rn32(bamax / d6))
            d = rn32(E4M3[sbyte] * g)
            rs.append(sbyte)
            for i, v in enumerate(row[16 * b:16 * b + 16]):
                sign = 8 if v < 0 else 0
                if d == 0:
                    rc.append(sign)
                    continue
                y = rn32(abs(v) / d)
                if draws is None:
                    rc.append(sign | e2m1_rne_sat(y))
                else:
                    rc.append(sign | e2m1_sr(y, draws[r][16 * b + i]))
        codes.append(rc)
        scales.append(rs)
    return codes, scales, g


def e2m1_sr(y: F, u16: int) -> int:
    """Stochastic rounding onto the E2M1 magnitudes: up with probability
    (y - lo) / (hi - lo), decided by u16 / 2^16; 6 and above give 6."""
    if y >= 6:
        return 7
    lo = max(k for k in range(8) if E2M1[k] <= y)
    return lo + 1 if F(u16, 65536) < (y - E2M1[lo]) / (E2M1[lo + 1] - E2M1[lo]) else lo
