"""Pins for the oracle's bf16 soft-float.

Independent references: an exhaustive table of every finite bf16 value
(numpy, built from the bit layout), torch's own float32 -> bfloat16
round-to-nearest-even, exact rational sums, and the worked addition example of
91haoming.cn/news/show-608006, section 四.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests.brute import bf16_value

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _finite_table():
    """Sorted finite non-negative bf16 values and their codes (from the bit layout)."""
    codes = np.arange(0, 0x7F80, dtype=np.uint32)           # +0 .. max finite
    vals = (codes << 16).view(np.float32).astype(np.float64)
    return vals, codes.astype(np.uint16)


VALS, CODES = _finite_table()


def _brute_round(x: Fraction, mode: str) -> int:
    """Round an exact rational to bf16 by searching the table of all values."""
    neg = x < 0
    a = -x if neg else x
    sign = 0x8000 if neg else 0
    if a == 0:
        return sign
    af = float(a)
    i = int(np.searchsorted(VALS, af, side="right")) - 1     # candidate lower neighbour
    i = max(0, min(i, len(VALS) - 1))
    while i > 0 and Fraction(VALS[i]) > a:
        i -= 1
    while i + 1 < len(VALS) and Fraction(VALS[i + 1]) <= a:
        i += 1
    lo = Fraction(VALS[i])
    if lo == a:
        return sign | int(CODES[i])
    hi_code = int(CODES[i]) + 1                              # 0x7F80 = inf above the max
    hi = Fraction(2 ** 128) if hi_code == 0x7F80 else Fraction(VALS[i + 1])
    mid = (lo + hi) / 2
    if mode == "rtz":
        pick = i
    elif mode == "rd":
        pick = i if not neg else None
    elif mode == "ru":
        pick = None if not neg else i
    elif mode == "rna":
        pick = i if a < mid else None
    else:  # rne
        if a < mid:
            pick = i
        elif a > mid:
            pick = None
        else:
            pick = i if int(CODES[i]) % 2 == 0 else None
    return sign | (int(CODES[pick]) if pick is not None else hi_code)


def test_decode_matches_bit_layout_exhaustively():
    allb = np.arange(65536, dtype=np.uint32)
    ref = (allb << 16).view(np.float32).astype(np.float64)
    got = oracle.bf16_decode(allb.astype(np.uint16))
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.all(np.isnan(got[np.isnan(ref)]))
    assert np.array_equal(np.isinf(got), np.isinf(ref))


def test_round_trip_every_finite_code():
    allb = np.arange(65536, dtype=np.uint32)
    vals = (allb << 16).view(np.float32).astype(np.float64)
    fin = np.isfinite(vals)
    for mode in oracle.MODES:
        back = oracle.bf16_from_double(vals[fin], mode)
        assert np.array_equal(back, allb[fin].astype(np.uint16)), mode


def test_rne_agrees_with_torch_float32_conversion():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    ours = oracle.bf16_from_double(x.astype(np.float64), "rne")
    theirs = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    # torch saturates nothing and keeps NaN handling aside; all inputs here are finite
    assert np.array_equal(ours, theirs)


@pytest.mark.parametrize("mode", list(oracle.MODES))
def test_rounding_modes_against_table_search(mode):
    rng = np.random.default_rng(11)
    xs = list(rng.standard_normal(400) * np.exp2(rng.integers(-140, 128, size=400)))
    # exact halfway points and neighbours of codes, both signs
    for c in rng.integers(1, 0x7F7F, size=200):
        lo = float(VALS[c])
        hi = float(VALS[c + 1])
        xs += [(lo + hi) / 2, -(lo + hi) / 2, np.nextafter((lo + hi) / 2, 0.0), np.nextafter((lo + hi) / 2, 10.0)]
    xs += [float(VALS[-1]) * (1 + 2 ** -9), float(VALS[-1]) * (1 + 2 ** -10), 2.0 ** -134, 3 * 2.0 ** -135]
    for x in xs:
        if not np.isfinite(x):
            continue
        want = _brute_round(Fraction(float(x)), mode)
        got = int(oracle.bf16_from_double(np.array([x]), mode)[0])
        assert got == want, (x, mode, hex(got), hex(want))


@pytest.mark.parametrize("mode", list(oracle.MODES))
def test_addition_is_one_rounding_of_the_exact_sum(mode):
    rng = np.random.default_rng(13)
    a = rng.integers(0, 0x7F80, size=3000).astype(np.uint16) | (rng.integers(0, 2, size=3000) << 15).astype(np.uint16)
    # bias toward close exponents, where significand overflow and cancellation happen
    b = (a.astype(np.int32) + rng.integers(-300, 300, size=3000)).clip(0, 0x7F7F).astype(np.uint16)
    b |= (rng.integers(0, 2, size=3000) << 15).astype(np.uint16)
    for x, y in zip(a, b):
        exact = bf16_value(int(x)) + bf16_value(int(y))
        assert oracle.bf16_add(int(x), int(y), mode) == _brute_round(exact, mode) or exact == 0


def test_worked_example_from_the_pages():
    g = json.load(open(os.path.join(GOLDEN, "worked_bf16_addition.json")))
    a_bits = int(g["operands"]["a_bits"], 16)
    b_bits = int(g["operands"]["b_bits"], 16)
    assert float(bf16_value(a_bits)) == g["operands"]["a"]
    assert float(bf16_value(b_bits)) == g["operands"]["b"]
    assert bf16_value(a_bits) + bf16_value(b_bits) == Fraction(g["exact_sum"])
    for mode, want in g["results"].items():
        got = oracle.bf16_add(a_bits, b_bits, mode)
        assert got == int(want, 16), (mode, hex(got))
    # significand overflow: the result's exponent is one above the operands'
    e_op = (a_bits >> 7) & 0xFF
    e_res = (oracle.bf16_add(a_bits, b_bits, "rne") >> 7) & 0xFF
    assert e_res == e_op + 1
    # a further negative addend sets the sticky bit: nearest-even then goes more negative
    s = g["sticky_case"]
    hi = g["exact_sum"] + s["extra_addend"]                  # exact in double
    assert Fraction(hi) == Fraction(g["exact_sum"]) + Fraction(s["extra_addend"])
    assert oracle.bf16_round2(hi, 0.0, "rne") == int(s["rne_bits_of_three_term_sum"], 16)


def test_round2_uses_the_low_part():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: the low part decides
    h = 1.0 + 2.0 ** -8
    assert oracle.bf16_round2(h, 0.0, "rne") == 0x3F80
    assert oracle.bf16_round2(h, 2.0 ** -80, "rne") == 0x3F81
    assert oracle.bf16_round2(h, -2.0 ** -80, "rna") == 0x3F80
    assert oracle.bf16_round2(1.0, -2.0 ** -80, "rd") == 0x3F7F
    assert oracle.bf16_round2(1.0, -2.0 ** -80, "rtz") == 0x3F7F
    assert oracle.bf16_round2(1.0, 2.0 ** -80, "ru") == 0x3F81
    assert oracle.bf16_round2(-1.0, 2.0 ** -80, "rd") == 0xBF80
