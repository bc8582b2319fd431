"""Pins of the oracle's key codec against things other than itself: numpy's
direct fp64->fp16 rounding, closed forms of the angle grid, 300-bit mpmath
angles (random and adversarially close to rounding boundaries), exact
rational checks of the magnitude rounding, numpy bit packing, and the
per-pair error bound of the quantiser.

Codec definition followed (the paper's abstract on the newx.sg / searcharxiv
pages, Abstract: a key is a scalar radius plus compact angle codes; the bit
layout is this library's): adjacent pairs, angle grid -pi + c 2pi/2^b,
magnitude grid c/(2^b - 1), nearest with ties rounded up."""
import json
import os
from fractions import Fraction

import mpmath
import numpy as np
import pytest

from oracle import oracle as O
from tests.util import near_boundary_pairs as _near_boundary_pairs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- fp16 radius
def test_fp16_matches_numpy_direct_rounding():
    rng = np.random.default_rng(1)
    e = rng.uniform(-30, 16, 300000)
    x = rng.uniform(1, 2, e.size) * 2.0 ** e
    x = x[x < 65504]
    ref = x.astype(np.float16).view(np.uint16)   # numpy rounds fp64 -> fp16 directly
    assert np.array_equal(O.f64_to_f16(x), ref)


def test_fp16_hand_cases():
    cases = {
        1 + 2 ** -11: 0x3C00,          # tie between 1 and 1+2^-10 -> even (1)
        1 + 3 * 2 ** -11: 0x3C02,      # tie between mantissa 1 and 2 -> 2
        1 + 2 ** -11 + 2 ** -40: 0x3C01,  # just above the tie; via fp32 it would be 1.0
        2 ** -25: 0x0000,              # half the smallest subnormal: tie -> even (0)
        3 * 2 ** -25: 0x0002,          # tie between 1 and 2 subnormal quanta -> 2
        2 ** -14 - 2 ** -25: 0x0400,   # tie between largest subnormal and 2^-14 -> 2^-14
        65504.0: 0x7BFF,
        65519.99: 0x7BFF,
        65520.0: 0x7BFF,               # would round to inf: saturates
        1e10: 0x7BFF,
        0.0: 0x0000,
    }
    for x, h in cases.items():
        assert O.f64_to_f16(np.array([x]))[0] == h, (x, hex(h))


# ---------------------------------------------------------------- angle codes
def _key_from_pairs(pairs):
    k = np.zeros(128, np.float32)
    for j, (x, y) in enumerate(pairs):
        k[2 * j], k[2 * j + 1] = x, y
    return k


def _theta_codes(pairs, tb, sb=4):
    pairs = list(pairs) + [(0.0, 0.0)] * (64 - len(pairs))
    _, th, s, st = O.encode(_key_from_pairs(pairs), tb, sb)
    assert st == O.OK
    return th[0], s[0]


@pytest.mark.parametrize("tb", [2, 3, 4, 8])
def test_theta_axes_closed_form(tb):
    N = 1 << tb
    th, _ = _theta_codes([(1, 0), (0, 1), (-1, 0), (0, -1), (0, 0), (-1.0, -0.0)], tb)
    # angle 0 -> N/2, pi/2 -> 3N/4, pi -> 0 (wraps), -pi/2 -> N/4, zero pair -> N/2,
    # (-1, -0) has atan2 = -pi -> code 0
    assert list(th[:6]) == [N // 2, 3 * N // 4, 0, N // 4, N // 2, 0]


def test_theta_two_bit_diagonal_ties():
    with open(os.path.join(GOLDEN, "theta2_diagonal_ties.json")) as f:
        g = json.load(f)
    pairs = [tuple(p) for p in g["pairs"]]
    th, _ = _theta_codes(pairs, 2, 3)
    assert list(th[: len(pairs)]) == g["codes"]


def _mp_theta_code(x, y, tb, prec=300):
    N = 1 << tb
    if x == 0 and y == 0:
        return N // 2
    with mpmath.workprec(prec):
        t = (mpmath.atan2(mpmath.mpf(float(y)), mpmath.mpf(float(x))) + mpmath.pi) / (2 * mpmath.pi) * N
        c = int(mpmath.floor(t + mpmath.mpf(0.5)))
        frac_dist = abs(t - mpmath.floor(t) - mpmath.mpf(0.5))
    return c % N, frac_dist


@pytest.mark.parametrize("tb", [2, 3, 4, 8])
def test_theta_random_vs_mpmath(tb):
    rng = np.random.default_rng(10 + tb)
    keys = (rng.standard_normal((40, 128)) * np.exp(rng.standard_normal((40, 128)))).astype(np.float32)
    _, th, _, st = O.encode(keys, tb, 4)
    assert st == O.OK
    for i in range(keys.shape[0]):
        for j in range(64):
            c, dist = _mp_theta_code(keys[i, 2 * j], keys[i, 2 * j + 1], tb, prec=120)
            assert dist > 1e-20      # random inputs are never exact ties
            assert th[i, j] == c


@pytest.mark.parametrize("tb", [3, 4, 8])
def test_theta_adversarial_boundaries(tb):
    pairs = _near_boundary_pairs(tb)
    in_band = 0
    for start in range(0, len(pairs), 64):
        chunk = pairs[start:start + 64]
        th, _ = _theta_codes(chunk, tb)
        for j, (x, y) in enumerate(chunk):
            c, dist = _mp_theta_code(x, y, tb)
            assert dist > mpmath.mpf(2) ** -90
            in_band += dist < mpmath.mpf(2) ** -30
            assert th[j] == c, (x, y, tb)
    # the construction really exercises the close-to-boundary path
    assert in_band > len(pairs) // 4


def test_theta_two_bit_near_diagonal():
    pairs = []
    for x in [1.0, 3.5, 1e-20, 7e30]:
        xf = np.float32(x)
        for y in [np.nextafter(xf, np.float32(0)), np.nextafter(xf, np.float32(np.inf))]:
            for sx in (1, -1):
                for sy in (1, -1):
                    pairs.append((sx * float(xf), sy * float(y)))
    th, _ = _theta_codes(pairs, 2, 3)
    for j, (x, y) in enumerate(pairs):
        c, dist = _mp_theta_code(x, y, 2)
        assert dist > 1e-12
        assert th[j] == c


# ------------------------------------------------------------ magnitude codes
def _exact_energy(x, y):
    return Fraction(float(x)) ** 2 + Fraction(float(y)) ** 2


@pytest.mark.parametrize("sb", [3, 4, 8])
def test_magnitude_rounding_exact(sb):
    rng = np.random.default_rng(20 + sb)
    keys = (rng.standard_normal((30, 128)) * np.exp(rng.standard_normal((30, 128)))).astype(np.float32)
    keys[0, :] = 0
    keys[0, 10] = 3.0                      # a single non-zero pair -> code L
    _, _, s, st = O.encode(keys, 4, sb)
    assert st == O.OK
    L = (1 << sb) - 1
    for i in range(keys.shape[0]):
        e = [_exact_energy(keys[i, 2 * j], keys[i, 2 * j + 1]) for j in range(64)]
        R2 = sum(e)
        for j in range(64):
            with mpmath.workprec(200):
                v = L * mpmath.sqrt(mpmath.mpf(e[j].numerator) / e[j].denominator
                                    / (mpmath.mpf(R2.numerator) / R2.denominator))
            # the oracle rounds the fp64 tree-summed norm; that perturbs v by
            # far less than 1e-9, so the nearest-integer rule must hold to that slack
            assert abs(v - int(s[i, j])) <= 0.5 + 1e-9
    assert s[0, 5] == L


@pytest.mark.parametrize("sb", [3, 4, 8])
def test_magnitude_exact_ties_round_up(sb):
    # four pairs (1, 0): R2 = 4 exactly, each s = 1/2, so L*s = L/2 is a tie
    # (L odd) and rounds up to (L+1)/2; the remaining zero pairs get 0.
    L = (1 << sb) - 1
    _, s = _theta_codes([(1.0, 0.0)] * 4, 4, sb)
    assert list(s[:4]) == [(L + 1) // 2] * 4
    assert (s[4:] == 0).all()


def test_zero_key():
    r16, th, s, st = O.encode(np.zeros((1, 128), np.float32), 4, 4)
    assert st == O.OK and r16[0] == 0 and (th == 8).all() and (s == 0).all()


def test_nonfinite_key_rejected():
    k = np.zeros((1, 128), np.float32)
    k[0, 7] = np.inf
    assert O.encode(k, 4, 4)[3] == O.EINVAL
    k[0, 7] = np.nan
    assert O.encode(k, 4, 4)[3] == O.EINVAL


# ------------------------------------------------------------------- radius
def test_radius_exact_sums():
    rng = np.random.default_rng(3)
    keys = rng.integers(-50, 51, (200, 128)).astype(np.float32)
    r16, _, _, _ = O.encode(keys, 4, 4)
    R2 = (keys.astype(np.float64) ** 2).sum(1)      # exact: small integers
    ref = np.sqrt(R2).astype(np.float16).view(np.uint16)
    assert np.array_equal(r16, ref)


def test_radius_random_vs_mpmath():
    rng = np.random.default_rng(4)
    keys = (rng.standard_normal((300, 128)) * 3).astype(np.float32)
    r16, _, _, _ = O.encode(keys, 4, 4)
    for i in range(keys.shape[0]):
        with mpmath.workprec(200):
            n = mpmath.sqrt(mpmath.fsum(mpmath.mpf(float(v)) ** 2 for v in keys[i]))
        assert r16[i] == np.float16(float(n)).view(np.uint16)


def test_radius_saturates():
    k = np.full((1, 128), 1e30, np.float32)
    r16, _, _, _ = O.encode(k, 4, 4)
    assert r16[0] == 0x7BFF


# ------------------------------------------------------------- bit strings
@pytest.mark.parametrize("b", [2, 3, 4, 8])
def test_bitstring_matches_numpy(b):
    rng = np.random.default_rng(b)
    codes = rng.integers(0, 1 << b, 64).astype(np.uint16)
    bits = ((codes[:, None].astype(np.int64) >> np.arange(b)) & 1).astype(np.uint8).reshape(-1)
    ref = np.packbits(bits, bitorder="little")
    got = O.bits_put(codes, b)
    assert np.array_equal(got, ref)
    assert np.array_equal(O.bits_get(got, b, 64), codes)


# ------------------------------------------------------- quantiser as a whole
@pytest.mark.parametrize("tier", [0, 1, 2])
def test_pair_error_bound_and_idempotence(tier):
    tb, sb = O.TIER_BITS[tier]
    rng = np.random.default_rng(40 + tier)
    keys = (rng.standard_normal((50, 128)) * np.exp(0.5 * rng.standard_normal(128))).astype(np.float32)
    r16, th, s, _ = O.encode(keys, tb, sb)
    N, L = 1 << tb, (1 << sb) - 1
    k64 = keys.astype(np.float64)
    r = np.sqrt((k64 ** 2).sum(1))
    u = k64 / r[:, None]
    ux, uy = u[:, 0::2], u[:, 1::2]
    sj = np.hypot(ux, uy)
    thq = -np.pi + th * 2 * np.pi / N
    uhx, uhy = s / L * np.cos(thq), s / L * np.sin(thq)
    err = np.hypot(ux - uhx, uy - uhy)
    bound = 2 * sj * np.sin(np.pi / N / 2) + 1 / (2 * L) + 1e-12
    assert (err <= bound).all()
    # re-encoding the dequantised key reproduces the angle codes wherever the
    # magnitude code is non-zero (the dequantised angle is a grid point)
    rhat = np.asarray(r16, np.uint16).view(np.float16).astype(np.float64)
    k2 = np.zeros_like(k64)
    k2[:, 0::2] = rhat[:, None] * uhx
    k2[:, 1::2] = rhat[:, None] * uhy
    _, th2, _, _ = O.encode(k2.astype(np.float32), tb, sb)
    mask = s > 0
    assert np.array_equal(th2[mask], th[mask])
