"""Pins of the CPU oracle's mxfp4 mode (reading R16).

"Quantization" (metalworking, newer-modes paragraph) and "Quantizing a Model
for MLX" ("Modes, bits and mixed recipes") name mxfp4 as a block-scaled float
mode with groups of 32, 4-bit codes and one exponent per group; the bit
layout is taken from the microscaling definition of that name.  Pinned here by
  * the E2M1 value set as that definition publishes it (a literal table,
    not the oracle's exponent/mantissa formula),
  * a brute force with exact rationals: the group exponent found by search
    (the X with 4 <= max|w| / 2^X < 8), every member's code by exhaustive
    nearest search over the table with the tie rule,
  * exact recovery of groups built from table values times 2^X,
  * the error bound (half a grid gap, or the saturation excess),
  * the special groups: all zero, -0 members, tiny groups at the clamp,
    non-finite members.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from group_wise_affine_aq_amd import inputs

# E2M1 magnitudes of codes 0..7 as the microscaling definition lists them
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_table():
    for c in range(8):
        assert oracle.e2m1_to_double(c) == E2M1[c]
        v = oracle.e2m1_to_double(c | 8)
        assert v == -E2M1[c] and np.signbit(v)  # code 8 is -0.0


def _group_exponent(ws):
    """X with 4 <= max|w| / 2^X < 8 by search (exact rationals), clamped."""
    amax = max(abs(Fraction(float(v))) for v in ws)
    if amax == 0:
        return -127
    X = 0
    while amax / Fraction(2) ** X >= 8:
        X += 1
    while amax / Fraction(2) ** X < 4:
        X -= 1
    return max(-127, min(127, X))


def _nearest(t):
    """Magnitude code nearest to t >= 0 by exhaustive search; a tie goes to the
    code with mantissa bit 0."""
    best = None
    for c in range(8):
        d = abs(t - Fraction(E2M1[c]))
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


def brute_force(ws):
    X = _group_exponent(ws)
    codes = []
    for v in ws:
        t = abs(Fraction(float(v))) / Fraction(2) ** X
        codes.append((8 if np.signbit(v) else 0) | _nearest(t))
    return X, codes


def _unpack(codes, K):
    return oracle.unpack(codes, K, 4)


@pytest.mark.parametrize("scale", [1.0, 1e-3, 37.0])
def test_brute_force(scale):
    w = inputs.weights(4, 128, seed=40, key=(int(scale * 1000),), outliers=True) * np.float32(scale)
    c, s = oracle.quantize_mxfp4(w)
    q = _unpack(c, 128)
    for n in range(4):
        for g in range(4):
            X, codes = brute_force(list(w[n, 32 * g:32 * g + 32]))
            assert int(s[n, g]) == X + 127, (n, g)
            assert list(q[n, 32 * g:32 * g + 32]) == codes, (n, g)


def test_ties_and_saturation():
    # max |w| = 7.5 -> X = 0; members at every midpoint of the grid and past 6
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.5, 7.0, 7.5]
    g = np.array((mids + [-m for m in mids] + [0.0] * 12)[:32], dtype=np.float32)
    c, s = oracle.quantize_mxfp4(g[None, :])
    assert int(s[0, 0]) == 127
    X, codes = brute_force(list(g))
    assert list(_unpack(c, 32)[0]) == codes
    # the ties resolve to the even mantissa: 0.25->0, 0.75->1, 1.25->1, 1.75->2,
    # 2.5->2, 3.5->4, 5->4; above 6 saturates to 6
    exp = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, 6.0, 6.0]
    got = oracle.dequantize_mxfp4_exact(c, s, 32)[0]
    assert list(got[:10]) == exp and list(got[10:20]) == [-e for e in exp]


@pytest.mark.parametrize("X", [-127, -20, -1, 0, 3, 60, 125])
def test_exact_recovery(X):
    rng = np.random.default_rng(X + 200)
    vals = rng.choice(E2M1, size=32) * rng.choice([-1.0, 1.0], size=32)
    vals[0] = 6.0 if X % 2 else 4.0  # max |w| / 2^X in [4, 8)
    w = (vals * 2.0 ** X).astype(np.float32)
    assert np.array_equal(w.astype(np.float64), vals * 2.0 ** X)  # exactly representable
    c, s = oracle.quantize_mxfp4(w[None, :])
    assert int(s[0, 0]) == X + 127
    assert np.array_equal(oracle.dequantize_mxfp4_exact(c, s, 32)[0], vals * 2.0 ** X)


def test_error_bound():
    w = inputs.weights(16, 256, seed=41, outliers=True)
    c, s = oracle.quantize_mxfp4(w)
    exact = oracle.dequantize_mxfp4_exact(c, s, 256)
    X = np.repeat(s.astype(np.int64) - 127, 32, axis=1)
    t = np.abs(w.astype(np.float64)) / np.ldexp(1.0, X)
    assert np.all((t >= 0) & (t < 8))
    grid = np.array(E2M1)
    # half the gap between the two grid points around t (beyond 6: the excess)
    hi_idx = np.clip(np.searchsorted(grid, t), 1, 7)
    half_gap = (grid[hi_idx] - grid[hi_idx - 1]) / 2
    bound = np.where(t > 6, t - 6, half_gap) * np.ldexp(1.0, X)
    assert np.all(np.abs(w.astype(np.float64) - exact) <= bound)
    # the group maximum never lands below 4 * 2^X (its exponent is X + 2)
    gmax = np.abs(w.astype(np.float64)).reshape(16, 8, 32).max(axis=2)
    assert np.all(gmax >= 4 * np.ldexp(1.0, s.astype(np.int64) - 127))


def test_special_groups():
    z = np.zeros((1, 32), dtype=np.float32)
    c, s = oracle.quantize_mxfp4(z)
    assert s[0, 0] == 0 and np.all(c == 0)                  # all zero: X = -127
    nz = -z
    c, s = oracle.quantize_mxfp4(nz)
    assert np.all(_unpack(c, 32) == 8)                       # -0 keeps its sign
    tiny = np.full((1, 32), 1e-40, dtype=np.float32)         # max|w| < 2^-125: clamped
    c, s = oracle.quantize_mxfp4(tiny)
    assert s[0, 0] == 0 and np.all(_unpack(c, 32) == 0)     # 1e-40 * 2^127 ~ 0.017 -> 0
    big = np.full((1, 32), 3e38, dtype=np.float32)           # X = 127 - 2 at the top
    c, s = oracle.quantize_mxfp4(big)
    X, codes = brute_force(list(big[0]))
    assert int(s[0, 0]) == X + 127 == 125 + 127 and list(_unpack(c, 32)[0]) == codes
    bad = np.zeros((1, 32), dtype=np.float32)
    bad[0, 5] = np.nan
    with pytest.raises(oracle.OracleError):
        oracle.quantize_mxfp4(bad)
    with pytest.raises(oracle.OracleError):
        oracle.quantize_mxfp4(np.zeros((1, 48), dtype=np.float32))


def test_dequantize_rounding():
    w = inputs.weights(8, 64, seed=42, outliers=True)
    c, s = oracle.quantize_mxfp4(w)
    exact = oracle.dequantize_mxfp4_exact(c, s, 64)
    assert np.array_equal(oracle.dequantize_mxfp4(c, s, 64, oracle.F32).astype(np.float64), exact)
    f16 = oracle.dequantize_mxfp4(c, s, 64, oracle.F16)
    assert np.array_equal(f16, exact.astype(np.float16).view(np.uint16))
    bf = oracle.dequantize_mxfp4(c, s, 64, oracle.BF16)
    for v, b in zip(exact.ravel()[:200], bf.ravel()[:200]):
        assert b == oracle.float_to_bf16_rne(np.float32(v))


def test_matmul_dense_small():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 32)); w = rng.standard_normal((3, 32))
    y, A = oracle.matmul_dense(x, w)
    for m in range(2):
        for n in range(3):
            assert abs(y[m, n] - sum(x[m, k] * w[n, k] for k in range(32))) < 1e-12
            assert abs(A[m, n] - sum(abs(x[m, k] * w[n, k]) for k in range(32))) < 1e-12
