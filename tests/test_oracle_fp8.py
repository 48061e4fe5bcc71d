"""Pins of the CPU oracle's mxfp8 and nvfp4 modes (readings R17, R18).

"Quantization" (metalworking, newer-modes paragraph) and "Quantizing a Model
for MLX" ("Modes, bits and mixed recipes") name mxfp8 (groups of 32, 8-bit
codes) and nvfp4 (groups of 16, 4-bit codes) as block-scaled float modes; the
ExecuTorch page lists nvfp4 as NVIDIA's FP4 format for weights, with group
size 16.  The bit layouts are taken from the microscaling (E4M3 codes, a
power-of-two scale) and NVFP4 (E2M1 codes, an E4M3 scale per 16, a tensor
scale) definitions.  Pinned here by
  * the E4M3 value set decoded by torch's float8_e4m3fn type (a library the
    oracle does not use), all 256 patterns,
  * torch's round-to-nearest-even cast to float8_e4m3fn: the mxfp8 codes of
    every member that the scale does not push past 448,
  * brute force with exact rationals: the mxfp8 group exponent by search,
    the nvfp4 group scale as the nearest E4M3 value to max|w| / (6 * 2^T)
    and every code as the nearest grid value, by exhaustive search with the
    tie rule,
  * exact recovery of groups built from grid values times their scales,
  * the special groups: zeros, -0 members, saturation at 448 and at 6,
    groups whose nvfp4 scale rounds to 0, non-finite members, bad shapes.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from group_wise_affine_aq_amd import inputs

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _torch_e4m3_table():
    import torch
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def _e4m3_mags():
    """The finite E4M3 magnitudes, codes 0..126, as exact rationals."""
    return [Fraction(float(v)) for v in _torch_e4m3_table()[:127]]


def test_e4m3_table_matches_torch():
    table = _torch_e4m3_table()
    for c in range(256):
        got, want = oracle.e4m3_to_double(c), table[c]
        if np.isnan(want):
            assert np.isnan(got), c
        else:
            assert got == want and np.signbit(got) == np.signbit(want), c
    assert oracle.e4m3_to_double(0x7E) == 448.0


def _nearest(t, mags):
    """The code whose magnitude is nearest to t >= 0 (exhaustive; a tie goes
    to the even code)."""
    best = None
    for c, m in enumerate(mags):
        d = abs(t - m)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


# ---- mxfp8 (R17) ---------------------------------------------------------------------
def _mx8_exponent(ws):
    """X with 256 <= max|w| / 2^X < 512 by search (exact rationals), clamped."""
    amax = max(abs(Fraction(float(v))) for v in ws)
    if amax == 0:
        return -127
    X = 0
    while amax / Fraction(2) ** X >= 512:
        X += 1
    while amax / Fraction(2) ** X < 256:
        X -= 1
    return max(-127, min(127, X))


def _bytes(codes):
    return np.ascontiguousarray(codes).view(np.uint8).reshape(codes.shape[0], -1)


@pytest.mark.parametrize("scale", [1.0, 3e-4, 50.0])
def test_mxfp8_brute_force(scale):
    w = inputs.weights(3, 96, seed=70, key=(int(scale * 1e4),), outliers=True) * np.float32(scale)
    c, s = oracle.quantize_mxfp8(w)
    q = _bytes(c)
    mags = _e4m3_mags()
    for n in range(3):
        for g in range(3):
            ws = list(w[n, 32 * g:32 * g + 32])
            X = _mx8_exponent(ws)
            assert int(s[n, g]) == X + 127
            for i, v in enumerate(ws):
                t = abs(Fraction(float(v))) / Fraction(2) ** X
                want = (0x80 if np.signbit(v) else 0) | _nearest(t, mags)
                assert q[n, 32 * g + i] == want, (n, g, i)


def test_mxfp8_codes_match_torch_cast():
    """Members not pushed past 448 take torch's nearest-even float8 cast."""
    import torch
    w = inputs.weights(16, 256, seed=71, outliers=True)
    c, s = oracle.quantize_mxfp8(w)
    X = np.repeat(s.astype(np.int64) - 127, 32, axis=1)
    t = np.ldexp(w.astype(np.float64), -X)          # exact: a power-of-two scaling
    ref = torch.from_numpy(t.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    inside = np.abs(t) <= 448
    assert inside.mean() > 0.95
    assert np.array_equal(_bytes(c)[inside], ref[inside])
    assert np.all(_bytes(c)[~inside] & 0x7F == 0x7E)  # the rest saturate to 448


def test_mxfp8_ties_saturation_and_recovery():
    # max |w| = 500 -> X = 0; members at E4M3 midpoints and past 448
    mids = [0.5 * (1 + 1.125), 0.5 * (1.125 + 1.25), 3 * 2.0 ** -10, 2.0 ** -10, 0.5 * (416 + 448),
            450.0, 463.0, 500.0]
    g = np.array((mids + [-m for m in mids] + [0.0] * 16)[:32], dtype=np.float32)
    c, s = oracle.quantize_mxfp8(g[None, :])
    assert int(s[0, 0]) == 127
    got = oracle.dequantize_mxfp8_exact(c, s, 32)[0]
    exp = [1.0, 1.25, 2 * 2.0 ** -9, 0.0, 448.0, 448.0, 448.0, 448.0]
    assert list(got[:8]) == exp and list(got[8:16]) == [-e for e in exp]
    # exact recovery of table values times 2^X, X from -127 to 119
    mags = np.array([float(m) for m in _e4m3_mags()])
    rng = np.random.default_rng(7)
    for X in (-127, -30, 0, 5, 119):
        vals = rng.choice(mags, 32) * rng.choice([-1.0, 1.0], 32)
        vals[0] = 448.0 if X % 2 else 256.0             # max |w| / 2^X in [256, 512)
        w = (vals * 2.0 ** X).astype(np.float32)
        assert np.array_equal(w.astype(np.float64), vals * 2.0 ** X)
        c, s = oracle.quantize_mxfp8(w[None, :])
        assert int(s[0, 0]) == X + 127
        assert np.array_equal(oracle.dequantize_mxfp8_exact(c, s, 32)[0], vals * 2.0 ** X)


def test_mxfp8_special_groups_and_errors():
    z = np.zeros((1, 32), dtype=np.float32)
    c, s = oracle.quantize_mxfp8(z)
    assert s[0, 0] == 0 and np.all(c == 0)
    c, s = oracle.quantize_mxfp8(-z)
    assert np.all(_bytes(c) == 0x80)                     # -0 keeps its sign
    big = np.full((1, 32), 3e38, dtype=np.float32)
    c, s = oracle.quantize_mxfp8(big)
    assert int(s[0, 0]) == 127 - 8 + 127                 # floor(log2 3e38) = 127
    bad = np.zeros((1, 32), dtype=np.float32)
    bad[0, 3] = np.inf
    with pytest.raises(oracle.OracleError):
        oracle.quantize_mxfp8(bad)
    with pytest.raises(oracle.OracleError):
        oracle.quantize_mxfp8(np.zeros((1, 16), dtype=np.float32))


def test_mxfp8_dequantize_rounding():
    w = inputs.weights(8, 64, seed=72, outliers=True)
    c, s = oracle.quantize_mxfp8(w)
    exact = oracle.dequantize_mxfp8_exact(c, s, 64)
    assert np.array_equal(oracle.dequantize_mxfp8(c, s, 64, oracle.F32).astype(np.float64), exact)
    assert np.array_equal(oracle.dequantize_mxfp8(c, s, 64, oracle.F16),
                          exact.astype(np.float16).view(np.uint16))
    # every code and scale byte: the table value times 2^X, NaN for the NaN codes
    codes = np.arange(256, dtype=np.uint8).reshape(8, 32).view(np.uint32)
    scales = np.array([[0], [1], [100], [127], [150], [200], [254], [255]], dtype=np.uint8)
    ex = oracle.dequantize_mxfp8_exact(codes, scales, 32)
    table = _torch_e4m3_table().reshape(8, 32)
    want = table * np.ldexp(1.0, scales.astype(np.int64) - 127)
    assert np.array_equal(np.isnan(ex), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(ex[ok], want[ok])


# ---- nvfp4 (R18) ---------------------------------------------------------------------
def _nv_brute(ws, T):
    mags = _e4m3_mags()
    amax = max(abs(Fraction(float(v))) for v in ws)
    sc = _nearest(amax / (6 * Fraction(2) ** T), mags)
    step = mags[sc] * Fraction(2) ** T
    codes = []
    for v in ws:
        mag = 0 if step == 0 else _nearest(abs(Fraction(float(v))) / step,
                                           [Fraction(e) for e in E2M1])
        codes.append((8 if np.signbit(v) else 0) | mag)
    return sc, codes


@pytest.mark.parametrize("scale,T", [(1.0, 0), (1.0, -14), (3e-4, -25), (40.0, -3), (1.0, 5)])
def test_nvfp4_brute_force(scale, T):
    w = inputs.weights(3, 64, seed=73, key=(int(scale * 1e4), T + 100), outliers=True)
    w = w * np.float32(scale)
    c, s = oracle.quantize_nvfp4(w, T)
    q = oracle.unpack(c, 64, 4)
    for n in range(3):
        for g in range(4):
            ws = list(w[n, 16 * g:16 * g + 16])
            sc, codes = _nv_brute(ws, T)
            assert int(s[n, g]) == sc, (n, g)
            assert list(q[n, 16 * g:16 * g + 16]) == codes, (n, g)


def test_nvfp4_scale_ties_saturation_and_zero():
    # max|w| / 6 exactly between E4M3 codes 56 (1.0) and 57 (1.125): tie -> 56
    g = np.zeros((4, 16), dtype=np.float32)
    g[0, 0] = 6 * 1.0625
    g[1, 0] = 6 * 1.1875                 # between 57 and 58: tie -> 58
    g[2, :] = 6 * 448 * 4.0              # beyond the largest scale: 448, codes saturate at 6
    g[3, :] = 6 * 2.0 ** -11             # below half the smallest E4M3 value: s = 0
    c, s = oracle.quantize_nvfp4(g)
    assert list(s[:, 0]) == [56, 58, 0x7E, 0]
    q = oracle.unpack(c, 16, 4)
    assert np.all(q[2] == 7)             # 4 * 448 * 6 / 448 = 24 -> 6
    assert np.all(q[3] == 0)             # s = 0: magnitude 0
    # E2M1 ties against s: members at the grid's midpoints times s = 1 (max 6)
    mids = [6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    h = np.array([mids + [-m for m in mids]], dtype=np.float32)
    c, s = oracle.quantize_nvfp4(h)
    assert int(s[0, 0]) == 56            # 6 / 6 = 1.0
    got = oracle.dequantize_nvfp4_exact(c, s, 16)[0]
    exp = [6.0, 0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]
    assert list(got[:8]) == exp and list(got[8:]) == [-e for e in exp]


@pytest.mark.parametrize("T", [-40, -14, 0, 20])
def test_nvfp4_exact_recovery(T):
    rng = np.random.default_rng(T + 300)
    mags = [float(m) for m in _e4m3_mags()]
    for sc in (8, 56, 100, 126):         # normal E4M3 scales
        vals = rng.choice(E2M1, 16) * rng.choice([-1.0, 1.0], 16)
        vals[0] = 6.0                    # max|w| / (6 * 2^T) = the scale exactly
        w = (vals * mags[sc] * 2.0 ** T).astype(np.float32)
        assert np.array_equal(w.astype(np.float64), vals * mags[sc] * 2.0 ** T)
        c, s = oracle.quantize_nvfp4(w[None, :], T)
        assert int(s[0, 0]) == sc
        assert np.array_equal(oracle.dequantize_nvfp4_exact(c, s, 16, T)[0], vals * mags[sc] * 2.0 ** T)


def test_nvfp4_error_bound_and_errors():
    w = inputs.weights(16, 128, seed=74, outliers=True)
    T = -14
    c, s = oracle.quantize_nvfp4(w, T)
    exact = oracle.dequantize_nvfp4_exact(c, s, 128, T)
    step = np.repeat(np.array([[oracle.e4m3_to_double(int(v)) for v in row] for row in s]), 16, axis=1)
    step = step * 2.0 ** T
    t = np.abs(w.astype(np.float64)) / step
    grid = np.array(E2M1)
    hi = np.clip(np.searchsorted(grid, t), 1, 7)
    bound = np.where(t > 6, t - 6, (grid[hi] - grid[hi - 1]) / 2) * step
    assert np.all(np.abs(w.astype(np.float64) - exact) <= bound * (1 + 1e-12))
    bad = np.zeros((1, 16), dtype=np.float32)
    bad[0, 1] = np.nan
    with pytest.raises(oracle.OracleError):
        oracle.quantize_nvfp4(bad)
    with pytest.raises(oracle.OracleError):
        oracle.quantize_nvfp4(np.zeros((1, 24), dtype=np.float32))
    with pytest.raises(oracle.OracleError):
        oracle.quantize_nvfp4(np.zeros((1, 16), dtype=np.float32), 101)


def test_nvfp4_dequantize_rounding():
    w = inputs.weights(8, 64, seed=75, outliers=True)
    c, s = oracle.quantize_nvfp4(w, -14)
    exact = oracle.dequantize_nvfp4_exact(c, s, 64, -14)
    assert np.array_equal(oracle.dequantize_nvfp4(c, s, 64, oracle.F32, -14).astype(np.float64),
                          exact)
    assert np.array_equal(oracle.dequantize_nvfp4(c, s, 64, oracle.F16, -14),
                          exact.astype(np.float16).view(np.uint16))
    bf = oracle.dequantize_nvfp4(c, s, 64, oracle.BF16, -14)
    for v, b in zip(exact.ravel()[:200], bf.ravel()[:200]):
        assert b == oracle.float_to_bf16_rne(np.float32(v))
