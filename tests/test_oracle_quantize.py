"""Pins of the CPU oracle quantizer.

The quantizer is an encoding (readings R1, R2 in the oracle's header):
per group of G weights along a row, bias = the group minimum rounded down to
fp16, scale = the smallest fp16 whose top grid point reaches the group
maximum, code = nearest grid index with ties to even.  These tests pin it by
  * an exact brute force with rational arithmetic on tiny inputs,
  * exact invariants (bias <= members, |w - w^| <= s/2, minimality),
  * grid-exact recovery and half-step ties,
  * group locality ("Quantizing a Model for MLX", 'What MLX quantization
    stores': an outlier can only distort its own group),
  * the degenerate groups (constant, all-zero, -0) and range errors.
"""
import bisect
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from group_wise_affine_aq_amd import inputs

# every finite fp16 value, ascending (numpy decodes the patterns)
_pos = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
FP16_SORTED = sorted(set((-_pos).tolist()) | set(_pos.tolist()))


def _h(v):
    return int(np.float16(v).view(np.uint16))


def brute_force_group(ws, bits):
    """Exact answer for one group, by enumeration with rationals."""
    L = (1 << bits) - 1
    lo, hi = Fraction(min(ws)), Fraction(max(ws))
    # bias: the largest fp16 value <= lo
    b = Fraction(FP16_SORTED[bisect.bisect_right(FP16_SORTED, lo) - 1])
    # scale: the smallest fp16 value >= (hi - b) / L
    target = (hi - b) / L
    s = Fraction(FP16_SORTED[bisect.bisect_left(FP16_SORTED, target)])
    assert s >= 0
    qs = []
    for w in ws:
        w = Fraction(w)
        if s == 0:
            qs.append(0)
            continue
        # nearest grid point over all q, ties broken towards the even q
        qs.append(min(range(L + 1), key=lambda q: (abs(w - (b + q * s)), q & 1)))
    return float(b), float(s), qs


def _check_against_brute_force(w, G, bits):
    codes, scales, biases = oracle.quantize(w, G, bits)
    q = oracle.unpack(codes, w.shape[1], bits)
    for n in range(w.shape[0]):
        for g in range(w.shape[1] // G):
            grp = [float(v) for v in w[n, g * G:(g + 1) * G]]
            b, s, qs = brute_force_group(grp, bits)
            assert biases[n, g] == _h(b), (n, g)
            assert scales[n, g] == _h(s), (n, g)
            assert list(q[n, g * G:(g + 1) * G]) == qs, (n, g)


@pytest.mark.parametrize("bits", range(2, 9))
@pytest.mark.parametrize("G", [32, 64, 128])
def test_brute_force_random(bits, G):
    w = inputs.weights(2, 2 * G, seed=1, key=(bits, G), std=0.02, outliers=False)
    _check_against_brute_force(w, G, bits)


@settings(max_examples=60, deadline=None)
@given(st.integers(2, 8), st.sampled_from([32, 64]), st.integers(0, 2**31),
       st.sampled_from([1e-6, 1e-3, 0.02, 1.0, 300.0]), st.floats(-2.0, 2.0))
def test_brute_force_hypothesis(bits, G, seed, scale, shift):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((1, G)) * scale + shift * scale).astype(np.float32)
    _check_against_brute_force(w, G, bits)


def _invariants(w, G, bits):
    codes, scales, biases = oracle.quantize(w, G, bits)
    N, K = w.shape
    L = (1 << bits) - 1
    q = oracle.unpack(codes, K, bits).astype(np.int64)
    s = scales.view(np.float16).astype(np.float64)
    b = biases.view(np.float16).astype(np.float64)
    assert q.min() >= 0 and q.max() <= L
    wg = w.astype(np.float64).reshape(N, K // G, G)
    qg = q.reshape(N, K // G, G)
    sb, bb = s[..., None], b[..., None]
    # bias never exceeds a member; top grid point reaches the max
    assert np.all(bb <= wg)
    assert np.all(b + L * s >= wg.max(axis=-1))
    # |w - w^| <= s/2 exactly: w in [b + (q-1/2)s, b + (q+1/2)s] (exact in binary64)
    assert np.all(bb + (qg - 0.5) * sb <= wg) and np.all(wg <= bb + (qg + 0.5) * sb)
    # bias = RD_fp16(min): the next fp16 up already exceeds the minimum
    nxt = np.nextafter(biases.view(np.float16), np.float16(np.inf)).astype(np.float64)
    assert np.all(nxt > wg.min(axis=-1))
    # scale minimal: the previous fp16 would not reach the maximum
    pos = s > 0
    prev = np.nextafter(scales.view(np.float16), np.float16(0)).astype(np.float64)
    assert np.all(b[pos] + L * prev[pos] < wg.max(axis=-1)[pos])
    assert np.all(s[~pos] == 0) and np.all(qg[~pos] == 0)
    return codes, scales, biases


@pytest.mark.parametrize("bits,G", [(4, 64), (3, 64), (2, 32), (8, 128), (5, 32), (6, 64), (7, 128)])
def test_invariants_workload_like(bits, G):
    w = inputs.weights(64, 8 * G, seed=2, key=(bits, G), outliers=True)
    _invariants(w, G, bits)


def test_group_locality():
    # one outlier changes only its own group's scale, bias and codes
    G, bits = 64, 4
    w = inputs.weights(4, 8 * G, seed=5)
    c0, s0, b0 = oracle.quantize(w, G, bits)
    w2 = w.copy()
    w2[2, 3 * G + 17] = 0.9
    c1, s1, b1 = oracle.quantize(w2, G, bits)
    q0 = oracle.unpack(c0, w.shape[1], bits)
    q1 = oracle.unpack(c1, w.shape[1], bits)
    diff_s = np.argwhere(s0 != s1)
    assert diff_s.tolist() == [[2, 3]]
    assert np.array_equal(np.delete(b0.ravel(), 2 * 8 + 3), np.delete(b1.ravel(), 2 * 8 + 3))
    dq = np.argwhere(q0 != q1)
    assert len(dq) > 0 and np.all(dq[:, 0] == 2) and np.all(dq[:, 1] // G == 3)


@pytest.mark.parametrize("bits", range(2, 9))
def test_grid_exact_recovery_and_ties(bits):
    L = (1 << bits) - 1
    G = 64
    rng = np.random.default_rng(bits)
    s0 = 2.0 ** -8
    b0 = float(np.float16(-0.37))
    q = rng.integers(0, L + 1, size=G)
    q[5], q[40] = 0, L  # both ends present fix the range
    w = (b0 + q * s0).astype(np.float32)[None, :]
    assert np.array_equal(w.astype(np.float64)[0], b0 + q * s0)  # exact inputs
    codes, scales, biases = oracle.quantize(w, G, bits)
    assert biases[0, 0] == _h(b0) and scales[0, 0] == _h(s0)
    assert np.array_equal(oracle.unpack(codes, G, bits)[0], q)
    # half steps: w = b0 + (j + 1/2) s0 must go to the even one of j, j+1
    j = rng.integers(0, L, size=G)
    wt = b0 + (j + 0.5) * s0
    wt[0], wt[1] = b0, b0 + L * s0
    wt32 = wt.astype(np.float32)[None, :]
    assert np.array_equal(wt32.astype(np.float64)[0], wt)
    codes, scales, biases = oracle.quantize(wt32, G, bits)
    assert biases[0, 0] == _h(b0) and scales[0, 0] == _h(s0)
    got = oracle.unpack(codes, G, bits)[0].astype(np.int64)
    want = np.where(j % 2 == 0, j, j + 1)
    want[0], want[1] = 0, L
    assert np.array_equal(got, want)


def test_degenerate_groups():
    G, bits = 32, 4
    L = (1 << bits) - 1
    w = np.zeros((4, G), dtype=np.float32)
    w[1, :] = -0.0
    w[2, :] = 0.123  # constant, not an fp16 value
    w[3, :] = -7.5   # constant, an fp16 value
    codes, scales, biases = oracle.quantize(w, G, bits)
    q = oracle.unpack(codes, G, bits)
    # all-zero and -0 groups: bias +0 (pattern 0), scale 0, codes 0
    assert biases[0, 0] == 0 and biases[1, 0] == 0
    assert scales[0, 0] == 0 and scales[1, 0] == 0 and np.all(q[:2] == 0)
    # fp16-exact constant: bias is the value, scale 0, codes 0
    assert biases[3, 0] == _h(-7.5) and scales[3, 0] == 0 and np.all(q[3] == 0)
    # other constants: bias rounds down, the smallest scale lifts the top
    # grid point onto the value, and every code is the top one
    v = float(np.float32(0.123))
    rd = FP16_SORTED[bisect.bisect_right(FP16_SORTED, v) - 1]
    assert biases[2, 0] == _h(rd) and rd < v
    s = float(scales[2:3].view(np.float16)[0, 0])
    assert s > 0 and rd + L * s >= v and np.all(q[2] == L)
    assert rd + L * float(np.nextafter(np.float16(s), np.float16(0))) < v


def test_range_errors():
    G, bits = 32, 4
    for bad in (np.inf, -np.inf, np.nan, -70000.0):
        w = np.zeros((1, G), dtype=np.float32)
        w[0, 3] = bad
        with pytest.raises(oracle.OracleError) as e:
            oracle.quantize(w, G, bits)
        assert e.value.status == oracle.ERR_RANGE
    # a range needing a scale above 65504 cannot be stored
    w = np.zeros((1, G), dtype=np.float32)
    w[0, 0], w[0, 1] = -3.0e38, 3.0e38
    with pytest.raises(oracle.OracleError):
        oracle.quantize(w, G, bits)
    # K not divisible by G is rejected
    with pytest.raises(oracle.OracleError) as e:
        oracle.quantize(np.zeros((1, 48), dtype=np.float32), 32, 4)
    assert e.value.status == oracle.ERR_ARG


def test_rtn_beats_any_other_code():
    # no other code in range gives a smaller error (exact check in binary64)
    G, bits = 64, 3
    w = inputs.weights(8, 4 * G, seed=9)
    codes, scales, biases = oracle.quantize(w, G, bits)
    q = oracle.unpack(codes, w.shape[1], bits).astype(np.int64)
    s = np.repeat(scales.view(np.float16).astype(np.float64), G, axis=1)
    b = np.repeat(biases.view(np.float16).astype(np.float64), G, axis=1)
    L = (1 << bits) - 1
    wd = w.astype(np.float64)
    best = np.abs(wd - (b + q * s))
    for alt in range(L + 1):
        assert np.all(best <= np.abs(wd - (b + alt * s)) + 1e-15)
