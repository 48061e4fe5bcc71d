"""GPU parity of the mxfp4 entry points (block-scaled E2M1 codes, one E8M0
exponent per 32 weights) against the CPU oracle.

Bar: quantize and dequantize bit-exact; the decode product within
2^-9 * A + 1e-6 per element, A = sum_k |x_k * w^_k| with w^ the oracle's
exact dequantized weight.  Codes and scales fed to the consumers come from
the oracle's quantizer or from the seeded generator, never from the device."""
import numpy as np
import pytest

import oracle
from group_wise_affine_aq_amd import inputs
from gpu_util import bits_to_dev, out_bits, out_to_f64, to_dev, torch_dtype

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def aq():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import group_wise_affine_aq_amd as mod
    mod.load_library()
    return mod


def _mx_to_dev(codes, scales):
    import torch
    c = torch.from_numpy(np.ascontiguousarray(codes).view(np.int32)).cuda()
    s = torch.from_numpy(np.ascontiguousarray(scales, dtype=np.uint8)).cuda()
    return c, s


def _mx_from_dev(codes, scales):
    return codes.cpu().numpy().view(np.uint32), scales.cpu().numpy()


def _special_rows():
    """Rows of 32-weight groups at the format's edges: zeros and -0, subnormal
    maxima (X clamped to -127), the smallest unclamped exponents, every
    midpoint of the E2M1 grid at several scales (ties), members above 6 * 2^X
    (saturation), the binary32 top (X = 125), mixed signs."""
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.5, 7.0, 7.5, 0.5, 1.0, 3.0, 6.0, 0.1,
                     4.0], dtype=np.float64)
    rows = []
    g = np.concatenate([mids, -mids])
    for X in (-127, -126, -125, -100, -3, 0, 7, 125):
        rows.append(np.ldexp(g, X))
    rows.append(np.zeros(32))
    rows.append(-np.zeros(32))
    rows.append(np.full(32, 1e-40))                                   # subnormal group
    rows.append(np.ldexp(np.linspace(-1.0, 1.0, 32), -124))           # just above the clamp
    rows.append(np.ldexp(np.linspace(-1.0, 1.0, 32), -126))           # max|w| = 2^-126
    rows.append(np.full(32, 3.4e38) * np.where(np.arange(32) % 2, 1, -1))
    rows.append(np.where(np.arange(32) == 7, 1.0, 1e-30))             # one large member
    return np.stack(rows).astype(np.float32)


# ---- quantize -------------------------------------------------------------------------
@pytest.mark.parametrize("wdt", ["f32", "f16", "bf16"])
def test_quantize_mxfp4_bitexact(aq, wdt):
    N, K = 37, 13 * 32
    w = inputs.weights(N, K, seed=60, key=(1,), outliers=True)
    if wdt != "f32":
        wb = inputs.to_bits(w, wdt)
        w = inputs.from_bits(wb, wdt).astype(np.float32)   # exactly the half values
        wd = bits_to_dev(wb, wdt)
    else:
        wd = to_dev(w)
    c, s = oracle.quantize_mxfp4(w)
    gc, gs = _mx_from_dev(*aq.aq_quantize_mxfp4(wd))
    assert np.array_equal(gs, s)
    assert np.array_equal(gc, c)


def test_quantize_mxfp4_special_groups(aq):
    w = _special_rows()
    # the same groups side by side in one row as well (several groups per row)
    w2 = np.ascontiguousarray(w.reshape(1, -1))
    for m in (w, w2):
        c, s = oracle.quantize_mxfp4(m)
        gc, gs = _mx_from_dev(*aq.aq_quantize_mxfp4(to_dev(m)))
        assert np.array_equal(gs, s)
        assert np.array_equal(gc, c)


@pytest.mark.parametrize("N,K", [(1, 32), (3, 64), (1000, 4096), (33, 14336 + 32)])
def test_quantize_mxfp4_shapes(aq, N, K):
    w = inputs.weights(N, K, seed=61, key=(N, K), outliers=True)
    c, s = oracle.quantize_mxfp4(w)
    gc, gs = _mx_from_dev(*aq.aq_quantize_mxfp4(to_dev(w)))
    assert np.array_equal(gs, s) and np.array_equal(gc, c)


# ---- dequantize -----------------------------------------------------------------------
@pytest.mark.parametrize("out", ["f32", "f16", "bf16"])
def test_dequantize_mxfp4_bitexact(aq, out):
    """Oracle-quantized weights plus arbitrary words and scale bytes over the
    whole byte range (254 and 255 overflow binary32 to +-inf for the larger
    codes)."""
    N, K = 29, 9 * 32
    w = inputs.weights(N, K, seed=62, outliers=True)
    c, s = oracle.quantize_mxfp4(w)
    rng = np.random.default_rng(62)
    rc = rng.integers(0, 2 ** 32, size=(N, K // 8), dtype=np.uint64).astype(np.uint32)
    rs = np.arange(N * K // 32, dtype=np.int64).reshape(N, K // 32) % 256
    rs = rs.astype(np.uint8)
    code = {"f32": oracle.F32, "f16": oracle.F16, "bf16": oracle.BF16}[out]
    for cc, ss in ((c, s), (rc, rs)):
        ref = oracle.dequantize_mxfp4(cc, ss, K, code)
        got = aq.aq_dequantize_mxfp4(*_mx_to_dev(cc, ss), K, out_dtype=torch_dtype(out))
        ref_bits = ref.view(np.uint32) if out == "f32" else ref
        assert np.array_equal(out_bits(got), ref_bits)


def test_dequantize_mxfp4_large(aq):
    N, K = 4096, 4096
    w = inputs.weights(N, K, seed=63)
    c, s = oracle.quantize_mxfp4(w)
    got = aq.aq_dequantize_mxfp4(*_mx_to_dev(c, s), K)
    assert np.array_equal(out_bits(got), oracle.dequantize_mxfp4(c, s, K, oracle.F32).view(np.uint32))


# ---- the decode product ---------------------------------------------------------------
def _qmv_check(aq, N, K, xdt, seed, w=None):
    if w is None:
        w = inputs.weights(N, K, seed=seed, key=(N, K), outliers=True)
    c, s = oracle.quantize_mxfp4(w)
    xb = inputs.activations(1, K, xdt, seed=seed, key=(N, K))
    y_ref, A = oracle.matmul_dense(inputs.from_bits(xb, xdt), oracle.dequantize_mxfp4_exact(c, s, K))
    y = aq.aq_qmv_mxfp4(bits_to_dev(xb, xdt), *_mx_to_dev(c, s))
    ok, ratio = oracle.within_tolerance(out_to_f64(y), y_ref, A)
    assert ok, f"qmv_mxfp4 N{N} K{K} {xdt}: worst error/bound = {ratio:.3f}"


# K: one chunk; 1..8 chunks per lane (ragged last passes: 4160 = 130 chunks,
# 9600 = 300); past 16384 the kernel that keeps x in LDS, up to its limit
_MX_K = [32, 96, 2048, 4160, 6176, 8192, 9600, 12288, 14336, 16384, 16416, 28672, 49152]


@pytest.mark.parametrize("K", _MX_K)
@pytest.mark.parametrize("xdt", ["f16", "bf16"])
def test_qmv_mxfp4_parity(aq, xdt, K):
    if xdt == "bf16" and K < 512:
        pytest.skip("bf16: the bound covers the result's own rounding from K = 512 on")
    _qmv_check(aq, 67, K, xdt, seed=64)


@pytest.mark.parametrize("N,K", [(1, 4096), (1024, 4096), (4096, 4096), (14336, 4096),
                                 (4096, 14336), (9000, 2048)])
def test_qmv_mxfp4_launch_shapes(aq, N, K):
    """The shapes that select each launch configuration (rows in flight,
    waves per workgroup, workgroups per CU)."""
    _qmv_check(aq, N, K, "f16", seed=65)


def test_qmv_mxfp4_many_rows_per_wave(aq):
    """More rows per wave than one output round: the ring refills."""
    _qmv_check(aq, 300000, 64, "f16", seed=66)


def test_qmv_mxfp4_special_groups(aq):
    """Groups of zeros, subnormal and clamped exponents, ties and saturated
    members (the groups near the binary32 top left out: their products
    overflow)."""
    w = _special_rows()
    w = w[np.abs(w).max(axis=1) < 1e4]
    w = np.ascontiguousarray(np.tile(w.reshape(1, -1), (5, 3)))
    _qmv_check(aq, w.shape[0], w.shape[1], "f16", seed=67, w=w)
