"""GPU parity of the block-scaled float modes (mxfp4, nvfp4, mxfp8: E2M1 or
E4M3 codes with a per-group scale) against the CPU oracle.

Bar: quantize and dequantize bit-exact (NaN where the oracle has NaN); the
decode product within 2^-9 * A + 1e-6 per element, A = sum_k |x_k * w^_k|
with w^ the oracle's exact dequantized weight.  Codes and scales fed to the
consumers come from the oracle's quantizer or from the seeded generator,
never from the device."""
import math

import numpy as np
import pytest

import oracle
from group_wise_affine_aq_amd import inputs
from gpu_util import bits_to_dev, out_bits, out_to_f64, to_dev, torch_dtype

pytestmark = pytest.mark.gpu

MODES = ["mxfp4", "nvfp4", "mxfp8"]
GROUP = {"mxfp4": 32, "nvfp4": 16, "mxfp8": 32}
BITS = {"mxfp4": 4, "nvfp4": 4, "mxfp8": 8}


@pytest.fixture(scope="module")
def aq():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import group_wise_affine_aq_amd as mod
    mod.load_library()
    return mod


def _tensor_exp(w, mode):
    """nvfp4's tensor exponent: the largest group scale near the top of E4M3
    (T = ceil(log2(max|W| / 2688))); 0 for the mx modes."""
    if mode != "nvfp4":
        return 0
    amax = float(np.abs(w).max())
    return 0 if amax == 0 else max(-100, min(100, math.ceil(math.log2(amax / 2688))))


def _oracle_quantize(w, mode, T):
    if mode == "mxfp4":
        return oracle.quantize_mxfp4(w)
    if mode == "mxfp8":
        return oracle.quantize_mxfp8(w)
    return oracle.quantize_nvfp4(w, T)


def _oracle_exact(c, s, K, mode, T):
    if mode == "mxfp4":
        return oracle.dequantize_mxfp4_exact(c, s, K)
    if mode == "mxfp8":
        return oracle.dequantize_mxfp8_exact(c, s, K)
    return oracle.dequantize_nvfp4_exact(c, s, K, T)


def _oracle_dequantize(c, s, K, mode, T, code):
    if mode == "mxfp4":
        return oracle.dequantize_mxfp4(c, s, K, code)
    if mode == "mxfp8":
        return oracle.dequantize_mxfp8(c, s, K, code)
    return oracle.dequantize_nvfp4(c, s, K, code, T)


def _to_dev(codes, scales):
    import torch
    c = torch.from_numpy(np.ascontiguousarray(codes).view(np.int32)).cuda()
    s = torch.from_numpy(np.ascontiguousarray(scales, dtype=np.uint8)).cuda()
    return c, s


def _from_dev(codes, scales):
    return codes.cpu().numpy().view(np.uint32), scales.cpu().numpy()


def _isnan_bits(b, out):
    if out == "f32":
        return np.isnan(b.view(np.float32))
    if out == "f16":
        return ((b & 0x7C00) == 0x7C00) & ((b & 0x03FF) != 0)
    return ((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0)


def _assert_same_bits(got, ref_bits, out):
    """Bit-exact, except that any NaN pattern matches any NaN pattern."""
    gn, rn = _isnan_bits(got, out), _isnan_bits(ref_bits, out)
    assert np.array_equal(gn, rn)
    assert np.array_equal(got[~gn], ref_bits[~rn])


def _special_rows():
    """Rows of 32 weights at the formats' edges: zeros and -0, subnormal
    maxima (exponents clamped), every E2M1 midpoint at several scales
    (ties), members past the largest code value (saturation), the binary32
    top, mixed signs, one large member among tiny ones."""
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
    rows.append(np.linspace(-500.0, 500.0, 32))                       # E4M3 ties and saturation
    return np.stack(rows).astype(np.float32)


# ---- quantize -------------------------------------------------------------------------
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("wdt", ["f32", "f16", "bf16"])
def test_quantize_fp_bitexact(aq, mode, wdt):
    N, K = 37, 13 * 32
    w = inputs.weights(N, K, seed=60, key=(1,), outliers=True)
    if wdt != "f32":
        wb = inputs.to_bits(w, wdt)
        w = inputs.from_bits(wb, wdt).astype(np.float32)   # exactly the half values
        wd = bits_to_dev(wb, wdt)
    else:
        wd = to_dev(w)
    T = _tensor_exp(w, mode)
    c, s = _oracle_quantize(w, mode, T)
    gc, gs = _from_dev(*aq.aq_quantize_fp(wd, mode, T))
    assert np.array_equal(gs, s)
    assert np.array_equal(gc, c)


@pytest.mark.parametrize("mode", MODES)
def test_quantize_fp_special_groups(aq, mode):
    w = _special_rows()
    w2 = np.ascontiguousarray(w.reshape(1, -1))  # the same groups side by side in one row
    for m in (w, w2):
        for T in ((0, -14, 60, -100) if mode == "nvfp4" else (0,)):
            c, s = _oracle_quantize(m, mode, T)
            gc, gs = _from_dev(*aq.aq_quantize_fp(to_dev(m), mode, T))
            assert np.array_equal(gs, s), T
            assert np.array_equal(gc, c), T


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("N,K", [(1, 32), (3, 64), (5, 48), (1000, 4096), (33, 14336 + 32)])
def test_quantize_fp_shapes(aq, mode, N, K):
    if K % GROUP[mode]:
        pytest.skip("K not a multiple of the group")
    w = inputs.weights(N, K, seed=61, key=(N, K), outliers=True)
    T = _tensor_exp(w, mode)
    c, s = _oracle_quantize(w, mode, T)
    gc, gs = _from_dev(*aq.aq_quantize_fp(to_dev(w), mode, T))
    assert np.array_equal(gs, s) and np.array_equal(gc, c)


# ---- dequantize -----------------------------------------------------------------------
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("out", ["f32", "f16", "bf16"])
def test_dequantize_fp_bitexact(aq, mode, out):
    """Oracle-quantized weights, plus arbitrary code words and every scale
    byte (NaN patterns and binary32 overflow included)."""
    N, K = 29, 9 * 32
    w = inputs.weights(N, K, seed=62, outliers=True)
    T = _tensor_exp(w, mode)
    c, s = _oracle_quantize(w, mode, T)
    rng = np.random.default_rng(62)
    rc = rng.integers(0, 2 ** 32, size=c.shape, dtype=np.uint64).astype(np.uint32)
    rs = (np.arange(s.size, dtype=np.int64).reshape(s.shape) % 256).astype(np.uint8)
    code = {"f32": oracle.F32, "f16": oracle.F16, "bf16": oracle.BF16}[out]
    for cc, ss, TT in ((c, s, T), (rc, rs, T), (rc, rs, 0)):
        ref = _oracle_dequantize(cc, ss, K, mode, TT, code)
        got = aq.aq_dequantize_fp(*_to_dev(cc, ss), K, mode, TT, out_dtype=torch_dtype(out))
        ref_bits = ref.view(np.uint32) if out == "f32" else ref
        _assert_same_bits(out_bits(got), ref_bits, out)


@pytest.mark.parametrize("mode", MODES)
def test_dequantize_fp_large(aq, mode):
    N, K = 4096, 4096
    w = inputs.weights(N, K, seed=63)
    T = _tensor_exp(w, mode)
    c, s = _oracle_quantize(w, mode, T)
    got = aq.aq_dequantize_fp(*_to_dev(c, s), K, mode, T)
    ref = _oracle_dequantize(c, s, K, mode, T, oracle.F32)
    assert np.array_equal(out_bits(got), ref.view(np.uint32))


# ---- the decode product ---------------------------------------------------------------
def _qmv_check(aq, mode, N, K, xdt, seed, w=None, T=None):
    if w is None:
        w = inputs.weights(N, K, seed=seed, key=(N, K), outliers=True)
    if T is None:
        T = _tensor_exp(w, mode)
    c, s = _oracle_quantize(w, mode, T)
    xb = inputs.activations(1, K, xdt, seed=seed, key=(N, K))
    y_ref, A = oracle.matmul_dense(inputs.from_bits(xb, xdt), _oracle_exact(c, s, K, mode, T))
    y = aq.aq_qmv_fp(bits_to_dev(xb, xdt), *_to_dev(c, s), mode, T)
    ok, ratio = oracle.within_tolerance(out_to_f64(y), y_ref, A)
    assert ok, f"qmv_fp {mode} N{N} K{K} {xdt} T{T}: worst error/bound = {ratio:.3f}"


# K: one chunk; 1..8 chunks per lane (ragged last passes: 4160 = 130 chunks,
# 9600 = 300); past 16384 the kernel that keeps x in LDS, up to its limit
_FP_K = [32, 96, 2048, 4160, 6176, 8192, 9600, 12288, 14336, 16384, 16416, 28672, 49152]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("K", _FP_K)
@pytest.mark.parametrize("xdt", ["f16", "bf16"])
def test_qmv_fp_parity(aq, mode, xdt, K):
    if xdt == "bf16" and K < 512:
        pytest.skip("bf16: the bound covers the result's own rounding from K = 512 on")
    _qmv_check(aq, mode, 67, K, xdt, seed=64)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("N,K", [(1, 4096), (1024, 4096), (4096, 4096), (14336, 4096),
                                 (4096, 14336), (9000, 2048)])
def test_qmv_fp_launch_shapes(aq, mode, N, K):
    """The shapes that select each launch configuration (rows in flight,
    waves per workgroup, workgroups per CU)."""
    _qmv_check(aq, mode, N, K, "f16", seed=65)


@pytest.mark.parametrize("mode", MODES)
def test_qmv_fp_many_rows_per_wave(aq, mode):
    """More rows per wave than one output round: the ring refills."""
    _qmv_check(aq, mode, 300000, 64, "f16", seed=66)


@pytest.mark.parametrize("mode", MODES)
def test_qmv_fp_special_groups(aq, mode):
    """Groups of zeros, subnormal and clamped exponents, ties and saturated
    members (the groups near the binary32 top left out: their products
    overflow); nvfp4 also without a tensor scale."""
    w = _special_rows()
    w = w[np.abs(w).max(axis=1) < 1e4]
    w = np.ascontiguousarray(np.tile(w.reshape(1, -1), (5, 3)))
    for T in ((None, 0) if mode == "nvfp4" else (None,)):
        _qmv_check(aq, mode, w.shape[0], w.shape[1], "f16", seed=67, w=w, T=T)


# ---- products for 2 and more rows of x (matrix cores) --------------------------------
def _mm_check(aq, mode, M, N, K, xdt, seed, w=None, T=None):
    if w is None:
        w = inputs.weights(N, K, seed=seed, key=(N, K), outliers=True)
    if T is None:
        T = _tensor_exp(w, mode)
    c, s = _oracle_quantize(w, mode, T)
    xb = inputs.activations(M, K, xdt, seed=seed, key=(M, N, K))
    y_ref, A = oracle.matmul_dense(inputs.from_bits(xb, xdt), _oracle_exact(c, s, K, mode, T))
    y = aq.aq_matmul_fp(bits_to_dev(xb, xdt), *_to_dev(c, s), mode, T)
    assert tuple(y.shape) == (M, N)
    ok, ratio = oracle.within_tolerance(out_to_f64(y), y_ref, A)
    assert ok, f"matmul_fp {mode} M{M} N{N} K{K} {xdt} T{T}: worst error/bound = {ratio:.3f}"


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("M", [2, 3, 4, 5, 8, 9, 16, 17, 40, 300])
@pytest.mark.parametrize("xdt", ["f16", "bf16"])
def test_matmul_fp_rows(aq, mode, M, xdt):
    """M rows of x in slices of 16 (17, 40, 300: a partial last slice), x loads
    carrying 4 chunks (M <= 4), 2 (M <= 8) or 1; N not a multiple of the
    32-row workgroup; K = 2080: 65 chunks, a partial last step of 4 chunks."""
    _mm_check(aq, mode, M, 100, 2080, xdt, seed=70)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("N,K", [(1, 32), (5, 96), (33, 160), (64, 4096), (257, 12288),
                                 (70, 49152)])
def test_matmul_fp_shapes(aq, mode, N, K):
    """One chunk, fewer chunks than a step, a row per workgroup block, the
    wave counts of the launch (2..8 waves splitting K) and the largest K."""
    _mm_check(aq, mode, 4, N, K, "f16", seed=71)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("N,K,M", [(14336, 4096, 4), (4096, 14336, 8)])
def test_matmul_fp_decode_shapes(aq, mode, N, K, M):
    """The speculative-decoding widths on the decode matrices."""
    _mm_check(aq, mode, M, N, K, "bf16", seed=72)


@pytest.mark.parametrize("mode", MODES)
def test_matmul_fp_special_groups(aq, mode):
    """Groups of zeros, subnormal and clamped exponents, ties and saturated
    members (as for M = 1); nvfp4 also without a tensor scale."""
    w = _special_rows()
    w = w[np.abs(w).max(axis=1) < 1e4]
    w = np.ascontiguousarray(np.tile(w.reshape(1, -1), (5, 3)))
    for T in ((None, 0) if mode == "nvfp4" else (None,)):
        _mm_check(aq, mode, 5, w.shape[0], w.shape[1], "f16", seed=73, w=w, T=T)


@pytest.mark.parametrize("mode", MODES)
def test_matmul_fp_one_row_is_qmv(aq, mode):
    """M = 1 goes to the decode product: the same bits as aq_qmv_fp."""
    import torch
    N, K = 300, 4096
    w = inputs.weights(N, K, seed=74, key=(N, K))
    T = _tensor_exp(w, mode)
    c, s = _oracle_quantize(w, mode, T)
    x = bits_to_dev(inputs.activations(1, K, "f16", seed=74, key=(N, K)), "f16")
    a = aq.aq_matmul_fp(x, *_to_dev(c, s), mode, T)
    b = aq.aq_qmv_fp(x, *_to_dev(c, s), mode, T)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# ---- the mixture-of-experts gather --------------------------------------------------------
def _gather_check(aq, mode, E, N, K, T, topk, xdt, seed, ids=None):
    """Experts quantized by the oracle; y_ref[t, j] = x[t] @ W_ids[t, j]^T with
    the oracle's exact weights (a zero row for an id outside [0, E))."""
    import torch
    ws = [inputs.weights(N, K, seed=seed, key=(e, N, K)) for e in range(E)]
    T_exp = _tensor_exp(np.concatenate(ws), mode)
    cs, ss, wx = [], [], []
    for w in ws:
        c, s = _oracle_quantize(w, mode, T_exp)
        cs.append(c)
        ss.append(s)
        wx.append(_oracle_exact(c, s, K, mode, T_exp))
    if ids is None:
        ids = inputs.expert_ids(T, E, topk, seed=seed)
    xb = inputs.activations(T, K, xdt, seed=seed, key=(T, K))
    xf = inputs.from_bits(xb, xdt)
    y_ref = np.zeros((T, topk, N))
    A = np.zeros((T, topk, N))
    for t in range(T):
        for j in range(topk):
            e = int(ids[t, j])
            if 0 <= e < E:
                y_ref[t, j], A[t, j] = (v[0] for v in oracle.matmul_dense(xf[t:t + 1], wx[e]))
    codes = torch.from_numpy(np.stack(cs).view(np.int32)).cuda()
    scales = torch.from_numpy(np.stack(ss)).cuda()
    y = aq.aq_gather_matmul_fp(bits_to_dev(xb, xdt), codes, scales, to_dev(ids), mode, T_exp)
    assert tuple(y.shape) == (T, topk, N)
    got = out_to_f64(y)
    ok, ratio = oracle.within_tolerance(got, y_ref, A)
    assert ok, f"gather_matmul_fp {mode} E{E} N{N} K{K} T{T}: worst error/bound = {ratio:.3f}"
    bad = (ids < 0) | (ids >= E)
    assert np.all(got[bad] == 0), "rows of ids outside the table must be zero"


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("xdt", ["f16", "bf16"])
def test_gather_matmul_fp(aq, mode, xdt):
    """8 experts, 40 tokens top-3 (about 15 pairs per expert: one batch of 16
    or two), N not a multiple of the 32-row workgroup, a partial last step."""
    _gather_check(aq, mode, 8, 100, 2080, 40, 3, xdt, seed=80)


@pytest.mark.parametrize("mode", MODES)
def test_gather_matmul_fp_crowded_and_bad_ids(aq, mode):
    """Every token on expert 1 (several batches of 16 and more than 256 ids,
    so several id rounds), one expert never chosen, and ids outside the
    table (zero rows)."""
    T, topk, E = 100, 3, 4
    ids = np.full((T, topk), 1, dtype=np.int32)
    ids[:, 1] = np.arange(T) % 2 * 2          # experts 0 and 2
    ids[5, 2], ids[17, 0], ids[63, 1] = -1, 4, 1 << 30
    _gather_check(aq, mode, E, 70, 544, T, topk, "f16", seed=81, ids=ids)


@pytest.mark.parametrize("mode", MODES)
def test_gather_matmul_fp_moe_shape(aq, mode):
    """The MoE workload's expert shape ([1408, 2048]) with 16 experts, 32
    tokens top-6."""
    _gather_check(aq, mode, 16, 1408, 2048, 32, 6, "f16", seed=82)


# ---- the prefill-size matrix ----------------------------------------------------------
@pytest.fixture(scope="module")
def prefill_weights():
    N, K = inputs.WORKLOADS["prefill"]["shapes"][0]
    return inputs.weights(N, K, seed=0, key=(inputs.WORKLOAD_ID["prefill"],))


@pytest.mark.parametrize("mode", MODES)
def test_fp_prefill_size(aq, prefill_weights, mode):
    """The benchmark's 28672 x 8192 matrix: quantize bit-exact on every
    element; dequantize to bf16 bit-exact on sampled rows."""
    import torch
    w = prefill_weights
    N, K = w.shape
    T = _tensor_exp(w, mode)
    wd = to_dev(w)
    gc, gs = aq.aq_quantize_fp(wd, mode, T)
    del wd
    c, s = _oracle_quantize(w, mode, T)
    assert np.array_equal(gs.cpu().numpy(), s)
    assert np.array_equal(gc.cpu().numpy().view(np.uint32), c)
    out = aq.aq_dequantize_fp(gc, gs, K, mode, T, out_dtype=torch.bfloat16)
    rows = np.unique(np.concatenate([np.random.default_rng(5).choice(N, 64, replace=False),
                                     [0, N - 1]]))
    ref = _oracle_dequantize(c[rows], s[rows], K, mode, T, oracle.BF16)
    _assert_same_bits(out_bits(out)[rows], ref, "bf16")
