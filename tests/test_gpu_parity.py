"""GPU parity of every libaq entry point against the CPU oracle, on seeded
inputs at sizes the oracle finishes in seconds, spanning several tiles,
slices and ragged tails, across all bit widths, group sizes and dtypes.

Bar: quantize and dequantize bit-exact; matmuls |y - y_ref| <= 2^-9*A + 1e-6
per element with A = sum_k |x_k * w^_k| (w^ the oracle's dequantized
weight).  Inputs come only from the seeded generator and the oracle."""
import numpy as np
import pytest

import oracle
from group_wise_affine_aq_amd import inputs
from gpu_util import (bits_to_dev, out_bits, out_to_f64, packed_from_dev, packed_to_dev,
                      to_dev, torch_dtype)

pytestmark = pytest.mark.gpu

ALL_BITS = [2, 3, 4, 5, 6, 7, 8]
GROUP_FOR_BITS = {2: 32, 3: 64, 4: 64, 5: 128, 6: 32, 7: 64, 8: 128}


@pytest.fixture(scope="module")
def aq():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import group_wise_affine_aq_amd as mod
    mod.load_library()
    return mod


def _quantized(N, K, G, bits, seed=0, outliers=True):
    w = inputs.weights(N, K, seed=seed, key=(G, bits, 17), outliers=outliers)
    return w, oracle.quantize(w, G, bits)


def _assert_close(y_dev, y_ref, A, what):
    ok, ratio = oracle.within_tolerance(out_to_f64(y_dev), y_ref, A)
    assert ok, f"{what}: worst error/bound = {ratio:.3f}"
    return ratio


# ---- quantize -------------------------------------------------------------------------
@pytest.mark.parametrize("bits", ALL_BITS)
@pytest.mark.parametrize("G", [32, 64, 128])
def test_quantize_bitexact_f32(aq, bits, G):
    N, K = 37, 6 * G
    w, (c, s, b) = _quantized(N, K, G, bits)
    gc, gs, gb = packed_from_dev(*aq.aq_quantize(to_dev(w), G, bits))
    assert np.array_equal(gs, s) and np.array_equal(gb, b)
    assert np.array_equal(gc, c)


def _check_mse(w, G, bits, steps, got):
    """Range search: bit-exact with the oracle wherever both pick the same
    candidate; elsewhere the device's candidate must tie the least error up to
    the rounding of the binary64 sums (the two add in different orders), and
    its scale, bias and codes must be exactly the oracle's for it."""
    c, s, b, chosen, errs = oracle.quantize_mse(w, G, bits, steps, details=True)
    gc, gs, gb = got
    K = w.shape[1]
    q_ref, q_dev = oracle.unpack(c, K, bits), oracle.unpack(gc, K, bits)
    same = (gs == s) & (gb == b)
    for n, g in zip(*np.nonzero(same)):
        assert np.array_equal(q_dev[n, g * G:(g + 1) * G], q_ref[n, g * G:(g + 1) * G]), (n, g)
    forced = {}
    for n, g in zip(*np.nonzero(~same)):
        for j in range(steps):
            if j not in forced:
                fc, fs, fb = oracle.quantize_mse(w, G, bits, steps, only=j)
                forced[j] = (oracle.unpack(fc, K, bits), fs, fb)
            fq, fs, fb = forced[j]
            if fs[n, g] == gs[n, g] and fb[n, g] == gb[n, g]:
                assert errs[n, g, j] <= errs[n, g].min() * (1 + 1e-12), (n, g, j)
                assert np.array_equal(q_dev[n, g * G:(g + 1) * G], fq[n, g * G:(g + 1) * G])
                break
        else:
            raise AssertionError(f"group {(n, g)}: device grid is no candidate")
    return int((~same).sum())


@pytest.mark.parametrize("bits", ALL_BITS)
@pytest.mark.parametrize("G", [32, 64, 128])
def test_quantize_mse(aq, bits, G):
    N, K, steps = 37, 6 * G, 30
    w = inputs.weights(N, K, seed=18, key=(G, bits), outliers=True)
    got = packed_from_dev(*aq.aq_quantize_mse(to_dev(w), G, bits, steps))
    assert _check_mse(w, G, bits, steps, got) <= N * K // G // 50


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("G", [32, 128])
def test_quantize_mse_same_sign_groups(aq, bits, G):
    """Groups whose members all share a sign (alternating positive and
    negative, some with one far member): the device follows the oracle,
    and its grids never reach below the min-max grid's bias nor use a larger
    scale (every candidate range lies inside [min, max])."""
    N, K, steps = 21, 6 * G, 50
    w = inputs.same_sign_weights(N, K, G, seed=22, key=(bits,))
    got = packed_from_dev(*aq.aq_quantize_mse(to_dev(w), G, bits, steps))
    _check_mse(w, G, bits, steps, got)
    _, s0, b0 = oracle.quantize(w, G, bits)
    f16 = lambda a: a.view(np.float16).astype(np.float64)
    assert (f16(got[2]) >= f16(b0)).all() and (f16(got[1]) <= f16(s0)).all()


def test_quantize_mse_one_step_and_half_inputs(aq):
    G, bits, N, K = 64, 4, 29, 512
    w = inputs.weights(N, K, seed=19, outliers=True)
    got = packed_from_dev(*aq.aq_quantize_mse(to_dev(w), G, bits, 1))
    for a, r in zip(got, oracle.quantize(w, G, bits)):
        assert np.array_equal(a, r)
    wb = inputs.to_bits(w, "bf16")
    w32 = inputs.from_bits(wb, "bf16").astype(np.float32)
    got = packed_from_dev(*aq.aq_quantize_mse(bits_to_dev(wb, "bf16"), G, 3, 50))
    _check_mse(w32, G, 3, 50, got)


@pytest.mark.parametrize("wdt", ["f16", "bf16"])
@pytest.mark.parametrize("bits", [3, 4, 8])
def test_quantize_bitexact_half_inputs(aq, wdt, bits):
    G, N, K = 64, 29, 512
    wb = inputs.to_bits(inputs.weights(N, K, seed=2, outliers=True), wdt)
    w32 = inputs.from_bits(wb, wdt).astype(np.float32)  # exact widening
    c, s, b = oracle.quantize(w32, G, bits)
    gc, gs, gb = packed_from_dev(*aq.aq_quantize(bits_to_dev(wb, wdt), G, bits))
    assert np.array_equal(gs, s) and np.array_equal(gb, b) and np.array_equal(gc, c)


@pytest.mark.parametrize("bits", ALL_BITS)
def test_quantize_edge_groups(aq, bits):
    """Constant, zero and -0 groups, fp32 subnormals, exact half-step ties,
    the fp16 range ends and groups spanning many binades."""
    G = 32
    L = (1 << bits) - 1
    rng = np.random.default_rng(bits)
    rows = []
    rows.append(np.zeros(G))
    rows.append(-np.zeros(G))
    rows.append(np.full(G, 0.123))
    rows.append(np.full(G, -7.5))
    rows.append(rng.standard_normal(G) * 1e-40)          # binary32 subnormals
    rows.append(rng.standard_normal(G) * 1e-6)           # fp16 subnormal range
    rows.append(np.linspace(-65504.0, 60000.0, G))        # fp16 range ends
    rows.append(rng.standard_normal(G) * 10.0 ** rng.integers(-8, 4, G))
    s0, b0 = 2.0 ** -8, float(np.float16(-0.37))
    j = rng.integers(0, L, G)
    t = b0 + (j + 0.5) * s0                                # exact ties
    t[0], t[1] = b0, b0 + L * s0
    rows.append(t)
    q = rng.integers(0, L + 1, G)
    q[0], q[1] = 0, L
    rows.append(b0 + q * s0)                               # exact grid points
    w = np.array(rows, dtype=np.float32)
    c, s, b = oracle.quantize(w, G, bits)
    gc, gs, gb = packed_from_dev(*aq.aq_quantize(to_dev(w), G, bits))
    assert np.array_equal(gb, b), np.argwhere(gb != b)
    assert np.array_equal(gs, s), np.argwhere(gs != s)
    assert np.array_equal(gc, c)
    _check_mse(w, G, bits, 50, packed_from_dev(*aq.aq_quantize_mse(to_dev(w), G, bits, 50)))


# ---- integer zero point -----------------------------------------------------------------
def _zp_from_dev(got):
    c, s, b = packed_from_dev(*got[:3])
    return c, s, b, got[3].cpu().numpy()


@pytest.mark.parametrize("bits", ALL_BITS)
@pytest.mark.parametrize("G", [32, 64, 128])
def test_quantize_zp_bitexact(aq, bits, G):
    """Codes, scales, biases and zero points bit-exact with the oracle, on
    Gaussian rows with outliers and on groups whose members share a sign."""
    N, K = 37, 6 * G
    w = np.concatenate([inputs.weights(N - 8, K, seed=40, key=(G, bits), outliers=True),
                        inputs.same_sign_weights(8, K, G, seed=41, key=(G, bits))])
    ref = oracle.quantize_zp(w, G, bits)
    got = _zp_from_dev(aq.aq_quantize_zp(to_dev(w), G, bits))
    for a, r, name in zip(got, ref, ("codes", "scales", "biases", "zeros")):
        assert np.array_equal(a, r), name


@pytest.mark.parametrize("wdt", ["f16", "bf16"])
def test_quantize_zp_half_inputs_and_edge_groups(aq, wdt):
    G, bits = 32, 4
    L = (1 << bits) - 1
    rng = np.random.default_rng(42)
    rows = [np.zeros(G), -np.zeros(G), np.full(G, 0.123), np.full(G, -7.5),
            rng.standard_normal(G) * 1e-6, np.linspace(-600.0, 500.0, G),
            np.linspace(0.25, 1.5, G), -np.linspace(0.25, 1.5, G)]
    s0, z0 = 2.0 ** -8, 5
    q = rng.integers(0, L + 1, G)
    q[0], q[1] = 0, L
    rows.append((q - z0) * s0)                                # exact grid points
    w32 = inputs.from_bits(inputs.to_bits(np.array(rows), wdt), wdt).astype(np.float32)
    ref = oracle.quantize_zp(w32, G, bits)
    got = _zp_from_dev(aq.aq_quantize_zp(bits_to_dev(inputs.to_bits(w32, wdt), wdt), G, bits))
    for a, r, name in zip(got, ref, ("codes", "scales", "biases", "zeros")):
        assert np.array_equal(a, r), name


def test_quantize_zp_without_zeros_output(aq):
    import torch
    import ctypes
    G, bits, N, K = 64, 4, 9, 256
    w = inputs.weights(N, K, seed=43, outliers=True)
    wd = to_dev(w)
    codes = torch.empty((N, K * bits // 32), dtype=torch.int32, device="cuda")
    scales = torch.empty((N, K // G), dtype=torch.float16, device="cuda")
    biases = torch.empty((N, K // G), dtype=torch.float16, device="cuda")
    lib = aq.load_library()
    st = lib.aq_quantize_zp(ctypes.c_void_p(wd.data_ptr()), 0, N, K, G, bits,
                            ctypes.c_void_p(codes.data_ptr()), ctypes.c_void_p(scales.data_ptr()),
                            ctypes.c_void_p(biases.data_ptr()), None,
                            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    ref = oracle.quantize_zp(w, G, bits)
    for a, r in zip(packed_from_dev(codes, scales, biases), ref[:3]):
        assert np.array_equal(a, r)


# ---- null biases (every bias +0) -----------------------------------------------------------
@pytest.mark.parametrize("bits,G", [(4, 64), (8, 128), (3, 64), (2, 32)])
def test_null_bias_consumers(aq, bits, G):
    """Every consumer with biases=None gives exactly the result of an all-zero
    bias array (the same kernels read +0), and that result matches the
    oracle with zero biases: bit-exact for dequantize and the embedding,
    within the bound for the matmuls (1, 3, 8, 40 and 130 rows, and the
    gathers)."""
    import torch
    N, K = 70, 8 * G
    w = inputs.weights(N, K, seed=44, key=(bits, G))
    c, s, _ = oracle.quantize(w, G, bits)
    zb = np.zeros_like(s)                                   # fp16 +0 biases
    dc, ds, dz = packed_to_dev(c, s, zb)
    for out in ("f32", "bf16"):
        code = {"f32": oracle.F32, "bf16": oracle.BF16}[out]
        ref = oracle.dequantize(c, s, zb, K, G, bits, code)
        a = out_bits(aq.aq_dequantize(dc, ds, None, G, bits, out_dtype=torch_dtype(out)))
        b = out_bits(aq.aq_dequantize(dc, ds, dz, G, bits, out_dtype=torch_dtype(out)))
        assert np.array_equal(a, b)
        assert np.array_equal(a, ref.view(np.uint32) if out == "f32" else ref)
    ids = np.array([3, 0, 69, -1, 70, 12], dtype=np.int32)
    a = out_bits(aq.aq_embedding(to_dev(ids), dc, ds, None, G, bits, out_dtype=torch.bfloat16))
    b = out_bits(aq.aq_embedding(to_dev(ids), dc, ds, dz, G, bits, out_dtype=torch.bfloat16))
    assert np.array_equal(a, b)
    for M in (1, 3, 8, 40, 130):
        xb = inputs.activations(M, K, "f16", seed=44, key=(M, bits))
        x = bits_to_dev(xb, "f16")
        y_ref, A = oracle.matmul(inputs.from_bits(xb, "f16"), c, s, zb, K, G, bits)
        fns = [aq.aq_quantized_matmul, aq.aq_qmm] + ([aq.aq_qmv] if M <= 8 else [])
        for fn in fns:
            y0, y1 = fn(x, dc, ds, None, G, bits), fn(x, dc, ds, dz, G, bits)
            assert np.array_equal(out_bits(y0), out_bits(y1)), (fn.__name__, M)
            _assert_close(y0, y_ref, A, f"null-bias {fn.__name__} M{M} b{bits}")
    E, T, topk = 5, 24, 3
    ce, se, _ = _experts(E, N, K, G, bits, seed=45)
    zbe = np.zeros_like(se)
    ide = inputs.expert_ids(T, E, topk, seed=45)
    xb = inputs.activations(T, K, "f16", seed=45)
    y_ref, A = oracle.gather_matmul(inputs.from_bits(xb, "f16"), ce, se, zbe, ide, K, G, bits)
    dce, dse, dze = packed_to_dev(ce, se, zbe)
    for fn in (aq.aq_gather_qmv, aq.aq_gather_qmm, aq.aq_gather_quantized_matmul):
        y0 = fn(bits_to_dev(xb, "f16"), dce, dse, None, to_dev(ide), G, bits)
        y1 = fn(bits_to_dev(xb, "f16"), dce, dse, dze, to_dev(ide), G, bits)
        assert np.array_equal(out_bits(y0), out_bits(y1)), fn.__name__
        _assert_close(y0, y_ref, A, f"null-bias {fn.__name__} b{bits}")


def test_zero_point_output_through_every_consumer(aq):
    """The zero-point quantizer's container feeds the consumers unchanged: the
    4-bit G=64 result through the decode, few-row and prefill kernels."""
    G, bits, N, K = 64, 4, 300, 4096
    w = inputs.weights(N, K, seed=46, outliers=True)
    c, s, b, _ = oracle.quantize_zp(w, G, bits)
    dev = packed_to_dev(c, s, b)
    for M in (1, 4, 24, 300):
        xb = inputs.activations(M, K, "bf16", seed=46, key=(M,))
        y_ref, A = oracle.matmul(inputs.from_bits(xb, "bf16"), c, s, b, K, G, bits)
        _assert_close(aq.aq_quantized_matmul(bits_to_dev(xb, "bf16"), *dev, G, bits), y_ref, A,
                      f"zero-point container M{M}")


# ---- dequantize -------------------------------------------------------------------------
@pytest.mark.parametrize("bits", ALL_BITS)
@pytest.mark.parametrize("out", ["f32", "f16", "bf16"])
def test_dequantize_bitexact(aq, bits, out):
    G = GROUP_FOR_BITS[bits]
    N, K = 23, 4 * G
    _, (c, s, b) = _quantized(N, K, G, bits, seed=3)
    code = {"f32": oracle.F32, "f16": oracle.F16, "bf16": oracle.BF16}[out]
    ref = oracle.dequantize(c, s, b, K, G, bits, code)
    got = aq.aq_dequantize(*packed_to_dev(c, s, b), G, bits, out_dtype=torch_dtype(out))
    ref_bits = ref.view(np.uint32) if out == "f32" else ref
    assert np.array_equal(out_bits(got), ref_bits)


@pytest.mark.parametrize("bits,out", [(4, "bf16"), (3, "f32"), (8, "f16")])
@pytest.mark.parametrize("lookup", [False, True])
def test_dequantize_stays_in_output(aq, bits, out, lookup):
    """The last wave's store span ends inside the output: elements past it are
    never written (a ragged tail of chunks inside one wave and one workgroup)."""
    import torch
    G = GROUP_FOR_BITS[bits]
    R, K = 37, 5 * G
    _, (c, s, b) = _quantized(R, K, G, bits, seed=21)
    code = {"f32": oracle.F32, "f16": oracle.F16, "bf16": oracle.BF16}[out]
    ids = np.random.default_rng(21).integers(-1, R + 1, size=29).astype(np.int32)
    rows = len(ids) if lookup else R
    slack = 4096
    buf = torch.full((rows * K + slack,), 3.0, dtype=torch_dtype(out), device="cuda")
    dst = buf[:rows * K].view(rows, K)
    if lookup:
        aq.aq_embedding(to_dev(ids), *packed_to_dev(c, s, b), G, bits, out=dst)
        ref = oracle.embedding(c, s, b, ids, K, G, bits, code)
    else:
        aq.aq_dequantize(*packed_to_dev(c, s, b), G, bits, out=dst)
        ref = oracle.dequantize(c, s, b, K, G, bits, code)
    assert torch.equal(buf[rows * K:].cpu(), torch.full((slack,), 3.0, dtype=torch_dtype(out)))
    ref_bits = ref.view(np.uint32) if out == "f32" else ref
    assert np.array_equal(out_bits(dst), ref_bits)


# ---- quantized embedding ---------------------------------------------------------------------
@pytest.mark.parametrize("bits", ALL_BITS)
@pytest.mark.parametrize("out", ["f32", "f16", "bf16"])
def test_embedding_bitexact(aq, bits, out):
    G = GROUP_FOR_BITS[bits]
    V, K = 41, 3 * G
    _, (c, s, b) = _quantized(V, K, G, bits, seed=8)
    ids = np.random.default_rng(bits).integers(0, V, size=300).astype(np.int32)
    ids[[5, 77, 299]] = [-1, V, 2**31 - 1]  # outside the table: zero rows
    code = {"f32": oracle.F32, "f16": oracle.F16, "bf16": oracle.BF16}[out]
    ref = oracle.embedding(c, s, b, ids, K, G, bits, code)
    got = aq.aq_embedding(to_dev(ids), *packed_to_dev(c, s, b), G, bits,
                          out_dtype=torch_dtype(out))
    ref_bits = ref.view(np.uint32) if out == "f32" else ref
    assert np.array_equal(out_bits(got), ref_bits)


@pytest.mark.parametrize("T", [1, 2, 7, 1025])
def test_embedding_token_counts(aq, T):
    V, K, G, bits = 50, 4096, 128, 8
    _, (c, s, b) = _quantized(V, K, G, bits, seed=9)
    ids = np.random.default_rng(T).integers(-2, V + 2, size=T).astype(np.int32)
    ref = oracle.embedding(c, s, b, ids, K, G, bits, oracle.BF16)
    got = aq.aq_embedding(to_dev(ids), *packed_to_dev(c, s, b), G, bits,
                          out_dtype=torch_dtype("bf16"))
    assert np.array_equal(out_bits(got), ref)


# ---- QMV (M <= 8) ---------------------------------------------------------------------------
@pytest.mark.parametrize("bits", ALL_BITS)
@pytest.mark.parametrize("M", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("xdt", ["f16", "bf16"])
def test_qmv_parity(aq, bits, M, xdt):
    G = GROUP_FOR_BITS[bits]
    N, K = 67, 4224 if G == 128 else 4160  # several slices at M=8, ragged tails
    _, (c, s, b) = _quantized(N, K, G, bits, seed=4)
    xb = inputs.activations(M, K, xdt, seed=4, key=(bits, M))
    y_ref, A = oracle.matmul(inputs.from_bits(xb, xdt), c, s, b, K, G, bits)
    y = aq.aq_qmv(bits_to_dev(xb, xdt), *packed_to_dev(c, s, b), G, bits)
    _assert_close(y, y_ref, A, f"qmv b{bits} M{M} {xdt}")


_QMV_SHAPES = [(1, 32, 32), (1, 64, 64), (3, 128, 128), (200, 96, 32), (129, 2048, 64),
               (5, 32768, 64)]


# bf16 only at K >= 512 (test_bf16_small_k), where the bound covers a bf16
# result's own rounding
@pytest.mark.parametrize("xdt,N,K,G", [("f16",) + t for t in _QMV_SHAPES] +
                         [("bf16",) + t for t in _QMV_SHAPES if t[1] >= 2048])
def test_qmv_shapes(aq, xdt, N, K, G):
    bits = 4
    _, (c, s, b) = _quantized(N, K, G, bits, seed=5)
    for M in (1, 4):
        xb = inputs.activations(M, K, xdt, seed=5, key=(N, K, M))
        y_ref, A = oracle.matmul(inputs.from_bits(xb, xdt), c, s, b, K, G, bits)
        y = aq.aq_qmv(bits_to_dev(xb, xdt), *packed_to_dev(c, s, b), G, bits)
        _assert_close(y, y_ref, A, f"qmv N{N} K{K} M{M}")


@pytest.mark.parametrize("bits", [3, 4, 8])
@pytest.mark.parametrize("G", [32, 64, 128])
@pytest.mark.parametrize("K", [9600, 14336, 16384])
def test_qmv_decode_long_rows(aq, bits, G, K):
    """M = 1 at 5..8 chunks per lane: 1, 2 and 4 staging loads of scales and
    biases per lane and row (128 groups each), a ragged last pass (K = 9600:
    300 chunks), and biases=None (a size-0 staging resource reads +0)."""
    N = 45
    _, (c, s, b) = _quantized(N, K, G, bits, seed=23)
    zb = np.zeros_like(b)
    xb = inputs.activations(1, K, "f16", seed=23, key=(bits, G, K))
    x = bits_to_dev(xb, "f16")
    y_ref, A = oracle.matmul(inputs.from_bits(xb, "f16"), c, s, b, K, G, bits)
    dc, ds, db = packed_to_dev(c, s, b)
    _assert_close(aq.aq_qmv(x, dc, ds, db, G, bits), y_ref, A, f"qmv1 b{bits} G{G} K{K}")
    y_ref, A = oracle.matmul(inputs.from_bits(xb, "f16"), c, s, zb, K, G, bits)
    _assert_close(aq.aq_qmv(x, dc, ds, None, G, bits), y_ref, A,
                  f"qmv1 b{bits} G{G} K{K} no bias")


def test_qmv_decode_many_rows_per_wave(aq):
    """M = 1 with more rows per wave than one output round (32 rows): each
    later round refills the ring, staged scales and biases included."""
    N, K, G, bits = 300000, 64, 32, 4
    _, (c, s, b) = _quantized(N, K, G, bits, seed=24)
    xb = inputs.activations(1, K, "f16", seed=24)
    y_ref, A = oracle.matmul(inputs.from_bits(xb, "f16"), c, s, b, K, G, bits)
    y = aq.aq_qmv(bits_to_dev(xb, "f16"), *packed_to_dev(c, s, b), G, bits)
    _assert_close(y, y_ref, A, "qmv1 many rows")


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("xdt,G,K", [(xdt, G, K) for G, K in ((32, 2144), (64, 2112), (128, 2176))
                                     for xdt in ("f16", "bf16")] + [("f16", 32, 96), ("f16", 64, 64)])
def test_qmv_few_rows_groups(aq, xdt, bits, G, K):
    """2..8 rows (the matrix-core path) at every group size, K ragged against
    the 128-code step and the per-wave K split, N ragged against 16-row tiles
    (bf16 only at K >= 2048, where the bound covers a bf16 result's own
    rounding)."""
    N = 45
    _, (c, s, b) = _quantized(N, K, G, bits, seed=14)
    for M in (2, 4, 6, 8):
        xb = inputs.activations(M, K, xdt, seed=14, key=(G, K, M, bits))
        y_ref, A = oracle.matmul(inputs.from_bits(xb, xdt), c, s, b, K, G, bits)
        y = aq.aq_qmv(bits_to_dev(xb, xdt), *packed_to_dev(c, s, b), G, bits)
        _assert_close(y, y_ref, A, f"qmv b{bits} G{G} K{K} M{M} {xdt}")


@pytest.mark.parametrize("bits,G", [(4, 64), (8, 128), (8, 32)])
def test_qmv_few_rows_tall(aq, bits, G):
    """Tall matrices (two 16-row blocks per workgroup), rows ragged against 32."""
    N, K = 8200, 256
    _, (c, s, b) = _quantized(N, K, G, bits, seed=16)
    for M in (3, 8):
        xb = inputs.activations(M, K, "f16", seed=16, key=(bits, G, M))
        y_ref, A = oracle.matmul(inputs.from_bits(xb, "f16"), c, s, b, K, G, bits)
        y = aq.aq_qmv(bits_to_dev(xb, "f16"), *packed_to_dev(c, s, b), G, bits)
        _assert_close(y, y_ref, A, f"qmv tall b{bits} G{G} M{M}")


def test_qmv_few_rows_long_rows(aq):
    """Long rows at 4-bit: 8 waves per workgroup with three steps in flight
    (rows ragged against 16, K ragged against the 128-code step, so the last
    wave's range ends inside a step)."""
    N, K, G, bits = 4100, 10016, 32, 4
    assert "W=8," in aq.aq_qmv_describe(4, N, K, G, bits, "bf16")
    _, (c, s, b) = _quantized(N, K, G, bits, seed=17)
    dev = packed_to_dev(c, s, b)
    for xdt in ("f16", "bf16"):
        for M in (2, 4, 5, 8):
            xb = inputs.activations(M, K, xdt, seed=17, key=(M,))
            y_ref, A = oracle.matmul(inputs.from_bits(xb, xdt), c, s, b, K, G, bits)
            y = aq.aq_qmv(bits_to_dev(xb, xdt), *dev, G, bits)
            _assert_close(y, y_ref, A, f"qmv long rows M{M} {xdt}")


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("xdt,G,K", [("f16", 32, 2144), ("bf16", 32, 2144), ("bf16", 64, 2112),
                                     ("f16", 128, 384), ("f16", 64, 64)])
def test_matmul_few_rows_sliced(aq, xdt, bits, G, K):
    """9..64 rows through the dispatcher: the matrix-core few-row kernel with
    16 rows of x per slot, slices of 16 rows past 16 (a partial last slice),
    row blocks (14) not a multiple of the 8-block slice mapping, K ragged.
    bf16 only at K >= 2048, where the bound covers a bf16 result's own
    rounding (fp16 holds it at any K)."""
    N = 213
    _, (c, s, b) = _quantized(N, K, G, bits, seed=21)
    for M in (9, 12, 16, 17, 31, 40, 64):
        xb = inputs.activations(M, K, xdt, seed=21, key=(G, K, M, bits))
        y_ref, A = oracle.matmul(inputs.from_bits(xb, xdt), c, s, b, K, G, bits)
        y = aq.aq_quantized_matmul(bits_to_dev(xb, xdt), *packed_to_dev(c, s, b), G, bits)
        _assert_close(y, y_ref, A, f"sliced b{bits} G{G} K{K} M{M} {xdt}")


@pytest.mark.parametrize("bits,G", [(4, 64), (8, 128), (8, 32), (4, 32)])
def test_matmul_few_rows_sliced_tall(aq, bits, G):
    """Tall matrices at 16..64 rows: two or four 16-row blocks per workgroup
    (four once the 64-row workgroups fill 3/4 of the chip: 8200 rows at 40 and
    64 rows of x, 12300 rows at 16 and 20; rows ragged against both); past 16
    rows two sets of 16 x rows per wave (slices of 32; 40 rows leave the
    second slice's second set empty)."""
    K = 256
    for N, Ms in ((8200, (16, 24, 40, 64)), (12300, (16, 20))):
        _, (c, s, b) = _quantized(N, K, G, bits, seed=22)
        for M in Ms:
            xb = inputs.activations(M, K, "f16", seed=22, key=(bits, G, M))
            y_ref, A = oracle.matmul(inputs.from_bits(xb, "f16"), c, s, b, K, G, bits)
            y = aq.aq_quantized_matmul(bits_to_dev(xb, "f16"), *packed_to_dev(c, s, b), G, bits)
            _assert_close(y, y_ref, A, f"sliced tall {N} b{bits} G{G} M{M}")


def test_qmv_unit_vectors(aq):
    """x = e_k picks column k of the dequantized matrix."""
    G, bits, N, K = 64, 4, 40, 256
    _, (c, s, b) = _quantized(N, K, G, bits, seed=6)
    wd = oracle.dequantize_exact(c, s, b, K, G, bits)
    for k in (0, 1, 7, 8, 63, 64, 200, 255):
        xb = np.zeros((1, K), dtype=np.uint16)
        xb[0, k] = 0x3C00  # 1.0 in fp16
        y = out_to_f64(aq.aq_qmv(bits_to_dev(xb, "f16"), *packed_to_dev(c, s, b), G, bits))
        assert np.all(np.abs(y[0] - wd[:, k]) <= np.ldexp(np.abs(wd[:, k]), -9) + 1e-6)


# ---- QMM (any M) ---------------------------------------------------------------------------
@pytest.mark.parametrize("bits", ALL_BITS)
@pytest.mark.parametrize("xdt", ["f16", "bf16"])
def test_qmm_parity(aq, bits, xdt):
    G = GROUP_FOR_BITS[bits]
    M, N, K = 130, 200, 4224 if G == 128 else 4160
    _, (c, s, b) = _quantized(N, K, G, bits, seed=7)
    xb = inputs.activations(M, K, xdt, seed=7, key=(bits,))
    y_ref, A = oracle.matmul(inputs.from_bits(xb, xdt), c, s, b, K, G, bits)
    y = aq.aq_qmm(bits_to_dev(xb, xdt), *packed_to_dev(c, s, b), G, bits)
    _assert_close(y, y_ref, A, f"qmm b{bits} {xdt}")


@pytest.mark.parametrize("M,N,K,G", [(1, 1, 32, 32), (7, 33, 96, 32), (64, 128, 64, 64),
                                     (257, 129, 160, 32), (33, 300, 1024, 128)])
def test_qmm_shapes_f16(aq, M, N, K, G):
    """Ragged tiles and K tails.  fp16: the dequantized weight (2^-11 relative)
    and the fp16 output rounding keep the error under the bound for any input."""
    bits, xdt = 4, "f16"
    _, (c, s, b) = _quantized(N, K, G, bits, seed=8)
    xb = inputs.activations(M, K, xdt, seed=8, key=(M, N, K))
    y_ref, A = oracle.matmul(inputs.from_bits(xb, xdt), c, s, b, K, G, bits)
    y = aq.aq_qmm(bits_to_dev(xb, xdt), *packed_to_dev(c, s, b), G, bits)
    _assert_close(y, y_ref, A, f"qmm {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K,G", [(1, 1, 2048, 32), (7, 33, 2080, 32), (257, 129, 2112, 64),
                                     (33, 300, 4096, 128)])
def test_qmm_shapes_bf16(aq, M, N, K, G):
    """bf16 at the workloads' depth (K >= 2048; 512..1408 in test_bf16_small_k).
    A bf16 output alone may be off by 2^-8*|y|, which the bound 2^-9*A covers
    only while |y| <= A/2 (|y|/A ~ 1/sqrt(K)); the kernel's rounding of the
    weights to bf16 adds to that, so below K ~ 512 it can leave the bound."""
    bits, xdt = 4, "bf16"
    _, (c, s, b) = _quantized(N, K, G, bits, seed=8)
    xb = inputs.activations(M, K, xdt, seed=8, key=(M, N, K))
    y_ref, A = oracle.matmul(inputs.from_bits(xb, xdt), c, s, b, K, G, bits)
    y = aq.aq_qmm(bits_to_dev(xb, xdt), *packed_to_dev(c, s, b), G, bits)
    _assert_close(y, y_ref, A, f"qmm {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K,G", [(300, 33029, 96, 32), (64, 51200, 160, 32),
                                     (300, 33029, 128, 64), (64, 51200, 256, 128)])
def test_qmm_tile_rounds(aq, M, N, K, G):
    """Shapes that fill the chip in rounds of 256-row tiles: 260 tiles (the
    last, partial round as 128-row tiles in a second launch; ragged rows,
    columns, K tail at G = 32) and 200 tiles (one launch of full tiles), with
    one group per chunk (G = 32) and with groups spanning chunks."""
    bits, xdt = 4, "f16"
    _, (c, s, b) = _quantized(N, K, G, bits, seed=23)
    xb = inputs.activations(M, K, xdt, seed=23, key=(M, N, K))
    y_ref, A = oracle.matmul(inputs.from_bits(xb, xdt), c, s, b, K, G, bits)
    y = aq.aq_qmm(bits_to_dev(xb, xdt), *packed_to_dev(c, s, b), G, bits)
    _assert_close(y, y_ref, A, f"qmm {M}x{N}x{K}")


def test_qmm_equals_gemm_of_dequantized(aq):
    """The matrix-core path multiplies exactly the bf16 weights that
    aq_dequantize produces (accumulation order aside)."""
    import torch
    G, bits, M, N, K = 64, 4, 96, 160, 512
    _, (c, s, b) = _quantized(N, K, G, bits, seed=9)
    xb = inputs.activations(M, K, "bf16", seed=9)
    x = bits_to_dev(xb, "bf16")
    dev = packed_to_dev(c, s, b)
    wq = aq.aq_dequantize(*dev, G, bits, out_dtype=torch.bfloat16)
    ref = (x.float() @ wq.float().T).double().cpu().numpy()
    y = out_to_f64(aq.aq_qmm(x, *dev, G, bits))
    assert np.max(np.abs(y - ref) / (np.abs(ref) + 1e-3)) < 2 ** -7


# ---- bf16 below the workloads' depth --------------------------------------------------------
@pytest.mark.parametrize("bits", [3, 4, 8])
@pytest.mark.parametrize("K,G", [(512, 64), (1024, 128), (1408, 64)])
def test_bf16_small_k(aq, bits, K, G):
    """bf16 activations at K = 512, 1024 and 1408 (an MoE down-projection
    width) through every matmul entry point: aq_qmv at 1, 3 and 8 rows,
    aq_qmm, aq_gather_qmv and aq_gather_qmm.  From K = 512 the bound covers a
    bf16 result's own rounding and the prefill kernel's rounding of the
    weights to bf16 (tests/test_oracle_matmul.py pins where it stops)."""
    xdt = "bf16"
    N = 100
    _, (c, s, b) = _quantized(N, K, G, bits, seed=25)
    dev = packed_to_dev(c, s, b)
    for M in (1, 3, 8):
        xb = inputs.activations(M, K, xdt, seed=25, key=(K, M, bits))
        y_ref, A = oracle.matmul(inputs.from_bits(xb, xdt), c, s, b, K, G, bits)
        _assert_close(aq.aq_qmv(bits_to_dev(xb, xdt), *dev, G, bits), y_ref, A,
                      f"qmv bf16 K{K} M{M} b{bits}")
    M = 130
    xb = inputs.activations(M, K, xdt, seed=25, key=(K, M, bits))
    y_ref, A = oracle.matmul(inputs.from_bits(xb, xdt), c, s, b, K, G, bits)
    _assert_close(aq.aq_qmm(bits_to_dev(xb, xdt), *dev, G, bits), y_ref, A,
                  f"qmm bf16 K{K} b{bits}")
    E, T, topk = 6, 40, 3
    ce, se, be = _experts(E, N, K, G, bits, seed=25)
    ids = inputs.expert_ids(T, E, topk, seed=25)
    xb = inputs.activations(T, K, xdt, seed=25, key=(K, bits))
    y_ref, A = oracle.gather_matmul(inputs.from_bits(xb, xdt), ce, se, be, ids, K, G, bits)
    deve = packed_to_dev(ce, se, be)
    _assert_close(aq.aq_gather_qmv(bits_to_dev(xb, xdt), *deve, to_dev(ids), G, bits), y_ref, A,
                  f"gather_qmv bf16 K{K} b{bits}")
    _assert_close(aq.aq_gather_qmm(bits_to_dev(xb, xdt), *deve, to_dev(ids), G, bits), y_ref, A,
                  f"gather_qmm bf16 K{K} b{bits}")


# ---- dispatch ----------------------------------------------------------------------------------
@pytest.mark.parametrize("M", [1, 3, 8, 9, 40, 64, 65, 200, 300])
def test_quantized_matmul_dispatch(aq, M):
    G, bits, N, K, xdt = 64, 4, 100, 640, "f16"
    _, (c, s, b) = _quantized(N, K, G, bits, seed=10)
    xb = inputs.activations(M, K, xdt, seed=10, key=(M,))
    y_ref, A = oracle.matmul(inputs.from_bits(xb, xdt), c, s, b, K, G, bits)
    y = aq.aq_quantized_matmul(bits_to_dev(xb, xdt), *packed_to_dev(c, s, b), G, bits)
    _assert_close(y, y_ref, A, f"dispatch M{M}")


@pytest.mark.parametrize("bits", [2, 3, 5, 6, 7])
def test_quantized_matmul_dispatch_other_widths(aq, bits):
    """9..256 rows with code widths the few-row kernel does not take: the
    dispatcher falls through to the prefill kernel."""
    G = GROUP_FOR_BITS[bits]
    N, K, xdt = 100, 640 if G != 128 else 768, "f16"
    _, (c, s, b) = _quantized(N, K, G, bits, seed=24)
    for M in (9, 40, 256):
        xb = inputs.activations(M, K, xdt, seed=24, key=(M, bits))
        y_ref, A = oracle.matmul(inputs.from_bits(xb, xdt), c, s, b, K, G, bits)
        y = aq.aq_quantized_matmul(bits_to_dev(xb, xdt), *packed_to_dev(c, s, b), G, bits)
        _assert_close(y, y_ref, A, f"dispatch b{bits} M{M}")


# ---- gather (MoE) ---------------------------------------------------------------------------------
def _experts(E, N, K, G, bits, seed):
    q = [oracle.quantize(inputs.weights(N, K, seed=seed, key=(e, G, bits)), G, bits)
         for e in range(E)]
    return (np.stack([a for a, _, _ in q]), np.stack([s for _, s, _ in q]),
            np.stack([b for _, _, b in q]))


@pytest.mark.parametrize("bits", ALL_BITS)
@pytest.mark.parametrize("xdt", ["f16", "bf16"])
def test_gather_parity(aq, bits, xdt):
    G = GROUP_FOR_BITS[bits]
    # bf16 at K >= 2048, where the bound covers a bf16 result's own rounding
    E, N, K, T, topk = 8, 100, 4 * G if xdt == "f16" else 2048 + 4 * G, 9, 3
    c, s, b = _experts(E, N, K, G, bits, seed=11)
    ids = inputs.expert_ids(T, E, topk, seed=11)
    xb = inputs.activations(T, K, xdt, seed=11)
    y_ref, A = oracle.gather_matmul(inputs.from_bits(xb, xdt), c, s, b, ids, K, G, bits)
    y = aq.aq_gather_qmv(bits_to_dev(xb, xdt), *packed_to_dev(c, s, b), to_dev(ids), G, bits)
    _assert_close(y, y_ref, A, f"gather b{bits} {xdt}")


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("G", [32, 64, 128])
def test_gather_groups(aq, bits, G):
    E, N, K, T, topk = 5, 37, 5 * G if G == 32 else 3 * G, 11, 2
    c, s, b = _experts(E, N, K, G, bits, seed=15)
    ids = inputs.expert_ids(T, E, topk, seed=15)
    xb = inputs.activations(T, K, "f16", seed=15)
    y_ref, A = oracle.gather_matmul(inputs.from_bits(xb, "f16"), c, s, b, ids, K, G, bits)
    y = aq.aq_gather_qmv(bits_to_dev(xb, "f16"), *packed_to_dev(c, s, b), to_dev(ids), G, bits)
    _assert_close(y, y_ref, A, f"gather b{bits} G{G}")


@pytest.mark.parametrize("bits,G", [(4, 32), (4, 64), (8, 128), (8, 32)])
@pytest.mark.parametrize("T,xdt,K", [(1, "f16", 384), (3, "f16", 9600), (4, "bf16", 2304)])
def test_gather_few_tokens(aq, bits, G, T, xdt, K):
    """At most one (token, slot) pair per expert on average: the launch with
    more waves per row (a ragged last block of rows, K split four ways)."""
    E, N, topk = 16, 100, 4
    c, s, b = _experts(E, N, K, G, bits, seed=19)
    ids = inputs.expert_ids(T, E, topk, seed=19, key=(T,))
    xb = inputs.activations(T, K, xdt, seed=19)
    y_ref, A = oracle.gather_matmul(inputs.from_bits(xb, xdt), c, s, b, ids, K, G, bits)
    y = aq.aq_gather_qmv(bits_to_dev(xb, xdt), *packed_to_dev(c, s, b), to_dev(ids), G, bits)
    _assert_close(y, y_ref, A, f"gather few T{T} b{bits} G{G} {xdt} K{K}")


@pytest.mark.parametrize("bits,G", [(4, 64), (8, 32), (8, 128)])
@pytest.mark.parametrize("E,T,topk,xdt", [(2, 21, 1, "f16"), (4, 40, 2, "f16"), (3, 150, 3, "f16"),
                                          (4, 37, 3, "bf16")])
def test_gather_crowded_experts(aq, bits, G, E, T, topk, xdt):
    """Experts with more than 8 routed pairs: batches of 16 x rows (a partial
    one included), a trailing batch of 8, and, past 256 pairs, several rounds
    of the id scan."""
    N, K = 100, 4 * G if xdt == "f16" else 2048 + 4 * G
    c, s, b = _experts(E, N, K, G, bits, seed=23)
    ids = inputs.expert_ids(T, E, topk, seed=23, key=(E, T))
    assert np.bincount(ids.ravel(), minlength=E).max() > 8
    xb = inputs.activations(T, K, xdt, seed=23)
    y_ref, A = oracle.gather_matmul(inputs.from_bits(xb, xdt), c, s, b, ids, K, G, bits)
    y = aq.aq_gather_qmv(bits_to_dev(xb, xdt), *packed_to_dev(c, s, b), to_dev(ids), G, bits)
    _assert_close(y, y_ref, A, f"gather crowded E{E} T{T} top{topk} b{bits} G{G} {xdt}")


def test_gather_expert_only_past_first_round(aq):
    """Experts whose pairs all lie past the first 256 (token, slot) pairs are
    still run (the first id scan lists only the first 256)."""
    G, bits, E, N, K, T, topk = 64, 4, 3, 70, 256, 100, 3
    c, s, b = _experts(E, N, K, G, bits, seed=25)
    ids = np.zeros((T, topk), dtype=np.int32)
    ids[90:, 1] = 1  # pairs 271.. only
    ids[95:, 2] = 2
    assert (ids.ravel()[:256] == 0).all()
    xb = inputs.activations(T, K, "f16", seed=25)
    y_ref, A = oracle.gather_matmul(inputs.from_bits(xb, "f16"), c, s, b, ids, K, G, bits)
    y = aq.aq_gather_qmv(bits_to_dev(xb, "f16"), *packed_to_dev(c, s, b), to_dev(ids), G, bits)
    _assert_close(y, y_ref, A, "gather expert only past the first round")


@pytest.mark.parametrize("K", [9600, 19200])
def test_gather_long_rows(aq, K):
    """Rows long enough that fewer 16-row blocks per workgroup fit the staged scales."""
    G, bits, E, N, T, topk = 32, 4, 3, 40, 5, 2
    c, s, b = _experts(E, N, K, G, bits, seed=17)
    ids = inputs.expert_ids(T, E, topk, seed=17)
    xb = inputs.activations(T, K, "f16", seed=17)
    y_ref, A = oracle.gather_matmul(inputs.from_bits(xb, "f16"), c, s, b, ids, K, G, bits)
    y = aq.aq_gather_qmv(bits_to_dev(xb, "f16"), *packed_to_dev(c, s, b), to_dev(ids), G, bits)
    _assert_close(y, y_ref, A, f"gather K{K}")


# ---- gather at prefill size (matrix cores) -------------------------------------------------
@pytest.mark.parametrize("bits", ALL_BITS)
@pytest.mark.parametrize("xdt,K", [("f16", 544), ("bf16", 2048)])
def test_gather_qmm_parity(aq, bits, xdt, K):
    """Several experts with ~180 routed rows each, N ragged against 256-column
    tiles, K with a 32-code tail (fp16) or at bf16 depth."""
    G = 32 if K % 64 else GROUP_FOR_BITS[bits]
    E, N, T, topk = 5, 300, 300, 3
    c, s, b = _experts(E, N, K, G, bits, seed=20)
    ids = inputs.expert_ids(T, E, topk, seed=20)
    xb = inputs.activations(T, K, xdt, seed=20, key=(bits, K))
    y_ref, A = oracle.gather_matmul(inputs.from_bits(xb, xdt), c, s, b, ids, K, G, bits)
    y = aq.aq_gather_qmm(bits_to_dev(xb, xdt), *packed_to_dev(c, s, b), to_dev(ids), G, bits)
    _assert_close(y, y_ref, A, f"gather_qmm b{bits} {xdt} K{K}")


def test_gather_qmm_crowded_and_bad_ids(aq):
    """One expert with 1398 routed rows (six 256-row tiles), an unused expert,
    and ids outside [0, E) (zero rows)."""
    G, bits, E, N, K, T, topk = 64, 4, 3, 250, 256, 700, 2
    c, s, b = _experts(E, N, K, G, bits, seed=21)
    ids = np.ones((T, topk), dtype=np.int32)
    ids[::7, 1] = 0
    ids[3, 0], ids[10, 1] = -1, E
    xb = inputs.activations(T, K, "f16", seed=21)
    import torch
    y = torch.full((T, topk, N), 7.0, dtype=torch.float16, device="cuda")
    aq.aq_gather_qmm(bits_to_dev(xb, "f16"), *packed_to_dev(c, s, b), to_dev(ids), G, bits, y=y)
    y = out_to_f64(y)
    assert np.all(y[3, 0] == 0) and np.all(y[10, 1] == 0)
    keep = (ids >= 0) & (ids < E)
    safe = np.where(keep, ids, 0).astype(np.int32)
    y_ref, A = oracle.gather_matmul(inputs.from_bits(xb, "f16"), c, s, b, safe, K, G, bits)
    ok, ratio = oracle.within_tolerance(y[keep], y_ref[keep], A[keep])
    assert ok, ratio


def test_gather_qmm_more_pairs_than_one_list(aq):
    """More pairs on one expert than one listing pass holds (4096): the scan
    resumes where the list filled up."""
    G, bits, E, N, K, T = 64, 4, 2, 40, 64, 4500
    c, s, b = _experts(E, N, K, G, bits, seed=22)
    ids = np.zeros((T, 1), dtype=np.int32)
    ids[::5, 0] = 1
    xb = inputs.activations(T, K, "f16", seed=22)
    y_ref, A = oracle.gather_matmul(inputs.from_bits(xb, "f16"), c, s, b, ids, K, G, bits)
    y = aq.aq_gather_qmm(bits_to_dev(xb, "f16"), *packed_to_dev(c, s, b), to_dev(ids), G, bits)
    _assert_close(y, y_ref, A, "gather_qmm multi-pass")


@pytest.mark.parametrize("T", [4, 200])
def test_gather_dispatch(aq, T):
    """Few rows per expert go to the matrix-vector gather, many to the
    matrix-core gather; both agree with the oracle."""
    G, bits, E, N, K, topk = 64, 4, 8, 70, 256, 2
    c, s, b = _experts(E, N, K, G, bits, seed=23)
    ids = inputs.expert_ids(T, E, topk, seed=23)
    xb = inputs.activations(T, K, "f16", seed=23)
    y_ref, A = oracle.gather_matmul(inputs.from_bits(xb, "f16"), c, s, b, ids, K, G, bits)
    y = aq.aq_gather_quantized_matmul(bits_to_dev(xb, "f16"), *packed_to_dev(c, s, b),
                                      to_dev(ids), G, bits)
    _assert_close(y, y_ref, A, f"gather dispatch T{T}")


def test_gather_crowded_expert_and_bad_ids(aq):
    """More tokens on one expert than one batch holds (processed in batches),
    unused experts, and ids outside [0, E) (their rows come back zero)."""
    G, bits, E, N, K, T, topk = 64, 4, 6, 70, 256, 21, 2
    c, s, b = _experts(E, N, K, G, bits, seed=12)
    ids = np.full((T, topk), 3, dtype=np.int32)
    ids[:, 1] = 1
    ids[5, 1] = 5
    xb = inputs.activations(T, K, "f16", seed=12)
    y_ref, A = oracle.gather_matmul(inputs.from_bits(xb, "f16"), c, s, b, ids, K, G, bits)
    y = aq.aq_gather_qmv(bits_to_dev(xb, "f16"), *packed_to_dev(c, s, b), to_dev(ids), G, bits)
    _assert_close(y, y_ref, A, "gather crowded")
    bad = ids.copy()
    bad[2, 0], bad[7, 1] = -1, E
    import torch
    yb = torch.full((T, topk, N), 7.0, dtype=torch.float16, device="cuda")
    aq.aq_gather_qmv(bits_to_dev(xb, "f16"), *packed_to_dev(c, s, b), to_dev(bad), G, bits, y=yb)
    yb = out_to_f64(yb)
    assert np.all(yb[2, 0] == 0) and np.all(yb[7, 1] == 0)
    keep = np.ones((T, topk), bool)
    keep[2, 0] = keep[7, 1] = False
    ok, _ = oracle.within_tolerance(yb[keep], y_ref[keep], A[keep])
    assert ok


def test_gather_all_same_expert_is_qmv(aq):
    G, bits, E, N, K, T = 64, 4, 4, 90, 512, 8
    c, s, b = _experts(E, N, K, G, bits, seed=13)
    ids = np.full((T, 1), 2, dtype=np.int32)
    xb = inputs.activations(T, K, "f16", seed=13)
    dev = packed_to_dev(c, s, b)
    yg = out_to_f64(aq.aq_gather_qmv(bits_to_dev(xb, "f16"), *dev, to_dev(ids), G, bits))
    yq = out_to_f64(aq.aq_qmv(bits_to_dev(xb, "f16"), dev[0][2].contiguous(),
                              dev[1][2].contiguous(), dev[2][2].contiguous(), G, bits))
    # the two kernels sum in different orders (M = 8 runs on the matrix cores),
    # so they agree through the oracle, each within the bound
    y_ref, A = oracle.matmul(inputs.from_bits(xb, "f16"), c[2], s[2], b[2], K, G, bits)
    for got, what in ((yg[:, 0, :], "gather"), (yq, "qmv")):
        ok, ratio = oracle.within_tolerance(got, y_ref, A)
        assert ok, f"{what}: worst error/bound = {ratio:.3f}"
