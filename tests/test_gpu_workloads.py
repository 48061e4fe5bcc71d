"""Parity at the full workload sizes, through the entry points the benchmark
times (shape dispatch for few rows, the matrix-core kernel for prefill, the
gather kernel for the experts).

  tiny     W [512, 512] 4-bit G=64, x fp16 [1, 512]
  decode   W [4096,4096], [1024,4096], [14336,4096], [4096,14336], 0.1% outliers
           x20, 4-bit G=64, x fp16 [1, K]
  specdec  W [14336,4096], [4096,14336] at 4-bit G=64 and 8-bit G=128,
           x bf16 [M, K], M in {2,3,4,6,8}; also M in {12,16,40,64} (sampled
           columns)
  prefill  X bf16 [2048, 8192], W [28672, 8192] at 4-bit G=64, 3-bit G=64,
           2-bit G=32 (outputs compared on a seeded sample of rows x columns)
  moe      64 experts [1408, 2048] 4-bit G=64, x fp16 [32, 2048], ids [32, 6];
           the same experts at prefill size, x fp16 [2048, 2048], ids [2048, 6]
           (sampled rows)
  embedding table [128256, 4096] 8-bit G=128, T in {1, 2048} token ids, bf16 out

Quantization is checked bit-exactly on every element (for the embedding table,
on every row a token refers to); embedding rows bit-exactly; matmul outputs against
|y - y_ref| <= 2^-9 * sum_k |x_k w^_k| + 1e-6."""
import numpy as np
import pytest

import oracle
from group_wise_affine_aq_amd import inputs
from gpu_util import bits_to_dev, out_bits, out_to_f64, packed_from_dev, packed_to_dev, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

WID = inputs.WORKLOAD_ID


@pytest.fixture(scope="module")
def aq():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import group_wise_affine_aq_amd as mod
    mod.load_library()
    return mod


def _check_quantize(aq, w, G, bits):
    """GPU quantize of W equals the oracle bit for bit; returns the packing."""
    ref = oracle.quantize(w, G, bits)
    got = packed_from_dev(*aq.aq_quantize(to_dev(w), G, bits))
    for name, a, b in zip(("codes", "scales", "biases"), got, ref):
        assert np.array_equal(a, b), f"{name} differ at {np.argwhere(a != b)[:5].tolist()}"
    return ref


def _close(y, y_ref, A, what):
    ok, ratio = oracle.within_tolerance(y, y_ref, A)
    assert ok, f"{what}: worst error/bound {ratio:.3f}"
    return ratio


def test_tiny(aq):
    N = K = 512
    w = inputs.weights(N, K, seed=0, key=(WID["tiny"],))
    c, s, b = _check_quantize(aq, w, 64, 4)
    xb = inputs.activations(1, K, "f16", seed=0, key=(WID["tiny"],))
    y_ref, A = oracle.matmul(inputs.from_bits(xb, "f16"), c, s, b, K, 64, 4)
    y = aq.aq_quantized_matmul(bits_to_dev(xb, "f16"), *packed_to_dev(c, s, b), 64, 4)
    _close(out_to_f64(y), y_ref, A, "tiny")


@pytest.mark.parametrize("N,K", inputs.WORKLOADS["decode"]["shapes"])
def test_decode(aq, N, K):
    w = inputs.weights(N, K, seed=0, key=(WID["decode"],), outliers=True)
    c, s, b = _check_quantize(aq, w, 64, 4)
    xb = inputs.activations(1, K, "f16", seed=0, key=(WID["decode"], N))
    y_ref, A = oracle.matmul(inputs.from_bits(xb, "f16"), c, s, b, K, 64, 4)
    y = aq.aq_quantized_matmul(bits_to_dev(xb, "f16"), *packed_to_dev(c, s, b), 64, 4)
    _close(out_to_f64(y), y_ref, A, f"decode {N}x{K}")


@pytest.mark.parametrize("bits,G", [(4, 64), (8, 128)])
@pytest.mark.parametrize("N,K", inputs.WORKLOADS["specdec"]["shapes"])
def test_specdec(aq, N, K, bits, G):
    w = inputs.weights(N, K, seed=0, key=(WID["specdec"],))
    c, s, b = _check_quantize(aq, w, G, bits)
    dev = packed_to_dev(c, s, b)
    for M in inputs.WORKLOADS["specdec"]["M"]:
        xb = inputs.activations(M, K, "bf16", seed=0, key=(WID["specdec"], N, M))
        y_ref, A = oracle.matmul(inputs.from_bits(xb, "bf16"), c, s, b, K, G, bits)
        y = aq.aq_quantized_matmul(bits_to_dev(xb, "bf16"), *dev, G, bits)
        _close(out_to_f64(y), y_ref, A, f"specdec {N}x{K} b{bits} M{M}")


@pytest.mark.parametrize("bits,G", [(4, 64), (8, 128)])
@pytest.mark.parametrize("N,K", inputs.WORKLOADS["specdec"]["shapes"])
def test_specdec_more_rows(aq, N, K, bits, G):
    """The same matrices at 12..64 rows of x (a batch of decoding sequences):
    the few-row kernel with 16 x rows per slot and slices of 16; every row,
    512 sampled output columns plus the first and last."""
    w = inputs.weights(N, K, seed=0, key=(WID["specdec"],))
    c, s, b = oracle.quantize(w, G, bits)
    dev = packed_to_dev(c, s, b)
    rng = np.random.default_rng(N + bits)
    cols = np.unique(np.concatenate([rng.choice(N, 512, replace=False), [0, N - 1]]))
    for M in sorted({12, 40, *inputs.WORKLOADS["specdec"]["M_batch"]}):
        xb = inputs.activations(M, K, "bf16", seed=0, key=(WID["specdec"], N, M))
        y_ref, A = oracle.matmul(inputs.from_bits(xb, "bf16"), c, s, b, K, G, bits, cols=cols)
        y = aq.aq_quantized_matmul(bits_to_dev(xb, "bf16"), *dev, G, bits)
        _close(out_to_f64(y)[:, cols], y_ref, A, f"specdec {N}x{K} b{bits} M{M}")


@pytest.fixture(scope="module")
def prefill_inputs():
    M, (N, K) = 2048, inputs.WORKLOADS["prefill"]["shapes"][0]
    w = inputs.weights(N, K, seed=0, key=(WID["prefill"],))
    xb = inputs.activations(M, K, "bf16", seed=0, key=(WID["prefill"],))
    return w, xb


@pytest.mark.parametrize("bits,G", [(4, 64), (3, 64), (2, 32)])
def test_prefill(aq, prefill_inputs, bits, G):
    w, xb = prefill_inputs
    N, K = w.shape
    c, s, b = _check_quantize(aq, w, G, bits)
    y = aq.aq_quantized_matmul(bits_to_dev(xb, "bf16"), *packed_to_dev(c, s, b), G, bits)
    rng = np.random.default_rng(bits)
    rows = np.sort(rng.choice(xb.shape[0], 96, replace=False))
    cols = np.sort(rng.choice(N, 384, replace=False))
    # include the tile edges
    rows = np.unique(np.concatenate([rows, [0, 127, 128, 2047]]))
    cols = np.unique(np.concatenate([cols, [0, 255, 256, N - 1]]))
    y_ref, A = oracle.matmul(inputs.from_bits(xb[rows], "bf16"), c, s, b, K, G, bits, cols=cols)
    got = out_to_f64(y)[np.ix_(rows, cols)]
    _close(got, y_ref, A, f"prefill b{bits} G{G}")


def test_moe(aq):
    cfg = inputs.WORKLOADS["moe"]
    (N, K), E, T, topk = cfg["shapes"][0], cfg["experts"], cfg["tokens"], cfg["topk"]
    packs = []
    for e in range(E):
        w = inputs.weights(N, K, seed=0, key=(WID["moe"], e))
        packs.append(_check_quantize(aq, w, 64, 4) if e < 2 else oracle.quantize(w, 64, 4))
    c = np.stack([p[0] for p in packs]); s = np.stack([p[1] for p in packs])
    b = np.stack([p[2] for p in packs])
    ids = inputs.expert_ids(T, E, topk, seed=0, key=(WID["moe"],))
    xb = inputs.activations(T, K, "f16", seed=0, key=(WID["moe"],))
    y_ref, A = oracle.gather_matmul(inputs.from_bits(xb, "f16"), c, s, b, ids, K, 64, 4)
    y = aq.aq_gather_qmv(bits_to_dev(xb, "f16"), *packed_to_dev(c, s, b), to_dev(ids), 64, 4)
    _close(out_to_f64(y), y_ref, A, "moe")


def test_moe_prefill(aq):
    """The same expert stack at prefill size through the matrix-core gather:
    2048 tokens top-6; 128 sampled (token, slot) rows checked against the
    oracle, all rows finite."""
    cfg = inputs.WORKLOADS["moe"]
    (N, K), E, T, topk = cfg["shapes"][0], cfg["experts"], cfg["prefill_tokens"], cfg["topk"]
    packs = [oracle.quantize(inputs.weights(N, K, seed=0, key=(WID["moe"], e)), 64, 4)
             for e in range(E)]
    c = np.stack([p[0] for p in packs]); s = np.stack([p[1] for p in packs])
    b = np.stack([p[2] for p in packs])
    ids = inputs.expert_ids(T, E, topk, seed=0, key=(WID["moe"], 1))
    xb = inputs.activations(T, K, "f16", seed=0, key=(WID["moe"], 1))
    y = out_to_f64(aq.aq_gather_quantized_matmul(bits_to_dev(xb, "f16"), *packed_to_dev(c, s, b),
                                                 to_dev(ids), 64, 4))
    assert np.all(np.isfinite(y))
    rng = np.random.default_rng(7)
    t = rng.integers(0, T, 128)
    j = rng.integers(0, topk, 128)
    x = inputs.from_bits(xb, "f16")[t]
    y_ref, A = oracle.gather_matmul(x, c, s, b, ids[t, j][:, None].astype(np.int32), K, 64, 4)
    _close(y[t, j][:, None, :], y_ref, A, "moe prefill")


def test_embedding(aq):
    import torch
    cfg = inputs.WORKLOADS["embedding"]
    (V, K), G, bits = cfg["shapes"][0], cfg["group_size"][0], cfg["bits"][0]
    w = inputs.weights_device(V, K, device=torch.device("cuda"), seed=0, key=(WID["embedding"],))
    c, s, b = aq.aq_quantize(w, G, bits)
    for T in cfg["tokens"]:
        ids = inputs.token_ids(T, V, seed=0, key=(WID["embedding"],))
        out = aq.aq_embedding(to_dev(ids), c, s, b, G, bits, out_dtype=torch.bfloat16)
        # the rows the tokens refer to, quantized again by the oracle
        rows = np.unique(ids)
        ri = torch.from_numpy(rows.astype(np.int64)).cuda()
        cr, sr, br = oracle.quantize(w[ri].cpu().numpy(), G, bits)
        got = packed_from_dev(c[ri].contiguous(), s[ri].contiguous(), b[ri].contiguous())
        for name, x, y in zip(("codes", "scales", "biases"), got, (cr, sr, br)):
            assert np.array_equal(x, y), f"{name} of referenced rows differ (T={T})"
        ref = oracle.embedding(cr, sr, br, np.searchsorted(rows, ids).astype(np.int32), K, G,
                               bits, oracle.BF16)
        assert np.array_equal(out_bits(out), ref), f"embedding rows differ (T={T})"

