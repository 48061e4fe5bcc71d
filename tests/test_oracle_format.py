"""Pins of the CPU oracle's format arithmetic and bit layout against what
the pages print (tests/golden/*.json) and against an independent decoder.

Not GPU tests: they run on the host only."""
import json
import os

import numpy as np
import pytest

import oracle
from group_wise_affine_aq_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --- sizes ------------------------------------------------------------------------
def test_bits_per_weight_g64_b4():
    # "Quantizing a Model for MLX", 'What MLX quantization stores': 4.5 bits/weight
    g = _golden("page_numbers.json")["bits_per_weight_g64_b4"]
    N, K = 7, 64 * 11
    assert oracle.qweight_bytes(N, K, 64, 4) * 8 / (N * K) == g["value"]


def test_size_prediction_70b():
    # 'Predict the size first': 70,553,706,496 params -> 39,686,459,904 bytes
    g = _golden("page_numbers.json")["llama33_70b_prediction"]
    assert g["params"] % 64 == 0
    assert oracle.qweight_bytes(1, g["params"], 64, 4) == g["predicted_bytes"]
    # the measured conversion is 2.1 MB larger (norms, headers): within 0.01%
    assert abs(g["measured_bytes"] - g["predicted_bytes"]) / g["measured_bytes"] < 1e-4


def test_converted_sizes_land_on_4p50():
    g = _golden("page_numbers.json")["converted_sizes_at_4p50_bpw"]
    for name in ("qwen3_14b", "llama31_8b"):
        p, b = g[name]["params"], g[name]["bytes"]
        assert round(b * 8 / p, 2) == 4.50
        pred = oracle.qweight_bytes(1, p - p % 64, 64, 4)
        assert abs(pred - b) / b < 2e-3


def test_bytes_per_param_and_ratio():
    g = _golden("page_numbers.json")["bytes_per_param_g64_b4"]
    assert oracle.qweight_bytes(1, 64, 64, 4) / 64 == g["value"]
    assert round(g["fp16_value"] / g["value"], 2) == g["ratio"]


def test_mlp_matrix_sizes():
    # Tutorial 10, s.4: 4096 x 14336 bf16 = 112 MB; 4-bit + scales ~= 30 MB (no biases)
    g = _golden("page_numbers.json")["mlp_matrix_4096x14336"]
    N, K = 4096, 14336
    assert N * K * 2 == g["bf16_bytes"]
    assert round(g["bf16_bytes"] / 2**20) == g["bf16_mb_printed"]
    with_biases = oracle.qweight_bytes(N, K, 64, 4)
    codes_and_scales = with_biases - N * (K // 64) * 2
    assert round(codes_and_scales / 2**20) == g["codes_plus_scales_mb_printed"]
    # the printed ratio is taken between the rounded sizes (112 / 30)
    mb = round(codes_and_scales / 2**20)
    assert round(g["bf16_mb_printed"] / mb, 1) == g["compression_printed"]


def test_words_per_row():
    for bits in range(2, 9):
        for K in (32, 64, 96, 4096):
            assert oracle.packed_words_per_row(K, bits) * 32 == K * bits


# --- bit layout ----------------------------------------------------------------------
def test_hand_worked_bit_layouts():
    for case in _golden("bit_layout.json")["cases"]:
        b = case["bits"]
        q = np.array([case["codes"]], dtype=np.uint8)
        words = oracle.pack(q, b)
        assert [f"0x{int(v):08x}" for v in words[0]] == case["words"], case
        assert np.array_equal(oracle.unpack(words, q.shape[1], b), q)


@pytest.mark.parametrize("bits", range(2, 9))
def test_pack_unpack_roundtrip(bits):
    rng = np.random.default_rng(bits)
    q = rng.integers(0, 1 << bits, size=(5, 32 * 7), dtype=np.uint8)
    codes = oracle.pack(q, bits)
    assert codes.shape == (5, 7 * bits)
    assert np.array_equal(oracle.unpack(codes, q.shape[1], bits), q)
    # bitstream property: the row as one big integer equals sum q_k << (k*b)
    for n in range(5):
        big = sum(int(v) << (32 * i) for i, v in enumerate(codes[n]))
        assert big == sum(int(v) << (k * bits) for k, v in enumerate(q[n]))


def _tutorial_style_decode(codes, scales, biases, group_size, bits, out="f32"):
    """Independent decoder written from Tutorial 10, s.3: each uint32 word is
    split with right shifts 0, b, 2b, ... and a (1<<b)-1 mask, values are
    flattened word by word, then values*scales + biases in float32 and a cast
    to the scales' dtype (here fp16).  Valid for b dividing 32."""
    assert 32 % bits == 0
    shifts = np.arange(0, 32, bits, dtype=np.uint32)
    vals = (codes[..., None] >> shifts) & np.uint32((1 << bits) - 1)
    vals = vals.reshape(codes.shape[0], -1).astype(np.float32)
    s = np.repeat(scales.view(np.float16).astype(np.float32), group_size, axis=-1)
    b = np.repeat(biases.view(np.float16).astype(np.float32), group_size, axis=-1)
    w32 = vals * s + b
    return w32 if out == "f32" else w32.astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("bits,G", [(2, 32), (4, 64), (8, 128), (4, 32), (8, 64), (2, 128)])
def test_tutorial_decoder_agrees(bits, G):
    w = inputs.weights(6, 4 * G, seed=3, key=(bits, G))
    codes, scales, biases = oracle.quantize(w, G, bits)
    K = w.shape[1]
    ref32 = _tutorial_style_decode(codes, scales, biases, G, bits)
    got32 = oracle.dequantize(codes, scales, biases, K, G, bits, oracle.F32)
    assert np.array_equal(ref32.view(np.uint32), got32.view(np.uint32))
    ref16 = _tutorial_style_decode(codes, scales, biases, G, bits, out="f16")
    got16 = oracle.dequantize(codes, scales, biases, K, G, bits, oracle.F16)
    assert np.array_equal(ref16, got16)
    exact = oracle.dequantize_exact(codes, scales, biases, K, G, bits)
    assert np.array_equal(exact.astype(np.float32).view(np.uint32), got32.view(np.uint32))


def test_three_bit_bytes():
    # b=3: eight codes per three bytes, least significant bits first
    rng = np.random.default_rng(7)
    q = rng.integers(0, 8, size=(3, 64), dtype=np.uint8)
    codes = oracle.pack(q, 3)
    raw = codes.view(np.uint8).reshape(3, -1)
    for n in range(3):
        for c in range(8):
            chunk = q[n, 8 * c:8 * c + 8]
            v = sum(int(x) << (3 * i) for i, x in enumerate(chunk))
            assert list(raw[n, 3 * c:3 * c + 3]) == [v & 255, (v >> 8) & 255, v >> 16]


# --- number-format helpers vs numpy / torch ------------------------------------------
def test_half_decode_all_patterns():
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(p)) for p in pats[::37]])
    r = ref[::37]
    both_nan = np.isnan(got) & np.isnan(r)
    assert np.all((got == r) | both_nan)


def test_half_rne_matches_numpy():
    rng = np.random.default_rng(11)
    xs = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(-9, 5, 3000),
                         [0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e-8, 2.0 ** -25, 3 * 2.0 ** -26]])
    with np.errstate(over="ignore"):  # 65520 and above round to inf, as they should
        for x in xs:
            assert oracle.double_to_half_rne(float(x)) == int(np.float16(x).view(np.uint16)), x
    # infinities stay infinite and NaN stays NaN (numpy agrees on the class)
    for x in (np.inf, -np.inf, np.nan, -np.nan):
        got = np.uint16(oracle.double_to_half_rne(float(x))).view(np.float16)
        want = np.float16(x)
        assert (np.isnan(got) and np.isnan(want)) or (got == want and np.signbit(got) == np.signbit(want))


def test_bf16_rne_matches_torch():
    import torch
    rng = np.random.default_rng(12)
    xs = (rng.standard_normal(4000) * 10.0 ** rng.integers(-30, 30, 4000)).astype(np.float32)
    xs = np.concatenate([xs, np.float32([0.0, -0.0, 3.3895314e38, 1e-45, -2.5e-40])])
    ref = torch.from_numpy(xs).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.float_to_bf16_rne(float(x)) for x in xs], dtype=np.uint16)
    assert np.array_equal(got, ref)
