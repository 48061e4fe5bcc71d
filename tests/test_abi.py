"""The C ABI of libaq: the library loads, exports every entry point that
include/aq.h declares, and rejects bad arguments on the host before anything
is enqueued (these calls never reach a kernel, so they run without a GPU)."""
import ctypes
import os
import re

import pytest

import group_wise_affine_aq_amd as aq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("aq.h", "aq_bench.h")]

OK, INVALID, UNSUPPORTED, ALIGN = 0, -1, -2, -3
F32, F16, BF16 = 0, 1, 2


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(aq_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(aq.lib_path()):
        pytest.skip("libaq.so not built (run python -m group_wise_affine_aq_amd.build)")
    return aq.load_library()


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("aq_quantize", "aq_quantize_mse", "aq_dequantize", "aq_qmv", "aq_qmm", "aq_gather_qmv",
              "aq_quantized_matmul", "aq_codes_words", "aq_qweight_bytes", "aq_status_string",
              "aq_quantize_fp", "aq_dequantize_fp", "aq_qmv_fp", "aq_matmul_fp", "aq_gather_matmul_fp"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    raw = ctypes.CDLL(aq.lib_path())
    for name in declared_functions():
        assert hasattr(raw, name), name


def test_host_helpers(lib):
    assert aq.aq_codes_words(4096, 4) == 512
    assert aq.aq_codes_words(4096, 3) == 384
    assert aq.aq_codes_words(33, 4) == -1
    # 4.5 bits per weight at G=64, 4 bits ("Quantizing a Model for MLX")
    assert aq.aq_qweight_bytes(4096, 14336, 64, 4) == 33030144
    assert aq.aq_qweight_bytes(1, 70553706496, 64, 4) == 39686459904
    assert aq.aq_qweight_bytes(10, 100, 64, 4) == -1
    assert "INVALID" in aq.aq_status_string(INVALID)
    assert aq.aq_status_string(12345) == "unknown aq_status"
    assert aq.aq_version().startswith("libaq")


P = 0x10000  # fake, 16-byte-aligned device addresses: never dereferenced
MIS = 0x10002


def qmv(lib, fn="aq_qmv", x=P, xdt=F16, M=1, codes=P, scales=P, biases=P, N=64, K=128, G=64,
        bits=4, y=P):
    return getattr(lib, fn)(x, xdt, M, codes, scales, biases, N, K, G, bits, y, None)


@pytest.mark.parametrize("fn", ["aq_qmv", "aq_qmm", "aq_quantized_matmul"])
def test_matmul_argument_errors(lib, fn):
    _matmul_argument_errors(lib, fn, 1)


@pytest.mark.parametrize("M", [16, 100, 300])
def test_dispatch_argument_errors_past_eight_rows(lib, M):
    """The shape dispatch validates before its shape heuristics run (a group
    size of 0 must come back as an error, not reach a division)."""
    assert qmv(lib, "aq_quantized_matmul", M=M, G=0) == INVALID
    _matmul_argument_errors(lib, "aq_quantized_matmul", M)


def _matmul_argument_errors(lib, fn, M):
    def call(**k):
        k.setdefault("M", M)
        return qmv(lib, fn, **k)

    assert call(bits=1) == INVALID
    assert call(bits=9) == INVALID
    assert call(G=16) == INVALID
    assert call(G=48) == INVALID
    assert call(K=96, G=64) == INVALID   # K % G != 0
    assert call(N=0) == INVALID
    assert call(K=0) == INVALID
    assert call(M=0) == INVALID
    assert call(xdt=F32) == INVALID
    assert call(xdt=7) == INVALID
    assert call(xdt=-3) == INVALID
    assert call(x=None) == INVALID
    assert call(y=None) == INVALID
    assert call(codes=None) == INVALID
    assert call(scales=None) == INVALID
    # biases=None is valid (every bias +0): test_consumers_take_null_biases
    assert call(x=MIS) == ALIGN
    assert call(y=MIS) == ALIGN
    assert call(codes=MIS) == ALIGN
    assert call(scales=MIS) == ALIGN


def test_qmv_rows_limit(lib):
    assert qmv(lib, "aq_qmv", M=9) == INVALID


def test_embedding_argument_errors(lib):
    def e(codes=P, scales=P, biases=P, V=100, K=128, G=64, bits=4, ids=P, T=3, out=P, dt=F16):
        return lib.aq_embedding(codes, scales, biases, V, K, G, bits, ids, T, out, dt, None)
    assert e(V=0) == INVALID
    assert e(T=0) == INVALID
    assert e(K=96) == INVALID
    assert e(G=16) == INVALID
    assert e(bits=9) == INVALID
    assert e(dt=7) == INVALID
    assert e(ids=None) == INVALID
    assert e(out=None) == INVALID
    assert e(codes=None) == INVALID
    assert e(ids=MIS) == ALIGN
    assert e(out=MIS) == ALIGN
    assert e(scales=MIS) == ALIGN


def test_bench_helper_argument_errors(lib):
    assert lib.aq_bench_stream_read(P, 0, 512, 4, P, None) == INVALID
    assert lib.aq_bench_stream_read(P, 24, 512, 4, P, None) == INVALID   # not a multiple of 16
    assert lib.aq_bench_stream_read(P, 1024, 0, 4, P, None) == INVALID
    assert lib.aq_bench_stream_read(P, 1024, 512, 3, P, None) == INVALID
    assert lib.aq_bench_stream_read(None, 1024, 512, 4, P, None) == INVALID
    assert lib.aq_bench_stream_read(MIS, 1024, 512, 4, P, None) == ALIGN
    assert lib.aq_bench_mfma_clock(0, 10, P, None) == INVALID
    assert lib.aq_bench_mfma_clock(4, 0, P, None) == INVALID
    assert lib.aq_bench_read_oneshot(P, 1024, 128, 8, P, None) == INVALID
    assert lib.aq_bench_read_oneshot(P, 1024, 256, 2, P, None) == INVALID
    assert lib.aq_bench_read_oneshot(P, 1000, 256, 8, P, None) == INVALID
    assert lib.aq_bench_read_oneshot(MIS, 1024, 256, 8, P, None) == ALIGN
    assert lib.aq_bench_read_oneshot(P, 1024, 256, 8, None, None) == INVALID
    assert lib.aq_bench_mfma_clock(4, 10, None, None) == INVALID


def test_qmm_depth_limit(lib):
    # 256 rows of x must stay below 2^31 bytes: K <= 4194303
    assert qmv(lib, "aq_qmm", M=16, K=4194304) == UNSUPPORTED
    assert qmv(lib, "aq_quantized_matmul", M=16, K=4194304) == UNSUPPORTED


def test_qmm_row_limit(lib):
    """The prefill grid holds at most 65535 row tiles of 128 rows."""
    assert qmv(lib, "aq_qmm", M=8388353) == UNSUPPORTED
    assert qmv(lib, "aq_quantized_matmul", M=8388353) == UNSUPPORTED


def test_quantize_dequantize_argument_errors(lib):
    q = lambda **k: lib.aq_quantize(k.get("w", P), k.get("dt", F32), k.get("N", 4), k.get("K", 64),
                                    k.get("G", 64), k.get("bits", 4), k.get("codes", P),
                                    k.get("scales", P), k.get("biases", P), None)
    assert q(bits=0) == INVALID
    assert q(G=256) == INVALID
    assert q(K=100) == INVALID
    assert q(dt=5) == INVALID
    assert q(w=None) == INVALID
    assert q(codes=None) == INVALID
    assert q(w=MIS) == ALIGN
    d = lambda **k: lib.aq_dequantize(k.get("codes", P), P, P, k.get("N", 4), k.get("K", 64), 64,
                                      k.get("bits", 4), k.get("out", P), k.get("dt", F16), None)
    assert d(bits=10) == INVALID
    assert d(dt=9) == INVALID
    assert d(out=None) == INVALID
    assert d(out=MIS) == ALIGN
    assert d(codes=MIS) == ALIGN


def test_qmv_describe(lib):
    d = aq.aq_qmv_describe
    assert d(1, 4096, 4096, 64, 4).startswith("qmv1_kernel<BITS=4, f16, CPL=2")
    assert d(1, 14336, 4096, 64, 4) != d(1, 1024, 4096, 64, 4)
    assert "CPL=7" in d(1, 4096, 14336, 64, 4, "bf16")
    assert d(1, 4096, 14336, 64, 4).endswith("W=8, SL=2>")
    assert d(1, 4096, 14336, 32, 4).endswith("SL=4>")
    assert d(1, 4096, 14336, 128, 8).endswith("SL=1>")
    assert d(4, 14336, 4096, 64, 4, "bf16").startswith("qmvm_kernel<bf16, BITS=4")
    assert d(3, 100, 256, 64, 3).startswith("qmv vector kernel")
    buf = ctypes.create_string_buffer(8)
    n = lib.aq_qmv_describe(1, 4096, 4096, 64, 4, F16, buf, 8)
    assert n > 8 and len(buf.value) == 7  # truncated, NUL-terminated
    for bad in (dict(M=0), dict(M=9), dict(K=100), dict(bits=1)):
        k = dict(M=1, K=4096, bits=4)
        k.update(bad)
        assert lib.aq_qmv_describe(k["M"], 64, k["K"], 64, k["bits"], F16, buf, 8) == -1


def test_quantize_mse_argument_errors(lib):
    q = lambda **k: lib.aq_quantize_mse(k.get("w", P), F32, 4, k.get("K", 64), 64, k.get("bits", 4),
                                        k.get("steps", 20), P, P, k.get("biases", P), None)
    assert q(steps=0) == INVALID
    assert q(steps=51) == INVALID
    assert q(bits=1) == INVALID
    assert q(K=96) == INVALID
    assert q(biases=None) == INVALID
    assert q(w=MIS) == ALIGN


def test_quantize_zp_argument_errors(lib):
    q = lambda **k: lib.aq_quantize_zp(k.get("w", P), k.get("dt", F32), 4, k.get("K", 64), 64,
                                       k.get("bits", 4), k.get("codes", P), P,
                                       k.get("biases", P), k.get("zeros", None), None)
    assert q(bits=1) == INVALID
    assert q(bits=9) == INVALID
    assert q(K=96) == INVALID
    assert q(dt=7) == INVALID
    assert q(w=None) == INVALID
    assert q(codes=None) == INVALID
    assert q(biases=None) == INVALID       # the quantizers always write biases
    assert q(w=MIS) == ALIGN
    assert q(zeros=MIS) == ALIGN           # zeros optional, aligned when given


def test_fp_mode_argument_errors(lib):
    """Block-scaled float modes: K a multiple of the mode's group (32, 16,
    32), a tensor exponent only for nvfp4 (|T| <= 100), every pointer
    required and 16-byte aligned; the decode product takes K a multiple of
    32 up to 49152."""
    MX4, NV4, MX8 = 0, 1, 2
    q = lambda **k: lib.aq_quantize_fp(k.get("w", P), k.get("dt", F32), k.get("N", 4),
                                       k.get("K", 64), k.get("mode", MX4), k.get("T", 0),
                                       k.get("codes", P), k.get("scales", P), None)
    assert q(K=48) == INVALID
    assert q(K=40, mode=NV4) == INVALID
    assert q(K=0) == INVALID
    assert q(N=0) == INVALID
    assert q(mode=3) == INVALID
    assert q(mode=-1) == INVALID
    assert q(T=1) == INVALID              # the mx modes take no tensor scale
    assert q(mode=MX8, T=-2) == INVALID
    assert q(mode=NV4, T=101) == INVALID
    assert q(mode=NV4, T=-101) == INVALID
    assert q(dt=3) == INVALID
    assert q(w=None) == INVALID
    assert q(scales=None) == INVALID
    assert q(w=MIS) == ALIGN
    assert q(mode=NV4, T=-100, scales=MIS) == ALIGN
    d = lambda **k: lib.aq_dequantize_fp(k.get("codes", P), k.get("scales", P), 4,
                                         k.get("K", 64), k.get("mode", MX8), k.get("T", 0),
                                         k.get("out", P), k.get("dt", F16), None)
    assert d(K=40) == INVALID
    assert d(mode=5) == INVALID
    assert d(dt=4) == INVALID
    assert d(out=None) == INVALID
    assert d(scales=None) == INVALID
    assert d(codes=MIS) == ALIGN
    assert d(mode=NV4, T=7, out=MIS) == ALIGN
    m = lambda **k: lib.aq_qmv_fp(k.get("x", P), k.get("dt", F16), k.get("codes", P),
                                  k.get("scales", P), k.get("N", 4), k.get("K", 64),
                                  k.get("mode", MX4), k.get("T", 0), k.get("y", P), None)
    assert m(dt=F32) == INVALID           # activations are fp16 or bf16
    assert m(K=33) == INVALID
    assert m(N=0) == INVALID
    assert m(y=None) == INVALID
    assert m(mode=MX8, T=3) == INVALID
    assert m(scales=MIS) == ALIGN
    assert m(x=MIS) == ALIGN
    assert m(K=49152 + 32) == UNSUPPORTED
    assert m(mode=NV4, K=48) == UNSUPPORTED  # a whole group, not a whole 32-code chunk
    mm = lambda **k: lib.aq_matmul_fp(k.get("x", P), k.get("dt", F16), k.get("M", 4),
                                      k.get("codes", P), k.get("scales", P), k.get("N", 4),
                                      k.get("K", 64), k.get("mode", MX4), k.get("T", 0),
                                      k.get("y", P), None)
    assert mm(M=0) == INVALID
    assert mm(M=-3) == INVALID
    assert mm(dt=F32) == INVALID
    assert mm(K=33) == INVALID
    assert mm(N=0) == INVALID
    assert mm(y=None) == INVALID
    assert mm(codes=None) == INVALID
    assert mm(mode=MX4, T=2) == INVALID
    assert mm(scales=MIS) == ALIGN
    assert mm(x=MIS) == ALIGN
    assert mm(K=49152 + 32) == UNSUPPORTED
    assert mm(mode=NV4, K=48) == UNSUPPORTED
    assert mm(M=16 * 65535 + 1) == UNSUPPORTED
    assert mm(M=1, K=33) == INVALID       # one row: the decode product's checks
    g = lambda **k: lib.aq_gather_matmul_fp(k.get("x", P), k.get("dt", F16), k.get("T", 4),
                                            k.get("codes", P), k.get("scales", P), k.get("E", 3),
                                            k.get("N", 4), k.get("K", 64), k.get("ids", P),
                                            k.get("topk", 2), k.get("mode", MX4), k.get("T_", 0),
                                            k.get("y", P), None)
    assert g(T=0) == INVALID
    assert g(E=0) == INVALID
    assert g(topk=0) == INVALID
    assert g(dt=F32) == INVALID
    assert g(K=33) == INVALID
    assert g(mode=4) == INVALID
    assert g(T_=1) == INVALID             # the mx modes take no tensor scale
    assert g(ids=None) == INVALID
    assert g(ids=MIS) == ALIGN
    assert g(y=MIS) == ALIGN
    assert g(K=49152 + 32) == UNSUPPORTED
    assert g(E=65536) == UNSUPPORTED
    assert g(mode=NV4, K=48) == UNSUPPORTED
    buf = ctypes.create_string_buffer(96)
    assert lib.aq_qmv_fp_describe(4096, 49152 + 32, MX4, F16, buf, 96) == -1
    assert lib.aq_qmv_fp_describe(4096, 100, MX4, F16, buf, 96) == -1
    assert lib.aq_qmv_fp_describe(4096, 4096, 9, F16, buf, 96) == -1
    d = aq.aq_qmv_fp_describe
    assert d(14336, 4096, "mxfp4") == "qmv1_fp_kernel<mxfp4, f16, CPL=2, UD=1, W=4>"
    assert d(4096, 14336, "mxfp8", "bf16") == "qmv1_fp_kernel<mxfp8, bf16, CPL=7, UD=1, W=8>"
    assert d(4096, 14336, "nvfp4") == "qmv1_fp_kernel<nvfp4, f16, CPL=7, UD=1, W=8>"
    assert d(4096, 16384, "nvfp4").startswith("qmv1_fp_lds_kernel<nvfp4")
    assert d(4096, 28672, "mxfp4").startswith("qmv1_fp_lds_kernel<mxfp4, f16")


def test_consumers_take_null_biases(lib):
    """A null bias array is accepted by every consumer (every bias +0); the
    other checks still run: a misaligned scale array is still refused, and a
    misaligned bias array too when one is given."""
    for fn in ("aq_qmv", "aq_qmm", "aq_quantized_matmul"):
        assert qmv(lib, fn, biases=None, scales=MIS) == ALIGN
        assert qmv(lib, fn, biases=None, bits=1) == INVALID
        assert qmv(lib, fn, biases=MIS) == ALIGN
        assert qmv(lib, fn, biases=None, codes=None) == INVALID
    assert lib.aq_dequantize(P, MIS, None, 4, 64, 64, 4, P, F16, None) == ALIGN
    assert lib.aq_dequantize(P, P, None, 4, 64, 64, 9, P, F16, None) == INVALID
    assert lib.aq_embedding(P, MIS, None, 4, 64, 64, 4, P, 2, P, F16, None) == ALIGN
    for name in ("aq_gather_qmv", "aq_gather_qmm", "aq_gather_quantized_matmul"):
        assert getattr(lib, name)(P, F16, 4, P, MIS, None, 8, 64, 128, P, 2, 64, 4, P,
                                  None) == ALIGN
        assert getattr(lib, name)(P, F16, 4, P, P, None, 8, 64, 128, P, 0, 64, 4, P,
                                  None) == INVALID


def test_gather_argument_errors(lib):
    g = lambda **k: lib.aq_gather_qmv(k.get("x", P), k.get("dt", F16), k.get("T", 4), P, P, P,
                                      k.get("E", 8), 64, k.get("K", 128), k.get("ids", P),
                                      k.get("topk", 2), k.get("G", 64), k.get("bits", 4),
                                      k.get("y", P), None)
    assert g(T=0) == INVALID
    assert g(E=0) == INVALID
    assert g(topk=0) == INVALID
    assert g(ids=None) == INVALID
    assert g(ids=MIS + 2) == ALIGN
    assert g(K=100) == INVALID
    assert g(dt=F32) == INVALID
    assert g(E=70000) == UNSUPPORTED
    for name in ("aq_gather_qmm", "aq_gather_quantized_matmul"):
        h = lambda **k: getattr(lib, name)(k.get("x", P), k.get("dt", F16), k.get("T", 4), P, P, P,
                                           k.get("E", 8), 64, k.get("K", 128), k.get("ids", P),
                                           k.get("topk", 2), 64, 4, k.get("y", P), None)
        assert h(T=0) == INVALID
        assert h(ids=None) == INVALID
        assert h(y=MIS) == ALIGN
        assert h(dt=F32) == INVALID
    # x too large for 32-bit offsets on the matrix-core gather
    assert lib.aq_gather_qmm(P, F16, 1 << 20, P, P, P, 8, 64, 1 << 11, P, 2, 64, 4, P,
                             None) == UNSUPPORTED


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(aq, "_lib", None)
    monkeypatch.setattr(aq, "lib_path", lambda: str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="libaq.so not found"):
        aq.load_library()
