"""CPU oracle for group-wise affine quantization.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``.  The product library never
imports, links or calls anything here, and this package shares no code with
it.  The arithmetic lives in ``aq_oracle.c`` (plain C, binary64); this module
only marshals numpy arrays into it.

Every function takes and returns numpy arrays:
  * weights ``w``: float32 [N, K]
  * codes: uint32 [N, K*bits/32]; scales, biases: uint16 (fp16 bits) [N, K/G]
  * activations: float64 arrays holding the exact fp16/bf16 values
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "aq_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

OK, ERR_ARG, ERR_UNSUPPORTED, ERR_RANGE, ERR_INDEX = 0, -1, -2, -5, -6
F32, F16, BF16 = 0, 1, 2


class OracleError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"oracle {what} failed with status {status}")
        self.status = status


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
             "-Wall", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        path = os.environ.get("AQ_ORACLE_LIB")  # the sanitizer build, if named
        if not path:
            build()
            path = _LIB
        lib = ctypes.CDLL(path)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        sig = {
            "oracle_num_threads": ([], i32),
            "oracle_set_num_threads": ([i32], None),
            "oracle_half_to_double": ([ctypes.c_uint16], ctypes.c_double),
            "oracle_bf16_to_double": ([ctypes.c_uint16], ctypes.c_double),
            "oracle_double_to_half_rne": ([ctypes.c_double], ctypes.c_uint16),
            "oracle_float_to_bf16_rne": ([ctypes.c_float], ctypes.c_uint16),
            "oracle_packed_words_per_row": ([i64, i32], i64),
            "oracle_qweight_bytes": ([i64, i64, i32, i32], i64),
            "oracle_pack": ([vp, i64, i64, i32, vp], i32),
            "oracle_unpack": ([vp, i64, i64, i32, vp], i32),
            "oracle_quantize": ([vp, i64, i64, i32, i32, vp, vp, vp], i32),
            "oracle_quantize_mse": ([vp, i64, i64, i32, i32, i32, i32, vp, vp, vp, vp, vp], i32),
            "oracle_quantize_zp": ([vp, i64, i64, i32, i32, vp, vp, vp, vp], i32),
            "oracle_dequantize_exact": ([vp, vp, vp, i64, i64, i32, i32, vp], i32),
            "oracle_dequantize": ([vp, vp, vp, i64, i64, i32, i32, i32, vp], i32),
            "oracle_embedding": ([vp, vp, vp, i64, i64, i32, i32, vp, i64, i32, vp], i32),
            "oracle_matmul_cols": ([vp, i64, vp, vp, vp, i64, i64, i32, i32, vp, i64, vp, vp], i32),
            "oracle_matmul": ([vp, i64, vp, vp, vp, i64, i64, i32, i32, vp, vp], i32),
            "oracle_gather_matmul": ([vp, i64, vp, vp, vp, i64, i64, i64, vp, i64, i32, i32, vp, vp],
                                     i32),
            "oracle_e2m1_to_double": ([i32], ctypes.c_double),
            "oracle_quantize_mxfp4": ([vp, i64, i64, vp, vp], i32),
            "oracle_dequantize_mxfp4_exact": ([vp, vp, i64, i64, vp], i32),
            "oracle_e4m3_to_double": ([i32], ctypes.c_double),
            "oracle_quantize_mxfp8": ([vp, i64, i64, vp, vp], i32),
            "oracle_dequantize_mxfp8_exact": ([vp, vp, i64, i64, vp], i32),
            "oracle_quantize_nvfp4": ([vp, i64, i64, i32, vp, vp], i32),
            "oracle_dequantize_nvfp4_exact": ([vp, vp, i64, i64, i32, vp], i32),
        }
        for name, (args, res) in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _lib = lib
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return _load().oracle_num_threads()


# --- scalar number-format helpers -------------------------------------------
def set_num_threads(n: int) -> None:
    """Threads used by the oracle's parallel loops from now on."""
    _load().oracle_set_num_threads(int(n))


def half_to_double(h: int) -> float:
    return _load().oracle_half_to_double(int(h))


def bf16_to_double(h: int) -> float:
    return _load().oracle_bf16_to_double(int(h))


def double_to_half_rne(x: float) -> int:
    return int(_load().oracle_double_to_half_rne(float(x)))


def float_to_bf16_rne(x: float) -> int:
    return int(_load().oracle_float_to_bf16_rne(float(x)))


# --- format arithmetic ---------------------------------------------------------
def packed_words_per_row(K: int, bits: int) -> int:
    return int(_load().oracle_packed_words_per_row(K, bits))


def qweight_bytes(N: int, K: int, group_size: int, bits: int) -> int:
    return int(_load().oracle_qweight_bytes(N, K, group_size, bits))


# --- packing -------------------------------------------------------------------
def pack(q: np.ndarray, bits: int) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    N, K = q.shape
    out = np.zeros((N, K * bits // 32), dtype=np.uint32)
    st = _load().oracle_pack(_p(q), N, K, bits, _p(out))
    if st:
        raise OracleError(st, "pack")
    return out


def unpack(codes: np.ndarray, K: int, bits: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint32)
    N = codes.shape[0]
    out = np.zeros((N, K), dtype=np.uint8)
    st = _load().oracle_unpack(_p(codes), N, K, bits, _p(out))
    if st:
        raise OracleError(st, "unpack")
    return out


# --- quantize / dequantize -----------------------------------------------------
def quantize(w: np.ndarray, group_size: int, bits: int):
    """-> (codes uint32 [N, K*b/32], scales uint16 [N, K/G], biases uint16 [N, K/G])"""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    if K % group_size:
        raise OracleError(ERR_ARG, "quantize")
    codes = np.zeros((N, K * bits // 32), dtype=np.uint32)
    scales = np.zeros((N, K // group_size), dtype=np.uint16)
    biases = np.zeros((N, K // group_size), dtype=np.uint16)
    st = _load().oracle_quantize(_p(w), N, K, group_size, bits, _p(codes), _p(scales), _p(biases))
    if st:
        raise OracleError(st, "quantize")
    return codes, scales, biases


def quantize_mse(w: np.ndarray, group_size: int, bits: int, steps: int, only: int = -1,
                 details: bool = False):
    """Range-search quantizer (reading R14): candidate i < steps moves both ends
    of [min, max] inwards by d_i = (max - min) * (i / 200), keeping the centred
    fraction (100 - i)/100 of the width; least binary64 squared error wins.
    only >= 0 evaluates that candidate alone.
    -> (codes, scales, biases), plus (chosen int32 [N, K/G], errs float64
    [N, K/G, steps]) when details."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    if K % group_size:
        raise OracleError(ERR_ARG, "quantize_mse")
    ng = K // group_size
    codes = np.zeros((N, K * bits // 32), dtype=np.uint32)
    scales = np.zeros((N, ng), dtype=np.uint16)
    biases = np.zeros((N, ng), dtype=np.uint16)
    chosen = np.zeros((N, ng), dtype=np.int32)
    errs = np.full((N, ng, steps), np.nan, dtype=np.float64)
    st = _load().oracle_quantize_mse(_p(w), N, K, group_size, bits, steps, only, _p(codes),
                                     _p(scales), _p(biases), _p(chosen), _p(errs))
    if st:
        raise OracleError(st, "quantize_mse")
    if details:
        return codes, scales, biases, chosen, errs
    return codes, scales, biases


def quantize_zp(w: np.ndarray, group_size: int, bits: int):
    """Integer-zero-point quantizer (reading R15): the smallest fp16 scale s
    admitting an integer zero point z in [0, 2^bits - 1] whose grid -z*s + q*s
    spans the group with -z*s an exact fp16 value; bias = -z*s.
    -> (codes, scales, biases, zeros uint8 [N, K/G])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    if K % group_size:
        raise OracleError(ERR_ARG, "quantize_zp")
    ng = K // group_size
    codes = np.zeros((N, K * bits // 32), dtype=np.uint32)
    scales = np.zeros((N, ng), dtype=np.uint16)
    biases = np.zeros((N, ng), dtype=np.uint16)
    zeros = np.zeros((N, ng), dtype=np.uint8)
    st = _load().oracle_quantize_zp(_p(w), N, K, group_size, bits, _p(codes), _p(scales),
                                    _p(biases), _p(zeros))
    if st:
        raise OracleError(st, "quantize_zp")
    return codes, scales, biases, zeros


def dequantize_exact(codes, scales, biases, K: int, group_size: int, bits: int) -> np.ndarray:
    """Exact w^ = q*s + b as float64 [N, K]."""
    N = codes.shape[0]
    out = np.zeros((N, K), dtype=np.float64)
    st = _load().oracle_dequantize_exact(_p(codes), _p(scales), _p(biases), N, K, group_size, bits,
                                         _p(out))
    if st:
        raise OracleError(st, "dequantize_exact")
    return out


def dequantize(codes, scales, biases, K: int, group_size: int, bits: int, out_dtype: int):
    """Dequantize to F32 (float32 array) or F16/BF16 (uint16 bit patterns)."""
    N = codes.shape[0]
    out = np.zeros((N, K), dtype=np.float32 if out_dtype == F32 else np.uint16)
    st = _load().oracle_dequantize(_p(codes), _p(scales), _p(biases), N, K, group_size, bits,
                                   out_dtype, _p(out))
    if st:
        raise OracleError(st, "dequantize")
    return out


def embedding(codes, scales, biases, ids, K: int, group_size: int, bits: int, out_dtype: int):
    """Quantized embedding ("Tutorial 10", s.6): out[t] = dequantize(row ids[t]);
    ids outside [0, V) give zero rows.  F32 -> float32, F16/BF16 -> uint16 bits."""
    ids = np.ascontiguousarray(ids, dtype=np.int32).reshape(-1)
    V, T = codes.shape[0], ids.shape[0]
    out = np.zeros((T, K), dtype=np.float32 if out_dtype == F32 else np.uint16)
    st = _load().oracle_embedding(_p(codes), _p(scales), _p(biases), V, K, group_size, bits,
                                  _p(ids), T, out_dtype, _p(out))
    if st:
        raise OracleError(st, "embedding")
    return out


# --- matmul / gather -------------------------------------------------------------
def matmul(x: np.ndarray, codes, scales, biases, K: int, group_size: int, bits: int, cols=None):
    """y = x @ W^T and A = |x| @ |W|^T (elementwise magnitudes), float64.

    ``x`` is float64 [M, K] (exact activation values).  With ``cols`` only
    those output columns are computed and y, A are [M, len(cols)]."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    M = x.shape[0]
    N = codes.shape[0]
    lib = _load()
    if cols is None:
        y = np.zeros((M, N)); A = np.zeros((M, N))
        st = lib.oracle_matmul(_p(x), M, _p(codes), _p(scales), _p(biases), N, K, group_size, bits,
                               _p(y), _p(A))
    else:
        cols = np.ascontiguousarray(cols, dtype=np.int64)
        y = np.zeros((M, len(cols))); A = np.zeros((M, len(cols)))
        st = lib.oracle_matmul_cols(_p(x), M, _p(codes), _p(scales), _p(biases), N, K, group_size,
                                    bits, _p(cols), len(cols), _p(y), _p(A))
    if st:
        raise OracleError(st, "matmul")
    return y, A


def gather_matmul(x: np.ndarray, codes, scales, biases, ids: np.ndarray, K: int, group_size: int,
                  bits: int):
    """MoE oracle: y[t, j, :] = x[t] @ W_{ids[t, j]}^T; returns (y, A) [T, topk, N]."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, topk = ids.shape
    E, N = codes.shape[0], codes.shape[1]
    y = np.zeros((T, topk, N)); A = np.zeros((T, topk, N))
    st = _load().oracle_gather_matmul(_p(x), T, _p(np.ascontiguousarray(codes)),
                                      _p(np.ascontiguousarray(scales)),
                                      _p(np.ascontiguousarray(biases)), E, N, K, _p(ids), topk,
                                      group_size, bits, _p(y), _p(A))
    if st:
        raise OracleError(st, "gather_matmul")
    return y, A


# --- mxfp4 (reading R16) ----------------------------------------------------------
def e2m1_to_double(code: int) -> float:
    """Value of a 4-bit E2M1 code (bit 3 sign, bits 2..1 exponent, bit 0 mantissa)."""
    return _load().oracle_e2m1_to_double(int(code))


def quantize_mxfp4(w: np.ndarray):
    """w float32 [N, K] (K % 32 == 0) -> (codes uint32 [N, K/8], scales uint8
    [N, K/32] holding X + 127): per group of 32, 2^X with X = floor(log2 max|w|)
    - 2 clamped to [-127, 127], codes the nearest E2M1 values of w / 2^X."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    codes = np.zeros((N, K // 8), dtype=np.uint32)
    scales = np.zeros((N, K // 32), dtype=np.uint8)
    st = _load().oracle_quantize_mxfp4(_p(w), N, K, _p(codes), _p(scales))
    if st:
        raise OracleError(st, "quantize_mxfp4")
    return codes, scales


def dequantize_mxfp4_exact(codes, scales, K: int) -> np.ndarray:
    """Exact code value * 2^X as float64 [N, K]."""
    codes = np.ascontiguousarray(codes, dtype=np.uint32)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    N = codes.shape[0]
    out = np.zeros((N, K), dtype=np.float64)
    st = _load().oracle_dequantize_mxfp4_exact(_p(codes), _p(scales), N, K, _p(out))
    if st:
        raise OracleError(st, "dequantize_mxfp4_exact")
    return out


def dequantize_mxfp4(codes, scales, K: int, out_dtype: int):
    """Dequantize to F32 (float32) or F16/BF16 (uint16 bit patterns), each the
    exact value rounded to nearest even (binary32 holds every value whose
    exponent fits it)."""
    exact = dequantize_mxfp4_exact(codes, scales, K)
    if out_dtype == F32:
        with np.errstate(over="ignore"):
            return exact.astype(np.float32)
    rnd = double_to_half_rne if out_dtype == F16 else (lambda v: float_to_bf16_rne(np.float32(v)))
    return np.vectorize(rnd, otypes=[np.uint16])(exact).astype(np.uint16)


def _round_exact(exact, out_dtype: int):
    if out_dtype == F32:
        with np.errstate(over="ignore", invalid="ignore"):
            return exact.astype(np.float32)

    def bf(v):
        with np.errstate(over="ignore", invalid="ignore"):
            return float_to_bf16_rne(np.float32(v))
    rnd = double_to_half_rne if out_dtype == F16 else bf
    return np.vectorize(rnd, otypes=[np.uint16])(exact).astype(np.uint16)


# --- mxfp8 (reading R17) and nvfp4 (reading R18) ---------------------------------------
def e4m3_to_double(code: int) -> float:
    """Value of an 8-bit E4M3 code (bit 7 sign, bits 6..3 exponent, bits 2..0
    mantissa; magnitude pattern 0x7F is NaN)."""
    return _load().oracle_e4m3_to_double(int(code))


def quantize_mxfp8(w: np.ndarray):
    """w float32 [N, K] (K % 32 == 0) -> (codes uint32 [N, K/4] (bytes in row
    order), scales uint8 [N, K/32] holding X + 127): per group of 32, 2^X with
    X = floor(log2 max|w|) - 8 clamped to [-127, 127], codes the nearest E4M3
    values of w / 2^X."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    codes = np.zeros((N, K // 4), dtype=np.uint32)
    scales = np.zeros((N, K // 32), dtype=np.uint8)
    st = _load().oracle_quantize_mxfp8(_p(w), N, K, _p(codes), _p(scales))
    if st:
        raise OracleError(st, "quantize_mxfp8")
    return codes, scales


def dequantize_mxfp8_exact(codes, scales, K: int) -> np.ndarray:
    """Exact code value * 2^X as float64 [N, K] (NaN for the NaN patterns)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint32)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    N = codes.shape[0]
    out = np.zeros((N, K), dtype=np.float64)
    st = _load().oracle_dequantize_mxfp8_exact(_p(codes), _p(scales), N, K, _p(out))
    if st:
        raise OracleError(st, "dequantize_mxfp8_exact")
    return out


def dequantize_mxfp8(codes, scales, K: int, out_dtype: int):
    """The exact values rounded to nearest even: float32 for F32, uint16 bit
    patterns for F16 / BF16."""
    return _round_exact(dequantize_mxfp8_exact(codes, scales, K), out_dtype)


def quantize_nvfp4(w: np.ndarray, T: int = 0):
    """w float32 [N, K] (K % 16 == 0) -> (codes uint32 [N, K/8], scales uint8
    [N, K/16] E4M3 patterns): with the tensor scale 2^T, per group of 16
    s = the E4M3 value nearest to max|w| / (6 * 2^T), codes the nearest E2M1
    values of w / (s * 2^T)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    codes = np.zeros((N, K // 8), dtype=np.uint32)
    scales = np.zeros((N, K // 16), dtype=np.uint8)
    st = _load().oracle_quantize_nvfp4(_p(w), N, K, int(T), _p(codes), _p(scales))
    if st:
        raise OracleError(st, "quantize_nvfp4")
    return codes, scales


def dequantize_nvfp4_exact(codes, scales, K: int, T: int = 0) -> np.ndarray:
    """Exact code value * s * 2^T as float64 [N, K] (NaN where s is a NaN pattern)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint32)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    N = codes.shape[0]
    out = np.zeros((N, K), dtype=np.float64)
    st = _load().oracle_dequantize_nvfp4_exact(_p(codes), _p(scales), N, K, int(T), _p(out))
    if st:
        raise OracleError(st, "dequantize_nvfp4_exact")
    return out


def dequantize_nvfp4(codes, scales, K: int, out_dtype: int, T: int = 0):
    """The exact values rounded to nearest even (as dequantize_mxfp8)."""
    return _round_exact(dequantize_nvfp4_exact(codes, scales, K, T), out_dtype)


def matmul_dense(x: np.ndarray, w: np.ndarray):
    """y = x @ w^T and A = |x| @ |w|^T in float64 for an exact dequantized w."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    return x @ w.T, np.abs(x) @ np.abs(w).T


def within_tolerance(y, y_ref, A):
    """The matmul acceptance test: |y - y_ref| <= 2^-9 * A + 1e-6 elementwise.

    Returns (ok, worst ratio err/bound)."""
    y = np.asarray(y, dtype=np.float64)
    bound = np.ldexp(1.0, -9) * A + 1e-6
    err = np.abs(y - y_ref)
    ratio = float(np.max(err / bound)) if err.size else 0.0
    return bool(np.all(err <= bound)), ratio
