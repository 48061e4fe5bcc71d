"""group_wise_affine_aq_amd -- group-wise affine weight-only quantization for
AMD Instinct MI355X.

Python binding over the C ABI of ``libaq.so`` (``include/aq.h``).  The
functions here only marshal torch tensors (device memory, the current HIP
stream) into the C entry points of the same names; every step of the
computation runs in the library's HIP kernels.  There is no fallback: if the
library has not been built, or a call fails, an exception is raised.

Packed weights use the layout of the pages' container ("Tutorial 10:
Quantization", s.4): codes uint32 [N, K*bits/32] (stored in torch as int32),
scales and biases fp16 [N, K/group_size].  Consumers accept biases=None
(every bias +0).
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "AQError", "lib_path", "load_library", "aq_status_string", "aq_version", "aq_codes_words",
    "aq_qweight_bytes", "aq_quantize", "aq_quantize_mse", "aq_quantize_zp", "aq_dequantize",
    "aq_embedding", "aq_qmv", "aq_qmm",
    "aq_quantized_matmul", "aq_gather_qmv", "aq_gather_qmm", "aq_gather_quantized_matmul",
    "aq_quantize_fp", "aq_dequantize_fp", "aq_qmv_fp", "aq_matmul_fp", "aq_gather_matmul_fp", "aq_qmv_fp_describe",
    "FP_MODES",
]

AQ_OK = 0
AQ_F32, AQ_F16, AQ_BF16 = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path() -> str:
    """The in-tree library, or the file AQ_LIB names (the sanitizer build)."""
    return os.environ.get("AQ_LIB") or os.path.join(_HERE, "libaq.so")


class AQError(RuntimeError):
    def __init__(self, status: int, fn: str):
        msg = _lib.aq_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{fn}: {msg} (status {status})")
        self.status = status


_lib = None


def load_library():
    """Load libaq.so (built by ``python -m group_wise_affine_aq_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"libaq.so not found at {path}; build it with "
                           "`python -m group_wise_affine_aq_amd.build`")
    lib = ctypes.CDLL(path)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    sigs = {
        "aq_status_string": ([i32], ctypes.c_char_p),
        "aq_version": ([], ctypes.c_char_p),
        "aq_codes_words": ([i64, i32], i64),
        "aq_qweight_bytes": ([i64, i64, i32, i32], i64),
        "aq_quantize": ([vp, i32, i64, i64, i32, i32, vp, vp, vp, vp], i32),
        "aq_quantize_mse": ([vp, i32, i64, i64, i32, i32, i32, vp, vp, vp, vp], i32),
        "aq_quantize_zp": ([vp, i32, i64, i64, i32, i32, vp, vp, vp, vp, vp], i32),
        "aq_qmv_describe": ([i64, i64, i64, i32, i32, i32, ctypes.c_char_p, i32], i32),
        "aq_dequantize": ([vp, vp, vp, i64, i64, i32, i32, vp, i32, vp], i32),
        "aq_embedding": ([vp, vp, vp, i64, i64, i32, i32, vp, i64, vp, i32, vp], i32),
        "aq_qmv": ([vp, i32, i64, vp, vp, vp, i64, i64, i32, i32, vp, vp], i32),
        "aq_qmm": ([vp, i32, i64, vp, vp, vp, i64, i64, i32, i32, vp, vp], i32),
        "aq_quantized_matmul": ([vp, i32, i64, vp, vp, vp, i64, i64, i32, i32, vp, vp], i32),
        "aq_gather_qmv": ([vp, i32, i64, vp, vp, vp, i64, i64, i64, vp, i32, i32, i32, vp, vp],
                          i32),
        "aq_gather_qmm": ([vp, i32, i64, vp, vp, vp, i64, i64, i64, vp, i32, i32, i32, vp, vp],
                          i32),
        "aq_gather_quantized_matmul": (
            [vp, i32, i64, vp, vp, vp, i64, i64, i64, vp, i32, i32, i32, vp, vp], i32),
        "aq_quantize_fp": ([vp, i32, i64, i64, i32, i32, vp, vp, vp], i32),
        "aq_dequantize_fp": ([vp, vp, i64, i64, i32, i32, vp, i32, vp], i32),
        "aq_qmv_fp": ([vp, i32, vp, vp, i64, i64, i32, i32, vp, vp], i32),
        "aq_matmul_fp": ([vp, i32, i64, vp, vp, i64, i64, i32, i32, vp, vp], i32),
        "aq_gather_matmul_fp": ([vp, i32, i64, vp, vp, i64, i64, i64, vp, i32, i32, i32, vp, vp],
                                i32),
        "aq_qmv_fp_describe": ([i64, i64, i32, i32, ctypes.c_char_p, i32], i32),
        "aq_bench_stream_read": ([vp, i64, i32, i32, vp, vp], i32),
        "aq_bench_read_oneshot": ([vp, i64, i32, i32, vp, vp], i32),
        "aq_bench_mfma_clock": ([i32, i32, vp, vp], i32),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


# ---- host helpers -------------------------------------------------------------------
def aq_status_string(status: int) -> str:
    return load_library().aq_status_string(status).decode()


def aq_version() -> str:
    return load_library().aq_version().decode()


def aq_codes_words(K: int, bits: int) -> int:
    return int(load_library().aq_codes_words(K, bits))


def aq_qweight_bytes(N: int, K: int, group_size: int, bits: int) -> int:
    return int(load_library().aq_qweight_bytes(N, K, group_size, bits))


# ---- marshalling -----------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    m = {torch.float32: AQ_F32, torch.float16: AQ_F16, torch.bfloat16: AQ_BF16}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def _torch_dtype(code: int):
    torch = _torch()
    return {AQ_F32: torch.float32, AQ_F16: torch.float16, AQ_BF16: torch.bfloat16}[code]


def _dev(t, name):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(st: int, fn: str):
    if st != AQ_OK:
        raise AQError(st, fn)


# ---- device operations -------------------------------------------------------------------
def aq_quantize(w, group_size: int, bits: int, codes=None, scales=None, biases=None, stream=None):
    """Quantize W [N, K] (fp32/fp16/bf16, device) -> (codes, scales, biases)."""
    torch = _torch()
    lib = load_library()
    N, K = w.shape
    if codes is None:
        codes = torch.empty((N, K * bits // 32), dtype=torch.int32, device=w.device)
    if scales is None:
        scales = torch.empty((N, K // group_size), dtype=torch.float16, device=w.device)
    if biases is None:
        biases = torch.empty((N, K // group_size), dtype=torch.float16, device=w.device)
    st = lib.aq_quantize(_dev(w, "w"), _dtype_code(w), N, K, group_size, bits,
                         _dev(codes, "codes"), _dev(scales, "scales"), _dev(biases, "biases"),
                         _stream(stream))
    _check(st, "aq_quantize")
    return codes, scales, biases


def aq_qmv_describe(M: int, N: int, K: int, group_size: int, bits: int, x_dtype="f16") -> str:
    """Name and compile-time shape of the kernel aq_qmv launches for this shape."""
    lib = load_library()
    code = {"f16": AQ_F16, "bf16": AQ_BF16}[x_dtype]
    buf = ctypes.create_string_buffer(160)
    n = lib.aq_qmv_describe(M, N, K, group_size, bits, code, buf, len(buf))
    if n < 0:
        raise AQError(-1, "aq_qmv_describe")
    return buf.value.decode()


def aq_quantize_mse(w, group_size: int, bits: int, steps: int, codes=None, scales=None,
                    biases=None, stream=None):
    """Range-search quantize W [N, K] over `steps` narrowed ranges -> (codes, scales, biases)."""
    torch = _torch()
    lib = load_library()
    N, K = w.shape
    if codes is None:
        codes = torch.empty((N, K * bits // 32), dtype=torch.int32, device=w.device)
    if scales is None:
        scales = torch.empty((N, K // group_size), dtype=torch.float16, device=w.device)
    if biases is None:
        biases = torch.empty((N, K // group_size), dtype=torch.float16, device=w.device)
    st = lib.aq_quantize_mse(_dev(w, "w"), _dtype_code(w), N, K, group_size, bits, steps,
                             _dev(codes, "codes"), _dev(scales, "scales"), _dev(biases, "biases"),
                             _stream(stream))
    _check(st, "aq_quantize_mse")
    return codes, scales, biases


def aq_quantize_zp(w, group_size: int, bits: int, codes=None, scales=None, biases=None,
                   zeros=None, stream=None):
    """Integer-zero-point quantize W [N, K] -> (codes, scales, biases, zeros),
    zeros uint8 [N, K/group_size] with bias = -zero * scale exactly."""
    torch = _torch()
    lib = load_library()
    N, K = w.shape
    if codes is None:
        codes = torch.empty((N, K * bits // 32), dtype=torch.int32, device=w.device)
    if scales is None:
        scales = torch.empty((N, K // group_size), dtype=torch.float16, device=w.device)
    if biases is None:
        biases = torch.empty((N, K // group_size), dtype=torch.float16, device=w.device)
    if zeros is None:
        zeros = torch.empty((N, K // group_size), dtype=torch.uint8, device=w.device)
    st = lib.aq_quantize_zp(_dev(w, "w"), _dtype_code(w), N, K, group_size, bits,
                            _dev(codes, "codes"), _dev(scales, "scales"), _dev(biases, "biases"),
                            _dev(zeros, "zeros"), _stream(stream))
    _check(st, "aq_quantize_zp")
    return codes, scales, biases, zeros


def aq_dequantize(codes, scales, biases, group_size: int, bits: int, out_dtype=None, out=None,
                  stream=None):
    """Dequantize packed weights -> [N, K] in out_dtype (default fp16)."""
    torch = _torch()
    lib = load_library()
    N = codes.shape[0]
    K = scales.shape[1] * group_size
    if out is None:
        out = torch.empty((N, K), dtype=out_dtype or torch.float16, device=codes.device)
    st = lib.aq_dequantize(_dev(codes, "codes"), _dev(scales, "scales"), _dev(biases, "biases"),
                           N, K, group_size, bits, _dev(out, "out"), _dtype_code(out),
                           _stream(stream))
    _check(st, "aq_dequantize")
    return out


def aq_embedding(ids, codes, scales, biases, group_size: int, bits: int, out_dtype=None,
                 out=None, stream=None):
    """Quantized embedding: out[t] = dequantize(table row ids[t]); ids int32 [T]."""
    torch = _torch()
    V = codes.shape[0]
    K = scales.shape[1] * group_size
    T = ids.numel()
    if out is None:
        out = torch.empty((T, K), dtype=out_dtype or torch.float16, device=codes.device)
    st = load_library().aq_embedding(_dev(codes, "codes"), _dev(scales, "scales"),
                                     _dev(biases, "biases"), V, K, group_size, bits,
                                     _dev(ids, "ids"), T, _dev(out, "out"), _dtype_code(out),
                                     _stream(stream))
    _check(st, "aq_embedding")
    return out


def _matmul(fname, x, codes, scales, biases, group_size, bits, y, stream):
    torch = _torch()
    lib = load_library()
    M, K = x.shape
    N = codes.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=x.dtype, device=x.device)
    st = getattr(lib, fname)(_dev(x, "x"), _dtype_code(x), M, _dev(codes, "codes"),
                             _dev(scales, "scales"), _dev(biases, "biases"), N, K, group_size,
                             bits, _dev(y, "y"), _stream(stream))
    _check(st, fname)
    return y


def aq_qmv(x, codes, scales, biases, group_size: int, bits: int, y=None, stream=None):
    """y = x @ W^T for x [M <= 8, K] (decode kernels)."""
    return _matmul("aq_qmv", x, codes, scales, biases, group_size, bits, y, stream)


def aq_qmm(x, codes, scales, biases, group_size: int, bits: int, y=None, stream=None):
    """y = x @ W^T for any M (matrix-core kernel)."""
    return _matmul("aq_qmm", x, codes, scales, biases, group_size, bits, y, stream)


def aq_quantized_matmul(x, codes, scales, biases, group_size: int, bits: int, y=None,
                        stream=None):
    """y = x @ W^T with the kernel chosen per shape."""
    return _matmul("aq_quantized_matmul", x, codes, scales, biases, group_size, bits, y, stream)


def aq_gather_qmv(x, codes, scales, biases, ids, group_size: int, bits: int, y=None,
                  stream=None):
    """MoE: y[t, j, :] = x[t] @ W_{ids[t, j]}^T; codes [E, N, K*bits/32]."""
    return _gather("aq_gather_qmv", x, codes, scales, biases, ids, group_size, bits, y, stream)


def aq_gather_qmm(x, codes, scales, biases, ids, group_size: int, bits: int, y=None,
                  stream=None):
    """MoE at prefill size (matrix cores): same operation as aq_gather_qmv."""
    return _gather("aq_gather_qmm", x, codes, scales, biases, ids, group_size, bits, y, stream)


def aq_gather_quantized_matmul(x, codes, scales, biases, ids, group_size: int, bits: int, y=None,
                               stream=None):
    """MoE with the kernel chosen by routed rows per expert."""
    return _gather("aq_gather_quantized_matmul", x, codes, scales, biases, ids, group_size, bits,
                   y, stream)


def _gather(name, x, codes, scales, biases, ids, group_size, bits, y, stream):
    torch = _torch()
    lib = load_library()
    T, K = x.shape
    E, N = codes.shape[0], codes.shape[1]
    topk = ids.shape[1]
    if y is None:
        y = torch.empty((T, topk, N), dtype=x.dtype, device=x.device)
    st = getattr(lib, name)(_dev(x, "x"), _dtype_code(x), T, _dev(codes, "codes"),
                            _dev(scales, "scales"), _dev(biases, "biases"), E, N, K,
                            _dev(ids, "ids"), topk, group_size, bits, _dev(y, "y"),
                            _stream(stream))
    _check(st, name)
    return y


# ---- measurement helpers (include/aq_bench.h) ----------------------------------------------
def aq_bench_stream_read(buf, blocks: int = 512, unroll: int = 4, sink=None, stream=None):
    """Read all of the device tensor `buf` once with a plain streaming kernel."""
    torch = _torch()
    if sink is None:
        sink = torch.zeros(4, dtype=torch.int32, device=buf.device)
    nbytes = buf.numel() * buf.element_size()
    st = load_library().aq_bench_stream_read(_dev(buf, "buf"), nbytes, blocks, unroll,
                                             _dev(sink, "sink"), _stream(stream))
    _check(st, "aq_bench_stream_read")
    return sink


def aq_bench_read_oneshot(buf, threads: int = 256, unroll: int = 8, sink=None, stream=None):
    """Read all of the device tensor `buf` once, every thread's loads issued up
    front, one contiguous block per workgroup."""
    torch = _torch()
    if sink is None:
        sink = torch.zeros(4, dtype=torch.int32, device=buf.device)
    nbytes = buf.numel() * buf.element_size()
    st = load_library().aq_bench_read_oneshot(_dev(buf, "buf"), nbytes, threads, unroll,
                                              _dev(sink, "sink"), _stream(stream))
    _check(st, "aq_bench_read_oneshot")
    return sink


def aq_bench_mfma_clock(blocks: int, iters: int, out=None, stream=None):
    """Per-wave (shader cycles, 100 MHz ticks) of an MFMA-only loop; int64 [4*blocks, 2]."""
    torch = _torch()
    if out is None:
        out = torch.zeros((4 * blocks, 2), dtype=torch.int64, device=torch.device("cuda"))
    st = load_library().aq_bench_mfma_clock(blocks, iters, _dev(out, "out"), _stream(stream))
    _check(st, "aq_bench_mfma_clock")
    return out


# ---- block-scaled float modes ---------------------------------------------------------
# mode -> (enum value, group size, code bits).  codes uint32 [N, K*bits/32]
# (int32 in torch); scales uint8 [N, K/group]: X + 127 for the mx modes, an
# E4M3 value for nvfp4 (with the tensor scale 2^tensor_exp).
FP_MODES = {"mxfp4": (0, 32, 4), "nvfp4": (1, 16, 4), "mxfp8": (2, 32, 8)}


def aq_quantize_fp(w, mode: str, tensor_exp: int = 0, codes=None, scales=None, stream=None):
    """Quantize W [N, K] (fp32/fp16/bf16, device) in a block-scaled float mode
    -> (codes, scales)."""
    torch = _torch()
    lib = load_library()
    m, g, bits = FP_MODES[mode]
    N, K = w.shape
    if codes is None:
        codes = torch.empty((N, K * bits // 32), dtype=torch.int32, device=w.device)
    if scales is None:
        scales = torch.empty((N, K // g), dtype=torch.uint8, device=w.device)
    st = lib.aq_quantize_fp(_dev(w, "w"), _dtype_code(w), N, K, m, tensor_exp,
                            _dev(codes, "codes"), _dev(scales, "scales"), _stream(stream))
    _check(st, "aq_quantize_fp")
    return codes, scales


def aq_dequantize_fp(codes, scales, K: int, mode: str, tensor_exp: int = 0, out_dtype=None,
                     out=None, stream=None):
    """Block-scaled codes/scales -> W^ [N, K] in out_dtype (default fp32)."""
    torch = _torch()
    lib = load_library()
    N = codes.shape[0]
    if out is None:
        out = torch.empty((N, K), dtype=out_dtype or torch.float32, device=codes.device)
    st = lib.aq_dequantize_fp(_dev(codes, "codes"), _dev(scales, "scales"), N, K,
                              FP_MODES[mode][0], tensor_exp, _dev(out, "out"), _dtype_code(out),
                              _stream(stream))
    _check(st, "aq_dequantize_fp")
    return out


def aq_qmv_fp(x, codes, scales, mode: str, tensor_exp: int = 0, y=None, stream=None):
    """y = x @ W^T for one row x [K] (or [1, K]) in fp16/bf16 and block-scaled W [N, K]."""
    torch = _torch()
    lib = load_library()
    K = x.shape[-1]
    if x.numel() != K:
        raise ValueError("aq_qmv_fp takes one row of x")
    N = codes.shape[0]
    if y is None:
        y = torch.empty(tuple(x.shape[:-1]) + (N,), dtype=x.dtype, device=x.device)
    st = lib.aq_qmv_fp(_dev(x, "x"), _dtype_code(x), _dev(codes, "codes"), _dev(scales, "scales"),
                       N, K, FP_MODES[mode][0], tensor_exp, _dev(y, "y"), _stream(stream))
    _check(st, "aq_qmv_fp")
    return y


def aq_matmul_fp(x, codes, scales, mode: str, tensor_exp: int = 0, y=None, stream=None):
    """y = x @ W^T for x [M, K] (fp16/bf16, device) and block-scaled W [N, K]."""
    torch = _torch()
    lib = load_library()
    M, K = (1, x.shape[-1]) if x.dim() == 1 else (x.shape[0], x.shape[1])
    if x.dim() > 2:
        raise ValueError("aq_matmul_fp takes x as [K] or [M, K]")
    N = codes.shape[0]
    if y is None:
        y = torch.empty(tuple(x.shape[:-1]) + (N,), dtype=x.dtype, device=x.device)
    st = lib.aq_matmul_fp(_dev(x, "x"), _dtype_code(x), M, _dev(codes, "codes"),
                          _dev(scales, "scales"), N, K, FP_MODES[mode][0], tensor_exp,
                          _dev(y, "y"), _stream(stream))
    _check(st, "aq_matmul_fp")
    return y


def aq_gather_matmul_fp(x, codes, scales, ids, mode: str, tensor_exp: int = 0, y=None,
                        stream=None):
    """y[t, j] = x[t] @ W_{ids[t, j]}^T: x [T, K] fp16/bf16, block-scaled experts
    codes [E, N, K*bits/32] (int32), scales [E, N, K/group] (uint8), ids [T, topk]
    (int32), all on the device; y [T, topk, N] in x's dtype."""
    torch = _torch()
    lib = load_library()
    T, K = x.shape
    E, N = codes.shape[0], codes.shape[1]
    topk = ids.shape[1]
    if y is None:
        y = torch.empty((T, topk, N), dtype=x.dtype, device=x.device)
    st = lib.aq_gather_matmul_fp(_dev(x, "x"), _dtype_code(x), T, _dev(codes, "codes"),
                                 _dev(scales, "scales"), E, N, K, _dev(ids, "ids"), topk,
                                 FP_MODES[mode][0], tensor_exp, _dev(y, "y"), _stream(stream))
    _check(st, "aq_gather_matmul_fp")
    return y


def aq_qmv_fp_describe(N: int, K: int, mode: str, x_dtype="f16") -> str:
    """Name and compile-time shape of the kernel aq_qmv_fp launches."""
    lib = load_library()
    code = {"f16": AQ_F16, "bf16": AQ_BF16}[x_dtype]
    buf = ctypes.create_string_buffer(160)
    n = lib.aq_qmv_fp_describe(N, K, FP_MODES[mode][0], code, buf, len(buf))
    if n < 0:
        raise AQError(-1, "aq_qmv_fp_describe")
    return buf.value.decode()
