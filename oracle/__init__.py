"""CPU oracle for weight-only block-32 int4/int8 matmul.

TEST INFRASTRUCTURE ONLY: the tests, the package smoke check and the bench's
CPU-baseline leg may use this module; the product library never does. It
shares no code with the HIP path. The arithmetic lives in ``wq_oracle.c``
(plain C, binary64 matmul); this file only builds and marshals it.

Functions follow the quantizer and matmul described in the TinyMOSS-Diarize
devpost page ("How we built it": weight-only, FP32 activations, dequantization
fused, never materialized), the moss-transcribe-diarize-litert card ("v2
decoder": int4 block-32) and the soniqo MOSS guide, RU implementation notes
(symmetric linear INT8 block-32).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "wq_oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
          "-shared", "-fPIC", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile the C oracle in-tree with gcc and return the library path."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build(force=False)
    lib = ctypes.CDLL(_SO)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I = ctypes.c_int
    lib.wqo_f16_bits_from_f32.argtypes = [ctypes.c_float]
    lib.wqo_f16_bits_from_f32.restype = ctypes.c_uint16
    lib.wqo_f64_from_f16_bits.argtypes = [ctypes.c_uint16]
    lib.wqo_f64_from_f16_bits.restype = ctypes.c_double
    lib.wqo_quantize.argtypes = [P, I64, I64, I, P, P]
    lib.wqo_decode.argtypes = [P, I64, I64, I, P]
    lib.wqo_dequant.argtypes = [P, P, I64, I64, I, P]
    lib.wqo_matmul.argtypes = [P, I64, I64, I64, I, P, P, I, P, P, I]
    lib.wqo_threads.argtypes = [I]
    lib.wqo_threads.restype = I
    lib.wqo_f16_bits_from_f32_array.argtypes = [P, I64, P]
    lib.wqo_f64_from_f16_bits_array.argtypes = [P, I64, P]
    for f in ("wqo_quantize", "wqo_decode", "wqo_dequant", "wqo_matmul",
              "wqo_f16_bits_from_f32_array", "wqo_f64_from_f16_bits_array"):
        getattr(lib, f).restype = None
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _check_bits(bits: int) -> None:
    if bits not in (4, 5, 8):
        raise ValueError("bits must be 4, 5 or 8")


def q_row_bytes(K: int, bits: int) -> int:
    return K * bits // 8


def f16_bits(a) -> np.ndarray:
    """binary32 -> binary16 bit patterns, round to nearest even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    _load().wqo_f16_bits_from_f32_array(_ptr(a), a.size, _ptr(out))
    return out


def f64_from_f16_bits(h) -> np.ndarray:
    """binary16 bit patterns -> binary64 values (exact)."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float64)
    _load().wqo_f64_from_f16_bits_array(_ptr(h), h.size, _ptr(out))
    return out


def quantize(w, bits: int):
    """Quantize + encode fp32 weights [N, K]. Returns (q uint8 [N, K*bits/8], scales uint16 [N, K/32])."""
    _check_bits(bits)
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    q = np.empty((N, q_row_bytes(K, bits)), dtype=np.uint8)
    s = np.empty((N, K // 32), dtype=np.uint16)
    _load().wqo_quantize(_ptr(w), N, K, bits, _ptr(q), _ptr(s))
    return q, s


def decode(q, K: int, bits: int) -> np.ndarray:
    """Packed bytes [N, K*bits/8] -> int8 codes [N, K] (int5: a row is the K/2
    bytes of low nibbles, then the K/8 bytes of bit 4)."""
    _check_bits(bits)
    q = np.ascontiguousarray(q, dtype=np.uint8)
    N = q.shape[0]
    assert q.shape[1] == q_row_bytes(K, bits)
    out = np.empty((N, K), dtype=np.int8)
    _load().wqo_decode(_ptr(q), N, K, bits, _ptr(out))
    return out


def dequant(q, scales, K: int, bits: int) -> np.ndarray:
    """Dequantized weights q*s as binary64 [N, K] (exact)."""
    _check_bits(bits)
    q = np.ascontiguousarray(q, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    N = q.shape[0]
    assert q.shape[1] == q_row_bytes(K, bits) and scales.shape == (N, K // 32)
    out = np.empty((N, K), dtype=np.float64)
    _load().wqo_dequant(_ptr(q), _ptr(scales), N, K, bits, _ptr(out))
    return out


def embed(ids, q, scales, K: int, bits: int) -> np.ndarray:
    """Tied token embedding lookup, binary64 [len(ids), K].

    The MOSS-Transcribe-Diarize LiteRT card ("Files") keeps one tied table for
    the token embedding and the lm_head (`embed_1`, `embed_128`, `logits`); a
    lookup is the table's row for each token. The table here is the packed
    block-32 tensor, so row ids[i] is that row of the dequantized weights.
    Ids outside [0, N) give rows of NaN (this library's convention).
    """
    w = dequant(q, scales, K, bits)
    ids = np.asarray(ids, dtype=np.int64).reshape(-1)
    out = np.full((ids.size, K), np.nan, dtype=np.float64)
    ok = (ids >= 0) & (ids < w.shape[0])
    out[ok] = w[ids[ok]]
    return out


def matmul(x, q, scales, bits: int, x16: bool = False, threads: int = 0):
    """y[m,n] = sum_k x[m,k] q[n,k] s[n,k/32] in binary64, with absum = sum_k |x||w^|.

    x: fp32 [M, K]; q, scales: packed [N, ...]. With x16=True, x is first rounded
    to binary16 (the fp16-activation diagnostic). Returns (y, absum), float64 [M, N].
    """
    _check_bits(bits)
    x = np.ascontiguousarray(x, dtype=np.float32)
    q = np.ascontiguousarray(q, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    M, K = x.shape
    N = q.shape[0]
    assert q.shape[1] == q_row_bytes(K, bits) and scales.shape == (N, K // 32)
    y = np.empty((M, N), dtype=np.float64)
    b = np.empty((M, N), dtype=np.float64)
    _load().wqo_matmul(_ptr(x), M, K, N, bits, _ptr(q), _ptr(scales), int(bool(x16)),
                       _ptr(y), _ptr(b), int(threads))
    return y, b


def threads_used(threads: int = 0) -> int:
    return int(_load().wqo_threads(int(threads)))
