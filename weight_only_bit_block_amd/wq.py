"""Python binding of the wq C ABI (libwq.so): argument marshalling only.

Tensors are PyTorch device tensors (PyTorch provides device memory and the
current stream); every computation runs in the library's HIP kernels. Each
function raises WqError when the library returns a non-zero status. The library
must be built (``python -m weight_only_bit_block_amd.build``); there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import List, Optional, Sequence, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libwq.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "wq.h")

BLOCK = 32
GEMV_MAX_M = 16
TABLE_ALIGN = 64

_lib = None


class WqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: wq status {status} ({strerror(status)})")


class WqDesc(ctypes.Structure):
    """Mirror of `struct wq_desc` (64 bytes)."""
    _fields_ = [
        ("bits", ctypes.c_int32),
        ("ws_slot", ctypes.c_int32),
        ("N", ctypes.c_int64),
        ("K", ctypes.c_int64),
        ("q_off", ctypes.c_uint64),
        ("s_off", ctypes.c_uint64),
        ("x", ctypes.c_void_p),
        ("y", ctypes.c_void_p),
        ("tile_begin", ctypes.c_int64),
    ]


assert ctypes.sizeof(WqDesc) == 64


def load(path: Optional[str] = None):
    """Load libwq.so (once). Raises if the library has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m weight_only_bit_block_amd.build`")
    lib = ctypes.CDLL(p)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    mm = [P, I64, I64, I64, I, P, P, P, P]
    lib.wq_q_bytes.argtypes = [I64, I64, I]
    lib.wq_q_bytes.restype = ctypes.c_size_t
    lib.wq_s_bytes.argtypes = [I64, I64]
    lib.wq_s_bytes.restype = ctypes.c_size_t
    lib.wq_pack.argtypes = [P, I64, I64, I, P, P, P]
    lib.wq_unpack.argtypes = [P, I64, I64, I, P, P]
    for f in ("wq_gemv", "wq_gemm", "wq_linear", "wq_gemm_noalloc"):
        getattr(lib, f).argtypes = mm
    lib.wq_table_layout.argtypes = [P, I, ctypes.POINTER(ctypes.c_uint64)]
    lib.wq_table_plan.argtypes = [P, I, I64, ctypes.POINTER(ctypes.c_int64)]
    lib.wq_table_plan_gemm.argtypes = [P, I, I64, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_uint64)]
    lib.wq_gemv_grouped.argtypes = [P, P, I, I64, I64, P]
    lib.wq_gemm_grouped.argtypes = [P, P, I, I64, I64, P, ctypes.c_uint64, P]
    lib.wq_embed.argtypes = [P, I64, I64, I64, I, P, P, P, P]
    lib.wq_strerror.argtypes = [I]
    lib.wq_strerror.restype = ctypes.c_char_p
    lib.wq_abi_version.argtypes = []
    for f in ("wq_pack", "wq_unpack", "wq_gemv", "wq_gemm", "wq_linear", "wq_gemm_noalloc", "wq_table_layout",
              "wq_table_plan", "wq_table_plan_gemm", "wq_gemv_grouped", "wq_gemm_grouped", "wq_embed",
              "wq_abi_version"):
        getattr(lib, f).restype = I
    _lib = lib
    return lib


def header_symbols(path: str = HEADER) -> List[str]:
    """Function names declared in include/wq.h."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(wq_[a-z_]+)\s*\(", text)))


def strerror(status: int) -> str:
    try:
        return load().wq_strerror(int(status)).decode()
    except Exception:  # library missing: still produce a message
        return "unknown"


def _check(status: int, where: str) -> None:
    if status != 0:
        raise WqError(status, where)


# ------------------------------------------------------------------ helpers
def _torch():
    import torch
    return torch


_raw_stream = None


def _stream(stream=None, device=None) -> int:
    """Raw hipStream_t of `stream`, else of the current stream of `device`."""
    global _raw_stream
    if stream is not None:
        return int(stream.cuda_stream)
    torch = _torch()
    if _raw_stream is None:
        _raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", False)
    if _raw_stream and device is not None:
        return int(_raw_stream(device))
    return int(torch.cuda.current_stream().cuda_stream)


def _ptr(t) -> int:
    return int(t.data_ptr())


def q_row_bytes(K: int, bits: int) -> int:
    return K * bits // 8


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _dev_tensor(t, dtype, name):
    torch = _torch()
    _need(isinstance(t, torch.Tensor), f"{name} must be a torch.Tensor")
    _need(t.is_cuda, f"{name} must be a device tensor")
    _need(t.dtype == dtype, f"{name} must be {dtype}, got {t.dtype}")
    _need(t.is_contiguous(), f"{name} must be contiguous")


# ------------------------------------------------------------------ entry points
def pack(w, bits: int, q=None, scales=None, check_range: bool = True, stream=None):
    """Quantize + pack fp32 weights w [N, K] -> (q uint8 [N, K*bits/8], scales int16 [N, K/32]).

    With check_range, rejects non-finite weights and blocks whose scale would
    overflow binary16 (max |w| > 65504 * Q) before packing.
    """
    torch = _torch()
    _dev_tensor(w, torch.float32, "w")
    _need(w.dim() == 2, "w must be [N, K]")
    N, K = w.shape
    if check_range and w.numel():
        Qmax = {4: 7, 5: 15}.get(bits, 127)
        _need(bool(torch.isfinite(w).all()), "w has non-finite values")
        _need(float(w.abs().max()) <= 65504.0 * Qmax, "a block scale would overflow binary16")
    if q is None:
        q = torch.empty((N, q_row_bytes(K, bits)), dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty((N, K // BLOCK), dtype=torch.int16, device=w.device)
    _check(load().wq_pack(_ptr(w), N, K, bits, _ptr(q), _ptr(scales), _stream(stream)), "wq_pack")
    return q, scales


def unpack(q, K: int, bits: int, stream=None):
    """Packed codes -> int8 codes [N, K]."""
    torch = _torch()
    _dev_tensor(q, torch.uint8, "q")
    N = q.shape[0]
    codes = torch.empty((N, K), dtype=torch.int8, device=q.device)
    _check(load().wq_unpack(_ptr(q), N, K, bits, _ptr(codes), _stream(stream)), "wq_unpack")
    return codes


def _matmul(fn: str, x, q, scales, bits: int, out=None, stream=None):
    torch = _torch()
    for t, dt, name in ((x, torch.float32, "x"), (q, torch.uint8, "q"), (scales, torch.int16, "scales")):
        if not (isinstance(t, torch.Tensor) and t.is_cuda and t.dtype == dt and t.is_contiguous()):
            _dev_tensor(t, dt, name)                # raises with the reason
    _need(x.dim() == 2, "x must be [M, K]")
    M, K = x.shape
    N = q.shape[0]
    _need(q.shape[1] == q_row_bytes(K, bits), "q has the wrong row length for K and bits")
    _need(tuple(scales.shape) == (N, K // BLOCK), "scales must be [N, K/32]")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    else:
        if not (isinstance(out, torch.Tensor) and out.is_cuda and out.dtype == torch.float32 and out.is_contiguous()):
            _dev_tensor(out, torch.float32, "out")
        _need(tuple(out.shape) == (M, N), "out must be [M, N]")
    st = getattr(load(), fn)(x.data_ptr(), M, K, N, bits, q.data_ptr(), scales.data_ptr(), out.data_ptr(),
                             _stream(stream, x.get_device()))
    if st:
        raise WqError(st, fn)
    return out


def gemv(x, q, scales, bits: int, out=None, stream=None):
    """Decode GEMV, 1 <= M <= 16: y = x @ dequant(q, scales).T in fp32."""
    return _matmul("wq_gemv", x, q, scales, bits, out, stream)


def gemm(x, q, scales, bits: int, out=None, stream=None):
    """Prefill GEMM (fp16 matrix cores, per-block fp32 scaling), any M."""
    return _matmul("wq_gemm", x, q, scales, bits, out, stream)


def gemm_noalloc(x, q, scales, bits: int, out=None, stream=None):
    """Prefill GEMM on the library's fixed per-device scratch (no device
    allocation by the library; the workspace must fit WQ_NOALLOC_SCRATCH_BYTES,
    and calls that overlap on one device race)."""
    return _matmul("wq_gemm_noalloc", x, q, scales, bits, out, stream)


def linear(x, q, scales, bits: int, out=None, stream=None):
    """Dispatch by M: M <= 16 -> gemv, else gemm."""
    return _matmul("wq_linear", x, q, scales, bits, out, stream)


def embed(ids, q, scales, K: int, bits: int, out=None, stream=None):
    """Tied token embedding: out[i] = dequantized row ids[i] of the packed table
    (q, scales) in fp32; ids outside [0, N) give rows of NaN."""
    torch = _torch()
    _dev_tensor(ids, torch.int32, "ids")
    _dev_tensor(q, torch.uint8, "q")
    _dev_tensor(scales, torch.int16, "scales")
    _need(ids.dim() == 1, "ids must be 1-D")
    N = q.shape[0]
    _need(q.shape[1] == q_row_bytes(K, bits), "q has the wrong row length for K and bits")
    _need(tuple(scales.shape) == (N, K // BLOCK), "scales must be [N, K/32]")
    n = ids.shape[0]
    if out is None:
        out = torch.empty((n, K), dtype=torch.float32, device=ids.device)
    else:
        _dev_tensor(out, torch.float32, "out")
        _need(tuple(out.shape) == (n, K), "out must be [len(ids), K]")
    _check(load().wq_embed(_ptr(ids), n, K, N, bits, _ptr(q), _ptr(scales), _ptr(out), _stream(stream)),
           "wq_embed")
    return out


# ------------------------------------------------------------------ package + grouped decode
def table_layout(specs: Sequence[Tuple[int, int, int]]):
    """specs: (bits, N, K) per tensor. Returns (ctypes WqDesc array, package bytes)."""
    arr = (WqDesc * len(specs))()
    for i, (bits, N, K) in enumerate(specs):
        arr[i].bits, arr[i].N, arr[i].K = bits, N, K
    total = ctypes.c_uint64(0)
    _check(load().wq_table_layout(ctypes.addressof(arr) if len(specs) else None, len(specs),
                                  ctypes.byref(total)), "wq_table_layout")
    return arr, int(total.value)


def table_plan(arr, M: int) -> int:
    """Set tile_begin for a grouped call with M rows; returns the total tile count."""
    total = ctypes.c_int64(0)
    _check(load().wq_table_plan(ctypes.addressof(arr) if len(arr) else None, len(arr), M,
                                ctypes.byref(total)), "wq_table_plan")
    return int(total.value)


def table_plan_gemm(arr, M: int) -> Tuple[int, int]:
    """Set tile_begin and ws_slot for a grouped prefill call with M rows;
    returns (launch size, workspace bytes)."""
    total = ctypes.c_int64(0)
    ws = ctypes.c_uint64(0)
    _check(load().wq_table_plan_gemm(ctypes.addressof(arr) if len(arr) else None, len(arr), M,
                                     ctypes.byref(total), ctypes.byref(ws)), "wq_table_plan_gemm")
    return int(total.value), int(ws.value)


class Package:
    """One device allocation holding packed tensors at 64-byte-aligned offsets,
    plus its host tensor table."""

    def __init__(self, specs: Sequence[Tuple[int, int, int]], device="cuda"):
        torch = _torch()
        self.specs = list(specs)
        self.table, self.nbytes = table_layout(self.specs)
        # over-allocate so the base can be aligned to 64 bytes
        self._buf = torch.empty(self.nbytes + TABLE_ALIGN, dtype=torch.uint8, device=device)
        off = (-_ptr(self._buf)) % TABLE_ALIGN
        self.data = self._buf[off: off + self.nbytes]
        self.base = _ptr(self.data)

    def q(self, i: int):
        bits, N, K = self.specs[i]
        o = int(self.table[i].q_off)
        return self.data[o: o + N * K * bits // 8].view(N, K * bits // 8)

    def scales(self, i: int):
        bits, N, K = self.specs[i]
        o = int(self.table[i].s_off)
        return self.data[o: o + N * (K // BLOCK) * 2].view(torch_int16()).view(N, K // BLOCK)

    def pack_into(self, i: int, w, check_range: bool = True, stream=None):
        bits, N, K = self.specs[i]
        _need(tuple(w.shape) == (N, K), f"tensor {i}: expected [{N}, {K}]")
        pack(w, bits, q=self.q(i), scales=self.scales(i), check_range=check_range, stream=stream)


def torch_int16():
    return _torch().int16


class GroupedCall:
    """A planned grouped launch: x / y pointers bound into a device table.
    prefill=False: the decode GEMV of every tensor (wq_gemv_grouped, M <= 16);
    prefill=True: the prefill GEMM of every tensor (wq_gemm_grouped, any M)."""

    def __init__(self, pkg: Package, xs: Sequence, ys: Sequence, M: int, device="cuda", prefill: bool = False):
        torch = _torch()
        _need(len(xs) == len(pkg.specs) and len(ys) == len(pkg.specs), "one x and one y per tensor")
        arr = (WqDesc * len(pkg.specs))()
        ctypes.memmove(arr, pkg.table, ctypes.sizeof(arr))
        for i, (bits, N, K) in enumerate(pkg.specs):
            x, y = xs[i], ys[i]
            _dev_tensor(x, torch.float32, f"x[{i}]")
            _dev_tensor(y, torch.float32, f"y[{i}]")
            _need(tuple(x.shape) == (M, K) and tuple(y.shape) == (M, N), f"tensor {i}: x/y shape")
            arr[i].x, arr[i].y = _ptr(x), _ptr(y)
        self.prefill = prefill
        self.ws_bytes = 0
        if prefill:
            self.total_tiles, self.ws_bytes = table_plan_gemm(arr, M)
        else:
            self.total_tiles = table_plan(arr, M)
        # the prefill workspace (prepared x per distinct input), 256-byte aligned
        self._wsbuf = torch.empty(self.ws_bytes + 256, dtype=torch.uint8, device=device)
        self.ws = _ptr(self._wsbuf) + (-_ptr(self._wsbuf)) % 256
        self.M = M
        self.count = len(pkg.specs)
        self.pkg = pkg
        self.host_table = arr
        raw = torch.frombuffer(bytearray(bytes(arr)), dtype=torch.uint8) if len(arr) else torch.empty(0, dtype=torch.uint8)
        self._tbuf = torch.empty(ctypes.sizeof(arr) + TABLE_ALIGN, dtype=torch.uint8, device=device)
        off = (-_ptr(self._tbuf)) % TABLE_ALIGN
        self.table_dev = self._tbuf[off: off + ctypes.sizeof(arr)]
        self.table_dev.copy_(raw)
        self.keep = (list(xs), list(ys))

    def __call__(self, stream=None):
        if self.prefill:
            _check(load().wq_gemm_grouped(self.pkg.base, _ptr(self.table_dev), self.count, self.total_tiles,
                                          self.M, self.ws, self.ws_bytes, _stream(stream)), "wq_gemm_grouped")
        else:
            _check(load().wq_gemv_grouped(self.pkg.base, _ptr(self.table_dev), self.count,
                                          self.total_tiles, self.M, _stream(stream)), "wq_gemv_grouped")
