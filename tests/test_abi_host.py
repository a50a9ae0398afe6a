"""Host-side checks of the C ABI (no GPU): the library loads, exports every
symbol the header declares, and rejects bad arguments before any launch.

Every call here fails validation on the host, so no HIP function runs.
"""
import ctypes

import pytest

import weight_only_bit_block_amd as wqa
from weight_only_bit_block_amd import wq as W

OK, NULL, SHAPE, BITS, ALIGN, MRANGE, HIP, TABLE = range(8)
FAKE = 0x10000          # 16-byte aligned, never dereferenced (validation fails first)
MIS = 0x10004           # misaligned


@pytest.fixture(scope="module")
def lib():
    return wqa.load()


def test_exports_every_header_symbol(lib):
    syms = W.header_symbols()
    assert {"wq_pack", "wq_unpack", "wq_gemv", "wq_gemm", "wq_linear", "wq_gemv_grouped",
            "wq_table_layout", "wq_table_plan", "wq_q_bytes", "wq_s_bytes", "wq_strerror",
            "wq_embed", "wq_abi_version", "wq_table_plan_gemm", "wq_gemm_grouped", "wq_gemm_noalloc"} <= set(syms)
    for s in syms:
        assert hasattr(lib, s), s
    assert lib.wq_abi_version() == 7


def test_sizes(lib):
    assert lib.wq_q_bytes(2048, 1024, 4) == 2048 * 512
    assert lib.wq_q_bytes(151936, 1024, 8) == 151936 * 1024
    assert lib.wq_s_bytes(2048, 1024) == 2048 * 32 * 2
    assert lib.wq_q_bytes(10, 33, 4) == 0 and lib.wq_q_bytes(10, 32, 6) == 0
    # int5: 5K/8 bytes per row, K % 128 == 0
    assert lib.wq_q_bytes(10, 128, 5) == 800 and lib.wq_q_bytes(10, 96, 5) == 0


@pytest.mark.parametrize("fn", ["wq_gemv", "wq_gemm", "wq_linear"])
def test_matmul_validation(lib, fn):
    f = getattr(lib, fn)
    # bits
    assert f(FAKE, 1, 32, 8, 6, FAKE, FAKE, FAKE, None) == BITS
    # shapes
    assert f(FAKE, 1, 33, 8, 4, FAKE, FAKE, FAKE, None) == SHAPE
    assert f(FAKE, 1, 96, 8, 5, FAKE, FAKE, FAKE, None) == SHAPE      # int5 needs K % 128 == 0
    assert f(None, 1, 128, 8, 5, FAKE, FAKE, FAKE, None) == NULL      # int5 accepted
    assert f(FAKE, 1, 0, 8, 4, FAKE, FAKE, FAKE, None) == SHAPE
    assert f(FAKE, -1, 32, 8, 4, FAKE, FAKE, FAKE, None) == SHAPE
    assert f(FAKE, 1, 32, -8, 4, FAKE, FAKE, FAKE, None) == SHAPE
    # empty calls succeed without launching, even with null pointers
    assert f(None, 0, 32, 8, 4, None, None, None, None) == OK
    assert f(None, 3, 32, 0, 8, None, None, None, None) == OK
    # nulls
    assert f(None, 1, 32, 8, 4, FAKE, FAKE, FAKE, None) == NULL
    assert f(FAKE, 1, 32, 8, 4, None, FAKE, FAKE, None) == NULL
    assert f(FAKE, 1, 32, 8, 4, FAKE, None, FAKE, None) == NULL
    assert f(FAKE, 1, 32, 8, 4, FAKE, FAKE, None, None) == NULL
    # alignment
    assert f(MIS, 1, 32, 8, 4, FAKE, FAKE, FAKE, None) == ALIGN
    assert f(FAKE, 1, 32, 8, 4, MIS, FAKE, FAKE, None) == ALIGN
    assert f(FAKE, 1, 32, 8, 4, FAKE, MIS, FAKE, None) == ALIGN
    assert f(FAKE, 1, 32, 8, 4, FAKE, FAKE, MIS, None) == ALIGN


def test_gemv_m_range(lib):
    assert lib.wq_gemv(FAKE, 17, 32, 8, 4, FAKE, FAKE, MIS, None) == ALIGN   # checks in order
    assert lib.wq_gemv(FAKE, 17, 32, 8, 4, FAKE, FAKE, FAKE + 16, None) == MRANGE


def test_pack_unpack_validation(lib):
    assert lib.wq_pack(FAKE, 4, 32, 3, FAKE, FAKE, None) == BITS
    assert lib.wq_pack(FAKE, 4, 32, 5, FAKE, FAKE, None) == SHAPE
    assert lib.wq_pack(None, 4, 128, 5, FAKE, FAKE, None) == NULL
    assert lib.wq_pack(FAKE, 4, 48, 4, FAKE, FAKE, None) == SHAPE
    assert lib.wq_pack(None, 4, 32, 4, FAKE, FAKE, None) == NULL
    assert lib.wq_pack(FAKE, 4, 32, 4, MIS, FAKE, None) == ALIGN
    assert lib.wq_pack(None, 0, 32, 4, None, None, None) == OK
    assert lib.wq_unpack(FAKE, 4, 32, 4, None, None) == NULL
    assert lib.wq_unpack(FAKE, 4, 32, 9, FAKE, None) == BITS


def test_embed_validation(lib):
    f = lib.wq_embed
    assert f(FAKE, 4, 32, 8, 6, FAKE, FAKE, FAKE, None) == BITS
    assert f(FAKE, 4, 48, 8, 8, FAKE, FAKE, FAKE, None) == SHAPE
    assert f(FAKE, -1, 32, 8, 8, FAKE, FAKE, FAKE, None) == SHAPE
    assert f(FAKE, 4, 32, -8, 8, FAKE, FAKE, FAKE, None) == SHAPE
    # empty lookups succeed without launching, even with null pointers
    assert f(None, 0, 32, 8, 8, None, None, None, None) == OK
    assert f(None, 4, 32, 8, 8, FAKE, FAKE, FAKE, None) == NULL
    assert f(FAKE, 4, 32, 8, 8, None, FAKE, FAKE, None) == NULL
    assert f(FAKE, 4, 32, 8, 8, FAKE, None, FAKE, None) == NULL
    assert f(FAKE, 4, 32, 8, 8, FAKE, FAKE, None, None) == NULL
    assert f(FAKE + 2, 4, 32, 8, 8, FAKE, FAKE, FAKE, None) == ALIGN
    assert f(FAKE, 4, 32, 8, 8, MIS, FAKE, FAKE, None) == ALIGN
    assert f(FAKE, 4, 32, 8, 8, FAKE, MIS, FAKE, None) == ALIGN
    assert f(FAKE, 4, 32, 8, 8, FAKE, FAKE, MIS, None) == ALIGN
    # an empty table needs no table pointers (every row is out of range)
    assert f(FAKE, 4, 32, 0, 8, None, None, MIS, None) == ALIGN


def test_table_layout_and_plan(lib):
    specs = [(4, 2048, 1024), (4, 1024, 1024), (8, 1024, 2048), (4, 3, 96), (8, 151936, 1024)]
    arr, total = wqa.table_layout(specs)
    end = 0
    for i, (bits, N, K) in enumerate(specs):
        d = arr[i]
        assert d.q_off % 64 == 0 and d.s_off % 64 == 0
        assert d.q_off >= end
        assert d.s_off >= d.q_off + N * K * bits // 8
        end = d.s_off + N * (K // 32) * 2
    assert total % 64 == 0 and total >= end and total - end < 64
    # plan needs x / y pointers
    with pytest.raises(wqa.WqError):
        wqa.table_plan(arr, 1)
    for i in range(len(specs)):
        arr[i].x, arr[i].y = FAKE, FAKE
    tiles = wqa.table_plan(arr, 1)
    begins = [arr[i].tile_begin for i in range(len(specs))]
    assert begins[0] == 0 and begins == sorted(begins) and tiles > begins[-1]
    with pytest.raises(wqa.WqError) as e:
        wqa.table_plan(arr, 17)
    assert e.value.status == MRANGE
    arr[1].x = MIS
    with pytest.raises(wqa.WqError) as e:
        wqa.table_plan(arr, 1)
    assert e.value.status == ALIGN
    arr[1].x = FAKE
    arr[2].q_off += 32
    with pytest.raises(wqa.WqError) as e:
        wqa.table_plan(arr, 1)
    assert e.value.status == ALIGN


def test_grouped_validation(lib):
    assert lib.wq_gemv_grouped(FAKE, FAKE, 3, 10, 0, None) == MRANGE
    assert lib.wq_gemv_grouped(FAKE, FAKE, 3, 10, 17, None) == MRANGE
    assert lib.wq_gemv_grouped(None, FAKE, 3, 10, 1, None) == NULL
    assert lib.wq_gemv_grouped(FAKE + 16, FAKE, 3, 10, 1, None) == ALIGN
    assert lib.wq_gemv_grouped(FAKE, FAKE + 16, 3, 10, 1, None) == ALIGN
    assert lib.wq_gemv_grouped(None, None, 0, 0, 1, None) == OK


def test_gemm_x_offset_limit(lib):
    """The prefill kernels address the binary16 copy of x with 32-bit byte
    offsets: M * K * 2 >= 2^32 is refused before anything is launched."""
    for fn in ("wq_gemm", "wq_linear"):
        assert getattr(lib, fn)(FAKE, 1 << 21, 1024, 8, 4, FAKE, FAKE, FAKE, None) == SHAPE


def _r256(b):
    return -(-b // 256) * 256


def _ksplit(M, K):
    """Work items per tile: long K loops of short prefills (M <= 128) are split
    into pieces of about 1024 of K (2 to 8 of them)."""
    return 1 if M > 128 else max(1, min(8, K // 1024))


def _gemm_items(M, N, K):
    bm = 64 if M <= 128 else 128
    return -(-M // bm) * -(-N // 128) * _ksplit(M, K)


def _header(M, items):
    """Split-K header of the workspace (M <= 128): a flag per item, then a
    64 x 128 fp32 partial tile per item."""
    return 0 if M > 128 else _r256(4 * items) + items * 64 * 128 * 4


def _ws_bytes(M, K):
    return _r256(M * K * 2) + _r256(M * 4)


@pytest.mark.parametrize("M", [1, 100, 128, 129, 512, 513, 1024, 4096])
def test_table_plan_gemm(lib, M):
    """Grouped prefill plan: longest K first (ties in table order), entries at
    multiples of 8 items, one tile shape per M."""
    specs = [(4, 2048, 1024), (4, 1024, 1024), (4, 1024, 2048), (8, 3, 96), (4, 1024, 3072),
             (5, 300, 1024)]
    arr, _ = wqa.table_layout(specs)
    with pytest.raises(wqa.WqError):
        wqa.table_plan_gemm(arr, M)                  # x / y not bound yet
    for i in range(len(specs)):
        arr[i].x, arr[i].y = FAKE + 4096 * i, FAKE
    total, ws = wqa.table_plan_gemm(arr, M)
    order = sorted(range(len(specs)), key=lambda i: (-specs[i][2], i))
    cur = 0
    for i in order:
        cur = -(-cur // 8) * 8
        assert arr[i].tile_begin == cur, (i, arr[i].tile_begin, cur)
        cur += _gemm_items(M, specs[i][1], specs[i][2])
    assert total == cur
    # every entry reads its own x here: one workspace slot each, in table order,
    # after the split-K header
    off = _header(M, total)
    for i, (bits, N, K) in enumerate(specs):
        assert arr[i].ws_slot * 256 == off
        off += _ws_bytes(M, K)
    assert ws == off


def test_table_plan_gemm_validation(lib):
    specs = [(4, 256, 1024), (8, 128, 64)]
    arr, _ = wqa.table_layout(specs)
    for i in range(len(specs)):
        arr[i].x, arr[i].y = FAKE, FAKE
    for M in (0, -1, (1 << 30) + 1):
        with pytest.raises(wqa.WqError) as e:
            wqa.table_plan_gemm(arr, M)
        assert e.value.status == MRANGE
    with pytest.raises(wqa.WqError) as e:
        wqa.table_plan_gemm(arr, 1 << 21)            # M * K * 2 >= 2^32
    assert e.value.status == SHAPE
    arr[1].y = MIS
    with pytest.raises(wqa.WqError) as e:
        wqa.table_plan_gemm(arr, 64)
    assert e.value.status == ALIGN
    arr[1].y = FAKE
    arr[0].bits = 6
    with pytest.raises(wqa.WqError) as e:
        wqa.table_plan_gemm(arr, 64)
    assert e.value.status == BITS
    arr[0].bits = 4
    total, ws = wqa.table_plan_gemm(arr, 64)
    assert total > 0 and ws == _header(64, total) + _ws_bytes(64, 1024) + _ws_bytes(64, 64)
    empty = (W.WqDesc * 0)()
    assert wqa.table_plan_gemm(empty, 64) == (0, 0)


def test_table_plan_gemm_shared_inputs(lib):
    """Entries reading the same x (pointer and K) with the same code order share
    a workspace slot; int8 (its own operand order) gets a slot of its own."""
    specs = [(4, 2048, 1024), (4, 1024, 1024), (8, 1024, 1024), (5, 512, 1024), (4, 1024, 3072),
             (8, 256, 1024)]
    arr, _ = wqa.table_layout(specs)
    xa, xb = FAKE, FAKE + 4096
    for i, x in enumerate([xa, xa, xa, xa, xb, xa]):
        arr[i].x, arr[i].y = x, FAKE
    M = 200                                           # no split-K header above M = 128
    _, ws = wqa.table_plan_gemm(arr, M)
    raw = [arr[i].ws_slot for i in range(len(specs))]
    # the first entry of each slot prepares it (ws_slot >= 0); later sharers hold the complement
    assert [r >= 0 for r in raw] == [True, False, True, False, True, False]
    s = [r if r >= 0 else ~r for r in raw]
    assert s[0] == s[1] == s[3] == 0                  # int4 / int5 order, x_a
    assert s[2] == s[5] == _ws_bytes(M, 1024) // 256  # int8 order, x_a
    assert s[4] == 2 * _ws_bytes(M, 1024) // 256      # x_b (K = 3072)
    assert ws == 2 * _ws_bytes(M, 1024) + _ws_bytes(M, 3072)


def test_gemm_grouped_validation(lib):
    g = lib.wq_gemm_grouped
    assert g(FAKE, FAKE, 3, 10, 0, FAKE, 256, None) == MRANGE
    assert g(FAKE, FAKE, 3, 10, (1 << 30) + 1, FAKE, 256, None) == MRANGE
    assert g(FAKE, FAKE, -1, 10, 64, FAKE, 256, None) == SHAPE
    assert g(FAKE, FAKE, 3, 1 << 31, 64, FAKE, 256, None) == SHAPE
    assert g(None, FAKE, 3, 10, 64, FAKE, 256, None) == NULL
    assert g(FAKE, FAKE, 3, 10, 64, None, 256, None) == NULL
    assert g(FAKE + 16, FAKE, 3, 10, 64, FAKE, 256, None) == ALIGN
    assert g(FAKE, FAKE + 16, 3, 10, 64, FAKE, 256, None) == ALIGN
    assert g(FAKE, FAKE, 3, 10, 64, FAKE + 64, 256, None) == ALIGN
    assert g(FAKE, FAKE, 3, 10, 64, FAKE, 256, None) == SHAPE     # smaller than the split-K header
    assert g(None, None, 0, 0, 64, None, 0, None) == OK


def test_gemm_noalloc_scratch_limit(lib):
    """wq_gemm_noalloc refuses, before anything is launched, a call whose
    workspace (ceil256(2 M K) + ceil256(4 M) bytes) exceeds its 32 MiB scratch,
    and validates arguments like wq_gemm."""
    SCRATCH = 8
    f = lib.wq_gemm_noalloc
    assert f(FAKE, 4097, 4096, 64, 4, FAKE, FAKE, FAKE, None) == SCRATCH    # 2 * 4097 * 4096 > 32 MiB
    assert f(FAKE, 16384, 1024, 64, 4, FAKE, FAKE, FAKE, None) == SCRATCH   # exactly 32 MiB of x + the factors
    assert f(FAKE, 100, 1024, 64, 6, FAKE, FAKE, FAKE, None) == BITS
    assert f(None, 100, 1024, 64, 4, FAKE, FAKE, FAKE, None) == NULL
    assert f(MIS, 100, 1024, 64, 4, FAKE, FAKE, FAKE, None) == ALIGN
    assert f(None, 0, 1024, 64, 4, None, None, None, None) == OK
    assert lib.wq_strerror(SCRATCH).decode().startswith("workspace larger")


def test_strerror(lib):
    for s in range(9):
        assert lib.wq_strerror(s).decode()
    assert lib.wq_strerror(99).decode() == "unknown status"
