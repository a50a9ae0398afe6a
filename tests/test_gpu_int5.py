"""GPU parity of the int5 path (pack, unpack, GEMV, GEMM, grouped decode and the
embedding lookup) against the CPU oracle.

int5 rows are the low-nibble plane (as int4) then the bit-4 plane; every
expected value comes from the oracle, and hand-packed rows go through the
oracle's decoder as well as the kernels.
"""
import numpy as np
import pytest

import oracle
import weight_only_bit_block_amd as wqa
from weight_only_bit_block_amd import inputs
from tests.gpu_util import check_gemm, check_gemv, note, scales_u16, to_dev, to_host, torch_cuda
from tests.test_gpu_kernels import _crafted, _weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    t = torch_cuda()
    wqa.load()
    oracle.build(force=False)
    return t


def pack5(codes: np.ndarray) -> np.ndarray:
    """int codes [N, K] in [-16, 15] -> int5 rows [N, 5K/8] (test-side packer)."""
    f = codes.astype(np.int64) & 31
    nib = f & 15
    lo = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    hb = ((f >> 4) & 1).reshape(codes.shape[0], -1, 8)
    hi = (hb << np.arange(8)).sum(axis=2).astype(np.uint8)
    return np.concatenate([lo, hi], axis=1)


@pytest.mark.parametrize("N,K", [(1, 128), (3, 256), (257, 1024), (64, 3072)])
def test_pack_unpack_int5(torch, N, K):
    for kind, w in [("normal", _weights(N, K, (60, N, K))), ("crafted", _crafted(N, K, 5, (61, N, K)))]:
        note(f"pack int5 {kind} N={N} K={K}")
        q_ref, s_ref = oracle.quantize(w, 5)
        q, s = wqa.pack(to_dev(w), 5)
        torch.cuda.synchronize()
        assert np.array_equal(to_host(q), q_ref), kind
        assert np.array_equal(scales_u16(s), s_ref), kind
        assert np.array_equal(to_host(wqa.unpack(q, K, 5)), oracle.decode(q_ref, K, 5)), kind


def test_unpack_every_field_int5(torch):
    """All 32 five-bit fields at every position of a block, -16 and -1 included."""
    codes = np.array([[((k + sh) % 32) - 16 for k in range(128)] for sh in range(32)])
    q = pack5(codes)
    assert np.array_equal(oracle.decode(q, 128, 5), codes)
    note("unpack int5 fields")
    assert np.array_equal(to_host(wqa.unpack(to_dev(q), 128, 5)), codes)


@pytest.mark.parametrize("K,N", [(128, 1), (256, 33), (384, 300), (1024, 2048), (2048, 1024), (3072, 1024),
                                 (4096, 129)])
def test_gemv_parity_int5(torch, K, N):
    w = _weights(N, K, (62, K, N))
    q_ref, s_ref = oracle.quantize(w, 5)
    q, s = to_dev(q_ref), to_dev(s_ref)
    for M in (1, 2, 3, 4, 5, 16):
        x = inputs.normal((M, K), seed=(63, K, N, M))
        if M > 2:
            x[1] *= 20
        y_ref, B = oracle.matmul(x, q_ref, s_ref, 5)
        note(f"gemv int5 M={M} K={K} N={N}")
        y = to_host(wqa.gemv(to_dev(x), q, s, 5))
        check_gemv(y, y_ref, B, f"gemv int5 M={M} K={K} N={N}")


def test_gemv_one_hot_extremes_int5(torch):
    """x = e_k reads out w^ bitwise (crafted weights, subnormal scales); codes
    -16..15 with zero scales; sign symmetry and power-of-two homogeneity bitwise."""
    K, N = 256, 70
    w = _crafted(N, K, 5, (64,))
    q_ref, s_ref = oracle.quantize(w, 5)
    wh = oracle.dequant(q_ref, s_ref, K, 5)
    q, s = to_dev(q_ref), to_dev(s_ref)
    eye = np.eye(K, dtype=np.float32)
    for m0 in range(0, K, 16):
        note(f"gemv int5 one-hot rows {m0}..")
        y = to_host(wqa.gemv(to_dev(eye[m0:m0 + 16]), q, s, 5))
        assert np.array_equal(y.astype(np.float64), wh[:, m0:m0 + 16].T)
    rng = inputs.generator((65,))
    codes = rng.integers(-16, 16, (96, 1024))
    codes[0::3] = -16
    q2 = pack5(codes)
    s2 = np.float16(rng.uniform(1e-3, 2e-2, (96, 32))).view(np.uint16)
    s2[5] = 0
    x = inputs.normal((4, 1024), seed=(66,))
    y_ref, B = oracle.matmul(x, q2, s2, 5)
    note("gemv int5 extremes")
    y = to_host(wqa.gemv(to_dev(x), to_dev(q2), to_dev(s2), 5))
    check_gemv(y, y_ref, B, "int5 extremes")
    assert np.all(y[:, 5] == 0)
    yn = to_host(wqa.gemv(to_dev(-x), to_dev(q2), to_dev(s2), 5))
    y8 = to_host(wqa.gemv(to_dev(x * np.float32(8.0)), to_dev(q2), to_dev(s2), 5))
    assert np.array_equal(yn, -y) and np.array_equal(y8, y * np.float32(8.0))


@pytest.mark.parametrize("K,N", [(128, 5), (256, 130), (1024, 256), (3072, 384), (2048, 257)])
def test_gemm_parity_int5(torch, K, N):
    w = _weights(N, K, (67, K, N))
    q_ref, s_ref = oracle.quantize(w, 5)
    q, s = to_dev(q_ref), to_dev(s_ref)
    for M in (1, 17, 64, 128, 130, 300):
        x = inputs.normal((M, K), seed=(68, K, N, M))
        x[M // 2] *= 20
        y_ref, _ = oracle.matmul(x, q_ref, s_ref, 5)
        y16, B16 = oracle.matmul(x, q_ref, s_ref, 5, x16=True)
        note(f"gemm int5 M={M} K={K} N={N}")
        y = to_host(wqa.gemm(to_dev(x), q, s, 5))
        check_gemm(y, y_ref, f"gemm int5 M={M} K={K} N={N}")
        check_gemv(y, y16, B16, f"gemm-vs-x16 int5 M={M} K={K} N={N}")
        for m in range(M):
            den = np.linalg.norm(y_ref[m])
            if den > 0:
                assert np.linalg.norm(y[m] - y_ref[m]) <= 2e-3 * den, m


def test_gemm_int5_long_prefill_shape(torch):
    """A long int5 prefill (at least 2 C tiles of 128 x 128, K = 1024: the shape
    that takes two workgroups per compute unit with three stages), with ragged M
    and N, on sampled columns against the oracle and against the binary16-x
    diagnostic reference elementwise."""
    M, K, N = 2100, 1024, 4000
    cols = np.sort(inputs.generator((71, 1)).choice(N, size=96, replace=False))
    w = _weights(N, K, (70, K, N))
    x = inputs.normal((M, K), seed=(72, K, N))
    x[::97] *= 20
    q_ref, s_ref = oracle.quantize(w, 5)
    qs, ss = oracle.quantize(w[cols], 5)
    y_ref, _ = oracle.matmul(x, qs, ss, 5)
    y16, B16 = oracle.matmul(x, qs, ss, 5, x16=True)
    note(f"gemm int5 long prefill M={M} K={K} N={N}")
    y = to_host(wqa.gemm(to_dev(x), to_dev(q_ref), to_dev(s_ref), 5))[:, cols]
    check_gemm(y, y_ref, "gemm int5 long prefill")
    check_gemv(y, y16, B16, "gemm int5 long prefill vs x16")


def test_gemm_one_hot_selection_int5(torch):
    K, N = 256, 150
    w = _crafted(N, K, 5, (69,))
    q_ref, s_ref = oracle.quantize(w, 5)
    wh = oracle.dequant(q_ref, s_ref, K, 5)
    note("gemm int5 one-hot")
    y = to_host(wqa.gemm(to_dev(np.eye(K, dtype=np.float32)), to_dev(q_ref), to_dev(s_ref), 5))
    assert np.array_equal(y.astype(np.float64), wh.T)
    K2, N2, M2 = 1024, 300, 200
    rng = inputs.generator((70,))
    pi = rng.integers(0, K2, N2)
    codes = np.zeros((N2, K2), dtype=np.int64)
    codes[np.arange(N2), pi] = -16                        # the one code with bit 4 set and nibble 0
    q2 = pack5(codes)
    s2 = np.full((N2, K2 // 32), 0x2C00, dtype=np.uint16)  # 1/16: code * scale = -1
    x2 = rng.integers(-1000, 1000, (M2, K2)).astype(np.float32)
    note("gemm int5 selection")
    y2 = to_host(wqa.gemm(to_dev(x2), to_dev(q2), to_dev(s2), 5))
    assert np.array_equal(y2, -x2[:, pi])


@pytest.mark.parametrize("M", [1, 4, 16])
def test_grouped_mixed_int4_int5_int8(torch, M):
    specs = [(5, 2048, 1024), (4, 1024, 1024), (5, 1024, 3072), (8, 1000, 1024), (5, 77, 128), (5, 0, 256)]
    pkg = wqa.Package(specs)
    refs = []
    for i, (bits, N, K) in enumerate(specs):
        q_ref, s_ref = oracle.quantize(_weights(N, K, (71, i)), bits)
        pkg.q(i).copy_(to_dev(q_ref))
        pkg.scales(i).copy_(to_dev(s_ref))
        refs.append((q_ref, s_ref))
    xs = [to_dev(inputs.normal((M, K), seed=(72, i, M))) for i, (_, _, K) in enumerate(specs)]
    ys = [torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda") for (_, N, _) in specs]
    call = wqa.GroupedCall(pkg, xs, ys, M)
    note(f"grouped int4/int5/int8 M={M}")
    call()
    torch.cuda.synchronize()
    for i, (bits, N, K) in enumerate(specs):
        got = to_host(ys[i])
        assert np.array_equal(got, to_host(wqa.gemv(xs[i], pkg.q(i), pkg.scales(i), bits))), i
        y_ref, B = oracle.matmul(to_host(xs[i]), refs[i][0], refs[i][1], bits)
        check_gemv(got, y_ref, B, f"grouped int5 mix tensor {i}")


def test_embed_int5(torch):
    N, K = 1000, 1024
    q_ref, s_ref = oracle.quantize(_weights(N, K, (73,)), 5)
    ids = inputs.generator((74,)).integers(0, N, 300).astype(np.int32)
    ids[1], ids[2] = -1, N
    note("embed int5")
    out = to_host(wqa.embed(to_dev(ids), to_dev(q_ref), to_dev(s_ref), K, 5)).astype(np.float64)
    ref = oracle.embed(ids, q_ref, s_ref, K, 5)
    assert np.all((out == ref) | (np.isnan(out) & np.isnan(ref)))
