"""GPU tests of the error claims at the edges of the activation range.

The GEMM rounds each row of x to binary16 after a per-row power-of-two scaling
(largest magnitude into [2^14, 2^15)); the matrix-core GEMV (3 <= M <= 16)
splits each (row, block) of x into three binary16 parts after a per-block
power-of-two scaling. Both are exact up to the rounding they state, so every
check here is an elementwise bound derived from that rounding, against the
oracle's binary64 result on the same fp32 x:

  GEMM:  |y - y_exact| <= 2^-11 B + 2^-25 2^-e_m W + 1e-5 B
         (B = sum_k |x||w^|, W = sum_k |w^|, 2^-e_m the row's scaling: values
         whose scaled magnitude is at least 2^-14 keep 11 significant bits,
         smaller ones an absolute error of half the binary16 subnormal step)
  GEMV (M >= 3): |y - y_exact| <= 1e-5 B + sum_b (2^-39 max_b |x| + 2^-151) W_b
         (W_b = sum over block b of |w^|; the three-part split is exact for
         values within 2^16 of their block's largest)
"""
import numpy as np
import pytest

import oracle
import weight_only_bit_block_amd as wqa
from weight_only_bit_block_amd import inputs
from tests.gpu_util import check_gemm, note, to_dev, to_host, torch_cuda
from tests.test_gpu_kernels import _weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    t = torch_cuda()
    wqa.load()
    oracle.build(force=False)
    return t


def _row_scale(x: np.ndarray) -> np.ndarray:
    """2^-e_m of each row: the power of two that the row's largest magnitude
    is divided by to land in [2^14, 2^15) (e capped at 126; 1 for zero rows)."""
    amax = np.abs(x.astype(np.float64)).max(axis=1)
    out = np.ones(len(x))
    nz = amax > 0
    E = np.frexp(amax[nz])[1]                       # amax = f 2^E, f in [0.5, 1)
    e = np.minimum(15 - E, 126)
    out[nz] = np.ldexp(1.0, -e)
    return out


# (largest magnitude of the row, kind): near and above binary16's largest
# finite 65504, far above it, near fp32's largest (one such value in a row of
# small ones), tiny, at the 2^-112 boundary of the relative claim and below it,
# rows spread over 2^16 .. 2^40 inside the row, and a zero row
ROWS = [(1.0, "n"), (6.0e4, "n"), (65504.0, "n"), (7.0e4, "n"), (1.0e6, "n"), (1.0e30, "n"), (1.0e36, "n"),
        (3.0e38, "one"), (1.0e-20, "n"), (1.0e-30, "n"), (2.0 ** -100, "n"), (2.0 ** -112, "n"), (1.0e-36, "n"),
        (1.0, "spread16"), (1.0, "spread24"), (1.0, "spread40"), (0.0, "n")]


def _range_rows(K: int, seed) -> np.ndarray:
    rng = inputs.generator(seed)
    x = np.empty((len(ROWS), K), dtype=np.float64)
    for i, (f, kind) in enumerate(ROWS):
        r = rng.standard_normal(K)
        if kind.startswith("spread"):
            # one value of 1, the rest log-uniform over 2^-bits .. 1
            bits = int(kind[6:])
            r = np.sign(r) * 2.0 ** rng.uniform(-bits, 0, K)
            r[rng.integers(0, K)] = 1.0
            x[i] = r * f
        elif kind == "one":
            r = r * 1e-3
            r[rng.integers(0, K)] = 1.0
            x[i] = r * f
        else:
            x[i] = r / np.abs(r).max() * f
    return x.astype(np.float32)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("K,N", [(1024, 300), (3072, 300), (1024, 33000)])
def test_gemm_activation_range(torch, bits, K, N):
    """Rows of x at every scale of fp32 (above binary16's range, near fp32's
    largest, tiny, and spread over up to 2^40 inside a row) through the prefill
    GEMM (the tile kernel; N = 33000: the skinny kernel): each output within the
    bound derived from the per-row binary16 rounding, and the per-call
    Frobenius claim on the rows it covers."""
    w = _weights(N, K, (90, bits, K))
    q_ref, s_ref = oracle.quantize(w, bits)
    x = _range_rows(K, (91, bits, K))
    M = len(x)
    cols = np.arange(N)
    if N > 300:
        cols = np.unique(np.concatenate([inputs.generator((96, bits)).choice(N, 400, replace=False), [N - 1]]))
    y_ref, B = oracle.matmul(x, q_ref[cols], s_ref[cols], bits)
    wh = oracle.dequant(q_ref[cols], s_ref[cols], K, bits)
    W = np.abs(wh).sum(axis=1)
    note(f"gemm activation range bits={bits} K={K} N={N} M={M}")
    y = to_host(wqa.gemm(to_dev(x), to_dev(q_ref), to_dev(s_ref), bits)).astype(np.float64)[:, cols]
    assert np.all(np.isfinite(y)) and np.all(np.abs(y_ref) < 1e38)
    bound = 2.0 ** -11 * B + 2.0 ** -25 * _row_scale(x)[:, None] * W[None, :] + 1e-5 * B
    err = np.abs(y - y_ref)
    worst = float(np.max(err / np.maximum(bound, 1e-300)))
    print(f"[info] gemm range bits={bits} K={K} N={N}: worst err/bound {worst:.3f}", flush=True)
    assert np.all(err <= bound), worst
    cover = np.abs(x).max(axis=1) >= 2.0 ** -112
    check_gemm(y[cover], y_ref[cover], f"gemm range bits={bits} K={K} N={N}")


@pytest.mark.parametrize("bits", [4, 8])
def test_gemm_nonfinite_rows_stay_in_their_rows(torch, bits):
    """A row holding inf or NaN gives non-finite outputs in that row only; every
    other row is bitwise what it is with that row set to zero (rows are scaled
    and rounded independently)."""
    K, N, M = 1024, 200, 40
    w = _weights(N, K, (92, bits))
    q_ref, s_ref = oracle.quantize(w, bits)
    q, s = to_dev(q_ref), to_dev(s_ref)
    x = inputs.normal((M, K), seed=(93, bits))
    x[7, 100] = np.inf
    x[20, 5] = np.nan
    x[21, 999] = -np.inf
    clean = x.copy()
    clean[[7, 20, 21]] = 0
    note(f"gemm non-finite rows bits={bits}")
    y = to_host(wqa.gemm(to_dev(x), q, s, bits))
    yc = to_host(wqa.gemm(to_dev(clean), q, s, bits))
    bad = [7, 20, 21]
    assert not np.isfinite(y[bad]).any(), "every output of a row with inf or NaN is non-finite"
    good = np.setdiff1d(np.arange(M), bad)
    assert np.array_equal(y[good], yc[good])


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("M", [3, 8, 16])
def test_gemv_mfma_block_range(torch, bits, M):
    """Matrix-core decode (3 <= M <= 16) with x blocks spread over 2^8, 2^16,
    2^24 and 2^40 around one value of 1 whose weight code is 0, so that the
    result is made of the small values alone: every output within the bound of
    the three-part split, and within the plain 1e-5 * sum|x||w^| bound where
    the split is exact (spreads up to 2^16)."""
    K, N = 1024, 300
    w = _weights(N, K, (94, bits, M))
    nb = K // 32
    spreads = [8, 16, 24, 40]
    rng = inputs.generator((95, bits, M))
    x = np.empty((M, K), dtype=np.float32)
    outl = rng.integers(0, 32, nb)                    # outlier position of each block
    for b in range(nb):
        sp = spreads[b % 4]
        v = np.sign(rng.standard_normal((M, 32))) * 2.0 ** rng.uniform(-sp, -sp + 1, (M, 32))
        v[:, outl[b]] = 1.0
        x[:, 32 * b: 32 * b + 32] = v
        w[:, 32 * b + outl[b]] = 0.0                  # code 0 at the outlier
    q_ref, s_ref = oracle.quantize(w, bits)
    wh = oracle.dequant(q_ref, s_ref, K, bits)
    assert np.all(wh[:, 32 * np.arange(nb) + outl] == 0)
    y_ref, B = oracle.matmul(x, q_ref, s_ref, bits)
    Wb = np.abs(wh).reshape(N, nb, 32).sum(axis=2)            # [N, nb]
    Eb = 2.0 ** -39 * np.abs(x.astype(np.float64)).reshape(M, nb, 32).max(axis=2) + 2.0 ** -151
    bound = 1e-5 * B + Eb @ Wb.T
    note(f"mgemv block range bits={bits} M={M}")
    y = to_host(wqa.gemv(to_dev(x), to_dev(q_ref), to_dev(s_ref), bits)).astype(np.float64)
    err = np.abs(y - y_ref)
    assert np.all(np.isfinite(y))
    assert np.all(err <= bound), float((err / bound).max())
    # where every block's spread is within 2^16, the plain bound holds too
    exact_blocks = np.array([spreads[b % 4] <= 16 for b in range(nb)])
    cols = np.repeat(exact_blocks, 32)
    xe = x * cols[None, :]
    y_e, B_e = oracle.matmul(xe, q_ref, s_ref, bits)
    ye = to_host(wqa.gemv(to_dev(xe), to_dev(q_ref), to_dev(s_ref), bits)).astype(np.float64)
    assert np.all(np.abs(ye - y_e) <= 1e-5 * B_e)
    plain = float((err / np.maximum(1e-5 * B, 1e-300)).max())
    print(f"[info] mgemv range bits={bits} M={M}: worst err / (1e-5 sum|x||w|) with 2^24 and 2^40 spreads = "
          f"{plain:.3f}", flush=True)
