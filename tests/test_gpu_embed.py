"""GPU parity of the tied-embedding lookup (wq_embed) against the CPU oracle.

Every output is an exact dequantized weight (a binary16 scale times an integer
code is exact in fp32), so the comparison is bitwise, NaN rows included.
"""
import numpy as np
import pytest

import oracle
import weight_only_bit_block_amd as wqa
from weight_only_bit_block_amd import inputs
from tests.gpu_util import note, to_dev, to_host, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    t = torch_cuda()
    wqa.load()
    oracle.build(force=False)
    return t


def _same(a: np.ndarray, b: np.ndarray) -> bool:
    a = a.astype(np.float64)
    return a.shape == b.shape and bool(np.all((a == b) | (np.isnan(a) & np.isnan(b))))


def _table(N, K, bits, seed):
    w = inputs.normal((N, K), seed=seed, sigma=0.02)
    w[:, :32] *= np.float32(1e-6)             # tiny first block: binary16-subnormal scales
    if N > 2:
        w[1] = 0                              # a zero row
    return oracle.quantize(w, bits)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("N,K", [(1, 32), (37, 96), (1000, 1024), (300, 3072)])
def test_embed_parity(torch, bits, N, K):
    q, s = _table(N, K, bits, (50, N, K, bits))
    qd, sd = to_dev(q), to_dev(s)
    rng = inputs.generator((51, N, K, bits))
    for n in (1, 7, 128, 300):
        ids = rng.integers(0, N, n).astype(np.int32)
        ids[0] = N - 1
        if n > 4:
            ids[1], ids[2], ids[3] = -1, N, np.iinfo(np.int32).max   # outside the table: NaN rows
            ids[4] = ids[5 % n]                                       # a repeated id
        note(f"embed bits={bits} N={N} K={K} n={n}")
        out = to_host(wqa.embed(to_dev(ids), qd, sd, K, bits))
        assert _same(out, oracle.embed(ids, q, s, K, bits)), (bits, N, K, n)


def test_embed_empty(torch):
    q, s = _table(5, 64, 8, (52,))
    ids = torch.empty(0, dtype=torch.int32, device="cuda")
    out = wqa.embed(ids, to_dev(q), to_dev(s), 64, 8)
    assert tuple(out.shape) == (0, 64)


@pytest.mark.parametrize("n", [1, 128, 4096])
def test_embed_full_lm_head(torch, n):
    """The int8 lm_head table at its full size (151936 x 1024), random codes and
    scales; the looked-up rows are checked against the oracle on those rows."""
    N, K = 151936, 1024
    rng = inputs.generator((53, n))
    q = rng.integers(0, 256, (N, K), dtype=np.uint8)
    s = rng.integers(0x0001, 0x2C00, (N, K // 32), dtype=np.uint16)
    ids = rng.integers(0, N, n).astype(np.int32)
    ids[0] = N - 1
    if n > 1:
        ids[1] = 0
    note(f"embed full lm_head n={n}")
    out = to_host(wqa.embed(to_dev(ids), to_dev(q), to_dev(s), K, 8))
    ref = oracle.embed(np.arange(n), q[ids], s[ids], K, 8)
    assert _same(out, ref)
