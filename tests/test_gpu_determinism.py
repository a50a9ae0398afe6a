"""Run-to-run determinism: every entry point gives the same bits when the same
call is repeated (no atomics, fixed reduction orders), 12 times in a row, with
other work on the device in between."""
import numpy as np
import pytest

import oracle
import weight_only_bit_block_amd as wqa
from weight_only_bit_block_amd import inputs
from tests.gpu_util import note, to_dev, to_host, torch_cuda
from tests.test_gpu_kernels import _weights

pytestmark = pytest.mark.gpu

REPEATS = 12


@pytest.fixture(scope="module")
def torch():
    t = torch_cuda()
    wqa.load()
    oracle.build(force=False)
    return t


def _repeat(torch, fn, outs, what):
    """Call fn REPEATS times; after each call every output tensor equals the
    first call's bits. The outputs are NaN-filled before each call and a
    device-wide fill of another buffer runs in between."""
    other = torch.empty(1 << 22, dtype=torch.float32, device="cuda")
    first = None
    for r in range(REPEATS):
        for y in outs:
            y.fill_(float("nan"))
        other.fill_(float(r))
        fn()
        torch.cuda.synchronize()
        got = [to_host(y).copy() for y in outs]
        if first is None:
            first = got
            assert all(np.all(np.isfinite(g)) for g in got), what
        else:
            for a, b in zip(first, got):
                assert np.array_equal(a, b), f"{what}: repeat {r} differs"


@pytest.mark.parametrize("M", [1, 2, 4, 16])
def test_grouped_decode_repeats(torch, M):
    specs = [(4, 2048, 1024), (8, 1024, 1024), (5, 1024, 2048), (4, 3072, 1024), (8, 4000, 1024)]
    pkg = wqa.Package(specs)
    for i, (bits, N, K) in enumerate(specs):
        pkg.pack_into(i, to_dev(_weights(N, K, (100, i))))
    xs = [to_dev(inputs.normal((M, K), seed=(101, i, M))) for i, (_, _, K) in enumerate(specs)]
    ys = [torch.empty((M, N), dtype=torch.float32, device="cuda") for (_, N, _) in specs]
    call = wqa.GroupedCall(pkg, xs, ys, M)
    note(f"determinism grouped decode M={M}")
    _repeat(torch, call, ys, f"grouped decode M={M}")


@pytest.mark.parametrize("M", [17, 128, 1024])
def test_grouped_prefill_repeats(torch, M):
    specs = [(4, 2048, 1024), (8, 1024, 1024), (5, 1024, 2048), (4, 1024, 3072), (4, 300, 96)]
    pkg = wqa.Package(specs)
    for i, (bits, N, K) in enumerate(specs):
        pkg.pack_into(i, to_dev(_weights(N, K, (102, i))))
    xs = [to_dev(inputs.normal((M, K), seed=(103, i, M))) for i, (_, _, K) in enumerate(specs)]
    ys = [torch.empty((M, N), dtype=torch.float32, device="cuda") for (_, N, _) in specs]
    call = wqa.GroupedCall(pkg, xs, ys, M, prefill=True)
    note(f"determinism grouped prefill M={M}")
    _repeat(torch, call, ys, f"grouped prefill M={M}")


@pytest.mark.parametrize("M,K,N,bits", [(4096, 1024, 3072, 4), (2000, 3072, 1024, 4), (300, 1024, 2000, 8),
                                        (64, 1024, 40000, 8), (40, 2048, 40000, 4), (3, 1024, 5000, 5)])
def test_single_call_repeats(torch, M, K, N, bits):
    """wq_linear at prefill shapes (tile kernels of every shape class and the
    skinny kernel) and one decode shape."""
    w = _weights(N, K, (104, M, bits))
    q, s = wqa.pack(to_dev(w), bits)
    x = to_dev(inputs.normal((M, K), seed=(105, M, bits)))
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    note(f"determinism linear M={M} K={K} N={N} bits={bits}")
    _repeat(torch, lambda: wqa.linear(x, q, s, bits, out=y), [y], f"linear M={M} K={K} N={N}")
