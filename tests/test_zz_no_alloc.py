"""wq_gemm_noalloc (the prefill GEMM on the library's fixed per-device scratch)
against wq_gemm through the C ABI: two calls in a row, the second smaller, each
bitwise equal to wq_gemm's output and within the GEMM bound of the oracle."""
import numpy as np
import pytest

import oracle
import weight_only_bit_block_amd as wqa
from weight_only_bit_block_amd import inputs
from tests.gpu_util import check_gemm, note, to_dev, to_host, torch_cuda


@pytest.mark.gpu
@pytest.mark.parametrize("bits", [4, 8])
def test_gemm_noalloc_matches_gemm(bits):
    torch = torch_cuda()
    K, N = 1024, 3000
    w = inputs.normal((N, K), seed=(70, bits), sigma=0.02)
    q_ref, s_ref = oracle.quantize(w, bits)
    q, s = to_dev(q_ref), to_dev(s_ref)
    for M in (1000, 130):          # the second call is smaller and reuses the same scratch
        x = inputs.normal((M, K), seed=(71, bits, M))
        x[M // 3] *= 20
        xd = to_dev(x)
        y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        note(f"gemm_noalloc bits={bits} M={M} K={K} N={N}")
        wqa.gemm_noalloc(xd, q, s, bits, out=y)
        ref = wqa.gemm(xd, q, s, bits)
        torch.cuda.synchronize()
        got = to_host(y)
        assert np.array_equal(got, to_host(ref)), f"M={M}: differs from wq_gemm"
        y_ref, _ = oracle.matmul(x, q_ref, s_ref, bits)
        check_gemm(got, y_ref, f"gemm_noalloc bits={bits} M={M}")
