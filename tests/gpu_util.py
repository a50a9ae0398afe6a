"""Helpers shared by the GPU parity tests: device transfer and the acceptance
rules. The expected values always come from the CPU oracle."""
import sys

import numpy as np
import pytest

GEMV_RTOL = 1e-5        # |y - y_ref| <= 1e-5 * sum_k |x||w^|, per output
GEMM_FROB = 2e-3        # ||Y - Y_ref||_F <= 2e-3 ||Y_ref||_F, per call


def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def note(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a fault can be attributed."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray):
    torch = torch_cuda()
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def scales_u16(t) -> np.ndarray:
    return to_host(t).view(np.uint16)


def check_gemv(y: np.ndarray, y_ref: np.ndarray, B: np.ndarray, what: str = "") -> float:
    """Elementwise bound; returns the worst error / bound ratio."""
    y = y.astype(np.float64)
    err = np.abs(y - y_ref)
    zero = B == 0
    assert np.all(y[zero] == 0), f"{what}: non-zero output where every product is zero"
    bound = GEMV_RTOL * B
    ratio = np.where(zero, 0.0, err / np.where(zero, 1.0, bound))
    worst = float(ratio.max()) if ratio.size else 0.0
    assert np.all(err <= bound), f"{what}: max err/bound = {worst:.3f}"
    assert np.all(np.isfinite(y)), what
    return worst


def check_gemm(y: np.ndarray, y_ref: np.ndarray, what: str = "") -> float:
    y = y.astype(np.float64)
    assert np.all(np.isfinite(y)), what
    den = float(np.linalg.norm(y_ref))
    num = float(np.linalg.norm(y - y_ref))
    if den == 0:
        assert np.all(y == 0), what
        return 0.0
    rel = num / den
    assert rel <= GEMM_FROB, f"{what}: relative Frobenius error {rel:.3e}"
    return rel
