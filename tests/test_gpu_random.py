"""Seeded random shapes for the calls whose kernel choice depends on the
shape: ngq_multi_gemm (one workgroup per tile at any T, or the persistent
kernel when an int5 / int8 projection has the SwiGLU epilogue), and the
split-K family (ngq_gemm_splitk, ngq_gemm_rescale, ngq_gemm_residual_rescale,
whose slice count follows K and N).  Every output column is checked against
the oracle, with the same gates as the fixed cases; the draws are fixed by
the seeds, so a failure names a reproducible case.
"""
import numpy as np
import pytest

import synthetic
from tests.test_gpu_multi import run_case as multi_case
from tests.test_gpu_parity import make
from tests.test_gpu_splitk import run as splitk_case
from tests.test_gpu_stack import draw_residual, gemm_rescale_case, residual_case

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ngq():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device visible")
    import groupwise_int_weight_amd as g

    g.lib()  # raises when the library is not built: no fallback exists
    return g


@pytest.fixture(scope="module")
def orc():
    import oracle

    oracle.lib()
    return oracle


def multi_draw(seed):
    g = np.random.default_rng(seed)
    T = int(g.integers(1, 9))
    K = 64 * int(g.integers(1, 33))  # up to 2048: X fits the persistent kernel at every T
    specs = []
    for _ in range(int(g.integers(1, 5))):
        bits = int(g.choice([4, 5, 8]))
        swiglu = bool(g.random() < 0.35)
        n = 4 * int(g.integers(0, 150)) if g.random() < 0.9 else 0
        specs.append((bits, bool(g.random() < 0.5), n, swiglu))
    return T, K, specs


@pytest.mark.parametrize("seed", range(24))
def test_multi_random_shapes(ngq, orc, seed):
    T, K, specs = multi_draw(1000 + seed)
    multi_case(ngq, orc, T, K, specs, seed=seed)


def split_draw(seed):
    g = np.random.default_rng(seed)
    T = int(g.integers(1, 9))
    K = 64 * int(g.integers(1, 161))  # up to 10240
    N = 4 * int(g.integers(1, 600))
    bits = int(g.choice([4, 5, 8]))
    return bits, bool(g.random() < 0.5), T, K, N


@pytest.mark.parametrize("seed", range(16))
def test_splitk_random_shapes(ngq, orc, seed):
    bits, sbf16, T, K, N = split_draw(2000 + seed)
    splitk_case(ngq, orc, bits, sbf16, T, K, N, seed=seed)


@pytest.mark.parametrize("seed", range(12))
def test_rescale_and_residual_random_shapes(ngq, orc, seed):
    bits, sbf16, T, K, N = split_draw(3000 + seed)
    _, (codes, scales, x) = make(bits, sbf16, T, K, N, seed=seed)
    what = f"random b{bits} T{T} K{K} N{N}"
    gemm_rescale_case(ngq, orc, bits, sbf16, codes, scales, x, None, "gemm_rescale " + what)
    residual_case(ngq, orc, bits, sbf16, codes, scales, x, draw_residual(T, N, seed), "residual " + what)
