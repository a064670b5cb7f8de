"""ngq_gemm_splitk_static (no allocation: partial sums in the library's fixed
device array) against ngq_gemm_splitk (caller's workspace) through the C ABI.

Both run the same kernels with the same split, so the outputs must be equal
bit for bit; the first call is also checked against the oracle.  Two calls
in a row, the second smaller, show that the array's contents from one call
do not leak into the next (the split kernels write every partial sum they
read), and a captured graph of the call replays to the same bits.
"""
import numpy as np
import pytest

import synthetic
from tests.parity import assert_parity, compare
from tests.test_gpu_parity import ORACLE_THREADS, dev_bf16, dev_scales, dev_u8, host_bits

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ngq():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device visible")
    import groupwise_int_weight_amd as g

    g.lib()  # raises when the library is not built: no fallback exists
    return g


def abi_static(ngq, T, K, N, x, wq, sc, y):
    st = ngq.lib().ngq_gemm_splitk_static(T, K, N, 4, 64, x.data_ptr(), wq.data_ptr(), sc.data_ptr(),
                                          y.data_ptr(), torch.cuda.current_stream().cuda_stream)
    return st


def abi_workspace(ngq, T, K, N, x, wq, sc, y):
    ws = torch.empty(ngq.ngq_splitk_workspace_bytes(K, N, 4), dtype=torch.uint8, device="cuda")
    st = ngq.lib().ngq_gemm_splitk(T, K, N, 4, 64, x.data_ptr(), wq.data_ptr(), sc.data_ptr(), y.data_ptr(),
                                   ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
    return st


def inputs(T, N, seed):
    w = synthetic.WORKLOADS["down"]  # K = 17408: split into 8 slices at T >= 5
    codes, scales, x = synthetic.make_inputs(w, T, seed=seed, N=N)
    return w.K, codes, scales, x


def test_static_matches_workspace_twice_then_smaller(ngq):
    import oracle

    for T, N, seed in [(8, 5120, 0), (5, 2560, 1)]:
        K, codes, scales, x = inputs(T, N, seed)
        xd, wq, sc = dev_bf16(x), dev_u8(ngq.ngq_pack(codes, 4)), dev_scales(scales, False)
        y_static = torch.full((T, N), -3.0, dtype=torch.bfloat16, device="cuda")
        y_ws = torch.full((T, N), 5.0, dtype=torch.bfloat16, device="cuda")
        assert abi_static(ngq, T, K, N, xd, wq, sc, y_static) == 0
        assert abi_workspace(ngq, T, K, N, xd, wq, sc, y_ws) == 0
        a, b = host_bits(y_static), host_bits(y_ws)
        assert np.array_equal(a, b), (T, N)
        if seed == 0:
            y64, axw, axs = oracle.gemm(x, oracle.pack(codes, 4), scales, K, N, 4, False, nthreads=ORACLE_THREADS,
                                        with_bounds=True)
            assert_parity(compare(a, y64, axw, axs, K, 4), f"static T{T}")


def test_static_graph_replay(ngq):
    T, N = 8, 1024
    K, codes, scales, x = inputs(T, N, 2)
    xd, wq, sc = dev_bf16(x), dev_u8(ngq.ngq_pack(codes, 4)), dev_scales(scales, False)
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    assert abi_static(ngq, T, K, N, xd, wq, sc, y) == 0
    ref = host_bits(y)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        assert abi_static(ngq, T, K, N, xd, wq, sc, y) == 0
    other = torch.empty((8, 2048), dtype=torch.bfloat16, device="cuda")
    for rep in range(3):
        y.fill_(1.0)
        # eager work on the same array between replays
        assert abi_static(ngq, 8, K, 2048, dev_bf16(inputs(8, 2048, 3)[3]), dev_u8(np.zeros(
            ngq.ngq_packed_bytes(K, 2048, 4), np.uint8)), torch.zeros((K // 64, 2048), dtype=torch.float16,
                                                                      device="cuda"), other) == 0
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(y), ref), rep


def test_static_unsplit_shapes_run_as_gemm(ngq):
    """No split (T K small, or enough tiles): no scratch used, the result is
    ngq_gemm's."""
    for T, K, N in [(4, 17408, 512), (8, 4096, 64), (8, 5120, 8192)]:
        g = np.random.default_rng(T + K + N)
        codes = synthetic.draw_codes(K, N, 4, g)
        scales = synthetic.draw_scales(K, N, 1e-3, 2e-2, False, g)
        x = synthetic.draw_x(T, K, g)
        xd, wq, sc = dev_bf16(x), dev_u8(ngq.ngq_pack(codes, 4)), dev_scales(scales, False)
        y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
        assert abi_static(ngq, T, K, N, xd, wq, sc, y) == 0
        assert np.array_equal(host_bits(y), host_bits(ngq.ngq_gemm(xd, wq, sc, 4, N)))
