"""ngq_gemm_splitk (K split over several workgroups per column tile) on the GPU.

The split applies where the 32-column tiles leave CUs idle and every slice
keeps 8 pairs (the down projection: 3 slices of 64-column tiles at any T).
Against the oracle on the down-projection shape and on ragged shapes (an odd
group count, so the last slice ends in half a pair; N not a multiple of the
64-column tile; every bit width and both scale types); bit for bit where the
partial sums are exact; run to run; and the shapes where no split applies,
which run as ngq_gemm.
"""
import numpy as np
import pytest

import synthetic
from tests.parity import assert_parity, compare
from tests.test_gpu_parity import ORACLE_THREADS, dev_bf16, dev_scales, dev_u8, host_bits, make

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


def run(ngq, orc, bits, sbf16, T, K, N, seed, cols=None):
    _, (codes, scales, x) = make(bits, sbf16, T, K, N, seed=seed)
    packed = ngq.ngq_pack(codes, bits)
    y = torch.full((T, N), -7.0, dtype=torch.bfloat16, device="cuda")
    ngq.ngq_gemm_splitk(dev_bf16(x), dev_u8(packed), dev_scales(scales, sbf16), bits, N, y=y)
    yb = host_bits(y)
    y64, axw, axs = orc.gemm(x, orc.pack(codes, bits), scales, K, N, bits, sbf16, cols=cols, nthreads=ORACLE_THREADS,
                             with_bounds=True)
    sub = yb if cols is None else yb[:, cols]
    assert_parity(compare(sub, y64, axw, axs, K, bits), f"splitk b{bits} T{T} K{K} N{N}")
    return yb


@pytest.mark.parametrize("bits,sbf16,T,K,N", [
    (4, False, 8, 12352, 100),   # 193 groups, 8 slices of 13 pairs: the last one ends in half a pair
    (5, True, 7, 16384, 36),     # 128 pairs: sixteen per slice
    (8, False, 5, 20480, 64),
    (4, True, 6, 12352, 260),    # 97 pairs, 5 tiles: 8 slices, a short last one
    (5, False, 7, 17408, 4),     # one narrow tile
    (4, False, 5, 17408, 5124),  # 81 tiles of 64 columns, the last one 4 wide: 3 slices
    (4, False, 1, 17408, 5120),  # T = 1
    (8, True, 2, 4096, 1000),    # 32 pairs: 4 slices; T = 2
    (5, True, 3, 2176, 192),     # 17 pairs: 2 slices, the second one pair short; T = 3
])
def test_splitk_small(ngq, orc, bits, sbf16, T, K, N):
    run(ngq, orc, bits, sbf16, T, K, N, seed=K + N + T)


@pytest.mark.parametrize("T", [5, 8, 1])
def test_splitk_down_shape(ngq, orc, T):
    w = synthetic.WORKLOADS["down"]
    codes, scales, x = synthetic.make_inputs(w, T, seed=0)
    packed = ngq.ngq_pack(codes, 4)
    xd, wd, sd = dev_bf16(x), dev_u8(packed), dev_scales(scales, False)
    y = host_bits(ngq.ngq_gemm_splitk(xd, wd, sd, 4, w.N))
    y64, axw, axs = orc.gemm(x, orc.pack(codes, 4), scales, w.K, w.N, 4, False, nthreads=ORACLE_THREADS,
                             with_bounds=True)
    assert_parity(compare(y, y64, axw, axs, w.K, 4), f"splitk down T{T}")
    # deterministic, and a captured graph replays to the same bits
    assert np.array_equal(y, host_bits(ngq.ngq_gemm_splitk(xd, wd, sd, 4, w.N)))
    ws = torch.empty(ngq.ngq_splitk_workspace_bytes(w.K, w.N, 4), dtype=torch.uint8, device="cuda")
    yg = torch.empty((T, w.N), dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ngq.ngq_gemm_splitk(xd, wd, sd, 4, w.N, y=yg, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ngq.ngq_gemm_splitk(xd, wd, sd, 4, w.N, y=yg, workspace=ws)
    for rep in range(3):
        yg.fill_(1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(yg), y), rep


@pytest.mark.parametrize("bits", [4, 5, 8])
def test_splitk_identity_scales_integer_x_bit_exact(ngq, orc, bits):
    """Scales 1 and small integer X: every slice sum and their total are
    integers below 2^24, exact in fp32 in any grouping."""
    T, K, N = 8, 12352, 96
    g = np.random.default_rng(70 + bits)
    lo, hi = synthetic.code_range(bits)
    codes = g.integers(lo, hi + 1, size=(K, N), dtype=np.int8)
    scales = np.full((K // 64, N), 0x3C00, np.uint16)
    x = synthetic.f32_to_bf16_bits(g.integers(-3, 4, size=(T, K)).astype(np.float32))
    y = ngq.ngq_gemm_splitk(dev_bf16(x), dev_u8(ngq.ngq_pack(codes, bits)), dev_scales(scales, False), bits, N)
    y64 = orc.gemm(x, orc.pack(codes, bits), scales, K, N, bits, False)
    assert np.array_equal(host_bits(y), orc.round_bf16_array(y64))


@pytest.mark.parametrize("T,K,N", [(4, 1024, 512), (8, 960, 64), (8, 10240, 8192), (1, 5120, 8192), (3, 0, 8)])
def test_splitk_without_a_split_runs_as_gemm(ngq, T, K, N):
    """Fewer than 16 pairs (no two slices of 8), tiles that fill the CUs, or
    K = 0: the call is ngq_gemm, bit for bit."""
    _, (codes, scales, x) = make(4, False, T, K, N, seed=5)
    packed = ngq.ngq_pack(codes, 4) if K else np.zeros(16, np.uint8)
    xd = dev_bf16(x) if K else torch.zeros((T, 0), dtype=torch.bfloat16, device="cuda")
    sd = dev_scales(scales, False) if K else torch.zeros((1, N), dtype=torch.float16, device="cuda")
    a = host_bits(ngq.ngq_gemm_splitk(xd, dev_u8(packed), sd, 4, N))
    b = host_bits(ngq.ngq_gemm(xd, dev_u8(packed), sd, 4, N))
    assert np.array_equal(a, b)
