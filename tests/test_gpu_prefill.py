"""ngq_gemm and ngq_swiglu_gemm with prefill-size T (token x column tiles,
K split over the waves, or the X tile shared by waves that split the columns)
on the GPU, against the CPU oracle.

Small ragged shapes (a token tail past every 64-token tile, a column tail,
odd group counts, every bit width and both scale types) for both variants,
the K-split kernel forced at decode and verify T (its 16-, 32- and 64-column
tiles), the full-size projections at T = 40 to 2048 on sampled columns, bit-exact cases, guard bands, K = 0, determinism and
graph replay.
"""
import numpy as np
import pytest

import synthetic
from tests.parity import bf16_bits_to_f64
from tests.test_gpu_parity import (check_swiglu, dev_bf16, dev_scales, dev_u8, host_bits, make, run_and_compare,
                                   sample_cols, swiglu_reference)

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


@pytest.fixture
def forced_tiled(ngq):
    prev = ngq.ngq_debug_force_kernel(ngq.NGQ_KERNEL_TILED)
    yield
    ngq.ngq_debug_force_kernel(prev)


@pytest.fixture
def forced_sx(ngq):
    prev = ngq.ngq_debug_force_kernel(ngq.NGQ_KERNEL_TILED_SX)
    yield
    ngq.ngq_debug_force_kernel(prev)


SMALL = [
    # bits, scale_bf16, T, K, N
    (4, False, 65, 320, 100),    # one past the verify range; 5 groups; column tail
    (5, True, 128, 1024, 520),   # two full token tiles
    (8, False, 129, 512, 300),   # one token past a tile
    (4, True, 200, 192, 36),     # 3 groups, one narrow tile
    (5, False, 96, 640, 68),
    (8, True, 70, 256, 4),       # a 4-column matrix
    (4, False, 300, 2048, 4100),
    (5, True, 77, 64, 40),       # a single group (waves 1..3 have none)
    (8, False, 150, 1088, 132),  # 17 groups
    # on 256 CUs the K-split kernel runs 16-column tiles for most shapes
    # above and 32-column ones for these two (66 tiles of 64 columns would
    # leave CUs idle, 264 of 16 two rounds); column tails of 20
    (5, True, 65, 320, 2100),
    (8, False, 100, 256, 2100),
]


@pytest.mark.parametrize("bits,sbf16,T,K,N", SMALL)
def test_prefill_small(ngq, orc, bits, sbf16, T, K, N):
    _, (codes, scales, x) = make(bits, sbf16, T, K, N, seed=T * 7 + K + N)
    run_and_compare(ngq, orc, bits, sbf16, codes, scales, x, what=f"prefill b{bits} T{T} K{K} N{N}")


@pytest.mark.parametrize("T", [1, 5, 8, 9, 16, 33, 64])
@pytest.mark.parametrize("bits,sbf16", [(4, False), (5, True), (8, False)])
def test_tiled_kernel_at_small_t(ngq, orc, forced_tiled, bits, sbf16, T):
    """The token x column kernel serves any T when forced (decode and verify
    sizes route elsewhere by default)."""
    _, (codes, scales, x) = make(bits, sbf16, T, 704, 196, seed=T + 3 * bits)
    run_and_compare(ngq, orc, bits, sbf16, codes, scales, x, what=f"tiled forced b{bits} T{T}")


@pytest.mark.parametrize("bits,sbf16,T,K,N", SMALL + [(4, False, 1, 320, 1000), (5, True, 8, 576, 264)])
def test_shared_x_kernel_small(ngq, orc, forced_sx, bits, sbf16, T, K, N):
    """The variant whose waves split the columns and share each X tile
    (large T routes to it) on the same ragged shapes, forced."""
    _, (codes, scales, x) = make(bits, sbf16, T, K, N, seed=T * 7 + K + N + 1)
    run_and_compare(ngq, orc, bits, sbf16, codes, scales, x, what=f"sx forced b{bits} T{T} K{K} N{N}")


INT4_SHAPES = [(sbf16, T, K, N) for bits, sbf16, T, K, N in SMALL if bits == 4] + \
    [(False, 1, 320, 1000), (True, 97, 576, 264), (False, 250, 1088, 516), (True, 129, 64, 4)]


@pytest.mark.parametrize("path_name", ["NGQ_KERNEL_TILED_SX96", "NGQ_KERNEL_TILED_SX128"])
@pytest.mark.parametrize("sbf16,T,K,N", INT4_SHAPES)
def test_shared_x_larger_token_tiles(ngq, orc, path_name, sbf16, T, K, N):
    """The shared-X kernel with 96- and 128-token tiles (int4), forced, on
    ragged shapes: token tails past a tile, column tails, odd group counts."""
    _, (codes, scales, x) = make(4, sbf16, T, K, N, seed=T * 5 + K + N)
    prev = ngq.ngq_debug_force_kernel(getattr(ngq, path_name))
    try:
        run_and_compare(ngq, orc, 4, sbf16, codes, scales, x, what=f"{path_name} T{T} K{K} N{N}")
    finally:
        ngq.ngq_debug_force_kernel(prev)


@pytest.mark.parametrize("path_name", ["NGQ_KERNEL_TILED_SX96", "NGQ_KERNEL_TILED_SX128"])
def test_shared_x_larger_token_tiles_swiglu(ngq, orc, path_name):
    T, K, N_ff = 200, 512, 100
    _, (codes, scales, x) = make(4, False, T, K, 2 * N_ff, seed=41)
    prev = ngq.ngq_debug_force_kernel(getattr(ngq, path_name))
    try:
        h = ngq.ngq_swiglu_gemm(dev_bf16(x), dev_u8(ngq.ngq_pack(codes, 4)), dev_scales(scales, False), 4, N_ff)
    finally:
        ngq.ngq_debug_force_kernel(prev)
    cols = np.arange(N_ff, dtype=np.int32)
    h64, g, u = swiglu_reference(orc, x, orc.pack(codes, 4), scales, K, N_ff, 4, False, cols)
    check_swiglu(host_bits(h), h64, g, u, f"{path_name} swiglu")


def test_larger_token_tiles_refuse_int5(ngq):
    x = torch.zeros((128, 64), dtype=torch.bfloat16, device="cuda")
    wq = torch.zeros(ngq.ngq_packed_bytes(64, 8, 5), dtype=torch.uint8, device="cuda")
    sc = torch.zeros((1, 8), dtype=torch.float16, device="cuda")
    y = torch.zeros((128, 8), dtype=torch.bfloat16, device="cuda")
    prev = ngq.ngq_debug_force_kernel(ngq.NGQ_KERNEL_TILED_SX128)
    try:
        st = ngq.lib().ngq_gemm(128, 64, 8, 5, 64, x.data_ptr(), wq.data_ptr(), sc.data_ptr(), y.data_ptr(),
                                torch.cuda.current_stream().cuda_stream)
    finally:
        ngq.ngq_debug_force_kernel(prev)
    assert st == ngq.NGQ_ERR_UNSUPPORTED


@pytest.mark.parametrize("bits,sbf16,T,K,N_ff", [(4, False, 65, 512, 100), (5, True, 130, 320, 36),
                                                  (8, False, 70, 256, 200)])
def test_shared_x_kernel_swiglu(ngq, orc, forced_sx, bits, sbf16, T, K, N_ff):
    _, (codes, scales, x) = make(bits, sbf16, T, K, 2 * N_ff, seed=K + N_ff + T + 1)
    packed = ngq.ngq_pack(codes, bits)
    h = ngq.ngq_swiglu_gemm(dev_bf16(x), dev_u8(packed), dev_scales(scales, sbf16), bits, N_ff)
    cols = np.arange(N_ff, dtype=np.int32)
    h64, g, u = swiglu_reference(orc, x, orc.pack(codes, bits), scales, K, N_ff, bits, sbf16, cols)
    check_swiglu(host_bits(h), h64, g, u, f"sx swiglu b{bits} T{T}")


@pytest.mark.parametrize("T,N", [(700, 1000), (1090, 520)])
def test_shared_x_bands_with_partial_last_band(ngq, orc, forced_sx, T, N):
    """Token tiles walked in bands of 4: 11 and 18 token tiles leave a last
    band of 3 and 2, next to a partial last column tile."""
    _, (codes, scales, x) = make(4, False, T, 256, N, seed=T + N)
    run_and_compare(ngq, orc, 4, False, codes, scales, x, what=f"sx bands T{T} N{N}")


def test_maximum_token_count(ngq, orc):
    """T = NGQ_MAX_T_PREFILL, the largest T the call takes (256 token tiles)."""
    T = ngq.NGQ_MAX_T_PREFILL
    _, (codes, scales, x) = make(5, True, T, 192, 36, seed=11)
    run_and_compare(ngq, orc, 5, True, codes, scales, x, what=f"max T{T}")


_FULL = {}


def full_inputs(name, T):
    key = (name, T)
    if key not in _FULL:
        w = synthetic.WORKLOADS[name]
        _FULL.clear()
        _FULL[key] = (w,) + tuple(synthetic.make_inputs(w, T, seed=2))
    return _FULL[key]


# qk at T = 1024 runs the shared-X variant with 64-token tiles, qk at 2048
# with 128, down at 2048 with 96, the others the K-split one (qk at 64 and
# down at 40 on 32-column tiles, the rest on 64)
@pytest.mark.parametrize("name,T", [("qk", 1024), ("gv", 256), ("qk8", 130), ("down", 256), ("qk", 2048),
                                    ("down", 2048), ("qk", 64), ("down", 40)])
def test_prefill_full_size(ngq, orc, name, T):
    w, codes, scales, x = full_inputs(name, T)
    cols = sample_cols(w.N, seed=T + 11, n_random=96)
    yb, _ = run_and_compare(ngq, orc, w.bits, w.scale_bf16, codes, scales, x, cols=cols,
                            what=f"prefill {name} T{T}")
    assert np.all(np.isfinite(bf16_bits_to_f64(yb)))


@pytest.mark.parametrize("bits,sbf16,T,K,N_ff", [(4, False, 65, 512, 100), (5, True, 130, 320, 36),
                                                  (8, False, 200, 256, 64), (4, True, 100, 1024, 260)])
def test_prefill_swiglu_small(ngq, orc, bits, sbf16, T, K, N_ff):
    _, (codes, scales, x) = make(bits, sbf16, T, K, 2 * N_ff, seed=K + N_ff + T)
    packed = ngq.ngq_pack(codes, bits)
    h = ngq.ngq_swiglu_gemm(dev_bf16(x), dev_u8(packed), dev_scales(scales, sbf16), bits, N_ff)
    cols = np.arange(N_ff, dtype=np.int32)
    h64, g, u = swiglu_reference(orc, x, orc.pack(codes, bits), scales, K, N_ff, bits, sbf16, cols)
    check_swiglu(host_bits(h), h64, g, u, f"prefill swiglu b{bits} T{T}")


def test_prefill_swiglu_full_size(ngq, orc):
    T = 256
    w, codes, scales, x = full_inputs("gate_up", T)
    N_ff = synthetic.N_FF
    packed = ngq.ngq_pack(codes, 4)
    h = ngq.ngq_swiglu_gemm(dev_bf16(x), dev_u8(packed), dev_scales(scales, False), 4, N_ff)
    cols = sample_cols(N_ff, seed=5, n_random=64)
    h64, g, u = swiglu_reference(orc, x, orc.pack(codes, 4), scales, w.K, N_ff, 4, False, cols)
    check_swiglu(host_bits(h)[:, cols], h64, g, u, "prefill swiglu gate_up T256")


@pytest.mark.parametrize("bits", [4, 5, 8])
def test_prefill_identity_scales_integer_x_bit_exact(ngq, orc, bits):
    """s = 1 and integer x: every partial sum is an integer below 2^24, so the
    fp32 result is exact and its bf16 rounding must equal the oracle's."""
    g = np.random.default_rng(240 + bits)
    T, K, N = 160, 576, 132
    codes = synthetic.draw_codes(K, N, bits, g)
    scales = np.full((K // 64, N), 0x3C00, np.uint16)
    xi = g.integers(-2, 3, size=(T, K))
    x = synthetic.f32_to_bf16_bits(xi.astype(np.float32))
    y = ngq.ngq_gemm(dev_bf16(x), dev_u8(ngq.ngq_pack(codes, bits)), dev_scales(scales, False), bits, N)
    exact = xi.astype(np.int64) @ codes.astype(np.int64)
    assert np.array_equal(host_bits(y), orc.round_bf16_array(exact.astype(np.float64)))


def test_prefill_one_hot_rows_bit_exact(ngq, orc):
    """One-hot x rows (k = row index + offset) with power-of-two scales read
    single weights back exactly: token t's output row is codes[k_t] s[k_t]."""
    K, N, T = 320, 72, 192
    g = np.random.default_rng(177)
    codes = synthetic.draw_codes(K, N, 5, g)
    exps = g.integers(-9, -3, size=(K // 64, N))
    scales = synthetic.f32_to_bf16_bits((2.0 ** exps).astype(np.float32))
    wq, sd = dev_u8(ngq.ngq_pack(codes, 5)), dev_scales(scales, True)
    for start in (0, 100):
        ks = (start + np.arange(T)) % K
        x = np.zeros((T, K), np.float32)
        x[np.arange(T), ks] = 1.0
        y = ngq.ngq_gemm(dev_bf16(synthetic.f32_to_bf16_bits(x)), wq, sd, 5, N)
        expect = codes[ks, :].astype(np.float64) * (2.0 ** exps[ks // 64, :])
        assert np.array_equal(host_bits(y), orc.round_bf16_array(expect)), start


def test_prefill_guard_bands_and_determinism(ngq, orc):
    T, K, N = 130, 320, 100
    _, (codes, scales, x) = make(4, False, T, K, N, seed=31)
    pad = 4096
    buf = torch.full((pad + T * N + pad,), 0x7E7E, dtype=torch.int16, device="cuda")
    y = buf[pad:pad + T * N].view(torch.bfloat16).view(T, N)
    args = (dev_bf16(x), dev_u8(ngq.ngq_pack(codes, 4)), dev_scales(scales, False), 4, N)
    ngq.ngq_gemm(*args, y=y)
    hb = host_bits(buf)
    assert np.all(hb[:pad] == 0x7E7E) and np.all(hb[pad + T * N:] == 0x7E7E)
    for _ in range(3):
        assert np.array_equal(host_bits(ngq.ngq_gemm(*args)), hb[pad:pad + T * N].reshape(T, N))


def test_prefill_k_zero_writes_zeros(ngq):
    T, N = 100, 8
    y = torch.full((T, N), 7.0, dtype=torch.bfloat16, device="cuda")
    wq = torch.zeros(16, dtype=torch.uint8, device="cuda")
    sc = torch.zeros((1, N), dtype=torch.float16, device="cuda")
    st = ngq.lib().ngq_gemm(T, 0, N, 4, 64, wq.data_ptr(), wq.data_ptr(), sc.data_ptr(), y.data_ptr(),
                            torch.cuda.current_stream().cuda_stream)
    assert st == 0
    assert np.all(host_bits(y) == 0)


@pytest.mark.parametrize("T", [256, 1024])  # K-split and shared-X variants
def test_prefill_graph_replay(ngq, T):
    w = synthetic.WORKLOADS["qk"]
    _, codes, scales, x = full_inputs("qk", T)
    args = (dev_bf16(x), dev_u8(ngq.ngq_pack(codes, 4)), dev_scales(scales, False), 4, w.N)
    ref = host_bits(ngq.ngq_gemm(*args))
    y = torch.empty((T, w.N), dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ngq.ngq_gemm(*args, y=y)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ngq.ngq_gemm(*args, y=y)
    for rep in range(3):
        y.fill_(1.0)
        torch.cuda.synchronize()
        g.replay()
        assert np.array_equal(host_bits(y), ref), rep
        ngq.ngq_gemm(*args)  # eager work between replays
        torch.cuda.synchronize()
