"""ngq_gemm and ngq_swiglu_gemm with 8 < T <= 64 tokens (the verify rounds of
several requests in one call) on the GPU, against the CPU oracle.  From 33
tokens on the calls route to the token x column tiles of prefill; the 64-row
verify kernel is also run there, forced.

Small ragged shapes (odd group counts, so the last pair has one group; a
column tail; every bit width and both scale types), every token-block
boundary (16, 32, 64 and one past), the full-size projections on sampled
columns, bit-exact cases, guard bands, K = 0, determinism and graph replay.
"""
import numpy as np
import pytest

import synthetic
from tests.parity import assert_parity, bf16_bits_to_f64, compare
from tests.test_gpu_parity import (check_swiglu, dev_bf16, dev_scales, dev_u8, host_bits, make, run_and_compare,
                                   swiglu_reference)

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


SMALL = [
    # bits, scale_bf16, T, K, N
    (4, False, 9, 320, 100),     # one past the decode range; 5 groups (a half pair)
    (5, True, 16, 1024, 520),    # one full token block
    (8, False, 17, 512, 300),
    (4, True, 33, 192, 36),      # 3 groups
    (5, False, 64, 640, 68),
    (8, True, 40, 256, 4),       # one narrow tile
    (4, False, 64, 2048, 4100),  # ragged column tail
    (5, True, 24, 64, 40),       # a single group
    (8, False, 48, 1088, 132),   # 17 groups
    (8, False, 32, 512, 12004),  # 48-column tiles (one per CU), a 4-column last tile
    (4, True, 16, 256, 10000),   # 48-column tiles, a 16-column last tile
    (5, False, 20, 384, 9000),   # 48-column tiles, int5
]


@pytest.mark.parametrize("bits,sbf16,T,K,N", SMALL)
def test_verify_small(ngq, orc, bits, sbf16, T, K, N):
    _, (codes, scales, x) = make(bits, sbf16, T, K, N, seed=T * 131 + K + N)
    run_and_compare(ngq, orc, bits, sbf16, codes, scales, x, what=f"verify b{bits} T{T} K{K} N{N}")


@pytest.mark.parametrize("T", [10, 15, 16, 17, 31, 32, 33, 47, 63, 64])
def test_verify_token_counts(ngq, orc, T):
    _, (codes, scales, x) = make(4, False, T, 640, 200, seed=T)
    run_and_compare(ngq, orc, 4, False, codes, scales, x, what=f"verify T{T}")


@pytest.mark.parametrize("bits,sbf16,T,K,N", [c for c in SMALL if c[2] > 32] + [(4, False, 33, 640, 200),
                                                                              (5, True, 63, 320, 100)])
def test_verify_wide_kernel_forced(ngq, orc, bits, sbf16, T, K, N):
    """33 <= T <= 64 routes to the token x column tiles by default; the 64-row
    verify kernel still serves it when forced."""
    _, (codes, scales, x) = make(bits, sbf16, T, K, N, seed=T * 131 + K + N)
    prev = ngq.ngq_debug_force_kernel(ngq.NGQ_KERNEL_WIDE)
    try:
        run_and_compare(ngq, orc, bits, sbf16, codes, scales, x, what=f"wide forced b{bits} T{T} K{K} N{N}")
    finally:
        ngq.ngq_debug_force_kernel(prev)


_FULL = {}


def full_inputs(name):
    if name not in _FULL:
        w = synthetic.WORKLOADS[name]
        _FULL.clear()
        _FULL[name] = (w,) + tuple(synthetic.make_inputs(w, 64, seed=1))
    return _FULL[name]


@pytest.mark.parametrize("name,T", [("qk", 64), ("qk", 16), ("qk", 40), ("gv", 64), ("gv", 24), ("qk8", 64),
                                    ("down", 64)])
def test_verify_full_size(ngq, orc, name, T):
    w, codes, scales, x = full_inputs(name)
    yb, _ = run_and_compare(ngq, orc, w.bits, w.scale_bf16, codes, scales, x[:T], what=f"verify {name} T{T}")
    assert np.all(np.isfinite(bf16_bits_to_f64(yb)))


@pytest.mark.parametrize("bits,sbf16,T,K,N_ff", [(4, False, 16, 512, 100), (5, True, 33, 320, 36),
                                                  (8, False, 64, 256, 64), (4, True, 40, 1024, 260)])
def test_verify_swiglu_small(ngq, orc, bits, sbf16, T, K, N_ff):
    _, (codes, scales, x) = make(bits, sbf16, T, K, 2 * N_ff, seed=K + N_ff + T)
    packed = ngq.ngq_pack(codes, bits)
    h = ngq.ngq_swiglu_gemm(dev_bf16(x), dev_u8(packed), dev_scales(scales, sbf16), bits, N_ff)
    cols = np.arange(N_ff, dtype=np.int32)
    h64, g, u = swiglu_reference(orc, x, orc.pack(codes, bits), scales, K, N_ff, bits, sbf16, cols)
    check_swiglu(host_bits(h), h64, g, u, f"verify swiglu b{bits} T{T}")


def test_verify_swiglu_full_size(ngq, orc):
    w, codes, scales, x = full_inputs("gate_up")
    N_ff = synthetic.N_FF
    packed = ngq.ngq_pack(codes, 4)
    h = ngq.ngq_swiglu_gemm(dev_bf16(x), dev_u8(packed), dev_scales(scales, False), 4, N_ff)
    cols = np.arange(N_ff, dtype=np.int32)
    h64, g, u = swiglu_reference(orc, x, orc.pack(codes, 4), scales, w.K, N_ff, 4, False, cols)
    check_swiglu(host_bits(h), h64, g, u, "verify swiglu gate_up T64")


@pytest.mark.parametrize("bits", [4, 5, 8])
def test_verify_identity_scales_integer_x_bit_exact(ngq, orc, bits):
    """s = 1 and integer x: every partial sum is an integer below 2^24, so the
    fp32 result is exact and its bf16 rounding must equal the oracle's."""
    g = np.random.default_rng(140 + bits)
    T, K, N = 64, 576, 132
    codes = synthetic.draw_codes(K, N, bits, g)
    scales = np.full((K // 64, N), 0x3C00, np.uint16)
    xi = g.integers(-2, 3, size=(T, K))
    x = synthetic.f32_to_bf16_bits(xi.astype(np.float32))
    y = ngq.ngq_gemm(dev_bf16(x), dev_u8(ngq.ngq_pack(codes, bits)), dev_scales(scales, False), bits, N)
    exact = xi.astype(np.int64) @ codes.astype(np.int64)
    assert np.array_equal(host_bits(y), orc.round_bf16_array(exact.astype(np.float64)))


def test_verify_one_hot_rows_bit_exact(ngq, orc):
    """64 one-hot x rows (k = row index + offset) with power-of-two scales read
    single weights back exactly: token t's output row is codes[k_t] s[k_t]."""
    K, N, T = 320, 72, 64
    g = np.random.default_rng(77)
    codes = synthetic.draw_codes(K, N, 5, g)
    exps = g.integers(-9, -3, size=(K // 64, N))
    scales = synthetic.f32_to_bf16_bits((2.0 ** exps).astype(np.float32))
    wq, sd = dev_u8(ngq.ngq_pack(codes, 5)), dev_scales(scales, True)
    for start in (0, 64, 256):
        ks = (start + np.arange(T)) % K
        x = np.zeros((T, K), np.float32)
        x[np.arange(T), ks] = 1.0
        y = ngq.ngq_gemm(dev_bf16(synthetic.f32_to_bf16_bits(x)), wq, sd, 5, N)
        expect = codes[ks, :].astype(np.float64) * (2.0 ** exps[ks // 64, :])
        assert np.array_equal(host_bits(y), orc.round_bf16_array(expect)), start


def test_verify_guard_bands_and_determinism(ngq, orc):
    T, K, N = 40, 320, 100
    _, (codes, scales, x) = make(4, False, T, K, N, seed=21)
    pad = 4096
    buf = torch.full((pad + T * N + pad,), 0x7E7E, dtype=torch.int16, device="cuda")
    y = buf[pad:pad + T * N].view(torch.bfloat16).view(T, N)
    args = (dev_bf16(x), dev_u8(ngq.ngq_pack(codes, 4)), dev_scales(scales, False), 4, N)
    ngq.ngq_gemm(*args, y=y)
    hb = host_bits(buf)
    assert np.all(hb[:pad] == 0x7E7E) and np.all(hb[pad + T * N:] == 0x7E7E)
    y64, axw, axs = orc.gemm(x, orc.pack(codes, 4), scales, K, N, 4, False, with_bounds=True)
    assert_parity(compare(hb[pad:pad + T * N].reshape(T, N), y64, axw, axs, K, 4))
    for _ in range(3):
        assert np.array_equal(host_bits(ngq.ngq_gemm(*args)), hb[pad:pad + T * N].reshape(T, N))


def test_verify_k_zero_writes_zeros(ngq):
    T, N = 20, 8
    y = torch.full((T, N), 7.0, dtype=torch.bfloat16, device="cuda")
    wq = torch.zeros(16, dtype=torch.uint8, device="cuda")
    sc = torch.zeros((1, N), dtype=torch.float16, device="cuda")
    st = ngq.lib().ngq_gemm(T, 0, N, 4, 64, wq.data_ptr(), wq.data_ptr(), sc.data_ptr(), y.data_ptr(),
                            torch.cuda.current_stream().cuda_stream)
    assert st == 0
    assert np.all(host_bits(y) == 0)


def test_verify_graph_replay(ngq):
    w = synthetic.WORKLOADS["qk"]
    T = 64
    _, codes, scales, x = full_inputs("qk")
    args = (dev_bf16(x[:T]), dev_u8(ngq.ngq_pack(codes, 4)), dev_scales(scales, False), 4, w.N)
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
