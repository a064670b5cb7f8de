"""GPU tests of the stacked-layer sweep: the RMS rescale kernel against the
oracle, the first layer's projections against the oracle, and properties of
the chained layers (finite, unit mean square per row, deterministic, and a
captured graph replays to the eager result bit for bit).

The oracle only ever sees generator inputs: the projections of layer 0 take
the seeded x0, the rescale takes seeded z.  Layers after the first consume
the GPU's own activations, so the chain is checked through properties that
hold at any depth rather than against the oracle.
"""
import math

import numpy as np
import pytest

import synthetic
from tests.parity import assert_parity, bf16_bits_to_f64, compare
from tests.test_gpu_parity import ORACLE_THREADS, check_swiglu, dev_bf16, host_bits, sample_cols, swiglu_reference

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


def cur_stream():
    return torch.cuda.current_stream().cuda_stream


# ---- RMS rescale ----------------------------------------------------------------------

def rescale_check(zb, gb, orc):
    """Bit-exact against the oracle, except an element whose GPU value is the
    other bf16 neighbour of a quotient within 2^-40 (relative) of their
    midpoint: the kernel sums the squares in a different order than the
    oracle, an fp64 difference of at most N 2^-53 relative in the mean
    square, half that in the root."""
    ob = orc.rms_rescale(zb)
    diff = ob != gb
    if not diff.any():
        return 0
    z = bf16_bits_to_f64(zb)
    ms = np.mean(z ** 2, axis=1, keepdims=True)
    q = z / np.sqrt(ms)
    mid = 0.5 * (bf16_bits_to_f64(ob) + bf16_bits_to_f64(gb))
    near = np.abs(q - mid) <= 2.0 ** -40 * np.abs(q)
    one = np.abs(ob.astype(np.int32) - gb.astype(np.int32)) == 1
    assert np.all((near & one)[diff]), np.argwhere(diff)[:5]
    return int(diff.sum())


@pytest.mark.parametrize("T,N", [(1, 5120), (8, 5120), (5, 17408), (3, 1000), (2, 4), (8, 8)])
def test_rms_rescale_matches_oracle(ngq, orc, T, N):
    g = np.random.default_rng(1000 * T + N)
    # rows of very different magnitudes, including bf16 subnormal entries
    mags = np.array([1.0, 1e-30, 3e20, 1e-3, 17.0, 1e-38, 2.0 ** 100, 0.5])[:T]
    z = synthetic.f32_to_bf16_bits((g.standard_normal((T, N)) * mags[:, None]).astype(np.float32))
    z[0, :3] = [0x8000, 0x0000, 0x0001]  # -0, +0 and the smallest subnormal
    x = ngq.ngq_rms_rescale(dev_bf16(z))
    exempt = rescale_check(z, host_bits(x), orc)
    assert exempt <= 2


def test_rms_rescale_in_place_and_zero_row(ngq, orc):
    g = np.random.default_rng(5)
    z = synthetic.f32_to_bf16_bits(g.standard_normal((4, 5120)).astype(np.float32))
    z[2] = 0
    zd = dev_bf16(z)
    out = host_bits(ngq.ngq_rms_rescale(zd))
    ngq.ngq_rms_rescale(zd, x=zd)  # in place
    assert np.array_equal(host_bits(zd), out)
    assert np.all(out[2] == 0)
    rescale_check(z, out, orc)


# ---- the down projection with the closing rescale (ngq_gemm_rescale) --------------------

def gemm_rescale_case(ngq, orc, bits, sbf16, codes, scales, x, cols, what):
    """y against the oracle (sampled columns), x_next against the oracle's
    rescale of the GPU's own y and bit for bit against ngq_rms_rescale(y)."""
    from tests.test_gpu_parity import dev_scales, dev_u8

    K, N = codes.shape
    packed = ngq.ngq_pack(codes, bits)
    args = (dev_bf16(x), dev_u8(packed), dev_scales(scales, sbf16), bits, N)
    y, xn = ngq.ngq_gemm_rescale(*args)
    yb, xb = host_bits(y), host_bits(xn)
    y64, axw, axs = orc.gemm(x, orc.pack(codes, bits), scales, K, N, bits, sbf16, cols=cols,
                             nthreads=ORACLE_THREADS, with_bounds=True)
    assert_parity(compare(yb if cols is None else yb[:, cols], y64, axw, axs, K, bits), what)
    assert np.array_equal(xb, host_bits(ngq.ngq_rms_rescale(y)))
    rescale_check(yb, xb, orc)
    return args, yb, xb


@pytest.mark.parametrize("T", [1, 4, 8])
def test_gemm_rescale_down_shape(ngq, orc, T):
    w = synthetic.WORKLOADS["down"]
    codes, scales, x = synthetic.make_inputs(w, T, seed=3)
    if T == 8:
        # rows of very different magnitudes, and a zero row (y = 0 -> x_next = 0)
        mags = np.array([1.0, 1e-30, 3e20, 1e-3, 17.0, 0.0, 2.0 ** 60, 0.5], np.float32)
        xf = (bf16_bits_to_f64(x) * mags[:, None]).astype(np.float32)
        x = synthetic.f32_to_bf16_bits(xf)
    args, yb, xb = gemm_rescale_case(ngq, orc, 4, False, codes, scales, x, None, f"gemm_rescale down T{T}")
    if T == 8:
        assert np.all(yb[5] == 0) and np.all(xb[5] == 0)
    # the split is ngq_gemm_splitk's at every T: the same y bits
    assert np.array_equal(yb, host_bits(ngq.ngq_gemm_splitk(*args)))
    # deterministic, and a captured graph replays to the same bits
    ws = torch.empty(ngq.ngq_splitk_workspace_bytes(w.K, w.N, 4), dtype=torch.uint8, device="cuda")
    yg = torch.empty((T, w.N), dtype=torch.bfloat16, device="cuda")
    xg = torch.empty((T, w.N), dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ngq.ngq_gemm_rescale(*args, y=yg, x_next=xg, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ngq.ngq_gemm_rescale(*args, y=yg, x_next=xg, workspace=ws)
    for rep in range(3):
        yg.fill_(1.0)
        xg.fill_(1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(yg), yb), rep
        assert np.array_equal(host_bits(xg), xb), rep
        ngq.ngq_rms_rescale(yg, x=xg)  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("bits,sbf16,T,K,N", [
    (4, False, 3, 12352, 100),  # split, N % 8 != 0: the plain reduction, then ngq_rms_rescale
    (5, True, 6, 16384, 4104),  # split, 65 tiles of 64 columns, the fused closing kernel
    (8, False, 2, 20480, 8),    # split, one tile
    (4, True, 4, 960, 64),      # 8 pairs: no split, ngq_gemm then ngq_rms_rescale
])
def test_gemm_rescale_ragged(ngq, orc, bits, sbf16, T, K, N):
    from tests.test_gpu_parity import make

    _, (codes, scales, x) = make(bits, sbf16, T, K, N, seed=K + N)
    args, yb, _ = gemm_rescale_case(ngq, orc, bits, sbf16, codes, scales, x, None, f"gemm_rescale b{bits} T{T} N{N}")
    if K == 960:
        assert np.array_equal(yb, host_bits(ngq.ngq_gemm(*args)))


# ---- the same with the residual added in the epilogue (ngq_gemm_residual_rescale) ------

def draw_residual(T, N, seed, scale=4.0):
    g = np.random.default_rng(seed)
    return synthetic.f32_to_bf16_bits((g.standard_normal((T, N)) * scale).astype(np.float32))


def residual_case(ngq, orc, bits, sbf16, codes, scales, x, r, what):
    """y = x W + r against the oracle (every column; the residual's magnitude
    joins the rounding bound), x_next bit for bit against ngq_rms_rescale(y)
    and against the oracle's rescale of the GPU's own y."""
    from tests.test_gpu_parity import dev_scales, dev_u8

    K, N = codes.shape
    packed = ngq.ngq_pack(codes, bits)
    args = (dev_bf16(x), dev_u8(packed), dev_scales(scales, sbf16), bits, N)
    rd = dev_bf16(r)
    y, xn = ngq.ngq_gemm_residual_rescale(*args, rd)
    yb, xb = host_bits(y), host_bits(xn)
    y64, axw, axs = orc.gemm(x, orc.pack(codes, bits), scales, K, N, bits, sbf16, nthreads=ORACLE_THREADS,
                             with_bounds=True)
    y64r, axwr = orc.add_residual(y64, r, axw)
    assert_parity(compare(yb, y64r, axwr, axs, K, bits), what)
    assert np.array_equal(xb, host_bits(ngq.ngq_rms_rescale(y)))
    rescale_check(yb, xb, orc)
    return args, rd, yb, xb


@pytest.mark.parametrize("T", [1, 4, 8])
def test_gemm_residual_rescale_down_shape(ngq, orc, T):
    w = synthetic.WORKLOADS["down"]
    codes, scales, x = synthetic.make_inputs(w, T, seed=5)
    r = draw_residual(T, w.N, seed=60 + T)
    if T == 8:
        # a zero row of x and of r: y = 0 and x_next = 0
        x[5] = 0
        r[5] = 0
    args, rd, yb, xb = residual_case(ngq, orc, 4, False, codes, scales, x, r, f"residual down T{T}")
    if T == 8:
        assert np.all(yb[5] == 0) and np.all(xb[5] == 0)
    # a zero residual: the same slices (3) and sums as ngq_gemm_rescale, so the
    # same y (as values: an fp32 sum of -0 plus +0 is +0)
    y0, _ = ngq.ngq_gemm_residual_rescale(*args, torch.zeros_like(rd))
    yr, _ = ngq.ngq_gemm_rescale(*args)
    assert torch.equal(y0.float(), yr.float())
    # deterministic, and a captured graph replays to the same bits
    ws = torch.empty(ngq.ngq_splitk_workspace_bytes(w.K, w.N, 4), dtype=torch.uint8, device="cuda")
    yg = torch.empty((T, w.N), dtype=torch.bfloat16, device="cuda")
    xg = torch.empty((T, w.N), dtype=torch.bfloat16, device="cuda")
    ngq.ngq_gemm_residual_rescale(*args, rd, y=yg, x_next=xg, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(yg), yb) and np.array_equal(host_bits(xg), xb)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ngq.ngq_gemm_residual_rescale(*args, rd, y=yg, x_next=xg, workspace=ws)
    for rep in range(3):
        yg.fill_(1.0)
        xg.fill_(1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(yg), yb), rep
        assert np.array_equal(host_bits(xg), xb), rep
        ngq.ngq_rms_rescale(yg, x=xg)  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("bits,sbf16,T,K,N", [
    (4, False, 3, 12352, 100),  # 8 slices (97 pairs, the last one group), N % 8 != 0: plain reduction + rescale
    (5, True, 6, 16384, 4104),  # 3 slices, 65 tiles of 64 columns, the fused closing kernel
    (8, False, 2, 20480, 8),    # 8 slices, one tile
    (4, True, 4, 4096, 64),     # 32 pairs: 4 slices, plain reduction
    (5, False, 5, 5120, 4096),  # 40 pairs, 64 tiles: 4 slices, the fused closing kernel
    (4, False, 8, 640, 5120),   # 5 pairs: one slice, the fused closing kernel
    (8, True, 7, 64, 4096),     # one group
])
def test_gemm_residual_rescale_ragged(ngq, orc, bits, sbf16, T, K, N):
    from tests.test_gpu_parity import make

    _, (codes, scales, x) = make(bits, sbf16, T, K, N, seed=K + N + 1)
    r = draw_residual(T, N, seed=K + N, scale=0.05)
    residual_case(ngq, orc, bits, sbf16, codes, scales, x, r, f"residual b{bits} T{T} K{K} N{N}")


def test_gemm_residual_rescale_zero_weights(ngq, orc):
    """Every code 0: the projection is 0, so y is the residual (up to the
    offset term's fp32 cancellation, which the parity bound covers) and
    x_next its rescale."""
    T, K, N = 8, 17408, 5120
    codes = np.zeros((K, N), dtype=np.int8)
    scales = synthetic.draw_scales(K, N, 1e-3, 2e-2, False, np.random.default_rng(2))
    x = synthetic.f32_to_bf16_bits(np.random.default_rng(3).standard_normal((T, K)).astype(np.float32))
    r = draw_residual(T, N, seed=4)
    residual_case(ngq, orc, 4, False, codes, scales, x, r, "residual, zero weights")


# ---- stacked layers -------------------------------------------------------------------

_STACK = {}


def stack_layers(ngq, layers):
    if _STACK.get("n", 0) < layers:
        _STACK.clear()
        torch.cuda.empty_cache()
        _STACK["w"] = synthetic.device_stack(layers, ngq.ngq_packed_bytes, seed=0)
        _STACK["n"] = layers
    return _STACK["w"][:layers]


def to_host_u8(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def to_host_u16(t):
    torch.cuda.synchronize()
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("T", [1, 8])
def test_stack_first_layer_matches_oracle(ngq, orc, T):
    from groupwise_int_weight_amd.stack import Stack

    layers = stack_layers(ngq, 2)
    st = Stack(layers, T)
    x0 = synthetic.stack_x0(T, seed=0)
    st.x.copy_(dev_bf16(x0))
    st.layer(0)
    torch.cuda.synchronize()
    for name, out, sbf16 in (("qk", st.q, False), ("gv", st.v, True)):
        w = synthetic.WORKLOADS[name]
        wq, s = layers[0][name]
        cols = sample_cols(w.N, seed=30 + T)
        y64, axw, axs = orc.gemm(x0, to_host_u8(wq), to_host_u16(s), w.K, w.N, w.bits, sbf16, cols=cols,
                                 nthreads=8, with_bounds=True)
        assert_parity(compare(host_bits(out)[:, cols], y64, axw, axs, w.K, w.bits), f"stack {name} T{T}")
    wq, s = layers[0]["gate_up"]
    cols = sample_cols(synthetic.N_FF, seed=40 + T)
    h64, g, u = swiglu_reference(orc, x0, to_host_u8(wq), to_host_u16(s), synthetic.HIDDEN, synthetic.N_FF, 4,
                                 False, cols)
    check_swiglu(host_bits(st.h)[:, cols], h64, g, u, f"stack swiglu T{T}")


@pytest.mark.parametrize("T,mode", [(1, "concurrent"), (8, "concurrent"), (8, "in_order"), (1, "fused"),
                                    (8, "fused")])
def test_stack_chain_properties_and_graph_replay(ngq, T, mode):
    from groupwise_int_weight_amd.stack import Stack

    L = 4
    layers = stack_layers(ngq, L)
    st = Stack(layers, T, concurrent=mode == "concurrent", fused=mode == "fused")
    x0 = dev_bf16(synthetic.stack_x0(T, seed=0))
    eager = to_host_u16(st.forward(x0))
    again = to_host_u16(st.forward(x0))
    assert np.array_equal(eager, again)  # deterministic
    if mode == "concurrent":
        # the side streams change only the order of independent work
        assert np.array_equal(eager, to_host_u16(Stack(layers, T).forward(x0)))
    if mode == "fused":
        # The split-K down projection groups its fp32 sums differently, so the
        # chain leaves the in-order one by rounding differences only.
        ref = bf16_bits_to_f64(to_host_u16(Stack(layers, T).forward(x0)))
        got = bf16_bits_to_f64(eager)
        assert np.linalg.norm(got - ref) <= 1e-2 * np.linalg.norm(ref)
    v = bf16_bits_to_f64(eager)
    assert np.all(np.isfinite(v))
    # every row leaves the rescale with unit mean square, up to bf16 rounding
    assert np.all(np.abs(np.mean(v ** 2, axis=1) - 1.0) < 2.0 ** -7)
    # the chain actually moves: the output is not the input
    assert not np.array_equal(eager, to_host_u16(x0))

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.x.copy_(x0)
        for i in range(L):  # warm-up on the capture stream
            st.layer(i, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        for i in range(L):
            st.layer(i)
    for rep in range(3):
        st.x.copy_(x0)
        graph.replay()
        got = to_host_u16(st.x)
        assert np.array_equal(got, eager), rep
        # eager work between replays
        st.forward(x0, layers=1)
        torch.cuda.synchronize()
    assert math.isfinite(float(v.sum()))
