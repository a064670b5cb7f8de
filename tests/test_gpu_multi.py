"""ngq_multi_gemm, several projections of one x in one launch, on the GPU.

Each projection of a fused call is checked against the oracle (every
column), and bit for bit against a single-projection call where one runs the
same tile code:
- when every projection is int4, or int5 / int8 without SwiGLU, the call
  runs one workgroup per tile: at T = 1 the VALU-step tile with 7 waves, so
  its SwiGLU projections must equal ngq_swiglu_gemm forced to the VALU kernel
  (7 waves too); its plain projections, and every projection at T >= 2 (the
  MFMA-step tile with 4 waves), have no single call with the same wave count
  (another order of the same sums) and are held to the oracle only;
- otherwise the persistent fused kernel runs the tile loop of the X-resident
  kernel with 8 waves (wave w takes pairs w, w + 8, ...; the wave partials
  are summed in wave order), so each projection must equal the single call
  forced to that kernel, whatever the tile width and the tile-to-workgroup
  assignment.
"""
import numpy as np
import pytest

import synthetic
from tests.parity import assert_parity, compare
from tests.test_gpu_parity import (ORACLE_THREADS, check_swiglu, dev_bf16, dev_scales, dev_u8, host_bits,
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


def draw(bits, sbf16, K, ncols, seed):
    g = np.random.default_rng(seed)
    codes = synthetic.draw_codes(K, ncols, bits, g)
    lo, hi = (5e-4, 1e-2) if sbf16 else (1e-3, 2e-2)
    scales = synthetic.draw_scales(K, ncols, lo, hi, sbf16, g)
    return codes, scales


def fused_tiles(K, specs):
    """Whether ngq_multi_gemm runs these projections as one workgroup per tile."""
    live = [(bits, swiglu) for bits, _, n, swiglu in specs if n > 0]
    return K > 0 and all(bits == 4 or not swiglu for bits, swiglu in live)


def single(ngq, x, p, path):
    """The same projection through ngq_gemm / ngq_swiglu_gemm on a forced
    kernel, or None when that kernel cannot serve the shape."""
    prev = ngq.ngq_debug_force_kernel(path)
    try:
        if p["swiglu"]:
            return ngq.ngq_swiglu_gemm(x, p["wq"], p["scales"], p["bits"], p["n"])
        return ngq.ngq_gemm(x, p["wq"], p["scales"], p["bits"], p["n"])
    except ngq.NgqError as e:
        if e.status == ngq.NGQ_ERR_UNSUPPORTED:
            return None
        raise
    finally:
        ngq.ngq_debug_force_kernel(prev)


def run_case(ngq, orc, T, K, specs, seed):
    g = np.random.default_rng(seed)
    x = synthetic.f32_to_bf16_bits(g.standard_normal((T, K)).astype(np.float32))
    xd = dev_bf16(x)
    host, projs = [], []
    for i, (bits, sbf16, n, swiglu) in enumerate(specs):
        ncols = 2 * n if swiglu else n
        codes, scales = draw(bits, sbf16, K, ncols, seed * 10 + i)
        packed = ngq.ngq_pack(codes, bits)
        host.append((codes, scales, orc.pack(codes, bits)))
        # outputs start as a pattern, so an unwritten element shows
        y = torch.full((T, n), -7.0, dtype=torch.bfloat16, device="cuda")
        projs.append(dict(wq=dev_u8(packed), scales=dev_scales(scales, sbf16), bits=bits, n=n, swiglu=swiglu, y=y))
    outs = ngq.ngq_multi_gemm(xd, projs)
    torch.cuda.synchronize()
    tiles = fused_tiles(K, specs)
    for i, ((bits, sbf16, n, swiglu), p, out) in enumerate(zip(specs, projs, outs)):
        what = f"T{T} K{K} proj{i} b{bits} n{n}{' swiglu' if swiglu else ''}"
        yb = host_bits(out)
        if n == 0:
            continue
        if not tiles:
            ref = single(ngq, xd, p, ngq.NGQ_KERNEL_XRES8)
        elif T == 1 and swiglu:
            ref = single(ngq, xd, p, ngq.NGQ_KERNEL_DOT)
            assert ref is not None, what
        else:
            ref = None
        if ref is not None:
            assert np.array_equal(yb, host_bits(ref)), what + ": differs from the single-projection kernel"
        codes, scales, packed_o = host[i]
        cols = np.arange(n, dtype=np.int32)
        if swiglu:
            h64, gg, u = swiglu_reference(orc, x, packed_o, scales, K, n, bits, sbf16, cols)
            check_swiglu(yb[:, cols], h64, gg, u, what)
        else:
            y64, axw, axs = orc.gemm(x, packed_o, scales, K, n, bits, sbf16, cols=cols, nthreads=ORACLE_THREADS,
                                     with_bounds=True)
            assert_parity(compare(yb[:, cols], y64, axw, axs, K, bits), what)
    return outs


CASES = [
    # T, K, [(bits, bf16 scales, n, swiglu)]
    (8, 1088, [(4, False, 96, False), (5, True, 100, False), (4, False, 36, True)]),   # odd group count
    (3, 320, [(4, True, 64, False), (4, False, 20, True), (5, False, 36, True), (5, True, 8, False)]),  # 4 kinds
    (6, 448, [(8, False, 64, False), (8, True, 100, True), (5, True, 4, False)]),       # int8, SwiGLU too
    (5, 512, [(4, False, 4, False)]),                                                   # one narrow tile
    (2, 64, [(5, True, 260, False), (4, False, 0, False), (4, False, 1028, True)]),     # one group; n = 0
    (7, 256, [(4, False, 16416, False), (5, True, 8224, True)]),                        # many tiles per workgroup
    (4, 17408, [(4, False, 520, False)]),                                               # long K, X per pair
    (8, 9216, [(4, False, 260, False), (5, True, 64, False)]),
    (4, 17408, [(8, True, 8, True), (8, False, 40, True)]),  # persistent: X staged in two rounds
    (3, 192, [(4, False, 72, False), (4, True, 36, True)]),                             # tiles, T = 3
    (7, 640, [(5, True, 96, False), (4, False, 44, True), (8, False, 28, False)]),      # tiles, T = 7
    # T = 1: the VALU-step tiles, unless a projection is int5 or int8 with SwiGLU
    (1, 1088, [(4, False, 96, False), (5, True, 100, False), (4, False, 36, True)]),   # odd group count
    (1, 448, [(8, False, 64, False), (8, True, 100, False), (4, True, 40, True), (5, False, 4, False)]),
    (1, 64, [(5, True, 260, False), (4, False, 0, False), (4, False, 1028, True)]),     # one group; n = 0
    (1, 256, [(4, False, 16416, False), (4, True, 8224, True)]),                        # many tiles
    (1, 320, [(4, True, 64, False), (4, False, 20, True), (5, False, 36, True)]),       # int5 SwiGLU: persistent
]


@pytest.mark.parametrize("T,K,specs", CASES)
def test_multi_small(ngq, orc, T, K, specs):
    run_case(ngq, orc, T, K, specs, seed=T * 100 + K)


@pytest.mark.parametrize("T", [1, 4, 8])
def test_multi_layer_shapes(ngq, orc, T):
    """The three projections of a stacked layer (QK int4, gate/value int5 with
    bf16 scales, gate/up int4 with the SwiGLU epilogue) in one call."""
    specs = [(4, False, 8192, False), (5, True, 12288, False), (4, False, synthetic.N_FF, True)]
    run_case(ngq, orc, T, synthetic.HIDDEN, specs, seed=T)


def test_multi_k_zero_and_t_zero(ngq):
    p = dict(wq=torch.zeros(16, dtype=torch.uint8, device="cuda"),
             scales=torch.zeros((1, 8), dtype=torch.float16, device="cuda"), bits=4, n=8,
             y=torch.full((3, 8), 5.0, dtype=torch.bfloat16, device="cuda"))
    x = torch.zeros((3, 0), dtype=torch.bfloat16, device="cuda")
    ngq.ngq_multi_gemm(x, [p])
    torch.cuda.synchronize()
    assert torch.all(p["y"] == 0)  # K = 0: an empty sum
    p["y"].fill_(5.0)
    ngq.ngq_multi_gemm(torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda"), [p])
    torch.cuda.synchronize()
    assert torch.all(p["y"] == 5.0)  # T = 0: nothing written


@pytest.mark.parametrize("T,specs", [(8, [(4, False, 4096, False), (5, True, 2048, True)]),
                                     (1, [(4, False, 4096, False), (5, True, 2048, False), (4, False, 2048, True)]),
                                     (4, [(4, False, 4096, False), (5, True, 2048, False), (4, False, 2048, True)])])
def test_multi_deterministic_and_graph_replay(ngq, T, specs):
    K = 1024
    g = np.random.default_rng(3)
    x = dev_bf16(synthetic.f32_to_bf16_bits(g.standard_normal((T, K)).astype(np.float32)))
    projs = []
    for i, (bits, sbf16, n, swiglu) in enumerate(specs):
        codes, scales = draw(bits, sbf16, K, 2 * n if swiglu else n, 50 + i)
        projs.append(dict(wq=dev_u8(ngq.ngq_pack(codes, bits)), scales=dev_scales(scales, sbf16), bits=bits, n=n,
                          swiglu=swiglu, y=torch.empty((T, n), dtype=torch.bfloat16, device="cuda")))
    first = [host_bits(o) for o in ngq.ngq_multi_gemm(x, projs)]
    again = [host_bits(o) for o in ngq.ngq_multi_gemm(x, projs)]
    assert all(np.array_equal(a, b) for a, b in zip(first, again))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ngq.ngq_multi_gemm(x, projs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ngq.ngq_multi_gemm(x, projs)
    for rep in range(3):
        for p in projs:
            p["y"].fill_(1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert all(np.array_equal(host_bits(p["y"]), f) for p, f in zip(projs, first)), rep
        ngq.ngq_multi_gemm(x, projs)  # eager work between replays
        torch.cuda.synchronize()
