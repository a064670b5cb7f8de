"""Every kernel path of ngq_gemm / ngq_swiglu_gemm against the oracle.

The library picks a kernel per shape (per-pair X with dynamic or static pair
assignment, X resident in LDS with 14 or 8 waves).  Here each path is forced
through the debug export and run on the same ragged shapes: odd group counts
(the last group pair has one group), N not a multiple of the tile, several
tiles per workgroup, long K, every bit width and both scale types.  The
(path, case) pairs a path does not serve are listed in UNSUPPORTED with the
reason; for them the call must refuse with NGQ_ERR_UNSUPPORTED, and a refusal
anywhere else fails the test.
"""
import numpy as np
import pytest

import synthetic
from tests.parity import assert_parity, compare
from tests.test_gpu_parity import dev_bf16, dev_scales, dev_u8, host_bits, make

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

PATHS = {1: "perpair_dyn", 2: "perpair_static", 3: "xres14", 4: "xres8", 10: "stream", 11: "dot"}


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
def forced(ngq, request):
    prev = ngq.ngq_debug_force_kernel(request.param)
    yield request.param
    ngq.ngq_debug_force_kernel(prev)


# (path, entry point, case) pairs that a forced path does not serve, with the
# reason; a case of None stands for every case of that entry point
UNSUPPORTED = {
    ("xres14", "swiglu", None): "the 14-wave X-resident kernel has no SwiGLU epilogue",
    ("perpair_dyn", "gemm", (4, True, 2, 17408, 64)):
        "one partial-sum block per pair (136 pairs at K = 17408) does not fit in LDS",
    ("perpair_dyn", "gemm", (8, False, 8, 17408, 96)): "the same",
    ("xres14", "gemm", (4, False, 8, 9216, 64)): "X exceeds the 14-wave kernel's prologue (6 chunks a thread)",
    ("xres14", "gemm", (8, False, 8, 17408, 96)): "the same",
    ("xres8", "gemm", (8, False, 8, 17408, 96)): "X (278 KB at T = 8) does not fit in LDS",
}


def run_checked(fn, path, entry, case):
    """The call's result, or None after checking that a listed pair refuses."""
    import groupwise_int_weight_amd as g

    if (path, entry, None) in UNSUPPORTED or (path, entry, case) in UNSUPPORTED:
        with pytest.raises(g.NgqError) as e:
            fn()
        assert e.value.status == g.NGQ_ERR_UNSUPPORTED
        return None
    return fn()


GEMM_CASES = [
    # bits, bf16 scales, T, K, N
    (4, False, 8, 5120, 96),
    (4, False, 3, 1088, 260),    # 17 groups: the last pair has one group
    (5, True, 8, 320, 36),       # 5 groups, N not a multiple of 32
    (5, False, 1, 1024, 100),
    (8, False, 5, 512, 64),
    (8, True, 8, 64, 4),         # one group, one narrow tile
    (4, True, 2, 17408, 64),     # long K
    (4, False, 8, 192, 520),
    (5, True, 7, 256, 16416),    # 513 tiles of 32 columns: several tiles per workgroup
    (4, False, 8, 9216, 64),     # X just fits in LDS: resident X staged in two rounds (streaming kernel)
    (8, False, 8, 17408, 96),    # X does not fit in LDS: X per pair (streaming kernel)
]


@pytest.mark.parametrize("forced", list(PATHS), ids=list(PATHS.values()), indirect=True)
@pytest.mark.parametrize("bits,sbf16,T,K,N", GEMM_CASES)
def test_gemm_path(ngq, orc, forced, bits, sbf16, T, K, N):
    _, (codes, scales, x) = make(bits, sbf16, T, K, N, seed=K + N + T)
    packed = ngq.ngq_pack(codes, bits)
    y = run_checked(lambda: ngq.ngq_gemm(dev_bf16(x), dev_u8(packed), dev_scales(scales, sbf16), bits, N),
                    PATHS[forced], "gemm", (bits, sbf16, T, K, N))
    if y is None:
        return
    yb = host_bits(y)
    y64, axw, axs = orc.gemm(x, orc.pack(codes, bits), scales, K, N, bits, sbf16, nthreads=8,
                             with_bounds=True)
    assert_parity(compare(yb, y64, axw, axs, K, bits), f"{PATHS[forced]} b{bits} T{T} K{K} N{N}")


SWIGLU_CASES = [
    (4, False, 8, 512, 100),
    (5, True, 3, 320, 36),
    (8, False, 1, 256, 64),
    (4, False, 4, 128, 8224),    # 257 tiles: several per workgroup
]


@pytest.mark.parametrize("forced", list(PATHS), ids=list(PATHS.values()), indirect=True)
@pytest.mark.parametrize("bits,sbf16,T,K,N_ff", SWIGLU_CASES)
def test_swiglu_path(ngq, orc, forced, bits, sbf16, T, K, N_ff):
    from tests.test_gpu_parity import check_swiglu, swiglu_reference

    _, (codes, scales, x) = make(bits, sbf16, T, K, 2 * N_ff, seed=K + N_ff)
    packed = ngq.ngq_pack(codes, bits)
    h = run_checked(lambda: ngq.ngq_swiglu_gemm(dev_bf16(x), dev_u8(packed), dev_scales(scales, sbf16), bits,
                                                N_ff), PATHS[forced], "swiglu", (bits, sbf16, T, K, N_ff))
    if h is None:
        return
    cols = np.arange(N_ff, dtype=np.int32)
    h64, g, u = swiglu_reference(orc, x, orc.pack(codes, bits), scales, K, N_ff, bits, sbf16, cols)
    check_swiglu(host_bits(h), h64, g, u, f"{PATHS[forced]} swiglu b{bits} T{T}")


@pytest.mark.parametrize("forced", list(PATHS), ids=list(PATHS.values()), indirect=True)
@pytest.mark.parametrize("bits", [4, 5, 8])
def test_identity_scales_integer_x_bit_exact_per_path(ngq, orc, forced, bits):
    """Scales 1 and small integer X: every partial sum is an integer below
    2^24, so every path must return the correctly rounded value exactly."""
    T, K, N = 8, 1088, 96
    g = np.random.default_rng(bits)
    lo, hi = synthetic.code_range(bits)
    codes = g.integers(lo, hi + 1, size=(K, N), dtype=np.int8)
    scales = np.full((K // 64, N), 0x3C00, np.uint16)  # fp16 1.0
    x = synthetic.f32_to_bf16_bits(g.integers(-3, 4, size=(T, K)).astype(np.float32))
    packed = ngq.ngq_pack(codes, bits)
    y = run_checked(lambda: ngq.ngq_gemm(dev_bf16(x), dev_u8(packed), dev_scales(scales, False), bits, N),
                    PATHS[forced], "gemm", (bits, False, T, K, N))
    if y is None:
        return
    y64 = orc.gemm(x, orc.pack(codes, bits), scales, K, N, bits, False)
    assert np.array_equal(host_bits(y), orc.round_bf16_array(y64)), PATHS[forced]

