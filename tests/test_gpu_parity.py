"""GPU parity of libngq against the CPU oracle, through the C ABI.

Every case draws seeded inputs from `synthetic`, packs them with the library's
packer (and, independently, with the oracle's), runs the HIP kernels and
compares element by element with the oracle (gates in tests/parity.py).
Full-size workloads are checked on every output column (the oracle computes a
whole T=8 projection in well under a second on the host's cores), plus
whole-output properties.
"""
import os
import math

import numpy as np
import pytest

import synthetic
from tests.parity import assert_parity, bf16_bits_to_f64, compare, rel_l2_gate

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


def dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to("cuda")


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).to("cuda").view(torch.bfloat16)


def dev_scales(bits, bf16):
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).to("cuda")
    return t.view(torch.bfloat16 if bf16 else torch.float16)


def host_bits(t):
    torch.cuda.synchronize()
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def make(bits, sbf16, T, K, N, seed, lo=1e-3, hi=2e-2, config_id=50):
    w = synthetic.Workload("case", K, N, bits, sbf16, lo, hi, config_id)
    return w, synthetic.make_inputs(w, T, seed=seed)


# host threads for the oracle on full-size cases
ORACLE_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def run_and_compare(ngq, orc, bits, sbf16, codes, scales, x, cols=None, what=""):
    K, N = codes.shape
    packed = ngq.ngq_pack(codes, bits)
    packed_o = orc.pack(codes, bits)
    assert np.array_equal(packed, packed_o)
    y = ngq.ngq_gemm(dev_bf16(x), dev_u8(packed), dev_scales(scales, sbf16), bits, N)
    yb = host_bits(y)
    y64, axw, axs = orc.gemm(x, packed_o, scales, K, N, bits, sbf16, cols=cols, nthreads=ORACLE_THREADS,
                             with_bounds=True)
    sub = yb if cols is None else yb[:, cols]
    rep = compare(sub, y64, axw, axs, K, bits)
    assert_parity(rep, what)
    return yb, rep


# ---- stage bit-exactness: unpack and dequant ---------------------------------

@pytest.mark.parametrize("bits", [4, 5, 8])
@pytest.mark.parametrize("K,N", [(64, 4), (320, 36), (1024, 260)])
def test_unpack_codes_bit_exact(ngq, bits, K, N):
    g = np.random.default_rng(100 + bits + K + N)
    codes = synthetic.draw_codes(K, N, bits, g)
    got = ngq.ngq_unpack_codes(dev_u8(ngq.ngq_pack(codes, bits)), K, N, bits)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), codes)


@pytest.mark.parametrize("bits,sbf16", [(4, False), (5, True), (8, False), (4, True)])
def test_dequant_bit_exact(ngq, orc, bits, sbf16):
    K, N = 256, 68
    _, (codes, scales, _) = make(bits, sbf16, 1, K, N, seed=5)
    w = ngq.ngq_dequant_f32(dev_u8(ngq.ngq_pack(codes, bits)), dev_scales(scales, sbf16), K, N, bits)
    torch.cuda.synchronize()
    ref = orc.dequant(orc.pack(codes, bits), scales, K, N, bits, sbf16)
    assert np.array_equal(w.cpu().numpy().view(np.uint32), ref.astype(np.float32).view(np.uint32))
    assert np.array_equal(ref.astype(np.float32).astype(np.float64), ref)  # c * s is exact in fp32


# ---- small shapes: every output against the oracle ------------------------------

SMALL = [
    # bits, scale_bf16, T, K, N
    (4, False, 1, 256, 256),      # the tiny int4 GEMV
    (4, False, 8, 1024, 1000),    # ragged column tail
    (4, True, 3, 320, 100),       # odd group count
    (5, True, 8, 1024, 520),
    (5, False, 5, 192, 36),
    (5, True, 2, 64, 4),          # a single group
    (8, False, 8, 512, 300),
    (8, True, 6, 320, 68),
    (4, False, 7, 2048, 4100),
    (5, True, 4, 5120, 192),
]


@pytest.mark.parametrize("bits,sbf16,T,K,N", SMALL)
def test_gemm_small(ngq, orc, bits, sbf16, T, K, N):
    _, (codes, scales, x) = make(bits, sbf16, T, K, N, seed=T * 131 + K + N)
    run_and_compare(ngq, orc, bits, sbf16, codes, scales, x, what=f"b{bits} T{T} K{K} N{N}")


@pytest.mark.parametrize("T", range(1, 9))
def test_gemm_every_t(ngq, orc, T):
    _, (codes, scales, x) = make(4, False, T, 640, 200, seed=T)
    run_and_compare(ngq, orc, 4, False, codes, scales, x, what=f"T{T}")


# ---- full-size workloads, every output column ------------------------------------

def sample_cols(N, seed, n_random=192):
    """Columns for cases too large for the oracle to compute whole in seconds
    (prefill-size T): both edges and random columns in between."""
    g = np.random.default_rng(seed)
    cols = np.unique(np.concatenate([np.arange(64), np.arange(N - 64, N), g.integers(0, N, n_random)]))
    return cols.astype(np.int32)


_FULL = {}


def full_inputs(name):
    if name not in _FULL:
        w = synthetic.WORKLOADS[name]
        codes, scales, x = synthetic.make_inputs(w, 8, seed=0)
        _FULL.clear()
        _FULL[name] = (w, codes, scales, x)
    return _FULL[name]


def closed_form_rms(w):
    ec2 = {4: 21.5, 5: 85.5, 8: (256 ** 2 - 1) / 12 + 0.25}[w.bits]
    es2 = (w.scale_lo ** 2 + w.scale_lo * w.scale_hi + w.scale_hi ** 2) / 3
    return math.sqrt(w.K * ec2 * es2)


# every T of one request's decode or verify step: each T has its own X layout
# in the kernels (T = 6 is the ninfer-ext README's recommended five drafts + 1)
@pytest.mark.parametrize("name,T", [("qk", t) for t in range(1, 9)] + [("gv", t) for t in range(1, 9)] +
                         [("qk8", 1), ("qk8", 8)])
def test_gemm_full_size(ngq, orc, name, T):
    w, codes, scales, x = full_inputs(name)
    yb, rep = run_and_compare(ngq, orc, w.bits, w.scale_bf16, codes, scales, x[:T], what=f"{name} T{T}")
    y = bf16_bits_to_f64(yb)
    assert np.all(np.isfinite(y))
    assert abs(math.sqrt(np.mean(y ** 2)) / closed_form_rms(w) - 1) < 0.03


def swiglu_reference(orc, x, packed_o, scales, K, N_ff, bits, sbf16, cols):
    both = np.concatenate([cols, cols + N_ff]).astype(np.int32)
    y64, axw, axs = orc.gemm(x, packed_o, scales, K, 2 * N_ff, bits, sbf16, cols=both, nthreads=ORACLE_THREADS,
                             with_bounds=True)
    n = cols.size
    g, u = y64[:, :n], y64[:, n:]
    h64 = orc.swiglu(g, u)
    return h64, g, u


def check_swiglu(hb, h64, g, u, what):
    """h = SiLU(g) u: the bf16 result against the exact value.  The error of
    fp32 g and u propagates with d h = SiLU'(g) u dg + SiLU(g) du, so the
    relative L2 gate is the same as for the projection."""
    hg = bf16_bits_to_f64(hb)
    rel, gate = rel_l2_gate(hg, h64)
    assert rel <= gate, (what, rel, gate)
    rms = math.sqrt(np.mean(h64 ** 2))
    h16 = bf16_bits_to_f64(__import__("oracle").round_bf16_array(h64))
    # one bf16 step of the output plus the propagated fp32 error of g and u
    step = np.abs(h16) * 2.0 ** -7 + 1e-30
    assert np.all(np.abs(hg - h16) <= np.maximum(1e-2 * rms, step)), what


@pytest.mark.parametrize("T", [1, 8])
def test_swiglu_and_down_full_size(ngq, orc, T):
    wgu = synthetic.WORKLOADS["gate_up"]
    wdn = synthetic.WORKLOADS["down"]
    N_ff = synthetic.N_FF
    codes, scales, x = synthetic.make_inputs(wgu, T, seed=0)
    packed = ngq.ngq_pack(codes, 4)
    packed_o = orc.pack(codes, 4)
    assert np.array_equal(packed, packed_o)
    h = ngq.ngq_swiglu_gemm(dev_bf16(x), dev_u8(packed), dev_scales(scales, False), 4, N_ff)
    hb = host_bits(h)
    cols = np.arange(N_ff, dtype=np.int32)
    h64, g, u = swiglu_reference(orc, x, packed_o, scales, wgu.K, N_ff, 4, False, cols)
    check_swiglu(hb, h64, g, u, f"swiglu T{T}")
    del codes, packed, packed_o
    # down projection: K = N_ff, its activations drawn by the generator (the
    # oracle never takes a GPU result as input)
    dcodes, dscales, dx = synthetic.make_inputs(wdn, T, seed=0)
    dpacked = ngq.ngq_pack(dcodes, 4)
    y = ngq.ngq_gemm(dev_bf16(dx), dev_u8(dpacked), dev_scales(dscales, False), 4, wdn.N)
    yb = host_bits(y)
    y64, axw, axs = orc.gemm(dx, orc.pack(dcodes, 4), dscales, wdn.K, wdn.N, 4, False, nthreads=ORACLE_THREADS,
                             with_bounds=True)
    assert_parity(compare(yb, y64, axw, axs, wdn.K, 4), f"down T{T}")


@pytest.mark.parametrize("bits,sbf16,T,K,N_ff", [(4, False, 8, 512, 100), (5, True, 3, 320, 36),
                                                  (8, False, 1, 256, 64), (4, True, 6, 1024, 260)])
def test_swiglu_small(ngq, orc, bits, sbf16, T, K, N_ff):
    _, (codes, scales, x) = make(bits, sbf16, T, K, 2 * N_ff, seed=K + N_ff)
    packed = ngq.ngq_pack(codes, bits)
    h = ngq.ngq_swiglu_gemm(dev_bf16(x), dev_u8(packed), dev_scales(scales, sbf16), bits, N_ff)
    cols = np.arange(N_ff, dtype=np.int32)
    h64, g, u = swiglu_reference(orc, x, orc.pack(codes, bits), scales, K, N_ff, bits, sbf16, cols)
    check_swiglu(host_bits(h), h64, g, u, f"swiglu b{bits} T{T}")


# ---- exact cases ------------------------------------------------------------------

@pytest.mark.parametrize("bits", [4, 5, 8])
def test_identity_scales_integer_x_bit_exact(ngq, orc, bits):
    """s = 1 and integer x: every partial sum is an integer below 2^24, so the
    fp32 result is exact and its bf16 rounding must equal the oracle's."""
    g = np.random.default_rng(40 + bits)
    T, K, N = 8, 512, 132
    codes = synthetic.draw_codes(K, N, bits, g)
    scales = np.full((K // 64, N), 0x3C00, np.uint16)
    xi = g.integers(-2, 3, size=(T, K))
    x = synthetic.f32_to_bf16_bits(xi.astype(np.float32))
    y = ngq.ngq_gemm(dev_bf16(x), dev_u8(ngq.ngq_pack(codes, bits)), dev_scales(scales, False), bits, N)
    exact = xi.astype(np.int64) @ codes.astype(np.int64)
    assert np.array_equal(host_bits(y), orc.round_bf16_array(exact.astype(np.float64)))


@pytest.mark.parametrize("bits,sbf16", [(4, False), (5, True), (8, False)])
def test_one_hot_x_bit_exact(ngq, orc, bits, sbf16):
    """One-hot x rows with power-of-two scales read single weights back: y =
    c * s is exact in bf16, so each output addresses one (k, n) exactly."""
    K, N = 320, 72
    g = np.random.default_rng(70 + bits)
    codes = synthetic.draw_codes(K, N, bits, g)
    exps = g.integers(-9, -3, size=(K // 64, N))
    sc = (2.0 ** exps).astype(np.float32)
    scales = synthetic.f32_to_bf16_bits(sc) if sbf16 else sc.astype(np.float16).view(np.uint16)
    wq = dev_u8(ngq.ngq_pack(codes, bits))
    sd = dev_scales(scales, sbf16)
    for start in range(0, K, 8):
        ks = np.arange(start, start + 8)
        x = np.zeros((8, K), np.float32)
        x[np.arange(8), ks] = 1.0
        y = ngq.ngq_gemm(dev_bf16(synthetic.f32_to_bf16_bits(x)), wq, sd, bits, N)
        expect = codes[ks, :].astype(np.float64) * (2.0 ** exps[ks // 64, :])
        assert np.array_equal(host_bits(y), orc.round_bf16_array(expect)), start


def test_metamorphic_scaling_and_sign(ngq):
    _, (codes, scales, x) = make(4, False, 8, 1024, 264, seed=9)
    wq = dev_u8(ngq.ngq_pack(codes, 4))
    xd = dev_bf16(x)
    base = ngq.ngq_gemm(xd, wq, dev_scales(scales, False), 4, 264)
    s2 = (scales.view(np.float16).astype(np.float32) * 2).astype(np.float16).view(np.uint16)
    twice = ngq.ngq_gemm(xd, wq, dev_scales(s2, False), 4, 264)
    neg = ngq.ngq_gemm(-xd, wq, dev_scales(scales, False), 4, 264)
    b = bf16_bits_to_f64(host_bits(base))
    assert np.array_equal(bf16_bits_to_f64(host_bits(twice)), 2 * b)
    assert np.array_equal(bf16_bits_to_f64(host_bits(neg)), -b)


def test_deterministic(ngq):
    _, (codes, scales, x) = make(5, True, 8, 5120, 1536, seed=3)
    args = (dev_bf16(x), dev_u8(ngq.ngq_pack(codes, 5)), dev_scales(scales, True), 5, 1536)
    a = host_bits(ngq.ngq_gemm(*args))
    for _ in range(3):
        assert np.array_equal(host_bits(ngq.ngq_gemm(*args)), a)


# ---- edge cases and memory safety ------------------------------------------------

def test_guard_bands_untouched(ngq, orc):
    T, K, N = 5, 320, 100
    _, (codes, scales, x) = make(4, False, T, K, N, seed=12)
    pad = 4096
    buf = torch.full((pad + T * N + pad,), 0x7E7E, dtype=torch.int16, device="cuda")
    y = buf[pad:pad + T * N].view(torch.bfloat16).view(T, N)
    ngq.ngq_gemm(dev_bf16(x), dev_u8(ngq.ngq_pack(codes, 4)), dev_scales(scales, False), 4, N, y=y)
    hb = host_bits(buf)
    assert np.all(hb[:pad] == 0x7E7E) and np.all(hb[pad + T * N:] == 0x7E7E)
    y64, axw, axs = orc.gemm(x, orc.pack(codes, 4), scales, K, N, 4, False, with_bounds=True)
    assert_parity(compare(hb[pad:pad + T * N].reshape(T, N), y64, axw, axs, K, 4))


def test_k_zero_writes_zeros(ngq):
    y = torch.full((3, 8), 7.0, dtype=torch.bfloat16, device="cuda")
    x = torch.zeros((3, 0), dtype=torch.bfloat16, device="cuda")
    wq = torch.zeros(16, dtype=torch.uint8, device="cuda")
    sc = torch.zeros((1, 8), dtype=torch.float16, device="cuda")
    st = ngq.lib().ngq_gemm(3, 0, 8, 4, 64, x.data_ptr() if x.numel() else wq.data_ptr(), wq.data_ptr(),
                            sc.data_ptr(), y.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0
    assert np.all(host_bits(y) == 0)


def test_t_zero_leaves_output(ngq):
    y = torch.full((1, 8), 7.0, dtype=torch.bfloat16, device="cuda")
    st = ngq.lib().ngq_gemm(0, 64, 8, 4, 64, None, None, None, y.data_ptr(), None)
    assert st == 0
    assert np.all(host_bits(y) == 0x40E0)


def test_stream_read_checksum(ngq):
    n = 1 << 20
    g = np.random.default_rng(1)
    words = g.integers(0, 2 ** 32, size=n, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).to("cuda")
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
    ngq.ngq_stream_read(buf, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words)


@pytest.mark.parametrize("bits,cols", [(4, 32), (5, 48), (8, 32), (5, 32)])
def test_stream_tiles_reads_every_word_once(ngq, bits, cols):
    """The calibration stream reads each packed P0 word of its tiles once:
    the per-tile XOR checksums equal the host's (as a multiset: workgroups
    take tiles in an XCD-grouped order)."""
    K, N = 1088, 192  # 17 groups (a half pair at the end); whole tiles of 32 or 48 columns
    g = np.random.default_rng(bits + cols)
    nb = ngq.ngq_packed_bytes(K, N, bits)
    packed = g.integers(0, 256, size=nb, dtype=np.uint8)
    scales = (g.uniform(1e-3, 2e-2, size=(K // 64, N))).astype(np.float16).view(np.uint16)
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
    ngq.ngq_stream_tiles(dev_u8(packed), dev_scales(scales, False), K, N, bits, cols, sink)
    torch.cuda.synchronize()
    rows = K // (4 if bits == 8 else 8)
    p0 = packed[: rows * N * 4].view("<u4").reshape(rows, N)
    ntiles = (N + cols - 1) // cols
    want = sorted(int(np.bitwise_xor.reduce(p0[:, t * cols:(t + 1) * cols], axis=None)) for t in range(ntiles))
    got = sorted(int(v) for v in sink.cpu().numpy().view(np.uint32)[:ntiles])
    assert got == want
