"""Pins of the CPU oracle to things other than itself.

The pages print no worked example of the groupwise-int projection, so the
oracle is pinned to: hand-worked examples (tests/golden), exact rational
brute force, an independent numpy float64 evaluation, IEEE decoders from the
Python standard library, closed-form statistics and algebraic invariants.
Each pin is chosen so that a plausible slip in the oracle (wrong nibble order,
transposed layout, wrong group index, wrong offset or sign, rounding through
fp32, wrong SiLU) fails at least one test here.
"""
import bisect
import json
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import synthetic

HERE = os.path.dirname(os.path.abspath(__file__))
BIAS = {4: 8, 5: 16, 8: 128}


def load_cases():
    with open(os.path.join(HERE, "golden", "worked_examples.json")) as f:
        return json.load(f)["cases"]


def words_to_bytes(words):
    return np.array([int(w, 16) for w in words], dtype="<u4").view(np.uint8)


def case_x(case):
    K = case["K"]
    spec = case["x"]
    xs = np.zeros(K)
    if spec["kind"] == "ones":
        xs[:] = 1.0
    elif spec["kind"] == "indicator_below":
        xs[: spec["limit"]] = 1.0
    elif spec["kind"] == "ramp_below":
        xs[: spec["limit"]] = np.arange(spec["limit"])
    elif spec["kind"] == "ramp_from_one_below":
        xs[: spec["limit"]] = np.arange(1, spec["limit"] + 1)
    elif spec["kind"] == "ramp_from_one":
        xs[:] = np.arange(1, K + 1)
    else:
        raise ValueError(spec)
    # every value used is a small integer, exact in bf16
    return synthetic.f32_to_bf16_bits(xs.astype(np.float32)).reshape(1, K)


# ---- independent IEEE decoders and an exhaustive bf16 rounding ----------------

def f16_ref(h):
    return struct.unpack("<e", int(h).to_bytes(2, "little"))[0]


def bf16_ref(b):
    return struct.unpack("<f", (int(b) << 16).to_bytes(4, "little"))[0]


_BF16_TABLE = None


def bf16_table():
    """All finite non-negative bf16 values as exact Fractions, ascending."""
    global _BF16_TABLE
    if _BF16_TABLE is None:
        vals = []
        for b in range(0x0000, 0x7F80):  # +0 .. max finite
            vals.append((Fraction(bf16_ref(b)), b))
        vals.sort()
        _BF16_TABLE = ([v for v, _ in vals], [b for _, b in vals])
    return _BF16_TABLE


def rne_bf16_fraction(v: Fraction) -> int:
    """Brute-force round-to-nearest-even of an exact rational to bf16 bits."""
    sign = 0x8000 if v < 0 else 0
    a = -v if v < 0 else v
    vals, bits = bf16_table()
    i = bisect.bisect_left(vals, a)
    if i < len(vals) and vals[i] == a:
        return sign | bits[i]
    if i == len(vals):
        # beyond max finite: the midpoint to 2^128 rounds to infinity (even)
        top = vals[-1]
        mid = (top + Fraction(2) ** 128) / 2
        return sign | (0x7F80 if a >= mid else bits[-1])
    lo, hi = vals[i - 1], vals[i]
    dlo, dhi = a - lo, hi - a
    if dlo < dhi:
        return sign | bits[i - 1]
    if dhi < dlo:
        return sign | bits[i]
    return sign | (bits[i - 1] if bits[i - 1] % 2 == 0 else bits[i])


# ---- worked examples ----------------------------------------------------------

@pytest.mark.parametrize("case", load_cases(), ids=lambda c: c["name"])
def test_worked_example(oracle_lib, case):
    o = oracle_lib
    K, N, bits = case["K"], case["N"], case["bits"]
    packed = np.concatenate([words_to_bytes(case["p0_words"]), words_to_bytes(case["p1_words"])]) \
        if case["p1_words"] else words_to_bytes(case["p0_words"])
    assert packed.size == o.packed_bytes(K, N, bits)
    scales = np.array([int(s, 16) for s in case["scales"]], dtype=np.uint16).reshape(K // 64, N)
    x = case_x(case)
    y = o.gemm(x, packed, scales, K, N, bits, case["scale_bf16"])
    assert y[0].tolist() == case["y"]
    yb = o.round_bf16_array(y)
    assert [hex(v).upper().replace("0X", "0x") for v in yb[0]] == case["y_bf16"]
    if "twos_complement_y" in case:
        assert y[0].tolist() != case["twos_complement_y"]


def test_worked_example_codes(oracle_lib):
    """The codes the fixtures' notes spell out, read back one by one."""
    o = oracle_lib
    c = {x["name"]: x for x in load_cases()}
    w1 = words_to_bytes(c["W1a_int4_first16"]["p0_words"])
    assert [o.code_at(w1, 64, 1, 4, k, 0) for k in range(20)] == [k - 8 for k in range(16)] + [0] * 4
    w2 = np.concatenate([words_to_bytes(c["W2a_int5_first16"]["p0_words"]),
                         words_to_bytes(c["W2a_int5_first16"]["p1_words"])])
    assert [o.code_at(w2, 64, 1, 5, k, 0) for k in range(18)] == list(range(16)) + [-8, -8]
    w3 = words_to_bytes(c["W3a_int8_ones"]["p0_words"])
    assert [o.code_at(w3, 64, 1, 8, k, 0) for k in range(6)] == [0, 1, -1, -128, 0, 0]


# ---- layout: round trips and single-field pins ----------------------------------

@pytest.mark.parametrize("bits", [4, 5, 8])
def test_pack_unpack_roundtrip(oracle_lib, bits):
    g = np.random.default_rng(11 + bits)
    K, N = 192, 20
    codes = synthetic.draw_codes(K, N, bits, g)
    packed = oracle_lib.pack(codes, bits)
    assert packed.size == oracle_lib.packed_bytes(K, N, bits)
    assert np.array_equal(oracle_lib.unpack(packed, K, N, bits), codes)
    # unpack then pack is the identity on arbitrary words
    words = g.integers(0, 256, size=packed.size, dtype=np.uint8)
    assert np.array_equal(oracle_lib.pack(oracle_lib.unpack(words, K, N, bits), bits), words)


@pytest.mark.parametrize("bits,k,n", [(4, 0, 0), (4, 7, 3), (4, 9, 1), (4, 63, 2),
                                      (5, 0, 0), (5, 4, 1), (5, 31, 3), (5, 33, 2),
                                      (8, 0, 0), (8, 3, 1), (8, 6, 2)])
def test_single_code_lands_in_its_field(oracle_lib, bits, k, n):
    """All codes zero except one at (k, n) set to the most negative value; the
    packed bytes must differ from the all-zero packing only in that field."""
    K, N = 64, 4
    zero = oracle_lib.pack(np.zeros((K, N), np.int8), bits)
    codes = np.zeros((K, N), np.int8)
    codes[k, n] = -(1 << (bits - 1))
    one = oracle_lib.pack(codes, bits)
    diff = np.flatnonzero(zero != one)
    z32 = zero.view("<u4")
    o32 = one.view("<u4")
    if bits == 4:
        wi = (k // 8) * N + n
        # u goes from 8 (0b1000) to 0: only bit 3 of nibble k%8 changes
        assert list(np.flatnonzero(z32 != o32)) == [wi]
        assert z32[wi] ^ o32[wi] == 1 << (4 * (k % 8) + 3)
    elif bits == 5:
        # u goes from 16 (0b10000) to 0: only the high-plane bit changes
        wi = (K // 8) * N + (k // 32) * N + n
        assert list(np.flatnonzero(z32 != o32)) == [wi]
        assert z32[wi] ^ o32[wi] == 1 << (k % 32)
    else:
        wi = (k // 4) * N + n
        assert list(np.flatnonzero(z32 != o32)) == [wi]
        assert z32[wi] ^ o32[wi] == 1 << (8 * (k % 4) + 7)
    assert diff.size == 1


def test_pack_rejects_out_of_range(oracle_lib):
    for bits, bad in [(4, 8), (4, -9), (5, 16), (5, -17)]:
        codes = np.zeros((64, 2), np.int8)
        codes[5, 1] = bad
        with pytest.raises(oracle_lib.OracleError):
            oracle_lib.pack(codes, bits)
    with pytest.raises(oracle_lib.OracleError):
        oracle_lib.pack(np.zeros((32, 2), np.int8), 4)  # K not a multiple of 64


# ---- IEEE decoding and rounding -------------------------------------------------

def test_f16_decode_exhaustive(oracle_lib):
    lib = oracle_lib.lib()
    for h in range(0x10000):
        ref = f16_ref(h)
        got = lib.oracle_f16_to_f64(h)
        if math.isnan(ref):
            assert math.isnan(got)
        else:
            assert got == ref and math.copysign(1, got) == math.copysign(1, ref)


def test_bf16_decode_exhaustive(oracle_lib):
    lib = oracle_lib.lib()
    for b in range(0x10000):
        ref = bf16_ref(b)
        got = lib.oracle_bf16_to_f64(b)
        if math.isnan(ref):
            assert math.isnan(got)
        else:
            assert got == ref and math.copysign(1, got) == math.copysign(1, ref)


@pytest.mark.parametrize("v,bits", [
    (1.0, 0x3F80), (-1.0, 0xBF80), (0.0, 0x0000), (-0.0, 0x8000),
    (1.0 + 2.0 ** -8, 0x3F80),           # exact tie -> even (down)
    (1.0 + 3 * 2.0 ** -8, 0x3F82),       # exact tie -> even (up)
    (1.0 + 2.0 ** -8 + 2.0 ** -40, 0x3F81),  # just above the tie: a detour through fp32 would lose this
    (3.0e38 * 10, 0x7F80), (-1e39, 0xFF80),
    (2.0 ** -133, 0x0001), (2.0 ** -134, 0x0000), (3 * 2.0 ** -134, 0x0002),
    (float("inf"), 0x7F80),
])
def test_round_bf16_pins(oracle_lib, v, bits):
    assert oracle_lib.round_bf16(v) == bits


def test_round_bf16_matches_brute_force(oracle_lib):
    g = np.random.default_rng(5)
    vals = np.concatenate([
        g.standard_normal(3000) * 10.0 ** g.integers(-40, 38, 3000),
        g.standard_normal(500) * 2.0 ** -130,           # subnormal range
        (1 + (2 * g.integers(0, 128, 300) + 1) * 2.0 ** -8) * 2.0 ** g.integers(-20, 20, 300),  # ties
    ])
    for v in vals:
        assert oracle_lib.round_bf16(float(v)) == rne_bf16_fraction(Fraction(float(v))), v


# ---- the projection -------------------------------------------------------------

def exact_projection(codes, scale_bits, x_bits, scale_bf16):
    """Brute force with exact rationals: y = sum_k x*c*s, then RNE to bf16."""
    K, N = codes.shape
    T = x_bits.shape[0]
    dec = bf16_ref if scale_bf16 else f16_ref
    S = [[Fraction(dec(scale_bits[g, n])) for n in range(N)] for g in range(K // 64)]
    X = [[Fraction(bf16_ref(x_bits[t, k])) for k in range(K)] for t in range(T)]
    out = np.zeros((T, N), np.uint16)
    exact = [[None] * N for _ in range(T)]
    for t in range(T):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += X[t][k] * int(codes[k, n]) * S[k // 64][n]
            exact[t][n] = acc
            out[t, n] = rne_bf16_fraction(acc)
    return exact, out


@pytest.mark.parametrize("bits,scale_bf16,K,N,T", [(4, False, 128, 6, 2), (5, True, 64, 5, 3),
                                                    (8, False, 128, 3, 1), (4, True, 192, 4, 2)])
def test_projection_brute_force_fractions(oracle_lib, bits, scale_bf16, K, N, T):
    w = synthetic.Workload("t", K, N, bits, scale_bf16, 1e-3, 2e-2, 90)
    codes, scales, x = synthetic.make_inputs(w, T, seed=3)
    packed = oracle_lib.pack(codes, bits)
    y64 = oracle_lib.gemm(x, packed, scales, K, N, bits, scale_bf16)
    exact, y16 = exact_projection(codes, scales, x, scale_bf16)
    assert np.array_equal(oracle_lib.round_bf16_array(y64), y16)
    for t in range(T):
        for n in range(N):
            # fp64 sum of exact products: error far below the output rounding
            assert abs(Fraction(y64[t, n]) - exact[t][n]) <= Fraction(1, 2 ** 40) * (1 + abs(exact[t][n]))


def exact_magnitudes(codes, scale_bits, x_bits, scale_bf16):
    """Brute force with exact rationals of the two magnitude sums the oracle
    returns beside y: A = sum_k |x c s| and B = sum_k |x| s, per output."""
    K, N = codes.shape
    T = x_bits.shape[0]
    dec = bf16_ref if scale_bf16 else f16_ref
    S = [[Fraction(dec(scale_bits[g, n])) for n in range(N)] for g in range(K // 64)]
    X = [[Fraction(bf16_ref(x_bits[t, k])) for k in range(K)] for t in range(T)]
    A = [[sum(abs(X[t][k] * int(codes[k, n]) * S[k // 64][n]) for k in range(K)) for n in range(N)]
         for t in range(T)]
    B = [[sum(abs(X[t][k]) * S[k // 64][n] for k in range(K)) for n in range(N)] for t in range(T)]
    return A, B


@pytest.mark.parametrize("bits,scale_bf16,K,N,T", [(4, False, 192, 5, 2), (5, True, 128, 4, 3),
                                                    (8, False, 128, 3, 2)])
def test_magnitude_sums_brute_force_fractions(oracle_lib, bits, scale_bf16, K, N, T):
    """The magnitudes sum|x w| and sum|x| s size the tie exemption of the parity
    gate, so they are pinned like y: against exact rational sums.  Every group
    has its own scales (U[1e-3, 2e-2]), so a wrong group index, a dropped or
    squared scale, or |x| c s in place of |x| s changes them by far more than
    the fp64 summation error (at most K 2^-53 relative)."""
    w = synthetic.Workload("t", K, N, bits, scale_bf16, 1e-3, 2e-2, 91)
    codes, scales, x = synthetic.make_inputs(w, T, seed=4)
    assert len({int(v) for v in scales[:, 0]}) == K // 64  # distinct per group
    y64, axw, axs = oracle_lib.gemm(x, oracle_lib.pack(codes, bits), scales, K, N, bits, scale_bf16,
                                    with_bounds=True)
    A, B = exact_magnitudes(codes, scales, x, scale_bf16)
    tol = Fraction(K, 2 ** 52)
    for t in range(T):
        for n in range(N):
            assert abs(Fraction(axw[t, n]) - A[t][n]) <= tol * A[t][n], (t, n)
            assert abs(Fraction(axs[t, n]) - B[t][n]) <= tol * B[t][n], (t, n)
            # triangle inequality and |c| <= 2^(bits-1): |y| <= A <= 2^(bits-1) B
            assert abs(y64[t, n]) <= axw[t, n] <= 2 ** (bits - 1) * axs[t, n]


def test_magnitude_sums_worked_example(oracle_lib):
    """Hand-worked: K=64, one column, codes k-8 on k<16 and 0 elsewhere
    (worked example W1's words), s = 0.5, x = 1 on k<16:
    sum|x c s| = 0.5 (8+7+...+1 + 0+1+...+7) = 0.5 * 64 = 32,
    sum|x| s = 16 * 0.5 = 8."""
    case = next(c for c in load_cases() if c["bits"] == 4 and c["x"]["kind"] == "indicator_below")
    packed = words_to_bytes(case["p0_words"])
    scales = np.array([int(s, 16) for s in case["scales"]], dtype=np.uint16).reshape(1, 1)
    assert scales[0, 0] == 0x3800
    y, axw, axs = oracle_lib.gemm(case_x(case), packed, scales, 64, 1, 4, False, with_bounds=True)
    assert (y[0, 0], axw[0, 0], axs[0, 0]) == (-4.0, 32.0, 8.0)


def test_residual_worked_example(oracle_lib):
    """Hand-worked: worked example W1 (y = -4.0, sum|x w| = 32) plus a
    residual of bf16 0x3FC0 = 1.5 gives y = -2.5 and the bound 33.5; the
    residual 0xBE80 = -0.25 gives -4.25 and 32.25.  (Read as fp16, 0x3FC0 would
    be 1.9375: a decode slip shows.)"""
    case = next(c for c in load_cases() if c["bits"] == 4 and c["x"]["kind"] == "indicator_below")
    packed = words_to_bytes(case["p0_words"])
    scales = np.array([int(s, 16) for s in case["scales"]], dtype=np.uint16).reshape(1, 1)
    y, axw, _ = oracle_lib.gemm(case_x(case), packed, scales, 64, 1, 4, False, with_bounds=True)
    for r_bits, want, bound in ((0x3FC0, -2.5, 33.5), (0xBE80, -4.25, 32.25), (0x0000, -4.0, 32.0)):
        yr, ar = oracle_lib.add_residual(y, np.array([[r_bits]], dtype=np.uint16), axw)
        assert (yr[0, 0], ar[0, 0]) == (want, bound), hex(r_bits)
    assert oracle_lib.add_residual(y, np.array([[0x3FC0]], dtype=np.uint16))[0, 0] == -2.5


def test_residual_zero_weights_give_the_residual(oracle_lib):
    """With every code 0 the projection is exactly 0, so y + r is r itself,
    decoded as bf16 (checked against the standard library's float decode)."""
    g = np.random.default_rng(11)
    T, K, N = 3, 128, 8
    codes = np.zeros((K, N), dtype=np.int8)
    scales = synthetic.draw_scales(K, N, 1e-3, 2e-2, False, g)
    x = synthetic.f32_to_bf16_bits(g.standard_normal((T, K)).astype(np.float32))
    r = synthetic.f32_to_bf16_bits(g.standard_normal((T, N)).astype(np.float32))
    y = oracle_lib.gemm(x, oracle_lib.pack(codes, 4), scales, K, N, 4, False)
    yr = oracle_lib.add_residual(y, r)
    assert all(yr[t, n] == bf16_ref(r[t, n]) for t in range(T) for n in range(N))


def numpy_projection(codes, scale_bits, x_bits, scale_bf16):
    K, N = codes.shape
    if scale_bf16:
        s = (scale_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    else:
        s = scale_bits.view(np.float16).astype(np.float64)
    w = codes.astype(np.float64) * np.repeat(s, 64, axis=0)
    x = (x_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x @ w


@pytest.mark.parametrize("name", ["qk", "gv"])
def test_projection_matches_numpy_float64(oracle_lib, name):
    """numpy's matmul on numpy-decoded operands, against the oracle reading the
    packed bytes: pins unpack, scale indexing, decoding and the sum together."""
    w = synthetic.WORKLOADS[name]
    K, N, T = 1024, 96, 8
    codes, scales, x = synthetic.make_inputs(w, T, seed=1, K=K, N=N)
    packed = oracle_lib.pack(codes, w.bits)
    y = oracle_lib.gemm(x, packed, scales, K, N, w.bits, w.scale_bf16)
    ref = numpy_projection(codes, scales, x, w.scale_bf16)
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_dequant_is_exact_product(oracle_lib):
    w = synthetic.WORKLOADS["gv"]
    codes, scales, _ = synthetic.make_inputs(w, 1, seed=2, K=128, N=10)
    packed = oracle_lib.pack(codes, 5)
    deq = oracle_lib.dequant(packed, scales, 128, 10, 5, True)
    for k in range(0, 128, 7):
        for n in range(10):
            assert Fraction(deq[k, n]) == int(codes[k, n]) * Fraction(bf16_ref(scales[k // 64, n]))


def test_identity_scales_integer_x_exact(oracle_lib):
    g = np.random.default_rng(4)
    K, N, T = 256, 12, 3
    codes = synthetic.draw_codes(K, N, 4, g)
    scales = np.full((K // 64, N), 0x3C00, np.uint16)  # fp16 1.0
    xi = g.integers(-3, 4, size=(T, K))
    x = synthetic.f32_to_bf16_bits(xi.astype(np.float32))
    y = oracle_lib.gemm(x, oracle_lib.pack(codes, 4), scales, K, N, 4, False)
    assert np.array_equal(y, xi.astype(np.int64) @ codes.astype(np.int64))


def test_thread_count_does_not_change_result(oracle_lib):
    w = synthetic.WORKLOADS["qk"]
    codes, scales, x = synthetic.make_inputs(w, 4, seed=7, K=512, N=64)
    packed = oracle_lib.pack(codes, 4)
    a = oracle_lib.gemm(x, packed, scales, 512, 64, 4, False, nthreads=1)
    b = oracle_lib.gemm(x, packed, scales, 512, 64, 4, False, nthreads=5)
    cols = np.array([63, 0, 17, 17, 5], np.int32)
    c = oracle_lib.gemm(x, packed, scales, 512, 64, 4, False, cols=cols, nthreads=3)
    assert np.array_equal(a, b)
    assert np.array_equal(c, a[:, cols])


def test_empty_shapes(oracle_lib):
    y = oracle_lib.gemm(np.zeros((2, 0), np.uint16), np.zeros(0, np.uint8), np.zeros((0, 3), np.uint16),
                        0, 3, 4, False)
    assert y.shape == (2, 3) and np.all(y == 0.0)  # K=0: the empty sum
    y = oracle_lib.gemm(np.zeros((0, 64), np.uint16), np.zeros(64 * 3 // 2, np.uint8),
                        np.zeros((1, 3), np.uint16), 64, 3, 4, False)
    assert y.shape == (0, 3)


@pytest.mark.parametrize("name,expected_rms", [("qk", 3.930), ("gv", 3.919)])
def test_output_rms_closed_form(oracle_lib, name, expected_rms):
    """E[y^2] = K E[x^2] E[c^2] E[s^2] for independent zero-mean x and codes.
    int4 uniform on [-8,7]: E[c^2] = 21.5; int5 on [-16,15]: 85.5;
    E[s^2] = (a^2 + ab + b^2)/3 for s ~ U[a, b]."""
    w = synthetic.WORKLOADS[name]
    lo, hi = w.scale_lo, w.scale_hi
    ec2 = {4: 21.5, 5: 85.5}[w.bits]
    es2 = (lo * lo + lo * hi + hi * hi) / 3
    assert abs(math.sqrt(w.K * ec2 * es2) - expected_rms) < 2e-3
    codes, scales, x = synthetic.make_inputs(w, 8, seed=0, N=256)
    y = oracle_lib.gemm(x, oracle_lib.pack(codes, w.bits), scales, w.K, 256, w.bits, w.scale_bf16)
    rms = math.sqrt(np.mean(y ** 2))
    assert abs(rms / expected_rms - 1) < 0.04  # 2048 samples: ~1.6% standard error


# ---- SwiGLU and the stack rescale ---------------------------------------------------

def test_swiglu_closed_forms(oracle_lib):
    g = np.array([0.0, math.log(3.0), -math.log(3.0), 40.0, -800.0, 2.5])
    u = np.array([5.0, 2.0, 2.0, 1.5, 3.0, 1.0])
    h = oracle_lib.swiglu(g, u)
    assert h[0] == 0.0
    assert abs(h[1] - u[1] * 0.75 * g[1]) < 1e-15          # 1 + e^-ln3 = 4/3
    assert abs(h[2] - u[2] * 0.25 * g[2]) < 1e-15          # 1 + e^ln3 = 4
    assert abs(h[3] - 40.0 * 1.5) < 1e-12                   # SiLU(g) -> g for large g
    assert h[4] == 0.0 or abs(h[4]) < 1e-300                # SiLU(g) -> 0 for very negative g
    # SiLU(g) - SiLU(-g) = g
    hp = oracle_lib.swiglu(np.array([2.5]), np.array([1.0]))[0]
    hm = oracle_lib.swiglu(np.array([-2.5]), np.array([1.0]))[0]
    assert abs((hp - hm) - 2.5) < 1e-15
    assert hp == h[5]


def test_rms_rescale(oracle_lib):
    z = synthetic.f32_to_bf16_bits(np.array([[3.0, 4.0, 3.0, 4.0], [2.0, 2.0, 2.0, 2.0]], np.float32))
    out = oracle_lib.rms_rescale(z)
    r = math.sqrt(12.5)
    assert out[0, 0] == oracle_lib.round_bf16(3 / r) and out[0, 1] == oracle_lib.round_bf16(4 / r)
    assert np.all(out[1] == 0x3F80)


def exact_rms_rescale_bits(z_bits):
    """Brute force: the quotient z / sqrt(mean z^2) to 80 significant digits
    (Decimal's square root is correctly rounded, and exact when the root is a
    terminating decimal), then the exhaustive bf16 rounding of that value."""
    import decimal

    ctx = decimal.Context(prec=80)
    out = np.zeros_like(z_bits)
    for t in range(z_bits.shape[0]):
        vals = [Fraction(bf16_ref(b)) for b in z_bits[t]]
        ms = sum(v * v for v in vals) / len(vals)
        if ms == 0:
            continue
        r = ctx.sqrt(ctx.divide(decimal.Decimal(ms.numerator), decimal.Decimal(ms.denominator)))
        for n, v in enumerate(vals):
            q = ctx.divide(decimal.Decimal(v.numerator), decimal.Decimal(v.denominator))
            out[t, n] = rne_bf16_fraction(Fraction(ctx.divide(q, r)))
    return out


def test_rms_rescale_brute_force(oracle_lib):
    g = np.random.default_rng(11)
    rows = [g.standard_normal(37) * 10.0 ** e for e in (-38, -5, 0, 3, 30)]
    rows.append(np.where(np.arange(37) == 5, 1e-3, 1e-42))  # one large entry, the rest subnormal
    z = synthetic.f32_to_bf16_bits(np.array(rows, np.float32))
    assert np.array_equal(oracle_lib.rms_rescale(z), exact_rms_rescale_bits(z))


def test_rms_rescale_scale_invariant_and_zero_row(oracle_lib):
    g = np.random.default_rng(12)
    z = synthetic.f32_to_bf16_bits(g.standard_normal((3, 512)).astype(np.float32))
    base = oracle_lib.rms_rescale(z)
    for j in (-20, -1, 1, 7):
        zs = synthetic.f32_to_bf16_bits((bf16_bits_f32(z) * np.float32(2.0 ** j)).astype(np.float32))
        assert np.array_equal(oracle_lib.rms_rescale(zs), base)  # power-of-two scaling cancels exactly
    # a row with zero mean square: zeros; the other rows are unaffected
    z[1] = 0
    out = oracle_lib.rms_rescale(z)
    assert np.all(out[1] == 0) and np.array_equal(out[[0, 2]], base[[0, 2]])
    # unit mean square up to the output rounding (relative half-ulp 2^-8 per element)
    v = bf16_bits_f32(out[[0, 2]]).astype(np.float64)
    assert np.all(np.abs(np.mean(v ** 2, axis=1) - 1.0) < 2.0 ** -7)


def bf16_bits_f32(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)
