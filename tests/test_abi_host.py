"""Host-side checks of libngq that need no GPU: the library loads, exports
every symbol the header declares, packs byte-identically to the oracle, and
rejects bad arguments with the documented status before any HIP call."""
import os
import re
import subprocess

import numpy as np
import pytest

import synthetic

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ngq.h")


@pytest.fixture(scope="module")
def ngq():
    import groupwise_int_weight_amd as g

    if not os.path.exists(g.LIB_PATH):
        from groupwise_int_weight_amd import build

        build.build()
    g.lib()
    return g


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ngq_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = header_functions()
    for required in ["ngq_pack", "ngq_gemm", "ngq_swiglu_gemm", "ngq_multi_gemm", "ngq_gemm_splitk", "ngq_gemm_rescale",
                     "ngq_gemm_residual_rescale", "ngq_packed_bytes",
                     "ngq_scale_bytes", "ngq_unpack_codes", "ngq_dequant_f32", "ngq_rms_rescale", "ngq_strerror"]:
        assert required in names


def test_library_exports_every_declared_symbol(ngq):
    names = header_functions()
    out = subprocess.run(["nm", "-D", "--defined-only", ngq.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT\s+(ngq_\w+)$", out, flags=re.M))
    assert set(names) <= exported, set(names) - exported
    # the binding knows the signature of every declared function, and nothing more
    assert set(ngq.SIGNATURES) == set(names)
    for n in names:
        assert getattr(ngq.lib(), n) is not None


def test_version_and_strerror(ngq):
    assert ngq.ngq_version() >= 1
    msgs = {s: ngq.ngq_strerror(s) for s in [0, -1, -2, -3, -4, -5]}
    assert len(set(msgs.values())) == 6
    assert ngq.ngq_strerror(-99) == "unknown status"


@pytest.mark.parametrize("bits", [4, 5, 8])
@pytest.mark.parametrize("K,N", [(64, 4), (192, 12), (320, 100), (1024, 36)])
def test_pack_matches_oracle_bytes(ngq, oracle_lib, bits, K, N):
    g = np.random.default_rng(K * 7 + N + bits)
    codes = synthetic.draw_codes(K, N, bits, g)
    mine = ngq.ngq_pack(codes, bits)
    ref = oracle_lib.pack(codes, bits)
    assert mine.size == ref.size == ngq.ngq_packed_bytes(K, N, bits)
    assert np.array_equal(mine, ref)


def test_pack_extreme_codes_match_oracle(ngq, oracle_lib):
    for bits in (4, 5, 8):
        lo, hi = synthetic.code_range(bits)
        codes = np.tile(np.array([lo, hi, 0, -1], np.int8), (128, 2))
        assert np.array_equal(ngq.ngq_pack(codes, bits), oracle_lib.pack(codes, bits))


def test_sizes(ngq):
    assert ngq.ngq_packed_bytes(5120, 8192, 4) == 5120 * 8192 // 2
    assert ngq.ngq_packed_bytes(5120, 12288, 5) == 5120 * 12288 // 2 + 5120 * 12288 // 8
    assert ngq.ngq_packed_bytes(5120, 8192, 8) == 5120 * 8192
    assert ngq.ngq_packed_bytes(5120, 12288, 5 | ngq.NGQ_SCALE_BF16) == ngq.ngq_packed_bytes(5120, 12288, 5)
    assert ngq.ngq_scale_bytes(5120, 8192, 4) == 80 * 8192 * 2
    assert ngq.ngq_packed_bytes(100, 8, 4) == 0     # K % 64
    assert ngq.ngq_packed_bytes(64, 6, 4) == 0      # N % 4
    assert ngq.ngq_packed_bytes(64, 8, 6) == 0      # bits
    assert ngq.ngq_packed_bytes(64, 8, 4, 32) == 0  # group
    assert ngq.ngq_packed_bytes(0, 8, 4) == 0


def test_pack_errors(ngq):
    L = ngq.lib()
    codes = np.zeros((64, 4), np.int8)
    out = np.zeros(1024, np.uint8)
    assert L.ngq_pack(64, 4, 6, 64, codes.ctypes.data, out.ctypes.data) == ngq.NGQ_ERR_UNSUPPORTED
    assert L.ngq_pack(64, 4, 4, 128, codes.ctypes.data, out.ctypes.data) == ngq.NGQ_ERR_UNSUPPORTED
    assert L.ngq_pack(32, 4, 4, 64, codes.ctypes.data, out.ctypes.data) == ngq.NGQ_ERR_SHAPE
    assert L.ngq_pack(64, 4, 4, 64, None, out.ctypes.data) == ngq.NGQ_ERR_ARG
    bad = codes.copy()
    bad[3, 2] = 8
    assert L.ngq_pack(64, 4, 4, 64, bad.ctypes.data, out.ctypes.data) == ngq.NGQ_ERR_ARG
    bad[3, 2] = -17
    assert L.ngq_pack(64, 4, 5, 64, bad.ctypes.data, out.ctypes.data) == ngq.NGQ_ERR_ARG


# Fake, never-dereferenced device addresses: every call below fails validation,
# which happens before any HIP call, so no GPU is needed.
X, W, S, Y = 0x100000, 0x200000, 0x300000, 0x400000


@pytest.mark.parametrize("args,status", [
    ((16385, 64, 4, 4, 64, X, W, S, Y), -2),    # T > 16384
    ((-1, 64, 4, 4, 64, X, W, S, Y), -2),       # T < 0
    ((1, 100, 4, 4, 64, X, W, S, Y), -2),       # K % 64
    ((1, 64, 6, 4, 64, X, W, S, Y), -2),        # N % 4
    ((1, 64, 4, 7, 64, X, W, S, Y), -3),        # bits
    ((1, 64, 4, 4 | 0x200, 64, X, W, S, Y), -3),  # unknown flag
    ((1, 64, 4, 4, 128, X, W, S, Y), -3),       # group
    ((1, 64, 4, 4, 64, X, W, S, None), -1),     # null y
    ((1, 64, 4, 4, 64, None, W, S, Y), -1),     # null x
    ((1, 64, 4, 4, 64, X, None, S, Y), -1),     # null wq
    ((1, 64, 4, 4, 64, X, W, None, Y), -1),     # null scales
    ((1, 64, 4, 4, 64, X + 8, W, S, Y), -4),    # misaligned x
    ((1, 64, 4, 5, 64, X, W + 4, S, Y), -4),    # misaligned wq
    ((1, 64, 4, 4, 64, X, W, S, Y + 2), -4),    # misaligned y
    ((1, 64, 4, 4, 64, X, W, S, X), -1),        # y overlaps x
    ((2, 64, 64, 4, 64, X, W, S, W + 16), -1),  # y overlaps wq
    ((1, 1 << 24, 512, 4, 64, X, W, S, Y), -3),  # packed weights >= 2 GiB
    ((64, 64, 4, 4, 64, X, W, S, Y + 2), -4),   # misaligned y, T = 64
    ((40, 64, 64, 4, 64, X, W, S, X + 64), -1),  # y overlaps x, T = 40
])
def test_gemm_rejects_bad_arguments(ngq, args, status):
    assert ngq.lib().ngq_gemm(*args, None) == status


def test_swiglu_rejects_bad_arguments(ngq):
    L = ngq.lib()
    assert L.ngq_swiglu_gemm(16385, 64, 4, 4, 64, X, W, S, Y, None) == -2
    assert L.ngq_swiglu_gemm(1, 64, 6, 4, 64, X, W, S, Y, None) == -2
    assert L.ngq_swiglu_gemm(1, 64, 4, 4, 64, X, W, S, None, None) == -1
    # the up half makes wq 2 N_ff columns wide: h must not overlap it either
    assert L.ngq_swiglu_gemm(1, 64, 8, 4, 64, X, W, S, W + 400, None) == -1


def test_empty_calls_are_no_ops(ngq):
    """T == 0 or N == 0 returns OK without touching any pointer or the GPU."""
    L = ngq.lib()
    assert L.ngq_gemm(0, 64, 4, 4, 64, None, None, None, None, None) == 0
    assert L.ngq_gemm(3, 64, 0, 4, 64, None, None, None, None, None) == 0
    assert L.ngq_swiglu_gemm(0, 64, 4, 4, 64, None, None, None, None, None) == 0
    assert L.ngq_unpack_codes(0, 4, 4, 64, None, None, None) == 0
    assert L.ngq_dequant_f32(64, 0, 4, 64, None, None, None, None) == 0
    assert L.ngq_stream_read(None, 0, None, None) == 0


@pytest.mark.parametrize("args,status", [
    ((-1, 64, X, Y), -2),            # T < 0
    ((1, -4, X, Y), -2),             # N < 0
    ((1, (1 << 24) + 1, X, Y), -2),  # N too large
    ((65536, 4, X, Y), -2),          # T too large
    ((1, 64, None, Y), -1),          # null z
    ((1, 64, X, None), -1),          # null x
    ((1, 64, X + 2, Y), -4),         # misaligned z
    ((1, 64, X, Y + 8), -4),         # misaligned x
    ((2, 64, X, X + 64), -1),        # partial overlap (in place, x == z, is allowed)
    ((65535, 1 << 15, X, Y), -3),    # block >= 2 GiB
])
def test_rms_rescale_rejects_bad_arguments(ngq, args, status):
    assert ngq.lib().ngq_rms_rescale(*args, None) == status


def test_rms_rescale_empty_is_no_op(ngq):
    L = ngq.lib()
    assert L.ngq_rms_rescale(0, 64, None, None, None) == 0
    assert L.ngq_rms_rescale(3, 0, None, None, None) == 0


def multi_call(ngq, T, K, projs, x=X, nproj=None, group=64):
    arr = (ngq.NgqProj * max(1, len(projs)))(*[ngq.NgqProj(*p) for p in projs])
    return ngq.lib().ngq_multi_gemm(T, K, group, x, arr, len(projs) if nproj is None else nproj, None)


# (bits, n, swiglu, reserved, wq, scales, y)
P_OK = (4, 64, 0, 0, W, S, Y)


@pytest.mark.parametrize("T,K,projs,nproj,status", [
    (1, 64, [P_OK], 0, -1),                                        # no projection
    (1, 64, [P_OK] * 4, 5, -1),                                    # more than NGQ_MAX_PROJ
    (9, 64, [P_OK], None, -2),                                     # T > 8
    (1, 100, [P_OK], None, -2),                                    # K % 64
    (1, 64, [(4, 66, 0, 0, W, S, Y)], None, -2),                   # n % 4
    (1, 64, [(7, 64, 0, 0, W, S, Y)], None, -3),                   # bits
    (1, 64, [(4, 64, 2, 0, W, S, Y)], None, -1),                   # swiglu flag
    (1, 64, [(4, 64, 0, 1, W, S, Y)], None, -1),                   # reserved field
    (1, 64, [(4, 64, 0, 0, W, S, None)], None, -1),                # null output
    (1, 64, [(4, 64, 0, 0, None, S, Y)], None, -1),                # null wq
    (1, 64, [(4, 64, 0, 0, W, S, Y + 2)], None, -4),               # misaligned output
    (1, 64, [(4, 64, 0, 0, W, S, X)], None, -1),                   # output overlaps x
    (1, 64, [P_OK, (5, 64, 0, 0, W + 4096, S, W + 16)], None, -1),  # output overlaps another wq
    (1, 64, [P_OK, (4, 64, 0, 0, W, S, Y + 64)], None, -1),        # two outputs overlap
    (8, 65536, [(5, 64, 1, 0, 0x1000000, 0x2000000, 0x3000000)], None, -3),  # int5 SwiGLU: X does not fit in LDS
])
def test_multi_rejects_bad_arguments(ngq, T, K, projs, nproj, status):
    assert multi_call(ngq, T, K, projs, nproj=nproj) == status


def test_multi_tile_kernels_have_no_lds_limit(ngq):
    """With int4 / plain int5 / plain int8 projections the fused call runs one
    workgroup per tile with X per pair: a K whose X exceeds the persistent
    kernel's LDS is served (no device here: the launch reports the missing
    device); with an int5 SwiGLU projection it is refused."""
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("host-only check: with a device these fake pointers would be launched")
    K = 131072  # X alone is 256 KB at T = 1
    p4 = (4, 64, 0, 0, 0x1000000, 0x2000000, 0x3000000)
    p5 = (5, 64, 0, 0, 0x4000000, 0x5000000, 0x3001000)
    p5s = (5, 64, 1, 0, 0x4000000, 0x5000000, 0x3001000)
    for T in (1, 2, 8):
        assert multi_call(ngq, T, K, [p4, p5]) == ngq.NGQ_ERR_HIP, T
        assert multi_call(ngq, T, K, [p4, p5s]) == ngq.NGQ_ERR_UNSUPPORTED, T


def test_multi_empty_calls_are_no_ops(ngq):
    """T == 0, or every projection zero-width, returns OK without a HIP call."""
    assert multi_call(ngq, 0, 64, [P_OK], x=None) == 0
    assert multi_call(ngq, 3, 64, [(4, 0, 0, 0, W, S, Y), (5, 0, 1, 0, W, S, Y)]) == 0
    assert ngq.lib().ngq_multi_gemm(1, 64, 64, X, None, 1, None) == -1


# Long-K calls (the down projection: 44.5 MB of packed weights) get addresses
# 256 MB apart, so that no buffer overlaps another unless a case says so and
# each case fails for the reason it names.
XL, WL, SL, YL, WSL, XNL, RL = (i << 28 for i in range(1, 8))
DOWN = (17408, 5120, 4, 64)


@pytest.mark.parametrize("args,status", [
    ((9, *DOWN, XL, WL, SL, YL, WSL, 1 << 21), -2),                   # T > 8
    ((8, 17400, 5120, 4, 64, XL, WL, SL, YL, WSL, 1 << 21), -2),      # K % 64
    ((8, 17408, 5120, 7, 64, XL, WL, SL, YL, WSL, 1 << 21), -3),      # bits
    ((8, *DOWN, XL, WL, SL, YL, None, 1 << 21), -1),                  # null workspace
    ((8, *DOWN, XL, WL, SL, YL, WSL + 8, 1 << 21), -4),               # misaligned workspace
    ((8, *DOWN, XL, WL, SL, YL, WSL, 1 << 16), -1),                   # workspace too small
    ((8, *DOWN, XL, WL, SL, YL, YL + 64, 1 << 21), -1),               # workspace overlaps y
    ((8, *DOWN, XL, WL, SL, XL, WSL, 1 << 21), -1),                   # y overlaps x
    ((8, *DOWN, XL, WL, SL, WL + 4096, WSL, 1 << 21), -1),            # y overlaps wq
    ((8, *DOWN, XL, WL, SL, YL, XL + 64, 1 << 21), -1),               # workspace overlaps x
])
def test_splitk_rejects_bad_arguments(ngq, args, status):
    assert ngq.lib().ngq_gemm_splitk(*args, None) == status


def test_splitk_workspace_and_empty_calls(ngq):
    L = ngq.lib()
    # fp32 partials of 8 slices at 8 tokens
    assert ngq.ngq_splitk_workspace_bytes(17408, 5120, 4) == 8 * 8 * 5120 * 4
    assert ngq.ngq_splitk_workspace_bytes(17408, 5122, 4) == 0
    assert ngq.ngq_splitk_workspace_bytes(100, 5120, 4) == 0
    assert L.ngq_gemm_splitk(0, 17408, 5120, 4, 64, None, None, None, None, None, 0, None) == 0


@pytest.mark.parametrize("args,status", [
    ((8, *DOWN, XL, WL, SL, YL, None, WSL, 1 << 21), -1),             # null x_next
    ((9, *DOWN, XL, WL, SL, YL, XNL, WSL, 1 << 21), -2),              # T > 8
    ((8, *DOWN, XL, WL, SL, YL, XNL + 8, WSL, 1 << 21), -4),          # misaligned x_next
    ((8, *DOWN, XL, WL, SL, YL, YL + 64, WSL, 1 << 21), -1),          # x_next overlaps y
    ((8, *DOWN, XL, WL, SL, YL, XL, WSL, 1 << 21), -1),               # x_next overlaps x
    ((8, *DOWN, XL, WL, SL, YL, WL + 4096, WSL, 1 << 21), -1),        # x_next overlaps wq
    ((8, *DOWN, XL, WL, SL, YL, WSL + 0x10000, WSL, 1 << 21), -1),    # x_next overlaps the workspace
    ((1, *DOWN, XL, WL, SL, YL, XNL, WSL, 1 << 15), -1),              # workspace too small (split at T = 1)
    ((8, *DOWN, XL, WL, SL, YL, XNL, None, 1 << 21), -1),             # null workspace
])
def test_gemm_rescale_rejects_bad_arguments(ngq, args, status):
    assert ngq.lib().ngq_gemm_rescale(*args, None) == status


def test_gemm_rescale_empty_calls(ngq):
    L = ngq.lib()
    assert L.ngq_gemm_rescale(0, 17408, 5120, 4, 64, None, None, None, None, XNL, None, 0, None) == 0
    assert L.ngq_gemm_rescale(0, 17408, 5120, 4, 64, None, None, None, None, None, None, 0, None) == -1


@pytest.mark.parametrize("args,status", [
    ((8, *DOWN, XL, WL, SL, None, YL, XNL, WSL, 1 << 21), -1),        # null residual
    ((8, *DOWN, XL, WL, SL, RL, YL, None, WSL, 1 << 21), -1),         # null x_next
    ((9, *DOWN, XL, WL, SL, RL, YL, XNL, WSL, 1 << 21), -2),          # T > 8
    ((8, *DOWN, XL, WL, SL, RL + 8, YL, XNL, WSL, 1 << 21), -4),      # misaligned residual
    ((8, *DOWN, XL, WL, SL, YL + 64, YL, XNL, WSL, 1 << 21), -1),     # residual overlaps y
    ((8, *DOWN, XL, WL, SL, XNL, YL, XNL, WSL, 1 << 21), -1),         # residual is x_next
    ((8, *DOWN, XL, WL, SL, WSL + 64, YL, XNL, WSL, 1 << 21), -1),    # residual overlaps the workspace
    ((8, *DOWN, XL, WL, SL, RL, YL, XNL, WSL, 1 << 16), -1),          # workspace too small
    ((8, *DOWN, XL, WL, SL, RL, YL, XNL, None, 1 << 21), -1),         # null workspace
    ((8, *DOWN, XL, WL, SL, RL, YL, YL, WSL, 1 << 21), -1),           # x_next is y
    # the residual is always split: even K = 64 (one slice) needs the workspace
    ((1, 64, 5120, 4, 64, XL, WL, SL, RL, YL, XNL, None, 0), -1),
])
def test_gemm_residual_rescale_rejects_bad_arguments(ngq, args, status):
    assert ngq.lib().ngq_gemm_residual_rescale(*args, None) == status


def test_gemm_residual_rescale_empty_calls(ngq):
    L = ngq.lib()
    # T == 0 touches nothing; the two pointers that define the call are still required
    assert L.ngq_gemm_residual_rescale(0, *DOWN, None, None, None, RL, None, XNL, None, 0, None) == 0
    assert L.ngq_gemm_residual_rescale(0, *DOWN, None, None, None, None, None, XNL, None, 0, None) == -1
    assert L.ngq_gemm_residual_rescale(0, *DOWN, None, None, None, RL, None, None, None, 0, None) == -1


def test_force_kernel_roundtrip(ngq):
    """The kernel-path override is host state only: set, read back, reject."""
    prev = ngq.ngq_debug_force_kernel(ngq.NGQ_KERNEL_XRES8)
    assert ngq.ngq_debug_force_kernel(prev) == ngq.NGQ_KERNEL_XRES8
    assert ngq.lib().ngq_debug_force_kernel(12) == ngq.NGQ_ERR_ARG
    assert ngq.lib().ngq_debug_force_kernel(-1) == ngq.NGQ_ERR_ARG
    assert ngq.ngq_debug_force_kernel(ngq.NGQ_KERNEL_AUTO) == prev


def test_debug_exports_reject_bad_arguments(ngq):
    L = ngq.lib()
    assert L.ngq_unpack_codes(100, 4, 4, 64, W, Y, None) == -2
    assert L.ngq_unpack_codes(64, 4, 4, 64, W, None, None) == -1
    assert L.ngq_unpack_codes(64, 4, 4, 64, W + 4, Y, None) == -4
    assert L.ngq_dequant_f32(64, 4, 4, 64, W, None, Y, None) == -1
    assert L.ngq_stream_read(X, 24, Y, None) == -2
    assert L.ngq_stream_tiles(64, 200, 4, 64, 32, W, S, Y, None) == -2   # ragged tiles
    assert L.ngq_stream_tiles(64, 192, 4, 64, 40, W, S, Y, None) == -3   # tile width
    assert L.ngq_stream_tiles(64, 192, 4, 64, 32, None, S, Y, None) == -1


def test_binding_refuses_host_tensors(ngq):
    torch = pytest.importorskip("torch")
    x = torch.zeros((1, 64), dtype=torch.bfloat16)
    # operands of the right sizes, but in host memory
    with pytest.raises(TypeError):
        ngq.ngq_gemm(x, torch.zeros(128, dtype=torch.uint8), torch.zeros((1, 4), dtype=torch.float16), 4, 4)


def test_binding_checks_sizes_before_any_call(ngq):
    """The library sizes its reads and writes from K and N, so the binding
    refuses tensors that do not hold what those sizes imply, before calling it
    (host tensors here: the size checks come before the device check)."""
    torch = pytest.importorskip("torch")
    bf, f16, u8 = torch.bfloat16, torch.float16, torch.uint8
    T, K, N = 2, 128, 8
    x = torch.zeros((T, K), dtype=bf)
    wq = torch.zeros(ngq.ngq_packed_bytes(K, N, 4), dtype=u8)  # 512 bytes
    sc = torch.zeros((K // 64, N), dtype=f16)
    y = torch.zeros((T, N), dtype=bf)
    with pytest.raises(ValueError, match="wq holds"):
        ngq.ngq_gemm(x, wq[:-16], sc, 4, N, y=y)
    with pytest.raises(ValueError, match="wq holds"):
        ngq.ngq_gemm(x, wq, sc, 5, N, y=y)  # an int4 buffer read as int5 (P1 missing)
    with pytest.raises(ValueError, match="scales hold"):
        ngq.ngq_gemm(x, wq, sc[:1], 4, N, y=y)
    with pytest.raises(ValueError, match="output shape"):
        ngq.ngq_gemm(x, wq, sc, 4, N, y=torch.zeros((T, N - 4), dtype=bf))
    with pytest.raises(TypeError, match="bfloat16"):
        ngq.ngq_gemm(x, wq, sc, 4, N, y=torch.zeros((T, N), dtype=f16))
    # SwiGLU: wq and scales cover 2 N_ff columns
    with pytest.raises(ValueError, match="wq holds"):
        ngq.ngq_swiglu_gemm(x, wq, sc, 4, N)
    with pytest.raises(ValueError, match="output shape"):
        ngq.ngq_swiglu_gemm(x, wq, sc, 4, N // 2, h=torch.zeros((T + 1, N // 2), dtype=bf))
    with pytest.raises(ValueError, match="output shape"):
        ngq.ngq_gemm_splitk(x, wq, sc, 4, N, y=torch.zeros((T, N), dtype=bf).t(), workspace=wq)
    with pytest.raises(ValueError, match="output shape"):
        ngq.ngq_gemm_rescale(x, wq, sc, 4, N, y=y, x_next=torch.zeros((1, N), dtype=bf), workspace=wq)
    with pytest.raises(ValueError, match="residual must be"):
        ngq.ngq_gemm_residual_rescale(x, wq, sc, 4, N, torch.zeros((T, N + 4), dtype=bf), y=y, workspace=wq)
    with pytest.raises(ValueError, match="residual must be"):
        ngq.ngq_gemm_residual_rescale(x, wq, sc, 4, N, torch.zeros((T, N), dtype=f16), y=y, workspace=wq)
    with pytest.raises(ValueError, match="projection 1"):
        ngq.ngq_multi_gemm(x, [dict(wq=wq, scales=sc, bits=4, n=N, y=y),
                               dict(wq=wq, scales=sc, bits=4, n=N, swiglu=True)])
    with pytest.raises(ValueError, match="output shape"):
        ngq.ngq_rms_rescale(y, x=torch.zeros((T, N + 4), dtype=bf))
    with pytest.raises(ValueError):
        ngq.ngq_unpack_codes(wq[:64], K, N, 4)
    with pytest.raises(ValueError):
        ngq.ngq_stream_read(wq, torch.zeros(16, dtype=torch.int32))


def test_multi_plan_cache_under_concurrent_eviction(ngq):
    """ngq_multi_gemm plans its tile split per shape and keeps the last 16
    plans.  Two threads asking for 40 distinct shapes each keep evicting
    plans the other is using; every call must still finish with the same
    status (no device here: planning succeeds, the launch reports the missing
    device), and a plan is never read after its eviction (it is copied into
    the launch arguments under the cache's lock)."""
    import threading

    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("host-only check: with a device these fake pointers would be launched")
    L = ngq.lib()
    results = []

    def worker(base):
        out = []
        for i in range(40):
            n = 64 + 4 * (base + i)
            arr = (ngq.NgqProj * 2)(ngq.NgqProj(4, n, 0, 0, W, S, Y), ngq.NgqProj(5, 2 * n, 0, 0, W + 0x40000, S, Y + 0x8000))
            out.append(L.ngq_multi_gemm(8, 1024, 64, X, arr, 2, None))
        results.append(out)

    th = [threading.Thread(target=worker, args=(b,)) for b in (0, 17)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    statuses = {st for out in results for st in out}
    assert len(results) == 2 and len(statuses) == 1 and statuses.pop() in (ngq.NGQ_ERR_HIP,), statuses
