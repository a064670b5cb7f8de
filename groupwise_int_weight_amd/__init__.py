"""Python binding of libngq: small-T groupwise-int projections on MI355X.

Thin ctypes marshalling over the C ABI declared in ``include/ngq.h``; every
step of the projection runs in the library's HIP kernels.  PyTorch is used
only for device memory and the current stream.  The names match the C entry
points: ``ngq_pack``, ``ngq_gemm``, ``ngq_swiglu_gemm`` and the debug exports.

The library must be built first (``python -m groupwise_int_weight_amd.build``);
importing a GPU entry point without it raises ``NgqLibraryMissing``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libngq.so")

NGQ_OK = 0
NGQ_ERR_ARG = -1
NGQ_ERR_SHAPE = -2
NGQ_ERR_UNSUPPORTED = -3
NGQ_ERR_ALIGN = -4
NGQ_ERR_HIP = -5
NGQ_INT4, NGQ_INT5, NGQ_INT8 = 4, 5, 8
NGQ_SCALE_BF16 = 0x100
NGQ_GROUP = 64
NGQ_MAX_T = 8
NGQ_MAX_T_VERIFY = 64  # several requests' verify rounds in one call
NGQ_MAX_T_PREFILL = 16384  # ngq_gemm / ngq_swiglu_gemm
NGQ_MAX_PROJ = 4
NGQ_STATIC_SCRATCH_BYTES = 4 << 20  # ngq_gemm_splitk_static's partial-sum array per device
NGQ_KERNEL_AUTO, NGQ_KERNEL_PERPAIR_DYN, NGQ_KERNEL_PERPAIR_STATIC, NGQ_KERNEL_XRES14, NGQ_KERNEL_XRES8 = 0, 1, 2, 3, 4
NGQ_KERNEL_WIDE, NGQ_KERNEL_TILED, NGQ_KERNEL_TILED_SX, NGQ_KERNEL_TILED_SX96, NGQ_KERNEL_TILED_SX128 = 5, 6, 7, 8, 9
NGQ_KERNEL_STREAM, NGQ_KERNEL_DOT = 10, 11

# Every function the header declares, with its ctypes signature.
_SIZE = ctypes.c_size_t
_INT = ctypes.c_int
_PTR = ctypes.c_void_p


class NgqProj(ctypes.Structure):
    """struct ngq_proj: one projection of an ngq_multi_gemm call."""
    _fields_ = [("bits", _INT), ("n", _INT), ("swiglu", _INT), ("reserved", _INT),
                ("wq", _PTR), ("scales", _PTR), ("y", _PTR)]


SIGNATURES = {
    "ngq_packed_bytes": (_SIZE, [_INT, _INT, _INT, _INT]),
    "ngq_scale_bytes": (_SIZE, [_INT, _INT, _INT, _INT]),
    "ngq_pack": (_INT, [_INT, _INT, _INT, _INT, _PTR, _PTR]),
    "ngq_gemm": (_INT, [_INT, _INT, _INT, _INT, _INT, _PTR, _PTR, _PTR, _PTR, _PTR]),
    "ngq_swiglu_gemm": (_INT, [_INT, _INT, _INT, _INT, _INT, _PTR, _PTR, _PTR, _PTR, _PTR]),
    "ngq_unpack_codes": (_INT, [_INT, _INT, _INT, _INT, _PTR, _PTR, _PTR]),
    "ngq_dequant_f32": (_INT, [_INT, _INT, _INT, _INT, _PTR, _PTR, _PTR, _PTR]),
    "ngq_multi_gemm": (_INT, [_INT, _INT, _INT, _PTR, ctypes.POINTER(NgqProj), _INT, _PTR]),
    "ngq_splitk_workspace_bytes": (_SIZE, [_INT, _INT, _INT, _INT]),
    "ngq_gemm_splitk": (_INT, [_INT, _INT, _INT, _INT, _INT, _PTR, _PTR, _PTR, _PTR, _PTR, _SIZE, _PTR]),
    "ngq_gemm_splitk_static": (_INT, [_INT, _INT, _INT, _INT, _INT, _PTR, _PTR, _PTR, _PTR, _PTR]),
    "ngq_rms_rescale": (_INT, [_INT, _INT, _PTR, _PTR, _PTR]),
    "ngq_gemm_rescale": (_INT, [_INT, _INT, _INT, _INT, _INT, _PTR, _PTR, _PTR, _PTR, _PTR, _PTR, _SIZE, _PTR]),
    "ngq_gemm_residual_rescale": (_INT, [_INT, _INT, _INT, _INT, _INT, _PTR, _PTR, _PTR, _PTR, _PTR, _PTR, _PTR,
                                         _SIZE, _PTR]),
    "ngq_stream_read": (_INT, [_PTR, _SIZE, _PTR, _PTR]),
    "ngq_stream_tiles": (_INT, [_INT, _INT, _INT, _INT, _INT, _PTR, _PTR, _PTR, _PTR]),
    "ngq_debug_force_kernel": (_INT, [_INT]),
    "ngq_strerror": (ctypes.c_char_p, [_INT]),
    "ngq_version": (_INT, []),
}


class NgqLibraryMissing(ImportError):
    pass


class NgqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {ngq_strerror(status)} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libngq.so (raises NgqLibraryMissing when it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise NgqLibraryMissing(
                f"{LIB_PATH} is not built; run `python -m groupwise_int_weight_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status: int, where: str):
    if status != NGQ_OK:
        raise NgqError(status, where)


def ngq_strerror(status: int) -> str:
    return lib().ngq_strerror(int(status)).decode()


def ngq_version() -> int:
    return int(lib().ngq_version())


def ngq_packed_bytes(K: int, N: int, bits: int, group: int = NGQ_GROUP) -> int:
    return int(lib().ngq_packed_bytes(K, N, bits, group))


def ngq_scale_bytes(K: int, N: int, bits: int, group: int = NGQ_GROUP) -> int:
    return int(lib().ngq_scale_bytes(K, N, bits, group))


def ngq_pack(codes: np.ndarray, bits: int, group: int = NGQ_GROUP) -> np.ndarray:
    """Pack int8 codes [K][N] (host) into the library's layout (host uint8 array)."""
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    K, N = codes.shape
    nbytes = ngq_packed_bytes(K, N, bits, group)
    out = np.zeros(max(nbytes, 16), dtype=np.uint8)
    _check(lib().ngq_pack(K, N, bits, group, codes.ctypes.data, out.ctypes.data), "ngq_pack")
    return out[:nbytes]


# ---- device entry points (torch tensors on the current HIP device) ----------

def _stream(stream):
    import torch

    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _dev_ptr(t, what):
    import torch

    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{what} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t.data_ptr()


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _check_operands(where, x, wq, scales, outs, K: int, ncols: int, bits: int, group: int):
    """Shapes, sizes, dtypes and devices of a projection's tensors, checked
    before the library is called: the library sizes its reads from K and N, so
    a buffer that is too small would be read or written past its end.
      wq     : ngq_packed_bytes(K, ncols, bits) bytes (nothing is read when K or ncols is 0)
      scales : (K / group) * ncols elements, float16 or bfloat16
      outs   : (tensor, rows, cols) triples, each bfloat16 of exactly that shape
    Every tensor must be on x's device.  With no token rows the call is a
    no-op that touches no buffer, so nothing is checked."""
    import torch

    if x.shape[0] == 0:
        return
    if K > 0 and ncols > 0:
        need = ngq_packed_bytes(K, ncols, int(bits) & 0xFF, group)
        if need == 0:
            raise ValueError(f"{where}: K={K}, columns={ncols}, bits={bits} is not a valid shape")
        if _nbytes(wq) != need:
            raise ValueError(f"{where}: wq holds {_nbytes(wq)} bytes, the packed {K} x {ncols} matrix {need}")
        if scales.numel() != (K // group) * ncols:
            raise ValueError(f"{where}: scales hold {scales.numel()} values, expected {(K // group) * ncols}")
    for t, rows, cols in outs:
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{where}: outputs must be bfloat16")
        if tuple(t.shape) != (rows, cols):
            raise ValueError(f"{where}: output shape {tuple(t.shape)}, expected {(rows, cols)}")
    for t in [wq, scales] + [o[0] for o in outs]:
        if t is not None and t.device != x.device:
            raise ValueError(f"{where}: every tensor must be on {x.device}, found one on {t.device}")


def _format_bits(bits: int, scales) -> int:
    import torch

    b = int(bits) & 0xFF
    if scales is not None and scales.dtype == torch.bfloat16:
        b |= NGQ_SCALE_BF16
    elif scales is not None and scales.dtype != torch.float16:
        raise TypeError("scales must be float16 or bfloat16")
    return b


def ngq_gemm(x, wq, scales, bits: int, N: int, y=None, group: int = NGQ_GROUP, stream=None):
    """y[T][N] (bf16) = x[T][K] (bf16) . dequant(wq) with scales [K/64][N]."""
    import torch

    T, K = x.shape
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    if y is None:
        y = torch.empty((T, N), dtype=torch.bfloat16, device=x.device)
    _check_operands("ngq_gemm", x, wq, scales, [(y, T, N)], K, N, bits, group)
    st = lib().ngq_gemm(T, K, N, _format_bits(bits, scales), group, _dev_ptr(x, "x"), _dev_ptr(wq, "wq"),
                        _dev_ptr(scales, "scales"), _dev_ptr(y, "y"), _stream(stream))
    _check(st, "ngq_gemm")
    return y


def ngq_swiglu_gemm(x, wq_gate_up, scales_gate_up, bits: int, N_ff: int, h=None, group: int = NGQ_GROUP,
                    stream=None):
    """h[T][N_ff] (bf16) = SiLU(x . W_gate) * (x . W_up), W = [gate | up] packed as K x 2N_ff."""
    import torch

    T, K = x.shape
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    if h is None:
        h = torch.empty((T, N_ff), dtype=torch.bfloat16, device=x.device)
    _check_operands("ngq_swiglu_gemm", x, wq_gate_up, scales_gate_up, [(h, T, N_ff)], K, 2 * N_ff, bits, group)
    st = lib().ngq_swiglu_gemm(T, K, N_ff, _format_bits(bits, scales_gate_up), group, _dev_ptr(x, "x"),
                               _dev_ptr(wq_gate_up, "wq_gate_up"), _dev_ptr(scales_gate_up, "scales_gate_up"),
                               _dev_ptr(h, "h"), _stream(stream))
    _check(st, "ngq_swiglu_gemm")
    return h


def ngq_splitk_workspace_bytes(K: int, N: int, bits: int, group: int = NGQ_GROUP) -> int:
    return int(lib().ngq_splitk_workspace_bytes(K, N, bits, group))


def ngq_gemm_splitk(x, wq, scales, bits: int, N: int, y=None, workspace=None, group: int = NGQ_GROUP, stream=None):
    """ngq_gemm with K split over several workgroups per column tile (long K,
    few tiles); `workspace` (a device uint8 tensor of at least
    ngq_splitk_workspace_bytes bytes) is allocated when not given."""
    import torch

    T, K = x.shape
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    if y is None:
        y = torch.empty((T, N), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        workspace = torch.empty(max(16, ngq_splitk_workspace_bytes(K, N, bits, group)), dtype=torch.uint8,
                                device=x.device)
    _check_operands("ngq_gemm_splitk", x, wq, scales, [(y, T, N)], K, N, bits, group)
    if workspace.device != x.device:
        raise ValueError("ngq_gemm_splitk: the workspace must be on x's device")
    st = lib().ngq_gemm_splitk(T, K, N, _format_bits(bits, scales), group, _dev_ptr(x, "x"), _dev_ptr(wq, "wq"),
                               _dev_ptr(scales, "scales"), _dev_ptr(y, "y"), _dev_ptr(workspace, "workspace"),
                               workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "ngq_gemm_splitk")
    return y


def ngq_gemm_splitk_static(x, wq, scales, bits: int, N: int, y=None, group: int = NGQ_GROUP, stream=None):
    """ngq_gemm_splitk with the partial sums in the library's fixed device
    array (no allocation by the library; calls on one device must not
    overlap).  `y` is allocated here when not given."""
    import torch

    T, K = x.shape
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    if y is None:
        y = torch.empty((T, N), dtype=torch.bfloat16, device=x.device)
    _check_operands("ngq_gemm_splitk_static", x, wq, scales, [(y, T, N)], K, N, bits, group)
    st = lib().ngq_gemm_splitk_static(T, K, N, _format_bits(bits, scales), group, _dev_ptr(x, "x"),
                                      _dev_ptr(wq, "wq"), _dev_ptr(scales, "scales"), _dev_ptr(y, "y"),
                                      _stream(stream))
    _check(st, "ngq_gemm_splitk_static")
    return y


def ngq_multi_gemm(x, projs, group: int = NGQ_GROUP, stream=None):
    """Several projections of the same x in one launch.  `projs` is a list of
    dicts with keys wq, scales, bits, n and optionally swiglu (False) and y;
    returns the list of outputs y[T][n] (bf16), each what ngq_gemm (or
    ngq_swiglu_gemm when swiglu) computes for its projection."""
    import torch

    T, K = x.shape
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    arr = (NgqProj * max(1, len(projs)))()
    outs = []
    for i, p in enumerate(projs):
        y = p.get("y")
        if y is None:
            y = torch.empty((T, int(p["n"])), dtype=torch.bfloat16, device=x.device)
        outs.append(y)
        n = int(p["n"])
        nsets = 2 if p.get("swiglu", False) else 1
        _check_operands(f"ngq_multi_gemm projection {i}", x, p["wq"], p["scales"], [(y, T, n)], K, nsets * n,
                        p["bits"], group)
    for i, (p, y) in enumerate(zip(projs, outs)):
        arr[i] = NgqProj(_format_bits(p["bits"], p["scales"]), int(p["n"]), int(bool(p.get("swiglu", False))), 0,
                         _dev_ptr(p["wq"], "wq"), _dev_ptr(p["scales"], "scales"), _dev_ptr(y, "y"))
    _check(lib().ngq_multi_gemm(T, K, group, _dev_ptr(x, "x"), arr, len(projs), _stream(stream)), "ngq_multi_gemm")
    return outs


def ngq_rms_rescale(z, x=None, stream=None):
    """x[t][:] (bf16) = z[t][:] / rms(z[t][:]); x may be z itself (in place)."""
    import torch

    T, N = z.shape
    if z.dtype != torch.bfloat16:
        raise TypeError("z must be bfloat16")
    if x is None:
        x = torch.empty_like(z)
    _check_operands("ngq_rms_rescale", z, None, None, [(x, T, N)], 0, N, NGQ_INT4, NGQ_GROUP)
    _check(lib().ngq_rms_rescale(T, N, _dev_ptr(z, "z"), _dev_ptr(x, "x"), _stream(stream)), "ngq_rms_rescale")
    return x


def ngq_gemm_rescale(x, wq, scales, bits: int, N: int, y=None, x_next=None, workspace=None,
                     group: int = NGQ_GROUP, stream=None):
    """The projection y = x . W (as ngq_gemm_splitk) and x_next = the RMS
    rescale of y (as ngq_rms_rescale) in one call; returns (y, x_next)."""
    import torch

    T, K = x.shape
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    if y is None:
        y = torch.empty((T, N), dtype=torch.bfloat16, device=x.device)
    if x_next is None:
        x_next = torch.empty((T, N), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        workspace = torch.empty(max(16, ngq_splitk_workspace_bytes(K, N, bits, group)), dtype=torch.uint8,
                                device=x.device)
    _check_operands("ngq_gemm_rescale", x, wq, scales, [(y, T, N), (x_next, T, N)], K, N, bits, group)
    if workspace.device != x.device:
        raise ValueError("ngq_gemm_rescale: the workspace must be on x's device")
    st = lib().ngq_gemm_rescale(T, K, N, _format_bits(bits, scales), group, _dev_ptr(x, "x"), _dev_ptr(wq, "wq"),
                                _dev_ptr(scales, "scales"), _dev_ptr(y, "y"), _dev_ptr(x_next, "x_next"),
                                _dev_ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                                _stream(stream))
    _check(st, "ngq_gemm_rescale")
    return y, x_next


def ngq_gemm_residual_rescale(x, wq, scales, bits: int, N: int, residual, y=None, x_next=None, workspace=None,
                              group: int = NGQ_GROUP, stream=None):
    """y = x . W + residual, rounded once to bf16, and x_next = the RMS rescale
    of y, in one call (K split, the residual added by the closing kernel);
    returns (y, x_next)."""
    import torch

    T, K = x.shape
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    if y is None:
        y = torch.empty((T, N), dtype=torch.bfloat16, device=x.device)
    if x_next is None:
        x_next = torch.empty((T, N), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        workspace = torch.empty(max(16, ngq_splitk_workspace_bytes(K, N, bits, group)), dtype=torch.uint8,
                                device=x.device)
    _check_operands("ngq_gemm_residual_rescale", x, wq, scales, [(y, T, N), (x_next, T, N)], K, N, bits, group)
    if residual.dtype != torch.bfloat16 or tuple(residual.shape) != (T, N):
        raise ValueError(f"ngq_gemm_residual_rescale: the residual must be bfloat16 of shape ({T}, {N}), "
                         f"not {residual.dtype} {tuple(residual.shape)}")
    for what, t in (("residual", residual), ("workspace", workspace)):
        if t.device != x.device:
            raise ValueError(f"ngq_gemm_residual_rescale: the {what} must be on x's device")
    st = lib().ngq_gemm_residual_rescale(T, K, N, _format_bits(bits, scales), group, _dev_ptr(x, "x"),
                                         _dev_ptr(wq, "wq"), _dev_ptr(scales, "scales"),
                                         _dev_ptr(residual, "residual"), _dev_ptr(y, "y"),
                                         _dev_ptr(x_next, "x_next"), _dev_ptr(workspace, "workspace"),
                                         workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "ngq_gemm_residual_rescale")
    return y, x_next


def ngq_unpack_codes(wq, K: int, N: int, bits: int, group: int = NGQ_GROUP, stream=None):
    import torch

    codes = torch.empty((K, N), dtype=torch.int8, device=wq.device)
    if K > 0 and _nbytes(wq) != ngq_packed_bytes(K, N, int(bits) & 0xFF, group):
        raise ValueError("ngq_unpack_codes: wq does not hold the packed K x N matrix")
    _check(lib().ngq_unpack_codes(K, N, int(bits) & 0xFF, group, _dev_ptr(wq, "wq"), _dev_ptr(codes, "codes"),
                                  _stream(stream)), "ngq_unpack_codes")
    return codes


def ngq_dequant_f32(wq, scales, K: int, N: int, bits: int, group: int = NGQ_GROUP, stream=None):
    import torch

    w = torch.empty((K, N), dtype=torch.float32, device=wq.device)
    if K > 0 and (_nbytes(wq) != ngq_packed_bytes(K, N, int(bits) & 0xFF, group) or
                  scales.numel() != (K // group) * N or scales.device != wq.device):
        raise ValueError("ngq_dequant_f32: wq or scales do not match the K x N matrix")
    _check(lib().ngq_dequant_f32(K, N, _format_bits(bits, scales), group, _dev_ptr(wq, "wq"),
                                 _dev_ptr(scales, "scales"), _dev_ptr(w, "w"), _stream(stream)),
           "ngq_dequant_f32")
    return w


def ngq_stream_read(buf, sink, stream=None):
    if _nbytes(sink) < 16384 or sink.device != buf.device:
        raise ValueError("ngq_stream_read: sink must hold 16384 bytes on the buffer's device")
    _check(lib().ngq_stream_read(_dev_ptr(buf, "buf"), buf.numel() * buf.element_size(), _dev_ptr(sink, "sink"),
                                 _stream(stream)), "ngq_stream_read")


def ngq_stream_tiles(wq, scales, K: int, N: int, bits: int, cols: int, sink, group: int = NGQ_GROUP, stream=None):
    """The weight stream of the streaming decode kernel alone (calibration);
    sink (device, >= 16384 bytes) receives per-tile checksums."""
    if K > 0 and _nbytes(wq) != ngq_packed_bytes(K, N, int(bits) & 0xFF, group):
        raise ValueError("ngq_stream_tiles: wq does not hold the packed K x N matrix")
    if _nbytes(sink) < 16384:
        raise ValueError("ngq_stream_tiles: sink must hold 16384 bytes")
    _check(lib().ngq_stream_tiles(K, N, _format_bits(bits, scales), group, cols, _dev_ptr(wq, "wq"),
                                  _dev_ptr(scales, "scales"), _dev_ptr(sink, "sink"), _stream(stream)),
           "ngq_stream_tiles")


def ngq_debug_force_kernel(path: int) -> int:
    """Force a kernel path for later calls (NGQ_KERNEL_AUTO restores the
    per-shape choice); returns the previous setting."""
    prev = int(lib().ngq_debug_force_kernel(int(path)))
    if prev < 0:
        raise NgqError(prev, "ngq_debug_force_kernel")
    return prev


__all__ = [
    "ngq_pack", "ngq_gemm", "ngq_swiglu_gemm", "ngq_multi_gemm", "ngq_gemm_splitk", "ngq_splitk_workspace_bytes",
    "ngq_gemm_splitk_static",
    "ngq_rms_rescale", "ngq_unpack_codes", "ngq_dequant_f32", "ngq_stream_read", "ngq_stream_tiles",
    "ngq_debug_force_kernel",
    "ngq_packed_bytes", "ngq_scale_bytes", "ngq_strerror", "ngq_version", "NgqError", "NgqLibraryMissing",
    "lib", "SIGNATURES", "NgqProj",
]
