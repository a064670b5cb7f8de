"""Stacked decode layers over libngq: the sequence of calls one layer makes.

Per layer, on the token block x (bf16 [T][5120]):
  q = x . W_qk        int4, K=5120, N=8192     (GDN QK projection)
  v = x . W_gv        int5, K=5120, N=12288    (attention gate/value projection)
  h = SiLU(x . W_g) * (x . W_u)                 int4, K=5120, N_ff=17408 (fused)
  z = h . W_down      int4, K=17408, N=5120
  x <- z / rms(z)     per token row (ngq_rms_rescale)
The projections are those the NInfer-4090 V3 topic ("What V3 did") routes at
T=8; only the down output feeds the next layer, the q and v outputs are
written and not used (they stand for the attention inputs, which are outside
this library).  Each step is one library call through the C ABI with raw
device pointers; this module only orders the calls and keeps the buffers.
"""
from __future__ import annotations

from . import NGQ_GROUP, NGQ_SCALE_BF16, NgqError, lib

HIDDEN = 5120
N_FF = 17408
# (name, K, N, bits, bf16 scales, kind): kind 'gemm' or 'swiglu' (N is N_ff)
LAYER_PLAN = (
    ("qk", HIDDEN, 8192, 4, False, "gemm"),
    ("gv", HIDDEN, 12288, 5, True, "gemm"),
    ("gate_up", HIDDEN, N_FF, 4, False, "swiglu"),
    ("down", N_FF, HIDDEN, 4, False, "gemm"),
)


def layer_bytes(T: int, packed_bytes) -> int:
    """Algorithmic HBM bytes of one layer at T tokens: every packed weight and
    scale once, every activation read and every output written once."""
    total = 0
    for name, K, N, bits, _, kind in LAYER_PLAN:
        ncols = 2 * N if kind == "swiglu" else N
        total += packed_bytes(K, ncols, bits) + (K // NGQ_GROUP) * ncols * 2 + 2 * T * K + 2 * T * N
    return total + 2 * (2 * T * HIDDEN)  # rescale: read z, write x


class Stack:
    """Layers of device weights (from `layers`: a list of {name: (packed, scales)})
    and the work buffers of one token count T."""

    def __init__(self, layers, T: int, device="cuda"):
        import torch

        if not 1 <= T <= 8:
            raise ValueError("T must be in 1..8")
        self.T = T
        self.layers = layers
        bf = torch.bfloat16
        self.q = torch.empty((T, 8192), dtype=bf, device=device)
        self.v = torch.empty((T, 12288), dtype=bf, device=device)
        self.h = torch.empty((T, N_FF), dtype=bf, device=device)
        self.z = torch.empty((T, HIDDEN), dtype=bf, device=device)
        self.x = torch.empty((T, HIDDEN), dtype=bf, device=device)  # the running activation
        self._calls = []
        for lw in layers:
            calls = []
            for name, K, N, bits, sbf16, kind in LAYER_PLAN:
                wq, s = lw[name]
                flag = bits | (NGQ_SCALE_BF16 if sbf16 else 0)
                calls.append((kind, K, N, flag, wq.data_ptr(), s.data_ptr()))
            self._calls.append(calls)

    def layer(self, i: int, stream: int):
        """Enqueue layer i on `stream` (a hipStream_t as int): x -> x."""
        L = lib()
        T = self.T
        xp, qp, vp, hp, zp = (t.data_ptr() for t in (self.x, self.q, self.v, self.h, self.z))
        (_, K0, N0, f0, w0, s0), (_, K1, N1, f1, w1, s1), (_, K2, N2, f2, w2, s2), (_, K3, N3, f3, w3, s3) = \
            self._calls[i]
        for st, where in (
            (L.ngq_gemm(T, K0, N0, f0, NGQ_GROUP, xp, w0, s0, qp, stream), "qk"),
            (L.ngq_gemm(T, K1, N1, f1, NGQ_GROUP, xp, w1, s1, vp, stream), "gv"),
            (L.ngq_swiglu_gemm(T, K2, N2, f2, NGQ_GROUP, xp, w2, s2, hp, stream), "gate_up"),
            (L.ngq_gemm(T, K3, N3, f3, NGQ_GROUP, hp, w3, s3, zp, stream), "down"),
            (L.ngq_rms_rescale(T, HIDDEN, zp, xp, stream), "rescale"),
        ):
            if st != 0:
                raise NgqError(st, f"layer {i} {where}")

    def forward(self, x0, stream: int, layers: int | None = None):
        """Copy x0 (device bf16 [T][5120]) into the running activation and enqueue
        the first `layers` layers (all by default).  Returns the activation."""
        self.x.copy_(x0)
        for i in range(len(self.layers) if layers is None else layers):
            self.layer(i, stream)
        return self.x
