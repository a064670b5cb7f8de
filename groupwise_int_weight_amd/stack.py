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
device pointers; this module only orders the calls (on up to three streams)
and keeps the buffers.  With `fused`, the three projections of x are one
ngq_multi_gemm call, and the down projection and the rescale one
ngq_gemm_rescale call.
"""
from __future__ import annotations

from . import NGQ_GROUP, NGQ_SCALE_BF16, NgqError, NgqProj, lib

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
    and the work buffers of one token count T.

    By default every call runs in order on the main stream.  With `fused` the
    QK, gate/value and gate/up projections are one ngq_multi_gemm launch (one
    launch cost, the tiles of all three spread over the CUs together) and the down
    projection with the rescale is ngq_gemm_rescale (K split, since its 160
    column tiles alone leave CUs idle, and the rescale done by the kernel
    that adds the slices).  With `concurrent`
    the QK and gate/value projections, which only read x, run on two side
    streams beside the gate/up and down projections, and the main stream waits
    for them before the rescale overwrites x.  On MI355X that is slower
    (measured): a kernel running beside another delays the workgroups that
    own its tiles, and the launch that finishes last sets the layer's time."""

    def __init__(self, layers, T: int, device="cuda", concurrent: bool = False, fused: bool = False):
        import torch

        if not 1 <= T <= 8:
            raise ValueError("T must be in 1..8")
        if concurrent and fused:
            raise ValueError("concurrent and fused are exclusive")
        self.fused = fused
        self.T = T
        self.layers = layers
        self.concurrent = concurrent
        bf = torch.bfloat16
        self.q = torch.empty((T, 8192), dtype=bf, device=device)
        self.v = torch.empty((T, 12288), dtype=bf, device=device)
        self.h = torch.empty((T, N_FF), dtype=bf, device=device)
        self.z = torch.empty((T, HIDDEN), dtype=bf, device=device)
        self.x = torch.empty((T, HIDDEN), dtype=bf, device=device)  # the running activation
        self.side = (torch.cuda.Stream(device=device), torch.cuda.Stream(device=device)) if concurrent else ()
        self.ws = None
        if fused:  # the split-K down projection's workspace
            _, K3, N3, bits3, _, _ = LAYER_PLAN[3]
            self.ws = torch.empty(lib().ngq_splitk_workspace_bytes(K3, N3, bits3, NGQ_GROUP), dtype=torch.uint8,
                                  device=device)
        self._calls = []
        self._multi = []
        for lw in layers:
            calls = []
            for name, K, N, bits, sbf16, kind in LAYER_PLAN:
                wq, s = lw[name]
                flag = bits | (NGQ_SCALE_BF16 if sbf16 else 0)
                calls.append((kind, K, N, flag, wq.data_ptr(), s.data_ptr()))
            self._calls.append(calls)
            # the projections of x as one ngq_multi_gemm call
            outs = (self.q, self.v, self.h)
            self._multi.append((NgqProj * 3)(*(NgqProj(f, N, int(kind == "swiglu"), 0, w, sc, o.data_ptr())
                                               for (kind, _, N, f, w, sc), o in zip(calls[:3], outs))))

    def project(self, i: int, stream=None):
        """Enqueue only the three projections of x of layer i (QK, gate/value,
        gate/up + SwiGLU) as one ngq_multi_gemm call."""
        import torch

        main = torch.cuda.current_stream() if stream is None else stream
        st = lib().ngq_multi_gemm(self.T, HIDDEN, NGQ_GROUP, self.x.data_ptr(), self._multi[i], 3, main.cuda_stream)
        if st != 0:
            raise NgqError(st, f"layer {i} qk+gv+gate_up")

    def layer(self, i: int, stream=None):
        """Enqueue layer i (x -> x) on `stream` (a torch.cuda.Stream; the current
        stream by default)."""
        import torch

        main = torch.cuda.current_stream() if stream is None else stream
        L = lib()
        T = self.T
        xp, qp, vp, hp, zp = (t.data_ptr() for t in (self.x, self.q, self.v, self.h, self.z))
        (_, K0, N0, f0, w0, s0), (_, K1, N1, f1, w1, s1), (_, K2, N2, f2, w2, s2), (_, K3, N3, f3, w3, s3) = \
            self._calls[i]

        def check(st, where):
            if st != 0:
                raise NgqError(st, f"layer {i} {where}")

        if self.fused:
            self.project(i, main)
            check(L.ngq_gemm_rescale(T, K3, N3, f3, NGQ_GROUP, hp, w3, s3, zp, xp, self.ws.data_ptr(),
                                     self.ws.numel(), main.cuda_stream), "down+rescale")
            return
        if self.concurrent:
            x_ready = torch.cuda.Event()
            x_ready.record(main)
            sq, sv = self.side
            sq.wait_event(x_ready)
            sv.wait_event(x_ready)
            check(L.ngq_gemm(T, K0, N0, f0, NGQ_GROUP, xp, w0, s0, qp, sq.cuda_stream), "qk")
            check(L.ngq_gemm(T, K1, N1, f1, NGQ_GROUP, xp, w1, s1, vp, sv.cuda_stream), "gv")
            q_done, v_done = torch.cuda.Event(), torch.cuda.Event()
            q_done.record(sq)
            v_done.record(sv)
        else:
            check(L.ngq_gemm(T, K0, N0, f0, NGQ_GROUP, xp, w0, s0, qp, main.cuda_stream), "qk")
            check(L.ngq_gemm(T, K1, N1, f1, NGQ_GROUP, xp, w1, s1, vp, main.cuda_stream), "gv")
        check(L.ngq_swiglu_gemm(T, K2, N2, f2, NGQ_GROUP, xp, w2, s2, hp, main.cuda_stream), "gate_up")
        check(L.ngq_gemm(T, K3, N3, f3, NGQ_GROUP, hp, w3, s3, zp, main.cuda_stream), "down")
        if self.concurrent:
            main.wait_event(q_done)  # x is overwritten next: QK and gate/value must be done reading it
            main.wait_event(v_done)
        check(L.ngq_rms_rescale(T, HIDDEN, zp, xp, main.cuda_stream), "rescale")

    def forward(self, x0, stream=None, layers: int | None = None):
        """Copy x0 (device bf16 [T][5120]) into the running activation and enqueue
        the first `layers` layers (all by default) on `stream`.  Returns the
        activation."""
        import torch

        main = torch.cuda.current_stream() if stream is None else stream
        with torch.cuda.stream(main):
            self.x.copy_(x0)
        for i in range(len(self.layers) if layers is None else layers):
            self.layer(i, main)
        return self.x
