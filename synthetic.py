"""Seeded synthetic inputs for the groupwise-int projection.

This module holds no arithmetic of the method: it only draws random codes,
scales and activations with the shapes and distributions of the workloads,
and describes those workloads.  The tests, the smoke check and the bench all
take their inputs from here, so the HIP path and the oracle see the same bits.

Workloads (shapes of the Qwen3.8-27B projections named on the pages: the GDN
QK projection, the attention gate/value projection and the SwiGLU MLP of the
NInfer-4090 V3 topic, section "What V3 did"; the pages give no sizes or
distributions, so these are readings):

  tiny      T=1, K=256,  N=256,   int4, fp16 scales U[1e-3, 2e-2]
  qk        T in 1..8, K=5120, N=8192,  int4, fp16 scales U[1e-3, 2e-2]
  gv        T in 1..8, K=5120, N=12288, int5, bf16 scales U[5e-4, 1e-2]
  gate_up   T in 1..8, K=5120, N=2*17408 (gate | up), int4, fp16 scales
  down      T in 1..8, K=17408, N=5120, int4, fp16 scales
  qk8       T in 1..8, K=5120, N=8192,  int8, fp16 scales (the QK shape in int8)

Codes are uniform over the full signed range of the width, X is N(0,1)
rounded to bf16, scales are uniform and rounded to the 16-bit scale type.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

GROUP = 64


@dataclass(frozen=True)
class Workload:
    name: str
    K: int
    N: int
    bits: int
    scale_bf16: bool
    scale_lo: float
    scale_hi: float
    config_id: int


WORKLOADS = {
    "tiny": Workload("tiny", 256, 256, 4, False, 1e-3, 2e-2, 0),
    "qk": Workload("qk", 5120, 8192, 4, False, 1e-3, 2e-2, 1),
    "gv": Workload("gv", 5120, 12288, 5, True, 5e-4, 1e-2, 2),
    "gate_up": Workload("gate_up", 5120, 2 * 17408, 4, False, 1e-3, 2e-2, 3),
    "down": Workload("down", 17408, 5120, 4, False, 1e-3, 2e-2, 3),
    # int8 is in the format list but in no measured workload: the QK shape
    "qk8": Workload("qk8", 5120, 8192, 8, False, 1e-3, 2e-2, 5),
}
N_FF = 17408
HIDDEN = 5120

# tensor ids of the seed streams
_CODES, _SCALES, _X = 0, 1, 2


def rng(seed: int, config_id: int, layer: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, config_id, layer, tensor_id]))


def code_range(bits: int):
    return -(1 << (bits - 1)), (1 << (bits - 1)) - 1


def draw_codes(K: int, N: int, bits: int, g: np.random.Generator) -> np.ndarray:
    lo, hi = code_range(bits)
    return g.integers(lo, hi + 1, size=(K, N), dtype=np.int8)


def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of fp32 values, rounded to nearest even by torch."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def draw_scales(K: int, N: int, lo: float, hi: float, bf16: bool, g: np.random.Generator) -> np.ndarray:
    v = g.uniform(lo, hi, size=(K // GROUP, N))
    if bf16:
        return f32_to_bf16_bits(v.astype(np.float32))
    return v.astype(np.float16).view(np.uint16)


def draw_x(T: int, K: int, g: np.random.Generator) -> np.ndarray:
    return f32_to_bf16_bits(g.standard_normal(size=(T, K)).astype(np.float32))


def make_inputs(w: Workload, T: int, seed: int = 0, layer: int = 0, K: int | None = None, N: int | None = None):
    """codes int8 [K][N], scales uint16 [K/64][N], x uint16 [T][K] (bf16 bits)."""
    K = w.K if K is None else K
    N = w.N if N is None else N
    codes = draw_codes(K, N, w.bits, rng(seed, w.config_id, layer, _CODES))
    scales = draw_scales(K, N, w.scale_lo, w.scale_hi, w.scale_bf16, rng(seed, w.config_id, layer, _SCALES))
    x = draw_x(T, K, rng(seed, w.config_id, layer, _X))
    return codes, scales, x


def random_words(nbytes: int, g: np.random.Generator) -> np.ndarray:
    """Uniformly random packed bytes.  Every field of every packed layout is
    then uniform over its range, i.e. codes uniform over the full signed range."""
    return g.integers(0, 256, size=nbytes, dtype=np.uint8)


def device_replicas(w: Workload, T: int, replicas: int, packed_bytes: int, seed: int = 0, device: str = "cuda"):
    """`replicas` distinct copies of a packed weight matrix and its scales, drawn
    on the device (uniform random bytes = uniform codes over the full range),
    plus one bf16 activation block [T][K].  Used to rotate through more memory
    than the caches hold when timing."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1_000_003 + w.config_id)
    wq = torch.randint(0, 256, (replicas, packed_bytes), dtype=torch.uint8, device=device, generator=g)
    s = torch.rand((replicas, w.K // GROUP, w.N), device=device, generator=g) * (w.scale_hi - w.scale_lo) + w.scale_lo
    s = s.to(torch.bfloat16 if w.scale_bf16 else torch.float16)
    x = torch.randn((T, w.K), device=device, generator=g).to(torch.bfloat16)
    return wq, s, x


# ---- the stacked-layer sweep ---------------------------------------------------------
# Per layer: the QK projection, the gate/value projection, the fused gate/up
# projection and the down projection, each with its own seeded weights.
STACK_PROJECTIONS = ("qk", "gv", "gate_up", "down")
STACK_CONFIG_ID = 4


def device_stack(layers: int, packed_bytes, seed: int = 0, device: str = "cuda"):
    """Distinct weights for `layers` stacked layers, drawn on the device: a list
    of {projection name: (packed uint8 tensor, scale tensor)}.  Packed bytes are
    uniform (uniform codes over the full range); scales are uniform over the
    workload's range, rounded to its 16-bit scale type.  `packed_bytes(K, N,
    bits)` gives the size of a packed matrix."""
    import torch

    out = []
    for layer in range(layers):
        d = {}
        for j, name in enumerate(STACK_PROJECTIONS):
            w = WORKLOADS[name]
            g = torch.Generator(device=device)
            g.manual_seed(((int(seed) * 1_000_003 + STACK_CONFIG_ID) * 4099 + layer) * 8 + j)
            wq = torch.randint(0, 256, (int(packed_bytes(w.K, w.N, w.bits)),), dtype=torch.uint8, device=device,
                               generator=g)
            s = torch.rand((w.K // GROUP, w.N), device=device, generator=g) * (w.scale_hi - w.scale_lo) + w.scale_lo
            d[name] = (wq, s.to(torch.bfloat16 if w.scale_bf16 else torch.float16))
        out.append(d)
    return out


def stack_x0(T: int, seed: int = 0) -> np.ndarray:
    """The first layer's input, bf16 bits [T][5120], N(0,1)."""
    return draw_x(T, HIDDEN, rng(seed, STACK_CONFIG_ID, 0, _X))
