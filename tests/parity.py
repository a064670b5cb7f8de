"""Comparison of GPU results with the oracle (helpers shared by the GPU tests,
the smoke check and the bench).

Gates, for bf16 outputs y_gpu against the oracle's exact fp64 result y64 and
its correctly rounded bf16 value y16:
  E1  ||y_gpu - y64||_2 / ||y64||_2 <= max(2e-3, 1.05 * floor), where floor
      is the same ratio for the correctly rounded y16: on a small sample the
      bf16 output rounding alone can exceed 2e-3, and no bf16 answer can beat
      the correctly rounded one
  E2  max_i |y_gpu,i - y16,i| <= 1e-2 * rms(y64), except elements where
      y_gpu,i is the other bf16 neighbour of y64,i and y64,i lies within eps_i
      of the midpoint of the two neighbours (an fp32 evaluation may round
      either way there).  eps_i = 4 * 2^-24 * (sum_k |x w| + off * sum_k |x| s)
      bounds the fp32 error of a sum whose terms are x * (c + off) * s, which
      is how the kernels evaluate it (off = 136, 144, 128 for int4/5/8).
"""
from __future__ import annotations

import numpy as np

OFFSET = {4: 136, 5: 144, 8: 128}


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def compare(y_gpu_bits: np.ndarray, y64: np.ndarray, abs_xw: np.ndarray, abs_xs: np.ndarray, K: int,
            bits: int) -> dict:
    import oracle

    y_gpu_bits = np.ascontiguousarray(y_gpu_bits, dtype=np.uint16)
    yg = bf16_bits_to_f64(y_gpu_bits)
    y16_bits = oracle.round_bf16_array(y64)
    y16 = bf16_bits_to_f64(y16_bits)
    norm = float(np.linalg.norm(y64))
    rel_l2 = float(np.linalg.norm(yg - y64)) / norm if norm > 0 else float(np.linalg.norm(yg))
    floor = float(np.linalg.norm(y16 - y64)) / norm if norm > 0 else 0.0
    rms = float(np.sqrt(np.mean(y64 ** 2))) if y64.size else 0.0
    tol = 1e-2 * rms
    err = np.abs(yg - y16)
    eps = 4.0 * 2.0 ** -24 * (abs_xw + OFFSET[bits] * abs_xs)
    neighbours = (np.abs(y_gpu_bits.astype(np.int32) - y16_bits.astype(np.int32)) == 1) & \
        ((y_gpu_bits & 0x8000) == (y16_bits & 0x8000))
    mid = 0.5 * (yg + y16)
    exempt = neighbours & (np.abs(y64 - mid) <= eps)
    over = err > tol
    return {
        "rel_l2": rel_l2,
        "rel_l2_rne_floor": floor,
        "rel_l2_gate": max(2e-3, 1.05 * floor),
        "max_err_over_rms": float(err.max() / rms) if err.size and rms > 0 else 0.0,
        "max_err_vs_y64_over_rms": float(np.abs(yg - y64).max() / rms) if err.size and rms > 0 else 0.0,
        "n": int(y64.size),
        "n_differ_from_rne": int(np.count_nonzero(y_gpu_bits != y16_bits)),
        "n_over_tol": int(np.count_nonzero(over)),
        "n_tie_exempt": int(np.count_nonzero(over & exempt)),
        "n_fail": int(np.count_nonzero(over & ~exempt)),
        "nonfinite": int(np.count_nonzero(~np.isfinite(yg))),
    }


def assert_parity(rep: dict, what: str = ""):
    assert rep["nonfinite"] == 0, (what, rep)
    assert rep["rel_l2"] <= rep["rel_l2_gate"], (what, rep)
    assert rep["n_fail"] == 0, (what, rep)


def rel_l2_gate(y_bits_or_f64, exact: np.ndarray) -> tuple:
    """(relative L2 error, gate) of a bf16 result against exact values, with the
    same floor rule as E1."""
    import oracle

    yg = y_bits_or_f64 if y_bits_or_f64.dtype == np.float64 else bf16_bits_to_f64(y_bits_or_f64)
    y16 = bf16_bits_to_f64(oracle.round_bf16_array(exact))
    norm = float(np.linalg.norm(exact))
    rel = float(np.linalg.norm(yg - exact)) / norm
    floor = float(np.linalg.norm(y16 - exact)) / norm
    return rel, max(2e-3, 1.05 * floor)
