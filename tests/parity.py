"""Helpers of the GPU parity tests: the output tolerance and oracle/GPU layer pairs."""
from __future__ import annotations

import os

import numpy as np

import oracle
from moe_synth import workloads as W


def oracle_threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def ulp_bf16(v: np.ndarray) -> np.ndarray:
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    u = np.exp2(e - 7)
    return np.where(a >= 2.0 ** -126, u, 2.0 ** -133)


def check_output(y_gpu_bits: np.ndarray, y_ref: np.ndarray, rows=None) -> float:
    """|y_gpu - y_ref| <= 1e-2 * rms(y_ref) + ulp_bf16(y_ref), elementwise over the checked rows
    (rms over the same rows).  Returns max error / rms."""
    g = bf16_to_f64(np.asarray(y_gpu_bits).view(np.uint16))
    r = np.asarray(y_ref, np.float64)
    if rows is not None:
        g, r = g[rows], r[rows]
    assert np.all(np.isfinite(r))
    rms = float(np.sqrt(np.mean(r * r)))
    err = np.abs(g - r)
    bound = 1e-2 * rms + ulp_bf16(r)
    bad = err > bound
    assert not bad.any(), (f"{bad.sum()} elements out of tolerance; worst err {err.max():.3e}, "
                           f"rms {rms:.3e}")
    return float(err.max() / rms) if rms > 0 else 0.0


def check_residual(h_next_bits: np.ndarray, h_in_bits: np.ndarray, y_ref: np.ndarray) -> float:
    """A residual update h' = bf16(h + y): |h'_gpu - (h + y_ref)| <= 1e-2 * rms(y_ref) +
    ulp_bf16(h + y_ref), elementwise (the output tolerance on y plus the final rounding)."""
    g = bf16_to_f64(np.asarray(h_next_bits).view(np.uint16))
    ref = bf16_to_f64(np.asarray(h_in_bits).view(np.uint16)) + np.asarray(y_ref, np.float64)
    assert np.all(np.isfinite(ref))
    rms = float(np.sqrt(np.mean(np.asarray(y_ref, np.float64) ** 2)))
    err = np.abs(g - ref)
    bad = err > 1e-2 * rms + ulp_bf16(ref)
    assert not bad.any(), (f"{bad.sum()} elements out of tolerance; worst err {err.max():.3e}, "
                           f"rms(y) {rms:.3e}")
    return float(err.max() / rms) if rms > 0 else 0.0


def check_route(ids_gpu, w_gpu, ids_ref, w_ref, gap_ref):
    """Ids bit-exact and weights within 2^-20 relative.  Tokens whose reference gap at the
    k boundary is below 1e-9 would be near-ties; none are expected in fp64."""
    assert np.all(gap_ref > 1e-9), f"near-tie token(s): min gap {gap_ref.min():.3e}"
    assert np.array_equal(ids_gpu, ids_ref)
    assert np.all(np.abs(w_gpu.astype(np.float64) - w_ref) <= 2.0 ** -20 * np.abs(w_ref))


def stack_workloads():
    """Test-only multi-layer shapes (RMSNorm eps 1e-6, independent draws per layer)."""
    return [
        W.Workload("stack_mid_mx", 15, 1024, 256, 24, 6, 1, W.WFMT_MXFP4, 1, bias_sigma=0.5,
                   n_layers=3),
        W.Workload("stack_mid_fp8", 16, 640, 384, 20, 4, 1, W.WFMT_FP8_B128, 1, n_layers=3),
    ]


def mid_workloads():
    """Test-only shapes the reference finishes in a second: several tiles, ragged tails."""
    return [
        W.Workload("mid_fp8", 11, 640, 384, 20, 4, 1, W.WFMT_FP8_B128, 1),
        W.Workload("mid_mx_bias", 12, 1024, 256, 24, 6, 1, W.WFMT_MXFP4, 1, bias_sigma=0.5),
        W.Workload("mid_mx_noshared", 13, 1152, 384, 12, 3, 0, W.WFMT_MXFP4, 1),
        W.Workload("mid_fp8_k1", 14, 1280, 256, 7, 1, 1, W.WFMT_FP8_B128, 1),
    ]
