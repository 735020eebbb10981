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


def check_route(ids_gpu, w_gpu, ids_ref, w_ref, gap_ref):
    """Ids bit-exact and weights within 2^-20 relative.  Tokens whose reference gap at the
    k boundary is below 1e-9 would be near-ties; none are expected in fp64."""
    assert np.all(gap_ref > 1e-9), f"near-tie token(s): min gap {gap_ref.min():.3e}"
    assert np.array_equal(ids_gpu, ids_ref)
    assert np.all(np.abs(w_gpu.astype(np.float64) - w_ref) <= 2.0 ** -20 * np.abs(w_ref))


def xn_bound(h_gpu_bits: np.ndarray, h_ref_bits: np.ndarray, gamma: np.ndarray,
             eps: float) -> np.ndarray:
    """Elementwise bound on |xn_gpu - xn_ref| where xn = bf16((h * r) * gamma), r = 1 /
    sqrt(mean(h^2) + eps), for two layer inputs h that may differ.  Rows with identical input
    have identical xn (one rounding of the same value), bound 0.  Otherwise the unrounded values
    of the two inputs differ by |a - b| and each side's rounding moves its value by at most half
    an ulp of its own magnitude."""
    hg = bf16_to_f64(np.asarray(h_gpu_bits).view(np.uint16))
    hr = bf16_to_f64(np.asarray(h_ref_bits).view(np.uint16))
    g = np.asarray(gamma, np.float64)
    rg = 1.0 / np.sqrt(np.mean(hg * hg, axis=1, keepdims=True) + eps)
    rr = 1.0 / np.sqrt(np.mean(hr * hr, axis=1, keepdims=True) + eps)
    a, b = hg * rg * g, hr * rr * g
    d = np.abs(a - b) + 0.5 * ulp_bf16(a) + 0.5 * ulp_bf16(b)
    same = np.all(hg == hr, axis=1)
    d[same] = 0.0
    return d


def check_stack(gpu_layers, h_out_gpu, ref_trace, h_out_ref, ref_layers, eps: float,
                n_experts: int, has_shared: int) -> dict:
    """Free-running comparison of a layer stack with the oracle's run from the same h0.

    gpu_layers[l] = (h_in bits [T][H], ids [T][S], w [T][S]) from the GPU's trace and
    ref_trace[l] = oracle.layer.stack_forward's record, both for the same T tokens.
    - Layer 0's input is h0 on both sides, bit for bit.
    - Layer l's input: |h_gpu - h_ref| within the sum over earlier layers of the one-layer output
      tolerance (1e-2 * rms(y_ref) + ulp_bf16 of the new residual), i.e. per-layer errors add.
    - Routing: a logit can move by at most B = max_e sum_k |Wr[e][k]| * xn_bound_k (+ 1e-9 for
      fp64 summation order).  Where the oracle's gap at the k boundary exceeds B the ids must
      match exactly and the weights agree within 2^-20 + 2.5 B relative (sigmoid slope <= 1/4,
      renormalized).  Where it does not, a differing pick is legitimate: that token is checked
      for valid ids from then on and leaves the comparison.
    - The final residual: same tolerance as an input.
    Returns counts of checked and diverged (token, layer) cases."""
    T = gpu_layers[0][0].shape[0]
    live = np.ones(T, bool)
    tol = None
    stats = {"checked": 0, "diverged": 0}

    def check_h(hg, hr, rows):
        g = bf16_to_f64(np.asarray(hg).view(np.uint16))[rows]
        r = bf16_to_f64(np.asarray(hr).view(np.uint16))[rows]
        err = np.abs(g - r)
        bad = err > tol[rows]
        assert not bad.any(), (f"{bad.sum()} residual elements out of tolerance; worst excess "
                               f"{(err - tol[rows]).max():.3e}")

    for l, ((hg, ig, wg), (hr, xnr, ir, wr, gap, y)) in enumerate(zip(gpu_layers, ref_trace)):
        R = ref_layers[l]
        if l == 0:
            assert np.array_equal(np.asarray(hg).view(np.uint16), hr)
        else:
            check_h(hg, hr, live)
        D = xn_bound(hg, hr, R.gamma, eps)
        B = (D @ np.abs(np.asarray(R.wr, np.float64)).T).max(axis=1) + 1e-9
        for t in range(T):
            if not live[t]:
                check_ids_valid(ig[t], n_experts, has_shared)
                continue
            stats["checked"] += 1
            if gap[t] > B[t]:
                assert np.array_equal(ig[t], ir[t]), f"layer {l} token {t}: ids differ, gap " \
                    f"{gap[t]:.3e} > bound {B[t]:.3e}"
                rel = 2.0 ** -20 + 2.5 * B[t]
                assert np.all(np.abs(wg[t].astype(np.float64) - wr[t]) <= rel * np.abs(wr[t]))
            elif not np.array_equal(ig[t], ir[t]):
                check_ids_valid(ig[t], n_experts, has_shared)
                live[t] = False
                stats["diverged"] += 1
        yv = np.asarray(y, np.float64)
        rms = np.sqrt(np.mean(yv * yv, axis=1, keepdims=True))
        hr_next = ref_trace[l + 1][0] if l + 1 < len(ref_trace) else h_out_ref
        step = 1e-2 * rms + ulp_bf16(bf16_to_f64(np.asarray(hr_next).view(np.uint16)))
        tol = step if tol is None else tol + step
    check_h(h_out_gpu, h_out_ref, live)
    return stats


def check_ids_valid(ids, n_experts: int, has_shared: int):
    """A legitimate routing of one token: distinct routed ids in [0, E), then the shared expert
    (stored last, id E = n_experts - 1) when the layer has one."""
    n_routed = n_experts - has_shared
    routed = ids[:-1] if has_shared else ids
    assert np.all((routed >= 0) & (routed < n_routed)) and len(set(routed.tolist())) == len(routed)
    if has_shared:
        assert ids[-1] == n_routed


def stack_workloads():
    """Test-only multi-layer shapes (RMSNorm eps 1e-6, independent draws per layer)."""
    return [
        W.Workload("stack_mid_mx", 15, 1024, 256, 24, 6, 1, W.WFMT_MXFP4, 1, bias_sigma=0.5,
                   n_layers=3),
        W.Workload("stack_mid_fp8", 16, 640, 384, 20, 4, 1, W.WFMT_FP8_B128, 1, n_layers=3),
    ]


def limit_workloads():
    """Shapes at the limits the C ABI accepts: 16 slots (15 routed + shared, 256 pairs at
    M = 16), 1024 routed experts, hidden 8192, the widest intermediate per format (FP8 4096,
    MXFP4 8192), and MXFP4 intermediates that are odd multiples of 32."""
    return [
        W.Workload("lim_mx_slots", 21, 256, 96, 24, 15, 1, W.WFMT_MXFP4, 1, bias_sigma=0.5),
        W.Workload("lim_mx_experts", 22, 128, 32, 1024, 8, 1, W.WFMT_MXFP4, 1, bias_sigma=0.5),
        W.Workload("lim_fp8_wide", 23, 8192, 128, 6, 2, 1, W.WFMT_FP8_B128, 1),
        W.Workload("lim_fp8_deep", 24, 128, 4096, 6, 2, 1, W.WFMT_FP8_B128, 1),
        W.Workload("lim_mx_deep", 25, 128, 8192, 4, 2, 0, W.WFMT_MXFP4, 1),
        W.Workload("lim_mx_wide", 26, 8192, 160, 4, 3, 1, W.WFMT_MXFP4, 1),
    ]


def mid_workloads():
    """Test-only shapes the reference finishes in a second: several tiles, ragged tails."""
    return [
        W.Workload("mid_fp8", 11, 640, 384, 20, 4, 1, W.WFMT_FP8_B128, 1),
        W.Workload("mid_mx_bias", 12, 1024, 256, 24, 6, 1, W.WFMT_MXFP4, 1, bias_sigma=0.5),
        W.Workload("mid_mx_noshared", 13, 1152, 384, 12, 3, 0, W.WFMT_MXFP4, 1),
        W.Workload("mid_fp8_k1", 14, 1280, 256, 7, 1, 1, W.WFMT_FP8_B128, 1),
        # the GLM intermediate (1536) at a small hidden: flattened down rows at M = 1, row
        # chunks with a workgroup per CU at M > 1
        W.Workload("mid_fp8_i1536", 27, 512, 1536, 12, 4, 1, W.WFMT_FP8_B128, 1),
        # FP8 hidden sizes with three, five and six 16-value chunks per lane (the GLM hidden
        # 5120 is five): the workgroup-per-CU gate/up at one and two units per step
        W.Workload("mid_fp8_h3072", 28, 3072, 128, 10, 3, 1, W.WFMT_FP8_B128, 1),
        W.Workload("mid_fp8_h5120", 29, 5120, 256, 9, 3, 1, W.WFMT_FP8_B128, 1),
        W.Workload("mid_fp8_h6144", 30, 6144, 128, 8, 2, 1, W.WFMT_FP8_B128, 1),
        # the GLM intermediate in MXFP4 (48 chunks, 96 eight-byte granules per down row):
        # flattened down rows at every token count
        W.Workload("mid_mx_i1536", 33, 512, 1536, 12, 4, 1, W.WFMT_MXFP4, 1),
        # FP8 intermediates that are not whole 128-blocks (partial last scale block along I)
        W.Workload("mid_fp8_i160", 31, 640, 160, 10, 3, 1, W.WFMT_FP8_B128, 1),
        W.Workload("mid_fp8_i192", 32, 1024, 192, 12, 4, 1, W.WFMT_FP8_B128, 1),
    ]


def draw_weights(L, Q, j):
    """fp64 weights of the distribution the next token is drawn from after j accepted drafts:
    max(0, p_j - q_j) at a rejection (p_j when that is zero everywhere), p_K after a full
    accept; p_i = softmax(row i), straight from its definition."""
    row = np.asarray(L[j], np.float64)
    p = np.exp(row - row.max())
    p /= p.sum()
    if Q is not None and j < Q.shape[0]:
        r = np.maximum(p - np.asarray(Q[j], np.float64), 0.0)
        if r.sum() > 0.0:
            return r
    return p


def check_verify_sampling(L, Q, d, u, got, tol=1e-5, mass_tol=2e-6):
    """A verify-acceptance result `got` (the accepted drafts then the drawn token) against the
    oracle on one sampling block.  The GPU sums fp32 exponentials (relative error ~1e-7) where
    the oracle uses fp64, so a decision within `tol` of its threshold may go either way.
    - Accepted count: equal to the oracle's unless the oracle saw an accept test that close; if
      the counts differ, the first position where the two sides disagree must be such a test
      (|p_i(d_i) - u_i q_i(d_i)| <= tol max(p, u q)).
    - Drawn token: equal to the oracle's when the counts agree and the oracle's draw was not
      that close to a bucket edge; otherwise u_K T must fall in the token's bucket of the draw's
      cumulative sum (index order, in probability units: T = 1 for p, the residual's mass after
      a rejection), widened on both sides by tol T plus mass_tol, the probability mass the
      GPU's fp32 exponentials can misplace (relative error <= ~1e-6 per value of p, so at most
      ~1e-6 of mass over a row).  A residual whose mass is of that order (p and q equal to fp32
      precision) is drawn from rounding noise on either side and only checked for validity.
    Returns (count exact, token exact)."""
    ref, (m_acc, m_draw) = oracle.verify(L, d, Q, u)
    got = np.asarray(got)
    K, V = L.shape[0] - 1, L.shape[1]
    n = len(got) - 1
    assert 0 <= n <= K and list(got[:n]) == list(d[:n]) and 0 <= got[n] < V, (got, ref)
    count_exact = m_acc > tol
    if count_exact:
        assert len(got) == len(ref), (got, ref, m_acc)
    elif len(got) != len(ref):
        i = min(len(got), len(ref)) - 1  # first position decided differently
        row = np.asarray(L[i], np.float64)
        pi = np.exp(row[d[i]] - row.max()) / np.exp(row - row.max()).sum()
        uq = float(u[i]) * float(Q[i, d[i]])
        assert abs(pi - uq) <= tol * max(pi, uq), (i, pi, uq)
    token_exact = count_exact and m_draw > tol
    if token_exact:
        assert got[n] == ref[n], (got, ref, m_draw)
    else:
        w = draw_weights(L, Q, n)
        c = np.cumsum(w)
        T = c[-1]
        t = float(u[K]) * T
        lo, hi = c[got[n]] - w[got[n]], c[got[n]]
        slack = tol * T + mass_tol
        assert lo - slack <= t < hi + slack, (int(got[n]), lo / T, hi / T, float(u[K]), T)
    return count_exact, token_exact


# ---- canary guards ---------------------------------------------------------------------------

GUARD_BYTES = 4096
GUARD_BYTE = 0xA5


class Guarded:
    """A device buffer of `nbytes` between two GUARD_BYTES regions filled with GUARD_BYTE: `inner`
    is the buffer handed to the library, `intact()` reports whether both guards still hold only
    the fill byte (anything written past either end of the buffer changes them)."""

    def __init__(self, nbytes: int, dtype=None, shape=None):
        import torch
        self.nbytes = int(nbytes)
        self.buf = torch.full((self.nbytes + 2 * GUARD_BYTES,), GUARD_BYTE, dtype=torch.uint8,
                              device="cuda")
        inner = self.buf[GUARD_BYTES:GUARD_BYTES + self.nbytes]
        if dtype is not None:
            inner = inner.view(dtype)
            if shape is not None:
                inner = inner.view(shape)
        self.inner = inner

    def intact(self) -> bool:
        import torch
        lo = self.buf[:GUARD_BYTES]
        hi = self.buf[GUARD_BYTES + self.nbytes:]
        return bool(torch.all(lo == GUARD_BYTE).item()) and bool(torch.all(hi == GUARD_BYTE).item())

