"""The parity checkers themselves, exercised on the CPU with the oracle's own results: an exact
copy passes, a planted mistake fails.  No GPU is involved."""
import os
import sys

import numpy as np
import pytest

import oracle
from moe_synth import workloads as W
from oracle.layer import RefLayer, stack_forward

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from parity import bf16_to_f64, check_output, check_stack, stack_workloads, xn_bound  # noqa: E402


@pytest.fixture(scope="module")
def stack_run():
    oracle.set_threads(min(8, os.cpu_count() or 1))
    wl = stack_workloads()[0].with_m(3)
    Rs = [RefLayer(wl, layer=l) for l in range(wl.n_layers)]
    h0 = W.tokens_bf16(wl, 5, 3)
    trace, h_out = stack_forward(Rs, h0, wl.rms_eps)
    return wl, Rs, trace, h_out


def _as_gpu(trace):
    return [(h.copy(), ids.copy(), w.astype(np.float32)) for (h, _, ids, w, _, _) in trace]


def test_stack_check_accepts_the_oracle_itself(stack_run):
    wl, Rs, trace, h_out = stack_run
    st = check_stack(_as_gpu(trace), h_out.copy(), trace, h_out, Rs, wl.rms_eps, wl.n_experts,
                     wl.has_shared)
    assert st == {"checked": 3 * wl.n_layers, "diverged": 0}


def test_stack_check_rejects_a_wrong_residual(stack_run):
    wl, Rs, trace, h_out = stack_run
    g = _as_gpu(trace)
    h = g[1][0]
    v = bf16_to_f64(h[0:1, 10:11])[0, 0]
    h[0, 10] = np.float32(v * 1.5 + 0.25).view(np.uint32) >> 16  # a 50% error in one element
    with pytest.raises(AssertionError):
        check_stack(g, h_out.copy(), trace, h_out, Rs, wl.rms_eps, wl.n_experts, wl.has_shared)


def test_stack_check_rejects_swapped_ids(stack_run):
    wl, Rs, trace, h_out = stack_run
    g = _as_gpu(trace)
    ids = g[2][1]
    ids[1, 0], ids[1, 1] = ids[1, 1], ids[1, 0]
    with pytest.raises(AssertionError):
        check_stack(g, h_out.copy(), trace, h_out, Rs, wl.rms_eps, wl.n_experts, wl.has_shared)


def test_stack_check_rejects_a_wrong_final_residual(stack_run):
    wl, Rs, trace, h_out = stack_run
    bad = h_out.copy()
    bad[2, 7] ^= 0x0100  # flip an exponent bit
    with pytest.raises(AssertionError):
        check_stack(_as_gpu(trace), bad, trace, h_out, Rs, wl.rms_eps, wl.n_experts,
                    wl.has_shared)


def test_xn_bound_zero_for_identical_rows_and_covers_a_perturbed_row(stack_run):
    wl, Rs, trace, h_out = stack_run
    h, xn = trace[1][0], trace[1][1]
    assert np.all(xn_bound(h, h, Rs[1].gamma, wl.rms_eps) == 0.0)
    h2 = h.copy()
    h2[0, 3] += 1  # one bf16 ulp in one element of token 0
    d = xn_bound(h2, h, Rs[1].gamma, wl.rms_eps)
    xn2 = oracle.rmsnorm(h2, Rs[1].gamma, wl.rms_eps)
    diff = np.abs(bf16_to_f64(xn2) - bf16_to_f64(xn))
    assert np.all(diff <= d)
    assert np.all(d[1:] == 0.0) and d[0].max() > 0.0


def test_output_check_rejects_a_dropped_term():
    rng = np.random.default_rng(3)
    y = rng.standard_normal((4, 256))
    bits = (y.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    check_output(bits, bf16_to_f64(bits))
    y2 = y.copy()
    y2[1, 5] += 0.5  # one term missing from one element
    with pytest.raises(AssertionError):
        check_output(bits, y2)
