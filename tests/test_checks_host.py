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
from parity import (bf16_to_f64, check_ids_valid, check_output, check_stack,  # noqa: E402
                    check_verify_sampling, draw_weights, stack_workloads, xn_bound)


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


def _verify_block(K, V, seed, noise, sigma):
    rng = np.random.default_rng(seed)
    L = (rng.standard_normal((K + 1, V)) * sigma).astype(np.float32)
    D = L[:K].astype(np.float64) + rng.standard_normal((K, V)) * noise
    Q = np.exp(D - D.max(axis=1, keepdims=True))
    Q = (Q / Q.sum(axis=1, keepdims=True)).astype(np.float32)
    d = np.array([rng.choice(V, p=Q[i].astype(np.float64) / Q[i].astype(np.float64).sum())
                  for i in range(K)], np.int32)
    u = rng.random(K + 1).astype(np.float32)
    return L, Q, d, u


def test_verify_sampling_check_accepts_the_oracle_itself():
    """The oracle's own results pass, exact and bucket-checked alike (flat rows put most draws
    into buckets narrower than the margin)."""
    seen_bucket = seen_exact = 0
    for trial in range(12):
        L, Q, d, u = _verify_block(4, 151552, 70 + trial, (0.5, 4.0)[trial % 2],
                                   6.0 if trial % 3 == 0 else 1.0)
        ref, _ = oracle.verify(L, d, Q, u)
        _, token_exact = check_verify_sampling(L, Q, d, u, ref)
        seen_bucket += not token_exact
        seen_exact += token_exact
    assert seen_bucket > 0 and seen_exact > 0


def test_verify_sampling_check_rejects_planted_errors():
    """A drawn token two buckets away, a token past the vocabulary, a wrong accepted prefix and
    an accepted count that differs at a position far from its threshold all fail."""
    L, Q, d, u = _verify_block(4, 4096, 5, 0.5, 1.0)
    ref, (m_acc, _) = oracle.verify(L, d, Q, u)
    assert m_acc > 1e-5
    n = len(ref) - 1
    w = draw_weights(L, Q, n)
    c = np.cumsum(w)
    far = int(np.searchsorted(c, (float(u[-1]) + 0.3) % 1.0 * c[-1], side="right"))
    for bad_tok in (far, 4096):
        bad = ref.copy()
        bad[n] = bad_tok
        with pytest.raises(AssertionError):
            check_verify_sampling(L, Q, d, u, bad)
    if n > 0:
        bad = ref.copy()
        bad[0] = (bad[0] + 1) % 4096
        with pytest.raises(AssertionError):
            check_verify_sampling(L, Q, d, u, bad)
    shorter = np.concatenate([ref[:max(n - 1, 0)], [ref[n]]]) if n > 0 else None
    longer = np.concatenate([d[:n + 1], [ref[n]]]) if n < 4 else None
    for bad in (shorter, longer):
        if bad is not None:
            with pytest.raises(AssertionError):
                check_verify_sampling(L, Q, d, u, bad)


def test_ids_validity_check():
    """The routing validity check of diverged stack tokens: distinct routed ids below E, then
    the shared expert's id E; a wrong shared id, a duplicate or an id past E fails."""
    E1 = 385  # 384 routed + shared
    ok = np.array([3, 7, 383, 0, 12, 99, 5, 200, 384])
    check_ids_valid(ok, E1, 1)
    for bad in ([3, 7, 383, 0, 12, 99, 5, 200, 385], [3, 3, 383, 0, 12, 99, 5, 200, 384],
                [3, 7, 384, 0, 12, 99, 5, 200, 384]):
        with pytest.raises(AssertionError):
            check_ids_valid(np.array(bad), E1, 1)
    check_ids_valid(np.array([0, 5, 2]), 8, 0)
    with pytest.raises(AssertionError):
        check_ids_valid(np.array([0, 5, 8]), 8, 0)
