"""Pins of the CPU reference against facts that do not come from the reference itself:
published tables and test vectors, library routines, closed forms, invariants and
brute force on tiny inputs.  CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch

import moe_synth
import oracle
from moe_synth import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---- seeded generator ------------------------------------------------------------------------

def test_splitmix64_published_vectors():
    g = gold("splitmix64_seed1234567.json")
    state, out = g["seed"], []
    for _ in range(5):
        state = (state + 0x9E3779B97F4A7C15) & 0xFFFFFFFFFFFFFFFF
        out.append(moe_synth.mix64(state))
    assert out == g["outputs"]


def test_generator_moments_and_determinism():
    key = moe_synth.stream_key(7, moe_synth.TAG_W13, 2, 5)
    v = moe_synth.normal_f32(key, 0, 1 << 20, 0.0, 0.02).astype(np.float64)
    assert abs(v.mean()) < 4 * 0.02 / 1024
    assert abs(v.std() / 0.02 - 1.0) < 5e-3
    # a slice starting mid-stream equals the same elements of the full stream
    w = moe_synth.normal_f32(key, 1000, 50, 0.0, 0.02)
    assert np.array_equal(w, v[1000:1050].astype(np.float32))
    g = moe_synth.normal_f32(moe_synth.stream_key(7, moe_synth.TAG_GAMMA), 0, 1 << 16, 1.0, 0.1)
    assert abs(g.mean() - 1.0) < 0.003 and abs(g.std() - 0.1) < 0.002
    b = moe_synth.normal_bf16(key, 0, 1 << 10, 0.0, 0.02)
    f = moe_synth.normal_f32(key, 0, 1 << 10, 0.0, 0.02)
    # bf16 bits are the nearest-even rounding of the fp32 values (checked through torch)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, ref)


# ---- element formats -------------------------------------------------------------------------

def test_e2m1_table_matches_mx_spec():
    g = gold("e2m1_ocp_table.json")
    vals = [oracle.e2m1_value(c) for c in range(16)]
    assert vals == g["values_by_code"]
    assert [math.copysign(1, v) for v in vals] == [math.copysign(1, v) for v in g["values_by_code"]]
    assert len(vals) == 16 and all(math.isfinite(v) for v in vals)
    assert max(vals) == 1.5 * 2 ** g["emax"]


def test_e8m0_values():
    assert oracle.e8m0_value(127) == 1.0
    assert oracle.e8m0_value(0) == 2.0 ** -127
    assert oracle.e8m0_value(254) == 2.0 ** 127
    assert math.isnan(oracle.e8m0_value(255))


def test_e4m3_decode_matches_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert nan.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(ref[~nan], got[~nan])
    assert oracle.e4m3_value(0x7E) == 448.0


def test_e4m3_rne_matches_torch_cast():
    rng = np.random.default_rng(1)
    t = np.concatenate([
        rng.uniform(0, 448, 20000), rng.uniform(0, 2 ** -6, 5000),
        np.exp(rng.uniform(np.log(2 ** -12), np.log(448), 20000)),
    ]).astype(np.float32)
    # every midpoint between adjacent finite codes, exactly (midpoints are fp32-representable)
    pos = np.array([oracle.e4m3_value(c) for c in range(0x7F)])
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    t = np.concatenate([t, mids, pos.astype(np.float32)])
    ref = torch.from_numpy(t).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_rne(float(v)) for v in t], np.uint8)
    assert np.array_equal(got, ref)
    assert oracle.e4m3_rne(460.0) == 0x7E and oracle.e4m3_rne(1e6) == 0x7E  # saturation


def test_e2m1_rne_midpoints_ties_to_even():
    # Grid 0,0.5,1,1.5,2,3,4,6 (codes 0..7); every midpoint goes to the even code.
    expect = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for t, c in expect.items():
        assert oracle.e2m1_rne(t) == c, t
    for c, v in enumerate([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]):
        assert oracle.e2m1_rne(v) == c
    eps = 2.0 ** -20
    assert oracle.e2m1_rne(0.25 + eps) == 1 and oracle.e2m1_rne(0.75 - eps) == 1
    assert oracle.e2m1_rne(5.0 + eps) == 7 and oracle.e2m1_rne(6.9) == 7 and oracle.e2m1_rne(1e9) == 7


def test_bf16_from_double_single_rounding():
    def bits(x):
        return oracle.bf16_from_double(x)
    assert bits(1.0) == 0x3F80
    assert bits(1.0 + 2 ** -8) == 0x3F80            # tie -> even (down)
    assert bits(1.0 + 3 * 2 ** -8) == 0x3F82        # tie -> even (up)
    assert bits(1.0 + 2 ** -8 + 2 ** -40) == 0x3F81  # just above the tie: one rounding only
    assert bits(-2.5) == 0xC020
    assert bits(2.0 ** -133) == 0x0001 and bits(2.0 ** -134) == 0x0000
    assert bits(3.0e38) == 0x7F62                   # 1.765625 * 2^127, nearest
    assert bits(3.3961e38) == 0x7F7F                # below the last finite midpoint
    assert bits(3.3963e38) == 0x7F80                # above it -> inf
    assert bits(1e39) == 0x7F80
    # agreement with fp32 -> bf16 nearest-even (torch) for values exact in fp32
    rng = np.random.default_rng(3)
    v = (rng.standard_normal(5000) * 10.0 ** rng.integers(-30, 30, 5000)).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([bits(float(x)) for x in v], np.uint16)
    assert np.array_equal(got, ref)


# ---- MXFP4 quantizer -------------------------------------------------------------------------

def _rand_w(rows, cols, seed, sigma=0.02):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((rows, cols)) * sigma).astype(np.float32)


def test_mxfp4_shared_exponent_closed_form():
    w = np.zeros((6, 32), np.float32)
    w[0, 5] = 1.0            # amax = 2^0  -> X = -2
    w[1, 0] = 0.75           # amax in [2^-1, 2^0) -> X = -3
    w[2, 31] = -6.0          # amax = 6 -> floor(log2 6) = 2 -> X = 0
    w[3, 7] = np.nextafter(np.float32(4.0), np.float32(0))  # just below 4 -> X = -1
    w[4, :] = 0.0            # all zero -> X = -127
    w[5, 3] = np.float32(2.0 ** -140)  # denormal amax -> clamp X = -127
    q, s, n = oracle.quant_mxfp4(w)
    assert n == 0
    assert list(s[:, 0].astype(int) - 127) == [-2, -3, 0, -1, -127, -127]
    # 1.0 / 2^-2 = 4 -> code 6 ; -6 / 2^0 -> code 7 | sign
    assert (q[0, 2] & 0xF0) >> 4 == 6 and (q[2, 15] >> 4) == 0xF
    assert np.all(q[4] == 0)


def test_mxfp4_exact_values_round_trip():
    rng = np.random.default_rng(5)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    for X in (-10, -3, 0, 4):
        v = grid[rng.integers(0, 8, (4, 64))] * rng.choice([-1, 1], (4, 64))
        v[:, ::32] = 6.0  # amax = 6 * 2^X fixes the block exponent to X
        w = (v * 2.0 ** X).astype(np.float32)
        q, s, _ = oracle.quant_mxfp4(w)
        assert np.all(s == X + 127)
        d = oracle.dequant(oracle.WFMT_MXFP4, q, s, 4, 64)
        assert np.array_equal(d, w.astype(np.float64))


def test_mxfp4_invariants():
    w = _rand_w(16, 256, 11)
    q, s, _ = oracle.quant_mxfp4(w)
    # sign symmetry: codes flip bit 3 of every nibble, scales unchanged
    qn, sn, _ = oracle.quant_mxfp4(-w)
    assert np.array_equal(qn, q ^ 0x88) and np.array_equal(sn, s)
    # power-of-two shift: same codes, scale + n
    for n in (-5, 3):
        qs, ss, _ = oracle.quant_mxfp4((w * np.float32(2.0 ** n)).astype(np.float32))
        assert np.array_equal(qs, q) and np.array_equal(ss.astype(int), s.astype(int) + n)
    # idempotence
    d = oracle.dequant(oracle.WFMT_MXFP4, q, s, 16, 256)
    q2, s2, _ = oracle.quant_mxfp4(d.astype(np.float32))
    assert np.array_equal(q2, q) and np.array_equal(s2, s)
    # error bound: half the local spacing (2^X * 0.5 * 2^max(e,0)) inside the grid, < 2*2^X when clipped
    scale = np.repeat(2.0 ** (s.astype(np.float64) - 127), 32, axis=1)
    t = np.abs(w.astype(np.float64)) / scale
    err = np.abs(d - w) / scale
    spacing = np.where(t < 2, 0.5, np.where(t < 4, 1.0, 2.0))
    inside = t <= 6
    assert np.all(err[inside] <= spacing[inside] / 2 + 1e-12)
    assert np.all(err[~inside] < 2.0)


def test_mxfp4_nonfinite_block():
    w = _rand_w(2, 64, 2)
    w[1, 40] = np.inf
    w[0, 3] = np.nan
    q, s, n = oracle.quant_mxfp4(w)
    assert n == 2
    assert s[1, 1] == 0xFF and s[0, 0] == 0xFF and np.all(q[1, 16:] == 0)
    assert s[0, 1] != 0xFF and s[1, 0] != 0xFF


def test_mxfp4_negative_zero_keeps_sign():
    w = np.zeros((1, 32), np.float32)
    w[0, 0] = 1.0
    w[0, 1] = -0.01  # |t| = 0.04 -> magnitude 0, sign kept -> code 8
    q, s, _ = oracle.quant_mxfp4(w)
    assert q[0, 0] == (6 | (8 << 4))


# ---- FP8 block-scaled quantizer ---------------------------------------------------------------

def test_fp8_b128_scale_and_codes():
    w = _rand_w(256, 384, 21)
    q, s, n = oracle.quant_fp8_b128(w)
    assert n == 0 and s.shape == (2, 3)
    for br in range(2):
        for bc in range(3):
            blk = w[br * 128:(br + 1) * 128, bc * 128:(bc + 1) * 128]
            amax = np.float32(np.abs(blk).max())
            assert s[br, bc] == amax / np.float32(448.0)  # numpy fp32 division (IEEE)
            t = (blk / s[br, bc]).astype(np.float32)
            ref = torch.from_numpy(np.ascontiguousarray(t)).to(torch.float8_e4m3fn)
            ref = ref.view(torch.uint8).numpy()
            assert np.array_equal(q[br * 128:(br + 1) * 128, bc * 128:(bc + 1) * 128], ref)
    d = oracle.dequant(oracle.WFMT_FP8_B128, q, s, 256, 384)
    big = np.abs(w) >= np.repeat(np.repeat(s, 128, 0), 128, 1) * 2.0 ** -6
    rel = np.abs(d - w)[big] / np.abs(w)[big]
    assert rel.max() <= 2.0 ** -4 + 1e-7


def test_fp8_exact_values_round_trip_and_zero_block():
    rng = np.random.default_rng(8)
    pos = np.array([oracle.e4m3_value(c) for c in range(0x7F)])
    v = pos[rng.integers(0, 0x7F, (128, 256))] * rng.choice([-1, 1], (128, 256))
    v[0, 0] = 448.0
    v[0, 128] = -448.0
    w = (v * 2.0 ** -9).astype(np.float32)
    w[:, 128:] = 0.0
    w[0, 128] = 0.0
    q, s, _ = oracle.quant_fp8_b128(w)
    assert s[0, 0] == np.float32(2.0 ** -9) and s[0, 1] == 1.0
    d = oracle.dequant(oracle.WFMT_FP8_B128, q, s, 128, 256)
    assert np.array_equal(d, w.astype(np.float64))
    assert np.all(q[:, 128:] == 0)


def test_fp8_ragged_blocks_equal_zero_padded_blocks():
    """A side that is not a multiple of 128 (a tensor-parallel rank's 192-wide slice of the GLM
    intermediate): the last block along it covers the remaining rows / columns only.  Zeros
    change neither a block's maximum nor any code, so the ragged matrix's codes, scales and
    dequantized values are those of the matrix zero-padded to whole blocks, cut back to shape
    (the whole-block quantizer is pinned above by the torch E4M3 cast)."""
    for rows, cols in ((200, 96), (384, 192), (5120 // 16, 192), (128, 176)):
        w = _rand_w(rows, cols, rows + cols)
        w[rows - 1, cols - 1] = 0.05  # a large value in the partial corner block
        pr, pc = -(-rows // 128) * 128, -(-cols // 128) * 128
        wp = np.zeros((pr, pc), np.float32)
        wp[:rows, :cols] = w
        q, s, n = oracle.quant_fp8_b128(w)
        qp, sp, n_p = oracle.quant_fp8_b128(wp)
        assert n == n_p == 0 and s.shape == (pr // 128, pc // 128)
        assert np.array_equal(s, sp)
        assert np.array_equal(q, qp[:rows, :cols])
        d = oracle.dequant(oracle.WFMT_FP8_B128, q, s, rows, cols)
        dp = oracle.dequant(oracle.WFMT_FP8_B128, qp, sp, pr, pc)
        assert np.array_equal(d, dp[:rows, :cols])
    # a non-finite value marks only its own (partial) block
    w = _rand_w(128, 192, 5)
    w[3, 150] = np.inf
    q, s, n = oracle.quant_fp8_b128(w)
    assert n == 1 and np.isnan(s[0, 1]) and np.isfinite(s[0, 0])
    assert np.all(q[:, 128:] == 0x7F) and not np.any(q[:, :128] == 0x7F)


def test_ffn_fp8_ragged_intermediate_matches_numpy():
    """The FFN on a 192-wide FP8 intermediate (partial last scale block along I) against a
    numpy float64 composition of the dequantized weights."""
    H, I, E = 256, 192, 3
    rng = np.random.default_rng(12)
    experts = {}
    for e in range(E):
        experts[e] = oracle.quant_fp8_b128(_rand_w(2 * I, H, 100 + e))[:2] + \
            oracle.quant_fp8_b128(_rand_w(H, I, 200 + e))[:2]
    x = (rng.standard_normal((2, H))).astype(np.float32)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    ids = np.array([[0, 2], [1, 2]], np.int32)
    wts = np.array([[0.25, 1.0], [0.75, 1.0]], np.float32)
    y = oracle.expert_ffn(oracle.WFMT_FP8_B128, H, I, E, experts, xb, ids, wts)
    xv = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = np.zeros((2, H))
    for t in range(2):
        for j in range(2):
            q13, s13, q2, s2 = experts[int(ids[t, j])]
            w13 = oracle.dequant(oracle.WFMT_FP8_B128, q13, s13, 2 * I, H)
            w2 = oracle.dequant(oracle.WFMT_FP8_B128, q2, s2, H, I)
            g, u = w13[:I] @ xv[t], w13[I:] @ xv[t]
            ref[t] += float(wts[t, j]) * (w2 @ (g / (1 + np.exp(-g)) * u))
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


# ---- W8A8: live FP8 activation quantizer -------------------------------------------------------

def _e4m3_nearest_brute(t):
    """Brute force: the E4M3FN magnitude code nearest |t| (ties to the even code), clamped to
    448, for fp32 t; the candidates are all 127 finite magnitudes."""
    pos = np.array([oracle.e4m3_value(c) for c in range(0x7F)])
    a = np.minimum(np.abs(np.asarray(t, np.float64)), 448.0)
    d = np.abs(a[..., None] - pos)
    best = d.min(axis=-1, keepdims=True)
    cand = np.where(d == best, np.arange(0x7F), 10 ** 6)
    even = np.where(cand % 2 == 0, cand, 10 ** 6).min(axis=-1)
    return np.where(even < 10 ** 6, even, cand.min(axis=-1)).astype(np.uint8)


def test_act_fp8_scales_and_codes_brute_force():
    rng = np.random.default_rng(31)
    M, n = 3, 1024
    # log-uniform magnitudes over 2^-30 .. 2^10 so blocks reach E4M3's subnormal range
    v = (2.0 ** rng.uniform(-30, 10, (M, n)) * rng.choice([-1, 1], (M, n))).astype(np.float32)
    v[1, 128:256] = 0.0                       # all-zero block: scale 1, codes 0
    v[2, 300] = -0.0
    v[2, 256:384] *= np.float32(2.0 ** -100)  # a block of fp32-subnormal-scale values
    q, s, nbad = oracle.quant_act_fp8(v)
    assert nbad == 0 and q.shape == v.shape and s.shape == (M, n // 128)
    for t in range(M):
        for b in range(n // 128):
            blk = v[t, b * 128:(b + 1) * 128]
            amax = np.float32(np.abs(blk).max())
            sc = np.float32(1.0) if amax == 0 else amax / np.float32(448.0)  # IEEE fp32 division
            assert s[t, b] == sc
            tt = (blk / sc).astype(np.float32)
            ref = _e4m3_nearest_brute(tt) | np.where(np.signbit(blk), 0x80, 0).astype(np.uint8)
            assert np.array_equal(q[t, b * 128:(b + 1) * 128], ref), (t, b)
            # the largest element takes the largest code, up to the rounding of the scale
            assert q[t, b * 128 + int(np.abs(blk).argmax())] & 0x7F >= (0x7E if amax else 0)
    # error bound: half an E4M3 ulp, relative 2^-4 in the normal range, absolute s*2^-10 below
    d = np.vectorize(oracle.e4m3_value)(q) * np.repeat(s.astype(np.float64), 128, axis=1)
    sc = np.repeat(s.astype(np.float64), 128, axis=1)
    err = np.abs(d - v.astype(np.float64))
    normal = np.abs(v) >= sc * 2.0 ** -6
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(v.astype(np.float64))[normal] * (1 + 1e-6))
    assert np.all(err[~normal] <= sc[~normal] * 2.0 ** -10 * (1 + 1e-6))
    assert q[1, 128:256].max() == 0 and s[1, 1] == 1.0 and q[2, 300] == 0x80


def test_act_fp8_exact_round_trip_and_nonfinite_block():
    rng = np.random.default_rng(32)
    pos = np.array([oracle.e4m3_value(c) for c in range(0x7F)])
    v = pos[rng.integers(0, 0x7F, (2, 384))] * rng.choice([-1, 1], (2, 384))
    v[:, ::128] = -448.0
    k = np.array([[-12], [3]])
    x = (v * np.repeat(2.0 ** np.repeat(k, 3, axis=1), 128, axis=1)).astype(np.float32)
    q, s, nbad = oracle.quant_act_fp8(x)
    assert nbad == 0 and np.array_equal(s, (2.0 ** np.repeat(k, 3, axis=1)).astype(np.float32))
    d = np.vectorize(oracle.e4m3_value)(q) * np.repeat(s.astype(np.float64), 128, axis=1)
    assert np.array_equal(d, x.astype(np.float64))
    y = x.copy()
    y[0, 130] = np.inf
    y[1, 383] = np.nan
    q2, s2, nbad2 = oracle.quant_act_fp8(y)
    assert nbad2 == 2 and np.isnan(s2[0, 1]) and np.isnan(s2[1, 2])
    assert np.all(q2[0, 128:256] == 0x7F) and np.all(q2[1, 256:] == 0x7F)
    keep = np.ones_like(s2, bool)
    keep[0, 1] = keep[1, 2] = False
    assert np.array_equal(s2[keep], s[keep])


def _act_fake_quant(v64):
    q, s, _ = oracle.quant_act_fp8(np.asarray(v64, np.float64).astype(np.float32))
    return np.vectorize(oracle.e4m3_value)(q) * np.repeat(s.astype(np.float64), 128, axis=-1)


def test_ffn_w8a8_quantizes_both_activations():
    """W8A8 FFN against a numpy composition: x and the SwiGLU output enter their projections as
    the values of their activation codes; the weights are the FP8_B128 ones."""
    H, I, E, M = 256, 256, 4, 2
    rng = np.random.default_rng(33)
    dense, packed = {}, {}
    for e in range(E):
        w13, w2 = _exact_fp8_matrix(2 * I, H, rng), _exact_fp8_matrix(H, I, rng)
        q13, s13, _ = oracle.quant(oracle.WFMT_FP8_B128, w13)
        q2, s2, _ = oracle.quant(oracle.WFMT_FP8_B128, w2)
        packed[e] = (q13, s13, q2, s2)
        dense[e] = (w13.astype(np.float64), w2.astype(np.float64))
    x = _bf16(rng.standard_normal((M, H)) * 3)
    ids = np.array([[2, 0, 3], [1, 3, 3]], np.int32)
    w = np.array([[0.6, 0.4, 1.0], [0.25, 0.75, 1.0]], np.float32)
    y8 = oracle.expert_ffn(oracle.WFMT_FP8_B128_A8, H, I, E, packed, x, ids, w)
    y16 = oracle.expert_ffn(oracle.WFMT_FP8_B128, H, I, E, packed, x, ids, w)
    xq = _act_fake_quant(_bf16_val(x))
    for t in range(M):
        ref = np.zeros(H)
        for j in range(3):
            w13, w2 = dense[ids[t, j]]
            a = _silu(w13[:I] @ xq[t]) * (w13[I:] @ xq[t])
            ref += np.float64(w[t, j]) * (w2 @ _act_fake_quant(a))
        assert np.allclose(y8[t], ref, rtol=1e-12, atol=1e-15 * np.abs(ref).max())
    # the variant is live: it differs from W8A16, by a few percent of the output's rms
    rel = np.abs(y8 - y16).max() / np.sqrt(np.mean(y16 ** 2))
    assert 1e-4 < rel < 0.2


# ---- router ----------------------------------------------------------------------------------

def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def _bf16_val(b):
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_router_brute_force_and_shared_slot():
    g = gold("page_numbers.json")["novita_shared_fusion"]
    E, H, k, M = g["n_routed"], 512, g["top_k_routed"], 5
    rng = np.random.default_rng(4)
    x = _bf16(rng.standard_normal((M, H)))
    wr = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    b = (rng.standard_normal(E) * 0.5).astype(np.float32)
    ids, w, logits, gap = oracle.route(x, wr, b, k, 1)
    assert ids.shape == (M, g["fused_top"])
    ref = _bf16_val(x) @ wr.astype(np.float64).T + b
    assert np.allclose(logits, ref, rtol=0, atol=1e-12)
    for t in range(M):
        order = np.lexsort((np.arange(E), -ref[t]))
        assert list(ids[t, :k]) == list(order[:k])
        sig = 1 / (1 + np.exp(-ref[t, order[:k]]))
        assert np.allclose(w[t, :k], sig / sig.sum(), rtol=1e-14)
        assert abs(w[t, :k].sum() - 1) < 1e-14
        assert ids[t, g["shared_position_1based"] - 1] == g["fused_total"] - 1  # shared = E
        assert w[t, k] == 1.0
        assert abs(gap[t] - (ref[t, order[k - 1]] - ref[t, order[k]])) < 1e-12


def test_router_ties_go_to_lower_index():
    E, H, k = 12, 64, 3
    x = _bf16(np.zeros((1, H)))
    wr = _rand_w(E, H, 1)
    ids, w, _, gap = oracle.route(x, wr, None, k, 1)
    assert list(ids[0]) == [0, 1, 2, E] and np.allclose(w[0, :k], 1 / k) and gap[0] == 0
    # duplicated router rows: equal logits, lower index wins
    rng = np.random.default_rng(9)
    x = _bf16(rng.standard_normal((1, H)))
    wr = _rand_w(E, H, 2)
    ids0, *_ = oracle.route(x, wr, None, 1, 0)
    top = int(ids0[0, 0])
    dup = E - 1 if top != E - 1 else 0
    wr2 = wr.copy()
    wr2[dup] = wr[top]
    ids1, *_ = oracle.route(x, wr2, None, 2, 0)
    assert list(ids1[0]) == sorted([top, dup])
    # bias-only ordering
    b = np.float32(np.arange(E)[::-1] * 0.1)
    b = np.ascontiguousarray(b[np.random.default_rng(3).permutation(E)])
    ids2, *_ = oracle.route(_bf16(np.zeros((1, H))), wr, b, 4, 0)
    assert list(ids2[0]) == list(np.argsort(-b, kind="stable")[:4])


# ---- expert FFN --------------------------------------------------------------------------------

def _exact_mx_matrix(rows, cols, rng):
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    v = grid[rng.integers(0, 8, (rows, cols))] * rng.choice([-1, 1], (rows, cols))
    v[:, ::32] = 6.0
    X = rng.integers(-9, -5, (rows, cols // 32))
    return (v * np.repeat(2.0 ** X, 32, axis=1)).astype(np.float32)


def _exact_fp8_matrix(rows, cols, rng):
    pos = np.array([oracle.e4m3_value(c) for c in range(0x7F)])
    v = pos[rng.integers(0, 0x7F, (rows, cols))] * rng.choice([-1, 1], (rows, cols))
    v[::128, ::128] = 448.0
    return (v * 2.0 ** -14).astype(np.float32)


def _silu(z):
    return z / (1 + np.exp(-z))


@pytest.mark.parametrize("wfmt", [oracle.WFMT_MXFP4, oracle.WFMT_FP8_B128])
def test_ffn_matches_numpy_on_exactly_representable_weights(wfmt):
    H, I, E, M, S = 256, 128, 5, 3, 3
    rng = np.random.default_rng(12 + wfmt)
    mk = _exact_mx_matrix if wfmt == oracle.WFMT_MXFP4 else _exact_fp8_matrix
    dense, packed = {}, {}
    for e in range(E):
        w13 = mk(2 * I, H, rng)
        w2 = mk(H, I, rng)
        q13, s13, _ = oracle.quant(wfmt, w13)
        q2, s2, _ = oracle.quant(wfmt, w2)
        packed[e] = (q13, s13, q2, s2)
        dense[e] = (w13.astype(np.float64), w2.astype(np.float64))
    x = _bf16(rng.standard_normal((M, H)))
    ids = np.array([[0, 3, 4], [2, 1, 4], [3, 0, 4]], np.int32)
    w = np.array([[0.6, 0.4, 1.0], [0.3, 0.7, 1.0], [0.5, 0.5, 1.0]], np.float32)
    y = oracle.expert_ffn(wfmt, H, I, E, packed, x, ids, w)
    xd = _bf16_val(x)
    for t in range(M):
        ref = np.zeros(H)
        for j in range(S):
            w13, w2 = dense[ids[t, j]]
            g, u = w13[:I] @ xd[t], w13[I:] @ xd[t]
            ref += np.float64(w[t, j]) * (w2 @ (_silu(g) * u))
        assert np.allclose(y[t], ref, rtol=1e-12, atol=1e-15 * np.abs(ref).max())


def _tiny_layer(seed=0):
    wl = W.WORKLOADS["tiny"]
    rng = np.random.default_rng(seed)
    packed = {}
    for e in range(wl.n_experts):
        q13, s13, _ = oracle.quant_mxfp4(_rand_w(2 * wl.inter, wl.hidden, 100 + e + seed))
        q2, s2, _ = oracle.quant_mxfp4(_rand_w(wl.hidden, wl.inter, 200 + e + seed))
        packed[e] = (q13, s13, q2, s2)
    x = _bf16(rng.standard_normal((4, wl.hidden)))
    return wl, packed, x


def _ffn(wl, packed, x, ids, w):
    return oracle.expert_ffn(wl.wfmt, wl.hidden, wl.inter, wl.n_experts, packed, x,
                             np.asarray(ids, np.int32), np.asarray(w, np.float32))


def test_ffn_fused_shared_equals_separate():
    wl, packed, x = _tiny_layer()
    E = wl.n_routed
    ids = np.array([[1, 5, E], [0, 7, E], [2, 2 + 1, E], [6, 4, E]], np.int32)
    w = np.array([[0.7, 0.3, 1.0], [0.2, 0.8, 1.0], [0.5, 0.5, 1.0], [0.9, 0.1, 1.0]], np.float32)
    fused = _ffn(wl, packed, x, ids, w)
    routed = _ffn(wl, packed, x, ids[:, :2], w[:, :2])
    shared = _ffn(wl, packed, x, ids[:, 2:], w[:, 2:])
    assert np.array_equal(fused, routed + shared)


def test_ffn_identical_experts_zero_input_relabel_rows():
    wl, packed, x = _tiny_layer(1)
    E = wl.n_routed
    same = {e: packed[0] for e in range(E)}
    same[E] = packed[E]
    w = np.array([[0.25, 0.75, 1.0]] * 4, np.float32)
    ya = _ffn(wl, same, x, [[1, 2, E]] * 4, w)
    yb = _ffn(wl, same, x, [[5, 7, E]] * 4, w)
    one = _ffn(wl, same, x, [[0, E]] * 4, [[1.0, 1.0]] * 4)
    assert np.allclose(ya, yb, rtol=1e-13) and np.allclose(ya, one, rtol=1e-12, atol=1e-15)
    z = _ffn(wl, packed, np.zeros_like(x), [[1, 2, E]] * 4, w)
    assert np.all(z == 0)
    # relabel experts: permute the stored experts and the ids together
    perm = np.random.default_rng(2).permutation(E)
    relab = {int(perm[e]): packed[e] for e in range(E)}
    relab[E] = packed[E]
    ids = np.array([[1, 6, E], [3, 0, E], [4, 5, E], [2, 7, E]], np.int32)
    ids_p = ids.copy()
    ids_p[:, :2] = perm[ids[:, :2]]
    assert np.array_equal(_ffn(wl, packed, x, ids, w), _ffn(wl, relab, x, ids_p, w))
    # each row of an M-token call equals the one-token call on that row
    full = _ffn(wl, packed, x, ids, w)
    for t in range(4):
        assert np.array_equal(full[t], _ffn(wl, packed, x[t:t + 1], ids[t:t + 1], w[t:t + 1])[0])


# ---- RMSNorm / residual ------------------------------------------------------------------------

def test_rmsnorm_against_numpy_and_invariants():
    rng = np.random.default_rng(6)
    H = 7168
    h = _bf16(rng.standard_normal((3, H)) * 3)
    gamma = (1 + 0.1 * rng.standard_normal(H)).astype(np.float32)
    out = oracle.rmsnorm(h, gamma, 1e-6)
    hv = _bf16_val(h)
    ref = hv / np.sqrt((hv ** 2).mean(axis=1, keepdims=True) + 1e-6) * gamma
    got = _bf16_val(out)
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-30)
    h2 = _bf16(_bf16_val(h) * 4.0)
    assert np.mean(oracle.rmsnorm(h2, gamma, 1e-6) == out) > 0.999
    c = _bf16(np.full((1, H), 2.0))
    assert np.array_equal(oracle.rmsnorm(c, gamma, 1e-6), _bf16(gamma.reshape(1, H)))


def test_residual_rounds_once():
    h = _bf16(np.array([1.0, -2.0, 0.0], np.float32))
    y = np.array([2.0 ** -8 + 2.0 ** -40, 2.0 ** -7, 1e-3])
    out = oracle.residual(h, y)
    assert list(out) == [0x3F81, oracle.bf16_from_double(-2.0 + 2.0 ** -7),
                         oracle.bf16_from_double(1e-3)]


# ---- byte model against the pages' arithmetic ------------------------------------------------

def test_bytes_model_against_pages():
    g = gold("page_numbers.json")
    s = g["sionic_bandwidth"]
    assert round(s["active_bytes_per_rank_gb"] / s["peak_tb_s"], 2) == s["ideal_ms"]
    for tbs, pct in s["effective"]:
        assert round(100 * tbs / s["peak_tb_s"]) == pct
    f = g["xiaomi_fp4_bytes"]
    wl = W.WORKLOADS["glm_mx_m4"]
    codes_fp4 = 3 * wl.hidden * wl.inter // 2
    assert codes_fp4 / (3 * wl.hidden * wl.inter) == f["fp4_over_fp8"]
    assert codes_fp4 / (2 * 3 * wl.hidden * wl.inter) == f["fp4_over_fp16"]
    n = g["novita_shared_fusion"]
    assert W.WORKLOADS["glm_fp8_m1"].inter // 8 == n["per_rank_inter_tp8"]
    assert W.WORKLOADS["glm_fp8_m1"].n_experts == n["fused_total"]
    assert W.WORKLOADS["glm_fp8_m1"].slots == n["fused_top"]


# ---- verify-acceptance of a speculative block ------------------------------------------------

def _softmax64(L):
    L = np.asarray(L, np.float64)
    e = np.exp(L - L.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def test_verify_greedy_prefix_and_ties():
    """Greedy: the drafts are accepted while they equal each row's argmax (lowest index on
    ties); the next token is that row's argmax (a correction, or the bonus token)."""
    rng = np.random.default_rng(41)
    K, V = 6, 300
    L = rng.standard_normal((K + 1, V)).astype(np.float32)
    g = L.argmax(axis=1)
    for n in range(K + 1):
        d = g[:K].copy()
        if n < K:
            d[n] = (g[n] + 1 + rng.integers(V - 1)) % V
        out, _ = oracle.verify(L, d)
        assert list(out) == list(g[:n]) + [int(g[n])], n
    # equal maxima: the lowest index wins
    L2 = np.zeros((2, 8), np.float32)
    L2[0, [3, 5]] = 2.0
    L2[1, [6, 1]] = 1.0
    assert list(oracle.verify(L2, np.array([3]))[0]) == [3, 1]
    assert list(oracle.verify(L2, np.array([5]))[0]) == [3]
    # out-of-range drafts are never accepted; K = 0 returns the argmax of row 0
    assert list(oracle.verify(L2, np.array([-1]))[0]) == [3]
    assert list(oracle.verify(L2[:1], np.zeros(0, np.int32))[0]) == [3]


def test_verify_sampling_special_cases():
    rng = np.random.default_rng(42)
    K, V = 4, 64
    L = (rng.standard_normal((K + 1, V)) * 2).astype(np.float32)
    P = _softmax64(L)
    # draft equal to the target: every draft token is accepted (u q < p for u < 1), and the
    # bonus token is the inverse-CDF draw from p_K
    Q = P[:K].astype(np.float32)
    for trial in range(20):
        d = np.array([rng.choice(V, p=P[i] / P[i].sum()) for i in range(K)], np.int32)
        d = np.where(Q[np.arange(K), d] > 0, d, P[:K].argmax(1)).astype(np.int32)
        u = rng.random(K + 1).astype(np.float32)
        out, _ = oracle.verify(L, d, Q, u)
        assert len(out) == K + 1 and list(out[:K]) == list(d)
        c = np.cumsum(P[K])
        assert out[K] == int(np.searchsorted(c, np.float64(u[K]) * c[-1], side="right"))
    # q(d) = 0 with p(d) > 0 is accepted; p(d) = 0 (logit -inf) is rejected
    L2 = L.copy()
    L2[0, 5] = -np.inf
    Q2 = np.full((K, V), 1.0 / V, np.float32)
    Q2[0, 7] = 0.0
    u = np.full(K + 1, 0.999, np.float32)
    out, _ = oracle.verify(L2, np.array([7, 0, 0, 0], np.int32), Q2, u)
    assert out[0] == 7
    out, _ = oracle.verify(L2, np.array([5, 0, 0, 0], np.int32), Q2, u)
    assert len(out) == 1 and out[0] != 5
    # a residual that sums to zero (q = 2 p: rejected for u >= 1/2) falls back to a draw from p
    Q3 = np.minimum(2 * P[:K], 1).astype(np.float32)
    d = P[:K].argmax(1).astype(np.int32)
    u = np.array([0.75, 0.1, 0.1, 0.1, 0.3], np.float32)
    out, _ = oracle.verify(L, d, Q3, u)
    c = np.cumsum(P[0])
    assert len(out) == 1 and out[0] == int(np.searchsorted(c, 0.3 * c[-1], side="right"))


def test_verify_sampling_is_lossless_on_a_tiny_vocabulary():
    """The property the pages name: rejection sampling leaves the output distribution unchanged.
    Over many draws of draft tokens d ~ q and uniforms, the first output token follows p_0, and
    the first draft token is accepted with probability sum_x min(p_0(x), q_0(x))."""
    rng = np.random.default_rng(43)
    K, V, trials = 2, 5, 40000
    L = (rng.standard_normal((K + 1, V)) * 1.5).astype(np.float32)
    P = _softmax64(L)
    Q = _softmax64(rng.standard_normal((K, V)) * 1.5).astype(np.float32)
    Qn = Q.astype(np.float64) / Q.astype(np.float64).sum(1, keepdims=True)
    first = np.zeros(V)
    accepted = 0
    for _ in range(trials):
        d = np.array([rng.choice(V, p=Qn[i]) for i in range(K)], np.int32)
        u = rng.random(K + 1).astype(np.float32)
        out, _ = oracle.verify(L, d, Q, u)
        first[out[0]] += 1
        accepted += len(out) > 1
    emp = first / trials
    sd = np.sqrt(P[0] * (1 - P[0]) / trials)
    assert np.all(np.abs(emp - P[0]) < 5 * sd + 1e-4), (emp, P[0])
    alpha = np.minimum(P[0], Q[0].astype(np.float64)).sum()
    assert abs(accepted / trials - alpha) < 5 * np.sqrt(alpha * (1 - alpha) / trials)


# ---- fused QK-norm + RoPE -----------------------------------------------------------------------

def _qk(x, nq, pos, gq, gk, eps=1e-6, theta=10000.0, rot=64):
    return oracle.qk_norm_rope(_bf16(x), nq, np.asarray(pos), gq, gk, eps, theta, rot)


def test_qk_norm_rope_position_zero_is_headwise_rmsnorm():
    rng = np.random.default_rng(51)
    M, nq, nh, hd = 3, 4, 6, 128
    x = rng.standard_normal((M, nh, hd)) * 2
    gq = (1 + 0.1 * rng.standard_normal(hd)).astype(np.float32)
    gk = (1 + 0.1 * rng.standard_normal(hd)).astype(np.float32)
    y, yb = _qk(x, nq, np.zeros(M), gq, gk, eps=1e-5)
    xb = _bf16_val(_bf16(x))
    r = 1 / np.sqrt((xb * xb).mean(axis=2, keepdims=True) + 1e-5)
    ref = xb * r * np.where(np.arange(nh)[None, :, None] < nq, gq.astype(np.float64),
                            gk.astype(np.float64))
    assert np.allclose(y, ref, rtol=1e-14, atol=0)
    assert np.array_equal(yb, _bf16(y.astype(np.float32))) or \
        np.all(np.abs(_bf16_val(yb) - y) <= np.abs(y) * 2.0 ** -8)


def test_qk_norm_rope_pairing_sign_and_frequencies():
    """One-hot heads pin the half-split pairing, the rotation's sign and the frequencies:
    with theta = 16 and rot = 8 the pair i turns by pos * 2^-i exactly."""
    hd, rot = 64, 8
    g = np.ones(hd, np.float32)
    for i in range(rot // 2):
        x = np.zeros((1, 1, hd))
        x[0, 0, i] = 1.0
        for pos in (1, 3, 100):
            y, _ = _qk(x, 1, [pos], g, g, eps=0.0, theta=16.0, rot=rot)
            n0 = np.sqrt(hd)  # the head's RMS is 1/sqrt(hd)
            ang = pos * 2.0 ** -i
            assert abs(y[0, 0, i] - n0 * np.cos(ang)) < 1e-12 * n0
            assert abs(y[0, 0, i + rot // 2] - n0 * np.sin(ang)) < 1e-12 * n0
            others = np.delete(y[0, 0], [i, i + rot // 2])
            assert np.all(others == 0)


def test_qk_norm_rope_invariants():
    """Rotation keeps every pair's length and leaves the dimensions past rot untouched, and the
    q.k product over the rotated dimensions depends only on the position difference (the
    property rotary embedding is built for)."""
    rng = np.random.default_rng(52)
    nq, nh, hd, rot = 1, 2, 128, 64
    x = rng.standard_normal((1, nh, hd))
    g = (1 + 0.1 * rng.standard_normal(hd)).astype(np.float32)
    y0, _ = _qk(x, nq, [0], g, g, rot=rot)
    ym, _ = _qk(x, nq, [37], g, g, rot=rot)
    h = rot // 2
    assert np.allclose(ym[..., :h] ** 2 + ym[..., h:rot] ** 2, y0[..., :h] ** 2 + y0[..., h:rot] ** 2,
                       rtol=1e-13)
    assert np.array_equal(ym[..., rot:], y0[..., rot:])
    dots = []
    for m, n in ((50, 20), (80, 50), (1030, 1000)):
        yq, _ = _qk(x, nq, [m], g, g, rot=rot)
        yk, _ = _qk(x, nq, [n], g, g, rot=rot)
        dots.append(float(yq[0, 0, :rot] @ yk[0, 1, :rot]))
    assert np.allclose(dots, dots[0], rtol=1e-11), dots
    yq, _ = _qk(x, nq, [51], g, g, rot=rot)
    assert abs(float(yq[0, 0, :rot] @ yk[0, 1, :rot]) - dots[0]) > 1e-6 * abs(dots[0])
