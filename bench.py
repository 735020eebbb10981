#!/usr/bin/env python3
"""Benchmark of the MoE decode layer on one MI355X.

One step = one pass of the decode hot path over one fresh token block: router, expert FFN
and combine in one call (moe_layer_decode: the results of moe_route_topk followed by
moe_expert_ffn_decode; with one token the gate/up kernel selects the experts itself), on the
GLM-4.7-shaped layer (hidden 5120, 160 routed + 1 shared expert fused as the
ninth slot, intermediate 1536, FP8 E4M3 weights with 128x128 fp32 block scales,
one decode token).  The value is the achieved HBM bandwidth on active expert
bytes: the packed bytes (codes + scales) of the distinct experts the step's
tokens selected, summed over the timed steps, divided by the timed wall time.

Weights are rotated over R independent layer copies (different seeds) so that
the 256 MB last-level cache cannot serve an expert from a previous step; tokens
come from a pool of 1000 pre-generated tokens.  All inputs are synthetic and
device-resident before timing starts.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_TBS = 8.0


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def active_bytes(ids: np.ndarray, wl) -> int:
    """Packed bytes of the distinct valid experts referenced by one step's ids [M][S]."""
    from moe_synth.workloads import packed_bytes_per_expert
    ex = np.unique(ids.reshape(-1))
    ex = ex[(ex >= 0) & (ex < wl.n_experts)]
    return int(ex.size) * packed_bytes_per_expert(wl)


def gateup_kernel_name(wl) -> str:
    """Name of the one-token gate/up kernel instantiation the library launches for this
    workload (the last argument, several W8A8 tokens, is false at one token)."""
    vals = 32 if wl.wfmt == 1 else 16
    ns = (wl.hidden // vals + 63) // 64
    fmt, a8 = (2, "true") if wl.wfmt == 3 else (wl.wfmt, "false")
    return f"gateup_kernel<{fmt}, {ns}, {a8}, false>"


def measure(wl, copies: int, steps: int, warmup: int, pool: int = 1000, one_launch=False):
    """Time `steps` decode steps of workload `wl` (moe_layer_decode, or with one_launch
    moe_layer_decode_one_launch).  Returns a dict of results."""
    import torch

    import bit_moe_expert_route_amd as moe
    from bit_moe_expert_route_amd.synthetic import GpuLayer, tokens

    M, S = wl.m, wl.slots
    t0 = time.time()
    staging = None
    layers = []
    for c in range(copies):
        g = GpuLayer(wl, layer=c, staging=staging)
        staging = g.staging
        layers.append(g)
    del staging
    for g in layers:
        g.staging = None
    torch.cuda.synchronize()
    log(f"{wl.name}: built {copies} layer copies in {time.time() - t0:.1f}s")
    descs = [g.desc for g in layers]
    ws = moe.new_workspace(descs, M)
    xpool = tokens(wl, 0, pool * M).view(pool, M, wl.hidden)
    n_total = warmup + steps
    ids_all = torch.empty((n_total, M, S), dtype=torch.int32, device="cuda")
    w_all = torch.empty((n_total, M, S), dtype=torch.float32, device="cuda")
    y = torch.empty((M, wl.hidden), dtype=torch.int16, device="cuda")

    decode = moe.layer_decode_one_launch if one_launch else moe.layer_decode

    def step(i):
        decode(descs[i % copies], xpool[i % pool], M, ids_all[i], w_all[i], y, ws,
               stream=torch.cuda.current_stream())

    def gate_up_only(i):
        moe.expert_gate_up(descs[i % copies], xpool[i % pool], M, ids_all[i], ws,
                           stream=torch.cuda.current_stream())

    def staged_step(i, ev_a, ev_b):
        """The same step with the gate/up stage (the dominant kernel) bracketed by events."""
        d = descs[i % copies]
        x = xpool[i % pool]
        s = torch.cuda.current_stream()
        moe.route_topk(d, x, M, ids_all[i], w_all[i], None, ws, stream=s)
        ev_a.record(s)
        moe.expert_gate_up(d, x, M, ids_all[i], ws, stream=s)
        ev_b.record(s)
        moe.expert_down_combine(d, M, ids_all[i], w_all[i], y, ws, stream=s)

    def ffn_only(i):
        d = descs[i % copies]
        moe.expert_ffn_decode(d, xpool[i % pool], M, ids_all[i], w_all[i], y, ws,
                              stream=torch.cuda.current_stream())

    # eager pass over every step (warm-up, fills the routing of every step)
    for i in range(n_total):
        step(i)
    torch.cuda.synchronize()
    # eager timing of the timed steps (host launch gaps included), also per step
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    pev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    start.record()
    pev[0].record()
    for k in range(steps):
        step(warmup + k)
        pev[k + 1].record()
    end.record()
    torch.cuda.synchronize()
    eager_ms = start.elapsed_time(end)
    step_us = np.array([1000.0 * pev[k].elapsed_time(pev[k + 1]) for k in range(steps)])
    # live duration of the gate/up launch inside eager steps (events on the launch stream)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for k in range(steps):
        staged_step(warmup + k, *evs[k])
    torch.cuda.synchronize()
    gateup_us = np.array([1000.0 * a.elapsed_time(b) for a, b in evs])
    # the same steps captured as one HIP graph: back-to-back launches, no host gaps
    g_step, g_ffn, g_gu = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g_step, stream=side):
            for k in range(steps):
                step(warmup + k)
        with torch.cuda.graph(g_ffn, stream=side):
            for k in range(steps):
                ffn_only(warmup + k)
        with torch.cuda.graph(g_gu, stream=side):
            for k in range(steps):
                gate_up_only(warmup + k)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g_step.replay()
    g_ffn.replay()
    g_gu.replay()
    torch.cuda.synchronize()
    start.record()
    g_step.replay()
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    start.record()
    g_ffn.replay()
    end.record()
    torch.cuda.synchronize()
    ffn_total_ms = start.elapsed_time(end)
    # the gate/up launches of the same steps back to back: its average launch duration
    start.record()
    g_gu.replay()
    end.record()
    torch.cuda.synchronize()
    gu_total_ms = start.elapsed_time(end)
    ids_np = ids_all[warmup:].cpu().numpy()
    bytes_steps = np.array([active_bytes(ids_np[k], wl) for k in range(steps)], np.float64)
    n_active = np.array([np.unique(ids_np[k]).size for k in range(steps)])
    total_bytes = float(bytes_steps.sum())
    from moe_synth.workloads import w13_bytes_per_expert
    w13_steps = np.array([np.unique(ids_np[k][(ids_np[k] >= 0) & (ids_np[k] < wl.n_experts)]).size
                          for k in range(steps)], np.float64) * w13_bytes_per_expert(wl)
    res = {
        "workload": wl.name, "hidden": wl.hidden, "inter": wl.inter, "n_routed": wl.n_routed,
        "shared": wl.has_shared, "top_k": wl.top_k, "m": M,
        "wfmt": {1: "mxfp4", 2: "fp8_e4m3_b128", 3: "fp8_e4m3_b128_w8a8"}[wl.wfmt],
        "copies": copies, "steps": steps,
        "us_per_layer": 1000.0 * total_ms / steps,
        "tb_s": total_bytes / (total_ms * 1e-3) / 1e12,
        "eager_us_per_layer": 1000.0 * eager_ms / steps,
        "eager_step_us_p10_p50_p90": [round(float(np.percentile(step_us, q)), 2)
                                      for q in (10, 50, 90)],
        "ffn_us_mean": 1000.0 * ffn_total_ms / steps,
        "ffn_tb_s": total_bytes / (ffn_total_ms * 1e-3) / 1e12,
        "active_experts_mean": float(n_active.mean()),
        "active_bytes_mean": float(bytes_steps.mean()),
        "gateup_kernel": gateup_kernel_name(wl),
        "gateup_us_mean": 1000.0 * gu_total_ms / steps,
        "gateup_us_eager_bracketed": float(gateup_us.mean()),
        "gateup_bytes_mean": float(w13_steps.mean()),
        "gateup_gb_s": float(w13_steps.sum() / (gu_total_ms * 1e-3) / 1e9),
        "total_ms": total_ms,
    }
    del layers, descs, ws, xpool
    torch.cuda.empty_cache()
    return res


def measure_verify(K: int, V: int, sampling: bool, calls: int, pool: int = 32):
    """Time moe_verify_accept on synthetic verify blocks: logits N(0, 9) [K+1][V], draft
    probabilities softmax(logits + N(0, 1)) and draft tokens drawn from them, uniforms in
    [0, 1).  `pool` distinct blocks (more bytes than the 256 MB memory-side cache) rotate over
    the calls, which are captured in one graph.  Bytes: the logits once, plus, for a block with
    a rejection, the rejected row of logits and draft probabilities once more."""
    import torch

    import bit_moe_expert_route_amd as moe
    g = torch.Generator(device="cuda")
    g.manual_seed(1234 + K + V + int(sampling))
    L = torch.randn((pool, K + 1, V), generator=g, device="cuda") * 3.0
    Q = torch.softmax(L[:, :K] + torch.randn((pool, K, V), generator=g, device="cuda"), dim=-1)
    d = torch.multinomial(Q.reshape(pool * K, V), 1, generator=g).reshape(pool, K).to(torch.int32)
    u = torch.rand((pool, K + 1), generator=g, device="cuda")
    ws = moe.new_verify_workspace(K, V)
    out = torch.zeros((calls, K + 1), dtype=torch.int32, device="cuda")
    cnt = torch.zeros((calls, 1), dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream()

    def call(i):
        b = i % pool
        moe.verify_accept(L[b], d[b], out[i], cnt[i], ws, draft_probs=Q[b] if sampling else None,
                          uniforms=u[b] if sampling else None, stream=torch.cuda.current_stream())

    for i in range(calls):
        call(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(s)
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for i in range(calls):
                call(i)
    s.wait_stream(side)
    graph.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    graph.replay()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end)
    n = cnt.cpu().numpy().reshape(-1)
    rejected = float(np.mean(n < K + 1)) if sampling else 0.0
    nbytes = (K + 1) * V * 4 + (2 * V * 4 * rejected if sampling else 0)
    us = 1000.0 * ms / calls
    pool_bytes = pool * ((2 * K + 1) if sampling else (K + 1)) * V * 4
    res = {"K": K, "V": V, "mode": "sampling" if sampling else "greedy", "calls": calls,
           "us_per_call": us, "gb_s": nbytes / (us * 1e-6) / 1e9,
           "tokens_per_block_mean": float(n.mean()), "pool_bytes": pool_bytes,
           "note": "latency-bound (two or four launches of short dependency chains)"}
    del L, Q, d, u, ws
    torch.cuda.empty_cache()
    return res


def measure_qk_norm_rope(M: int, calls: int, nq: int = 96, nk: int = 8, hd: int = 128,
                         rot: int = 64, pool: int = 64):
    """Time moe_qk_norm_rope on GLM-shaped attention heads (96 query + 8 key heads of 128,
    half of each rotated, V heads after them in the row): synthetic bf16 N(0, 1) rows, random
    positions below 2^20.  `pool` row blocks rotate over the calls (in place, so each call
    normalizes an already normalized block: the work is the same), captured in one graph.
    Bytes: the q and k heads read and written once."""
    import torch

    import bit_moe_expert_route_amd as moe
    g = torch.Generator(device="cuda")
    g.manual_seed(77 + M)
    stride = (nq + 2 * nk) * hd
    qk = (torch.randn((pool, M, stride), generator=g, device="cuda")).to(torch.bfloat16)
    qk = qk.view(torch.int16)
    pos = torch.randint(0, 1 << 20, (pool, M), generator=g, device="cuda", dtype=torch.int32)
    gq = 1 + 0.1 * torch.randn(hd, generator=g, device="cuda")
    gk = 1 + 0.1 * torch.randn(hd, generator=g, device="cuda")
    s = torch.cuda.current_stream()

    def call(i):
        b = i % pool
        moe.qk_norm_rope(qk[b], M, nq, nk, hd, stride, pos[b], gq, gk, 1e-5, 1e6, rot,
                         stream=torch.cuda.current_stream())

    for i in range(pool):
        call(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(s)
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for i in range(calls):
                call(i)
    s.wait_stream(side)
    graph.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    graph.replay()
    end.record()
    torch.cuda.synchronize()
    us = 1000.0 * start.elapsed_time(end) / calls
    nbytes = 2 * M * (nq + nk) * hd * 2
    res = {"M": M, "heads": f"{nq}+{nk}x{hd}", "rot": rot, "calls": calls, "us_per_call": us,
           "gb_s": nbytes / (us * 1e-6) / 1e9,
           "note": "latency-bound; the rotating row blocks stay in the caches, so gb_s is not "
                   "an HBM figure"}
    del qk, pos
    torch.cuda.empty_cache()
    return res


def measure_stack(wl, M: int, steps: int, warmup: int):
    """Time the layer stack (moe_layer_stack_persistent over wl.n_layers layers) on fresh
    M-token blocks: each step updates its own pre-generated h block in place.  Active bytes
    come from an untimed traced pass over the same blocks (the path is deterministic)."""
    import torch

    import bit_moe_expert_route_amd as moe
    from bit_moe_expert_route_amd.synthetic import GpuLayer, tokens
    from moe_synth.workloads import packed_bytes_per_expert

    wl = wl.with_m(M)
    L, H, S = wl.n_layers, wl.hidden, wl.slots
    staging = None
    layers = []
    for l in range(L):
        g = GpuLayer(wl, layer=l, staging=staging)
        staging = g.staging
        layers.append(g)
    del staging
    for g in layers:
        g.staging = None
    descs = [g.desc for g in layers]
    arr = (moe.Layer * L)(*descs)
    ws = moe.new_workspace(descs, M)
    n_total = warmup + steps
    h0 = tokens(wl, 0, n_total * M).view(n_total, M, H)
    h = h0.clone()
    rec = M * H * 2 + 8 * M * S
    trace = torch.empty(L * rec, dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream()
    active = np.zeros(steps)
    for k in range(steps):  # traced pass: routing of every timed step
        moe.layer_stack_persistent(arr, L, wl.rms_eps, h[warmup + k], M, ws, trace=trace, stream=s)
        tr = trace.cpu().numpy()
        for l in range(L):
            r = tr[l * rec + M * H * 2:l * rec + M * H * 2 + 4 * M * S].view(np.int32)
            active[k] += np.unique(r).size * packed_bytes_per_expert(wl)
    h.copy_(h0)
    for i in range(warmup):
        moe.layer_stack_persistent(arr, L, wl.rms_eps, h[i], M, ws, stream=s)
    torch.cuda.synchronize()
    # graphs of at most 100 steps each (each step on its own block), replayed back to back
    graphs = []
    side = torch.cuda.Stream()
    side.wait_stream(s)
    with torch.cuda.stream(side):
        for k0 in range(0, steps, 100):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                for k in range(k0, min(steps, k0 + 100)):
                    moe.layer_stack_persistent(arr, L, wl.rms_eps, h[warmup + k], M, ws,
                                               stream=side)
            graphs.append(g)
    s.wait_stream(side)
    torch.cuda.synchronize()
    h[warmup:].copy_(h0[warmup:])
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for g in graphs:
        g.replay()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end)
    res = {"m": M, "layers": L, "wfmt": "mxfp4" if wl.wfmt == 1 else "fp8_e4m3_b128",
           "us_per_step": 1000.0 * ms / steps, "us_per_layer": 1000.0 * ms / steps / L,
           "tb_s": float(active.sum()) / (ms * 1e-3) / 1e12,
           "active_bytes_per_step": float(active.mean()), "steps": steps}
    res["frac_of_peak"] = res["tb_s"] / HBM_PEAK_TBS
    del layers, descs, ws, h, h0, trace, graphs
    torch.cuda.empty_cache()
    return res


def traffic_per_launch(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None when the
    summary is missing or was taken on other kernel sources than the ones built here."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "gateup_glm_fp8_m1_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in ("ffn.hip", "ffn_body.h", "ffn_common.h", "moe_device.h", "act_quant.h",
              "route_select.h"):
        h.update(open(os.path.join(ROOT, "bit_moe_expert_route_amd", "csrc", f), "rb").read())
    if vals.get("kernel") != kernel or vals.get("source_sha256") != h.hexdigest():
        return None
    return float(vals["hbm_bytes_per_launch"])


def copy_probe(nbytes: int = 256 << 20) -> None:
    """One plain device copy of known size, outside any timed region: the reference that
    scales the HBM byte counters of a profile of this command."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def read_ceiling(nbytes: int = 4 << 30, reps: int = 10):
    """The achievable-bandwidth reference: a plain streaming read (16-byte non-temporal loads)
    of a device buffer much larger than the caches, timed over `reps` reads."""
    import torch

    import moe_synth
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    moe_synth.gpu_read_probe(buf.data_ptr(), nbytes, sink.data_ptr(), s)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        moe_synth.gpu_read_probe(buf.data_ptr(), nbytes, sink.data_ptr(), s)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / reps
    del buf, sink
    torch.cuda.empty_cache()
    return {"bytes": nbytes, "us_per_read": 1000.0 * ms, "tb_s": nbytes / (ms * 1e-3) / 1e12,
            "frac_of_peak": nbytes / (ms * 1e-3) / 1e12 / HBM_PEAK_TBS}


def read_at_size(nbytes: int, rotate_bytes: int = 2 << 30, reps_per_copy: int = 8):
    """A plain streaming read of `nbytes` per launch, as a kernel of that size sees it: launches
    back to back in one graph over rotating copies (together past the memory-side cache), so
    each read comes from HBM and pays its own ramp and drain.  Best of three replays."""
    import torch

    import moe_synth
    copies = max(2, rotate_bytes // nbytes)
    bufs = [torch.ones(nbytes, dtype=torch.uint8, device="cuda") for _ in range(copies)]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    reps = reps_per_copy * copies
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        s = torch.cuda.current_stream().cuda_stream
        for r in range(reps):
            moe_synth.gpu_read_probe(bufs[r % copies].data_ptr(), nbytes, sink.data_ptr(), s)
    g.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = None
    for _ in range(3):
        start.record()
        g.replay()
        end.record()
        torch.cuda.synchronize()
        us = 1000.0 * start.elapsed_time(end) / reps
        best = us if best is None else min(best, us)
    del bufs, sink, g
    torch.cuda.empty_cache()
    return {"bytes": nbytes, "copies": copies, "us_per_read": best,
            "tb_s": nbytes / (best * 1e-6) / 1e12}


def sync_probe(chain: int = 1000, barriers: int = 1000):
    """What one grid-wide dependency costs on this GPU: as the boundary between two dependent
    launches of a full resident grid (a graph of `chain` launches that only store a word per
    workgroup), and as an in-kernel grid barrier (`barriers` device-scope counter barriers in
    one launch, without and with the release / acquire fences a data hand-off needs)."""
    import torch

    import moe_synth
    s = torch.cuda.current_stream().cuda_stream
    words = torch.zeros(4096, dtype=torch.int32, device="cuda")
    for _ in range(3):
        moe_synth.gpu_sync_step(words.data_ptr(), s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(chain):
            moe_synth.gpu_sync_step(words.data_ptr(), torch.cuda.current_stream().cuda_stream)
    g.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    g.replay()
    end.record()
    torch.cuda.synchronize()
    res = {"chain": chain, "barriers": barriers,
           "kernel_boundary_us": 1000.0 * start.elapsed_time(end) / chain}
    del g
    for fenced in (False, True):
        times = []
        for _ in range(3):
            words.zero_()
            torch.cuda.synchronize()
            start.record()
            moe_synth.gpu_grid_barrier(words.data_ptr(), barriers, fenced, s)
            end.record()
            torch.cuda.synchronize()
            if int(words[1].item()) != 0:  # a wait gave up: no time to report
                times = None
                break
            times.append(1000.0 * start.elapsed_time(end) / barriers)
        res["grid_barrier_fenced_us" if fenced else "grid_barrier_us"] = (
            min(times) if times else None)
    del words
    torch.cuda.empty_cache()
    return res


def cpu_baseline(wl, n_tokens: int = 6):
    """The CPU reference, as it stands, on a bounded sample: route + expert FFN of n_tokens
    single-token steps of the same workload (expert packing is setup, not timed)."""
    import oracle
    from moe_synth import workloads as W
    from oracle.layer import RefLayer

    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    threads = max(1, cores or 1)
    oracle.set_threads(threads)
    R = RefLayer(wl)
    xs = [W.tokens_bf16(wl, t, wl.m) for t in range(n_tokens)]
    routes = [R.route(x) for x in xs]
    for ids, *_ in routes:  # pack the experts the sample needs (untimed setup)
        for e in np.unique(ids):
            R.packed(int(e))
    t0 = time.perf_counter()
    total_bytes = 0
    for x in xs:
        y, ids, w, _ = R.forward(x)
        total_bytes += active_bytes(ids, wl)
    dt = time.perf_counter() - t0
    # the same oracle on one thread, over the first two of those steps
    oracle.set_threads(1)
    t1 = time.perf_counter()
    for x in xs[:2]:
        R.forward(x)
    dt1 = (time.perf_counter() - t1) / 2
    oracle.set_threads(threads)
    return {"value": total_bytes / dt / 1e12, "unit": "TB/s", "cores": cores,
            "threads": threads, "nproc": os.cpu_count(),
            "kind": "oracle", "us_per_layer": 1e6 * dt / n_tokens,
            "one_thread_us_per_layer": 1e6 * dt1,
            "sample": f"{n_tokens} decode steps (route + expert FFN, fp64) of {wl.name} "
                      f"with M={wl.m}, experts packed beforehand; one-thread figure over 2 of "
                      f"them"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other layers reported under 'extra'")
    ap.add_argument("--only-extra", default="",
                    help="comma-separated layer lines of 'extra' to run alone (to profile one)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the decode path "
              "runs on one GPU and has no multi-GPU sharding", file=sys.stderr)
        sys.exit(2)

    import torch
    from moe_synth import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    wl = W.WORKLOADS["glm_fp8_m1"]
    main_res = measure(wl, args.copies, args.steps, args.warmup)
    copy_probe()
    log(json.dumps(main_res))
    extra = {}
    keys = ("m", "wfmt", "us_per_layer", "tb_s", "ffn_us_mean", "ffn_tb_s", "eager_us_per_layer",
            "eager_step_us_p10_p50_p90", "active_experts_mean", "copies")
    only = set(filter(None, args.only_extra.split(",")))
    if not args.no_extra:
        n_x, w_x = max(20, args.steps // 4), max(5, args.warmup // 2)
        # the tensor-parallel ranks move ~14-26 MB per step: 64 layer copies put more than the
        # memory-side cache between two uses of a copy's shared expert
        for name, copies in (("glm_w8a8_m1", 8), ("glm_fp8_m4", 8), ("glm_w8a8_m4", 8),
                             ("glm_mx_m4", 8), ("t1_mx_m16", 4), ("tp8_glm_fp8", 64),
                             ("tp8_glm_mx", 64), ("tp8_t1_mx", 64)):
            if only and name not in only:
                continue
            r = measure(W.WORKLOADS[name], copies, n_x, w_x)
            log(json.dumps(r))
            extra[name] = {k: r[k] for k in keys}
            extra[name]["frac_of_peak"] = r["tb_s"] / HBM_PEAK_TBS
            if name == "glm_w8a8_m1":  # its dominant kernel, timed as the main line's
                extra[name]["gateup_kernel"] = r["gateup_kernel"]
                extra[name]["gateup_us"] = r["gateup_us_mean"]
                extra[name]["gateup_gb_s"] = r["gateup_gb_s"]
            if name.startswith("tp8"):
                extra[name]["note"] = "latency-bound: one rank's share moves few bytes per launch"
        if not only:
            # the main layer without rotation: its 212 MB of active experts partly stay in the
            # 256 MB memory-side cache between steps (cache-assisted, not an HBM figure)
            r = measure(wl, 1, n_x, w_x)
            extra["glm_fp8_m1_hot"] = {k: r[k] for k in keys}
            extra["glm_fp8_m1_hot"]["note"] = "cache-assisted: one layer copy, no rotation"
            # the same layer as ONE launch per step (moe_layer_decode_one_launch)
            r = measure(wl, args.copies, n_x, w_x, one_launch=True)
            log(json.dumps(r))
            extra["glm_fp8_m1_one_launch"] = {k: r[k] for k in keys}
            extra["glm_fp8_m1_one_launch"]["frac_of_peak"] = r["tb_s"] / HBM_PEAK_TBS
            # the 8-layer stack, 1000 timed steps (each on its own token block)
            for M in (1, 4):
                r = measure_stack(W.WORKLOADS["stack8"], M, 1000, w_x)
                log(json.dumps(r))
                extra[f"stack8_m{M}"] = r
            for K, sampling, pool in ((15, False, 32), (15, True, 32), (4, True, 96)):
                r = measure_verify(K, 151552, sampling, 200, pool=pool)
                log(json.dumps(r))
                extra[f"verify_k{K}_v151552_{r['mode']}"] = r
            for M in (1, 16):
                r = measure_qk_norm_rope(M, 200)
                log(json.dumps(r))
                extra[f"qk_norm_rope_glm_m{M}"] = r
            r = read_ceiling()
            log(json.dumps(r))
            extra["read_ceiling"] = r
            # the same plain read at the main line's kernel sizes (W13 and W2 bytes per launch)
            gu = int(main_res["gateup_bytes_mean"]) // 16 * 16
            dn = int(main_res["active_bytes_mean"] - main_res["gateup_bytes_mean"]) // 16 * 16
            r = {"gateup_bytes": read_at_size(gu), "down_bytes": read_at_size(dn)}
            log(json.dumps(r))
            extra["read_at_kernel_sizes"] = r
            r = sync_probe()
            log(json.dumps(r))
            extra["sync_probe"] = r
    gu_gbs = main_res["gateup_gb_s"]
    out = {
        "metric": "MoE-layer decode µs/layer + achieved HBM TB/s (active expert bytes) at M=1,4,16",
        "value": round(main_res["tb_s"], 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["us_per_layer"] / 1000.0, 5),
        "us_per_layer": round(main_res["us_per_layer"], 2),
        "eager_us_per_layer": round(main_res["eager_us_per_layer"], 2),
        "eager_step_us_p10_p50_p90": main_res["eager_step_us_p10_p50_p90"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "glm_fp8_m1: hidden 5120, 160 routed + 1 shared (top-9 of 161), "
                               "intermediate 1536, FP8 E4M3 128x128 fp32 scales, M=1",
                   "weights": "fp8_e4m3_b128 (decoded exactly to bf16)", "activations": "bf16",
                   "products": "v_dot2_f32_bf16", "accumulate": "fp32",
                   "layer_copies": args.copies, "token_pool": 1000, "parallelism": "none"},
        "roofline": {"bound": "hbm", "kernel": main_res["gateup_kernel"],
                     "timed_as": "a graph of the same steps' moe_expert_gate_up calls (experts "
                                 "from the step's ids; the step itself selects them inside the "
                                 "same kernel, about 1 us more)",
                     "achieved": round(gu_gbs, 1), "peak": HBM_PEAK_TBS * 1000.0,
                     "unit": "GB/s", "frac": round(gu_gbs / (HBM_PEAK_TBS * 1000.0), 4),
                     "traffic": traffic_per_launch(main_res["gateup_kernel"]),
                     "per_launch_us": round(main_res["gateup_us_mean"], 3),
                     "per_launch_us_eager_bracketed": round(main_res["gateup_us_eager_bracketed"],
                                                            3),
                     "algorithmic_bytes_per_launch": round(main_res["gateup_bytes_mean"]),
                     "ffn_tb_s": round(main_res["ffn_tb_s"], 4),
                     "ffn_us_per_call": round(main_res["ffn_us_mean"], 2)},
        "frac_of_peak": round(main_res["tb_s"] / HBM_PEAK_TBS, 4),
        "extra": extra,
    }
    if "read_at_kernel_sizes" in extra:
        # a plain read of the kernel's bytes per launch, against the kernel's time
        plain = extra["read_at_kernel_sizes"]["gateup_bytes"]["us_per_read"]
        out["roofline"]["plain_read_same_bytes_us"] = round(plain, 3)
        out["roofline"]["frac_of_plain_read_same_bytes"] = round(
            plain / main_res["gateup_us_mean"], 4)
    if not args.no_cpu_baseline:
        try:
            out["cpu_baseline"] = cpu_baseline(wl)
        except Exception as exc:  # the baseline is context; report why it is missing
            out["cpu_baseline"] = {"error": repr(exc)}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
