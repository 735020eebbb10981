"""Workload-level use of the CPU reference -- TEST INFRASTRUCTURE ONLY.

Generates a workload's fp32 expert weights with the shared seeded generator,
packs them with the reference quantizers (never with the GPU's), and runs the
reference router, expert FFN and layer stack on them.
"""
from __future__ import annotations

import numpy as np

from moe_synth import workloads as W

from . import expert_ffn, quant, residual, rmsnorm, route


class RefLayer:
    """One layer of a workload, experts packed by the reference quantizer on demand."""

    def __init__(self, wl: W.Workload, layer: int = 0):
        self.wl = wl
        self.layer = layer
        self._packed: dict[int, tuple] = {}
        self._wr = None
        self._b = None
        self._gamma = None

    @property
    def wr(self):
        if self._wr is None:
            self._wr = W.router_w(self.wl, self.layer)
        return self._wr

    @property
    def bias(self):
        if self._b is None and self.wl.bias_sigma:
            self._b = W.router_b(self.wl, self.layer)
        return self._b

    @property
    def gamma(self):
        if self._gamma is None:
            self._gamma = W.rms_gamma(self.wl, self.layer)
        return self._gamma

    def packed(self, e: int):
        """(q13, s13, q2, s2) for expert e, quantized by the reference."""
        if e not in self._packed:
            q13, s13, n1 = quant(self.wl.wfmt, W.w13_f32(self.wl, self.layer, e))
            q2, s2, n2 = quant(self.wl.wfmt, W.w2_f32(self.wl, self.layer, e))
            assert n1 == 0 and n2 == 0
            self._packed[e] = (q13, s13, q2, s2)
        return self._packed[e]

    def route(self, x_bf16: np.ndarray):
        wl = self.wl
        return route(x_bf16, self.wr, self.bias, wl.top_k, wl.has_shared)

    def ffn(self, x_bf16, ids, w, token_mask=None):
        wl = self.wl
        needed = set()
        for t in range(ids.shape[0]):
            if token_mask is None or token_mask[t]:
                needed.update(int(e) for e in ids[t])
        experts = {e: self.packed(e) for e in sorted(needed)}
        return expert_ffn(wl.wfmt, wl.hidden, wl.inter, wl.n_experts, experts, x_bf16, ids,
                          np.asarray(w, np.float32), token_mask)

    def forward(self, x_bf16, token_mask=None):
        """Route then FFN: returns (y fp64, ids, w fp32, gap)."""
        ids, w, _, gap = self.route(x_bf16)
        w32 = w.astype(np.float32)
        return self.ffn(x_bf16, ids, w32, token_mask), ids, w32, gap


def stack_forward(layers: list[RefLayer], h0_bf16: np.ndarray, eps: float):
    """Pre-norm residual stack: h <- bf16(h + MoE_l(RMSNorm_l(h))).  Returns the per-layer
    records [(h_in, xn, ids, w, gap, y)] and the final h."""
    h = np.ascontiguousarray(h0_bf16, dtype=np.uint16)
    trace = []
    for L in layers:
        xn = rmsnorm(h, L.gamma, eps)
        y, ids, w, gap = L.forward(xn)
        trace.append((h, xn, ids, w, gap, y))
        h = residual(h, y)
    return trace, h
