"""The five synthetic MoE decode workloads and their seeded tensors.

Shapes and distributions follow the workloads the pages discuss: a tiny
sanity layer; a GLM-4.7-shaped layer (hidden 5120, 160 routed experts plus one
shared expert fused as the ninth slot of a top-9, intermediate 1536; Novita,
"Optimizing GLM4-MoE for production", section 1, shared-expert fusion) in FP8
at one token and in MXFP4 at a 4-token verify block; a 1T-class layer (hidden
7168, 384+1 experts, intermediate 2048) in MXFP4 at a 16-token verify block with
a per-expert router bias that skews routing (molayo, "Xiaomi ... 1,000 tokens
per second", section 1 on routing imbalance, section 2 on expert-only MXFP4,
section 3 on block verification); and an 8-layer stack of the 1T-class layer.

Every tensor is a pure function of (seed, tag, layer, index, element): expert
weights N(0, 0.02) per element, router weights N(0, 0.02), router bias
N(0, 0.5) where the workload skews routing, RMSNorm gamma N(1, 0.1), tokens
bf16(N(0, 1)).  Seeds are 1000 * (workload number - 1).
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

from . import (TAG_BIAS, TAG_GAMMA, TAG_W13, TAG_W2, TAG_WR, TAG_X, normal_bf16, normal_f32,
               stream_key)

WFMT_MXFP4 = 1
WFMT_FP8_B128 = 2
WFMT_FP8_B128_A8 = 3  # FP8_B128 weights, activations quantized live (W8A8)


@dataclass(frozen=True)
class Workload:
    name: str
    number: int
    hidden: int
    inter: int
    n_routed: int
    top_k: int
    has_shared: int
    wfmt: int
    m: int
    bias_sigma: float = 0.0     # 0 -> no router bias
    n_layers: int = 1
    rms_eps: float = 1e-6
    w_sigma: float = 0.02
    wr_sigma: float = 0.02

    @property
    def seed(self) -> int:
        return 1000 * (self.number - 1)

    @property
    def n_experts(self) -> int:
        """Stored experts: routed plus the shared one (stored last)."""
        return self.n_routed + self.has_shared

    @property
    def slots(self) -> int:
        return self.top_k + self.has_shared

    def with_m(self, m: int) -> "Workload":
        return replace(self, m=m)

    def with_wfmt(self, wfmt: int, name: str | None = None) -> "Workload":
        """The same draws (same number, so same weights and tokens) in another format."""
        return replace(self, wfmt=wfmt, name=name or self.name)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 256, 128, 8, 2, 1, WFMT_MXFP4, 1),
    "glm_fp8_m1": Workload("glm_fp8_m1", 2, 5120, 1536, 160, 8, 1, WFMT_FP8_B128, 1),
    # the same layer (same draws) with live FP8 activation quantization (W8A8)
    "glm_w8a8_m1": Workload("glm_w8a8_m1", 2, 5120, 1536, 160, 8, 1, WFMT_FP8_B128_A8, 1),
    # a 4-token verify block of the same layer, W8A16 and W8A8
    "glm_fp8_m4": Workload("glm_fp8_m4", 2, 5120, 1536, 160, 8, 1, WFMT_FP8_B128, 4),
    "glm_w8a8_m4": Workload("glm_w8a8_m4", 2, 5120, 1536, 160, 8, 1, WFMT_FP8_B128_A8, 4),
    "glm_mx_m4": Workload("glm_mx_m4", 3, 5120, 1536, 160, 8, 1, WFMT_MXFP4, 4),
    "t1_mx_m16": Workload("t1_mx_m16", 4, 7168, 2048, 384, 8, 1, WFMT_MXFP4, 16, bias_sigma=0.5),
    "stack8": Workload("stack8", 5, 7168, 2048, 384, 8, 1, WFMT_MXFP4, 1, bias_sigma=0.5,
                       n_layers=8),
    # one GPU's share of a tensor-parallel-8 deployment: every expert split along the
    # intermediate axis (GLM: 1536 / 8 = 192; 1T: 2048 / 8 = 256)
    "tp8_glm_mx": Workload("tp8_glm_mx", 6, 5120, 192, 160, 8, 1, WFMT_MXFP4, 1),
    "tp8_t1_mx": Workload("tp8_t1_mx", 7, 7168, 256, 384, 8, 1, WFMT_MXFP4, 1, bias_sigma=0.5),
    # the FP8 GLM-4.7 deployment's rank (Novita, section 1: TP8, intermediate 192 per rank); the
    # FP8 block scales' last 128-block along the intermediate axis covers 64 values
    "tp8_glm_fp8": Workload("tp8_glm_fp8", 8, 5120, 192, 160, 8, 1, WFMT_FP8_B128, 1),
}


def packed_bytes_per_expert(wl: Workload) -> int:
    """Packed bytes of one expert's three matrices (codes plus scales)."""
    h, i = wl.hidden, wl.inter
    if wl.wfmt == WFMT_MXFP4:
        return 3 * h * i // 2 + 3 * h * i // 32
    # FP8: one fp32 scale per 128x128 block, the last block along the intermediate axis
    # partial when it is not a whole one
    return 3 * h * i + 4 * (h // 128) * (-(-2 * i // 128) + -(-i // 128))


def w13_bytes_per_expert(wl: Workload) -> int:
    """Packed bytes of one expert's gate/up matrix [2I][H] (codes plus scales)."""
    h, i = wl.hidden, wl.inter
    if wl.wfmt == WFMT_MXFP4:
        return 2 * h * i // 2 + 2 * h * i // 32
    return 2 * h * i + 4 * (h // 128) * -(-2 * i // 128)


# ---- host-side tensors (numpy) -------------------------------------------------------------

def w13_f32(wl: Workload, layer: int, expert: int) -> np.ndarray:
    """Expert gate/up weights [2I][H]: gate rows [0, I), up rows [I, 2I)."""
    key = stream_key(wl.seed, TAG_W13, layer, expert)
    n = 2 * wl.inter * wl.hidden
    return normal_f32(key, 0, n, 0.0, wl.w_sigma).reshape(2 * wl.inter, wl.hidden)


def w2_f32(wl: Workload, layer: int, expert: int) -> np.ndarray:
    """Expert down weights [H][I]."""
    key = stream_key(wl.seed, TAG_W2, layer, expert)
    n = wl.hidden * wl.inter
    return normal_f32(key, 0, n, 0.0, wl.w_sigma).reshape(wl.hidden, wl.inter)


def router_w(wl: Workload, layer: int = 0) -> np.ndarray:
    """Router weights [E][H] fp32 (routed experts only)."""
    key = stream_key(wl.seed, TAG_WR, layer, 0)
    return normal_f32(key, 0, wl.n_routed * wl.hidden, 0.0, wl.wr_sigma).reshape(
        wl.n_routed, wl.hidden)


def router_b(wl: Workload, layer: int = 0):
    if wl.bias_sigma == 0.0:
        return None
    key = stream_key(wl.seed, TAG_BIAS, layer, 0)
    return normal_f32(key, 0, wl.n_routed, 0.0, wl.bias_sigma)


def rms_gamma(wl: Workload, layer: int = 0) -> np.ndarray:
    key = stream_key(wl.seed, TAG_GAMMA, layer, 0)
    return normal_f32(key, 0, wl.hidden, 1.0, 0.1)


def tokens_bf16(wl: Workload, first_token: int, n_tokens: int) -> np.ndarray:
    """Tokens [n][H] as bf16 bit patterns (uint16); token t is a fixed slice of one stream."""
    key = stream_key(wl.seed, TAG_X, 0, 0)
    h = wl.hidden
    return normal_bf16(key, first_token * h, n_tokens * h, 0.0, 1.0).reshape(n_tokens, h)
