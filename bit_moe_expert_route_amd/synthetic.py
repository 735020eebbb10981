"""Synthetic MoE layers resident in device memory.

Expert weights are drawn on the GPU by the shared seeded generator (moe_synth),
one expert at a time into an fp32 staging buffer, and packed by the library's
own moe_quant_mx straight into the layer's contiguous expert tensors, so a
9 GB layer never exists in fp32 or crosses PCIe.
"""
from __future__ import annotations

import torch

import moe_synth
from moe_synth import workloads as W

from . import Layer, quant_mx


def packed_sizes(wl: W.Workload):
    """(w13 code bytes, w13 scale elems, w2 code bytes, w2 scale elems) per expert."""
    H, I = wl.hidden, wl.inter
    if wl.wfmt == W.WFMT_MXFP4:
        return 2 * I * H // 2, 2 * I * H // 32, H * I // 2, H * I // 32
    # FP8: 128x128 block scales, the last block along a side partial when it is not a whole one
    return 2 * I * H, -(-2 * I // 128) * (H // 128), H * I, (H // 128) * -(-I // 128)


class GpuLayer:
    """One workload layer on the GPU: packed experts, router, optional bias and gamma."""

    def __init__(self, wl: W.Workload, layer: int = 0, device: str = "cuda",
                 staging: torch.Tensor | None = None):
        self.wl = wl
        self.layer = layer
        E1, H, I = wl.n_experts, wl.hidden, wl.inter
        c13, s13, c2, s2 = packed_sizes(wl)
        sdt = torch.uint8 if wl.wfmt == W.WFMT_MXFP4 else torch.float32
        self.w13 = torch.empty(E1 * c13, dtype=torch.uint8, device=device)
        self.w13_scale = torch.empty(E1 * s13, dtype=sdt, device=device)
        self.w2 = torch.empty(E1 * c2, dtype=torch.uint8, device=device)
        self.w2_scale = torch.empty(E1 * s2, dtype=sdt, device=device)
        self.nonfinite = torch.zeros(1, dtype=torch.int32, device=device)
        need = 2 * I * H
        if staging is None or staging.numel() < need:
            staging = torch.empty(need, dtype=torch.float32, device=device)
        self.staging = staging
        stream = torch.cuda.current_stream().cuda_stream
        for e in range(E1):
            st = staging[:need].view(2 * I, H)
            moe_synth.gpu_normal_f32(moe_synth.stream_key(wl.seed, moe_synth.TAG_W13, layer, e),
                                     0, need, 0.0, wl.w_sigma, st.data_ptr(), stream)
            quant_mx(wl.wfmt, st, self.w13[e * c13:(e + 1) * c13],
                     self.w13_scale[e * s13:(e + 1) * s13], self.nonfinite)
            st = staging[:H * I].view(H, I)
            moe_synth.gpu_normal_f32(moe_synth.stream_key(wl.seed, moe_synth.TAG_W2, layer, e),
                                     0, H * I, 0.0, wl.w_sigma, st.data_ptr(), stream)
            quant_mx(wl.wfmt, st, self.w2[e * c2:(e + 1) * c2],
                     self.w2_scale[e * s2:(e + 1) * s2], self.nonfinite)
        self.router_w = torch.empty(wl.n_routed * H, dtype=torch.float32, device=device)
        moe_synth.gpu_normal_f32(moe_synth.stream_key(wl.seed, moe_synth.TAG_WR, layer, 0), 0,
                                 wl.n_routed * H, 0.0, wl.wr_sigma, self.router_w.data_ptr(),
                                 stream)
        self.router_b = None
        if wl.bias_sigma:
            self.router_b = torch.empty(wl.n_routed, dtype=torch.float32, device=device)
            moe_synth.gpu_normal_f32(moe_synth.stream_key(wl.seed, moe_synth.TAG_BIAS, layer, 0),
                                     0, wl.n_routed, 0.0, wl.bias_sigma,
                                     self.router_b.data_ptr(), stream)
        self.gamma = torch.empty(H, dtype=torch.float32, device=device)
        moe_synth.gpu_normal_f32(moe_synth.stream_key(wl.seed, moe_synth.TAG_GAMMA, layer, 0), 0,
                                 H, 1.0, 0.1, self.gamma.data_ptr(), stream)

    @property
    def desc(self) -> Layer:
        wl = self.wl
        return Layer(wl.wfmt, wl.hidden, wl.inter, wl.n_routed, wl.top_k, wl.has_shared,
                     self.w13.data_ptr(), self.w13_scale.data_ptr(), self.w2.data_ptr(),
                     self.w2_scale.data_ptr(), self.router_w.data_ptr(),
                     None if self.router_b is None else self.router_b.data_ptr(),
                     self.gamma.data_ptr())

    def expert_packed(self, e: int):
        """(q13, s13, q2, s2) of expert e as host numpy arrays, shaped like the reference's."""
        wl = self.wl
        H, I = wl.hidden, wl.inter
        c13, s13, c2, s2 = packed_sizes(wl)
        q13 = self.w13[e * c13:(e + 1) * c13].cpu().numpy()
        sc13 = self.w13_scale[e * s13:(e + 1) * s13].cpu().numpy()
        q2 = self.w2[e * c2:(e + 1) * c2].cpu().numpy()
        sc2 = self.w2_scale[e * s2:(e + 1) * s2].cpu().numpy()
        if wl.wfmt == W.WFMT_MXFP4:
            return (q13.reshape(2 * I, H // 2), sc13.reshape(2 * I, H // 32),
                    q2.reshape(H, I // 2), sc2.reshape(H, I // 32))
        return (q13.reshape(2 * I, H), sc13.reshape(-(-2 * I // 128), H // 128),
                q2.reshape(H, I), sc2.reshape(H // 128, -(-I // 128)))


def tokens(wl: W.Workload, first_token: int, n_tokens: int, device: str = "cuda"):
    """bf16 tokens [n][H] (as int16 bit patterns) drawn on the GPU."""
    out = torch.empty(n_tokens * wl.hidden, dtype=torch.int16, device=device)
    moe_synth.gpu_normal_bf16(moe_synth.stream_key(wl.seed, moe_synth.TAG_X, 0, 0),
                              first_token * wl.hidden, n_tokens * wl.hidden, 0.0, 1.0,
                              out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    return out.view(n_tokens, wl.hidden)
