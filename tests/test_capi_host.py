"""The C-ABI library loads, exports every function include/moe_mx.h declares, and rejects
invalid arguments on the host before any GPU work.  CPU only (no HIP call is reached)."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

import bit_moe_expert_route_amd as moe

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "moe_mx.h")

pytestmark = pytest.mark.skipif(not os.path.exists(moe.LIB_PATH),
                                reason="libmoe_mx.so not built")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_function():
    names = header_functions()
    assert set(names) == set(moe.EXPORTS)
    lib = moe.lib()
    for n in names:
        assert hasattr(lib, n), n


def _layer(**kw):
    d = dict(wfmt=moe.WFMT_MXFP4, hidden=256, inter=128, n_routed=8, top_k=2, has_shared=1,
             w13=0x1000, w13_scale=0x2000, w2=0x3000, w2_scale=0x4000, router_w=0x5000,
             router_b=None, rms_gamma=None)
    d.update(kw)
    return moe.Layer(**d)


def test_status_strings():
    assert moe.status_str(moe.MOE_OK) == "MOE_OK"
    assert moe.status_str(moe.MOE_ERR_WORKSPACE) == "MOE_ERR_WORKSPACE"


def test_workspace_sizing():
    L = _layer()
    n1 = moe.workspace_bytes(L, 1)
    n16 = moe.workspace_bytes(L, 16)
    assert 0 < n1 < n16 and n16 % 256 == 0
    assert moe.workspace_bytes(L, 0) == 0 and moe.workspace_bytes(L, 17) == 0
    assert moe.workspace_bytes(_layer(hidden=200), 1) == 0
    assert moe.workspace_bytes(_layer(top_k=9), 1) == 0
    assert moe.workspace_bytes(_layer(wfmt=4), 1) == 0


def _route(L, M=1, x=0x10000, ids=0x20000, w=0x30000, ws=0x40000, ws_bytes=1 << 30):
    return moe.lib().moe_route_topk(ctypes.byref(L), x, M, ids, w, None, ws, ws_bytes, None)


def _ffn(L, M=1, x=0x10000, ids=0x20000, w=0x30000, y=0x50000, ws=0x40000, ws_bytes=1 << 30):
    return moe.lib().moe_expert_ffn_decode(ctypes.byref(L), x, M, ids, w, y, ws, ws_bytes, None,
                                           None)


def _gate_up(L, M=1, x=0x10000, ids=0x20000, ws=0x40000, ws_bytes=1 << 30):
    return moe.lib().moe_expert_gate_up(ctypes.byref(L), x, M, ids, ws, ws_bytes, None, None)


def _down(L, M=1, ids=0x20000, w=0x30000, y=0x50000, ws=0x40000, ws_bytes=1 << 30):
    return moe.lib().moe_expert_down_combine(ctypes.byref(L), M, ids, w, y, ws, ws_bytes, None,
                                             None)


@pytest.mark.parametrize("bad", [
    dict(wfmt=0), dict(hidden=100), dict(inter=80), dict(n_routed=0), dict(top_k=0),
    dict(top_k=9), dict(has_shared=2), dict(n_routed=2000, top_k=2), dict(hidden=-128),
])
def test_invalid_layer_rejected(bad):
    L = _layer(**bad)
    assert _route(L) == moe.MOE_ERR_INVALID
    assert _ffn(L) == moe.MOE_ERR_INVALID
    assert _gate_up(L) == moe.MOE_ERR_INVALID
    assert _down(L) == moe.MOE_ERR_INVALID


def test_stage_calls_rejected_before_launch():
    L = _layer()
    assert _gate_up(L, x=None) == moe.MOE_ERR_INVALID
    assert _gate_up(L, ids=None) == moe.MOE_ERR_INVALID
    assert _gate_up(L, M=17) == moe.MOE_ERR_INVALID
    assert _gate_up(L, ws_bytes=16) == moe.MOE_ERR_WORKSPACE
    assert _gate_up(_layer(w13_scale=None)) == moe.MOE_ERR_INVALID
    assert _down(L, w=None) == moe.MOE_ERR_INVALID
    assert _down(L, y=None) == moe.MOE_ERR_INVALID
    assert _down(L, M=0) == moe.MOE_ERR_INVALID
    assert _down(L, ws=0x40010) == moe.MOE_ERR_WORKSPACE
    assert _down(_layer(w2=0x3004)) == moe.MOE_ERR_INVALID


def test_invalid_calls_rejected_before_launch():
    L = _layer()
    assert moe.lib().moe_route_topk(None, 0x10000, 1, 0x20000, 0x30000, None, 0x40000, 1 << 30,
                                    None) == moe.MOE_ERR_INVALID
    assert _route(L, M=0) == moe.MOE_ERR_INVALID
    assert _route(L, M=17) == moe.MOE_ERR_INVALID
    assert _route(L, x=None) == moe.MOE_ERR_INVALID
    assert _route(L, x=0x10008) == moe.MOE_ERR_INVALID          # misaligned activations
    assert _route(_layer(router_w=None)) == moe.MOE_ERR_INVALID
    assert _route(L, ws=None) == moe.MOE_ERR_WORKSPACE
    assert _route(L, ws=0x40010) == moe.MOE_ERR_WORKSPACE       # misaligned workspace
    assert _route(L, ws_bytes=16) == moe.MOE_ERR_WORKSPACE
    assert _ffn(_layer(w13=None)) == moe.MOE_ERR_INVALID
    assert _ffn(_layer(w2=0x3004)) == moe.MOE_ERR_INVALID       # misaligned codes
    assert _ffn(L, y=None) == moe.MOE_ERR_INVALID
    assert _ffn(L, ws_bytes=moe.workspace_bytes(L, 1) - 1) == moe.MOE_ERR_WORKSPACE
    q = moe.lib().moe_quant_mx
    assert q(moe.WFMT_MXFP4, None, 32, 32, 0x1000, 0x2000, None, None) == moe.MOE_ERR_INVALID
    assert q(moe.WFMT_MXFP4, 0x1000, 32, 48, 0x2000, 0x3000, None, None) == moe.MOE_ERR_INVALID
    assert q(moe.WFMT_FP8_B128, 0x1000, 64, 136, 0x2000, 0x3000, None,
             None) == moe.MOE_ERR_INVALID                       # rows of codes not 16-byte
    assert q(moe.WFMT_FP8_B128, 0x1000, 64, 128, 0x2000, 0x3002, None,
             None) == moe.MOE_ERR_INVALID                       # misaligned fp32 scales
    assert q(7, 0x1000, 128, 128, 0x2000, 0x3000, None, None) == moe.MOE_ERR_INVALID
    assert q(moe.WFMT_MXFP4, 0x1000, 0, 32, 0x2000, 0x3000, None, None) == moe.MOE_OK  # no-op
    assert moe.lib().moe_workspace_init(None, 16, None) == moe.MOE_ERR_WORKSPACE


def _stack(layers, n=None, eps=1e-6, h=0x10000, M=1, ws=0x40000, ws_bytes=1 << 30, trace=None):
    arr = (moe.Layer * len(layers))(*layers)
    return moe.lib().moe_layer_stack_persistent(arr, len(layers) if n is None else n, eps, h, M,
                                                ws, ws_bytes, trace, None)


def test_stack_rejected_before_launch():
    L = _layer(rms_gamma=0x6000)
    assert _stack([L], n=0) == moe.MOE_ERR_INVALID
    assert _stack([L], M=0) == moe.MOE_ERR_INVALID
    assert _stack([L], M=17) == moe.MOE_ERR_INVALID
    assert _stack([L], h=None) == moe.MOE_ERR_INVALID
    assert _stack([L], eps=-1.0) == moe.MOE_ERR_INVALID
    assert _stack([L], eps=float("nan")) == moe.MOE_ERR_INVALID
    assert _stack([_layer()]) == moe.MOE_ERR_INVALID                     # no gamma
    assert _stack([_layer(rms_gamma=0x6004)]) == moe.MOE_ERR_INVALID     # misaligned gamma
    assert _stack([L, _layer(rms_gamma=0x6000, inter=256)]) == moe.MOE_ERR_INVALID
    assert _stack([L, _layer(rms_gamma=0x6000, top_k=3)]) == moe.MOE_ERR_INVALID
    assert _stack([L], ws_bytes=64) == moe.MOE_ERR_WORKSPACE
    assert _stack([L], trace=0x70008) == moe.MOE_ERR_INVALID


def test_tensor_parallel_shard_shapes():
    """A tensor-parallel shard's intermediate slice: a multiple of 32 in both formats (FP8 with a
    partial last 128-block of scales along the intermediate axis); W8A8 keeps whole 128-value
    activation blocks."""
    # an accepted shape stops at the (too small) workspace, so nothing is ever launched
    ok = _layer(inter=192)
    assert moe.workspace_bytes(ok, 1) > 0
    assert _ffn(ok, ws_bytes=16) == moe.MOE_ERR_WORKSPACE
    assert _ffn(_layer(inter=96), ws_bytes=16) == moe.MOE_ERR_WORKSPACE
    assert _ffn(_layer(inter=80)) == moe.MOE_ERR_INVALID
    fp8 = dict(wfmt=moe.WFMT_FP8_B128)
    for inter in (192, 96, 160):
        assert moe.workspace_bytes(_layer(inter=inter, **fp8), 4) > 0
        assert _ffn(_layer(inter=inter, **fp8), ws_bytes=16) == moe.MOE_ERR_WORKSPACE
        assert _route(_layer(inter=inter, **fp8), ws_bytes=16) == moe.MOE_ERR_WORKSPACE
    assert _ffn(_layer(inter=80, **fp8)) == moe.MOE_ERR_INVALID
    a8 = dict(wfmt=moe.WFMT_FP8_B128_A8)
    assert _ffn(_layer(inter=192, **a8)) == moe.MOE_ERR_UNSUPPORTED
    assert _route(_layer(inter=192, **a8)) == moe.MOE_ERR_UNSUPPORTED


def test_w8a8_layer_checks():
    """W8A8 (FP8_B128_A8): FP8 shape rules (whole 128x128 blocks).  Every hidden size up to the
    8192 limit is accepted at one and at several tokens, by each FFN call and the layer stack."""
    a8 = dict(wfmt=moe.WFMT_FP8_B128_A8)
    assert moe.workspace_bytes(_layer(**a8), 1) > 0
    for M in (1, 2, 16):  # accepted shapes stop at the (too small) workspace
        assert _ffn(_layer(**a8), M=M, ws_bytes=16) == moe.MOE_ERR_WORKSPACE
        assert _gate_up(_layer(**a8), M=M, ws_bytes=16) == moe.MOE_ERR_WORKSPACE
    assert _ffn(_layer(inter=192, **a8)) == moe.MOE_ERR_UNSUPPORTED
    wide = dict(hidden=8192, **a8)
    for M in (1, 2, 16):  # accepted: stops at the (too small) workspace
        assert _ffn(_layer(**wide), M=M, ws_bytes=16) == moe.MOE_ERR_WORKSPACE
        assert _gate_up(_layer(**wide), M=M, ws_bytes=16) == moe.MOE_ERR_WORKSPACE
        assert _down(_layer(**wide), M=M, ws_bytes=16) == moe.MOE_ERR_WORKSPACE
        assert _stack([_layer(rms_gamma=0x6000, **wide)], M=M,
                      ws_bytes=16) == moe.MOE_ERR_WORKSPACE
    q = moe.lib().moe_quant_mx
    assert q(moe.WFMT_FP8_B128_A8, 0x1000, 64, 120, 0x2000, 0x3000, None,
             None) == moe.MOE_ERR_INVALID


def test_unsupported_sizes():
    assert _route(_layer(wfmt=moe.WFMT_FP8_B128, hidden=8192 + 128)) == moe.MOE_ERR_UNSUPPORTED
    assert _ffn(_layer(inter=8192 + 128)) == moe.MOE_ERR_UNSUPPORTED
    assert _route(_layer(hidden=16384)) == moe.MOE_ERR_UNSUPPORTED
    assert _route(_layer(hidden=8192), ws_bytes=16) == moe.MOE_ERR_WORKSPACE  # accepted shape


def _verify(K=4, V=1000, L=0x10000, Q=None, d=0x20000, u=0x30000, out=0x40000, cnt=0x50000,
            ws=0x60000, ws_bytes=1 << 30):
    return moe.lib().moe_verify_accept(L, Q, d, u, K, V, out, cnt, ws, ws_bytes, None)


def test_verify_rejected_before_launch():
    assert moe.verify_workspace_bytes(4, 151552) > 0
    assert moe.verify_workspace_bytes(15, 1 << 24) > moe.verify_workspace_bytes(15, 151552)
    assert moe.verify_workspace_bytes(16, 100) == 0 and moe.verify_workspace_bytes(-1, 100) == 0
    assert moe.verify_workspace_bytes(4, 0) == 0 and moe.verify_workspace_bytes(4, (1 << 24) + 1) == 0
    assert _verify(K=16) == moe.MOE_ERR_INVALID
    assert _verify(V=0) == moe.MOE_ERR_INVALID
    assert _verify(L=None) == moe.MOE_ERR_INVALID
    assert _verify(d=None) == moe.MOE_ERR_INVALID
    assert _verify(out=None) == moe.MOE_ERR_INVALID
    assert _verify(cnt=None) == moe.MOE_ERR_INVALID
    assert _verify(Q=0x70000, u=None) == moe.MOE_ERR_INVALID  # sampling needs uniforms
    assert _verify(L=0x10002) == moe.MOE_ERR_INVALID           # misaligned logits
    assert _verify(ws=None) == moe.MOE_ERR_WORKSPACE
    assert _verify(ws=0x60010) == moe.MOE_ERR_WORKSPACE
    assert _verify(ws_bytes=moe.verify_workspace_bytes(4, 1000) - 1) == moe.MOE_ERR_WORKSPACE
    assert _verify(K=0, d=None, ws_bytes=16) == moe.MOE_ERR_WORKSPACE  # K = 0 needs no drafts


def _qk(qk=0x10000, M=1, nq=4, nk=1, hd=128, stride=640, pos=0x20000, gq=0x30000, gk=0x40000,
        eps=1e-6, theta=1e4, rot=64):
    return moe.lib().moe_qk_norm_rope(qk, M, nq, nk, hd, stride, pos, gq, gk, eps, theta, rot,
                                      None)


def test_qk_norm_rope_rejected_before_launch():
    assert _qk(qk=None) == moe.MOE_ERR_INVALID
    assert _qk(pos=None) == moe.MOE_ERR_INVALID
    assert _qk(gk=None) == moe.MOE_ERR_INVALID
    assert _qk(M=0) == moe.MOE_ERR_INVALID
    assert _qk(nq=0, nk=0) == moe.MOE_ERR_INVALID
    assert _qk(nq=-1) == moe.MOE_ERR_INVALID
    assert _qk(hd=96, stride=480) == moe.MOE_ERR_INVALID      # head_dim 64, 128 or 256
    assert _qk(rot=130) == moe.MOE_ERR_INVALID                # rot_dim <= head_dim
    assert _qk(rot=62) == moe.MOE_ERR_INVALID                 # a multiple of head_dim / 32
    assert _qk(stride=639) == moe.MOE_ERR_INVALID             # stride covers the heads ...
    assert _qk(stride=644) == moe.MOE_ERR_INVALID             # ... and is a multiple of 8
    assert _qk(qk=0x10008) == moe.MOE_ERR_INVALID             # 16-byte aligned
    assert _qk(eps=-1.0) == moe.MOE_ERR_INVALID
    assert _qk(theta=0.0) == moe.MOE_ERR_INVALID


def _ld(L, M=1, x=0x10000, ids=0x20000, w=0x30000, y=0x50000, ws=0x40000, ws_bytes=1 << 30):
    return moe.lib().moe_layer_decode(ctypes.byref(L), x, M, ids, w, None, y, ws, ws_bytes, None,
                                      None)


def test_layer_decode_rejected_before_launch():
    L = _layer()
    assert _ld(_layer(wfmt=0)) == moe.MOE_ERR_INVALID
    assert _ld(L, x=None) == moe.MOE_ERR_INVALID
    assert _ld(L, ids=None) == moe.MOE_ERR_INVALID
    assert _ld(L, w=None) == moe.MOE_ERR_INVALID
    assert _ld(L, y=None) == moe.MOE_ERR_INVALID
    assert _ld(_layer(router_w=None)) == moe.MOE_ERR_INVALID
    assert _ld(L, M=0) == moe.MOE_ERR_INVALID
    assert _ld(L, M=17) == moe.MOE_ERR_INVALID
    assert _ld(L, ws_bytes=16) == moe.MOE_ERR_WORKSPACE
    # several W8A8 tokens at the widest hidden size: accepted (stops at the small workspace)
    assert _ld(_layer(wfmt=moe.WFMT_FP8_B128_A8, hidden=8192), M=2,
               ws_bytes=16) == moe.MOE_ERR_WORKSPACE


def test_bench_refuses_several_gpus():
    """bench.py measures one GPU: asked for more it exits with a message and prints no result
    line, before importing torch or touching a device."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=root)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""
