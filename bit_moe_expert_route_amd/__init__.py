"""Python binding of libmoe_mx.so, the gfx950 MoE decode-layer library.

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  Tensors are torch tensors (device memory and streams); the C ABI is
declared in include/moe_mx.h.  The library must be built (``build.build()``);
nothing here falls back to another implementation.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# MOE_LIB_PATH selects another build of the library (the host-sanitized one of the CPU tests)
LIB_PATH = os.environ.get("MOE_LIB_PATH") or os.path.join(PKG, "libmoe_mx.so")

MOE_OK, MOE_ERR_INVALID, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
WFMT_MXFP4 = 1
WFMT_FP8_B128 = 2
WFMT_FP8_B128_A8 = 3  # FP8_B128 weights, activations quantized live (W8A8)
MAX_TOKENS = 16
STATIC_SCRATCH_BYTES = 16 << 20  # MOE_STATIC_SCRATCH_BYTES
MAX_SLOTS = 16
MAX_EXPERTS = 1024

EXPORTS = ("moe_quant_mx", "moe_route_topk", "moe_expert_ffn_decode", "moe_expert_gate_up",
           "moe_expert_down_combine", "moe_layer_decode", "moe_layer_decode_one_launch",
           "moe_layer_decode_static",
           "moe_layer_stack_persistent",
           "moe_qk_norm_rope",
           "moe_verify_accept",
           "moe_verify_workspace_bytes", "moe_workspace_bytes", "moe_workspace_init",
           "moe_status_str")


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {status_str(status)} ({status})")
        self.status = status


class Layer(ctypes.Structure):
    """Mirror of the C ``moe_layer`` descriptor (device pointers as integers)."""
    _fields_ = [("wfmt", ctypes.c_int32), ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_routed", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("has_shared", ctypes.c_int32), ("w13", ctypes.c_void_p),
                ("w13_scale", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("w2_scale", ctypes.c_void_p), ("router_w", ctypes.c_void_p),
                ("router_b", ctypes.c_void_p), ("rms_gamma", ctypes.c_void_p)]


_lib = None


def lib():
    """Load the library; raises if it is not built (there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "bit_moe_expert_route_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        LP = ctypes.POINTER(Layer)
        sig = {
            "moe_quant_mx": ([i32, P, i64, i64, P, P, P, P], ctypes.c_int),
            "moe_route_topk": ([LP, P, i32, P, P, P, P, sz, P], ctypes.c_int),
            "moe_expert_ffn_decode": ([LP, P, i32, P, P, P, P, sz, P, P], ctypes.c_int),
            "moe_expert_gate_up": ([LP, P, i32, P, P, sz, P, P], ctypes.c_int),
            "moe_expert_down_combine": ([LP, i32, P, P, P, P, sz, P, P], ctypes.c_int),
            "moe_layer_decode": ([LP, P, i32, P, P, P, P, P, sz, P, P], ctypes.c_int),
            "moe_layer_decode_one_launch": ([LP, P, i32, P, P, P, P, P, sz, P, P], ctypes.c_int),
            "moe_layer_decode_static": ([LP, P, i32, P, P, P, P, P, P], ctypes.c_int),
            "moe_layer_stack_persistent": ([LP, i32, ctypes.c_float, P, i32, P, sz, P, P],
                                           ctypes.c_int),
            "moe_verify_accept": ([P, P, P, P, i32, i32, P, P, P, sz, P], ctypes.c_int),
            "moe_verify_workspace_bytes": ([i32, i32], sz),
            "moe_qk_norm_rope": ([P, i32, i32, i32, i32, i64, P, P, P, ctypes.c_float,
                                  ctypes.c_float, i32, P], ctypes.c_int),
            "moe_workspace_bytes": ([LP, i32, i32], sz),
            "moe_workspace_init": ([P, sz, P], ctypes.c_int),
            "moe_status_str": ([ctypes.c_int], ctypes.c_char_p),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().moe_status_str(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != MOE_OK:
        raise MoeError(fn, status)


# MOE_TRACE=<path>: every entry-point call made outside a graph capture is bracketed by two
# timing events on its stream; trace_records() returns (function, milliseconds) per call, and at
# exit the records not yet taken go to <path> as JSON lines ("-": standard error).
TRACE = os.environ.get("MOE_TRACE") or None
_trace_events: list = []


def _torch_stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, int):
        return torch.cuda.ExternalStream(stream)
    return stream


def _call(fn: str, stream, *args) -> None:
    """Call the library's entry point fn with args (its stream last) and raise on a status."""
    f = getattr(lib(), fn)
    if TRACE is None:
        _check(fn, f(*args))
        return
    import torch
    if torch.cuda.is_current_stream_capturing():
        _check(fn, f(*args))
        return
    s = _torch_stream(stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    status = f(*args)
    e1.record(s)
    _trace_events.append((fn, e0, e1))
    _check(fn, status)


def trace_records() -> list:
    """The traced calls since the last call of this function: [(function, ms)] (synchronizes)."""
    import torch
    if not _trace_events:
        return []
    torch.cuda.synchronize()
    out = [(fn, float(e0.elapsed_time(e1))) for fn, e0, e1 in _trace_events]
    _trace_events.clear()
    return out


def _dump_trace() -> None:
    if TRACE is None or not _trace_events:
        return
    import json
    import sys
    recs = trace_records()
    f = sys.stderr if TRACE == "-" else open(TRACE, "a")
    for fn, ms in recs:
        f.write(json.dumps({"fn": fn, "ms": round(ms, 6)}) + "\n")
    if f is not sys.stderr:
        f.close()


if TRACE is not None:
    import atexit
    atexit.register(_dump_trace)


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def quant_mx(wfmt: int, w, q_out, scale_out, nonfinite=None, stream=None) -> None:
    """moe_quant_mx on a 2-D fp32 device tensor w [rows][cols]."""
    rows, cols = w.shape
    _call("moe_quant_mx", stream, wfmt, _ptr(w), rows, cols, _ptr(q_out), _ptr(scale_out),
          _ptr(nonfinite), _stream(stream))


def route_topk(layer: Layer, x, M: int, topk_ids, topk_w, logits=None, ws=None,
               ws_bytes: int | None = None, stream=None) -> None:
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None and ws is not None else ws_bytes
    _call("moe_route_topk", stream,
        ctypes.byref(layer), _ptr(x), M, _ptr(topk_ids), _ptr(topk_w), _ptr(logits), _ptr(ws),
        nbytes or 0, _stream(stream))


def expert_ffn_decode(layer: Layer, x, M: int, topk_ids, topk_w, y, ws, ws_bytes=None,
                      dev_status=None, stream=None) -> None:
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _call("moe_expert_ffn_decode", stream,
        ctypes.byref(layer), _ptr(x), M, _ptr(topk_ids), _ptr(topk_w), _ptr(y), _ptr(ws),
        nbytes, _ptr(dev_status), _stream(stream))


def expert_gate_up(layer: Layer, x, M: int, topk_ids, ws, ws_bytes=None, dev_status=None,
                   stream=None) -> None:
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _call("moe_expert_gate_up", stream,
        ctypes.byref(layer), _ptr(x), M, _ptr(topk_ids), _ptr(ws), nbytes, _ptr(dev_status),
        _stream(stream))


def expert_down_combine(layer: Layer, M: int, topk_ids, topk_w, y, ws, ws_bytes=None,
                        dev_status=None, stream=None) -> None:
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _call("moe_expert_down_combine", stream,
        ctypes.byref(layer), M, _ptr(topk_ids), _ptr(topk_w), _ptr(y), _ptr(ws), nbytes,
        _ptr(dev_status), _stream(stream))


def layer_stack_persistent(layers, n_layers: int, rms_eps: float, h, M: int, ws,
                           ws_bytes=None, trace=None, stream=None) -> None:
    arr = layers if isinstance(layers, ctypes.Array) else (Layer * n_layers)(*layers)
    nbytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _call("moe_layer_stack_persistent", stream,
        arr, n_layers, rms_eps, _ptr(h), M, _ptr(ws), nbytes, _ptr(trace), _stream(stream))


def workspace_bytes(layers, M: int) -> int:
    if isinstance(layers, Layer):
        layers = [layers]
    arr = (Layer * len(layers))(*layers)
    return int(lib().moe_workspace_bytes(arr, len(layers), M))


def workspace_init(ws, stream=None) -> None:
    _call("moe_workspace_init", stream,
        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))


def new_workspace(layers, M: int, device="cuda"):
    """Allocate (torch) and zero-fill a workspace for these layers and up to M tokens."""
    import torch
    n = workspace_bytes(layers, M)
    if n == 0:
        raise ValueError("invalid layer description for workspace sizing")
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    workspace_init(ws)
    return ws


def verify_workspace_bytes(K: int, V: int) -> int:
    return int(lib().moe_verify_workspace_bytes(K, V))


def new_verify_workspace(K: int, V: int, device="cuda"):
    """Allocate (torch) and zero-fill a workspace for moe_verify_accept."""
    import torch
    n = verify_workspace_bytes(K, V)
    if n == 0:
        raise ValueError("verify shape outside the limits")
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    workspace_init(ws)
    return ws


def verify_accept(logits, draft_tokens, out_tokens, out_count, ws, draft_probs=None,
                  uniforms=None, ws_bytes=None, stream=None) -> None:
    """logits [K+1][V] fp32, draft_tokens [K] int32, draft_probs [K][V] fp32 or None (greedy),
    uniforms [K+1] fp32; out_tokens [K+1] int32, out_count [1] int32 (device tensors)."""
    K1, V = logits.shape
    n = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _call("moe_verify_accept", stream,
        _ptr(logits), _ptr(draft_probs), _ptr(draft_tokens), _ptr(uniforms), K1 - 1, V,
        _ptr(out_tokens), _ptr(out_count), _ptr(ws), n, _stream(stream))


def qk_norm_rope(qk, M: int, n_q_heads: int, n_k_heads: int, head_dim: int, token_stride: int,
                 positions, gamma_q, gamma_k, eps: float, theta: float, rot_dim: int,
                 stream=None) -> None:
    """In place on qk (bf16 bits as an int16 tensor): head-wise RMSNorm of the query and key
    heads, then rotary embedding of their first rot_dim values."""
    _call("moe_qk_norm_rope", stream,
        _ptr(qk), M, n_q_heads, n_k_heads, head_dim, token_stride, _ptr(positions),
        _ptr(gamma_q), _ptr(gamma_k), float(eps), float(theta), rot_dim, _stream(stream))


def layer_decode(layer: Layer, x, M: int, topk_ids, topk_w, y, ws, logits=None, ws_bytes=None,
                 dev_status=None, stream=None) -> None:
    """Route + expert FFN + combine of one layer (the two calls' results, in fewer launches)."""
    n = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _call("moe_layer_decode", stream,
        ctypes.byref(layer), _ptr(x), M, _ptr(topk_ids), _ptr(topk_w), _ptr(logits), _ptr(y),
        _ptr(ws), n, _ptr(dev_status), _stream(stream))


def layer_decode_one_launch(layer: Layer, x, M: int, topk_ids, topk_w, y, ws, logits=None,
                            ws_bytes=None, dev_status=None, stream=None) -> None:
    """The one-token layer as a single kernel launch (same results as layer_decode)."""
    n = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _call("moe_layer_decode_one_launch", stream,
        ctypes.byref(layer), _ptr(x), M, _ptr(topk_ids), _ptr(topk_w), _ptr(logits), _ptr(y),
        _ptr(ws), n, _ptr(dev_status), _stream(stream))


def layer_decode_static(layer: Layer, x, M: int, topk_ids, topk_w, y, logits=None,
                        dev_status=None, stream=None) -> None:
    """moe_layer_decode on the library's own per-GPU scratch: no workspace, no allocation."""
    _call("moe_layer_decode_static", stream,
        ctypes.byref(layer), _ptr(x), M, _ptr(topk_ids), _ptr(topk_w), _ptr(logits), _ptr(y),
        _ptr(dev_status), _stream(stream))
