"""ctypes binding of the CPU reference (``moe_oracle.c``) -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never does, and this
package never imports the GPU library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
# MOE_ORACLE_LIB selects another build (the sanitized one of the CPU tests)
LIB = os.environ.get("MOE_ORACLE_LIB") or os.path.join(_DIR, "libmoe_oracle.so")

WFMT_MXFP4 = 1
WFMT_FP8_B128 = 2
WFMT_FP8_B128_A8 = 3  # FP8_B128 weights, activations quantized live (W8A8)


def build(out: str = LIB, sanitize: bool = False) -> str:
    """Compile the oracle with gcc (sanitize: with AddressSanitizer and UndefinedBehaviorSanitizer,
    for a process that preloads gcc's libasan)."""
    extra = (["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
              "-fno-omit-frame-pointer", "-g"] if sanitize else [])
    subprocess.check_call(["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-shared",
                           "-fPIC", "-Wall", *extra, os.path.join(_DIR, "moe_oracle.c"), "-lm",
                           "-o", out + ".tmp"])
    os.replace(out + ".tmp", out)
    return out


class _Experts(ctypes.Structure):
    _fields_ = [("wfmt", ctypes.c_int32), ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("w13_q", ctypes.POINTER(ctypes.c_void_p)),
                ("w13_s", ctypes.POINTER(ctypes.c_void_p)),
                ("w2_q", ctypes.POINTER(ctypes.c_void_p)),
                ("w2_s", ctypes.POINTER(ctypes.c_void_p))]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        i32, i64, u32, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_double
        sig = {
            "orc_set_threads": ([i32], None), "orc_get_threads": ([], i32),
            "orc_e2m1_value": ([u32], f64), "orc_e8m0_value": ([u32], f64),
            "orc_e4m3_value": ([u32], f64), "orc_e2m1_rne": ([f64], u32),
            "orc_e4m3_rne": ([f64], u32), "orc_bf16_from_double": ([f64], ctypes.c_uint16),
            "orc_quant_mxfp4": ([P, i64, i64, P, P], i64),
            "orc_quant_fp8_b128": ([P, i64, i64, P, P], i64),
            "orc_quant_act_fp8": ([P, i64, P, P], i64),
            "orc_dequant": ([i32, P, P, i64, i64, P], None),
            "orc_route": ([P, i32, i32, P, P, i32, i32, i32, P, P, P, P], None),
            "orc_expert_ffn": ([ctypes.POINTER(_Experts), P, i32, P, P, i32, P, P], None),
            "orc_rmsnorm": ([P, i32, i32, P, f64, P], None),
            "orc_residual": ([P, P, i64, P], None),
            "orc_verify": ([P, P, P, P, i32, i32, P, P], i32),
            "orc_qk_norm_rope": ([P, i32, i32, i32, i32, i64, P, P, P, f64, f64, i32, P, P],
                                 None),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data


def set_threads(n: int) -> None:
    lib().orc_set_threads(int(n))


def get_threads() -> int:
    return int(lib().orc_get_threads())


def e2m1_value(code: int) -> float:
    return float(lib().orc_e2m1_value(code))


def e8m0_value(code: int) -> float:
    return float(lib().orc_e8m0_value(code))


def e4m3_value(code: int) -> float:
    return float(lib().orc_e4m3_value(code))


def e2m1_rne(t: float) -> int:
    return int(lib().orc_e2m1_rne(float(t)))


def e4m3_rne(t: float) -> int:
    return int(lib().orc_e4m3_rne(float(t)))


def bf16_from_double(d: float) -> int:
    return int(lib().orc_bf16_from_double(float(d)))


def quant_mxfp4(w: np.ndarray):
    """fp32 [rows][cols] -> (codes u8 [rows][cols/2], E8M0 scales u8 [rows][cols/32], nonfinite)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, cols = w.shape
    assert cols % 32 == 0
    q = np.empty((rows, cols // 2), np.uint8)
    s = np.empty((rows, cols // 32), np.uint8)
    n = lib().orc_quant_mxfp4(w.ctypes.data, rows, cols, q.ctypes.data, s.ctypes.data)
    return q, s, int(n)


def quant_fp8_b128(w: np.ndarray):
    """fp32 [rows][cols] -> (E4M3 codes u8 [rows][cols], fp32 scales
    [ceil(rows/128)][ceil(cols/128)], nonfinite); a last block along a side may be partial."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, cols = w.shape
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((-(-rows // 128), -(-cols // 128)), np.float32)
    n = lib().orc_quant_fp8_b128(w.ctypes.data, rows, cols, q.ctypes.data, s.ctypes.data)
    return q, s, int(n)


def quant_act_fp8(v: np.ndarray):
    """fp32 [..., n] (n % 128 == 0) -> (E4M3 codes u8 [..., n], fp32 scales [..., n/128],
    nonfinite): the W8A8 variant's live activation quantizer, per 128 consecutive values."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    assert v.shape[-1] % 128 == 0
    q = np.empty(v.shape, np.uint8)
    s = np.empty(v.shape[:-1] + (v.shape[-1] // 128,), np.float32)
    n = lib().orc_quant_act_fp8(v.ctypes.data, v.size, q.ctypes.data, s.ctypes.data)
    return q, s, int(n)


def quant(wfmt: int, w: np.ndarray):
    return quant_mxfp4(w) if wfmt == WFMT_MXFP4 else quant_fp8_b128(w)


def dequant(wfmt: int, q: np.ndarray, s: np.ndarray, rows: int, cols: int) -> np.ndarray:
    out = np.empty((rows, cols), np.float64)
    lib().orc_dequant(wfmt, q.ctypes.data, s.ctypes.data, rows, cols, out.ctypes.data)
    return out


def route(x_bf16: np.ndarray, wr: np.ndarray, b: np.ndarray | None, k: int, has_shared: int):
    """x bf16 bits [M][H] -> (ids int32 [M][S], w fp64 [M][S], logits fp64 [M][E], gap fp64 [M])."""
    x_bf16 = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    wr = np.ascontiguousarray(wr, dtype=np.float32)
    M, H = x_bf16.shape
    E = wr.shape[0]
    S = k + (1 if has_shared else 0)
    ids = np.empty((M, S), np.int32)
    w = np.empty((M, S), np.float64)
    logits = np.empty((M, E), np.float64)
    gap = np.empty(M, np.float64)
    bb = None if b is None else np.ascontiguousarray(b, dtype=np.float32)
    lib().orc_route(x_bf16.ctypes.data, M, H, wr.ctypes.data, _ptr(bb), E, k,
                    1 if has_shared else 0, ids.ctypes.data, w.ctypes.data, logits.ctypes.data,
                    gap.ctypes.data)
    return ids, w, logits, gap


def expert_ffn(wfmt: int, hidden: int, inter: int, n_experts: int, experts: dict,
               x_bf16: np.ndarray, ids: np.ndarray, w: np.ndarray,
               token_mask: np.ndarray | None = None) -> np.ndarray:
    """experts: {e: (q13, s13, q2, s2)} for every referenced e.  Returns y fp64 [M][H]."""
    x_bf16 = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    w32 = np.ascontiguousarray(w, dtype=np.float32)
    M, S = ids.shape
    arrs = [(ctypes.c_void_p * n_experts)() for _ in range(4)]
    keep = []
    for e, tensors in experts.items():
        for a, t in zip(arrs, tensors):
            t = np.ascontiguousarray(t)
            keep.append(t)
            a[e] = t.ctypes.data
    L = _Experts(wfmt, hidden, inter, n_experts,
                 *[ctypes.cast(a, ctypes.POINTER(ctypes.c_void_p)) for a in arrs])
    y = np.empty((M, hidden), np.float64)
    mask = None if token_mask is None else np.ascontiguousarray(token_mask, dtype=np.uint8)
    lib().orc_expert_ffn(ctypes.byref(L), x_bf16.ctypes.data, M, ids.ctypes.data,
                         w32.ctypes.data, S, _ptr(mask), y.ctypes.data)
    return y


def rmsnorm(h_bf16: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    h_bf16 = np.ascontiguousarray(h_bf16, dtype=np.uint16)
    M, H = h_bf16.shape
    g = np.ascontiguousarray(gamma, dtype=np.float32)
    out = np.empty_like(h_bf16)
    lib().orc_rmsnorm(h_bf16.ctypes.data, M, H, g.ctypes.data, float(eps), out.ctypes.data)
    return out


def residual(h_bf16: np.ndarray, y: np.ndarray) -> np.ndarray:
    h_bf16 = np.ascontiguousarray(h_bf16, dtype=np.uint16)
    y = np.ascontiguousarray(y, dtype=np.float64)
    out = np.empty_like(h_bf16)
    lib().orc_residual(h_bf16.ctypes.data, y.ctypes.data, h_bf16.size, out.ctypes.data)
    return out


def verify(logits: np.ndarray, draft: np.ndarray, q: np.ndarray | None = None,
           u: np.ndarray | None = None):
    """Verify-acceptance of one speculative block.  logits fp32 [K+1][V], draft int32 [K],
    q fp32 [K][V] draft probabilities (None: greedy), u fp32 [K+1] uniforms.
    Returns (tokens int32 [n+1], (accept margin, draw margin)): the smallest relative distance
    of an accept test, and of the draw, to its threshold (inf when there is none)."""
    L = np.ascontiguousarray(logits, dtype=np.float32)
    K1, V = L.shape
    K = K1 - 1
    d = np.ascontiguousarray(draft, dtype=np.int32).reshape(K)
    Q = None if q is None else np.ascontiguousarray(q, dtype=np.float32)
    assert Q is None or Q.shape == (K, V)
    uu = np.ascontiguousarray(np.zeros(K + 1) if u is None else u, dtype=np.float32)
    assert uu.shape == (K + 1,)
    out = np.empty(K + 1, np.int32)
    margin = np.zeros(2, np.float64)
    n = lib().orc_verify(L.ctypes.data, _ptr(Q), d.ctypes.data, uu.ctypes.data, K, V,
                         out.ctypes.data, margin.ctypes.data)
    return out[:n].copy(), (float(margin[0]), float(margin[1]))


def qk_norm_rope(x_bf16: np.ndarray, nq: int, pos: np.ndarray, gamma_q: np.ndarray,
                 gamma_k: np.ndarray, eps: float, theta: float, rot: int):
    """x bf16 bits [M][nh][hd] -> (y fp64 [M][nh][hd] unrounded, y bf16 bits [M][nh][hd])."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    M, nh, hd = x.shape
    p = np.ascontiguousarray(pos, dtype=np.int32).reshape(M)
    gq = np.ascontiguousarray(gamma_q, dtype=np.float32).reshape(hd)
    gk = np.ascontiguousarray(gamma_k, dtype=np.float32).reshape(hd)
    y64 = np.empty((M, nh, hd), np.float64)
    yb = np.empty((M, nh, hd), np.uint16)
    lib().orc_qk_norm_rope(x.ctypes.data, M, nq, nh, hd, nh * hd, p.ctypes.data, gq.ctypes.data,
                           gk.ctypes.data, float(eps), float(theta), int(rot), y64.ctypes.data,
                           yb.ctypes.data)
    return y64, yb
