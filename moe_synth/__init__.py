"""Seeded synthetic inputs for the MoE decode layer.

The generator (splitmix64 counter stream -> standardised 8-term Irwin-Hall
sum -> mu + sigma*z -> fp32 / bf16) is defined in ``synth.h`` and implemented
twice with identical bits: ``synth_cpu.c`` (host) and ``synth_gpu.hip``
(device, for multi-gigabyte weights).  This package holds no MoE arithmetic;
both the CPU reference and the GPU library's tests draw their inputs from it.  The GPU half also
carries the benchmark's streaming-read probe (the achievable-bandwidth reference).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
CPU_LIB = os.path.join(_DIR, "libmoe_synth_cpu.so")
GPU_LIB = os.path.join(_DIR, "libmoe_synth_gpu.so")

TAG_W13, TAG_W2, TAG_WR, TAG_BIAS, TAG_GAMMA, TAG_X = 1, 2, 3, 4, 5, 6

HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(gpu: bool = True) -> None:
    """Compile the host generator with gcc and, if asked, the device one with hipcc."""
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-shared", "-fPIC",
                           os.path.join(_DIR, "synth_cpu.c"), "-o", CPU_LIB + ".tmp"])
    os.replace(CPU_LIB + ".tmp", CPU_LIB)
    if gpu:
        subprocess.check_call(["hipcc", *HIP_FLAGS, "-shared", "-fPIC",
                               os.path.join(_DIR, "synth_gpu.hip"), "-o", GPU_LIB + ".tmp"])
        os.replace(GPU_LIB + ".tmp", GPU_LIB)


_cpu = None
_gpu = None


def _cpu_lib():
    global _cpu
    if _cpu is None:
        if not os.path.exists(CPU_LIB):
            build(gpu=False)
        lib = ctypes.CDLL(CPU_LIB)
        lib.synth_mix64.argtypes = [ctypes.c_uint64]
        lib.synth_mix64.restype = ctypes.c_uint64
        lib.synth_stream_key.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                         ctypes.c_uint32]
        lib.synth_stream_key.restype = ctypes.c_uint64
        for name in ("synth_normal_f32", "synth_normal_bf16"):
            fn = getattr(lib, name)
            fn.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_double,
                           ctypes.c_double, ctypes.c_void_p]
            fn.restype = None
        _cpu = lib
    return _cpu


def _gpu_lib():
    global _gpu
    if _gpu is None:
        if not os.path.exists(GPU_LIB):
            raise RuntimeError(f"{GPU_LIB} is not built; run moe_synth.build()")
        lib = ctypes.CDLL(GPU_LIB)
        for name in ("synth_gpu_normal_f32", "synth_gpu_normal_bf16"):
            fn = getattr(lib, name)
            fn.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_double,
                           ctypes.c_double, ctypes.c_void_p, ctypes.c_void_p]
            fn.restype = ctypes.c_int
        lib.synth_gpu_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                             ctypes.c_void_p]
        lib.synth_gpu_read_probe.restype = ctypes.c_int
        lib.synth_gpu_sync_step.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        lib.synth_gpu_sync_step.restype = ctypes.c_int
        lib.synth_gpu_grid_barrier.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_void_p]
        lib.synth_gpu_grid_barrier.restype = ctypes.c_int
        _gpu = lib
    return _gpu


def mix64(z: int) -> int:
    return int(_cpu_lib().synth_mix64(z & 0xFFFFFFFFFFFFFFFF))


def stream_key(seed: int, tag: int, layer: int = 0, index: int = 0) -> int:
    return int(_cpu_lib().synth_stream_key(seed, tag, layer, index))


def normal_f32(key: int, first: int, n: int, mu: float, sigma: float) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    if n:
        _cpu_lib().synth_normal_f32(key, first, n, mu, sigma, out.ctypes.data)
    return out


def normal_bf16(key: int, first: int, n: int, mu: float, sigma: float) -> np.ndarray:
    """bf16 values as raw uint16 bit patterns."""
    out = np.empty(n, dtype=np.uint16)
    if n:
        _cpu_lib().synth_normal_bf16(key, first, n, mu, sigma, out.ctypes.data)
    return out


def gpu_normal_f32(key: int, first: int, n: int, mu: float, sigma: float, dev_ptr: int,
                   stream: int = 0) -> None:
    rc = _gpu_lib().synth_gpu_normal_f32(key, first, n, mu, sigma, dev_ptr, stream)
    if rc != 0:
        raise RuntimeError(f"synth_gpu_normal_f32 failed: hip error {rc}")


def gpu_normal_bf16(key: int, first: int, n: int, mu: float, sigma: float, dev_ptr: int,
                    stream: int = 0) -> None:
    rc = _gpu_lib().synth_gpu_normal_bf16(key, first, n, mu, sigma, dev_ptr, stream)
    if rc != 0:
        raise RuntimeError(f"synth_gpu_normal_bf16 failed: hip error {rc}")


def gpu_read_probe(dev_ptr: int, nbytes: int, sink_ptr: int, stream: int = 0) -> None:
    """One streaming read of nbytes of device memory (the benchmark's read ceiling)."""
    rc = _gpu_lib().synth_gpu_read_probe(dev_ptr, nbytes, sink_ptr, stream)
    if rc != 0:
        raise RuntimeError(f"synth_gpu_read_probe failed: hip error {rc}")


def gpu_sync_step(words_ptr: int, stream: int = 0) -> None:
    """One launch of the resident grid that only stores a word per workgroup (a chain of them
    times the boundary between dependent launches)."""
    rc = _gpu_lib().synth_gpu_sync_step(words_ptr, stream)
    if rc != 0:
        raise RuntimeError(f"synth_gpu_sync_step failed: hip error {rc}")


def gpu_grid_barrier(words_ptr: int, iters: int, fenced: bool, stream: int = 0) -> None:
    """One launch of `iters` grid-wide barriers (words[0..1] zero beforehand; words[1] != 0
    afterwards means a wait gave up)."""
    rc = _gpu_lib().synth_gpu_grid_barrier(words_ptr, iters, int(fenced), stream)
    if rc != 0:
        raise RuntimeError(f"synth_gpu_grid_barrier failed: hip error {rc}")


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)
