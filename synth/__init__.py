"""Seeded synthetic inputs shared by the oracle harness and the GPU path.

Host draws come from libsynth_host.so (plain C, synth_host.c); device draws
come from libsynth_dev.so (synth_dev.hip), which evaluates the same integer
recipe so both are bit-identical.  Nothing here computes any part of the
decode step.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from typing import Optional

import numpy as np

from . import workloads  # noqa: F401
from .workloads import KV_SIGMA, V_TILE, TensorSpec, Workload, kv_layout, tensor_inventory  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_SO = os.path.join(_HERE, "libsynth_host.so")
DEV_SO = os.path.join(_HERE, "libsynth_dev.so")

# standard deviation of the sum of four uniform 16-bit integers
_IH4_SD = math.sqrt(4.0 * (65536.0 ** 2 - 1.0) / 12.0)
BF16_ONE = 0x3F80


def build(verbose: bool = False) -> None:
    """Compile both generator libraries in place."""
    src = os.path.join(_HERE, "synth_host.c")
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", HOST_SO + ".tmp", src]
    subprocess.check_call(cmd)
    os.replace(HOST_SO + ".tmp", HOST_SO)
    dsrc = os.path.join(_HERE, "synth_dev.hip")
    cmd = ["hipcc", "--offload-arch=gfx950", "-O3", "-shared", "-fPIC",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-o", DEV_SO + ".tmp", dsrc]
    subprocess.check_call(cmd, stderr=None if verbose else subprocess.DEVNULL)
    os.replace(DEV_SO + ".tmp", DEV_SO)


_host = None
_dev = None


def _host_lib():
    global _host
    if _host is None:
        if not os.path.exists(HOST_SO):
            raise RuntimeError(f"{HOST_SO} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(HOST_SO)
        lib.synth_key.restype = ctypes.c_uint64
        lib.synth_key.argtypes = [ctypes.c_uint64, ctypes.c_char_p]
        lib.synth_normal_bf16.argtypes = [ctypes.c_uint64, ctypes.c_float, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64]
        lib.synth_normal_f32.argtypes = [ctypes.c_uint64, ctypes.c_float, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64]
        lib.synth_uniform_i32.argtypes = [ctypes.c_uint64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64]
        lib.synth_fill_u16.argtypes = [ctypes.c_uint16, ctypes.c_void_p, ctypes.c_int64]
        _host = lib
    return _host


def _dev_lib():
    global _dev
    if _dev is None:
        if not os.path.exists(DEV_SO):
            raise RuntimeError(f"{DEV_SO} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(DEV_SO)
        for fn, extra in (("synth_dev_normal_bf16", ctypes.c_float), ("synth_dev_normal_f32", ctypes.c_float),
                          ("synth_dev_uniform_i32", ctypes.c_int32)):
            f = getattr(lib, fn)
            f.restype = ctypes.c_int
            f.argtypes = [ctypes.c_uint64, extra, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
        lib.synth_dev_normal_bf16_tiles.restype = ctypes.c_int
        lib.synth_dev_normal_bf16_tiles.argtypes = [ctypes.c_uint64, ctypes.c_float, ctypes.c_void_p, ctypes.c_int64,
                                                    ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
        lib.synth_dev_fill_u16.restype = ctypes.c_int
        lib.synth_dev_fill_u16.argtypes = [ctypes.c_uint16, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        _dev = lib
    return _dev


def key(seed: int, name: str) -> int:
    return int(_host_lib().synth_key(ctypes.c_uint64(seed), name.encode()))


def scale_for(sigma: float) -> float:
    """fp32 multiplier that maps the centred Irwin-Hall sum to N(0, sigma)."""
    return float(np.float32(sigma / _IH4_SD))


# ---------------------------------------------------------------- host draws
def normal_bf16(seed: int, name: str, n: int, sigma: float, offset: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    _host_lib().synth_normal_bf16(key(seed, name), scale_for(sigma), out.ctypes.data, n, offset)
    return out


def normal_f32(seed: int, name: str, n: int, sigma: float, offset: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    _host_lib().synth_normal_f32(key(seed, name), scale_for(sigma), out.ctypes.data, n, offset)
    return out


def uniform_i32(seed: int, name: str, n: int, hi: int, offset: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    _host_lib().synth_uniform_i32(key(seed, name), hi, out.ctypes.data, n, offset)
    return out


def weight_host(w: Workload, spec: TensorSpec) -> np.ndarray:
    """One weight tensor as bf16 bits, shape [rows, cols]."""
    seed = w.seed("weights")
    if spec.kind == "gain":
        if spec.sigma == 0.0:
            out = np.full(spec.numel, BF16_ONE, dtype=np.uint16)
        else:
            # 1 + N(0, sigma), drawn in fp32 and rounded to bf16
            z = normal_f32(seed, spec.name, spec.numel, spec.sigma)
            out = f32_to_bf16_bits(np.float32(1.0) + z)
    else:
        out = normal_bf16(seed, spec.name, spec.numel, spec.sigma)
    return out.reshape(spec.rows, spec.cols)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest-even), returned as uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def tokens(w: Workload, batch: int, step: int = 0) -> np.ndarray:
    return uniform_i32(w.seed("tokens"), f"tokens.step{step}", batch, w.vocab)


def kv_layer_host(w: Workload, layer: int) -> np.ndarray:
    """Initial cache (bf16 bits) or state (fp32) of one layer, full max_batch/max_ctx shape.

    Rows at positions >= context are drawn too (they are overwritten before
    being read)."""
    lay, _ = kv_layout(w)
    kind, _, nbytes, shape, dt = lay[layer]
    if kind == "kda":
        n = int(np.prod(shape))
        return normal_f32(w.seed("state"), f"L{layer}.kda_state", n, KV_SIGMA).reshape(shape)
    if kind == "gqa":
        n = int(np.prod(shape))
        k = normal_bf16(w.seed("kv"), f"L{layer}.k_cache", n, KV_SIGMA).reshape(shape)
        v = normal_bf16(w.seed("kv"), f"L{layer}.v_cache", n, KV_SIGMA).reshape(shape)
        return np.stack([k, v])
    n = int(np.prod(shape))
    return normal_bf16(w.seed("kv"), f"L{layer}.mla_cache", n, KV_SIGMA).reshape(shape)


# -------------------------------------------------------------- device draws
def _dev_check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"synth device draw {what} failed: hip error {rc}")


def weight_device(w: Workload, spec: TensorSpec, ptr: int, stream: int = 0) -> None:
    """Draw one weight tensor straight into device memory at `ptr`."""
    seed = w.seed("weights")
    lib = _dev_lib()
    if spec.kind == "gain":
        # gains are tiny: draw on the host and let the caller copy; here only
        # the all-ones case is handled on device.
        if spec.sigma != 0.0:
            raise ValueError("random gains are drawn on the host (weight_host)")
        _dev_check(lib.synth_dev_fill_u16(BF16_ONE, ptr, spec.numel, stream), spec.name)
        return
    _dev_check(lib.synth_dev_normal_bf16(key(seed, spec.name), scale_for(spec.sigma), ptr, spec.numel, 0, stream),
               spec.name)


def kv_layer_device(w: Workload, layer: int, ptr: int, stream: int = 0) -> None:
    lay, _ = kv_layout(w)
    kind, _, nbytes, shape, dt = lay[layer]
    lib = _dev_lib()
    n = int(np.prod(shape))
    if kind == "kda":
        _dev_check(lib.synth_dev_normal_f32(key(w.seed("state"), f"L{layer}.kda_state"), scale_for(KV_SIGMA),
                                            ptr, n, 0, stream), "state")
    elif kind == "gqa":
        _dev_check(lib.synth_dev_normal_bf16(key(w.seed("kv"), f"L{layer}.k_cache"), scale_for(KV_SIGMA),
                                             ptr, n, 0, stream), "k")
        # V is stored in V_TILE-position tiles, dim-major within a tile
        rows = n // w.head_dim
        _dev_check(lib.synth_dev_normal_bf16_tiles(key(w.seed("kv"), f"L{layer}.v_cache"), scale_for(KV_SIGMA),
                                                   ptr + n * 2, rows, w.head_dim, V_TILE, stream), "v")
    else:
        _dev_check(lib.synth_dev_normal_bf16(key(w.seed("kv"), f"L{layer}.mla_cache"), scale_for(KV_SIGMA),
                                             ptr, n, 0, stream), "mla")
