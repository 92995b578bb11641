"""ORACLE -- test infrastructure only.

Plain CPU reference for one decode step (and the speculative verify step) of
the megakernel's model.  liboracle.so (oracle.c) holds the arithmetic of each
block in fp64; step.py composes the blocks in the order the model defines.
Only tests/, the smoke entry and the benchmark's CPU-baseline leg may import
this package.  It shares no code with the GPU library; its inputs come from
the `synth` generator only.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SO = os.path.join(_HERE, "liboracle.so")


def build() -> None:
    src = os.path.join(_HERE, "oracle.c")
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-Wall", "-shared", "-fPIC", "-o", SO + ".tmp", src, "-lm"])
    os.replace(SO + ".tmp", SO)


_lib = None

P = ctypes.c_void_p
I = ctypes.c_int
I64 = ctypes.c_int64
D = ctypes.c_double


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(SO):
            raise RuntimeError(f"{SO} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(SO)
        L.orc_bf16.restype = D
        L.orc_bf16.argtypes = [ctypes.c_uint16]
        L.orc_to_bf16.restype = ctypes.c_uint16
        L.orc_to_bf16.argtypes = [D]
        L.orc_rmsnorm.argtypes = [I, P, P, D, P]
        L.orc_matvec.argtypes = [I64, I64, P, P, P]
        L.orc_rope.argtypes = [I, P, I64, D]
        L.orc_silu.restype = D
        L.orc_silu.argtypes = [D]
        L.orc_sigmoid.restype = D
        L.orc_sigmoid.argtypes = [D]
        L.orc_softmax.argtypes = [I, P]
        L.orc_gqa_block.restype = I
        L.orc_gqa_block.argtypes = [I, I, I, I, D, D, P, P, P, P, P, P, I64, P, P, I64]
        L.orc_mla_block.restype = I
        L.orc_mla_block.argtypes = [I, I, I, I, I, I, I, D, D, P, P, P, P, P, P, P, P, P, I64, P, I64]
        L.orc_kda_block.restype = I
        L.orc_kda_block.argtypes = [I, I, I, I, I, D, P, P, P, P, P, P, P, P, P]
        L.orc_swiglu_add.argtypes = [I, I, P, P, P, P, D, P]
        L.orc_router.argtypes = [I, I, I, I, P, P, P, P, P]
        L.orc_head.restype = ctypes.c_int32
        L.orc_head.argtypes = [I, I64, D, P, P, P, P]
        L.orc_embed.argtypes = [I, P, ctypes.c_int32, P]
        _lib = L
    return _lib


def ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


# thin numpy-facing wrappers of the building blocks (used by the pin tests)
def rmsnorm(x: np.ndarray, g_bits: np.ndarray, eps: float) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    g = np.ascontiguousarray(g_bits, dtype=np.uint16)
    y = np.empty_like(x)
    lib().orc_rmsnorm(x.size, ptr(x), ptr(g), eps, ptr(y))
    return y


def matvec(W_bits: np.ndarray, x: np.ndarray) -> np.ndarray:
    W = np.ascontiguousarray(W_bits, dtype=np.uint16)
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty(W.shape[0], dtype=np.float64)
    lib().orc_matvec(W.shape[0], W.shape[1], ptr(W), ptr(x), ptr(y))
    return y


def rope(v: np.ndarray, pos: int, theta: float) -> np.ndarray:
    v = np.array(v, dtype=np.float64)
    lib().orc_rope(v.size, ptr(v), pos, theta)
    return v


def softmax(s: np.ndarray) -> np.ndarray:
    s = np.array(s, dtype=np.float64)
    lib().orc_softmax(s.size, ptr(s))
    return s


def to_bf16(d: float) -> int:
    return int(lib().orc_to_bf16(float(d)))


def router(wr_bits: np.ndarray, xn: np.ndarray, k: int, norm_topk: int = 1):
    wr = np.ascontiguousarray(wr_bits, dtype=np.uint16)
    xn = np.ascontiguousarray(xn, dtype=np.float64)
    E, H = wr.shape
    ids = np.empty(k, dtype=np.int32)
    w = np.empty(k, dtype=np.float64)
    lg = np.empty(E, dtype=np.float32)
    lib().orc_router(H, E, k, norm_topk, ptr(wr), ptr(xn), ptr(ids), ptr(w), ptr(lg))
    return ids, w, lg


def swiglu_add(wg, wu, wd, xn, scale, acc):
    wg, wu, wd = (np.ascontiguousarray(a, dtype=np.uint16) for a in (wg, wu, wd))
    xn = np.ascontiguousarray(xn, dtype=np.float64)
    assert acc.dtype == np.float64 and acc.flags["C_CONTIGUOUS"]
    F, H = wg.shape
    lib().orc_swiglu_add(H, F, ptr(wg), ptr(wu), ptr(wd), ptr(xn), scale, ptr(acc))
    return acc
