"""Seeded synthetic inputs shared by the oracle side and the GPU side.

Nothing here computes any step of the method: this package only draws tensors
with the distributions of the workloads (see ``workloads.py``) from a
counter-based generator implemented in ``synth.c``.  bf16 tensors are returned
as ``uint16`` numpy arrays holding the bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsynth.so")
SRC_PATH = os.path.join(_HERE, "synth.c")

NORMAL, UNIT_ROWS, SIGMOID_NORMAL, UNIFORM, CONST = 0, 1, 2, 3, 4
F32, BF16, F64 = 0, 1, 2

_lib = None


def build(force: bool = True) -> str:
    """Compile synth.c into libsynth.so with gcc (host code only)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        cmd = ["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c11",
               "-ffp-contract=off", SRC_PATH, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(LIB_PATH)
        i64, u64, dbl, vp = ctypes.c_int64, ctypes.c_uint64, ctypes.c_double, ctypes.c_void_p
        L.synth_fill.restype = ctypes.c_int
        L.synth_fill.argtypes = [ctypes.c_int, ctypes.c_int, u64, u64,
                                 i64, i64, i64, i64,
                                 i64, i64, i64, i64, i64, i64,
                                 dbl, dbl, vp, i64, i64, i64]
        L.synth_raw_uniform.restype = None
        L.synth_raw_uniform.argtypes = [u64, u64, u64, i64, vp]
        L.synth_raw_bits.restype = None
        L.synth_raw_bits.argtypes = [u64, u64, u64, i64, vp]
        _lib = L
    return _lib


_NP = {F32: np.float32, BF16: np.uint16, F64: np.float64}


def fill(kind: int, dtype: int, seed: int, stream: int, shape, block=None,
         mean: float = 0.0, std: float = 1.0, out: np.ndarray | None = None) -> np.ndarray:
    """Generate ``block`` = ((b0, nb), (t0, nt), (h0, nh)) of a logical
    [B, T, H, D] tensor.  Returns (or writes into ``out``) an array of shape
    [nb, nt, nh, D].  ``out`` may be a strided view whose last axis is
    contiguous."""
    B, T, H, D = (int(x) for x in shape)
    if block is None:
        block = ((0, B), (0, T), (0, H))
    (b0, nb), (t0, nt), (h0, nh) = block
    if out is None:
        out = np.empty((nb, nt, nh, D), dtype=_NP[dtype])
    if out.shape != (nb, nt, nh, D) or out.dtype != _NP[dtype]:
        raise ValueError(f"out has shape {out.shape} / {out.dtype}, need {(nb, nt, nh, D)} / {_NP[dtype]}")
    if out.size == 0:
        return out
    if out.strides[3] != out.itemsize:
        raise ValueError("last axis of out must be contiguous")
    osb, ost, osh = (s // out.itemsize for s in out.strides[:3])
    rc = lib().synth_fill(kind, dtype, seed, stream, B, T, H, D, b0, nb, t0, nt, h0, nh,
                          float(mean), float(std), out.ctypes.data, osb, ost, osh)
    if rc != 0:
        raise ValueError("synth_fill rejected its arguments")
    return out


def raw_uniform(seed: int, stream: int, i0: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    lib().synth_raw_uniform(seed, stream, i0, n, out.ctypes.data)
    return out


def raw_bits(seed: int, stream: int, i0: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    lib().synth_raw_bits(seed, stream, i0, n, out.ctypes.data)
    return out


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (a.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest even); returns bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = 0x7FC0
    return r
