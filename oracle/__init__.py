"""KDA oracle package — TEST INFRASTRUCTURE ONLY.

Plain fp64 CPU implementations of what the KDA forward computes, written from
"Kimi K3: KDA, Attention Residuals and Stable LatentMoE" (sections 2.1-2.3
and 10.2).  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import it.  It shares no code with the GPU library.

``kda_ref``  : numpy, small cases (sequential, chunked, gate, (M, S~) pairs).
``forward_c``: the C/OpenMP twin (kda_oracle.c) for large workloads.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from . import kda_ref  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "kda_oracle.c")
_lib = None


def build(force: bool = True) -> str:
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.run(["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-ffp-contract=off",
                        SRC_PATH, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(LIB_PATH)
        i64, dbl, vp = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        L.kda_oracle_forward.restype = ctypes.c_int
        L.kda_oracle_forward.argtypes = [i64, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp,
                                         dbl, dbl, ctypes.c_int, dbl, vp, vp, vp, dbl, vp, vp, vp,
                                         ctypes.c_int, ctypes.c_int]
        _lib = L
    return _lib


def _f32(a):
    """fp32 contiguous copy; uint16 arrays are bf16 bit patterns (exact)."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        a = (a.astype(np.uint32) << 16).view(np.float32)
    return np.ascontiguousarray(a, dtype=np.float32)


def _ptr(a):
    return None if a is None else a.ctypes.data


def forward_c(q, k, v, beta, z, A, S0=None, gate=None, w=None, g_min=-5.0, scale=1.0,
              l2norm=True, l2_eps=1e-6, rms_eps=1e-6, want_o=True, nthreads=0, decay="k3"):
    """Run the C oracle.  q, k, z: [B, T, H, dk]; v, gate: [B, T, H, dv];
    beta: [B, T, H]; A: [H]; S0: [B, H, dk, dv] fp64/fp32 or None.
    Returns dict with S_T (fp64) and o / y when requested."""
    q, k, v, beta, z, A = (_f32(x) for x in (q, k, v, beta, z, A))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or z.shape != q.shape or v.shape[:3] != (B, T, H) or beta.shape != (B, T, H):
        raise ValueError("shape mismatch")
    s0 = None if S0 is None else np.ascontiguousarray(S0, dtype=np.float64)
    if s0 is not None and s0.shape != (B, H, dk, dv):
        raise ValueError("S0 shape")
    g = None if gate is None else _f32(gate)
    wh = None if w is None else _f32(w)
    o = np.empty((B, T, H, dv)) if want_o else None
    y = np.empty((B, T, H, dv)) if g is not None else None
    ST = np.empty((B, H, dk, dv))
    rc = _load().kda_oracle_forward(B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(z),
                                    _ptr(A), g_min, scale, int(bool(l2norm)), l2_eps, _ptr(s0),
                                    _ptr(g), _ptr(wh), rms_eps, _ptr(o), _ptr(y), _ptr(ST), int(nthreads),
                                    {"k3": 0, "softplus": 1}[decay])
    if rc != 0:
        raise RuntimeError(f"kda_oracle_forward failed ({rc})")
    out = {"S_T": ST}
    if o is not None:
        out["o"] = o
    if y is not None:
        out["y"] = y
    return out
