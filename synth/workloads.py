"""The five synthetic workloads (shapes, dtypes and value distributions).

Shapes follow the KDA layers of Kimi K3 (96 heads, head dim 128, up to a
1M-token context).  No trained weights exist, so decay scales A_h are drawn
from U(-1, 1) (or fixed at their initial value 0) and every activation is a
seeded random tensor.  Layouts: q, k, v, z, gate are [B, T, H, D]; beta is
[B, T, H]; A is [H]; S0 is [B, H, D, D] (row index = key channel).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import BF16, CONST, F32, NORMAL, SIGMOID_NORMAL, UNIFORM, UNIT_ROWS, fill

# stream ids (one independent random stream per tensor)
ST_Q, ST_K, ST_V, ST_BETA, ST_Z, ST_A, ST_GATE, ST_S0 = 1, 2, 3, 4, 5, 6, 7, 8


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    B: int
    T: int
    H: int
    D: int
    dtype: str                 # "f32" or "bf16": storage type of q, k, v, beta, z, gate
    z_std: float = 1.0
    z_split_pinned: bool = False  # heads h >= H/2 get z = +30 (decay pinned at g_min)
    A_kind: str = "zero"       # "zero" or "uniform" (U(-1, 1) per head)
    gate: bool = False
    s0_std: float = 0.0        # 0 -> no initial state
    chunk: int = 64
    g_min: float = -5.0
    note: str = ""

    @property
    def seed(self) -> int:
        return 1000 + self.index

    @property
    def in_dtype(self) -> int:
        return F32 if self.dtype == "f32" else BF16

    @property
    def token_heads(self) -> int:
        return self.B * self.T * self.H


WORKLOADS = {
    "tiny": Workload("tiny", 0, B=1, T=128, H=2, D=64, dtype="f32", z_std=1.0, A_kind="zero",
                     note="fp32 path, output o only"),
    "prefill": Workload("prefill", 1, B=4, T=4096, H=32, D=128, dtype="bf16", z_std=2.0,
                        A_kind="uniform", gate=True),
    "k3_layer": Workload("k3_layer", 2, B=1, T=65536, H=96, D=128, dtype="bf16", z_std=1.0,
                         z_split_pinned=True, A_kind="zero", gate=True,
                         note="heads >= 48 have z = +30 so every step sits at g_min"),
    "long_context": Workload("long_context", 3, B=1, T=1 << 20, H=96, D=128, dtype="bf16",
                             z_std=2.0, A_kind="uniform", gate=True),
    "decode": Workload("decode", 4, B=256, T=64, H=96, D=128, dtype="bf16", z_std=2.0,
                       A_kind="uniform", gate=True, s0_std=0.1,
                       note="64 single-token steps over 256 sequences from a random fp32 state"),
}


def gen_A(wl: Workload, heads=None) -> np.ndarray:
    h0, nh = (0, wl.H) if heads is None else heads
    if wl.A_kind == "zero":
        return np.zeros(nh, dtype=np.float32)
    a = fill(UNIFORM, F32, wl.seed, ST_A, (1, 1, wl.H, 1), ((0, 1), (0, 1), (h0, nh)), mean=-1.0, std=1.0)
    return a.reshape(nh).copy()


def gen_inputs(wl: Workload, batch=None, time=None, heads=None, with_gate=None) -> dict:
    """Generate the inputs of ``wl`` restricted to a block of (batch, time,
    heads), each given as (start, count).  bf16 tensors are uint16 bit
    patterns; everything else is fp32."""
    b0, nb = (0, wl.B) if batch is None else batch
    t0, nt = (0, wl.T) if time is None else time
    h0, nh = (0, wl.H) if heads is None else heads
    blk = ((b0, nb), (t0, nt), (h0, nh))
    shp = (wl.B, wl.T, wl.H, wl.D)
    dt = wl.in_dtype
    out = {}
    out["q"] = fill(UNIT_ROWS, dt, wl.seed, ST_Q, shp, blk)
    out["k"] = fill(UNIT_ROWS, dt, wl.seed, ST_K, shp, blk)
    out["v"] = fill(NORMAL, dt, wl.seed, ST_V, shp, blk)
    out["beta"] = fill(SIGMOID_NORMAL, dt, wl.seed, ST_BETA, (wl.B, wl.T, wl.H, 1), blk).reshape(nb, nt, nh)
    z = np.empty((nb, nt, nh, wl.D), dtype=np.float32 if dt == F32 else np.uint16)
    if wl.z_split_pinned:
        half = wl.H // 2
        for lo, hi, pinned in ((0, half, False), (half, wl.H, True)):
            a, b = max(lo, h0), min(hi, h0 + nh)
            if a >= b:
                continue
            sub = z[:, :, a - h0:b - h0, :]
            if pinned:
                fill(CONST, dt, wl.seed, ST_Z, shp, ((b0, nb), (t0, nt), (a, b - a)), mean=30.0, out=sub)
            else:
                fill(NORMAL, dt, wl.seed, ST_Z, shp, ((b0, nb), (t0, nt), (a, b - a)),
                     mean=0.0, std=wl.z_std, out=sub)
    else:
        fill(NORMAL, dt, wl.seed, ST_Z, shp, blk, mean=0.0, std=wl.z_std, out=z)
    out["z"] = z
    out["A"] = gen_A(wl, (h0, nh))
    if wl.gate if with_gate is None else with_gate:
        out["gate"] = fill(NORMAL, dt, wl.seed, ST_GATE, shp, blk)
    if wl.s0_std > 0:
        s = fill(NORMAL, F32, wl.seed, ST_S0, (wl.B, 1, wl.H, wl.D * wl.D), ((b0, nb), (0, 1), (h0, nh)),
                 std=wl.s0_std)
        out["S0"] = s.reshape(nb, nh, wl.D, wl.D)
    return out


def gen_prep_inputs(B: int, T: int, H: int, D: int, W: int, dtype: str, seed: int, with_state: bool = True) -> dict:
    """Inputs of the input steps before the core (projections of q, k, v and
    the beta logits, N(0, 1); depthwise conv taps N(0, 0.5^2) [H D, W] fp32;
    a conv state N(0, 1) [B, 3, W - 1, H D] fp32).  bf16 tensors are uint16
    bit patterns."""
    dt = BF16 if dtype == "bf16" else F32
    shp = (B, T, H, D)
    out = {n: fill(NORMAL, dt, seed, 40 + i, shp) for i, n in enumerate(("xq", "xk", "xv"))}
    out["beta_logits"] = fill(NORMAL, dt, seed, 43, (B, T, H, 1)).reshape(B, T, H)
    for i, n in enumerate(("wq", "wk", "wv")):
        out[n] = fill(NORMAL, F32, seed, 44 + i, (1, 1, H * D, W), std=0.5).reshape(H * D, W)
    if with_state and W > 1:
        out["state"] = fill(NORMAL, F32, seed, 47, (B, 3, W - 1, H * D))
    return out
