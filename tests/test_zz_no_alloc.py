"""The workspace-free forward (kda_chunk_fwd_noalloc, per-GPU scratch array)
against the workspace forward (kda_chunk_fwd) through the C ABI, and against
the fp64 oracle: two calls in a row, the second with a smaller input, then a
shape whose sequence needs several segments of the scratch array.

Source: "Kimi K3: KDA, Attention Residuals and Stable LatentMoE", sections
2.1-2.3 (the same computation as kda_chunk_fwd)."""
import numpy as np
import pytest
import torch

import oracle
from synth.workloads import Workload, gen_inputs
from kda_gpu_util import dev, host64, log, rel_l2

pytestmark = pytest.mark.gpu
TOL = 3e-3


@pytest.fixture(scope="module")
def kda():
    import gated_delta_rule_84_amd as m
    m.lib()
    return m


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def _both(kda, B, T, H, D, seed, s0=0.1):
    wl = Workload("noalloc", 90 + seed, B=B, T=T, H=H, D=D, dtype="bf16", z_std=2.0, A_kind="uniform", gate=True,
                  s0_std=s0)
    x = gen_inputs(wl)
    t = {n: dev(x[n]) for n in ("q", "k", "v", "beta", "z", "A", "gate")}
    S0 = dev(x["S0"]) if "S0" in x else None
    log(f"[noalloc] B={B} T={T} H={H} D={D}")
    a = kda.chunk_fwd_noalloc(t["q"], t["k"], t["v"], t["beta"], t["z"], t["A"], S0=S0, gate=t["gate"])
    torch.cuda.synchronize()
    b = kda.chunk_fwd(t["q"], t["k"], t["v"], t["beta"], t["z"], t["A"], S0=S0, gate=t["gate"])
    torch.cuda.synchronize()
    ref = oracle.forward_c(x["q"], x["k"], x["v"], x["beta"], x["z"], x["A"], S0=x.get("S0"), gate=x["gate"])
    for key in ("o", "y", "S_T"):
        assert torch.equal(_bits(a[key]), _bits(b[key])), key  # same kernels, same rounding
        e = rel_l2(host64(a[key]), ref[key])
        log(f"[noalloc] {key} rel_l2={e:.3e}")
        assert e <= TOL, key


def test_noalloc_two_calls_second_smaller(kda):
    _both(kda, 2, 700, 3, 128, 1)
    _both(kda, 1, 130, 2, 64, 2)


def test_noalloc_several_segments(kda):
    """B * H = 256 at d = 128: one chunk of records and states takes ~32 MB, so
    the 128 MiB array holds a few chunks and the 16-chunk sequence runs in
    several segments with the state carried between them."""
    _both(kda, 8, 1024, 32, 128, 3)


def test_noalloc_rejects_what_does_not_fit(kda):
    """B * H = 2048 at d = 128: one chunk needs more than the array; nothing runs."""
    desc = kda.make_desc(16, 64, 128, 128, kda.KDA_BF16, kda.KDA_BF16)
    import ctypes
    z = ctypes.c_void_p(256)
    rc = kda.lib().kda_chunk_fwd_noalloc(ctypes.byref(desc), z, z, z, z, z, z, None, None, None, z, None, None, None)
    assert rc == 6  # KDA_ERR_WORKSPACE
