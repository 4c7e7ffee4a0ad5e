"""Long-context workload on the GPU: B1, T = 1,048,576, H96, d128, bf16 inputs,
fp32 state, output gate -- the whole sequence in one kda_chunk_fwd call.

Inputs are generated slab by slab (65,536 tokens, all heads) into device
buffers; the fp64 C oracle walks the same slabs with its state carried from
slab to slab.  Checked: o and y of four sampled heads over the whole
sequence, and the final state S_T of every head, each within relative L2
3e-3 (the bf16-input / fp32-state bar).  About 2.5 minutes, most of it CPU.
"""
import time

import numpy as np
import pytest
import torch

import oracle
from synth.workloads import WORKLOADS, gen_inputs

from kda_gpu_util import dev, host64, log, rel_l2

TOL_BF16 = 3e-3
SAMPLED = [0, 31, 64, 95]
SLAB = 65536


@pytest.fixture(scope="module")
def kda():
    import gated_delta_rule_84_amd as m
    assert torch.cuda.is_available()
    m.lib()
    return m


@pytest.mark.gpu
@pytest.mark.slow
@pytest.mark.timeout(1200)
def test_long_context_sampled_heads_and_every_state(kda):
    wl = WORKLOADS["long_context"]
    B, T, H, D = wl.B, wl.T, wl.H, wl.D
    assert B == 1 and T % SLAB == 0
    log(f"[long] {wl}")
    cuda = torch.device("cuda")
    torch.cuda.empty_cache()
    bufs = {n: torch.empty((B, T, H, D), dtype=torch.bfloat16, device=cuda) for n in ("q", "k", "v", "z", "gate")}
    bufs["beta"] = torch.empty((B, T, H), dtype=torch.bfloat16, device=cuda)
    A = None
    S_all = None                      # oracle state of every head, fp64
    S_smp = None                      # oracle state of the sampled heads (carried by the sampled pass)
    ref_o = np.empty((T, len(SAMPLED), D))
    ref_y = np.empty((T, len(SAMPLED), D))
    t_start = time.time()
    for t0 in range(0, T, SLAB):
        x = gen_inputs(wl, time=(t0, SLAB))
        for n in ("q", "k", "v", "z", "gate", "beta"):
            bufs[n][:, t0:t0 + SLAB].copy_(dev(x[n]))
        if A is None:
            A = x["A"]
        # every head, state only
        r = oracle.forward_c(x["q"], x["k"], x["v"], x["beta"], x["z"], A, S0=S_all, want_o=False)
        S_all = r["S_T"]
        # sampled heads with o and y
        xs = {n: np.ascontiguousarray(x[n][:, :, SAMPLED]) for n in ("q", "k", "v", "beta", "z", "gate")}
        rs = oracle.forward_c(xs["q"], xs["k"], xs["v"], xs["beta"], xs["z"], A[SAMPLED], S0=S_smp, gate=xs["gate"])
        S_smp = rs["S_T"]
        ref_o[t0:t0 + SLAB] = rs["o"][0]
        ref_y[t0:t0 + SLAB] = rs["y"][0]
        del x, xs, r, rs
        log(f"[long] tokens {t0 + SLAB}/{T} generated and run on the oracle ({time.time() - t_start:.0f} s)")
    assert np.array_equal(S_smp, S_all[:, SAMPLED])  # the two oracle passes agree exactly

    torch.cuda.synchronize()
    t_gpu = time.time()
    r = kda.chunk_fwd(bufs["q"], bufs["k"], bufs["v"], bufs["beta"], bufs["z"], dev(A), gate=bufs["gate"])
    torch.cuda.synchronize()
    log(f"[long] GPU forward {time.time() - t_gpu:.2f} s")
    o = host64(r["o"][0, :, SAMPLED])
    y = host64(r["y"][0, :, SAMPLED])
    S = host64(r["S_T"])
    for j, h in enumerate(SAMPLED):
        eo = rel_l2(o[:, j], ref_o[:, j])
        ey = rel_l2(y[:, j], ref_y[:, j])
        log(f"[long] head {h}: o={eo:.3e} y={ey:.3e}")
        assert eo <= TOL_BF16 and ey <= TOL_BF16
    es = [rel_l2(S[0, h], S_all[0, h]) for h in range(H)]
    log(f"[long] S_T over {H} heads: max {max(es):.3e}, all {rel_l2(S, S_all):.3e}")
    assert max(es) <= TOL_BF16
