"""Prefix-cache snapshots on the GPU (kda_chunk_fwd_snapshots).

K3 blog, section 13.1: a cached prefix of a KDA layer can only be reused as
the recurrent state at a chunk-aligned boundary.  The forward therefore also
stores the state after every N-th chunk.  Checked here:
  * each snapshot against the fp64 oracle's final state over that prefix
    (relative L2 within the bar of the input precision);
  * resuming: a forward over the remaining tokens started from snapshot j
    gives outputs and final state bit-identical to the full run's suffix;
  * asking for snapshots changes no other output (bit-identical);
  * with T a multiple of the snapshot period the last snapshot is S_T.
"""
import numpy as np
import pytest
import torch

import oracle
from synth.workloads import Workload, gen_inputs

from kda_gpu_util import dev, host64, log, rel_l2

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 3e-3}
NAMES = ("q", "k", "v", "beta", "z", "gate")


@pytest.fixture(scope="module")
def kda():
    import gated_delta_rule_84_amd as m
    assert torch.cuda.is_available()
    m.lib()
    return m


def _wl(B, T, H, D, dtype, seed):
    return Workload("custom", 900 + seed, B=B, T=T, H=H, D=D, dtype=dtype, z_std=2.0, A_kind="uniform",
                    gate=True, s0_std=0.1)


def _bit_equal(a, b):
    if a.dtype == torch.bfloat16:
        a, b = a.view(torch.int16), b.view(torch.int16)
    return torch.equal(a, b)


def _fwd(kda, t, S0, **kw):
    r = kda.chunk_fwd(t["q"], t["k"], t["v"], t["beta"], t["z"], t["A"], S0=S0, gate=t["gate"], **kw)
    torch.cuda.synchronize()
    return r


@pytest.mark.parametrize("B,T,H,D,dtype,every", [(2, 1000, 3, 128, "bf16", 2), (1, 640, 2, 64, "f32", 1),
                                                 (3, 512, 2, 128, "bf16", 4), (1, 333, 2, 64, "bf16", 1)])
def test_snapshots_match_oracle_prefix_states(kda, B, T, H, D, dtype, every):
    x = gen_inputs(_wl(B, T, H, D, dtype, seed=T + every))
    t = {n: dev(x[n]) for n in NAMES + ("A", "S0")}
    n = T // (64 * every)
    log(f"[snapshots] B={B} T={T} H={H} D={D} {dtype} every={every} -> {n}")
    r = _fwd(kda, t, t["S0"], overlap=False, snapshot_chunks=every)
    assert tuple(r["snapshots"].shape) == (B, n, H, D, D)
    snaps = host64(r["snapshots"])
    for j in range(n):
        tj = (j + 1) * 64 * every
        ref = oracle.forward_c(*(x[m][:, :tj] for m in ("q", "k", "v", "beta", "z")), x["A"], S0=x["S0"],
                               want_o=False)["S_T"]
        e = rel_l2(snaps[:, j], ref)
        log(f"  snapshot {j} (after token {tj - 1}): rel_l2 {e:.3e}")
        assert e <= TOL[dtype], j
    if T % (64 * every) == 0:
        assert torch.equal(r["snapshots"][:, -1], r["S_T"])


@pytest.mark.parametrize("fused,overlap,seg,sched", [(True, True, None, "fused"), (False, False, None, "segments"),
                                                     (False, True, 128, "pipelined"), (False, True, 128, "overlapped")])
def test_resume_from_snapshot_is_bit_identical(kda, fused, overlap, seg, sched):
    B, T, H, D, every = 2, 900, 3, 128, 3
    x = gen_inputs(_wl(B, T, H, D, "bf16", seed=17))
    t = {n: dev(x[n]) for n in NAMES + ("A", "S0")}
    kw = dict(overlap=overlap, segment_tokens=seg, fused=fused)
    if sched == "overlapped":  # two segments of records: the double-buffered schedule
        desc = kda.make_desc(B, T, H, D, kda.KDA_BF16, kda.KDA_BF16, segment_tokens=seg, overlap=True, fused=False)
        kw["workspace"] = torch.empty(kda.workspace_size(desc, 2 * seg), dtype=torch.uint8, device="cuda")
        assert kda.schedule(desc, kw["workspace"].numel())[1] == "overlapped"
    elif sched == "pipelined":
        desc = kda.make_desc(B, T, H, D, kda.KDA_BF16, kda.KDA_BF16, segment_tokens=seg, overlap=True, fused=False)
        assert kda.schedule(desc, kda.workspace_size(desc))[1] == "pipelined"
    plain = _fwd(kda, t, t["S0"], **kw)
    full = _fwd(kda, t, t["S0"], snapshot_chunks=every, **kw)
    for key in ("o", "y", "S_T"):
        assert _bit_equal(plain[key], full[key]), key
    n = full["snapshots"].shape[1]
    assert n == T // (64 * every) == 4
    for j in range(n):
        tj = (j + 1) * 64 * every
        rest = {m: t[m][:, tj:].contiguous() for m in NAMES}
        rest["A"] = t["A"]
        r = _fwd(kda, rest, full["snapshots"][:, j].contiguous(), **kw)
        log(f"[resume] {kw} from snapshot {j} (token {tj})")
        for key in ("o", "y"):
            assert _bit_equal(r[key], full[key][:, tj:].contiguous()), (j, key)
        assert _bit_equal(r["S_T"], full["S_T"]), j


@pytest.mark.parametrize("fused", [True, False])
def test_snapshots_only(kda, fused):
    """Snapshots without o, y or S_T (a prefill that only fills the cache)."""
    B, T, H, D = 1, 300, 2, 64
    x = gen_inputs(_wl(B, T, H, D, "bf16", seed=5))
    t = {n: dev(x[n]) for n in NAMES + ("A", "S0")}
    ref = _fwd(kda, t, t["S0"], overlap=False, snapshot_chunks=1, fused=False)
    only = kda.chunk_fwd(t["q"], t["k"], t["v"], t["beta"], t["z"], t["A"], S0=t["S0"], want_o=False,
                         want_state=False, overlap=False, snapshot_chunks=1, fused=fused)
    torch.cuda.synchronize()
    assert set(only) == {"snapshots"}
    assert torch.equal(only["snapshots"], ref["snapshots"])
    assert np.isfinite(host64(only["snapshots"])).all()
