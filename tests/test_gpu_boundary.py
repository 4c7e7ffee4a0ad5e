"""GPU tests of the boundary's failure handling and memory discipline: state
pool slots outside the pool, the status word of the two-stream schedules
(with a producer the host withholds, so that the scan's own bounded wait runs
out while every kernel still exits normally), guard bands around the
workspace and the outputs, and a forward captured into a HIP graph.

Source of the computation: "Kimi K3: KDA, Attention Residuals and Stable
LatentMoE", sections 2.1-2.3."""
import os

import numpy as np
import pytest
import torch

from synth.workloads import Workload, gen_inputs
from kda_gpu_util import dev, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    import gated_delta_rule_84_amd as m
    m.lib()
    return m


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def _inputs(B, T, H, D, seed, s0=0.1):
    wl = Workload("boundary", 130 + seed, B=B, T=T, H=H, D=D, dtype="bf16", z_std=2.0, A_kind="uniform", gate=True,
                  s0_std=s0)
    x = gen_inputs(wl)
    t = {n: dev(x[n]) for n in ("q", "k", "v", "beta", "z", "A", "gate")}
    t["S0"] = dev(x["S0"]) if "S0" in x else None
    return t


def test_decode_skips_and_flags_out_of_range_slots(kda):
    n, H, D, n_slots = 4, 2, 128, 6
    t = _inputs(n, 1, H, D, seed=1, s0=0.0)
    step = {k: t[k][:, 0].contiguous() for k in ("q", "k", "v", "beta", "z", "gate")}
    pool = torch.randn((n_slots, H, D, D), device="cuda") * 0.1
    slot = torch.tensor([5, -1, 2, 6], dtype=torch.int32, device="cuda")  # -1 and 6 lie outside [0, 6)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    before = pool.clone()
    o = torch.full((n, H, D), 7.0, device="cuda")
    kda.recurrent_step(step["q"], step["k"], step["v"], step["beta"], step["z"], t["A"], pool, slot=slot,
                       gate=step["gate"], out_dtype=torch.float32, out={"o": o}, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == kda.FLAG_BAD_SLOT
    for s in (0, 1, 3, 4):  # rows no valid slot names are untouched
        assert torch.equal(pool[s], before[s]), s
    assert not torch.equal(pool[5], before[5]) and not torch.equal(pool[2], before[2])
    assert torch.all(o[1] == 7.0) and torch.all(o[3] == 7.0)  # skipped sequences' outputs untouched
    assert torch.isfinite(o[0]).all() and torch.isfinite(o[2]).all()
    # in-range slots only: the flag stays clear
    status.zero_()
    kda.recurrent_step(step["q"], step["k"], step["v"], step["beta"], step["z"], t["A"], pool,
                       slot=torch.tensor([0, 1, 2, 3], dtype=torch.int32, device="cuda"), gate=step["gate"],
                       status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0


def test_state_io_skips_and_flags_out_of_range_slots(kda):
    H, D, n_slots = 3, 64, 4
    pool = torch.randn((n_slots, H, D, D), device="cuda")
    user = torch.randn((3, H, D, D), device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    before = pool.clone()
    slot = torch.tensor([2, 4, 100], dtype=torch.int32, device="cuda")
    kda.state_io(kda.STATE_IMPORT, pool, user, slot=slot, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == kda.FLAG_BAD_SLOT
    assert torch.equal(pool[2], user[0])
    for s in (0, 1, 3):
        assert torch.equal(pool[s], before[s]), s


def test_status_word_reports_a_withheld_producer(kda):
    """Pipelined schedule (sixteen 128-token segments); the host launches only
    the first segment's producer, so the scan's bounded wait for the second
    runs out (about a second): outputs are invalid (NaN) and
    kda_chunk_fwd_status says so.  A normal call through the same workspace
    reports KDA_OK again."""
    B, T, H, D = 1, 2048, 2, 128
    t = _inputs(B, T, H, D, seed=2)
    desc = kda.make_desc(B, T, H, D, kda.KDA_BF16, kda.KDA_BF16, segment_tokens=128)
    ws = torch.empty(kda.workspace_size(desc), dtype=torch.uint8, device="cuda")
    assert kda.schedule(desc, ws.numel())[1] == "pipelined"

    def run():
        return kda.chunk_fwd(t["q"], t["k"], t["v"], t["beta"], t["z"], t["A"], S0=t["S0"], gate=t["gate"],
                             workspace=ws, segment_tokens=128)

    good = {k: v.clone() for k, v in run().items()}
    assert kda.call_status(desc, ws) == 0
    os.environ["KDA_TEST_PRODUCED_SEGMENTS"] = "1"
    try:
        log("[status] producer withheld: the scan's bounded wait runs out (about a second)")
        bad = run()
        assert kda.call_status(desc, ws) == 8  # KDA_ERR_TIMEOUT
    finally:
        del os.environ["KDA_TEST_PRODUCED_SEGMENTS"]
    assert torch.isnan(bad["o"].float()).any()
    again = run()
    assert kda.call_status(desc, ws) == 0
    for key in ("o", "y", "S_T"):
        assert torch.equal(_bits(again[key]), _bits(good[key])), key


@pytest.mark.parametrize("sched,head_first", [("pipelined", False), ("overlapped", False), ("segments", False),
                                              ("pipelined", True), ("segments", True)])
def test_guard_bands_around_workspace_and_outputs(kda, sched, head_first):
    """Workspace, o, y and S_T carved out of one buffer with 64 KiB guard bands
    of a fixed pattern between them; after the call every guard is intact
    (token major, and head first)."""
    B, T, H, D = 1, 1536, 3, 128
    t = _inputs(B, T, H, D, seed=3)
    tok = (B, T, H, D)
    if head_first:
        for n in ("q", "k", "v", "z", "gate"):
            t[n] = t[n].permute(0, 2, 1, 3).contiguous()
        t["beta"] = t["beta"].permute(0, 2, 1).contiguous()
        tok = (B, H, T, D)
    seg = 128
    desc = kda.make_desc(B, T, H, D, kda.KDA_BF16, kda.KDA_BF16, segment_tokens=seg if sched != "segments" else 0,
                         overlap=sched != "segments", head_first=head_first)
    if sched == "pipelined":
        ws_bytes = kda.workspace_size(desc)
    elif sched == "overlapped":
        ws_bytes = kda.workspace_size(desc, 2 * seg)
    else:
        ws_bytes = kda.workspace_size(desc, 256)
    assert kda.schedule(desc, ws_bytes)[1] == sched
    G = 64 << 10
    sizes = [ws_bytes, B * T * H * D * 2, B * T * H * D * 2, B * H * D * D * 4]
    offs, at = [], G
    for sz in sizes:
        offs.append(at)
        at += (sz + 255) // 256 * 256 + G
    buf = torch.empty(at, dtype=torch.uint8, device="cuda")
    pattern = torch.arange(at, device="cuda", dtype=torch.int64).remainder(251).to(torch.uint8)
    buf.copy_(pattern)
    ws = buf[offs[0]:offs[0] + ws_bytes]
    out = {"o": buf[offs[1]:offs[1] + sizes[1]].view(torch.bfloat16).view(tok),
           "y": buf[offs[2]:offs[2] + sizes[2]].view(torch.bfloat16).view(tok),
           "S_T": buf[offs[3]:offs[3] + sizes[3]].view(torch.float32).view(B, H, D, D)}
    r = kda.chunk_fwd(t["q"], t["k"], t["v"], t["beta"], t["z"], t["A"], S0=t["S0"], gate=t["gate"], out=out,
                      workspace=ws, segment_tokens=seg if sched != "segments" else 256,
                      overlap=sched != "segments", head_first=head_first)
    torch.cuda.synchronize()
    assert kda.call_status(desc, ws) == 0
    used = torch.zeros(at, dtype=torch.bool, device="cuda")
    for o_, sz in zip(offs, sizes):
        used[o_:o_ + sz] = True
    assert torch.equal(buf[~used], pattern[~used]), "a guard band was written"
    ref = kda.chunk_fwd(t["q"], t["k"], t["v"], t["beta"], t["z"], t["A"], S0=t["S0"], gate=t["gate"],
                        overlap=False, head_first=head_first)
    for key in ("o", "y", "S_T"):
        assert torch.equal(_bits(r[key]), _bits(ref[key])), key


@pytest.mark.parametrize("head_first", [False, True])
def test_forward_captured_in_a_graph(kda, head_first):
    """A call whose stream is being captured takes the one-stream schedule (no
    in-kernel waits for producers a graph may order after the scan); the graph
    replays, with eager work and synchronisations in between, give the eager
    result bit for bit every time (token major, and head first)."""
    B, T, H, D = 1, 2048, 2, 128
    t = _inputs(B, T, H, D, seed=4)
    tok = (B, T, H, D)
    if head_first:
        for n in ("q", "k", "v", "z", "gate"):
            t[n] = t[n].permute(0, 2, 1, 3).contiguous()
        t["beta"] = t["beta"].permute(0, 2, 1).contiguous()
        tok = (B, H, T, D)
    desc = kda.make_desc(B, T, H, D, kda.KDA_BF16, kda.KDA_BF16, head_first=head_first)
    ws = torch.empty(kda.workspace_size(desc), dtype=torch.uint8, device="cuda")
    out = {"o": torch.empty(tok, dtype=torch.bfloat16, device="cuda"),
           "y": torch.empty(tok, dtype=torch.bfloat16, device="cuda"),
           "S_T": torch.empty((B, H, D, D), device="cuda")}
    eager = {k: v.clone() for k, v in kda.chunk_fwd(t["q"], t["k"], t["v"], t["beta"], t["z"], t["A"], S0=t["S0"],
                                                     gate=t["gate"], out=out, workspace=ws,
                                                     head_first=head_first).items()}
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            kda.chunk_fwd(t["q"], t["k"], t["v"], t["beta"], t["z"], t["A"], S0=t["S0"], gate=t["gate"], out=out,
                          workspace=ws, head_first=head_first)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        for v_ in out.values():
            v_.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for key in ("o", "y", "S_T"):
            assert torch.equal(_bits(out[key]), _bits(eager[key])), (rep, key)
        junk = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        del junk
