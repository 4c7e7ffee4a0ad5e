"""Head-first token layout (kda_desc.tokens = KDA_TOKENS_BHTD): the forward
with q, k, z, v, gate, o, y as [B, H, T, D] and beta as [B, H, T] gives
bit-identical results to the token-major call on the same values, on every
schedule that takes it (one stream with the split scan and with one
workgroup per head, the overlapped and pipelined schedules, the fused
kernel, prefix-cache snapshots, the no-alloc entry point) and for fp32
inputs.  The token-major path itself is checked against the fp64 oracle by
the other GPU tests; a second, oracle-checked case here covers a head-first
call directly."""
import pytest
import torch

import oracle
from synth.workloads import Workload, gen_inputs
from kda_gpu_util import dev, host64, log, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    import gated_delta_rule_84_amd as m
    assert torch.cuda.is_available()
    m.lib()
    return m


def _inputs(B, T, H, D, dtype, seed):
    wl = Workload("layout", 900 + seed, B=B, T=T, H=H, D=D, dtype=dtype, z_std=2.0, A_kind="uniform",
                  gate=True, s0_std=0.1)
    x = gen_inputs(wl)
    return {n: dev(x[n]) for n in ("q", "k", "v", "beta", "z", "A", "gate", "S0")}, x


def _head_first(t):
    """The same values with the token and head axes swapped (contiguous)."""
    out = dict(t)
    for n in ("q", "k", "v", "z", "gate"):
        out[n] = t[n].permute(0, 2, 1, 3).contiguous()
    out["beta"] = t["beta"].permute(0, 2, 1).contiguous()
    return out


def _call(kda, t, noalloc=False, **kw):
    fn = kda.chunk_fwd_noalloc if noalloc else kda.chunk_fwd
    r = fn(t["q"], t["k"], t["v"], t["beta"], t["z"], t["A"], S0=t["S0"], gate=t["gate"], **kw)
    torch.cuda.synchronize()
    return r


def _bit_equal(a, b):
    if a.dtype == torch.bfloat16:
        a, b = a.view(torch.int16), b.view(torch.int16)
    return torch.equal(a, b)


CASES = [
    # name, B, T, H, D, dtype, schedule expected, call options
    ("one stream, split scan", 2, 300, 3, 128, "bf16", "segments", {"overlap": False, "fused": False}),
    ("one stream, one workgroup per head", 2, 200, 80, 128, "bf16", "segments", {"overlap": False, "fused": False}),
    ("pipelined", 1, 9000, 4, 128, "bf16", "pipelined", {"fused": False}),
    ("overlapped", 2, 2048, 4, 128, "bf16", "overlapped", {"fused": False, "segment_tokens": 64,
                                                           "ws_segment": 128}),
    ("fused", 1, 500, 2, 128, "bf16", "fused", {"fused": True}),
    ("fp32 inputs, d = 64", 1, 333, 2, 64, "f32", "segments", {"overlap": False, "fused": False}),
    ("snapshots", 1, 700, 2, 128, "bf16", None, {"overlap": False, "fused": False, "snapshot_chunks": 3}),
    ("no-alloc entry point", 2, 150, 3, 128, "bf16", None, {"noalloc": True}),
    ("one token", 2, 1, 3, 128, "bf16", None, {"fused": False}),
    ("no tokens (state copied)", 2, 0, 3, 128, "bf16", None, {"fused": False}),
    ("o only, ragged, d = 64", 1, 65, 2, 64, "bf16", None, {"fused": False, "want_y": False}),
]


@pytest.mark.parametrize("name,B,T,H,D,dtype,sched,opts", CASES, ids=[c[0] for c in CASES])
def test_head_first_matches_token_major(kda, name, B, T, H, D, dtype, sched, opts):
    opts = dict(opts)
    ws_segment = opts.pop("ws_segment", None)
    t, _ = _inputs(B, T, H, D, dtype, seed=B * 100 + H)
    kdt = kda.KDA_BF16 if dtype == "bf16" else kda.KDA_F32
    extra = {}
    if sched is not None:
        desc = kda.make_desc(B, T, H, D, kdt, kdt, segment_tokens=opts.get("segment_tokens", 0),
                             overlap=opts.get("overlap", True), fused=opts.get("fused"), head_first=True)
        nbytes = kda.workspace_size(desc, ws_segment)
        assert kda.schedule(desc, nbytes)[1] == sched
        if ws_segment is not None:
            extra["workspace"] = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    log(f"[layout] {name}: B={B} T={T} H={H} D={D} {dtype}")
    ref = _call(kda, t, **opts, **extra)
    hf = _call(kda, _head_first(t), head_first=True, **opts, **extra)
    keys = [k for k in ("o", "y", "S_T", "snapshots") if ref.get(k) is not None]
    assert {"o", "S_T"} <= set(keys) and all(k in hf for k in keys)
    for key in keys:
        got = hf[key].permute(0, 2, 1, 3) if key in ("o", "y") else hf[key]
        assert tuple(got.shape) == tuple(ref[key].shape), key
        assert _bit_equal(got.contiguous(), ref[key]), key


def test_head_first_pipelined_vs_oracle(kda):
    """A head-first call on the pipelined schedule against the fp64 oracle of
    the same values (token-major there): o, y and S_T within the bf16 bar."""
    B, T, H, D = 1, 8256, 2, 128
    t, x = _inputs(B, T, H, D, "bf16", seed=77)
    desc = kda.make_desc(B, T, H, D, kda.KDA_BF16, kda.KDA_BF16, head_first=True)
    assert kda.schedule(desc, kda.workspace_size(desc))[1] == "pipelined"
    r = _call(kda, _head_first(t), head_first=True, fused=False)
    ref = oracle.forward_c(x["q"], x["k"], x["v"], x["beta"], x["z"], x["A"], S0=x["S0"], gate=x["gate"])
    errs = {"o": rel_l2(host64(r["o"].permute(0, 2, 1, 3)), ref["o"]),
            "y": rel_l2(host64(r["y"].permute(0, 2, 1, 3)), ref["y"]),
            "S_T": rel_l2(host64(r["S_T"]), ref["S_T"])}
    log(f"[layout] head first vs oracle: " + " ".join(f"{k}={v:.3e}" for k, v in errs.items()))
    assert all(v <= 3e-3 for v in errs.values()), errs


def test_head_first_pipelined_windows(kda):
    """Head first on the pipelined schedule in windows (a workspace of 512
    chunks of records: two windows, the second short and ragged, each
    starting at a token offset): bit-identical to the token-major call with
    the same workspace, snapshots across the windows included."""
    B, T, H, D = 1, 625 * 64 - 20, 3, 128
    t, _ = _inputs(B, T, H, D, "bf16", seed=55)
    desc = kda.make_desc(B, T, H, D, kda.KDA_BF16, kda.KDA_BF16, head_first=True)
    nbytes = kda.workspace_size(desc, 512 * 64)
    assert kda.schedule(desc, nbytes)[1] == "pipelined"
    assert kda.launches(desc, nbytes) == ["intra", "scan"] * 2
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    log(f"[layout] pipelined windows head first: B={B} T={T} H={H}")
    ref = _call(kda, t, fused=False, workspace=ws, snapshot_chunks=100)
    hf = _call(kda, _head_first(t), head_first=True, fused=False, workspace=ws, snapshot_chunks=100)
    assert kda.call_status(desc, ws) == 0
    for key in ("o", "y", "S_T", "snapshots"):
        got = hf[key].permute(0, 2, 1, 3) if key in ("o", "y") else hf[key]
        assert _bit_equal(got.contiguous(), ref[key]), key
