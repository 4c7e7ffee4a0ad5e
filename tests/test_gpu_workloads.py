"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times, against the fp64 oracle (relative L2 <= 3e-3, bf16 inputs,
fp32 state).

prefill   : B4 T4096 H32 d128 with gate; every head checked (o, y, S_T).
k3_layer  : B1 T65536 H96 d128 with gate; the benchmark's exact call (y and
            S_T, the workspace the size query offers) and its no-gate side
            call (o and S_T); every head against the oracle over the whole
            sequence.
decode    : 256 sequences x 96 heads from a random fp32 state, 64 decode
            steps; compared with the chunked forward of the same 64 tokens
            from the same state, and with the oracle on 16 sequences.
"""
import numpy as np
import pytest
import torch

import oracle
from synth.workloads import WORKLOADS, gen_inputs
from kda_gpu_util import dev, host64, log, rel_l2

pytestmark = pytest.mark.gpu
TOL = 3e-3


@pytest.fixture(scope="module")
def kda():
    import gated_delta_rule_84_amd as m
    m.lib()
    return m


def _fwd(kda, x, **kw):
    t = {n: dev(x[n]) for n in ("q", "k", "v", "beta", "z", "A")}
    r = kda.chunk_fwd(t["q"], t["k"], t["v"], t["beta"], t["z"], t["A"],
                      S0=dev(x["S0"]) if "S0" in x else None,
                      gate=dev(x["gate"]) if "gate" in x else None, **kw)
    torch.cuda.synchronize()
    return r


@pytest.mark.timeout(300)
def test_prefill_workload_all_heads(kda):
    wl = WORKLOADS["prefill"]
    log(f"[prefill] generating {wl}")
    x = gen_inputs(wl)
    r = _fwd(kda, x, want_o=True)
    log("[prefill] oracle")
    ref = oracle.forward_c(x["q"], x["k"], x["v"], x["beta"], x["z"], x["A"], gate=x["gate"])
    for key in ("o", "y", "S_T"):
        e = rel_l2(host64(r[key]), ref[key])
        log(f"[prefill] {key} rel_l2={e:.3e}")
        assert e <= TOL, key


def _bench_call(kda, t, out, ws, gate=True):
    """The call bench.py times: y and S_T out (no o), the workspace the size
    query offers (every record resident: the pipelined schedule), or, without
    the gate, o and S_T (bench.py's o_only side line)."""
    kda.chunk_fwd(t["q"], t["k"], t["v"], t["beta"], t["z"], t["A"], gate=t["gate"] if gate else None,
                  want_o=not gate, out=out, workspace=ws)
    torch.cuda.synchronize()


@pytest.mark.timeout(600)
def test_k3_layer_workload_all_heads(kda):
    """Every head of the K3 layer (B1 T65536 H96): y and S_T of the benchmark's
    exact call, and o and S_T of its no-gate side call, against the oracle run
    over the whole sequence of each head (16 heads at a time)."""
    wl = WORKLOADS["k3_layer"]
    log(f"[k3_layer] generating {wl}")
    x = gen_inputs(wl)
    t = {n: dev(x[n]) for n in ("q", "k", "v", "beta", "z", "A", "gate")}
    del x
    B, T, H, D = wl.B, wl.T, wl.H, wl.D
    desc = kda.make_desc(B, T, H, D, kda.KDA_BF16, kda.KDA_BF16)
    ws_bytes = kda.workspace_size(desc)
    log(f"[k3_layer] schedule {kda.schedule(desc, ws_bytes)}")
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    out_y = {"y": torch.empty((B, T, H, D), dtype=torch.bfloat16, device="cuda"),
             "S_T": torch.empty((B, H, D, D), device="cuda")}
    _bench_call(kda, t, out_y, ws)
    y, S_y = out_y["y"].cpu(), out_y["S_T"].cpu()
    out_o = {"o": out_y.pop("y"), "S_T": out_y["S_T"]}
    _bench_call(kda, t, out_o, ws, gate=False)
    o, S_o = out_o["o"].cpu(), out_o["S_T"].cpu()
    del t, out_o, out_y, ws
    torch.cuda.empty_cache()
    assert torch.equal(S_y, S_o)  # the gate never changes the state
    num = {k: 0.0 for k in ("o", "y", "S_T")}
    den = dict(num)
    worst = dict(num)
    G = 16
    for h0 in range(0, H, G):
        log(f"[k3_layer] oracle on heads {h0}..{h0 + G - 1}")
        xs = gen_inputs(wl, heads=(h0, G))
        ref = oracle.forward_c(xs["q"], xs["k"], xs["v"], xs["beta"], xs["z"], xs["A"], gate=xs["gate"])
        got = {"o": o[:, :, h0:h0 + G].float().numpy().astype(np.float64),
               "y": y[:, :, h0:h0 + G].float().numpy().astype(np.float64),
               "S_T": S_y[:, h0:h0 + G].numpy().astype(np.float64)}
        for key in num:
            for i in range(G):
                a = got[key][:, :, i] if key != "S_T" else got[key][:, i]
                r = ref[key][:, :, i] if key != "S_T" else ref[key][:, i]
                d2, r2 = float(np.sum((a - r) ** 2)), float(np.sum(r * r))
                num[key] += d2
                den[key] += r2
                worst[key] = max(worst[key], (d2 / max(r2, 1e-300)) ** 0.5)
        del xs, ref, got
    for key in num:
        e = (num[key] / den[key]) ** 0.5
        log(f"[k3_layer] {key}: rel_l2 over all heads {e:.3e}, worst head {worst[key]:.3e}")
        assert e <= TOL and worst[key] <= TOL, key


@pytest.mark.timeout(300)
def test_decode_workload_vs_chunked_and_oracle(kda):
    wl = WORKLOADS["decode"]
    log(f"[decode] generating {wl}")
    x = gen_inputs(wl)
    n, T, H, D = wl.B, wl.T, wl.H, wl.D
    # chunked forward of the same 64 tokens from the same state
    ch = _fwd(kda, x, out_dtype=torch.float32)
    pool = dev(x["S0"]).clone()
    A = dev(x["A"])
    o_dec = torch.empty((n, T, H, D), device="cuda")
    y_dec = torch.empty((n, T, H, D), device="cuda")
    full = {nm: dev(x[nm]) for nm in ("q", "k", "v", "beta", "z", "gate")}
    for t in range(T):
        st = {nm: full[nm][:, t].contiguous() for nm in full}
        res = kda.recurrent_step(st["q"], st["k"], st["v"], st["beta"], st["z"], A, pool, gate=st["gate"],
                                 out_dtype=torch.float32)
        o_dec[:, t] = res["o"]
        y_dec[:, t] = res["y"]
    torch.cuda.synchronize()
    for key, a, b in (("o", o_dec, ch["o"]), ("y", y_dec, ch["y"]), ("S", pool, ch["S_T"])):
        e = rel_l2(host64(a), host64(b))
        log(f"[decode] decode vs chunked {key}: {e:.3e}")
        assert e <= TOL, key
    m = 16
    ref = oracle.forward_c(x["q"][:m], x["k"][:m], x["v"][:m], x["beta"][:m], x["z"][:m], x["A"],
                           S0=x["S0"][:m], gate=x["gate"][:m])
    for key, a, tol in (("o", o_dec, 1e-5), ("y", y_dec, 1e-5), ("S_T", pool, 1e-5)):
        e = rel_l2(host64(a[:m]), ref[key])
        log(f"[decode] decode vs oracle {key}: {e:.3e}")
        assert e <= tol, key
    for key in ("o", "y", "S_T"):
        e = rel_l2(host64(ch[key][:m]), ref[key])
        log(f"[decode] chunked vs oracle {key}: {e:.3e}")
        assert e <= TOL, key
