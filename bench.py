"""Benchmark of the KDA forward hot path on one MI355X.

One step = one kda_chunk_fwd call over the K3-shaped layer workload
(B1, T65536, H96, d128, bf16 inputs, fp32 state, output gate, y and S_T
outputs), inputs already resident in HBM.  Prints ONE JSON line.

The library picks the schedule for the workspace the size query offers (the
pipelined two-kernel schedule for long sequences: every chunk record resident,
one scan launch, or windows of records beyond the query's cap); --schedule
forces one (the fused kernel measured slower at every size tried).
--workload selects another configuration (long ones are generated slab by
slab on the device).  K timed steps follow W warm-up steps; the JSON line
gives their mean (ms_per_step, and `value`), median and minimum.

Roofline (`roofline`): the dominant kernel is the one with the longest
average launch (the pipelined schedule's single scan launch, which spans the
step); its achieved bandwidth is the path's algorithmic bytes of the
token-heads one launch processes -- 1,538 B per token-head at d = 128: q, k, z,
v, gate logits in and y out at 2d bytes each, beta 2 bytes -- plus the state,
over the launch's average duration measured with HIP events that the library
records around each of its launches on the launch stream
(kda_chunk_fwd_traced, in the order kda_chunk_fwd_launches reports).
`kernel_share` gives the same kernel's own inputs and outputs instead:
  intra-chunk : q, k, z (3 * 2d B) + beta (2 B) per token-head
  state scan  : v, gate logits in, y out (3 * 2d B) per token-head + final state
After the timed loop (outside it) the timed outputs are checked: finite, the
library's status word clear (kda_chunk_fwd_status), and, in the CPU-baseline
leg, y of the first and last sampled head against the fp64 oracle (<= 3e-3).
Side measurements (skipped with their --no-* flags): the same forward
without the output gate (o and S_T out, 1,282 B per token-head; sequences up
to 65,536 tokens), the prefill workload (B4 T4096 H32), the input steps, the
decode step and the state export, the same K3-layer forward with the
tensors head first ([B, H, T, d]: y checked bit for bit against the
headline call's), and the long-context workload (B1
T1,048,576 H96, the workspace the size query offers; up to 5 timed calls
after its inputs are generated, which takes about a minute).  The CPU
baseline is the fp64 C oracle on every host core the process may use, over
a bounded sample of heads.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA fwd tokens·heads/s at T=64K,H=96,d=128 bf16; % MFMA/HBM peak"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA


def kernel_bytes(name: str, token_heads: int, d: int, BH: int, T: int) -> float:
    """Algorithmic HBM bytes of one kernel's launches in a step (its share of
    the path's inputs and outputs; intermediates between the two kernels are
    not algorithmic)."""
    if name == "fused":
        return token_heads * (6 * 2 * d + 2) + 2 * BH * d * d * 4  # every input and output
    if name == "intra":
        return token_heads * (3 * 2 * d + 2)          # q, k, z, beta
    if name == "scan":
        return token_heads * (3 * 2 * d) + BH * d * d * 4  # v, gate in, y out; final state
    raise KeyError(name)


def kernel_source_hash() -> str:
    """sha256 over the HIP sources of the library (what a traffic profile was taken with)."""
    import hashlib
    csrc = os.path.join(ROOT, "gated_delta_rule_84_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".hpp", ".cpp")):
            h.update(name.encode())
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def profiled_traffic(kernel: str, workload: str):
    """Measured HBM bytes per launch of `kernel` from the committed counter
    summary profiles/hbm_traffic_<workload>.txt (rocprofv3 FETCH_SIZE and
    WRITE_SIZE scaled by a plain-copy calibration), or None when that summary
    is missing or was taken with different kernel sources."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            key, _, val = line.partition(":")
            vals[key.strip()] = val.strip()
    if vals.get("source_sha256") != kernel_source_hash():
        return None
    try:
        return float(vals[f"{kernel}_hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def profiled_counters(workload: str):
    """MFMA figures measured by rocprofv3 SQ counters, from the committed
    summary profiles/counters_<workload>.txt (MFMA busy share of the SIMDs a
    kernel occupies, achieved MFMA TFLOP/s, LDS bank-conflict share), or None
    when that summary is missing or was taken with different kernel sources."""
    path = os.path.join(ROOT, "profiles", f"counters_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals, sha = {}, None
    for line in open(path):
        if line.startswith("# source_sha256:"):
            sha = line.split(":", 1)[1].strip()
        elif ":" in line and not line.startswith(("#", "[")):
            key, _, val = line.partition(":")
            vals[key.strip()] = val.strip()
    if sha != kernel_source_hash():
        return None
    keys = ("scan_mfma_busy_own_cus", "scan_mfma_busy_chip", "scan_mfma_tflops", "intra_mfma_busy_chip",
            "intra_mfma_tflops", "scan_lds_bank_conflict_share", "intra_lds_bank_conflict_share")
    try:
        out = {k: float(vals[k]) for k in keys if k in vals}
    except ValueError:
        return None
    if not out:
        return None
    out["bf16_mfma_peak_TFLOPs"] = BF16_PEAK_TFLOPS
    out["source"] = f"profiles/counters_{workload}.txt"
    return out


def path_bytes_per_token_head(d: int) -> int:
    # q, k, z, v, gate logits in and y out (bf16, 2d bytes each) + beta (2 bytes): 1,538 B at d = 128
    return 6 * 2 * d + 2


def path_flops_per_token_head(d: int, C: int = 64) -> float:
    # 6 d^2 (state products) + 5 (C + 16) d (sub-tile products) + C^2 / 3 (UT inverse)
    return 6 * d * d + 5 * (C + 16) * d + C * C / 3


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, heads: int, y_gpu=None) -> dict:
    """The fp64 C oracle (sequential recurrence + gate, OpenMP over heads) on
    every host core the process may use, over heads 0 .. heads - 1 of the
    workload; with y_gpu (the GPU's y of those heads from the timed loop) the
    oracle's y also spot-checks it (relative L2 on the first and last sampled
    head)."""
    import oracle
    from synth.workloads import gen_inputs

    threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    x = gen_inputs(wl, heads=(0, heads))
    t0 = time.perf_counter()
    ref = oracle.forward_c(x["q"], x["k"], x["v"], x["beta"], x["z"], x["A"], gate=x["gate"], nthreads=threads,
                           want_o=False)
    dt = time.perf_counter() - t0
    th = wl.B * wl.T * heads
    res = {"value": th / dt, "unit": "tokens·heads/s", "cores": threads, "kind": "oracle",
           "nproc": os.cpu_count(), "cpu_model": cpu_model(),
           "sample": f"fp64 C oracle (sequential recurrence + gate, OpenMP over heads) on heads 0..{heads - 1} "
                     f"of the {wl.name} workload, all {wl.T} tokens ({th} token-heads, {dt:.1f} s, "
                     f"{threads} threads)"}
    if y_gpu is not None:
        errs = {}
        for hh in sorted({0, heads - 1}):
            a = y_gpu[:, :, hh].astype(np.float64)
            r = ref["y"][:, :, hh]
            errs[f"head_{hh}"] = float(np.linalg.norm(a - r) / np.linalg.norm(r))
        res["parity_y_rel_l2"] = errs
        res["parity_ok"] = all(e <= 3e-3 for e in errs.values())
    return res


def all_finite(x) -> bool:
    """Whether every element of a device tensor is finite, checked in slices
    along its second dimension so that no temporary larger than about 256 MB
    is allocated (a T = 1M output is 26 GB)."""
    import torch
    x = x.reshape(x.shape[0], x.shape[1], -1) if x.dim() > 2 else x.reshape(1, x.shape[0], -1)
    per = max(1, (256 << 20) // max(1, x.shape[0] * x.shape[2]))
    for t0 in range(0, x.shape[1], per):
        if not bool(torch.isfinite(x[:, t0:t0 + per]).all().item()):
            return False
    return True


def time_calls(fn, steps: int, warmup: int):
    """Mean, median and minimum milliseconds of `steps` calls of fn (events on
    the current stream between the calls)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    marks[0].record()
    for k in range(steps):
        fn()
        marks[k + 1].record()
    torch.cuda.synchronize()
    per = [marks[k].elapsed_time(marks[k + 1]) for k in range(steps)]
    return marks[0].elapsed_time(marks[-1]) / steps, float(np.median(per)), float(np.min(per))


def time_prefill(kda, wl, steps: int, warmup: int) -> dict:
    """The prefill workload (B4 T4096 H32 d128, bf16, gate; y and S_T out) with
    the library's own schedule for the workspace its size query offers."""
    import torch
    from synth.workloads import gen_inputs

    x = gen_inputs(wl)
    t = {k: torch.from_numpy(np.ascontiguousarray(v).view(np.int16) if v.dtype == np.uint16 else v).cuda()
         for k, v in x.items()}
    for k, v in x.items():
        if v.dtype == np.uint16:
            t[k] = t[k].view(torch.bfloat16)
    del x
    B, T, H, D = wl.B, wl.T, wl.H, wl.D
    desc = kda.make_desc(B, T, H, D, kda.KDA_BF16, kda.KDA_BF16)
    ws = torch.empty(kda.workspace_size(desc), dtype=torch.uint8, device="cuda")
    out = {"y": torch.empty((B, T, H, D), dtype=torch.bfloat16, device="cuda"),
           "S_T": torch.empty((B, H, D, D), device="cuda")}

    def call():
        kda.chunk_fwd(t["q"], t["k"], t["v"], t["beta"], t["z"], t["A"], gate=t["gate"], want_o=False, out=out,
                      workspace=ws)

    ms, med, mn = time_calls(call, steps, warmup)
    th = B * T * H
    nbytes = th * path_bytes_per_token_head(D) + 2 * B * H * D * D * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": wl.name, "B": B, "T": T, "H": H, "d": D, "schedule": kda.schedule(desc, ws.numel())[1],
            "ms": ms, "ms_median": med, "ms_min": mn, "token_heads_per_s": th / (ms * 1e-3),
            "algorithmic_bytes": nbytes, "achieved_GBs": gbs, "frac_hbm": gbs / HBM_PEAK_GBS,
            "outputs_finite": all_finite(out["y"])}


def load_inputs(wl, dev) -> dict:
    """The workload's seeded inputs as device tensors (bf16 as torch.bfloat16).
    Long sequences are generated slab by slab straight into the device
    tensors (the whole host copy would be ~150 GB at 1M tokens)."""
    import torch
    from synth.workloads import gen_inputs

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    slab = 65536
    if wl.T > slab and wl.T % slab == 0:
        t = {}
        for t0 in range(0, wl.T, slab):
            x = gen_inputs(wl, time=(t0, slab))
            for k, v in x.items():
                if k in ("A", "S0"):
                    t.setdefault(k, to_dev(v))
                    continue
                if k not in t:
                    t[k] = torch.empty((wl.B, wl.T) + v.shape[2:],
                                       dtype=torch.bfloat16 if v.dtype == np.uint16 else torch.float32, device=dev)
                t[k][:, t0:t0 + slab].copy_(to_dev(v))
            del x
            print(f"inputs {wl.name}: tokens {t0 + slab}/{wl.T}", file=sys.stderr, flush=True)
        return t
    x = gen_inputs(wl)
    return {k: to_dev(v) for k, v in x.items()}


def time_long_context(kda, wl, steps: int, warmup: int) -> dict:
    """The long-context workload (B1 T1,048,576 H96 d128, bf16, gate; y and
    S_T out) with the workspace the size query offers (the pipelined
    schedule over windows of records within its cap)."""
    import torch

    dev = torch.device("cuda:0")
    t_gen = time.perf_counter()
    t = load_inputs(wl, dev)
    t_gen = time.perf_counter() - t_gen
    B, T, H, D = wl.B, wl.T, wl.H, wl.D
    desc = kda.make_desc(B, T, H, D, kda.KDA_BF16, kda.KDA_BF16)
    ws_bytes = kda.workspace_size(desc)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    out = {"y": torch.empty((B, T, H, D), dtype=torch.bfloat16, device=dev),
           "S_T": torch.empty((B, H, D, D), device=dev)}

    def call():
        kda.chunk_fwd(t["q"], t["k"], t["v"], t["beta"], t["z"], t["A"], S0=t.get("S0"), gate=t["gate"],
                      want_o=False, out=out, workspace=ws)

    ms, med, mn = time_calls(call, steps, warmup)
    th = B * T * H
    nbytes = th * path_bytes_per_token_head(D) + 2 * B * H * D * D * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    res = {"workload": wl.name, "B": B, "T": T, "H": H, "d": D, "schedule": kda.schedule(desc, ws_bytes)[1],
           "workspace_bytes": ws_bytes, "launches": len(kda.launches(desc, ws_bytes)),
           "ms": ms, "ms_median": med, "ms_min": mn, "steps": steps, "warmup": warmup,
           "token_heads_per_s": th / (ms * 1e-3), "algorithmic_bytes": nbytes, "achieved_GBs": gbs,
           "frac_hbm": gbs / HBM_PEAK_GBS, "input_setup_s": t_gen,
           "outputs_finite": all_finite(out["y"]) and all_finite(out["S_T"]),
           "library_status_ok": kda.call_status(desc, ws) == 0}
    del t, out, ws
    torch.cuda.empty_cache()
    return res


def measure_peaks(kda) -> dict:
    """What this GPU achieves against the published peaks (8 TB/s HBM, 2.5
    PFLOP/s dense bf16 MFMA, 157.3 TFLOP/s fp32): the library's state copy
    (kda_state_io export, non-temporal 16-byte loads and stores) over a pool
    of 1,536 x 96 states (2 x 9.7 GB moved per call), a torch device copy of
    4 GiB, and square GEMMs of torch (hipBLASLt) at n = 8,192."""
    import torch

    res = {"hbm_peak_GBs": HBM_PEAK_GBS, "bf16_mfma_peak_TFLOPs": BF16_PEAK_TFLOPS, "fp32_peak_TFLOPs": 157.3}
    pool = torch.zeros((1536, 96, 128, 128), device="cuda")
    user = torch.empty_like(pool)
    ms, med, _ = time_calls(lambda: kda.state_io(kda.STATE_EXPORT, pool, user), 10, 2)
    nbytes = 2 * pool.numel() * 4
    res["state_copy"] = {"bytes": nbytes, "ms_median": med, "GBs": nbytes / (med * 1e-3) / 1e9}
    del pool, user
    a = torch.empty(1 << 30, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    ms, med, _ = time_calls(lambda: b.copy_(a), 10, 2)
    res["torch_copy"] = {"bytes": 2 * a.numel() * 4, "ms_median": med, "GBs": 2 * a.numel() * 4 / (med * 1e-3) / 1e9}
    del a, b
    n = 8192
    for dt, name in ((torch.bfloat16, "gemm_bf16"), (torch.float32, "gemm_fp32")):
        x = torch.randn((n, n), device="cuda").to(dt)
        y = torch.randn((n, n), device="cuda").to(dt)
        ms, med, _ = time_calls(lambda: torch.mm(x, y), 10, 3)
        res[name] = {"n": n, "ms_median": med, "TFLOPs": 2 * n ** 3 / (med * 1e-3) / 1e12}
        del x, y
    torch.cuda.empty_cache()
    return res


def time_head_first(kda, t, out, ws, B, T, H, D, steps: int, warmup: int) -> dict:
    """The same forward with the per-token tensors head first ([B, H, T, d],
    beta [B, H, T]; kda_desc.tokens = KDA_TOKENS_BHTD), as a caller whose
    projections write each head's tokens in one block would pass them; y is
    compared bit for bit with the token-major call's (its last timed step)."""
    import torch

    hf = {n: t[n].permute(0, 2, 1, 3).contiguous() for n in ("q", "k", "v", "z", "gate")}
    hf["beta"] = t["beta"].permute(0, 2, 1).contiguous()
    y_hf = torch.empty((B, H, T, D), dtype=out["y"].dtype, device=out["y"].device)
    st_hf = torch.empty_like(out["S_T"])

    def call():
        kda.chunk_fwd(hf["q"], hf["k"], hf["v"], hf["beta"], hf["z"], t["A"], S0=t.get("S0"), gate=hf["gate"],
                      want_o=False, out={"y": y_hf, "S_T": st_hf}, workspace=ws, head_first=True)

    ms, med, mn = time_calls(call, steps, warmup)
    same = all(torch.equal(y_hf[:, h].view(torch.int16), out["y"][:, :, h].view(torch.int16)) for h in range(H))
    same = same and torch.equal(st_hf, out["S_T"])
    th = B * T * H
    nbytes = th * path_bytes_per_token_head(D) + 2 * B * H * D * D * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    del hf, y_hf, st_hf
    torch.cuda.empty_cache()
    return {"layout": "[B, H, T, d]", "ms": ms, "ms_median": med, "ms_min": mn, "token_heads_per_s": th / (ms * 1e-3),
            "algorithmic_bytes": nbytes, "achieved_GBs": gbs, "frac_hbm": gbs / HBM_PEAK_GBS,
            "bit_identical_to_token_major": bool(same)}


def time_input_prep(kda, t, B, T, H, D, steps, warmup, workload, W=4):
    """The input steps before the core (q, k, v = Swish(ShortConv(x)), beta =
    Sigmoid(logit)) at the workload's shapes: the workload's q, k, v, beta
    tensors stand in for the projections (the timing does not depend on the
    values); taps seeded.  Algorithmic bytes: x_q, x_k, x_v and the beta
    logit read, q, k, v and beta written = 3 * 2 * 2D + 2 * 2 per token-head."""
    import torch
    from synth.workloads import gen_prep_inputs
    w = gen_prep_inputs(1, 1, H, D, W, "bf16", seed=5, with_state=False)
    ws = [torch.from_numpy(w[n]).cuda() for n in ("wq", "wk", "wv")]
    out = {n: torch.empty_like(t["q"]) for n in ("q", "k", "v")}
    out["beta"] = torch.empty_like(t["beta"])

    def call():
        kda.input_prep(t["q"], t["k"], t["v"], *ws, beta_logits=t["beta"], out=out)

    for _ in range(warmup):
        call()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        call()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    nbytes = B * T * H * (3 * 2 * 2 * D + 2 * 2)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"conv_width": W, "ms": ms, "algorithmic_bytes": nbytes, "achieved_GBs": gbs,
            "frac_hbm": gbs / HBM_PEAK_GBS, "launches": 2,
            "traffic": profiled_traffic("prep_conv", workload)}


def time_decode(kda, H, D, steps, warmup, n=256):
    """Decode steps (kda_recurrent_step) for n sequences of H heads, one token
    each, with the fp32 state pool [n, H, D, D] updated in place and y = the
    gated output (bf16), as in the decode workload.  Inputs are seeded random
    values (the timing does not depend on them).  Algorithmic bytes per
    call: the state read and written (8 D^2) plus q, k, v, z, gate read and y
    written (12 D) and beta (2) per token-head."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(7)
    bf = torch.bfloat16
    x = {nm: torch.randn((n, H, D), generator=g, device="cuda").to(bf) for nm in ("q", "k", "v", "z", "gate")}
    beta = torch.sigmoid(torch.randn((n, H), generator=g, device="cuda")).to(bf)
    A = torch.rand((H,), generator=g, device="cuda") * 2 - 1
    pool = torch.randn((n, H, D, D), generator=g, device="cuda") * 0.1
    out = {"y": torch.empty((n, H, D), dtype=bf, device="cuda")}

    def call():
        kda.recurrent_step(x["q"], x["k"], x["v"], beta, x["z"], A, pool, gate=x["gate"], want_o=False, out=out)

    for _ in range(warmup):
        call()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        call()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    nbytes = n * H * (8 * D * D + 12 * D + 2)
    gbs = nbytes / (ms * 1e-3) / 1e9
    res = {"sequences": n, "heads": H, "d": D, "ms": ms, "token_heads_per_s": n * H / (ms * 1e-3),
           "algorithmic_bytes": nbytes, "achieved_GBs": gbs, "frac_hbm": gbs / HBM_PEAK_GBS, "launches": 1}
    # state export of the same pool (kda_state_io, KV layout): 4 D^2 bytes read and written per head-slot
    user = torch.empty_like(pool)
    for _ in range(warmup):
        kda.state_io(kda.STATE_EXPORT, pool, user)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        kda.state_io(kda.STATE_EXPORT, pool, user)
    stop.record()
    torch.cuda.synchronize()
    ms_io = start.elapsed_time(stop) / steps
    io_bytes = 2 * n * H * D * D * 4
    res["state_export"] = {"ms": ms_io, "algorithmic_bytes": io_bytes,
                           "achieved_GBs": io_bytes / (ms_io * 1e-3) / 1e9,
                           "frac_hbm": io_bytes / (ms_io * 1e-3) / 1e9 / HBM_PEAK_GBS}
    return res


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="k3_layer")
    ap.add_argument("--cpu-heads", type=int, default=0, help="heads in the CPU-baseline sample (0: all heads)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--schedule", choices=("auto", "fused", "overlapped", "pipelined", "segments"), default="auto",
                    help="the library's choice (default), the fused kernel, or a two-kernel schedule "
                         "(overlapped: two segments of records, double-buffered; pipelined: every record)")
    ap.add_argument("--segment-tokens", type=int, default=0,
                    help="tokens per segment of the two-kernel schedules; 0: library default")
    ap.add_argument("--decay", choices=("k3", "softplus"), default="k3",
                    help="decay map: K3's bounded map (the method), or Kimi Linear's softplus map (ablation)")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode-step side measurement")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prefill workload's side measurement (B4 T4096 H32)")
    ap.add_argument("--no-o-only", action="store_true", help="skip the side measurement without the output gate")
    ap.add_argument("--no-head-first", action="store_true",
                    help="skip the side measurement with the inputs and outputs head first ([B, H, T, d])")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the long-context workload's side measurement (B1 T1,048,576 H96, about a minute "
                         "of input generation)")
    ap.add_argument("--no-input-prep", action="store_true",
                    help="skip timing the input steps (ShortConv + Swish, Sigmoid) on the workload's shapes")
    ap.add_argument("--copy-calibration", type=float, default=0.0, metavar="GIB",
                    help="only run a plain device copy of GIB GiB (reference for HBM byte counters)")
    ap.add_argument("--peaks", action="store_true",
                    help="only measure what this GPU achieves against its published peaks: the library's state "
                         "copy over 24 GB, a plain torch device copy, and bf16 / fp32 GEMMs of torch (hipBLASLt)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(heads and sequence would shard as described in the design notes). Run with --gpus 1.",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import gated_delta_rule_84_amd as kda
    from synth.workloads import WORKLOADS

    wl = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration > 0:
        nbytes = int(args.copy_calibration * (1 << 30))
        a = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        b_ = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            b_.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": nbytes, "reads_per_copy": nbytes, "writes_per_copy": nbytes}))
        return 0
    if args.peaks:
        print(json.dumps(measure_peaks(kda)), flush=True)
        return 0
    kda.lib()

    t_gen = time.perf_counter()
    t = load_inputs(wl, dev)
    t_gen = time.perf_counter() - t_gen
    B, T, H, D = wl.B, wl.T, wl.H, wl.D
    token_heads = B * T * H
    odt = torch.bfloat16
    out = {"y": torch.empty((B, T, H, D), dtype=odt, device=dev),
           "S_T": torch.empty((B, H, D, D), dtype=torch.float32, device=dev)}
    fused = {"auto": None, "fused": True}.get(args.schedule, False)
    overlap = args.schedule in ("auto", "overlapped", "pipelined")
    seg_arg = args.segment_tokens or None
    desc = kda.make_desc(B, T, H, D, kda.KDA_BF16, kda.KDA_BF16, segment_tokens=seg_arg if overlap else 0,
                         overlap=overlap, fused=fused, decay=args.decay)
    if args.schedule == "overlapped":   # two segments of records: the double-buffered schedule
        ws_bytes = kda.workspace_size(desc, 2 * (seg_arg or 8192))
    elif args.schedule == "pipelined":  # every record of the call (also past the size query's cap)
        ws_bytes = kda.workspace_size(desc, T)
    elif overlap or fused or not seg_arg:
        ws_bytes = kda.workspace_size(desc)
    else:
        ws_bytes = kda.workspace_size(desc, seg_arg)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    seg, sched = kda.schedule(desc, ws_bytes)
    assert args.schedule == "auto" or sched == args.schedule or (
        args.schedule == "overlapped" and sched in ("segments", "pipelined")), sched
    # the kernel launches of one call, in the order the library brackets them with events
    names = kda.launches(desc, ws_bytes)

    def step(events=None):
        kda.chunk_fwd(t["q"], t["k"], t["v"], t["beta"], t["z"], t["A"], S0=t.get("S0"), gate=t["gate"],
                      want_o=False, out=out, workspace=ws, events=events, segment_tokens=seg_arg,
                      overlap=overlap, fused=fused, decay=args.decay)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # per-step kernel events (created by a first record, then re-recorded by the library)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * len(names))] for _ in range(args.steps)]
    for row in ev:
        for e in row:
            e.record()
    torch.cuda.synchronize()
    handles = [[e.cuda_event for e in row] for row in ev]
    # step boundaries on the caller's stream (each call joins the library's streams back into it)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]

    torch.cuda.synchronize()
    marks[0].record()
    for k in range(args.steps):
        step(events=handles[k])
        marks[k + 1].record()
    torch.cuda.synchronize()
    total_ms = marks[0].elapsed_time(marks[-1])
    ms = total_ms / args.steps
    step_ms = [marks[k].elapsed_time(marks[k + 1]) for k in range(args.steps)]
    # the timed outputs are checked outside the timed region
    status_ok = kda.call_status(desc, ws) == 0
    finite = all_finite(out["y"]) and all_finite(out["S_T"])

    per = {n: [] for n in set(names)}
    for row in ev:
        tot = {n: 0.0 for n in per}
        for i, n in enumerate(names):
            tot[n] += row[2 * i].elapsed_time(row[2 * i + 1])
        for n in per:
            per[n].append(tot[n])
    kern_ms = {n: float(np.mean(v)) for n, v in per.items()}  # per step, summed over its launches
    launches = {n: names.count(n) for n in per}
    dom = max(kern_ms, key=lambda n: kern_ms[n] / launches[n])  # longest average launch
    avg_launch_ms = kern_ms[dom] / launches[dom]
    path_bytes = token_heads * path_bytes_per_token_head(D) + 2 * B * H * D * D * 4
    # headline roofline: the path's algorithmic bytes of the token-heads one launch of
    # the dominant kernel processes (all of them for the pipelined schedule's single
    # scan launch) over that launch's average duration
    dom_path_bytes = path_bytes / launches[dom]
    achieved = dom_path_bytes / (avg_launch_ms * 1e-3) / 1e9
    # secondary: the kernel's own share of the path's bytes (its inputs and outputs)
    share_bytes = kernel_bytes(dom, token_heads, D, B * H, T)
    share_gbs = share_bytes / (kern_ms[dom] * 1e-3) / 1e9
    path_gbs = path_bytes / (ms * 1e-3) / 1e9
    path_tflops = token_heads * path_flops_per_token_head(D) / (ms * 1e-3) / 1e12

    result = {
        "metric": METRIC,
        "value": token_heads / (ms * 1e-3),
        "unit": "tokens·heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_median": float(np.median(step_ms)),
        "ms_min": float(np.min(step_ms)),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "baseline_note": "the source pages give no KDA throughput figure on stated hardware; none is invented",
        "dtype": "bf16",
        "data": "synthetic (seeded; K3 layer shapes, no trained weights)",
        "config": {"workload": wl.name, "B": B, "T": T, "H": H, "d_k": D, "d_v": D, "chunk": 64,
                   "inputs": "bf16", "layout": "[B, T, H, d] (token major)", "state": "fp32",
                   "outputs": "y (bf16) + S_T (fp32)", "gate": True,
                   "schedule": sched, "segment_tokens": seg, "decay": args.decay},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": profiled_traffic(dom, wl.name),
                     "algorithmic_bytes_per_launch": dom_path_bytes,
                     "launches_per_step": launches[dom], "avg_launch_ms": avg_launch_ms,
                     "kernel_share": {"algorithmic_bytes_per_launch": share_bytes / launches[dom],
                                      "achieved_GBs": share_gbs, "frac": share_gbs / HBM_PEAK_GBS}},
        "path_roofline": {"achieved_GBs": path_gbs, "frac_hbm": path_gbs / HBM_PEAK_GBS,
                          "achieved_TFLOPs": path_tflops, "frac_bf16_mfma": path_tflops / BF16_PEAK_TFLOPS,
                          "algorithmic_bytes": path_bytes},
        "counters": profiled_counters(wl.name),
        "kernel_ms": kern_ms,
        "checks": {"outputs_finite": finite, "library_status_ok": status_ok},
        "input_setup_s": t_gen,
    }
    if not args.no_o_only and T <= 65536:
        # the same forward without the output gate: o (bf16) and S_T out (skipped for
        # the long workloads, whose extra o buffer would not fit beside the records)
        out_o = {"o": torch.empty((B, T, H, D), dtype=odt, device=dev), "S_T": out["S_T"]}

        def step_o():
            kda.chunk_fwd(t["q"], t["k"], t["v"], t["beta"], t["z"], t["A"], S0=t.get("S0"), out=out_o,
                          workspace=ws, segment_tokens=seg_arg, overlap=overlap, fused=fused, decay=args.decay)

        ms_o, med_o, min_o = time_calls(step_o, args.steps, args.warmup)
        o_bytes = token_heads * (5 * 2 * D + 2) + 2 * B * H * D * D * 4  # q, k, z, v, beta in; o out; S0, S_T
        result["o_only"] = {"ms": ms_o, "ms_median": med_o, "ms_min": min_o,
                            "token_heads_per_s": token_heads / (ms_o * 1e-3),
                            "algorithmic_bytes": o_bytes, "achieved_GBs": o_bytes / (ms_o * 1e-3) / 1e9,
                            "frac_hbm": o_bytes / (ms_o * 1e-3) / 1e9 / HBM_PEAK_GBS}
        del out_o
    if not args.no_head_first and args.schedule == "auto" and wl.name == "k3_layer":
        result["head_first"] = time_head_first(kda, t, out, ws, B, T, H, D, args.steps, args.warmup)
    if not args.no_input_prep:
        result["input_prep"] = time_input_prep(kda, t, B, T, H, D, args.steps, args.warmup, wl.name)
    if not args.no_decode:
        result["decode"] = time_decode(kda, H, D, args.steps, args.warmup)
    if not args.no_prefill and wl.name != "prefill":
        result["prefill"] = time_prefill(kda, WORKLOADS["prefill"], args.steps, args.warmup)
    if not args.no_cpu_baseline:
        heads = args.cpu_heads or H
        y_host = out["y"][:, :, :min(heads, H)].float().cpu().numpy()  # the last timed step's output
        result["cpu_baseline"] = cpu_baseline(wl, min(heads, H), y_host)
    if not args.no_long and wl.name != "long_context":
        del t, out
        torch.cuda.empty_cache()
        result["long_context"] = time_long_context(kda, WORKLOADS["long_context"], min(args.steps, 5),
                                                   min(args.warmup, 2))
    print(json.dumps(result), flush=True)
    valid = finite and status_ok and result.get("cpu_baseline", {}).get("parity_ok", True)
    if not valid:
        print("bench: the timed outputs failed their checks (see 'checks' / 'cpu_baseline')", file=sys.stderr)
        return 3
    return 0


if __name__ == "__main__":
    sys.exit(main())
