"""GPU parity on small inputs: the HIP path (through the C ABI) against the
fp64 oracle, element by element on the same seeded inputs.

Tolerances (relative L2 over the whole checked tensor, fp64):
  fp32 inputs / fp32 outputs   <= 1e-5
  bf16 inputs / fp32 state     <= 3e-3
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import kda_ref as R
import synth
from synth.workloads import WORKLOADS, Workload, gen_inputs
from kda_gpu_util import dev, host64, log, rel_l2, widen

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_BF16 = 3e-3


@pytest.fixture(scope="module")
def kda():
    import gated_delta_rule_84_amd as m
    assert torch.cuda.is_available()
    m.lib()
    return m


def _run(kda, x, out_dtype=None, gate=True, S0=True, **kw):
    t = {n: dev(x[n]) for n in ("q", "k", "v", "beta", "z", "A")}
    g = dev(x["gate"]) if (gate and "gate" in x) else None
    s0 = dev(x["S0"]) if (S0 and "S0" in x) else None
    r = kda.chunk_fwd(t["q"], t["k"], t["v"], t["beta"], t["z"], t["A"], S0=s0, gate=g, out_dtype=out_dtype, **kw)
    torch.cuda.synchronize()
    return r


def _oracle(x, gate=True, S0=True):
    return oracle.forward_c(x["q"], x["k"], x["v"], x["beta"], x["z"], x["A"],
                            S0=x.get("S0") if S0 else None, gate=x.get("gate") if gate else None)


def test_tiny_fp32_workload(kda):
    """Workload 'tiny': B1 T128 H2 d64, fp32 path, o only."""
    wl = WORKLOADS["tiny"]
    x = gen_inputs(wl)
    log(f"[tiny] {wl}")
    r = _run(kda, x, gate=False)
    ref = R.kda_forward_heads(x["q"], x["k"], x["v"], x["beta"], x["z"], x["A"])
    e_o = rel_l2(host64(r["o"]), ref["o"])
    e_s = rel_l2(host64(r["S_T"]), ref["S_T"])
    log(f"[tiny] rel_l2 o={e_o:.3e} S_T={e_s:.3e}")
    assert e_o <= TOL_F32 and e_s <= TOL_F32


def _custom(B, T, H, D, dtype, seed, z_std=2.0, s0=0.1):
    return Workload("custom", 50 + seed, B=B, T=T, H=H, D=D, dtype=dtype, z_std=z_std, A_kind="uniform",
                    gate=True, s0_std=s0)


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("B,T,H,D", [(2, 200, 3, 128), (1, 64, 2, 128), (3, 77, 2, 64), (1, 1, 1, 128),
                                     (2, 333, 1, 64)])
def test_bf16_small_ragged(kda, B, T, H, D, fused):
    wl = _custom(B, T, H, D, "bf16", seed=B * 1000 + T)
    x = gen_inputs(wl)
    log(f"[bf16 small] B={B} T={T} H={H} D={D} fused={fused}")
    ref = _oracle(x)
    for odt in (torch.float32, torch.bfloat16):
        r = _run(kda, x, out_dtype=odt, fused=fused)
        e_o = rel_l2(host64(r["o"]), ref["o"])
        e_y = rel_l2(host64(r["y"]), ref["y"])
        e_s = rel_l2(host64(r["S_T"]), ref["S_T"])
        log(f"  out={odt} o={e_o:.3e} y={e_y:.3e} S_T={e_s:.3e}")
        assert e_o <= TOL_BF16 and e_y <= TOL_BF16 and e_s <= TOL_BF16


@pytest.mark.parametrize("B,T,H,D", [(2, 130, 2, 128), (1, 200, 3, 64)])
def test_fp32_small_ragged(kda, B, T, H, D):
    wl = _custom(B, T, H, D, "f32", seed=7 + T)
    x = gen_inputs(wl)
    log(f"[fp32 small] B={B} T={T} H={H} D={D}")
    ref = _oracle(x)
    r = _run(kda, x)
    for key in ("o", "y", "S_T"):
        e = rel_l2(host64(r[key]), ref[key])
        log(f"  {key}={e:.3e}")
        assert e <= TOL_F32, key


def test_outputs_fully_written_and_deterministic(kda):
    wl = _custom(2, 150, 2, 128, "bf16", seed=3)
    x = gen_inputs(wl)
    shp = (2, 150, 2, 128)
    outs = []
    for _ in range(2):
        pre = {"o": torch.full(shp, float("nan"), dtype=torch.bfloat16, device="cuda"),
               "y": torch.full(shp, float("nan"), dtype=torch.bfloat16, device="cuda"),
               "S_T": torch.full((2, 2, 128, 128), float("nan"), device="cuda")}
        r = _run(kda, x, out=pre)
        for key in ("o", "y", "S_T"):
            assert not torch.isnan(r[key]).any(), key
        outs.append({k: v.clone() for k, v in r.items()})
    for key in ("o", "y", "S_T"):
        assert torch.equal(outs[0][key].view(torch.int16) if outs[0][key].dtype == torch.bfloat16 else outs[0][key],
                           outs[1][key].view(torch.int16) if outs[1][key].dtype == torch.bfloat16 else outs[1][key])


def _bit_equal(a, b):
    if a.dtype == torch.bfloat16:
        a, b = a.view(torch.int16), b.view(torch.int16)
    return torch.equal(a, b)


def test_segmented_workspace_matches_single_pass(kda):
    """A workspace that only holds one chunk runs the sequence in 64-token
    segments (state carried through memory); results are bit-identical."""
    wl = _custom(2, 300, 2, 128, "bf16", seed=11)
    x = gen_inputs(wl)
    full = _run(kda, x, overlap=False, fused=False)
    small = _run(kda, x, overlap=False, segment_tokens=64, fused=False)
    for key in ("o", "y", "S_T"):
        assert _bit_equal(full[key], small[key]), key


@pytest.mark.parametrize("B,T,H,D,seg", [(2, 1000, 3, 128, 128), (1, 777, 2, 64, 256), (3, 300, 4, 128, 64)])
def test_overlapped_schedule_matches_one_stream(kda, B, T, H, D, seg):
    """The overlapped schedule (intra-chunk kernel of the next segment on one
    library stream while the scan of the current one runs on another, records
    double-buffered) gives bit-identical results to the one-stream schedule,
    including a ragged last segment and a state carried over many segments."""
    wl = _custom(B, T, H, D, "bf16", seed=B * 100 + T)
    x = gen_inputs(wl)
    log(f"[overlap] B={B} T={T} H={H} D={D} segment={seg}")
    # two segments of records (every record would select the pipelined schedule)
    desc = kda.make_desc(B, T, H, D, kda.KDA_BF16, kda.KDA_BF16, segment_tokens=seg, overlap=True, fused=False)
    ws = torch.empty(kda.workspace_size(desc, 2 * seg), dtype=torch.uint8, device="cuda")
    assert kda.schedule(desc, ws.numel())[1] == "overlapped"
    one = _run(kda, x, overlap=False, fused=False)
    two = _run(kda, x, overlap=True, segment_tokens=seg, fused=False, workspace=ws)
    for key in ("o", "y", "S_T"):
        assert _bit_equal(one[key], two[key]), key
    # work enqueued on the caller's stream after the call sees the finished
    # results (the call joins its streams back into the caller's stream)
    t = {n: dev(x[n]) for n in ("q", "k", "v", "beta", "z", "A", "gate", "S0")}
    torch.cuda.synchronize()
    r = kda.chunk_fwd(t["q"], t["k"], t["v"], t["beta"], t["z"], t["A"], S0=t["S0"], gate=t["gate"],
                      overlap=True, segment_tokens=seg, fused=False, workspace=ws)
    snap = {key: val.clone() for key, val in r.items()}  # on the current stream
    torch.cuda.current_stream().synchronize()
    for key in ("o", "y", "S_T"):
        assert _bit_equal(one[key], snap[key]), key


def test_overlapped_schedule_reuses_workspace(kda):
    """Many short segments (the scan of each waits inside the kernel for its
    records' counters) and three consecutive calls on different inputs with
    one workspace: every call equals the one-stream schedule bit for bit, so
    no counter of an earlier call lets a scan start early."""
    B, T, H, D, seg = 2, 2048, 4, 128, 64
    desc = kda.make_desc(B, T, H, D, kda.KDA_BF16, kda.KDA_BF16, segment_tokens=seg, overlap=True, fused=False)
    # two segments of records (every record would select the pipelined schedule)
    ws = torch.empty(kda.workspace_size(desc, 2 * seg), dtype=torch.uint8, device="cuda")
    assert kda.schedule(desc, ws.numel())[1] == "overlapped"
    outs = []
    for seed in (1, 2, 3):
        x = gen_inputs(_custom(B, T, H, D, "bf16", seed=700 + seed))
        log(f"[overlap reuse] seed={seed} segments={T // seg}")
        t = {n: dev(x[n]) for n in ("q", "k", "v", "beta", "z", "A", "gate", "S0")}
        r = kda.chunk_fwd(t["q"], t["k"], t["v"], t["beta"], t["z"], t["A"], S0=t["S0"], gate=t["gate"],
                          overlap=True, segment_tokens=seg, fused=False, workspace=ws)
        outs.append((x, r))
    torch.cuda.synchronize()
    for x, r in outs:
        one = _run(kda, x, overlap=False, fused=False)
        for key in ("o", "y", "S_T"):
            assert _bit_equal(one[key], r[key]), key


@pytest.mark.parametrize("B,T,H,D,seg,opts", [
    (1, 9000, 4, 128, 0, {}),                                   # default: 71 segments of 2 chunks (the last 1)
    (2, 3000, 3, 128, 256, {}),                                 # ragged last chunk, 4-chunk steady segments
    (1, 2065, 2, 64, 64, {"out_dtype": torch.float32}),         # d = 64, 33 one-chunk segments, fp32 outputs
    (3, 1100, 2, 128, 128, {"gate": False}),                    # o only; 18 chunks in 2-chunk segments
    (2, 1300, 3, 128, 192, {"S0": False}),                      # zero initial state, 3-chunk segments
    (1, 2000, 2, 128, 128, {"want_state": False}),              # no S_T: the scan ends in the workspace
])
def test_pipelined_schedule_matches_one_stream(kda, B, T, H, D, seg, opts):
    """The pipelined schedule (every chunk record in the workspace, ONE
    intra-chunk launch on one library stream beside ONE scan launch over the
    sequence that waits inside the kernel for each segment's record counters,
    producers paced by the scan's progress) gives bit-identical results to
    the one-stream schedule; the launch-order query matches what the call
    does (the intra-chunk launch, then the scan: should the library's two
    streams share a hardware queue, the scan then finds every record
    written)."""
    wl = _custom(B, T, H, D, "bf16", seed=B * 1000 + T)
    x = gen_inputs(wl)
    desc = kda.make_desc(B, T, H, D, kda.KDA_BF16, kda.KDA_BF16, segment_tokens=seg, overlap=True, fused=False)
    nbytes = kda.workspace_size(desc)
    assert kda.schedule(desc, nbytes)[1] == "pipelined"
    order = kda.launches(desc, nbytes)
    # the one intra-chunk launch first, then the one scan launch
    assert order == ["intra", "scan"]
    log(f"[pipelined] B={B} T={T} H={H} D={D} segment={seg} launches={len(order)}")
    one = _run(kda, x, overlap=False, fused=False, **opts)
    pip = _run(kda, x, overlap=True, segment_tokens=seg, fused=False, **opts)
    keys = [k for k in ("o", "y", "S_T") if k in one]
    assert keys and all(k in pip for k in keys)
    for key in keys:
        assert _bit_equal(one[key], pip[key]), key


def test_pipelined_one_chunk_segments(kda):
    """201 chunks (ragged) counted in 201 one-chunk segments (a record wait
    at every chunk step, pacing lead of 7 chunks) by the one intra-chunk
    launch: the results still equal the one-stream schedule bit for bit."""
    B, T, H, D, seg = 1, 64 * 201 - 30, 2, 64, 64
    x = gen_inputs(_custom(B, T, H, D, "bf16", seed=4201))
    desc = kda.make_desc(B, T, H, D, kda.KDA_BF16, kda.KDA_BF16, segment_tokens=seg, overlap=True, fused=False)
    nbytes = kda.workspace_size(desc)
    order = kda.launches(desc, nbytes)
    assert kda.schedule(desc, nbytes) == (64, "pipelined") and order == ["intra", "scan"], order
    log(f"[pipelined one-chunk segments] T={T} launches={len(order)}")
    one = _run(kda, x, overlap=False, fused=False)
    pip = _run(kda, x, overlap=True, segment_tokens=seg, fused=False)
    for key in ("o", "y", "S_T"):
        assert _bit_equal(one[key], pip[key]), key


def test_pipelined_schedule_reuses_workspace_and_traces(kda):
    """Three consecutive pipelined calls on different inputs with one
    workspace (counters re-zeroed by each call; 32 one-chunk segments) each
    equal the one-stream schedule bit for bit; events bracket every launch in
    the reported order."""
    B, T, H, D, seg = 2, 2048, 4, 128, 64
    desc = kda.make_desc(B, T, H, D, kda.KDA_BF16, kda.KDA_BF16, segment_tokens=seg, overlap=True, fused=False)
    ws = torch.empty(kda.workspace_size(desc), dtype=torch.uint8, device="cuda")
    assert kda.schedule(desc, ws.numel())[1] == "pipelined"
    order = kda.launches(desc, ws.numel())
    assert order == ["intra", "scan"]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * len(order))]
    for e in ev:
        e.record()
    torch.cuda.synchronize()
    outs = []
    for seed in (1, 2, 3):
        x = gen_inputs(_custom(B, T, H, D, "bf16", seed=900 + seed))
        log(f"[pipelined reuse] seed={seed}")
        t = {n: dev(x[n]) for n in ("q", "k", "v", "beta", "z", "A", "gate", "S0")}
        r = kda.chunk_fwd(t["q"], t["k"], t["v"], t["beta"], t["z"], t["A"], S0=t["S0"], gate=t["gate"],
                          overlap=True, segment_tokens=seg, fused=False, workspace=ws,
                          events=[e.cuda_event for e in ev] if seed == 3 else None)
        outs.append((x, r))
    torch.cuda.synchronize()
    ms = [ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(len(order))]
    assert all(m >= 0.0 for m in ms) and ms[-1] > 0.0
    for x, r in outs:
        one = _run(kda, x, overlap=False, fused=False)
        for key in ("o", "y", "S_T"):
            assert _bit_equal(one[key], r[key]), key


@pytest.mark.parametrize("B,T,H,D,opts", [
    (2, 1000, 3, 128, {}),
    (1, 777, 2, 64, {}),
    (3, 130, 2, 128, {"out_dtype": torch.float32}),
    (2, 64, 4, 128, {"S0": False}),
    (1, 65, 2, 64, {"gate": False}),
    (2, 300, 2, 128, {"rms_w": True}),
    (1, 200, 3, 128, {"want_o": False}),
    (2, 129, 2, 64, {"want_state": False, "out_dtype": torch.float32}),
])
def test_fused_matches_two_kernel_schedules(kda, B, T, H, D, opts):
    """The fused kernel (records built in LDS by producer waves) and the
    two-kernel schedules run the same arithmetic: bit-identical o, y, S_T."""
    wl = _custom(B, T, H, D, "bf16", seed=7 * B + T + H)
    x = gen_inputs(wl)
    opts = dict(opts)
    log(f"[fused] B={B} T={T} H={H} D={D} {opts}")
    if opts.pop("rms_w", False):
        opts["rms_w"] = torch.linspace(0.5, 1.5, H * D, device="cuda").reshape(H, D)
    gate = opts.pop("gate", True)
    S0 = opts.pop("S0", True)
    ref = _run(kda, x, gate=gate, S0=S0, fused=False, overlap=False, **opts)
    fus = _run(kda, x, gate=gate, S0=S0, fused=True, **opts)
    assert set(ref) == set(fus)
    for key in ref:
        assert _bit_equal(ref[key], fus[key]), key
    _, sched = kda.schedule(kda.make_desc(B, T, H, D, kda.KDA_BF16, kda.KDA_BF16, fused=True), 0)
    assert sched == "fused"
    # left to the library, a two-kernel schedule is taken
    desc = kda.make_desc(B, T, H, D, kda.KDA_BF16, kda.KDA_BF16)
    assert kda.schedule(desc, kda.workspace_size(desc))[1] != "fused"


def test_state_only_and_zero_length(kda):
    wl = _custom(1, 100, 2, 64, "bf16", seed=5)
    x = gen_inputs(wl)
    ref = _oracle(x)
    r = _run(kda, x, gate=False, want_o=False)
    assert set(r) == {"S_T"}
    assert rel_l2(host64(r["S_T"]), ref["S_T"]) <= TOL_BF16
    x0 = gen_inputs(_custom(1, 0, 2, 64, "bf16", seed=6))
    r0 = _run(kda, x0, gate=False)
    assert torch.equal(r0["S_T"], dev(x0["S0"]))


def test_prepass_decay_and_subtile_bound(kda):
    """Pre-pass G against the fp64 chunk-local cumulative sum of the decay map;
    every aligned 16-token sub-tile's log-decay lies in [-80, 0] in fp32,
    reaching -80 exactly on the pinned heads of the k3_layer workload."""
    wl = WORKLOADS["k3_layer"]
    x = gen_inputs(wl, time=(0, 256), heads=(40, 16))
    q, k, z = dev(x["q"]), dev(x["k"]), dev(x["z"])
    A = dev(x["A"])
    G, rq, rk = kda.prepass(q, k, z, A)
    torch.cuda.synchronize()
    Gh = host64(G)[0]  # [T, H, D]
    g = R.decay_log(widen(x["z"])[0], x["A"][None, :, None])
    Gref = np.cumsum(g.reshape(4, 64, 16, 128), axis=1).reshape(256, 16, 128)
    assert np.abs(Gh - Gref).max() <= 2e-4
    # sub-tile sums: G at the end of each sub-tile minus G at the end of the previous
    Gc = Gh.reshape(4, 4, 16, 16, 128)
    ends = Gc[:, :, 15]
    starts = np.concatenate([np.zeros((4, 1, 16, 128)), Gc[:, :-1, 15]], axis=1)
    sub = ends - starts
    assert sub.max() <= 0.0 and sub.min() >= -80.0
    assert sub[:, :, 8:].min() == -80.0  # heads 48.. are pinned at g_min
    qn = np.linalg.norm(widen(x["q"]).astype(np.float64), axis=-1)
    np.testing.assert_allclose(host64(rq)[0], 1 / np.sqrt(qn[0] ** 2 + 1e-6), rtol=1e-5)
    kn = np.linalg.norm(widen(x["k"]).astype(np.float64), axis=-1)
    np.testing.assert_allclose(host64(rk)[0], 1 / np.sqrt(kn[0] ** 2 + 1e-6), rtol=1e-5)


@pytest.mark.parametrize("D,dtype", [(128, "bf16"), (64, "f32"), (128, "f32")])
def test_decode_steps_match_oracle(kda, D, dtype):
    n, H, steps = 6, 3, 5
    wl = _custom(n, steps, H, D, dtype, seed=21 + D)
    x = gen_inputs(wl)
    log(f"[decode] D={D} dtype={dtype}")
    ref = _oracle(x)
    pool = torch.zeros((n + 3, H, D, D), device="cuda")
    slot = torch.tensor([3, 0, 5, 1, 8, 2], dtype=torch.int32, device="cuda")
    kda.state_io(kda.STATE_IMPORT, pool, user=dev(x["S0"]), slot=slot)
    ys, os_ = [], []
    for t in range(steps):
        step = {nm: dev(np.ascontiguousarray(x[nm][:, t])) for nm in ("q", "k", "v", "beta", "z", "gate")}
        r = kda.recurrent_step(step["q"], step["k"], step["v"], step["beta"], step["z"], dev(x["A"]), pool,
                               slot=slot, gate=step["gate"], out_dtype=torch.float32)
        os_.append(host64(r["o"]))
        ys.append(host64(r["y"]))
    torch.cuda.synchronize()
    o = np.stack(os_, axis=1)
    y = np.stack(ys, axis=1)
    ST = torch.empty((n, H, D, D), device="cuda")
    kda.state_io(kda.STATE_EXPORT, pool, user=ST, slot=slot)
    torch.cuda.synchronize()
    tol = TOL_F32 if dtype == "f32" else 1e-5  # fp32 state and fp32 math on both paths
    for name, a, b in (("o", o, ref["o"]), ("y", y, ref["y"]), ("S", host64(ST), ref["S_T"])):
        e = rel_l2(a, b)
        log(f"  {name}={e:.3e}")
        assert e <= tol, name


def test_state_io_layouts(kda):
    H, D = 2, 64
    user = torch.randn((3, H, D, D), device="cuda")
    pool = torch.full((5, H, D, D), 7.0, device="cuda")
    slot = torch.tensor([4, 0, 2], dtype=torch.int32, device="cuda")
    kda.state_io(kda.STATE_IMPORT, pool, user=user, slot=slot)
    out_t = torch.empty_like(user)
    kda.state_io(kda.STATE_EXPORT, pool, user=out_t, slot=slot, layout=kda.LAYOUT_VK)
    kda.state_io(kda.STATE_ZERO, pool, slot=slot[:1], n=1)
    torch.cuda.synchronize()
    assert torch.equal(pool[0], user[1]) and torch.equal(pool[2], user[2])
    assert torch.equal(out_t, user.transpose(-1, -2))
    assert torch.count_nonzero(pool[4]) == 0
    assert torch.all(pool[1] == 7.0) and torch.all(pool[3] == 7.0)


@pytest.mark.parametrize("D", [64, 128])
def test_state_io_vector_and_element_paths(kda, D):
    """Same-layout import / export / zero: 16-byte vectors when both pointers
    are 16-byte aligned, element by element when one is only 4-byte aligned
    (buffers offset by one float); both give exact copies."""
    H = 3
    user = torch.randn((4, H, D, D), device="cuda")
    pool = torch.randn((6, H, D, D), device="cuda")
    keep = pool.clone()
    slot = torch.tensor([5, 1, 3, 0], dtype=torch.int32, device="cuda")

    def offset(shape):  # a view whose data pointer is 4 bytes past a 256-byte boundary
        flat = torch.empty(int(np.prod(shape)) + 1, device="cuda")
        return flat[1:].view(shape)

    kda.state_io(kda.STATE_IMPORT, pool, user=user, slot=slot)
    out = torch.empty_like(user)
    kda.state_io(kda.STATE_EXPORT, pool, user=out, slot=slot)
    p1, u1, out1 = offset(pool.shape), offset(user.shape), offset(user.shape)
    assert p1.data_ptr() % 16 == 4
    p1.copy_(keep)
    u1.copy_(user * 2)
    kda.state_io(kda.STATE_IMPORT, p1, user=u1, slot=slot)
    kda.state_io(kda.STATE_EXPORT, p1, user=out1, slot=slot)
    kda.state_io(kda.STATE_ZERO, p1, slot=slot[:2], n=2)
    kda.state_io(kda.STATE_ZERO, pool, slot=slot[2:], n=2)
    torch.cuda.synchronize()
    assert torch.equal(out, user) and torch.equal(out1, user * 2)
    for i, r in enumerate(slot.tolist()):
        assert torch.equal(pool[r], torch.zeros_like(pool[r]) if i >= 2 else user[i])
        assert torch.equal(p1[r], torch.zeros_like(p1[r]) if i < 2 else user[i] * 2)
    for r in (2, 4):  # rows no slot names are untouched
        assert torch.equal(pool[r], keep[r]) and torch.equal(p1[r], keep[r])


def test_fused_with_heads_filling_the_device(kda):
    """B * H at the CU count: left to the library a two-kernel schedule is
    taken; the forced fused kernel gives the same results bit for bit."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    B, T, H, D = 2, 130, (cus + 1) // 2, 64
    desc = kda.make_desc(B, T, H, D, kda.KDA_BF16, kda.KDA_BF16)
    assert kda.schedule(desc, kda.workspace_size(desc))[1] != "fused"
    x = gen_inputs(_custom(B, T, H, D, "bf16", seed=4))
    auto = _run(kda, x, fused=True)
    ref = _run(kda, x, fused=False, overlap=False)
    for key in ("o", "y", "S_T"):
        assert _bit_equal(auto[key], ref[key]), key


@pytest.mark.parametrize("B,T,H,opts", [
    (4, 4096, 32, {}),                                           # the prefill workload's shape: 256 workgroups
    (1, 1000, 3, {}),                                            # ragged last chunk, 6 workgroups (a partial group of 16)
    (2, 700, 5, {"out_dtype": torch.float32, "rms_w": True}),    # fp32 outputs, RMSNorm weight
    (1, 640, 2, {"gate": False}),                                # o and S_T only: no row-sum exchange
    (3, 512, 2, {"S0": False, "want_o": False}),                 # zero initial state, y and S_T only
    (1, 2048, 4, {"snapshot_chunks": 8}),                        # prefix-cache snapshots from both halves
])
def test_split_scan_matches_unsplit(kda, monkeypatch, B, T, H, opts):
    """One-stream calls with 2 B H within the device's compute units split
    each head's value columns between two scan workgroups that exchange their
    RMSNorm row sums; the result equals the unsplit scan workgroup's bit for
    bit (o, y, S_T, snapshots) and the fp64 oracle within 3e-3."""
    D = 128
    x = gen_inputs(_custom(B, T, H, D, "bf16", seed=5000 + B * T + H))
    opts = dict(opts)
    kw = {"overlap": False, "fused": False}
    if opts.pop("rms_w", False):
        w = torch.from_numpy(np.random.default_rng(7).uniform(0.5, 1.5, (H, D)).astype(np.float32)).cuda()
        kw["rms_w"] = w
    for k_ in ("out_dtype", "want_o", "snapshot_chunks"):
        if k_ in opts:
            kw[k_] = opts.pop(k_)
    log(f"[split] B={B} T={T} H={H} {sorted(kw)}")
    split = _run(kda, x, **opts, **kw)
    monkeypatch.setenv("KDA_TEST_NO_SPLIT", "1")
    whole = _run(kda, x, **opts, **kw)
    monkeypatch.delenv("KDA_TEST_NO_SPLIT")
    keys = [k_ for k_ in ("o", "y", "S_T", "snapshots") if k_ in whole]
    assert keys and all(k_ in split for k_ in keys)
    for key in keys:
        assert _bit_equal(split[key], whole[key]), key
    if "rms_w" not in kw and kw.get("snapshot_chunks", 0) == 0:
        ref = _oracle(x, gate=opts.get("gate", True), S0=opts.get("S0", True))
        for key in keys:
            e = rel_l2(host64(split[key]), ref[key])
            log(f"[split] {key} rel_l2={e:.3e}")
            assert e <= TOL_BF16, key


@pytest.mark.parametrize("B,T,H,D,windows", [
    (1, 625 * 64 - 20, 3, 128, 2),        # 512 + 113 chunks, the last window short and ragged
    (1, 4 * 512 * 64 + 1000, 1, 64, 5),   # four full windows and one of 16 chunks, d = 64
])
def test_pipelined_windows_match_one_stream(kda, B, T, H, D, windows):
    """A workspace that holds 512 chunks of records but not all of them: the
    pipelined schedule runs in windows of 512 chunks (per window one
    intra-chunk launch and one scan launch, the state carried across, a
    window's producers waiting for the previous window's scan), bit-identical
    to the one-stream schedule (outputs and prefix-cache snapshots) and within
    3e-3 of the oracle."""
    x = gen_inputs(_custom(B, T, H, D, "bf16", seed=7000 + T + H))
    desc = kda.make_desc(B, T, H, D, kda.KDA_BF16, kda.KDA_BF16, overlap=True, fused=False)
    nbytes = kda.workspace_size(desc, 512 * 64)
    assert kda.schedule(desc, nbytes)[1] == "pipelined"
    assert kda.launches(desc, nbytes) == ["intra", "scan"] * windows
    log(f"[pipelined windows] B={B} T={T} H={H} D={D} windows={windows}")
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    pip = _run(kda, x, overlap=True, fused=False, workspace=ws, snapshot_chunks=100)
    assert kda.call_status(desc, ws) == 0
    one = _run(kda, x, overlap=False, fused=False, snapshot_chunks=100)
    for key in ("o", "y", "S_T", "snapshots"):  # snapshots every 100 chunks, across the windows
        assert _bit_equal(one[key], pip[key]), key
    ref = _oracle(x)
    for key in ("o", "y", "S_T"):
        e = rel_l2(host64(pip[key]), ref[key])
        log(f"[pipelined windows] {key} rel_l2={e:.3e}")
        assert e <= TOL_BF16, key
