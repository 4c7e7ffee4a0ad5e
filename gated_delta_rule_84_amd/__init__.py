"""Python binding of libkda (MI355X / gfx950 Kimi Delta Attention).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI of ``include/kda.h``.  PyTorch provides device memory
and the current HIP stream.  There is no fallback path: if ``libkda.so`` has
not been built, every call raises.
"""
from __future__ import annotations

import atexit
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "kda.h")

KDA_F32, KDA_BF16 = 0, 1
STATE_ZERO, STATE_IMPORT, STATE_EXPORT = 0, 1, 2
LAYOUT_KV, LAYOUT_VK = 0, 1
STATUS = {0: "KDA_OK", 1: "KDA_ERR_NULL_ARG", 2: "KDA_ERR_BAD_SHAPE", 3: "KDA_ERR_BAD_DTYPE",
          4: "KDA_ERR_MISALIGNED", 5: "KDA_ERR_UNSUPPORTED", 6: "KDA_ERR_WORKSPACE", 7: "KDA_ERR_HIP",
          8: "KDA_ERR_TIMEOUT"}


class KdaDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("g_min", ctypes.c_float), ("q_scale", ctypes.c_float), ("l2_eps", ctypes.c_float),
                ("rms_eps", ctypes.c_float), ("qk_l2norm", ctypes.c_int32),
                ("in_dtype", ctypes.c_int), ("out_dtype", ctypes.c_int),
                ("segment_tokens", ctypes.c_int32), ("overlap", ctypes.c_int32), ("fused", ctypes.c_int32),
                ("decay", ctypes.c_int), ("tokens", ctypes.c_int)]


ABI_VERSION = 6  # KDA_ABI_VERSION of include/kda.h that KdaDesc mirrors


DECAYS = {"k3": 0, "softplus": 1}


class KdaError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {STATUS.get(code, code)}")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    """Load libkda.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python __graft_entry__.py` "
                               "(no CPU fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
        dp = ctypes.POINTER(KdaDesc)
        L.kda_abi_version.restype = ctypes.c_int
        if L.kda_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} has ABI version {L.kda_abi_version()}, this binding expects "
                               f"{ABI_VERSION}: rebuild it with `python __graft_entry__.py`")
        L.kda_status_str.restype = ctypes.c_char_p
        L.kda_status_str.argtypes = [ctypes.c_int]
        L.kda_desc_init.restype = ctypes.c_int
        L.kda_desc_init.argtypes = [dp, i32, i32, i32, i32, ctypes.c_int, ctypes.c_int]
        L.kda_chunk_fwd_workspace_size.restype = sz
        L.kda_chunk_fwd_workspace_size.argtypes = [dp]
        L.kda_chunk_fwd_workspace_size_for.restype = sz
        L.kda_chunk_fwd_workspace_size_for.argtypes = [dp, i32]
        L.kda_chunk_fwd_snapshots.restype = ctypes.c_int
        L.kda_chunk_fwd_snapshots.argtypes = [dp] + [vp] * 13 + [i32, vp, sz, vp]
        L.kda_chunk_fwd_kcp.restype = ctypes.c_int
        L.kda_chunk_fwd_kcp.argtypes = [dp, i32] + [vp] * 13 + [sz, vp]
        L.kda_chunk_fwd_kcp_workspace_size.restype = sz
        L.kda_chunk_fwd_kcp_workspace_size.argtypes = [dp, i32]
        L.kda_input_prep.restype = ctypes.c_int
        L.kda_input_prep.argtypes = [dp, i32] + [vp] * 14
        L.kda_snapshot_count.restype = i32
        L.kda_snapshot_count.argtypes = [dp, i32]
        L.kda_release_resources.restype = ctypes.c_int
        L.kda_release_resources.argtypes = []
        L.kda_chunk_fwd_schedule.restype = ctypes.c_int
        L.kda_chunk_fwd_schedule.argtypes = [dp, sz, ctypes.POINTER(i32), ctypes.POINTER(i32)]
        L.kda_chunk_fwd_launches.restype = ctypes.c_int
        L.kda_chunk_fwd_launches.argtypes = [dp, sz, ctypes.POINTER(i32), i32, ctypes.POINTER(i32)]
        L.kda_chunk_fwd.restype = ctypes.c_int
        L.kda_chunk_fwd.argtypes = [dp] + [vp] * 13 + [sz, vp]
        L.kda_chunk_fwd_status.restype = ctypes.c_int
        L.kda_chunk_fwd_status.argtypes = [dp, vp, sz, vp]
        L.kda_chunk_fwd_noalloc.restype = ctypes.c_int
        L.kda_chunk_fwd_noalloc.argtypes = [dp] + [vp] * 13
        L.kda_chunk_fwd_traced.restype = ctypes.c_int
        L.kda_chunk_fwd_traced.argtypes = [dp] + [vp] * 13 + [sz, vp, ctypes.POINTER(vp), i32]
        L.kda_recurrent_step.restype = ctypes.c_int
        L.kda_recurrent_step.argtypes = [dp] + [vp] * 7 + [i32] + [vp] * 7
        L.kda_state_io.restype = ctypes.c_int
        L.kda_state_io.argtypes = [ctypes.c_int, i32, i32, i32, i32, ctypes.c_int, vp, i32, vp, vp, vp, vp]
        L.kda_prepass.restype = ctypes.c_int
        L.kda_prepass.argtypes = [dp] + [vp] * 7 + [vp]
        _lib = L
        atexit.register(release_resources)
    return _lib


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _expect(name, t, shape, dtype=None):
    """A tensor argument's shape (and element type); None passes."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _check_forward_args(q, k, v, beta, z, A, S0, gate, rms_w, out, head_first):
    """Shapes and element types of a forward call's tensors (the C ABI sees
    only pointers, so a mismatch here would make the kernels read or write
    past a tensor).  Returns (B, T, H, D)."""
    if q.dim() != 4:
        raise ValueError(f"q must be 4-D ({'[B, H, T, D]' if head_first else '[B, T, H, D]'}), got {tuple(q.shape)}")
    if head_first:
        B, H, T, D = q.shape
        tok, per_tok = (B, H, T, D), (B, H, T)
    else:
        B, T, H, D = q.shape
        tok, per_tok = (B, T, H, D), (B, T, H)

    expect = _expect

    for name, t in (("k", k), ("v", v), ("z", z), ("gate", gate)):
        expect(name, t, tok, q.dtype)
    expect("beta", beta, per_tok, q.dtype)
    expect("A", A, (H,), torch.float32)
    expect("S0", S0, (B, H, D, D), torch.float32)
    expect("rms_w", rms_w, (H, D), torch.float32)
    for name in ("o", "y"):
        if out and out.get(name) is not None and tuple(out[name].shape) != tok:
            raise ValueError(f"out['{name}'] has shape {tuple(out[name].shape)}, expected {tok}")
    if out and out.get("S_T") is not None:
        expect("out['S_T']", out["S_T"], (B, H, D, D), torch.float32)
    return B, T, H, D


def make_desc(B, T, H, D, in_dtype, out_dtype, g_min=-5.0, q_scale=1.0, l2_eps=1e-6, rms_eps=1e-6,
              qk_l2norm=True, segment_tokens=0, overlap=True, fused=None, decay="k3", head_first=False) -> KdaDesc:
    d = KdaDesc()
    rc = lib().kda_desc_init(ctypes.byref(d), B, T, H, D, in_dtype, out_dtype)
    if rc != 0:
        raise KdaError("kda_desc_init", rc)
    d.g_min, d.q_scale, d.l2_eps, d.rms_eps, d.qk_l2norm = g_min, q_scale, l2_eps, rms_eps, int(bool(qk_l2norm))
    d.segment_tokens, d.overlap = int(segment_tokens or 0), int(bool(overlap))
    d.fused = 1 if fused is None else (2 if fused else 0)  # None: the library decides
    d.decay = DECAYS[decay]
    d.tokens = 1 if head_first else 0  # KDA_TOKENS_BHTD / KDA_TOKENS_BTHD
    return d


def workspace_size(desc: KdaDesc, segment_tokens: int | None = None) -> int:
    """Workspace bytes: the descriptor's preferred schedule (None), or one
    segment of ``segment_tokens`` tokens processed in turn."""
    if segment_tokens is None:
        return int(lib().kda_chunk_fwd_workspace_size(ctypes.byref(desc)))
    return int(lib().kda_chunk_fwd_workspace_size_for(ctypes.byref(desc), int(segment_tokens)))


def release_resources() -> None:
    """Synchronise and destroy the library's own streams and events (the
    two-stream schedules create them again when needed).  Registered to run at
    interpreter exit, while the HIP runtime is still up."""
    if _lib is not None:
        _lib.kda_release_resources()


SCHEDULES = {0: "segments", 1: "overlapped", 2: "fused", 3: "pipelined"}
LAUNCH_KINDS = {0: "intra", 1: "scan", 2: "fused"}


def call_status(desc: KdaDesc, workspace) -> int:
    """kda_chunk_fwd_status: waits for the current stream, then 0 (KDA_OK) or
    8 (KDA_ERR_TIMEOUT: the last call through `workspace` had an in-kernel
    wait for chunk records give up, so its outputs are invalid)."""
    return int(lib().kda_chunk_fwd_status(ctypes.byref(desc), _ptr(workspace), workspace.numel(),
                                          _stream(workspace.device)))


def schedule(desc: KdaDesc, ws_bytes: int) -> tuple[int, str]:
    """(tokens per segment, schedule name) that kda_chunk_fwd uses on the
    current device for this descriptor and workspace size."""
    seg, sch = ctypes.c_int32(0), ctypes.c_int32(0)
    rc = lib().kda_chunk_fwd_schedule(ctypes.byref(desc), int(ws_bytes), ctypes.byref(seg), ctypes.byref(sch))
    if rc != 0:
        raise KdaError("kda_chunk_fwd_schedule", rc)
    return int(seg.value), SCHEDULES[int(sch.value)]


def launches(desc: KdaDesc, ws_bytes: int) -> list[str]:
    """Kinds of the kernel launches ('intra', 'scan', 'fused'), in the order
    that chunk_fwd(..., events=...) brackets them, for this descriptor and
    workspace size on the current device."""
    n = ctypes.c_int32(0)
    rc = lib().kda_chunk_fwd_launches(ctypes.byref(desc), int(ws_bytes), None, 0, ctypes.byref(n))
    if rc != 0:
        raise KdaError("kda_chunk_fwd_launches", rc)
    kinds = (ctypes.c_int32 * max(n.value, 1))()
    rc = lib().kda_chunk_fwd_launches(ctypes.byref(desc), int(ws_bytes), kinds, n.value, ctypes.byref(n))
    if rc != 0:
        raise KdaError("kda_chunk_fwd_launches", rc)
    return [LAUNCH_KINDS[int(kinds[i])] for i in range(n.value)]


def chunk_fwd(q, k, v, beta, z, A, S0=None, gate=None, rms_w=None, *, out_dtype=None, want_o=True,
              want_y=None, want_state=True, workspace=None, segment_tokens=None, overlap=True, fused=None,
              out=None, events=None, snapshot_chunks=0, kcp_parts=0, head_first=False, **opts):
    """KDA forward over whole sequences.  q, k, z: [B, T, H, D]; v (and gate):
    [B, T, H, D]; beta: [B, T, H]; A: [H] fp32; S0: [B, H, D, D] fp32 or None.
    Returns a dict with 'o' / 'y' (out_dtype, default the input dtype) and
    'S_T' (fp32).  ``out`` may supply preallocated output tensors; ``events``
    (raw hipEvent_t handles) selects the traced entry point.  With
    ``fused`` True (bf16 inputs) one fused kernel runs the whole forward (None:
    the library's choice, currently the two-kernel schedules); otherwise, with
    ``overlap`` the library may run the pipelined schedule (records counted in
    segments of ``segment_tokens`` tokens, default 128) or the overlapped one
    (segments of ``segment_tokens``, default 8192), as the workspace allows;
    without it, ``segment_tokens`` sizes the segments processed in turn on
    one stream (default: as many as the workspace holds).  With
    ``snapshot_chunks`` = N > 0 the result also holds 'snapshots'
    [B, n, H, D, D]: the state after every N-th chunk (prefix-cache resume
    points, n = T // (64 N)).  With ``kcp_parts`` = P > 1 the sequence runs as P
    parallel segments folded through their (M, S~) pairs (kda_chunk_fwd_kcp).
    With ``head_first`` the per-token tensors are [B, H, T, D] (beta
    [B, H, T]) and o, y come out the same way."""
    B, T, H, D = _check_forward_args(q, k, v, beta, z, A, S0, gate, rms_w, out, head_first)
    tok_shape = (B, H, T, D) if head_first else (B, T, H, D)
    in_dt = _dt(q)
    odt = q.dtype if out_dtype is None else out_dtype
    desc = make_desc(B, T, H, D, in_dt, _dt(torch.empty(0, dtype=odt)),
                     segment_tokens=(segment_tokens or 0) if overlap else 0, overlap=overlap, fused=fused,
                     head_first=head_first, **opts)
    want_y = (gate is not None) if want_y is None else want_y
    res = dict(out or {})
    dev = q.device
    if want_o and "o" not in res:
        res["o"] = torch.empty(tok_shape, dtype=odt, device=dev)
    if want_y and "y" not in res:
        res["y"] = torch.empty(tok_shape, dtype=odt, device=dev)
    if want_state and "S_T" not in res:
        res["S_T"] = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    if workspace is None:
        nbytes = workspace_size(desc, None if overlap else segment_tokens)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    if kcp_parts and kcp_parts > 1:
        nb = int(lib().kda_chunk_fwd_kcp_workspace_size(ctypes.byref(desc), int(kcp_parts)))
        if nb == 0:
            raise KdaError("kda_chunk_fwd_kcp_workspace_size", 5)
        kws = torch.empty(nb, dtype=torch.uint8, device=dev)
        rc = lib().kda_chunk_fwd_kcp(
            ctypes.byref(desc), int(kcp_parts), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(z), _ptr(A), _ptr(S0),
            _ptr(gate), _ptr(rms_w), _ptr(res.get("o")), _ptr(res.get("y")), _ptr(res.get("S_T")), _ptr(kws),
            kws.numel(), _stream(dev))
        if rc != 0:
            raise KdaError("kda_chunk_fwd_kcp", rc)
        return res
    if snapshot_chunks:
        n = int(lib().kda_snapshot_count(ctypes.byref(desc), int(snapshot_chunks)))
        if "snapshots" not in res:
            res["snapshots"] = torch.empty((B, n, H, D, D), dtype=torch.float32, device=dev)
        rc = lib().kda_chunk_fwd_snapshots(
            ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(z), _ptr(A), _ptr(S0), _ptr(gate),
            _ptr(rms_w), _ptr(res.get("o")), _ptr(res.get("y")), _ptr(res.get("S_T")), _ptr(res["snapshots"]),
            int(snapshot_chunks), _ptr(workspace), workspace.numel(), _stream(dev))
        if rc != 0:
            raise KdaError("kda_chunk_fwd_snapshots", rc)
        return res
    args = (ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(z), _ptr(A), _ptr(S0), _ptr(gate),
            _ptr(rms_w), _ptr(res.get("o")), _ptr(res.get("y")), _ptr(res.get("S_T")), _ptr(workspace),
            workspace.numel(), _stream(dev))
    if events is None:
        rc = lib().kda_chunk_fwd(*args)
    else:
        arr = (ctypes.c_void_p * len(events))(*[ctypes.c_void_p(e) for e in events])
        rc = lib().kda_chunk_fwd_traced(*args, arr, len(events))
    if rc != 0:
        raise KdaError("kda_chunk_fwd", rc)
    return res


NOALLOC_SCRATCH_BYTES = 128 << 20  # KDA_NOALLOC_SCRATCH_BYTES


def chunk_fwd_noalloc(q, k, v, beta, z, A, S0=None, gate=None, rms_w=None, *, out_dtype=None, want_o=True,
                      want_y=None, want_state=True, out=None, head_first=False, **opts):
    """kda_chunk_fwd_noalloc: the forward without a workspace (the library's
    per-GPU scratch array, one-stream schedule).  Arguments and result as
    chunk_fwd; only the outputs are allocated here, by the caller's side."""
    B, T, H, D = _check_forward_args(q, k, v, beta, z, A, S0, gate, rms_w, out, head_first)
    tok_shape = (B, H, T, D) if head_first else (B, T, H, D)
    odt = q.dtype if out_dtype is None else out_dtype
    desc = make_desc(B, T, H, D, _dt(q), _dt(torch.empty(0, dtype=odt)), head_first=head_first, **opts)
    want_y = (gate is not None) if want_y is None else want_y
    res = dict(out or {})
    dev = q.device
    if want_o and "o" not in res:
        res["o"] = torch.empty(tok_shape, dtype=odt, device=dev)
    if want_y and "y" not in res:
        res["y"] = torch.empty(tok_shape, dtype=odt, device=dev)
    if want_state and "S_T" not in res:
        res["S_T"] = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    rc = lib().kda_chunk_fwd_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(z), _ptr(A),
                                     _ptr(S0), _ptr(gate), _ptr(rms_w), _ptr(res.get("o")), _ptr(res.get("y")),
                                     _ptr(res.get("S_T")), _stream(dev))
    if rc != 0:
        raise KdaError("kda_chunk_fwd_noalloc", rc)
    return res


def input_prep(xq, xk, xv, wq, wk, wv, beta_logits=None, state_in=None, state_out=None, *, out=None):
    """Input steps before the core: q, k, v = Swish(ShortConv(x)), beta =
    Sigmoid(beta_logits).  x*: [B, T, H, D] (bf16 or fp32); w*: [H * D, W]
    fp32 taps (W = 1..4, the last tap on the current token); state_in /
    state_out: [B, 3, W - 1, H * D] fp32 conv windows (None: zeros / not
    written; they may be the same tensor).  Returns a dict with q, k, v (and
    beta)."""
    if xq.dim() != 4 or wq.dim() != 2:
        raise ValueError("xq must be [B, T, H, D] and wq [H * D, W]")
    B, T, H, D = xq.shape
    W = wq.shape[1]
    for name, t in (("xk", xk), ("xv", xv)):
        _expect(name, t, xq.shape, xq.dtype)
    _expect("beta_logits", beta_logits, (B, T, H), xq.dtype)
    for name, t in (("wq", wq), ("wk", wk), ("wv", wv)):
        _expect(name, t, (H * D, W), torch.float32)
    for name, t in (("state_in", state_in), ("state_out", state_out)):
        _expect(name, t, (B, 3, W - 1, H * D), torch.float32)
    for name in ("q", "k", "v"):
        _expect(f"out['{name}']", (out or {}).get(name), (B, T, H, D), xq.dtype)
    _expect("out['beta']", (out or {}).get("beta"), (B, T, H), xq.dtype)
    desc = make_desc(B, T, H, D, _dt(xq), _dt(xq))
    res = dict(out or {})
    for n in ("q", "k", "v"):
        if n not in res:
            res[n] = torch.empty((B, T, H, D), dtype=xq.dtype, device=xq.device)
    if beta_logits is not None and "beta" not in res:
        res["beta"] = torch.empty((B, T, H), dtype=xq.dtype, device=xq.device)
    rc = lib().kda_input_prep(ctypes.byref(desc), int(W), _ptr(xq), _ptr(xk), _ptr(xv), _ptr(beta_logits),
                              _ptr(wq), _ptr(wk), _ptr(wv), _ptr(state_in), _ptr(state_out), _ptr(res["q"]),
                              _ptr(res["k"]), _ptr(res["v"]), _ptr(res.get("beta")), _stream(xq.device))
    if rc != 0:
        raise KdaError("kda_input_prep", rc)
    return res


def recurrent_step(q, k, v, beta, z, A, S_pool, slot=None, gate=None, rms_w=None, *, out_dtype=None,
                   want_o=True, want_y=None, out=None, status=None, **opts):
    """One decode token for n sequences.  q, k, v, z (and gate): [n, H, D];
    beta [n, H]; S_pool [n_slots, H, D, D] fp32 updated in place; slot: int32
    [n] or None.  status: a device uint32 tensor that collects
    KDA_FLAG_BAD_SLOT for slots outside [0, n_slots) (those are skipped)."""
    if q.dim() != 3 or S_pool.dim() != 4:
        raise ValueError("q must be [n, H, D] and S_pool [n_slots, H, D, D]")
    n, H, D = q.shape
    for name, t in (("k", k), ("v", v), ("z", z), ("gate", gate)):
        _expect(name, t, (n, H, D), q.dtype)
    _expect("beta", beta, (n, H), q.dtype)
    _expect("A", A, (H,), torch.float32)
    _expect("S_pool", S_pool, (S_pool.shape[0], H, D, D), torch.float32)
    _expect("slot", slot, (n,), torch.int32)
    _expect("rms_w", rms_w, (H, D), torch.float32)
    for name in ("o", "y"):
        _expect(f"out['{name}']", (out or {}).get(name), (n, H, D))
    odt = q.dtype if out_dtype is None else out_dtype
    desc = make_desc(n, 1, H, D, _dt(q), _dt(torch.empty(0, dtype=odt)), **opts)
    want_y = (gate is not None) if want_y is None else want_y
    res = dict(out or {})
    if want_o and "o" not in res:
        res["o"] = torch.empty((n, H, D), dtype=odt, device=q.device)
    if want_y and "y" not in res:
        res["y"] = torch.empty((n, H, D), dtype=odt, device=q.device)
    rc = lib().kda_recurrent_step(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(z), _ptr(A),
                                  _ptr(S_pool), int(S_pool.shape[0]), _ptr(slot), _ptr(gate), _ptr(rms_w),
                                  _ptr(res.get("o")), _ptr(res.get("y")), _ptr(status), _stream(q.device))
    if rc != 0:
        raise KdaError("kda_recurrent_step", rc)
    return res


FLAG_BAD_SLOT = 1  # KDA_FLAG_BAD_SLOT


def state_io(op: int, pool, user=None, slot=None, n=None, layout: int = LAYOUT_KV, status=None):
    """ZERO / IMPORT / EXPORT states between ``pool`` [n_slots, H, D, D] and
    ``user`` [n, H, D, D] (layout KV) or its transpose (layout VK).  status:
    as for recurrent_step."""
    if pool.dim() != 4:
        raise ValueError("pool must be [n_slots, H, D, D]")
    n_slots, H, Dk, Dv = pool.shape
    _expect("pool", pool, pool.shape, torch.float32)
    if n is None:
        n = user.shape[0] if user is not None else (slot.numel() if slot is not None else pool.shape[0])
    _expect("user", user, (n, H, Dk, Dv) if layout == LAYOUT_KV else (n, H, Dv, Dk), torch.float32)
    _expect("slot", slot, (n,), torch.int32)
    rc = lib().kda_state_io(op, n, H, Dk, Dv, layout, _ptr(pool), int(n_slots), _ptr(slot), _ptr(user), _ptr(status),
                            _stream(pool.device))
    if rc != 0:
        raise KdaError("kda_state_io", rc)


def prepass(q, k, z, A, **opts):
    """Chunk-local cumulative log-decay G [B, T, H, D] and inverse norms rq, rk
    [B, T, H] (diagnostic view of the first step of chunk_fwd)."""
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, D]")
    B, T, H, D = q.shape
    for name, t in (("k", k), ("z", z)):
        _expect(name, t, q.shape, q.dtype)
    _expect("A", A, (H,), torch.float32)
    desc = make_desc(B, T, H, D, _dt(q), KDA_F32, **opts)
    G = torch.empty((B, T, H, D), dtype=torch.float32, device=q.device)
    rq = torch.empty((B, T, H), dtype=torch.float32, device=q.device)
    rk = torch.empty((B, T, H), dtype=torch.float32, device=q.device)
    rc = lib().kda_prepass(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(z), _ptr(A), _ptr(G), _ptr(rq), _ptr(rk),
                           _stream(q.device))
    if rc != 0:
        raise KdaError("kda_prepass", rc)
    return G, rq, rk


def build():
    from . import _build
    return _build.build()
