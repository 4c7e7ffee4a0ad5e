"""C-ABI checks that need no GPU: the library loads, exports every function
include/kda.h declares, and rejects bad arguments on the host before any HIP
call (the pointers below are never dereferenced)."""
import ctypes
import re

import pytest

import gated_delta_rule_84_amd as kda

FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced by host validation


def _declared():
    src = open(kda.HEADER_PATH).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = kda.lib()
    names = _declared()
    assert {"kda_chunk_fwd", "kda_recurrent_step", "kda_state_io"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    assert L.kda_abi_version() == kda.ABI_VERSION == int(re.search(r"#define KDA_ABI_VERSION (\d+)", open(kda.HEADER_PATH).read()).group(1))
    assert L.kda_status_str(6) == b"workspace missing or too small"


def _desc(**kw):
    d = kda.KdaDesc()
    rc = kda.lib().kda_desc_init(ctypes.byref(d), 2, 100, 3, 128, kda.KDA_BF16, kda.KDA_BF16)
    assert rc == 0
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def P(i):
    """The i-th of several disjoint fake device ranges (4 GiB apart)."""
    return FAKE + i * (1 << 32)


def _fwd(d, q=P(0), k=P(1), v=P(2), beta=P(3), z=P(4), A=P(5), S0=None, gate=None, w=None, o=P(6), y=None,
         ST=None, ws=P(7), nbytes=1 << 40):
    return kda.lib().kda_chunk_fwd(ctypes.byref(d), q, k, v, beta, z, A, S0, gate, w, o, y, ST, ws, nbytes, None)


def test_desc_validation():
    L = kda.lib()
    d = kda.KdaDesc()
    assert L.kda_desc_init(ctypes.byref(d), 1, 10, 1, 96, 1, 1) == 5     # head dim 96 unsupported
    assert L.kda_desc_init(ctypes.byref(d), 0, 10, 1, 128, 1, 1) == 2    # B = 0
    assert L.kda_desc_init(ctypes.byref(d), 1, -1, 1, 128, 1, 1) == 2    # T < 0
    assert L.kda_desc_init(ctypes.byref(d), 1, 10, 1, 128, 7, 1) == 3    # bad dtype
    assert L.kda_desc_init(None, 1, 10, 1, 128, 1, 1) == 1
    assert L.kda_desc_init(ctypes.byref(d), 1, 10, 1, 64, 0, 0) == 0
    assert d.chunk == 64 and d.g_min == -5.0 and d.qk_l2norm == 1


def test_forward_host_errors():
    assert _fwd(_desc(), q=None) == 1
    assert _fwd(_desc(), o=None, y=None, ST=None) == 1
    assert _fwd(_desc(), y=P(8), gate=None) == 1                  # y needs the gate logits
    assert _fwd(_desc(), v=P(2) + 2) == 4                         # misaligned
    assert _fwd(_desc(), beta=P(3) + 1) == 4
    # workspace errors exist only for the two-kernel schedules (the fused one
    # needs none and would launch here)
    assert _fwd(_desc(fused=0), ws=None) == 6
    assert _fwd(_desc(fused=0), nbytes=1024) == 6                 # smaller than one chunk needs
    assert _fwd(_desc(fused=3)) == 2                              # flag out of range
    assert _fwd(_desc(g_min=-6.0)) == 5                           # 16 * g_min < -88: e^80 bound lost
    assert _fwd(_desc(g_min=0.0)) == 5
    assert _fwd(_desc(chunk=32)) == 5
    assert _fwd(_desc(d_v=64)) == 5


def test_forward_rejects_overlapping_outputs():
    """o, y, S_T over an input or over each other are refused before any
    launch (S_T over S0 is the allowed in-place update)."""
    d = _desc(fused=0)
    assert _fwd(d, o=P(0)) == 5                                   # o over q
    assert _fwd(d, o=P(2) + 1024) == 5                            # o starts inside v
    assert _fwd(d, o=None, y=P(4), gate=P(9)) == 5                # y over z
    assert _fwd(d, o=P(9), y=P(10), gate=P(9)) == 5               # o over the gate logits
    assert _fwd(d, y=P(6) + 512, gate=P(9)) == 5                  # y overlaps o
    assert _fwd(d, S0=P(10), ST=P(10) + 4) == 5                   # S_T overlaps S0 without equalling it
    assert _fwd(d, ST=P(5)) == 5                                  # S_T over A
    assert _fwd(d, S0=P(10), ST=P(10), ws=None) == 6              # S_T == S0 passes on to the workspace check


def test_workspace_sizes():
    L = kda.lib()
    d = _desc(fused=0)
    one = L.kda_chunk_fwd_workspace_size_for(ctypes.byref(d), 1)
    two = L.kda_chunk_fwd_workspace_size_for(ctypes.byref(d), 65)
    full = L.kda_chunk_fwd_workspace_size(ctypes.byref(d))
    assert 0 < one < two == full  # T = 100 -> 2 chunks
    bad = _desc(d_k=96, d_v=96)
    assert L.kda_chunk_fwd_workspace_size(ctypes.byref(bad)) == 0


def test_decode_and_state_io_host_errors():
    L = kda.lib()
    d = _desc()
    args = [FAKE] * 6
    assert L.kda_recurrent_step(ctypes.byref(d), *args, FAKE, 64, None, None, None, FAKE, None, None, None) == 2  # T != 1
    d.T = 1
    assert L.kda_recurrent_step(ctypes.byref(d), *args, None, 64, None, None, None, FAKE, None, None, None) == 1  # no pool
    assert L.kda_recurrent_step(ctypes.byref(d), *args, FAKE, 64, None, None, None, None, FAKE, None, None) == 1  # y, no gate
    # pool rows: at least one, and B of them for the identity mapping
    assert L.kda_recurrent_step(ctypes.byref(d), *args, FAKE, 0, None, None, None, FAKE, None, None, None) == 2
    assert L.kda_recurrent_step(ctypes.byref(d), *args, FAKE, d.B - 1, None, None, None, FAKE, None, None, None) == 2
    assert L.kda_recurrent_step(ctypes.byref(d), *args, FAKE, 64, FAKE + 2, None, None, FAKE, None, None, None) == 4
    assert L.kda_state_io(9, 1, 1, 128, 128, 0, FAKE, 1, None, FAKE, None, None) == 5
    assert L.kda_state_io(1, 1, 1, 128, 64, 0, FAKE, 1, None, FAKE, None, None) == 5
    assert L.kda_state_io(1, 1, 1, 128, 128, 0, FAKE, 1, None, None, None, None) == 1
    assert L.kda_state_io(0, -1, 1, 128, 128, 0, FAKE, 1, None, None, None, None) == 2
    # pool row counts: at least one, and enough rows for the identity mapping
    assert L.kda_state_io(0, 2, 1, 128, 128, 0, FAKE, 0, None, None, None, None) == 2
    assert L.kda_state_io(0, 3, 1, 128, 128, 0, FAKE, 2, None, None, None, None) == 2
    assert L.kda_state_io(1, 1, 1, 128, 128, 0, FAKE, 1, None, FAKE, FAKE + 2, None) == 4  # status alignment
    assert L.kda_state_io(1, 0, 1, 128, 128, 0, FAKE, 1, None, FAKE, None, None) == 0  # nothing to do


def test_no_cpu_fallback(monkeypatch, tmp_path):
    """The binding refuses to run without the built library."""
    monkeypatch.setattr(kda, "_lib", None)
    monkeypatch.setattr(kda, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        kda.lib()


def _snap(d, snaps=P(8), every=1, o=P(6), ST=None):
    return kda.lib().kda_chunk_fwd_snapshots(ctypes.byref(d), P(0), P(1), P(2), P(3), P(4), P(5), None, None, None,
                                             o, None, ST, snaps, every, P(7), 1 << 40, None)


def test_snapshot_host_errors_and_count():
    L = kda.lib()
    d = _desc(T=1000)                                             # 15 full chunks + a tail
    assert L.kda_snapshot_count(ctypes.byref(d), 1) == 15
    assert L.kda_snapshot_count(ctypes.byref(d), 4) == 3
    assert L.kda_snapshot_count(ctypes.byref(d), 16) == 0
    assert L.kda_snapshot_count(ctypes.byref(d), 0) == 0
    assert L.kda_snapshot_count(ctypes.byref(_desc(d_k=96, d_v=96)), 1) == 0
    assert _snap(d, every=0) == 2
    assert _snap(d, snaps=None) == 1                              # 15 boundaries need the buffer
    assert _snap(d, snaps=P(8) + 2) == 4
    assert _snap(_desc(T=1000, chunk=32)) == 5
    assert _snap(d, every=16, snaps=None, o=None) == 0            # no boundary, no output: nothing to do


def test_schedule_query():
    L = kda.lib()
    seg, sch = ctypes.c_int32(0), ctypes.c_int32(0)
    assert _desc().fused == 1                                     # the default: the library decides
    d = _desc(T=70000, fused=2)                                   # forced
    assert L.kda_chunk_fwd_schedule(ctypes.byref(d), 0, ctypes.byref(seg), ctypes.byref(sch)) == 0
    assert sch.value == 2 and seg.value == 70016                  # fused: whole sequence, no workspace
    assert L.kda_chunk_fwd_workspace_size(ctypes.byref(d)) == 256
    d32 = _desc(T=70000, in_dtype=kda.KDA_F32, fused=2)           # fp32 inputs: two-kernel schedules
    assert L.kda_chunk_fwd_schedule(ctypes.byref(d32), 0, ctypes.byref(seg), ctypes.byref(sch)) == 6
    d2 = _desc(T=1000, fused=0, overlap=0)
    ws = L.kda_chunk_fwd_workspace_size(ctypes.byref(d2))
    assert L.kda_chunk_fwd_schedule(ctypes.byref(d2), ws, ctypes.byref(seg), ctypes.byref(sch)) == 0
    assert sch.value == 0 and seg.value == 1024


def _launches(d, ws):
    L = kda.lib()
    n = ctypes.c_int32(0)
    assert L.kda_chunk_fwd_launches(ctypes.byref(d), ws, None, 0, ctypes.byref(n)) == 0
    kinds = (ctypes.c_int32 * max(n.value, 1))()
    assert L.kda_chunk_fwd_launches(ctypes.byref(d), ws, kinds, n.value, ctypes.byref(n)) == 0
    return [kinds[i] for i in range(n.value)]


def test_workspace_and_launch_queries():
    """Without a GPU the two-stream schedules are unavailable, so the library
    plans the one-stream segments; the size query still offers the pipelined
    schedule's workspace for bf16 inputs: every record up to its cap, beyond
    it the largest window that fits the cap."""
    L = kda.lib()
    rec = 61952                                                   # bytes per chunk record at d = 128, fp16 entries
    d = _desc(B=1, T=65536, H=96, fused=0)
    ws = L.kda_chunk_fwd_workspace_size(ctypes.byref(d))
    assert ws >= 96 * 1024 * rec and ws < 96 * 1024 * rec + (64 << 20)   # every record, plus state and counters
    big = _desc(B=1, T=1 << 20, H=96, fused=0)                    # every record would be 97 GB: windows
    ws_big = L.kda_chunk_fwd_workspace_size(ctypes.byref(big))
    cap = 8 << 30                                                 # the largest window of the pipelined schedule
    assert cap - 96 * 2 * rec - (64 << 20) <= ws_big <= cap       # within the cap, less than a segment short of it
    f32 = _desc(B=1, T=65536, H=96, fused=0, in_dtype=kda.KDA_F32)  # fp32: no pipelined schedule
    assert L.kda_chunk_fwd_workspace_size(ctypes.byref(f32)) < 96 * 1024 * rec
    # launch order of the one-stream plan: (intra, scan) per segment
    seg = L.kda_chunk_fwd_workspace_size_for(ctypes.byref(d), 8192)
    assert _launches(d, seg) == [0, 1] * 8
    assert _launches(_desc(T=70000, fused=2), 0) == [2]
    n = ctypes.c_int32(0)
    assert L.kda_chunk_fwd_launches(ctypes.byref(d), seg, None, 4, ctypes.byref(n)) == 1      # kinds NULL
    assert L.kda_chunk_fwd_launches(ctypes.byref(d), 0, None, 0, ctypes.byref(n)) == 6        # no workspace


def _prep(d, width=4, xq=FAKE, beta_logits=FAKE, beta=FAKE, st_in=None, st_out=None, q=FAKE):
    return kda.lib().kda_input_prep(ctypes.byref(d), width, xq, FAKE, FAKE, beta_logits, FAKE, FAKE, FAKE,
                                    st_in, st_out, q, FAKE, FAKE, beta, None)


def test_input_prep_host_errors():
    d = _desc()
    assert _prep(d, width=0) == 5 and _prep(d, width=5) == 5          # widths 1..4
    assert _prep(d, beta=None) == 1                                  # beta logits without an output
    assert _prep(d, beta_logits=None) == 1
    assert _prep(d, xq=None) == 1 and _prep(d, q=None) == 1
    assert _prep(d, xq=FAKE + 2) == 4                                # 16-byte vectors
    assert _prep(d, st_in=FAKE + 2) == 4
    assert _prep(_desc(d_k=96, d_v=96)) == 5


def test_input_prep_rejects_overlapping_outputs():
    """q, k, v written over an input (or each other) are rejected before any
    launch.  (The allowed aliases, beta over its logits and the state updated
    in place, are exercised on the GPU by the input-step tests.)"""
    L = kda.lib()
    d = _desc(B=1, T=8, H=2, d_k=64, d_v=64)
    xb = 8 * 2 * 64 * 2                                               # bytes of one [B, T, H, d] bf16 tensor
    X = [FAKE + i * (1 << 20) for i in range(10)]                     # disjoint fake device ranges

    def call(q=X[3], k=X[4], v=X[5], beta=X[6], bl=X[7], st_in=X[8], st_out=X[9]):
        return L.kda_input_prep(ctypes.byref(d), 4, X[0], X[1], X[2], bl, X[0], X[1], X[2], st_in, st_out,
                                q, k, v, beta, None)
    assert call(q=X[0]) == 5                                          # q over x_q
    assert call(k=X[0] + xb - 16) == 5                                # k starts inside x_q
    assert call(v=X[3] + 16) == 5                                     # v overlaps q
    assert call(st_out=X[8] + 16) == 5                                # state_out overlaps state_in, not equal
    assert call(beta=X[2]) == 5                                       # beta over x_v


def test_kcp_host_errors():
    L = kda.lib()
    d = _desc(T=1000)                                                # 1000 is not a multiple of 128
    assert L.kda_chunk_fwd_kcp_workspace_size(ctypes.byref(d), 2) == 0
    assert L.kda_chunk_fwd_kcp(ctypes.byref(d), 2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, FAKE, None,
                               None, FAKE, 1 << 40, None) == 5
    assert L.kda_chunk_fwd_kcp(ctypes.byref(d), 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, FAKE, None,
                               None, FAKE, 1 << 40, None) == 2
    d2 = _desc(T=1024)
    one = L.kda_chunk_fwd_kcp_workspace_size(ctypes.byref(d2), 1)
    four = L.kda_chunk_fwd_kcp_workspace_size(ctypes.byref(d2), 4)
    assert one == L.kda_chunk_fwd_workspace_size(ctypes.byref(d2)) and four >= 3 * 2 * 4 * 3 * 128 * 128 * 4


def test_token_layout_field():
    """kda_desc.tokens: token major by default; head first is accepted by the
    forward, rejected (KDA_ERR_UNSUPPORTED, before any GPU work) by the
    entry points that take token-major tensors only; other values are
    rejected."""
    L = kda.lib()
    assert _desc().tokens == 0
    assert kda.make_desc(1, 64, 2, 128, kda.KDA_BF16, kda.KDA_BF16, head_first=True).tokens == 1
    assert _fwd(_desc(tokens=2)) == 5
    hf = _desc(T=1024, tokens=1)
    assert L.kda_chunk_fwd_workspace_size(ctypes.byref(hf)) == L.kda_chunk_fwd_workspace_size(ctypes.byref(_desc(T=1024)))
    assert L.kda_chunk_fwd_kcp_workspace_size(ctypes.byref(hf), 2) == 0
    assert L.kda_chunk_fwd_kcp(ctypes.byref(hf), 2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, FAKE, None,
                               None, FAKE, 1 << 40, None) == 5
    assert L.kda_prepass(ctypes.byref(hf), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 5
    assert L.kda_input_prep(ctypes.byref(hf), 4, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, None,
                            FAKE, FAKE, FAKE, None, None) == 5


def test_decay_map_field():
    assert _desc().decay == 0                                        # K3 map by default
    assert _fwd(_desc(decay=2)) == 5                                 # unknown map


def test_noalloc_rejects_oversized_shapes_on_the_host():
    """kda_chunk_fwd_noalloc: a shape whose single chunk of records and states
    exceeds the per-GPU scratch array is refused before anything is enqueued
    (no GPU needed); invalid descriptors are refused too."""
    L = kda.lib()
    d = kda.make_desc(16, 64, 128, 128, kda.KDA_BF16, kda.KDA_BF16)  # B * H = 2048
    p = ctypes.c_void_p(256)
    assert L.kda_chunk_fwd_noalloc(ctypes.byref(d), p, p, p, p, p, p, None, None, None, p, None, None, None) == 6
    d.chunk = 32
    assert L.kda_chunk_fwd_noalloc(ctypes.byref(d), p, p, p, p, p, p, None, None, None, p, None, None, None) == 5
    assert kda.NOALLOC_SCRATCH_BYTES == 128 << 20
