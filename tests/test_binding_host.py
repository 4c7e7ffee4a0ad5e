"""The Python binding's argument checks, on the CPU (no GPU work): a
forward call whose tensors disagree in shape or element type is refused
before any pointer reaches the library."""
import pytest
import torch

import gated_delta_rule_84_amd as kda


def _tensors(B=1, T=70, H=2, D=64, head_first=False, dtype=torch.bfloat16):
    tok = (B, H, T, D) if head_first else (B, T, H, D)
    per = (B, H, T) if head_first else (B, T, H)
    t = {n: torch.zeros(tok, dtype=dtype) for n in ("q", "k", "v", "z", "gate")}
    t["beta"] = torch.zeros(per, dtype=dtype)
    t["A"] = torch.zeros((H,), dtype=torch.float32)
    t["S0"] = torch.zeros((B, H, D, D), dtype=torch.float32)
    return t


def _call(t, fn=None, **kw):
    fn = fn or kda.chunk_fwd
    return fn(t["q"], t["k"], t["v"], t["beta"], t["z"], t["A"], S0=t["S0"], gate=t["gate"], **kw)


@pytest.mark.parametrize("head_first", [False, True])
@pytest.mark.parametrize("fn", [kda.chunk_fwd, kda.chunk_fwd_noalloc])
def test_forward_refuses_mismatched_tensors(fn, head_first):
    bad = [
        ("k", torch.zeros((1, 71, 2, 64), dtype=torch.bfloat16)),      # one token more
        ("v", torch.zeros((1, 70, 2, 64), dtype=torch.float32)),       # other element type
        ("beta", torch.zeros((1, 70, 2, 1), dtype=torch.bfloat16)),    # not [B, T, H]
        ("A", torch.zeros((3,), dtype=torch.float32)),                 # one decay scale per head
        ("A", torch.zeros((2,), dtype=torch.bfloat16)),
        ("S0", torch.zeros((1, 2, 64, 32), dtype=torch.float32)),
        ("gate", torch.zeros((1, 70, 2, 128), dtype=torch.bfloat16)),
    ]
    for name, tensor in bad:
        t = _tensors(head_first=head_first)
        if head_first and tensor.dim() == 4 and name != "S0":
            tensor = tensor.permute(0, 2, 1, 3)
        t[name] = tensor
        with pytest.raises(ValueError, match=name):
            _call(t, fn, head_first=head_first)
    t = _tensors(head_first=head_first)
    with pytest.raises(ValueError, match="out"):
        _call(t, fn, head_first=head_first, out={"y": torch.zeros((1, 2, 2, 2), dtype=torch.bfloat16)})
    # consistent CPU tensors pass the shape checks and stop at the device check
    with pytest.raises(ValueError, match="GPU"):
        _call(_tensors(head_first=head_first), fn, head_first=head_first)


def test_decode_state_io_prep_prepass_refuse_mismatched_tensors():
    bf = torch.bfloat16
    n, H, D = 3, 2, 64
    q = torch.zeros((n, H, D), dtype=bf)
    pool = torch.zeros((5, H, D, D))
    A = torch.zeros((H,))
    with pytest.raises(ValueError, match="beta"):
        kda.recurrent_step(q, q, q, torch.zeros((n, H + 1), dtype=bf), q, A, pool)
    with pytest.raises(ValueError, match="slot"):
        kda.recurrent_step(q, q, q, torch.zeros((n, H), dtype=bf), q, A, pool, slot=torch.zeros((n,), dtype=torch.int64))
    with pytest.raises(ValueError, match="S_pool"):
        kda.recurrent_step(q, q, q, torch.zeros((n, H), dtype=bf), q, A, torch.zeros((5, H, D, D), dtype=torch.float64))
    with pytest.raises(ValueError, match="user"):
        kda.state_io(kda.STATE_EXPORT, pool, torch.zeros((n, H, D, D // 2)))
    with pytest.raises(ValueError, match="slot"):
        kda.state_io(kda.STATE_EXPORT, pool, torch.zeros((n, H, D, D)), slot=torch.zeros((n + 1,), dtype=torch.int32))
    x = torch.zeros((1, 10, H, D), dtype=bf)
    w = torch.zeros((H * D, 4))
    with pytest.raises(ValueError, match="xv"):
        kda.input_prep(x, x, torch.zeros((1, 11, H, D), dtype=bf), w, w, w)
    with pytest.raises(ValueError, match="state_in"):
        kda.input_prep(x, x, x, w, w, w, state_in=torch.zeros((1, 3, 4, H * D)))
    with pytest.raises(ValueError, match="wk"):
        kda.input_prep(x, x, x, w, torch.zeros((H * D, 3)), w)
    with pytest.raises(ValueError, match="z"):
        kda.prepass(x, x, torch.zeros((1, 10, H, D)), A)
