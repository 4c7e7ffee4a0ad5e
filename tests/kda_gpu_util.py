"""Helpers for the GPU parity tests (no method arithmetic here)."""
import numpy as np
import torch

import synth


def dev(a, device="cuda"):
    """numpy -> device tensor; uint16 arrays are bf16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def host64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def widen(a):
    return synth.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a


def rel_l2(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm((x - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-300))


def log(msg):
    print(msg, flush=True)
