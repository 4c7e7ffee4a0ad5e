"""Planted mistakes: each pin set must catch a plausible error in the oracle.

Every case below rewrites one expression of oracle/kda_ref.py (a dropped term,
a flipped sign, a transposed operand, a wrong diagonal, a wrong axis or
reduction), loads the rewritten source as a separate module on the CPU, and
runs the pins of test_oracle_pins.py against it.  At least one pin must fail
for every mistake; the unmodified oracle passes them all.
"""
import importlib.util
import inspect
import os
import types

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = open(os.path.join(ROOT, "oracle", "kda_ref.py")).read()

# (name, exact text in the oracle, planted replacement)
MUTANTS = [
    ("decay_rows_vs_cols", "S = alpha[t][:, None] * S", "S = S * alpha[t][None, :]"),
    ("delta_sign", "np.outer(kt, v[t] - S.T @ kt)", "np.outer(kt, v[t] + S.T @ kt)"),
    ("readout_transposed", "o[t] = S.T @ q[t]", "o[t] = S @ q[t]"),
    ("literal_order", "M = (eye - beta[t] * np.outer(kt, kt)) @ np.diag(alpha[t])",
     "M = np.diag(alpha[t]) @ (eye - beta[t] * np.outer(kt, kt))"),
    ("ut_includes_diagonal", "L = np.tril(bc[:, None] * (Kf @ Kb.T), -1)", "L = np.tril(bc[:, None] * (Kf @ Kb.T), 0)"),
    ("ut_beta_on_columns", "L = np.tril(bc[:, None] * (Kf @ Kb.T), -1)", "L = np.tril((Kf @ Kb.T) * bc[None, :], -1)"),
    ("aqk_strict", "Aqk = np.tril(Qf @ Kb.T)", "Aqk = np.tril(Qf @ Kb.T, -1)"),
    ("gamma_exclusive", "G = np.cumsum(g[c0:c1], axis=0)", "G = np.cumsum(g[c0:c1], axis=0) - g[c0:c1]"),
    ("chunk_state_decay_dropped", "S = Gam[-1][:, None] * S + ", "S = S + "),
    ("decay_scale_not_exponentiated", "sigmoid(np.exp(np.float64(A_h)) * np.asarray(z",
     "sigmoid(np.float64(A_h) * np.asarray(z"),
    ("decay_sign", "return g_min * sigmoid(", "return -g_min * sigmoid("),
    ("rms_sum_not_mean", "np.mean(o * o, axis=-1, keepdims=True)", "np.sum(o * o, axis=-1, keepdims=True)"),
    ("l2_eps_outside_sqrt", "np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)",
     "(np.sqrt(np.sum(x * x, axis=-1, keepdims=True)) + eps)"),
    ("compose_order", "return M2 @ M1, S2 + M2 @ S1", "return M1 @ M2, S2 + M2 @ S1"),
    ("step_matrix_order",
     "return (np.eye(k_t.size) - beta_t * np.outer(k_t, k_t)) @ np.diag(np.asarray(alpha_t, dtype=np.float64))",
     "return np.diag(np.asarray(alpha_t, dtype=np.float64)) @ (np.eye(k_t.size) - beta_t * np.outer(k_t, k_t))"),
    ("conv_taps_flipped", "y += w[:, j] * ext[j:j + T]", "y += w[:, W - 1 - j] * ext[j:j + T]"),
    ("conv_state_newest_first", "ext = np.concatenate([prev, x], axis=0)",
     "ext = np.concatenate([prev[::-1], x], axis=0)"),
    ("conv_state_not_advanced", "return y, ext[T:].copy()", "return y, ext[:W - 1].copy()"),
    ("swish_sign", "return x * sigmoid(x)", "return x * sigmoid(-x)"),
    ("softplus_scale_dropped", "return -np.exp(np.float64(A_h)) * np.logaddexp(0.0, z)",
     "return -np.logaddexp(0.0, z)"),
    ("softplus_as_relu", "return -np.exp(np.float64(A_h)) * np.logaddexp(0.0, z)",
     "return -np.exp(np.float64(A_h)) * np.maximum(z, 0.0)"),
    ("q_scale_on_keys", "return q * scale, k", "return q, k * scale"),
    ("l2norm_flag_ignored", "    if l2norm:\n        q = l2_normalize(q, eps)", "    if True:\n        q = l2_normalize(q, eps)"),
]


def _load_variant(src: str, tag: str) -> types.ModuleType:
    spec = importlib.util.spec_from_loader(f"kda_ref_{tag}", loader=None)
    mod = importlib.util.module_from_spec(spec)
    exec(compile(src, f"<kda_ref {tag}>", "exec"), mod.__dict__)
    return mod


def _pins():
    spec = importlib.util.spec_from_file_location("_pins", os.path.join(ROOT, "tests", "test_oracle_pins.py"))
    pins = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(pins)
    return pins


def _run_pins(pins, ref, golden_dir):
    """Run every pin against module `ref`; return the names of those that fail."""
    failed = []
    saved = pins.R
    pins.R = ref
    pins.RNG = np.random.default_rng(12345)
    try:
        for name, fn in sorted(vars(pins).items()):
            if not name.startswith("test_") or not callable(fn):
                continue
            if name.startswith("test_c_oracle"):
                continue  # compare the C oracle with the (unmodified) numpy one
            params = inspect.signature(fn).parameters
            calls = [{}]
            if "chunk" in params:
                calls = [{"chunk": 16, "T": 65}, {"chunk": 64, "T": 100}]
            if "name" in params:
                calls = [{"name": "tiny"}]
            for kw in calls:
                if "golden_dir" in params:
                    kw = dict(kw, golden_dir=golden_dir)
                try:
                    fn(**kw)
                except Exception:  # noqa: BLE001 - any failure of the pin counts
                    failed.append(name)
                    break
    finally:
        pins.R = saved
    return failed


def test_unmodified_oracle_passes_every_pin(golden_dir):
    pins = _pins()
    assert _run_pins(pins, _load_variant(SRC, "orig"), golden_dir) == []


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, old, new, golden_dir):
    assert SRC.count(old) >= 1, f"mutation site of {name} not found in the oracle"
    mutated = SRC.replace(old, new, 1)
    pins = _pins()
    failed = _run_pins(pins, _load_variant(mutated, name), golden_dir)
    assert failed, f"no pin catches the planted mistake {name}"
