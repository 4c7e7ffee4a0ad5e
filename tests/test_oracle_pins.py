"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: closed forms
that special cases of the recurrence reduce to, a hand-worked example, exact
rational arithmetic, the pages' printed numbers, algebraic identities (the
(M, S~) composition law) and invariants.  Together they are chosen so that a
dropped term, a wrong sign, a transposed operand or a mis-ordered step in the
oracle fails at least one of them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import kda_ref as R
import synth
from synth.workloads import WORKLOADS, gen_inputs

RNG = np.random.default_rng(12345)


def _rand_head(T, dk, dv, rng, z_std=1.0):
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    v = rng.standard_normal((T, dv))
    beta = rng.uniform(0.05, 0.95, T)
    z = rng.standard_normal((T, dk)) * z_std
    return q, k, v, beta, z


# ---------------------------------------------------------------- pages' numbers
def test_pages_decay_facts(golden_dir):
    """Numbers printed in section 2.2 of the source page."""
    f = json.load(open(os.path.join(golden_dir, "pages_decay_facts.json")))["facts"]
    g_min = f["g_min"]["value"]
    assert R.G_MIN == g_min
    # the map's range (g_min, 0): at A_h = 0 (its initial value) sample widely
    z = np.linspace(-60, 60, 20001)
    g = R.decay_log(z, f["A_h_init"]["value"])
    assert np.all(g >= g_min) and np.all(g <= 0)
    assert np.all(g[np.abs(z) < 30] > g_min) and np.all(g[np.abs(z) < 30] < 0)
    # alpha > e^-5 ~ 6.7e-3
    amin = math.exp(g_min)
    assert abs(amin - f["alpha_min"]["value"]) / f["alpha_min"]["value"] < f["alpha_min"]["rel_tol"]
    assert np.exp(g).min() >= amin
    # sub-tile reciprocal bound e^{-g_min * 16} = e^80 < bf16 max ~ 3.39e38 ~ e^88.7
    n = f["subtile_tokens"]["value"]
    assert -g_min * n == f["recip_bound_exp"]["value"]
    bf16_max = float(np.float32(synth.bf16_bits_to_f32(np.array([0x7F7F], np.uint16))[0]))
    assert abs(bf16_max - f["bf16_max"]["value"]) / f["bf16_max"]["value"] < f["bf16_max"]["rel_tol"]
    assert abs(math.log(bf16_max) - f["bf16_max_log"]["value"]) < f["bf16_max_log"]["abs_tol"]
    assert math.exp(f["recip_bound_exp"]["value"]) < bf16_max
    # four steps at the bound: e^-20 ~ 2e-9
    four = math.exp(4 * g_min)
    assert abs(four - f["four_pinned_steps"]["value"]) / f["four_pinned_steps"]["value"] < f["four_pinned_steps"]["rel_tol"]


def test_decay_map_values():
    """g = g_min * sigmoid(e^A z): sigmoid(0) = 1/2, e^{ln 2} = 2, limits."""
    assert R.decay_log(0.0, 0.0) == pytest.approx(-2.5, abs=1e-15)
    assert R.decay_log(1.0, math.log(2.0)) == pytest.approx(-5.0 / (1.0 + math.exp(-2.0)), rel=1e-15)
    assert R.decay_log(-3.0, 0.0) == pytest.approx(-5.0 * math.exp(-3.0) / (1 + math.exp(-3.0)), rel=1e-14)
    assert R.decay_log(1e4, 0.0) == -5.0
    assert R.decay_log(-1e4, 0.0) == 0.0
    # symmetry of the logistic: g(z) + g(-z) = g_min
    z = np.linspace(-7, 7, 57)
    np.testing.assert_allclose(R.decay_log(z, 0.3) + R.decay_log(-z, 0.3), -5.0, rtol=0, atol=1e-14)


@pytest.mark.parametrize("name", ["tiny", "prefill", "k3_layer", "long_context", "decode"])
def test_subtile_logdecay_bound(name):
    """Every aligned 16-token sub-tile's cumulative log-decay lies in (-80, 0]
    (section 2.2) for every workload's z distribution, in fp64; and in fp32
    the pinned heads reach exactly -80, never below."""
    wl = WORKLOADS[name]
    T = min(wl.T, 1024)
    H = wl.H
    inp = gen_inputs(wl, batch=(0, 1), time=(0, T))
    z = inp["z"]
    zf = synth.bf16_bits_to_f32(z) if z.dtype == np.uint16 else z
    g = R.decay_log(zf[0], inp["A"][None, :, None])  # [T, H, dk]
    sub = g[: (T // 16) * 16].reshape(T // 16, 16, H, wl.D).sum(axis=1)
    assert sub.max() <= 0.0 and sub.min() > -80.0
    # fp32 evaluation of the same map and sums
    e = np.exp(inp["A"].astype(np.float32))[None, :, None]
    g32 = np.float32(-5.0) / (np.float32(1.0) + np.exp(-(e * zf[0]).astype(np.float32)))
    c32 = np.cumsum(g32[: (T // 16) * 16].reshape(T // 16, 16, H, wl.D), axis=1, dtype=np.float32)
    assert c32.max() <= 0.0 and c32.min() >= -80.0
    if wl.z_split_pinned:
        assert c32[:, -1, H // 2:, :].min() == np.float32(-80.0)
        assert sub[:, H // 2:, :].min() > -80.0 and sub[:, H // 2:, :].min() < -79.99999


# ---------------------------------------------------------------- closed forms
def test_beta_zero_is_pure_decay():
    """beta = 0 removes the delta write: S_t = Diag(exp sum_{s<=t} g_s) S_0,
    i.e. each key-channel row decays on its own, o_t = S_t^T q_t."""
    T, dk, dv = 40, 6, 5
    q, k, v, _, z = _rand_head(T, dk, dv, RNG)
    z = z - 3.0
    S0 = RNG.standard_normal((dk, dv))
    o, S = R.kda_recurrent(q, k, v, np.zeros(T), z=z, A_h=0.2, S0=S0)
    g = R.decay_log(z, 0.2)
    qn = q / np.sqrt((q * q).sum(1, keepdims=True) + 1e-6)
    for t in range(T):
        St = np.exp(g[: t + 1].sum(0))[:, None] * S0
        np.testing.assert_allclose(o[t], St.T @ qn[t], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S, np.exp(g.sum(0))[:, None] * S0, rtol=1e-12)


def test_overwrite_with_orthonormal_keys():
    """alpha = 1 and beta = 1 with orthonormal keys: each write overwrites the
    value stored under its key; afterwards S = sum_j k_j v_j^T +
    (I - sum_j k_j k_j^T) S_0 and reading with q = k_j returns v_j exactly."""
    dk, dv, m = 8, 8, 5
    Qm, _ = np.linalg.qr(RNG.standard_normal((dk, dk)))
    keys = Qm[:, :m].T
    vals = RNG.standard_normal((m, dv))
    S0 = RNG.standard_normal((dk, dv))
    z = np.full((m, dk), -1e4)  # sigmoid underflows -> g = 0 -> alpha = 1
    o, S = R.kda_recurrent(keys, keys, vals, np.ones(m), z=z, S0=S0, l2norm=False)
    P = keys.T @ keys
    np.testing.assert_allclose(S, keys.T @ vals + (np.eye(dk) - P) @ S0, atol=1e-13)
    np.testing.assert_allclose(o, vals, atol=1e-13)  # o_t = S_t^T k_t = v_t
    for j in range(m):
        np.testing.assert_allclose(S.T @ keys[j], vals[j], atol=1e-13)


def test_scalar_worked_example(golden_dir):
    """d_k = d_v = 1 reduces to a first-order linear recurrence; hand-worked
    values in tests/golden/scalar_worked_example.json."""
    ex = json.load(open(os.path.join(golden_dir, "scalar_worked_example.json")))
    st = ex["steps"]
    fr = lambda s: float(Fraction(s))  # noqa: E731
    q = np.array([[fr(s["q"])] for s in st])
    k = np.array([[fr(s["k"])] for s in st])
    v = np.array([[fr(s["v"])] for s in st])
    beta = np.array([fr(s["beta"]) for s in st])
    g = np.log(np.array([[fr(s["alpha"])] for s in st]))
    o, S = R.kda_recurrent(q, k, v, beta, g=g, S0=np.array([[fr(ex["s0"])]]), l2norm=False)
    np.testing.assert_allclose(o[:, 0], [fr(s["o"]) for s in st], rtol=1e-15, atol=1e-15)
    assert S[0, 0] == pytest.approx(fr(st[-1]["s"]), rel=1e-15)
    oc, Sc = R.kda_chunked(q, k, v, beta, g=g, S0=np.array([[fr(ex["s0"])]]), l2norm=False, chunk=2)
    np.testing.assert_allclose(oc[:, 0], [fr(s["o"]) for s in st], rtol=1e-14, atol=1e-15)


def test_exact_rational_recurrence():
    """The fp64 oracle matches the recurrence evaluated in exact rational
    arithmetic (alpha given directly as rationals, no L2 norm)."""
    T, dk, dv = 6, 3, 2
    rng = np.random.default_rng(7)
    to_fr = lambda a: [[Fraction(int(x), 16) for x in row] for row in a]  # noqa: E731
    qi = rng.integers(-16, 17, (T, dk))
    ki = rng.integers(-16, 17, (T, dk))
    vi = rng.integers(-32, 33, (T, dv))
    ai = rng.integers(1, 17, (T, dk))
    bi = rng.integers(0, 17, T)
    S0i = rng.integers(-16, 17, (dk, dv))
    Q, K, V, Al, S = to_fr(qi), to_fr(ki), to_fr(vi), to_fr(ai), to_fr(S0i)
    Bt = [Fraction(int(x), 16) for x in bi]
    outs = []
    for t in range(T):
        # M = (I - beta k k^T) Diag(alpha); S = M S + beta k v^T
        M = [[((1 if i == j else 0) - Bt[t] * K[t][i] * K[t][j]) * Al[t][j] for j in range(dk)] for i in range(dk)]
        S = [[sum(M[i][l] * S[l][j] for l in range(dk)) + Bt[t] * K[t][i] * V[t][j] for j in range(dv)]
             for i in range(dk)]
        outs.append([sum(S[i][j] * Q[t][i] for i in range(dk)) for j in range(dv)])
    o, Sf = R.kda_recurrent(qi / 16, ki / 16, vi / 16, bi / 16, g=np.log(ai / 16), S0=S0i / 16, l2norm=False)
    np.testing.assert_allclose(o, np.array(outs, dtype=float), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(Sf, np.array(S, dtype=float), rtol=1e-13, atol=1e-14)
    oc, Sc = R.kda_chunked(qi / 16, ki / 16, vi / 16, bi / 16, g=np.log(ai / 16), S0=S0i / 16,
                           l2norm=False, chunk=4)
    np.testing.assert_allclose(oc, np.array(outs, dtype=float), rtol=1e-12, atol=1e-13)


def test_l2_normalize_values():
    x = np.array([[3.0, 4.0], [0.0, 0.0], [1e-4, 0.0]])
    y = R.l2_normalize(x)
    np.testing.assert_allclose(y[0], [3 / math.sqrt(25 + 1e-6), 4 / math.sqrt(25 + 1e-6)], rtol=1e-15)
    np.testing.assert_array_equal(y[1], [0.0, 0.0])  # eps keeps the zero row finite
    assert y[2, 0] == pytest.approx(1e-4 / math.sqrt(1e-8 + 1e-6), rel=1e-14)


def test_gate_closed_forms():
    """Section 2.3 gate without projections: sigmoid(0) = 1/2; RMSNorm maps
    c * 1 to sign(c) * 1 up to eps; a one-hot o = a e_j maps to
    a / sqrt(a^2 / d + eps) e_j."""
    d = 16
    y = R.output_gate(np.full((1, d), 3.0), np.zeros((1, d)))
    np.testing.assert_allclose(y, 0.5 * 3.0 / math.sqrt(9.0 + 1e-6), rtol=1e-15)
    y = R.output_gate(np.full((1, d), -2.0), np.full((1, d), 50.0), eps=0.0)
    np.testing.assert_allclose(y, -1.0, rtol=1e-15)
    o = np.zeros((1, d))
    o[0, 5] = 0.25
    y = R.output_gate(o, np.full((1, d), math.log(3.0)))  # sigmoid(ln 3) = 3/4
    ref = np.zeros((1, d))
    ref[0, 5] = 0.75 * 0.25 / math.sqrt(0.0625 / d + 1e-6)
    np.testing.assert_allclose(y, ref, rtol=1e-14, atol=1e-300)
    w = np.linspace(0.5, 2.0, d)
    np.testing.assert_allclose(R.output_gate(o, np.zeros((1, d)), w=w)[0, 5], 0.5 * 0.25 / math.sqrt(0.0625 / d + 1e-6) * w[5])


# ---------------------------------------------------------------- identities and invariants
@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("T", [1, 15, 17, 63, 65, 100])
def test_chunked_equals_sequential(chunk, T):
    dk, dv = 12, 10
    q, k, v, beta, z = _rand_head(T, dk, dv, RNG, z_std=2.0)
    S0 = RNG.standard_normal((dk, dv))
    o1, S1 = R.kda_recurrent(q, k, v, beta, z=z, A_h=0.4, S0=S0)
    o2, S2 = R.kda_chunked(q, k, v, beta, z=z, A_h=0.4, S0=S0, chunk=chunk)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12 * max(1, np.abs(o1).max()))
    np.testing.assert_allclose(S2, S1, rtol=0, atol=1e-12 * np.abs(S1).max())


def test_literal_and_rank1_forms_agree():
    q, k, v, beta, z = _rand_head(30, 7, 9, RNG)
    S0 = RNG.standard_normal((7, 9))
    o1, S1 = R.kda_recurrent(q, k, v, beta, z=z, A_h=-0.3, S0=S0)
    o2, S2 = R.kda_recurrent(q, k, v, beta, z=z, A_h=-0.3, S0=S0, literal=True)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S1, S2, rtol=1e-12, atol=1e-13)


def test_state_pair_composition():
    """Section 10.2: S_T = S~ + M S_0 (linearity in the entry state); splitting
    the sequence anywhere and composing (M, S~) pairs reproduces S_T, and the
    composition is associative."""
    T, dk, dv = 48, 6, 4
    q, k, v, beta, z = _rand_head(T, dk, dv, RNG)
    # weak decay (g ~ -0.1 per step) keeps every transfer M of order one, so
    # a mis-ordered product cannot hide below the tolerance
    z = z - 4.0
    S0 = RNG.standard_normal((dk, dv))
    _, ST = R.kda_recurrent(q, k, v, beta, z=z, A_h=0.1, S0=S0)
    M, St = R.segment_pair(q, k, v, beta, z=z, A_h=0.1)
    np.testing.assert_allclose(St + M @ S0, ST, atol=1e-12)
    cuts = [0, 7, 20, 21, 48]
    pairs = [R.segment_pair(q[a:b], k[a:b], v[a:b], beta[a:b], z=z[a:b], A_h=0.1) for a, b in zip(cuts, cuts[1:])]
    acc = pairs[0]
    for p in pairs[1:]:
        acc = R.compose(p, acc)
    np.testing.assert_allclose(acc[0], M, atol=1e-12)
    np.testing.assert_allclose(acc[1] + acc[0] @ S0, ST, atol=1e-12)
    a, b, c = pairs[:3]
    left = R.compose(c, R.compose(b, a))
    right = R.compose(R.compose(c, b), a)
    np.testing.assert_allclose(left[0], right[0], atol=1e-13)
    np.testing.assert_allclose(left[1], right[1], atol=1e-13)
    # split-and-resume through the sequential oracle is bit-identical
    o_a, S_a = R.kda_recurrent(q[:20], k[:20], v[:20], beta[:20], z=z[:20], A_h=0.1, S0=S0)
    o_b, S_b = R.kda_recurrent(q[20:], k[20:], v[20:], beta[20:], z=z[20:], A_h=0.1, S0=S_a)
    o_f, S_f = R.kda_recurrent(q, k, v, beta, z=z, A_h=0.1, S0=S0)
    assert np.array_equal(np.concatenate([o_a, o_b]), o_f) and np.array_equal(S_b, S_f)


def test_state_norm_bound():
    """With |k| = 1, beta in [0, 1] and alpha <= 1 the step matrix has
    spectral norm <= 1, so |S_t|_2 <= |S_{t-1}|_2 + beta_t |v_t|."""
    T, dk, dv = 64, 10, 10
    q, k, v, beta, z = _rand_head(T, dk, dv, RNG)
    S = RNG.standard_normal((dk, dv))
    for t in range(T):
        _, Sn = R.kda_recurrent(q[t:t + 1], k[t:t + 1], v[t:t + 1], beta[t:t + 1], z=z[t:t + 1], S0=S)
        assert np.linalg.norm(Sn, 2) <= np.linalg.norm(S, 2) + beta[t] * np.linalg.norm(v[t]) + 1e-12
        S = Sn


def test_c_oracle_matches_numpy_oracle():
    wl = WORKLOADS["tiny"]
    x = gen_inputs(wl)
    g = RNG.standard_normal(x["v"].shape).astype(np.float32)
    S0 = RNG.standard_normal((wl.B, wl.H, wl.D, wl.D)) * 0.1
    ref = R.kda_forward_heads(x["q"], x["k"], x["v"], x["beta"], x["z"], x["A"], S0=S0, gate=g)
    c = oracle.forward_c(x["q"], x["k"], x["v"], x["beta"], x["z"], x["A"], S0=S0, gate=g)
    for key in ("o", "y", "S_T"):
        np.testing.assert_allclose(c[key], ref[key], rtol=1e-12, atol=1e-13)


def test_c_oracle_bf16_inputs_and_head_subset():
    """The C oracle on a head subset equals the same heads of a full run."""
    wl = WORKLOADS["decode"]
    full = gen_inputs(wl, batch=(0, 2), time=(0, 8), heads=(0, 6))
    part = gen_inputs(wl, batch=(0, 2), time=(0, 8), heads=(2, 3))
    for key in ("q", "k", "v", "z", "gate"):
        assert np.array_equal(full[key][:, :, 2:5], part[key])
    a = oracle.forward_c(full["q"], full["k"], full["v"], full["beta"], full["z"], full["A"], S0=full["S0"],
                         gate=full["gate"])
    b = oracle.forward_c(part["q"], part["k"], part["v"], part["beta"], part["z"], part["A"], S0=part["S0"],
                         gate=part["gate"])
    assert np.array_equal(a["o"][:, :, 2:5], b["o"]) and np.array_equal(a["S_T"][:, 2:5], b["S_T"])


# ---- input steps before the core (section 2.1: ShortConv, Swish, Sigmoid) ----

def test_swish_and_sigmoid_values():
    # Sigmoid(0) = 1/2, Sigmoid(ln 3) = 3/4 exactly; Swish(x) = x Sigmoid(x)
    assert R.sigmoid(np.array([0.0]))[0] == 0.5
    assert abs(R.sigmoid(np.array([math.log(3.0)]))[0] - 0.75) < 1e-15
    assert R.swish(np.array([0.0]))[0] == 0.0
    assert abs(R.swish(np.array([math.log(3.0)]))[0] - 0.75 * math.log(3.0)) < 1e-15
    # Swish(-x) = Swish(x) - x (Sigmoid(-x) = 1 - Sigmoid(x)); limits
    x = np.linspace(-6, 6, 25)
    assert np.allclose(R.swish(-x), R.swish(x) - x, atol=1e-14)
    assert abs(R.swish(np.array([40.0]))[0] - 40.0) < 1e-12 and abs(R.swish(np.array([-40.0]))[0]) < 1e-12


def test_short_conv_is_causal_convolution():
    """Against numpy's convolution (an independent routine): y[t] =
    sum_m h[m] x[t - m] with h[m] = w[W - 1 - m] and zeros before token 0."""
    rng = np.random.default_rng(3)
    T, C, W = 37, 5, 4
    x = rng.standard_normal((T, C))
    w = rng.standard_normal((C, W))
    y, st = R.short_conv(x, w)
    for c in range(C):
        ref = np.convolve(x[:, c], w[c, ::-1])[:T]
        assert np.allclose(y[:, c], ref, atol=1e-13)
    assert np.array_equal(st, x[T - (W - 1):])          # last W-1 inputs, oldest first


def test_short_conv_tap_direction_and_state():
    """The last tap multiplies the current token; the first tap the token
    W-1 steps back, which before token 0 comes from the state (oldest first)."""
    T, C, W = 6, 2, 4
    x = np.arange(1.0, T * C + 1).reshape(T, C)
    state = -np.arange(1.0, (W - 1) * C + 1).reshape(W - 1, C)     # times -3, -2, -1
    cur = np.zeros((C, W)); cur[:, W - 1] = 1.0
    first = np.zeros((C, W)); first[:, 0] = 1.0
    y, _ = R.short_conv(x, cur, state)
    assert np.array_equal(y, x)
    y, _ = R.short_conv(x, first, state)
    assert np.array_equal(y[:W - 1], state) and np.array_equal(y[W - 1:], x[:T - (W - 1)])
    y, _ = R.short_conv(x, first)                                   # no state: zeros
    assert np.array_equal(y[:W - 1], np.zeros((W - 1, C)))
    # a sequence shorter than the window: the new state mixes old state and inputs
    _, st = R.short_conv(x[:1], first, state)
    assert np.array_equal(st, np.concatenate([state[1:], x[:1]]))


def test_input_prep_chains_through_its_state():
    """Running T tokens at once equals running them in two calls with the
    state carried (the decode / prefix-resume contract)."""
    rng = np.random.default_rng(4)
    B, T, H, d, W = 2, 23, 2, 4, 4
    xs = [rng.standard_normal((B, T, H, d)) for _ in range(3)]
    bl = rng.standard_normal((B, T, H))
    ws = [rng.standard_normal((H * d, W)) for _ in range(3)]
    full = R.input_prep(*xs, bl, *ws)
    a = R.input_prep(*(x[:, :9] for x in xs), bl[:, :9], *ws)
    b = R.input_prep(*(x[:, 9:] for x in xs), bl[:, 9:], *ws, state=a["state"])
    for n in ("q", "k", "v", "beta"):
        assert np.allclose(np.concatenate([a[n], b[n]], axis=1), full[n], atol=1e-14), n
    assert np.array_equal(b["state"], full["state"])
    # the output is Swish of the convolution, per stream
    y, _ = R.short_conv(xs[1][0].reshape(T, H * d), ws[1])
    assert np.allclose(full["k"][0].reshape(T, H * d), y / (1.0 + np.exp(-y)), atol=1e-14)


# ---- Kimi Linear decay map (the one K3's section 2.2 replaces) ----

def test_softplus_decay_values():
    # Softplus(0) = ln 2, so g(0) = -ln 2 and alpha = 1/2 exactly at A = 0
    assert abs(R.decay_log_softplus(np.array([0.0]), 0.0)[0] + math.log(2.0)) < 1e-15
    assert abs(R.decay_log_softplus(np.array([0.0]), math.log(3.0))[0] + 3.0 * math.log(2.0)) < 1e-14
    # unbounded below, close to -z e^A for large z; close to -e^{z + A} for very negative z
    assert abs(R.decay_log_softplus(np.array([60.0]), 0.0)[0] + 60.0) < 1e-12
    assert abs(R.decay_log_softplus(np.array([-30.0]), 0.5)[0] + math.exp(-30.0 + 0.5)) < 1e-25
    assert np.all(R.decay_log_softplus(np.linspace(-20, 20, 41), -0.3) < 0)


def test_softplus_decay_halves_the_state():
    """beta = 0 and z = 0, A = 0: every step multiplies the state by exactly
    1/2 (powers of two are exact in fp64), for the numpy and the C oracle."""
    rng = np.random.default_rng(8)
    T, d = 7, 4
    q, k, v = rng.standard_normal((T, d)), rng.standard_normal((T, d)), rng.standard_normal((T, d))
    S0 = rng.standard_normal((d, d))
    o, S = R.kda_recurrent(q, k, v, np.zeros(T), z=np.zeros((T, d)), A_h=0.0, S0=S0, decay="softplus")
    assert np.array_equal(S, S0 * 2.0 ** -T)
    qn = q / np.sqrt((q * q).sum(1, keepdims=True) + 1e-6)
    assert np.allclose(o, np.stack([(S0 * 2.0 ** -(t + 1)).T @ qn[t] for t in range(T)]), atol=1e-15)
    f32 = lambda a: a.astype(np.float32)[None, :, None]
    rc = oracle.forward_c(f32(q), f32(k), f32(v), np.zeros((1, T, 1), np.float32), np.zeros((1, T, 1, d), np.float32),
                          np.zeros(1, np.float32), S0=S0[None, None], decay="softplus")
    assert np.array_equal(rc["S_T"][0, 0], S0 * 2.0 ** -T)


def test_c_oracle_softplus_matches_numpy():
    rng = np.random.default_rng(9)
    T, d, H = 40, 8, 2
    q, k, v = (rng.standard_normal((1, T, H, d)).astype(np.float32) for _ in range(3))
    z = rng.standard_normal((1, T, H, d)).astype(np.float32) * 3
    beta = (1 / (1 + np.exp(-rng.standard_normal((1, T, H))))).astype(np.float32)
    A = np.array([0.4, -0.7], np.float32)
    rc = oracle.forward_c(q, k, v, beta, z, A, decay="softplus")
    for h in range(H):
        o, S = R.kda_recurrent(q[0, :, h], k[0, :, h], v[0, :, h], beta[0, :, h], z=z[0, :, h], A_h=A[h],
                               decay="softplus")
        assert np.allclose(rc["o"][0, :, h], o, atol=1e-12) and np.allclose(rc["S_T"][0, h], S, atol=1e-12)


# ---- the C oracle's optional branches: RMSNorm weight, q scale, L2Norm off ----

def _c_and_numpy(x, S0, g, **kw):
    c = oracle.forward_c(x["q"], x["k"], x["v"], x["beta"], x["z"], x["A"], S0=S0, gate=g, **kw)
    ref = R.kda_forward_heads(x["q"], x["k"], x["v"], x["beta"], x["z"], x["A"], S0=S0, gate=g,
                              **{k: v for k, v in kw.items() if k in ("w", "scale", "l2norm")})
    return c, ref


@pytest.mark.parametrize("scale,l2norm", [(0.37, True), (1.0, False), (2.5, False)])
def test_c_oracle_options_match_numpy_oracle(scale, l2norm):
    """Section 2.1 (L2Norm on q, k; q scale, reading R5) and section 2.3 (RMSNorm
    weight): the C twin takes the same branches as the numpy oracle."""
    wl = WORKLOADS["tiny"]
    x = gen_inputs(wl)
    rng = np.random.default_rng(77)
    if not l2norm:  # rows of norm in [0.5, 1] so that the recurrence stays bounded without L2Norm
        for key in ("q", "k"):
            x[key] = (x[key] * rng.uniform(0.5, 1.0, x[key].shape[:3] + (1,))).astype(np.float32)
    g = rng.standard_normal(x["v"].shape).astype(np.float32)
    w = rng.uniform(0.25, 2.0, (wl.H, wl.D)).astype(np.float32)
    S0 = rng.standard_normal((wl.B, wl.H, wl.D, wl.D)) * 0.1
    c, ref = _c_and_numpy(x, S0, g, w=w, scale=scale, l2norm=l2norm)
    for key in ("o", "y", "S_T"):
        np.testing.assert_allclose(c[key], ref[key], rtol=1e-11, atol=1e-12)


def test_q_scale_is_linear_in_the_output():
    """o_t = S_t^T (scale q_t) (section 2.1): o scales with the query scale and
    the state does not see it, in both oracles."""
    wl = WORKLOADS["tiny"]
    x = gen_inputs(wl)
    S0 = np.random.default_rng(5).standard_normal((wl.B, wl.H, wl.D, wl.D)) * 0.1
    for fwd in (lambda **kw: oracle.forward_c(x["q"], x["k"], x["v"], x["beta"], x["z"], x["A"], S0=S0, **kw),
                lambda **kw: R.kda_forward_heads(x["q"], x["k"], x["v"], x["beta"], x["z"], x["A"], S0=S0, **kw)):
        a, b = fwd(scale=1.0), fwd(scale=0.125)
        np.testing.assert_allclose(b["o"], 0.125 * a["o"], rtol=1e-13, atol=1e-15)
        np.testing.assert_array_equal(a["S_T"], b["S_T"])


def test_l2norm_off_on_prenormalised_rows_equals_l2norm_on():
    """Section 2.1 puts L2Norm on q and k inside the layer: switching it off and
    feeding rows already divided by sqrt(|x|^2 + eps) (done here with plain
    numpy) gives the same result, in both oracles."""
    rng = np.random.default_rng(9)
    B, T, H, D = 1, 40, 2, 16
    q = rng.standard_normal((B, T, H, D)) * rng.uniform(0.2, 5.0, (B, T, H, 1))
    k = rng.standard_normal((B, T, H, D)) * rng.uniform(0.2, 5.0, (B, T, H, 1))
    v = rng.standard_normal((B, T, H, D))
    beta = rng.uniform(0.1, 0.9, (B, T, H))
    z = rng.standard_normal((B, T, H, D))
    A = rng.uniform(-1, 1, H)
    qn = q / np.sqrt((q * q).sum(-1, keepdims=True) + 1e-6)
    kn = k / np.sqrt((k * k).sum(-1, keepdims=True) + 1e-6)
    f32 = lambda a: a.astype(np.float32)
    # the C oracle reads fp32: round the inputs once and normalise the rounded values
    q32, k32 = f32(q), f32(k)
    qn32 = q32 / np.sqrt((q32.astype(np.float64) ** 2).sum(-1, keepdims=True) + 1e-6)
    kn32 = k32 / np.sqrt((k32.astype(np.float64) ** 2).sum(-1, keepdims=True) + 1e-6)
    on = R.kda_forward_heads(q, k, v, beta, z, A)
    off = R.kda_forward_heads(qn, kn, v, beta, z, A, l2norm=False)
    for key in ("o", "S_T"):
        np.testing.assert_allclose(off[key], on[key], rtol=1e-12, atol=1e-13)
    con = oracle.forward_c(q32, k32, f32(v), f32(beta), f32(z), f32(A))
    # fp32 inputs of the normalised rows lose ~1e-8 relative; the check allows that
    coff = oracle.forward_c(f32(qn32), f32(kn32), f32(v), f32(beta), f32(z), f32(A), l2norm=False)
    for key in ("o", "S_T"):
        np.testing.assert_allclose(coff[key], con[key], rtol=0, atol=1e-6 * np.abs(con[key]).max())
    # and without normalisation the result really differs (the branch is taken)
    raw = oracle.forward_c(q32, k32, f32(v), f32(beta), f32(z), f32(A), l2norm=False)
    assert np.abs(raw["o"] - con["o"]).max() > 1e-2


def test_c_oracle_rms_weight_scales_each_channel():
    """Section 2.3 with a per-(head, channel) RMSNorm weight [H, d_v]: y(w) =
    y(1) * w channel by channel, per head (C oracle)."""
    wl = WORKLOADS["tiny"]
    x = gen_inputs(wl)
    rng = np.random.default_rng(13)
    g = rng.standard_normal(x["v"].shape).astype(np.float32)
    w = rng.uniform(0.25, 2.0, (wl.H, wl.D)).astype(np.float32)
    a = oracle.forward_c(x["q"], x["k"], x["v"], x["beta"], x["z"], x["A"], gate=g)
    b = oracle.forward_c(x["q"], x["k"], x["v"], x["beta"], x["z"], x["A"], gate=g, w=w)
    np.testing.assert_allclose(b["y"], a["y"] * w.astype(np.float64)[None, None], rtol=1e-14, atol=1e-300)
    np.testing.assert_array_equal(a["o"], b["o"])
