"""KDA oracle: plain, slow, fp64 CPU reference of what the KDA forward computes.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  It shares no code with the GPU
library and the GPU library never calls it.

Source pages: "Kimi K3: KDA, Attention Residuals and Stable LatentMoE"
(hs-black.github.io/posts/kimi-k3), section 2.1 (the per-head recurrence, the
chunked output formula and the input steps ShortConv / Swish / Sigmoid before
the core), section 2.2 (the bounded decay map and the
16-token sub-tile bound), section 2.3 (the full-rank output gate) and section
10.2 (the (M, S~) pair composition used for context parallelism).

Conventions (single head unless noted):
  q, k : [T, dk]    v : [T, dv]    beta : [T]    z : [T, dk]    A : scalar
  S    : [dk, dv]   (row index = key channel; o_t = S_t^T q_t)
Readings where the pages leave a step open are listed in each docstring.

Parity pins: every function here is pinned by tests/test_oracle_pins.py
against closed forms, exact rational arithmetic or the pages' own numbers.
"""
from __future__ import annotations

import numpy as np

G_MIN = -5.0
L2_EPS = 1e-6
RMS_EPS = 1e-6


def sigmoid(x):
    """Numerically stable logistic function in fp64."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def decay_log(z, A_h, g_min: float = G_MIN):
    """K3 bounded log-decay (section 2.2): g = g_min * Sigmoid(e^{A_h} z),
    which lies in (g_min, 0); the per-channel retention is alpha = e^g."""
    return g_min * sigmoid(np.exp(np.float64(A_h)) * np.asarray(z, dtype=np.float64))


def decay_log_softplus(z, A_h):
    """Kimi Linear's log-decay map, the one section 2.2 replaces:
    g = -e^{A_h} Softplus(z), unbounded below (Softplus(z) = log(1 + e^z))."""
    z = np.asarray(z, dtype=np.float64)
    return -np.exp(np.float64(A_h)) * np.logaddexp(0.0, z)


def l2_normalize(x, eps: float = L2_EPS):
    """Per-row L2 normalisation (section 2.1 applies L2Norm to q and k).
    Reading: eps is added under the square root, x / sqrt(sum x^2 + eps)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def _prep(q, k, l2norm, eps, scale):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    if l2norm:
        q = l2_normalize(q, eps)
        k = l2_normalize(k, eps)
    return q * scale, k


def kda_recurrent(q, k, v, beta, z=None, A_h=0.0, g=None, S0=None, g_min=G_MIN,
                  l2norm=True, l2_eps=L2_EPS, scale=1.0, literal=False, decay="k3"):
    """Token-by-token KDA recurrence of section 2.1, single head, fp64:

        S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
        o_t = S_t^T q_t

    alpha_t = e^{g_t} with g_t from ``decay_log(z_t, A_h)`` (``decay`` "k3")
    or ``decay_log_softplus(z_t, A_h)`` ("softplus", the Kimi Linear map),
    unless the log decay ``g`` ([T, dk]) is given directly (tests only).

    ``literal=True`` forms the d_k x d_k matrix (I - beta k k^T) Diag(alpha)
    and multiplies, exactly as printed.  The default applies the same step
    in rank-1 form: S <- Diag(alpha) S, then S <- S + beta k (v - S^T k)^T.

    Readings: o_t reads the state after the write of token t; the state is
    d_k x d_v with the key channel as row index; q is multiplied by
    ``scale`` (1 by default: the pages show no scaling) after L2Norm.

    Returns (o [T, dv], S_T [dk, dv]).
    """
    q, k = _prep(q, k, l2norm, l2_eps, scale)
    v = np.asarray(v, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64).reshape(-1)
    T, dk = k.shape
    dv = v.shape[1]
    if g is None:
        g = decay_log(z, A_h, g_min) if decay == "k3" else decay_log_softplus(z, A_h)
    g = np.asarray(g, dtype=np.float64)
    alpha = np.exp(g)
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64, copy=True)
    o = np.empty((T, dv))
    eye = np.eye(dk)
    for t in range(T):
        kt = k[t]
        if literal:
            M = (eye - beta[t] * np.outer(kt, kt)) @ np.diag(alpha[t])
            S = M @ S + beta[t] * np.outer(kt, v[t])
        else:
            S = alpha[t][:, None] * S
            S = S + beta[t] * np.outer(kt, v[t] - S.T @ kt)
        o[t] = S.T @ q[t]
    return o, S


def kda_chunked(q, k, v, beta, z=None, A_h=0.0, g=None, S0=None, g_min=G_MIN,
                l2norm=True, l2_eps=L2_EPS, scale=1.0, chunk=64):
    """Chunked form of the same recurrence, fp64 (section 2.1's block output
    formula O = (Gamma . Q) S + Tril[(Q . Gamma)(K / Gamma)^T](U - W S)).

    The pages defer U and W to the Kimi Linear paper; this is the reading
    derived from the recurrence itself.  Within a chunk with entry state S,
    G = inclusive cumulative sum of g over the chunk's tokens (per channel),
    Gamma = e^G, and
        L  = StrictTril(Diag(beta) (K . Gamma)(K / Gamma)^T)
        Tm = (I + L)^{-1}
        W  = Tm Diag(beta) (K . Gamma),   U = Tm Diag(beta) V
        U' = U - W S
        O  = (Q . Gamma) S + Tril[(Q . Gamma)(K / Gamma)^T] U'
        S  <- Diag(Gamma_last) S + (K . (Gamma_last / Gamma))^T U'
    Tril keeps the diagonal (o_t sees the write of token t); the UT system
    uses the strict part.  Decays are anchored at the chunk start, which is
    safe in fp64 for chunk * |g_min| < 700.  The last chunk may be short.
    """
    q, k = _prep(q, k, l2norm, l2_eps, scale)
    v = np.asarray(v, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64).reshape(-1)
    T, dk = k.shape
    dv = v.shape[1]
    if g is None:
        g = decay_log(z, A_h, g_min)
    g = np.asarray(g, dtype=np.float64)
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64, copy=True)
    o = np.empty((T, dv))
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        n = c1 - c0
        Qc, Kc, Vc, bc = q[c0:c1], k[c0:c1], v[c0:c1], beta[c0:c1]
        G = np.cumsum(g[c0:c1], axis=0)
        Gam = np.exp(G)
        Kf, Kb, Qf = Kc * Gam, Kc / Gam, Qc * Gam
        L = np.tril(bc[:, None] * (Kf @ Kb.T), -1)
        Tm = np.linalg.inv(np.eye(n) + L)
        W = Tm @ (bc[:, None] * Kf)
        U = Tm @ (bc[:, None] * Vc)
        Up = U - W @ S
        Aqk = np.tril(Qf @ Kb.T)
        o[c0:c1] = Qf @ S + Aqk @ Up
        S = Gam[-1][:, None] * S + (Kc * (Gam[-1] / Gam)).T @ Up
    return o, S


def output_gate(o, gate_logit, w=None, eps: float = RMS_EPS):
    """Output gate of section 2.3 without the projections:
    y = Sigmoid(gate_logit) * RMSNorm(o).  Reading: RMSNorm over the d_v
    channels of one head and token, eps added to the mean square, optional
    per-channel weight w (1 when absent)."""
    o = np.asarray(o, dtype=np.float64)
    r = o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    if w is not None:
        r = r * np.asarray(w, dtype=np.float64)
    return sigmoid(gate_logit) * r


def step_matrix(k_t, beta_t, alpha_t):
    """M_t = (I - beta_t k_t k_t^T) Diag(alpha_t), the d_k x d_k transfer of
    one token (section 10.2)."""
    k_t = np.asarray(k_t, dtype=np.float64)
    return (np.eye(k_t.size) - beta_t * np.outer(k_t, k_t)) @ np.diag(np.asarray(alpha_t, dtype=np.float64))


def segment_pair(q, k, v, beta, z=None, A_h=0.0, g=None, g_min=G_MIN, l2norm=True,
                 l2_eps=L2_EPS):
    """(M, S~) of a segment (section 10.2): M = M_T ... M_1 and S~ the state
    reached from S = 0."""
    _, kk = _prep(q, k, l2norm, l2_eps, 1.0)
    if g is None:
        g = decay_log(z, A_h, g_min)
    alpha = np.exp(np.asarray(g, dtype=np.float64))
    beta = np.asarray(beta, dtype=np.float64).reshape(-1)
    M = np.eye(kk.shape[1])
    for t in range(kk.shape[0]):
        M = step_matrix(kk[t], beta[t], alpha[t]) @ M
    _, St = kda_recurrent(q, k, v, beta, z=z, A_h=A_h, g=g, S0=None, g_min=g_min,
                          l2norm=l2norm, l2_eps=l2_eps)
    return M, St


def compose(p2, p1):
    """(M2, S2) o (M1, S1) = (M2 M1, S2 + M2 S1): apply segment 1, then 2."""
    M2, S2 = p2
    M1, S1 = p1
    return M2 @ M1, S2 + M2 @ S1


def kda_forward_heads(q, k, v, beta, z, A, S0=None, gate=None, w=None, g_min=G_MIN,
                      l2norm=True, l2_eps=L2_EPS, rms_eps=RMS_EPS, scale=1.0):
    """Multi-head, multi-batch driver: q, k, z: [B, T, H, dk]; v, gate:
    [B, T, H, dv]; beta [B, T, H]; A [H]; S0 [B, H, dk, dv] or None.
    Returns dict with o [B, T, H, dv], S_T [B, H, dk, dv] and y if gated."""
    q = np.asarray(q, dtype=np.float64)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.empty((B, T, H, dv))
    ST = np.empty((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            s0 = None if S0 is None else S0[b, h]
            o[b, :, h], ST[b, h] = kda_recurrent(q[b, :, h], k[b, :, h], v[b, :, h], beta[b, :, h],
                                                 z=z[b, :, h], A_h=A[h], S0=s0, g_min=g_min,
                                                 l2norm=l2norm, l2_eps=l2_eps, scale=scale)
    out = {"o": o, "S_T": ST}
    if gate is not None:
        wh = None if w is None else np.asarray(w)[None, None]
        out["y"] = output_gate(o, gate, wh, rms_eps)
    return out


def swish(x):
    """Swish(x) = x * Sigmoid(x), applied after ShortConv to q, k and v
    (section 2.1; section 4's SwiGLU discussion gives the same definition)."""
    x = np.asarray(x, dtype=np.float64)
    return x * sigmoid(x)


def short_conv(x, w, state=None):
    """ShortConv of section 2.1: a depthwise causal convolution over time.
    x: [T, C]; w: [C, W] taps -- w[:, W-1] multiplies the current token and
    w[:, W-1-j] the token j steps back; state: [W-1, C] inputs before token 0,
    oldest first (None: zeros).  Returns (y [T, C], new_state [W-1, C]), the
    new state being the last W-1 inputs of the extended sequence.
    Reading: the pages give neither the width nor a bias; the width is a
    parameter and there is no bias."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    T, C = x.shape
    W = w.shape[1]
    prev = np.zeros((W - 1, C)) if state is None else np.asarray(state, dtype=np.float64).reshape(W - 1, C)
    ext = np.concatenate([prev, x], axis=0)  # ext[i] = input at time i - (W - 1)
    y = np.zeros((T, C))
    for j in range(W):  # tap j meets the input at time t - (W - 1) + j
        y += w[:, j] * ext[j:j + T]
    return y, ext[T:].copy()


def input_prep(xq, xk, xv, beta_logit, wq, wk, wv, state=None):
    """The core's inputs from the projections (section 2.1):
        q = Swish(ShortConv(x_q)), k = Swish(ShortConv(x_k)),
        v = Swish(ShortConv(x_v)), beta = Sigmoid(beta_logit).
    The L2Norm of q and k belongs to the core (kda_recurrent / kda_chunked
    apply it).  xq, xk, xv: [B, T, H, d]; beta_logit: [B, T, H]; w*: [H d, W];
    state: [B, 3, W-1, H d] (q, k, v windows) or None.  Returns a dict with
    q, k, v [B, T, H, d], beta [B, T, H] and the new state [B, 3, W-1, H d]."""
    xs = [np.asarray(a, dtype=np.float64) for a in (xq, xk, xv)]
    ws = (wq, wk, wv)
    B, T, H, d = xs[0].shape
    C = H * d
    W = np.asarray(wq).shape[1]
    out = {n: np.empty((B, T, H, d)) for n in ("q", "k", "v")}
    new_state = np.empty((B, 3, W - 1, C))
    for b in range(B):
        for i, n in enumerate(("q", "k", "v")):
            st = None if state is None else np.asarray(state, dtype=np.float64)[b, i]
            y, new_state[b, i] = short_conv(xs[i][b].reshape(T, C), ws[i], st)
            out[n][b] = swish(y).reshape(T, H, d)
    out["beta"] = sigmoid(beta_logit)
    out["state"] = new_state
    return out
