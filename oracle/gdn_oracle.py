"""Plain fp64 CPU oracle for the Gated DeltaNet token mixer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: it exists so that the tests, the smoke check and the
bench's CPU-baseline leg have an obviously correct reference to compare the
HIP kernels against.  It shares no code with the HIP path.

Everything here is computed in float64 with numpy, token by token, exactly as
the method is stated:

* causal depthwise short convolution of width 4 over the concatenated q/k/v
  channels, then SiLU ("Inside Qwen3.5", section 5: the kernel-4 causal
  convolution gives cheap local mixing; the conv state is a (channels,
  width-1) buffer as in "Mamba hybrid model selection", per-request memory
  section);
* L2 normalisation of q and k per head ("Inside Qwen3.5", section 5: the
  L2-norm on q/k keeps the recurrence bounded);
* the gated delta rule ("Inside Qwen3.5", sections 4-5: the update
  S <- a*S + b*(v - S*k)*k^T with per-token, per-head a and b), read with the
  decay applied first, i.e. S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T
  and o_t = S_t q_t.  V head h reads QK head h // (H_v / H_qk);
* with erase=False, the same recurrence without the error-correcting write:
  S_t = a_t S_{t-1} + b_t v_t k_t^T, the additive linear attention of
  "Inside Qwen3.5", section 2 (S = sum v k^T, o = S q) with the decay gate of
  section 5 kept and the correction term dropped.

Readings where the pages are silent:
  * eps = 1e-6 inside the square root of the L2 norm;
  * conv tap W-1 multiplies the current token; the conv state holds the last
    W-1 inputs in chronological order (oldest first); positions before a
    sequence start read the conv state, or zero when none is given;
  * the query scale is 1 unless the caller passes another one;
  * g is log(alpha) and beta is the write strength, both given per token and
    per V head.

The *_backward functions are reverse-mode differentiation of the same
definitions, written out step by step (each forward step taken back in the
opposite order), for the training row: gradients of a scalar loss with
respect to every input, given its gradients with respect to every output.

Parity pins for every function live in tests/test_oracle_pins.py and
tests/test_oracle_backward_pins.py.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "silu",
    "l2_normalize",
    "causal_conv1d",
    "split_qkv",
    "gated_delta_rule",
    "gdn_layer",
    "layer_channels",
    "decode_step",
    "chunked_gated_delta_rule",
    "unrolled_product_form",
    "round_to_bf16",
    "ring_to_chronological",
    "l2_normalize_backward",
    "gated_delta_rule_backward",
    "causal_conv1d_backward",
]


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def _bounds(total, cu_seqlens):
    if cu_seqlens is None:
        return [0, int(total)]
    b = [int(c) for c in np.asarray(cu_seqlens).reshape(-1)]
    assert b[0] == 0 and b[-1] == total and all(x <= y for x, y in zip(b, b[1:]))
    return b


def silu(y):
    """SiLU(y) = y * sigmoid(y) = y / (1 + e^-y), applied after the conv."""
    y = _f64(y)
    return y / (1.0 + np.exp(-y))


def l2_normalize(x, eps=1e-6):
    """x / sqrt(sum(x^2) + eps) over the last axis ("Inside Qwen3.5", section 5)."""
    x = _f64(x)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def causal_conv1d(x, weight, bias=None, conv_state=None, cu_seqlens=None, activation="silu"):
    """Causal depthwise conv of width W over each packed sequence.

    x          [T, C]     packed tokens (sequences given by cu_seqlens)
    weight     [C, W]     tap W-1 multiplies the current token
    bias       [C] or None
    conv_state [N, C, W-1] inputs that precede each sequence, oldest first,
               or None for zeros
    returns (y [T, C], new_state [N, C, W-1]) where new_state holds the last
    W-1 entries of (old state ++ sequence inputs), oldest first.
    """
    x, weight, bias = _f64(x), _f64(weight), _f64(bias)
    T, C = x.shape
    W = weight.shape[1]
    b = _bounds(T, cu_seqlens)
    N = len(b) - 1
    state = np.zeros((N, C, W - 1)) if conv_state is None else _f64(conv_state).copy()
    y = np.zeros((T, C))
    new_state = np.zeros((N, C, W - 1))
    for n in range(N):
        s, e = b[n], b[n + 1]
        L = e - s
        # padded history: W-1 earlier inputs, then the sequence itself
        xp = np.concatenate([state[n].T, x[s:e]], axis=0)  # [(W-1)+L, C]
        acc = np.zeros((L, C))
        for j in range(W):
            acc += weight[:, j] * xp[j:j + L]
        if bias is not None:
            acc += bias
        y[s:e] = acc
        new_state[n] = xp[L:].T  # the last W-1 rows of the padded history
    if activation == "silu":
        y = silu(y)
    else:
        assert activation in (None, "none")
    return y, new_state


def ring_to_chronological(conv_state, conv_head):
    """The conv state of each sequence in chronological order (oldest first).

    conv_state [N, C, M] holds the last M = W-1 inputs of every channel in a
    ring of M slots; conv_head [N] is the slot of the oldest one, so the j-th
    oldest input sits in slot (head + j) mod M.  A ring is a storage layout of
    the same (channels, width - 1) conv buffer the per-request memory section
    of "Mamba hybrid model selection" describes: a decode step can overwrite
    the oldest slot and advance the head instead of moving every slot.
    """
    cs = _f64(conv_state)
    heads = np.asarray(conv_head).reshape(-1)
    N, _, M = cs.shape
    out = np.empty_like(cs)
    for n in range(N):
        h = int(heads[n]) % M
        for j in range(M):
            out[n, :, j] = cs[n, :, (h + j) % M]
    return out


def split_qkv(y, h_qk, d_k, h_v, d_v):
    """Split the concatenated channels [q | k | v] into per-head tensors."""
    T = y.shape[0]
    nq = h_qk * d_k
    q = y[:, :nq].reshape(T, h_qk, d_k)
    k = y[:, nq:2 * nq].reshape(T, h_qk, d_k)
    v = y[:, 2 * nq:2 * nq + h_v * d_v].reshape(T, h_v, d_v)
    return q, k, v


def gated_delta_rule(q, k, v, g, beta, initial_state=None, cu_seqlens=None, scale=1.0,
                     l2norm_qk=True, eps=1e-6, v_heads=None, erase=True):
    """Sequential gated delta rule, one token at a time, in fp64.

    q, k  [T, H_qk, d_k];  v [T, H_v, d_v];  g, beta [T, H_v]
    initial_state [N, H_v, d_v, d_k] or None (zeros)
    v_heads: optional subset of V heads to evaluate (results are indexed in
             that order); every V head is independent of the others.
    returns o [T, len(heads), d_v], final_state [N, len(heads), d_v, d_k]

    Per V head h with QK head h // (H_v / H_qk):
        S  <- exp(g_t) * S                      (decay: forget)
        S  <- S + beta_t * (v_t - S k_t) k_t^T   (delta write against the decayed S)
        o_t = scale * S q_t
    which equals S_t = a_t S_{t-1}(I - b_t k_t k_t^T) + b_t v_t k_t^T.
    erase=False drops the S k_t term: S_t = a_t S_{t-1} + b_t v_t k_t^T.
    """
    q, k, v, g, beta = _f64(q), _f64(k), _f64(v), _f64(g), _f64(beta)
    T, h_qk, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    assert h_v % h_qk == 0
    grp = h_v // h_qk
    heads = np.arange(h_v) if v_heads is None else np.asarray(v_heads, dtype=np.int64)
    qk_of = heads // grp
    if l2norm_qk:
        q = l2_normalize(q, eps)
        k = l2_normalize(k, eps)
    b = _bounds(T, cu_seqlens)
    N = len(b) - 1
    H = len(heads)
    S_all = np.zeros((N, H, d_v, d_k))
    if initial_state is not None:
        S_all[:] = _f64(initial_state)[:, heads]
    o = np.zeros((T, H, d_v))
    for n in range(N):
        S = S_all[n].copy()
        for t in range(b[n], b[n + 1]):
            kt = k[t, qk_of]                      # [H, d_k]
            qt = q[t, qk_of]                      # [H, d_k]
            S = np.exp(g[t, heads])[:, None, None] * S
            pred = np.matmul(S, kt[:, :, None])[:, :, 0] if erase else 0.0  # S k   [H, d_v]
            err = beta[t, heads][:, None] * (v[t, heads] - pred)  # b (v - S k)
            S = S + err[:, :, None] * kt[:, None, :]
            o[t] = scale * np.matmul(S, qt[:, :, None])[:, :, 0]
        S_all[n] = S
    return o, S_all


def layer_channels(h_qk, d_k, h_v, d_v, v_heads=None):
    """Indices of the conv channels that the given V heads read, ordered
    [q of their QK heads | k of their QK heads | v of the heads]."""
    grp = h_v // h_qk
    heads = np.arange(h_v) if v_heads is None else np.asarray(v_heads, dtype=np.int64)
    qks = np.unique(heads // grp)
    nq = h_qk * d_k
    return np.concatenate([
        (qks[:, None] * d_k + np.arange(d_k)).reshape(-1),
        nq + (qks[:, None] * d_k + np.arange(d_k)).reshape(-1),
        2 * nq + (heads[:, None] * d_v + np.arange(d_v)).reshape(-1),
    ])


def gdn_layer(x, conv_weight, g, beta, h_qk, d_k, h_v, d_v, conv_bias=None, conv_state=None,
              initial_state=None, cu_seqlens=None, scale=1.0, activation="silu", l2norm_qk=True,
              v_heads=None, x_is_selected=False, erase=True):
    """The whole token mixer for packed sequences: conv(+SiLU) -> split -> recurrence.

    With v_heads given, only the channels those heads read are convolved (the
    conv is depthwise, so each channel is independent); x_is_selected=True
    means x, conv_weight, conv_bias and conv_state already hold just those
    channels, in layer_channels() order.
    returns o, final_state, new_conv_state (the latter over the channels used,
    [N, C_used, W-1], in layer_channels() order).
    """
    grp = h_v // h_qk
    heads = np.arange(h_v) if v_heads is None else np.asarray(v_heads, dtype=np.int64)
    qks = np.unique(heads // grp)
    ch = slice(None) if x_is_selected else layer_channels(h_qk, d_k, h_v, d_v, v_heads)
    x = _f64(x)[:, ch]
    cs = None if conv_state is None else _f64(conv_state)[:, ch]
    bias = None if conv_bias is None else _f64(conv_bias)[ch]
    y, new_cs = causal_conv1d(x, _f64(conv_weight)[ch], bias, cs, cu_seqlens, activation)
    nqs = len(qks) * d_k
    q = y[:, :nqs].reshape(-1, len(qks), d_k)
    k = y[:, nqs:2 * nqs].reshape(-1, len(qks), d_k)
    vv = y[:, 2 * nqs:].reshape(-1, len(heads), d_v)
    # re-index: local V head i reads the local slot of QK head heads[i] // grp
    local_qk = np.searchsorted(qks, heads // grp)
    qh = q[:, local_qk]
    kh = k[:, local_qk]
    gh = _f64(g)[:, heads]
    bh = _f64(beta)[:, heads]
    s0 = None if initial_state is None else _f64(initial_state)[:, heads]
    # one QK slot per V head (explicitly repeated), so the grouping is trivial
    o, S = gated_delta_rule(qh, kh, vv, gh, bh, s0, cu_seqlens, scale, l2norm_qk, erase=erase)
    return o, S, new_cs


def decode_step(x, conv_weight, g, beta, state, conv_state, h_qk, d_k, h_v, d_v, conv_bias=None,
                scale=1.0, activation="silu", l2norm_qk=True, round_state_bf16=False, erase=True):
    """One new token for each of N independent sequences.

    x [N, C] pre-conv inputs; conv_state [N, C, W-1]; state [N, H_v, d_v, d_k];
    g, beta [N, H_v].  conv_weight None means q|k|v arrive already mixed (no
    conv, no activation).  Returns (o [N, H_v, d_v], new_state, new_conv_state).
    This is the same recurrence as gated_delta_rule applied to a length-1
    sequence per request ("Inside Qwen3.5", section 8: decode is a
    read-modify-write of the fixed-size state every token).
    round_state_bf16 is a diagnostic that rounds the new state to bf16.
    """
    x = _f64(x)
    N = x.shape[0]
    cu = np.arange(N + 1)
    if conv_weight is None:
        y, new_cs = x, None if conv_state is None else _f64(conv_state).copy()
    else:
        y, new_cs = causal_conv1d(x, conv_weight, conv_bias, conv_state, cu, activation)
    q, k, v = split_qkv(y, h_qk, d_k, h_v, d_v)
    o, S = gated_delta_rule(q, k, v, g, beta, state, cu, scale, l2norm_qk, erase=erase)
    if round_state_bf16:
        S = round_to_bf16(S)
    return o, S, new_cs


def chunked_gated_delta_rule(q, k, v, g, beta, initial_state, chunk, scale=1.0, l2norm_qk=True,
                             eps=1e-6, erase=True):
    """The chunked (WY / UT-transform) rearrangement of the same recurrence, fp64.

    Used only to pin the algebra of the chunked prefill in tests; it is never
    the reference a kernel is compared against.  Single sequence.  Within a
    chunk with cumulative log-decay G_r = sum_{i<=r} g_i and gamma_r = e^{G_r}:
        A   = strict_lower(beta_r e^{G_r-G_j} k_r.k_j),  Tm = (I + A)^-1
        U   = Tm diag(beta) (V - diag(gamma) K S^T)
        O   = diag(gamma) Q S^T + (lower_incl(e^{G_r-G_j}) * Q K^T) U
        S'  = gamma_last S + U^T diag(e^{G_last - G}) K
    With erase=False there is no correction: A = 0 (Tm = I) and U = diag(beta) V.
    """
    q, k, v, g, beta = _f64(q), _f64(k), _f64(v), _f64(g), _f64(beta)
    T, h_qk, d_k = q.shape
    h_v, d_v = v.shape[1:]
    grp = h_v // h_qk
    if l2norm_qk:
        q = l2_normalize(q, eps)
        k = l2_normalize(k, eps)
    S_all = np.zeros((h_v, d_v, d_k)) if initial_state is None else _f64(initial_state).reshape(h_v, d_v, d_k).copy()
    o = np.zeros((T, h_v, d_v))
    for h in range(h_v):
        hq = h // grp
        S = S_all[h]
        for c0 in range(0, T, chunk):
            c1 = min(c0 + chunk, T)
            n = c1 - c0
            K, Q, V = k[c0:c1, hq], q[c0:c1, hq], v[c0:c1, h]
            b = beta[c0:c1, h]
            G = np.cumsum(g[c0:c1, h])
            gam = np.exp(G)
            incl = np.tril(np.ones((n, n), dtype=bool))
            D = np.where(incl, G[:, None] - G[None, :], 0.0)
            Gam = np.where(incl, np.exp(D), 0.0)
            if erase:
                A = np.tril(b[:, None] * Gam * (K @ K.T), -1)
                Tm = np.linalg.inv(np.eye(n) + A)
                U = Tm @ (b[:, None] * (V - gam[:, None] * (K @ S.T)))
            else:
                U = b[:, None] * V
            o[c0:c1, h] = scale * (gam[:, None] * (Q @ S.T) + (Gam * (Q @ K.T)) @ U)
            S = gam[-1] * S + (U * np.exp(G[-1] - G)[:, None]).T @ K
        S_all[h] = S
    return o, S_all


def unrolled_product_form(k, v, g, beta, S0):
    """S_T = S_0 A_1...A_T + sum_s beta_s v_s k_s^T A_{s+1}...A_T with
    A_t = alpha_t (I - beta_t k_t k_t^T) formed explicitly.  Single head,
    k already normalised; tiny T only."""
    k, v, g, beta, S0 = _f64(k), _f64(v), _f64(g), _f64(beta), _f64(S0)
    T, d_k = k.shape
    A = [np.exp(g[t]) * (np.eye(d_k) - beta[t] * np.outer(k[t], k[t])) for t in range(T)]

    def prod(lo):  # A_lo ... A_{T-1}
        P = np.eye(d_k)
        for t in range(lo, T):
            P = P @ A[t]
        return P

    S = S0 @ prod(0)
    for s in range(T):
        S = S + beta[s] * np.outer(v[s], k[s]) @ prod(s + 1)
    return S


def round_to_bf16(a):
    """Round to the nearest bfloat16 value, ties to even (via float32 bits)."""
    a32 = np.asarray(a, dtype=np.float32)
    u = a32.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


# ------------------------------------------------------------------ backward

def l2_normalize_backward(x, d_xhat, eps=1e-6):
    """Gradient through xhat = x / n, n = sqrt(sum(x^2) + eps), over the last
    axis: dx = d_xhat / n - x (x . d_xhat) / n^3."""
    x, d_xhat = _f64(x), _f64(d_xhat)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)
    return d_xhat / n - x * np.sum(x * d_xhat, axis=-1, keepdims=True) / n ** 3


def gated_delta_rule_backward(q, k, v, g, beta, d_o, initial_state=None, d_final_state=None,
                              cu_seqlens=None, scale=1.0, l2norm_qk=True, eps=1e-6, erase=True,
                              segment=16):
    """Reverse-mode gradients of gated_delta_rule, token by token, in fp64.

    Inputs as gated_delta_rule, plus d_o [T, H_v, d_v] (gradient of the loss
    with respect to o) and d_final_state [N, H_v, d_v, d_k] or None (zero).
    Returns dq, dk [T, H_qk, d_k], dv [T, H_v, d_v], dg, dbeta [T, H_v],
    d_initial_state [N, H_v, d_v, d_k].

    Each token's forward step, per V head with a = e^{g_t}:
        Sd = a S_prev;  p = Sd k;  e = b (v - p);  S = Sd + e k^T;  o = scale S q
    is taken back in the opposite order, with dS the gradient of S:
        dS += scale do q^T;           dq = scale S^T do
        de = dS k;  dk = dS^T e;      dSd = dS
        dv = b de;  db = (v - p).de;  dp = -b de
        dSd += dp k^T;                dk += Sd^T dp
        da = <dSd, S_prev>;  dg = a da;  dS_prev = a dSd
    (without erase, p = 0 and its two lines drop out).  The gradients of a QK
    head add up over the V heads that read it, then pass through the L2 norm.
    The states S_prev are recomputed from checkpoints every `segment` tokens.
    """
    q, k, v, g, beta, d_o = _f64(q), _f64(k), _f64(v), _f64(g), _f64(beta), _f64(d_o)
    T, h_qk, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    grp = h_v // h_qk
    qk_of = np.arange(h_v) // grp
    qn, kn = (l2_normalize(q, eps), l2_normalize(k, eps)) if l2norm_qk else (q, k)
    b = _bounds(T, cu_seqlens)
    N = len(b) - 1
    S0 = np.zeros((N, h_v, d_v, d_k)) if initial_state is None else _f64(initial_state).copy()
    dSf = np.zeros((N, h_v, d_v, d_k)) if d_final_state is None else _f64(d_final_state)
    dqn = np.zeros((T, h_v, d_k))
    dkn = np.zeros((T, h_v, d_k))
    dv = np.zeros((T, h_v, d_v))
    dg = np.zeros((T, h_v))
    db = np.zeros((T, h_v))
    dS0 = np.zeros((N, h_v, d_v, d_k))

    def step(S, t):
        kt, a = kn[t, qk_of], np.exp(g[t])[:, None, None]
        Sd = a * S
        p = np.matmul(Sd, kt[:, :, None])[:, :, 0] if erase else np.zeros((h_v, d_v))
        e = beta[t][:, None] * (v[t] - p)
        return Sd, p, e, Sd + e[:, :, None] * kt[:, None, :]

    for n in range(N):
        s0, s1 = b[n], b[n + 1]
        # forward sweep: the state before each segment's first token
        starts = list(range(s0, s1, segment))
        ckpt = []
        S = S0[n].copy()
        for st in starts:
            ckpt.append(S.copy())
            for t in range(st, min(st + segment, s1)):
                S = step(S, t)[3]
        dS = dSf[n].copy()
        for st, Sst in reversed(list(zip(starts, ckpt))):
            prev = [Sst]
            for t in range(st, min(st + segment, s1)):
                prev.append(step(prev[-1], t)[3])
            for t in reversed(range(st, min(st + segment, s1))):
                Sp = prev[t - st]
                Sd, p, e, S = step(Sp, t)
                kt, qt = kn[t, qk_of], qn[t, qk_of]
                a = np.exp(g[t])
                dS = dS + scale * d_o[t][:, :, None] * qt[:, None, :]
                dqn[t] = scale * np.matmul(np.swapaxes(S, 1, 2), d_o[t][:, :, None])[:, :, 0]
                de = np.matmul(dS, kt[:, :, None])[:, :, 0]
                dk_t = np.matmul(np.swapaxes(dS, 1, 2), e[:, :, None])[:, :, 0]
                dSd = dS
                dv[t] = beta[t][:, None] * de
                db[t] = np.sum((v[t] - p) * de, axis=1)
                if erase:
                    dp = -beta[t][:, None] * de
                    dSd = dSd + dp[:, :, None] * kt[:, None, :]
                    dk_t = dk_t + np.matmul(np.swapaxes(Sd, 1, 2), dp[:, :, None])[:, :, 0]
                dkn[t] = dk_t
                da = np.sum(dSd * Sp, axis=(1, 2))
                dg[t] = a * da
                dS = a[:, None, None] * dSd
        dS0[n] = dS
    # each QK head collects the gradients of the V heads that read it
    dq = np.zeros((T, h_qk, d_k))
    dk = np.zeros((T, h_qk, d_k))
    for h in range(h_v):
        dq[:, qk_of[h]] += dqn[:, h]
        dk[:, qk_of[h]] += dkn[:, h]
    if l2norm_qk:
        dq = l2_normalize_backward(q, dq, eps)
        dk = l2_normalize_backward(k, dk, eps)
    return dq, dk, dv, dg, db, dS0


def causal_conv1d_backward(x, weight, dy, bias=None, conv_state=None, cu_seqlens=None,
                           activation="silu", d_new_state=None):
    """Gradients of causal_conv1d: returns dx [T, C], dweight [C, W], dbias [C]
    (None without bias) and d_conv_state [N, C, W-1].

    Per sequence the padded history xp = (state ++ x) gives z = sum_j w_j
    xp[j : j+L] (+ bias) and y = SiLU(z); new_state = the last W-1 rows of xp.
    Back: dz = dy SiLU'(z), SiLU'(z) = s (1 + z (1 - s)) with s = sigmoid(z);
    dxp[j : j+L] += w_j dz, dw_j = sum over tokens of dz xp[j : j+L],
    dbias = sum of dz, and the new-state gradient adds onto the rows of xp it
    copied.  dx and d_conv_state are the two parts of dxp.
    """
    x, weight, dy = _f64(x), _f64(weight), _f64(dy)
    bias = _f64(bias)
    T, C = x.shape
    W = weight.shape[1]
    b = _bounds(T, cu_seqlens)
    N = len(b) - 1
    state = np.zeros((N, C, W - 1)) if conv_state is None else _f64(conv_state)
    dx = np.zeros((T, C))
    dw = np.zeros((C, W))
    dbias = np.zeros(C)
    dstate = np.zeros((N, C, W - 1))
    for n in range(N):
        s, e = b[n], b[n + 1]
        L = e - s
        xp = np.concatenate([state[n].T, x[s:e]], axis=0)
        z = np.zeros((L, C))
        for j in range(W):
            z += weight[:, j] * xp[j:j + L]
        if bias is not None:
            z += bias
        if activation == "silu":
            sg = 1.0 / (1.0 + np.exp(-z))
            dz = dy[s:e] * sg * (1.0 + z * (1.0 - sg))
        else:
            assert activation in (None, "none")
            dz = dy[s:e].copy()
        dxp = np.zeros((W - 1 + L, C))
        for j in range(W):
            dxp[j:j + L] += weight[:, j] * dz
            dw[:, j] += np.sum(dz * xp[j:j + L], axis=0)
        dbias += np.sum(dz, axis=0)
        if d_new_state is not None:
            dxp[L:] += _f64(d_new_state)[n].T
        dx[s:e] = dxp[W - 1:]
        dstate[n] = dxp[:W - 1].T
    return dx, dw, (dbias if bias is not None else None), dstate
