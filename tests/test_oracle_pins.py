"""Pins for the fp64 oracle against what the pages and the mathematics fix.

None of these checks retypes the oracle's own loop: each one compares it with
a hand-worked fixture, a closed form, a special case that reduces to another
formula printed on the pages, an exact rational evaluation, a library
routine, or an invariant.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import gdn_inputs
from oracle import gdn_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _unit(a):
    return a / np.linalg.norm(a, axis=-1, keepdims=True)


def _rand_case(rng, T=9, h_qk=2, h_v=4, d_k=5, d_v=3, S0=True):
    q = rng.standard_normal((T, h_qk, d_k))
    k = rng.standard_normal((T, h_qk, d_k))
    v = rng.standard_normal((T, h_v, d_v))
    g = -np.logaddexp(0, -rng.standard_normal((T, h_v)))
    beta = 1 / (1 + np.exp(-rng.standard_normal((T, h_v))))
    s0 = 0.3 * rng.standard_normal((1, h_v, d_v, d_k)) if S0 else None
    return q, k, v, g, beta, s0


# ---------------------------------------------------------------- recurrence

def test_worked_example_by_hand():
    """Hand-worked 2x2 example of the decay-first update (tests/golden/worked_2x2.json)."""
    fx = json.load(open(os.path.join(GOLDEN, "worked_2x2.json")))
    k = np.array(fx["k"])[:, None, :]
    q = np.array(fx["q"])[:, None, :]
    v = np.array(fx["v"])[:, None, :]
    g = np.log(np.array(fx["alpha"]))[:, None]
    beta = np.array(fx["beta"])[:, None]
    S0 = np.array(fx["S0"])[None, None]
    o1, S1 = orc.gated_delta_rule(q[:1], k[:1], v[:1], g[:1], beta[:1], S0, l2norm_qk=False)
    assert np.allclose(S1[0, 0], fx["S1"], atol=1e-15)
    assert not np.allclose(S1[0, 0], fx["S1_same_time_reading"])
    o, S2 = orc.gated_delta_rule(q, k, v, g, beta, S0, l2norm_qk=False)
    assert np.allclose(S2[0, 0], fx["S2"], atol=1e-14)
    assert np.allclose(o[:, 0], fx["o"], atol=1e-14)


def test_exact_rational_arithmetic():
    """Brute force in exact rational arithmetic (fractions) on tiny inputs,
    from the matrix statement S_t = a S (I - b k k^T) + b v k^T, o = S q."""
    rng = np.random.default_rng(1)
    T, dk, dv = 5, 3, 2

    def rat(x):
        return Fraction(int(round(x * 64)), 64)

    K = [[rat(x) for x in row] for row in rng.uniform(-1, 1, (T, dk))]
    V = [[rat(x) for x in row] for row in rng.uniform(-1, 1, (T, dv))]
    Q = [[rat(x) for x in row] for row in rng.uniform(-1, 1, (T, dk))]
    A = [Fraction(int(a), 16) for a in rng.integers(1, 16, T)]
    B = [Fraction(int(b), 16) for b in rng.integers(0, 17, T)]
    S = [[rat(x) for x in row] for row in rng.uniform(-1, 1, (dv, dk))]
    S_init = [row[:] for row in S]
    outs = []
    for t in range(T):
        # M = I - b k k^T ;  S <- a S M + b v k^T
        M = [[(1 if i == j else 0) - B[t] * K[t][i] * K[t][j] for j in range(dk)] for i in range(dk)]
        S = [[A[t] * sum(S[r][m] * M[m][c] for m in range(dk)) + B[t] * V[t][r] * K[t][c]
              for c in range(dk)] for r in range(dv)]
        outs.append([sum(S[r][c] * Q[t][c] for c in range(dk)) for r in range(dv)])
    f = np.vectorize(float)
    o, Sf = orc.gated_delta_rule(f(np.array(Q, dtype=object))[:, None], f(np.array(K, dtype=object))[:, None],
                                 f(np.array(V, dtype=object))[:, None],
                                 np.log([float(a) for a in A])[:, None], np.array([float(b) for b in B])[:, None],
                                 f(np.array(S_init, dtype=object))[None, None], l2norm_qk=False)
    assert np.allclose(Sf[0, 0], f(np.array(S, dtype=object)), rtol=0, atol=1e-13)
    assert np.allclose(o[:, 0], f(np.array(outs, dtype=object)), rtol=0, atol=1e-13)


def test_no_decay_no_write_keeps_state():
    """alpha = 1, beta = 0: the state is unchanged and o_t = S_0 q_t."""
    rng = np.random.default_rng(2)
    q, k, v, g, beta, s0 = _rand_case(rng)
    o, S = orc.gated_delta_rule(q, k, v, 0 * g, 0 * beta, s0)
    assert np.array_equal(S, s0)
    qn = orc.l2_normalize(q)
    for h in range(4):
        assert np.allclose(o[:, h], qn[:, h // 2] @ s0[0, h].T, atol=1e-14)


def test_beta_zero_closed_form():
    """beta = 0: S_T = (prod alpha) S_0 and o_t = (prod_{s<=t} alpha_s) S_0 q_t."""
    rng = np.random.default_rng(3)
    q, k, v, g, beta, s0 = _rand_case(rng)
    o, S = orc.gated_delta_rule(q, k, v, g, 0 * beta, s0)
    decay = np.exp(np.cumsum(g, axis=0))  # [T, H_v]
    assert np.allclose(S[0], decay[-1][:, None, None] * s0[0], atol=1e-14)
    qn = orc.l2_normalize(q)
    for h in range(4):
        assert np.allclose(o[:, h], decay[:, h:h + 1] * (qn[:, h // 2] @ s0[0, h].T), atol=1e-14)


def test_full_write_to_unit_key_stores_value():
    """beta = 1 with a unit key: after the write, S_t k_t = v_t for any alpha
    (the error-correcting write replaces the association; "Inside Qwen3.5", section 5)."""
    rng = np.random.default_rng(4)
    q, k, v, g, beta, s0 = _rand_case(rng, T=12)
    k = _unit(k)
    for t in range(1, 13):
        _, S = orc.gated_delta_rule(q[:t], k[:t], v[:t], g[:t], np.ones_like(beta[:t]), s0,
                                    l2norm_qk=False)
        for h in range(4):
            assert np.allclose(S[0, h] @ k[t - 1, h // 2], v[t - 1, h], atol=1e-13)


def test_ungated_equals_deltanet_as_printed():
    """g = 0 reduces to DeltaNet as printed on "Hybrid Mamba-Transformer MoE"
    (Gated DeltaNet section): S_t = S_{t-1} - b (S_{t-1} k) k^T + b v k^T."""
    rng = np.random.default_rng(5)
    q, k, v, g, beta, s0 = _rand_case(rng, h_qk=1, h_v=1)
    kn, qn = orc.l2_normalize(k), orc.l2_normalize(q)
    S = s0[0, 0].copy()
    outs = []
    for t in range(len(k)):
        kt, b = kn[t, 0], beta[t, 0]
        S = S - b * np.outer(S @ kt, kt) + b * np.outer(v[t, 0], kt)
        outs.append(S @ qn[t, 0])
    o, Sf = orc.gated_delta_rule(q, k, v, 0 * g, beta, s0)
    assert np.allclose(Sf[0, 0], S, atol=1e-14)
    assert np.allclose(o[:, 0], np.array(outs), atol=1e-14)


def test_orthogonal_keys_reduce_to_gated_linear_attention():
    """Mutually orthogonal unit keys and S_0 = 0: the erase term vanishes and
    S_t = sum_s (prod_{r=s+1..t} alpha_r) beta_s v_s k_s^T -- decayed linear
    attention; with alpha = beta = 1 it is S = sum v k^T, o = S q
    ("Inside Qwen3.5", section 2)."""
    rng = np.random.default_rng(6)
    T, d = 6, 8
    perm = rng.permutation(d)[:T]
    k = np.eye(d)[perm][:, None, :]
    q = rng.standard_normal((T, 1, d))
    v = rng.standard_normal((T, 1, 3))
    g = -np.logaddexp(0, -rng.standard_normal((T, 1)))
    beta = 1 / (1 + np.exp(-rng.standard_normal((T, 1))))
    o, S = orc.gated_delta_rule(q, k, v, g, beta, None, l2norm_qk=False)
    G = np.cumsum(g[:, 0])
    ref = sum(np.exp(G[-1] - G[s]) * beta[s, 0] * np.outer(v[s, 0], k[s, 0]) for s in range(T))
    assert np.allclose(S[0, 0], ref, atol=1e-14)
    o1, S1 = orc.gated_delta_rule(q, k, v, 0 * g, np.ones_like(beta), None, l2norm_qk=False)
    la = sum(np.outer(v[s, 0], k[s, 0]) for s in range(T))
    assert np.allclose(S1[0, 0], la, atol=1e-14)
    assert np.allclose(o1[-1, 0], la @ q[-1, 0], atol=1e-14)


def test_unrolled_product_form():
    """S_T = S_0 A_1..A_T + sum_s b_s v_s k_s^T A_{s+1}..A_T with explicit A_t."""
    rng = np.random.default_rng(7)
    q, k, v, g, beta, s0 = _rand_case(rng, T=7, h_qk=1, h_v=1)
    _, S = orc.gated_delta_rule(q, k, v, g, beta, s0)
    ref = orc.unrolled_product_form(orc.l2_normalize(k[:, 0]), v[:, 0], g[:, 0], beta[:, 0], s0[0, 0])
    assert np.allclose(S[0, 0], ref, atol=1e-14)


@pytest.mark.parametrize("chunk", [1, 2, 3, 4, 16, 64])
def test_chunked_equals_sequential(chunk):
    """Brute force: the chunked (UT-transform) algebra equals the sequential
    recurrence, with partial last chunks, grouped heads and S_0 != 0."""
    rng = np.random.default_rng(8)
    q, k, v, g, beta, s0 = _rand_case(rng, T=37, h_qk=2, h_v=6, d_k=8, d_v=5)
    o, S = orc.gated_delta_rule(q, k, v, g, beta, s0)
    oc, Sc = orc.chunked_gated_delta_rule(q, k, v, g, beta, s0[0], chunk)
    assert np.abs(o - oc).max() < 1e-12
    assert np.abs(S[0] - Sc).max() < 1e-12


def test_linearity_in_values_and_initial_state():
    rng = np.random.default_rng(9)
    q, k, v, g, beta, s0 = _rand_case(rng)
    _, _, v2, _, _, s2 = _rand_case(rng)
    a, b = 0.7, -1.3
    o1, S1 = orc.gated_delta_rule(q, k, v, g, beta, s0)
    o2, S2 = orc.gated_delta_rule(q, k, v2, g, beta, s2)
    o3, S3 = orc.gated_delta_rule(q, k, a * v + b * v2, g, beta, a * s0 + b * s2)
    assert np.allclose(o3, a * o1 + b * o2, atol=1e-13)
    assert np.allclose(S3, a * S1 + b * S2, atol=1e-13)


def test_stability_bound():
    """||I - b k k^T||_2 = 1 for b in [0,1] and unit k, so
    ||S_t||_2 <= alpha_t ||S_{t-1}||_2 + b_t ||v_t||_2 at every step."""
    rng = np.random.default_rng(10)
    q, k, v, g, beta, s0 = _rand_case(rng, T=30, h_qk=1, h_v=1, d_k=6, d_v=6)
    prev = np.linalg.norm(s0[0, 0], 2)
    for t in range(1, 31):
        _, S = orc.gated_delta_rule(q[:t], k[:t], v[:t], g[:t], beta[:t], s0)
        cur = np.linalg.norm(S[0, 0], 2)
        assert cur <= math.exp(g[t - 1, 0]) * prev + beta[t - 1, 0] * np.linalg.norm(v[t - 1, 0]) + 1e-12
        prev = cur


def test_grouped_heads_equal_repeated_heads():
    """V head h reads QK head h // (H_v/H_qk): same as repeating each QK head."""
    rng = np.random.default_rng(11)
    q, k, v, g, beta, s0 = _rand_case(rng, h_qk=2, h_v=6)
    o, S = orc.gated_delta_rule(q, k, v, g, beta, s0)
    o2, S2 = orc.gated_delta_rule(np.repeat(q, 3, axis=1), np.repeat(k, 3, axis=1), v, g, beta, s0)
    assert np.array_equal(o, o2) and np.array_equal(S, S2)
    o3, S3 = orc.gated_delta_rule(q, k, v, g, beta, s0, v_heads=[4, 1])
    assert np.array_equal(o3, o[:, [4, 1]]) and np.array_equal(S3, S[:, [4, 1]])


def test_varlen_packed_equals_per_sequence():
    rng = np.random.default_rng(12)
    lens = [5, 1, 0, 9, 3]
    T = sum(lens)
    q, k, v, g, beta, _ = _rand_case(rng, T=T)
    s0 = 0.3 * rng.standard_normal((len(lens), 4, 3, 5))
    cu = np.concatenate([[0], np.cumsum(lens)])
    o, S = orc.gated_delta_rule(q, k, v, g, beta, s0, cu_seqlens=cu)
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        on, Sn = orc.gated_delta_rule(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], s0[n:n + 1])
        assert np.array_equal(o[a:b], on) and np.array_equal(S[n], Sn[0])
    assert np.array_equal(S[2], s0[2])  # an empty sequence passes its state through


def test_split_prefill_equals_whole():
    """prefill(T1) then prefill(T2) from its state equals prefill(T1 + T2)."""
    rng = np.random.default_rng(13)
    q, k, v, g, beta, s0 = _rand_case(rng, T=20)
    o, S = orc.gated_delta_rule(q, k, v, g, beta, s0)
    oa, Sa = orc.gated_delta_rule(q[:7], k[:7], v[:7], g[:7], beta[:7], s0)
    ob, Sb = orc.gated_delta_rule(q[7:], k[7:], v[7:], g[7:], beta[7:], Sa)
    assert np.allclose(np.concatenate([oa, ob]), o, atol=1e-14) and np.allclose(Sb, S, atol=1e-14)


# ------------------------------------------------------------------ conv etc.

def test_conv_matches_torch_conv1d():
    """The causal depthwise conv equals torch's conv1d (cross-correlation,
    groups = channels) over the zero-left-padded input, in float64."""
    rng = np.random.default_rng(14)
    T, C, W = 17, 6, 4
    x = rng.standard_normal((T, C))
    w = rng.standard_normal((C, W))
    bias = rng.standard_normal(C)
    y, st = orc.causal_conv1d(x, w, bias, activation=None)
    xt = torch.from_numpy(x.T[None])
    ref = torch.nn.functional.conv1d(torch.nn.functional.pad(xt, (W - 1, 0)),
                                     torch.from_numpy(w[:, None, :]), torch.from_numpy(bias), groups=C)
    assert np.allclose(y, ref[0].numpy().T, atol=1e-14)
    assert np.array_equal(st[0], x[-(W - 1):].T)


def test_conv_tap_and_state_order():
    rng = np.random.default_rng(15)
    T, C = 10, 3
    x = rng.standard_normal((T, C))
    st = rng.standard_normal((1, C, 3))
    e3 = np.zeros((C, 4)); e3[:, 3] = 1
    y, _ = orc.causal_conv1d(x, e3, conv_state=st, activation=None)
    assert np.array_equal(y, x)  # the last tap is the current token
    e0 = np.zeros((C, 4)); e0[:, 0] = 1
    y, new = orc.causal_conv1d(x, e0, conv_state=st, activation=None)
    assert np.array_equal(y[:3], st[0].T) and np.array_equal(y[3:], x[:-3])  # shift by 3, oldest first
    # a sequence shorter than the window keeps its older state entries
    _, new2 = orc.causal_conv1d(x[:2], e0, conv_state=st, activation=None)
    assert np.array_equal(new2[0], np.concatenate([st[0][:, 2:], x[:2].T], axis=1))


def test_conv_varlen_has_no_leakage():
    rng = np.random.default_rng(16)
    lens = [4, 1, 0, 7]
    cu = np.concatenate([[0], np.cumsum(lens)])
    x = rng.standard_normal((sum(lens), 5))
    w = rng.standard_normal((5, 4))
    st = rng.standard_normal((4, 5, 3))
    y, new = orc.causal_conv1d(x, w, conv_state=st, cu_seqlens=cu)
    for n in range(4):
        yn, sn = orc.causal_conv1d(x[cu[n]:cu[n + 1]], w, conv_state=st[n:n + 1])
        assert np.array_equal(y[cu[n]:cu[n + 1]], yn) and np.array_equal(new[n], sn[0])
    assert np.array_equal(new[2], st[2])


def test_silu_and_l2norm_against_library():
    x = np.linspace(-30, 30, 1001)
    assert np.allclose(orc.silu(x), torch.nn.functional.silu(torch.from_numpy(x)).numpy(), atol=1e-15)
    a = np.random.default_rng(17).standard_normal((7, 3, 128))
    assert np.allclose(orc.l2_normalize(a, eps=0.0), a / np.linalg.norm(a, axis=-1, keepdims=True),
                       atol=1e-15)


def test_layer_and_decode_handoff():
    """conv+recurrence over T tokens, then one decode step from the emitted
    recurrent and conv states, equals the layer over T + 1 tokens."""
    rng = np.random.default_rng(18)
    hq, hv, d = 2, 4, 8
    C = 2 * hq * d + hv * d
    T = 11
    x = rng.standard_normal((T + 1, C))
    w = 0.5 * rng.standard_normal((C, 4))
    g = -np.logaddexp(0, -rng.standard_normal((T + 1, hv)))
    beta = 1 / (1 + np.exp(-rng.standard_normal((T + 1, hv))))
    s0 = 0.1 * rng.standard_normal((1, hv, d, d))
    o, S, cs = orc.gdn_layer(x, w, g, beta, hq, d, hv, d, initial_state=s0)
    oa, Sa, csa = orc.gdn_layer(x[:T], w, g[:T], beta[:T], hq, d, hv, d, initial_state=s0)
    od, Sd, csd = orc.decode_step(x[T:], w, g[T:], beta[T:], Sa, csa, hq, d, hv, d)
    assert np.allclose(od[0], o[T], atol=1e-13)
    assert np.allclose(Sd, S, atol=1e-13) and np.allclose(csd, cs, atol=0)
    # sampled heads give the same rows as the whole layer
    o2, S2, _ = orc.gdn_layer(x, w, g, beta, hq, d, hv, d, initial_state=s0, v_heads=[3, 0])
    assert np.allclose(o2, o[:, [3, 0]], atol=1e-14) and np.allclose(S2, S[:, [3, 0]], atol=1e-14)


# ------------------------------------------------------- erase-off variant

def test_erase_off_closed_form_any_keys():
    """Without the correcting write the recurrence is additive: for any keys
    S_t = (prod_{r<=t} a_r) S_0 + sum_{s<=t} (prod_{s<r<=t} a_r) b_s v_s k_s^T
    and o_t = scale S_t q_t -- the linear attention S = sum v k^T, o = S q of
    "Inside Qwen3.5", section 2, with the decay gate of section 5."""
    rng = np.random.default_rng(40)
    T = 8
    q, k, v, g, beta, s0 = _rand_case(rng, T=T, h_qk=1, h_v=1)
    o, S = orc.gated_delta_rule(q, k, v, g, beta, s0, scale=0.7, erase=False)
    kn = k[:, 0] / np.sqrt((k[:, 0] ** 2).sum(-1, keepdims=True) + 1e-6)
    qn = q[:, 0] / np.sqrt((q[:, 0] ** 2).sum(-1, keepdims=True) + 1e-6)
    G = np.cumsum(g[:, 0])
    for t in range(T):
        St = np.exp(G[t]) * s0[0, 0] + sum(np.exp(G[t] - G[s]) * beta[s, 0] * np.outer(v[s, 0], kn[s])
                                           for s in range(t + 1))
        assert np.allclose(o[t, 0], 0.7 * St @ qn[t], atol=1e-13)
    assert np.allclose(S[0, 0], St, atol=1e-13)


def test_erase_off_plain_linear_attention():
    """a = b = 1 and S_0 = 0: S_t = sum_{s<=t} v_s k_s^T and o_t = S_t q_t,
    as printed in "Inside Qwen3.5", section 2 (prefix sums by torch.cumsum)."""
    rng = np.random.default_rng(41)
    T, d = 7, 5
    q, k, v = rng.standard_normal((T, 1, d)), rng.standard_normal((T, 1, d)), rng.standard_normal((T, 1, 3))
    o, S = orc.gated_delta_rule(q, k, v, np.zeros((T, 1)), np.ones((T, 1)), None, l2norm_qk=False,
                                erase=False)
    outer = torch.from_numpy(np.einsum("ti,tj->tij", v[:, 0], k[:, 0]))
    St = torch.cumsum(outer, dim=0).numpy()
    assert np.allclose(S[0, 0], St[-1], atol=1e-14)
    assert np.allclose(o[:, 0], np.einsum("tij,tj->ti", St, q[:, 0]), atol=1e-13)


def test_erase_off_equals_erase_on_for_orthogonal_keys():
    """Mutually orthogonal unit keys and S_0 = 0: S_{t-1} k_t = 0, so the
    correcting term vanishes and the two forms agree."""
    rng = np.random.default_rng(42)
    T, d = 6, 8
    k = np.eye(d)[rng.permutation(d)[:T]][:, None, :]
    q = rng.standard_normal((T, 1, d))
    v = rng.standard_normal((T, 1, 3))
    g = -np.logaddexp(0, -rng.standard_normal((T, 1)))
    beta = 1 / (1 + np.exp(-rng.standard_normal((T, 1))))
    o1, S1 = orc.gated_delta_rule(q, k, v, g, beta, None, l2norm_qk=False)
    o0, S0 = orc.gated_delta_rule(q, k, v, g, beta, None, l2norm_qk=False, erase=False)
    assert np.allclose(o1, o0, atol=1e-14) and np.allclose(S1, S0, atol=1e-14)
    # with a repeated key they differ: the erase-on form replaces, the other adds
    k2 = k.copy()
    k2[3] = k2[1]
    _, Sa = orc.gated_delta_rule(q, k2, v, g, beta, None, l2norm_qk=False)
    _, Sb = orc.gated_delta_rule(q, k2, v, g, beta, None, l2norm_qk=False, erase=False)
    assert np.abs(Sa - Sb).max() > 1e-3


@pytest.mark.parametrize("chunk", [1, 3, 16, 64])
def test_erase_off_chunked_equals_sequential(chunk):
    """Brute force: the chunked form with no correction (A = 0, U = diag(b) V)
    equals the sequential additive recurrence, partial chunks and S_0 != 0."""
    rng = np.random.default_rng(43)
    q, k, v, g, beta, s0 = _rand_case(rng, T=37, h_qk=2, h_v=6, d_k=8, d_v=5)
    o, S = orc.gated_delta_rule(q, k, v, g, beta, s0, erase=False)
    oc, Sc = orc.chunked_gated_delta_rule(q, k, v, g, beta, s0[0], chunk, erase=False)
    assert np.abs(o - oc).max() < 1e-12
    assert np.abs(S[0] - Sc).max() < 1e-12


def test_erase_off_layer_and_decode_handoff():
    """Erase off: the layer over T tokens, then one decode step from its
    states, equals the layer over T + 1 tokens."""
    rng = np.random.default_rng(44)
    hq, hv, d = 1, 3, 8
    C = 2 * hq * d + hv * d
    T = 9
    x = rng.standard_normal((T + 1, C))
    w = 0.5 * rng.standard_normal((C, 4))
    g = -np.logaddexp(0, -rng.standard_normal((T + 1, hv)))
    beta = 1 / (1 + np.exp(-rng.standard_normal((T + 1, hv))))
    s0 = 0.1 * rng.standard_normal((1, hv, d, d))
    o, S, cs = orc.gdn_layer(x, w, g, beta, hq, d, hv, d, initial_state=s0, erase=False)
    oa, Sa, csa = orc.gdn_layer(x[:T], w, g[:T], beta[:T], hq, d, hv, d, initial_state=s0, erase=False)
    od, Sd, _ = orc.decode_step(x[T:], w, g[T:], beta[T:], Sa, csa, hq, d, hv, d, erase=False)
    assert np.allclose(od[0], o[T], atol=1e-13) and np.allclose(Sd, S, atol=1e-13)


def test_bf16_rounding_is_nearest_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1e-3, 3.0e38])
    ref = torch.from_numpy(vals.astype(np.float32)).to(torch.bfloat16).float().numpy()
    assert np.array_equal(orc.round_to_bf16(vals), ref.astype(np.float64))


# ------------------------------------------------------------------- sizes

def test_sizes_match_the_pages():
    fx = json.load(open(os.path.join(GOLDEN, "sizes_27b.json")))
    cfg = gdn_inputs.CONFIGS["qwen35_27b_prefill"]
    assert (cfg["h_qk"], cfg["h_v"], cfg["d_k"], cfg["width"]) == (fx["h_qk"], fx["h_v"], fx["d"], fx["conv_width"])
    assert cfg["d_k"] * cfg["d_v"] == fx["floats_per_head"]
    state = cfg["h_v"] * cfg["d_v"] * cfg["d_k"] * 4
    conv = gdn_inputs.channels(cfg) * cfg["width"] * 2
    assert state == fx["state_bytes_per_layer_fp32"] and conv == fx["conv_buffer_bytes_bf16_4_taps"]
    assert state + conv == fx["layer_bytes"]
    assert fx["layer_bytes"] // fx["kv_bytes_per_token"] == fx["break_even_tokens"]
    assert round(fx["linear_layers"] * fx["layer_bytes"] / 2 ** 20) == fx["state_mb_48_layers"]


def test_varlen_lengths_recipe():
    rng = np.random.default_rng(0)
    L = gdn_inputs.varlen_lengths(8, 262144, 4096, 65536, rng)
    assert L.sum() == 262144 and L.min() >= 4096 and L.max() <= 65536 and len(L) == 8


def test_ring_to_chronological_by_hand():
    """Hand-worked ring of three slots holding inputs a, b, c of one channel:
    with head 1 the oldest input is slot 1, so the order is (b, c, a); with
    head 2 it is (c, a, b); head 0 is the chronological layout itself."""
    a, b, c = 1.0, 2.0, 3.0
    ring = np.array([[[a, b, c]]] * 3)  # three sequences, one channel, slots 0..2
    got = orc.ring_to_chronological(ring, np.array([0, 1, 2]))
    assert got[0, 0].tolist() == [a, b, c]
    assert got[1, 0].tolist() == [b, c, a]
    assert got[2, 0].tolist() == [c, a, b]


def test_ring_step_equals_shift():
    """Writing the new input over the oldest slot and advancing the head holds
    the same chronological conv state as shifting the slots, step after step,
    for every starting head; the decode oracle consumes that state."""
    rng = np.random.default_rng(5)
    N, C, M = 3, 4, 3
    ring = rng.standard_normal((N, C, M))
    head = np.array([0, 1, 2])
    chrono = orc.ring_to_chronological(ring, head)
    for _ in range(7):
        x = rng.standard_normal((N, C))
        for n in range(N):                       # ring step: one slot, head + 1
            ring[n, :, head[n]] = x[n]
        head = (head + 1) % M
        chrono = np.concatenate([chrono[:, :, 1:], x[:, :, None]], axis=2)  # shift step
        assert np.array_equal(orc.ring_to_chronological(ring, head), chrono)
    # and the conv over one more token reads the same history either way
    w = rng.standard_normal((C, M + 1))
    xt = rng.standard_normal((1, C))
    y_ring, _ = orc.causal_conv1d(xt, w, conv_state=orc.ring_to_chronological(ring, head)[:1], activation=None)
    expect = sum(w[:, j] * chrono[0, :, j] for j in range(M)) + w[:, M] * xt[0]
    assert np.allclose(y_ring[0], expect, rtol=0, atol=1e-12)
