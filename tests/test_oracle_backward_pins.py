"""Pins for the oracle's backward functions.

None of them retypes the backward loop.  Each one checks it against
something fixed independently of it:
- central finite differences of the pinned forward definitions, for every
  input entry;
- the adjoint identity of the map (V, S_0) -> (O, S_T), which is linear
  for fixed q, k, g, beta, so it is exact up to rounding;
- the closed form of the beta = 0 case;
- invariants.
"""
import numpy as np
import pytest

from oracle import gdn_oracle as orc


def _case(rng, lens, h_qk, h_v, d_k, d_v):
    T = sum(lens)
    q = rng.standard_normal((T, h_qk, d_k))
    k = rng.standard_normal((T, h_qk, d_k))
    v = rng.standard_normal((T, h_v, d_v))
    g = -np.logaddexp(0, -rng.standard_normal((T, h_v)))
    beta = 1 / (1 + np.exp(-rng.standard_normal((T, h_v))))
    s0 = 0.3 * rng.standard_normal((len(lens), h_v, d_v, d_k))
    cu = np.cumsum([0] + lens)
    return q, k, v, g, beta, s0, cu


def _fd(f, x, h=1e-6):
    """Central differences of the scalar f at every entry of x (x is restored)."""
    out = np.zeros_like(x)
    flat, of = x.reshape(-1), out.reshape(-1)
    for i in range(flat.size):
        keep = flat[i]
        flat[i] = keep + h
        fp = f()
        flat[i] = keep - h
        fm = f()
        flat[i] = keep
        of[i] = (fp - fm) / (2 * h)
    return out


@pytest.mark.parametrize("erase", [True, False])
@pytest.mark.parametrize("l2", [True, False])
def test_recurrence_backward_matches_finite_differences(erase, l2):
    """Every gradient of L = <o, Ro> + <S_T, Rs> against central differences of
    gated_delta_rule itself: two packed sequences (one of them a single token),
    grouped heads, non-zero S_0, a non-unit scale."""
    rng = np.random.default_rng(5)
    q, k, v, g, beta, s0, cu = _case(rng, [5, 1, 4], 2, 4, 3, 2)
    Ro = rng.standard_normal((q.shape[0], 4, 2))
    Rs = rng.standard_normal(s0.shape)
    scale = 0.7

    def loss():
        o, S = orc.gated_delta_rule(q, k, v, g, beta, s0, cu, scale, l2norm_qk=l2, erase=erase)
        return float(np.sum(o * Ro) + np.sum(S * Rs))

    got = orc.gated_delta_rule_backward(q, k, v, g, beta, Ro, s0, Rs, cu, scale, l2norm_qk=l2,
                                        erase=erase, segment=2)
    for name, x, gx in zip(["q", "k", "v", "g", "beta", "S0"], [q, k, v, g, beta, s0], got):
        ref = _fd(loss, x)
        err = np.max(np.abs(gx - ref)) / max(np.max(np.abs(ref)), 1e-12)
        assert err < 1e-7, (name, err)


def test_recurrence_backward_segment_invariant():
    """The checkpoint spacing only changes where states are recomputed."""
    rng = np.random.default_rng(6)
    q, k, v, g, beta, s0, cu = _case(rng, [13, 7], 1, 3, 4, 4)
    do = rng.standard_normal(v.shape)
    dsf = rng.standard_normal(s0.shape)
    a = orc.gated_delta_rule_backward(q, k, v, g, beta, do, s0, dsf, cu, segment=1)
    b = orc.gated_delta_rule_backward(q, k, v, g, beta, do, s0, dsf, cu, segment=64)
    for x, y in zip(a, b):
        assert np.allclose(x, y, rtol=0, atol=1e-13)


def test_adjoint_identity_in_values_and_initial_state():
    """For fixed q, k, g, beta the map (V, S_0) -> (O, S_T) is linear, so
    <dV, V'> + <dS_0, S_0'> = <dO, O'> + <dS_T, S_T'>, where (O', S_T') is
    the forward run on (V', S_0'), holds exactly (to rounding) for any V', S_0'."""
    rng = np.random.default_rng(7)
    q, k, v, g, beta, s0, cu = _case(rng, [9, 0, 6], 2, 4, 5, 3)
    do = rng.standard_normal(v.shape)
    dsf = rng.standard_normal(s0.shape)
    _, _, dv, _, _, ds0 = orc.gated_delta_rule_backward(q, k, v, g, beta, do, s0, dsf, cu)
    v2 = rng.standard_normal(v.shape)
    s2 = rng.standard_normal(s0.shape)
    o2, S2 = orc.gated_delta_rule(q, k, v2, g, beta, s2, cu)
    lhs = np.sum(dv * v2) + np.sum(ds0 * s2)
    rhs = np.sum(do * o2) + np.sum(dsf * S2)
    assert abs(lhs - rhs) < 1e-12 * max(1.0, abs(rhs))


def test_beta_zero_closed_form():
    """beta = 0: S_t = P_t S_0 with P_t = exp(sum_{s<=t} g_s), o_t = scale P_t S_0 q^_t.
    Then dS_0 = P_T dS_T + sum_t scale P_t do_t q^_t^T, dV = dK = 0, and
    dg_s = sum_{t>=s} scale P_t <do_t, S_0 q^_t> + P_T <dS_T, S_0>."""
    rng = np.random.default_rng(8)
    T, dk_, dv_ = 7, 4, 3
    q, k, v, g, beta, s0, cu = _case(rng, [T], 1, 1, dk_, dv_)
    beta[:] = 0.0
    do = rng.standard_normal(v.shape)
    dsf = rng.standard_normal(s0.shape)
    scale = 1.3
    dq, dk, dv, dg, db, ds0 = orc.gated_delta_rule_backward(q, k, v, g, beta, do, s0, dsf, cu, scale)
    qn = q[:, 0] / np.sqrt(np.sum(q[:, 0] ** 2, axis=1, keepdims=True) + 1e-6)
    S0 = s0[0, 0]
    P = np.exp(np.cumsum(g[:, 0]))
    want_ds0 = P[-1] * dsf[0, 0] + sum(scale * P[t] * np.outer(do[t, 0], qn[t]) for t in range(T))
    term = np.array([scale * P[t] * do[t, 0] @ (S0 @ qn[t]) for t in range(T)])
    want_dg = np.array([term[s:].sum() for s in range(T)]) + P[-1] * np.sum(dsf[0, 0] * S0)
    assert np.allclose(ds0[0, 0], want_ds0, atol=1e-12)
    assert np.allclose(dg[:, 0], want_dg, atol=1e-12)
    assert np.max(np.abs(dv)) == 0.0 and np.max(np.abs(dk)) == 0.0
    # beta's own gradient is not zero at beta = 0: db_t = <dS_t, v_t k^_t^T - S_dec k^_t k^_t^T>


def test_l2_backward_orthogonal_without_eps():
    """x / |x| is scale invariant, so its gradient is orthogonal to x (eps = 0)."""
    rng = np.random.default_rng(9)
    x = rng.standard_normal((6, 2, 5))
    d = orc.l2_normalize_backward(x, rng.standard_normal(x.shape), eps=0.0)
    assert np.max(np.abs(np.sum(x * d, axis=-1))) < 1e-13


@pytest.mark.parametrize("act", ["silu", None])
def test_conv_backward_matches_finite_differences(act):
    """dx, dweight, dbias, d_conv_state of L = <y, Ry> + <new_state, Rs> against
    central differences of causal_conv1d: three packed sequences, one of them
    shorter than the conv state (its new state keeps older entries)."""
    rng = np.random.default_rng(10)
    lens, C, W = [6, 2, 5], 3, 4
    T = sum(lens)
    cu = np.cumsum([0] + lens)
    x = rng.standard_normal((T, C))
    w = 0.5 * rng.standard_normal((C, W))
    bias = 0.1 * rng.standard_normal(C)
    cs = rng.standard_normal((3, C, W - 1))
    Ry = rng.standard_normal((T, C))
    Rs = rng.standard_normal((3, C, W - 1))

    def loss():
        y, ns = orc.causal_conv1d(x, w, bias, cs, cu, act)
        return float(np.sum(y * Ry) + np.sum(ns * Rs))

    got = orc.causal_conv1d_backward(x, w, Ry, bias, cs, cu, act, Rs)
    for name, a, ga in zip(["x", "w", "bias", "state"], [x, w, bias, cs], got):
        ref = _fd(loss, a)
        assert np.max(np.abs(ga - ref)) < 1e-7 * max(1.0, np.max(np.abs(ref))), name


def test_conv_backward_identity_tap():
    """With only the current tap (w = e_{W-1}) and no activation, y = x, so
    dx = dy and the state gets only what new_state copied."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((8, 2))
    w = np.zeros((2, 4))
    w[:, 3] = 1.0
    dy = rng.standard_normal(x.shape)
    dx, dw, _, dst = orc.causal_conv1d_backward(x, w, dy, activation=None)
    assert np.array_equal(dx, dy)
    assert np.array_equal(dst, np.zeros_like(dst))
    assert np.allclose(dw[:, 3], np.sum(dy * x, axis=0))
