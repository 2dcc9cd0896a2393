"""Pins of the oracle's recurrence backward (derivatives of the gated delta rule) against central finite
differences of the oracle's forward -- itself pinned in test_oracle_pins.py -- and a closed form."""
import numpy as np
import pytest

import oracle as O


def _chain(rng, L, dk, dv):
    q, k = rng.standard_normal((L, dk)), rng.standard_normal((L, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((L, dv))
    alpha = rng.uniform(0.5, 1.0, L)
    beta = rng.uniform(0.1, 1.0, L)
    S0 = 0.3 * rng.standard_normal((dk, dv))
    return q, k, v, alpha, beta, S0


@pytest.mark.parametrize("scale", [1.0, 0.7])
def test_chain_backward_matches_finite_differences(scale):
    """L = sum dy . y + <dS_L, S_L>; every partial derivative by central differences (h = 1e-6)."""
    rng = np.random.default_rng(21)
    L, dk, dv = 6, 3, 4
    args = list(_chain(rng, L, dk, dv))
    dy, dSf = rng.standard_normal((L, dv)), rng.standard_normal((dk, dv))

    def loss(a):
        y, S = O.gated_delta_rule(*a, scale=scale)
        return float(np.sum(dy * y) + np.sum(dSf * S))

    got = O.gated_delta_rule_backward(*args, dy, dSf, scale)
    names = ["q", "k", "v", "alpha", "beta", "S0"]
    grads = {"q": got[0], "k": got[1], "v": got[2], "alpha": got[3], "beta": got[4], "S0": got[5]}
    h = 1e-6
    for i, name in enumerate(names):
        x = args[i]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            ap, am = list(args), list(args)
            ap[i], am[i] = xp, xm
            fd[idx] = (loss(ap) - loss(am)) / (2 * h)
        assert np.allclose(grads[name], fd, rtol=1e-6, atol=1e-8), name


def test_layer_backward_sums_over_value_heads():
    """Two value heads read one QK head: dq, dk are the sum of both chains' derivatives; packed
    sequences are independent. Finite differences over the layer forward."""
    rng = np.random.default_rng(22)
    cu = np.array([0, 3, 7])
    T, HK, HV, d = 7, 1, 2, 3
    q, k = rng.standard_normal((T, HK, d)), rng.standard_normal((T, HK, d))
    v = rng.standard_normal((T, HV, d))
    alpha, beta = rng.uniform(0.5, 1, (T, HV)), rng.uniform(0.1, 1, (T, HV))
    S0 = 0.3 * rng.standard_normal((2, HV, d, d))
    dy, dSf = rng.standard_normal((T, HV, d)), rng.standard_normal((2, HV, d, d))

    def loss(qq, kk):
        y, S = O.recurrence_layer(qq, kk, v, alpha, beta, S0, cu)
        return float(np.sum(dy * y) + np.sum(dSf * S))

    dq, dk, *_ = O.recurrence_layer_backward(q, k, v, alpha, beta, S0, cu, dy, dSf)
    h = 1e-6
    for x, g, which in ((q, dq, 0), (k, dk, 1)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            fd[idx] = ((loss(xp, k) - loss(xm, k)) if which == 0 else (loss(q, xp) - loss(q, xm))) / (2 * h)
        assert np.allclose(g, fd, rtol=1e-6, atol=1e-8)


def test_frozen_state_closed_form():
    """alpha = 1, beta = 0: the state never changes, y_t = S0^T q_t, so dq_t = S0 dy_t,
    dS0 = sum_t q_t dy_t^T + dS_L, and k, v get no gradient."""
    rng = np.random.default_rng(23)
    L, dk, dv = 9, 5, 4
    q, k, v, _, _, S0 = _chain(rng, L, dk, dv)
    dy, dSf = rng.standard_normal((L, dv)), rng.standard_normal((dk, dv))
    dq, dkk, dvv, _, _, dS0 = O.gated_delta_rule_backward(q, k, v, np.ones(L), np.zeros(L), S0, dy, dSf)
    assert np.allclose(dq, dy @ S0.T, rtol=1e-13)
    assert np.allclose(dS0, q.T @ dy + dSf, rtol=1e-13)
    assert np.all(dkk == 0) and np.all(dvv == 0)


def test_mixer_backward_matches_finite_differences():
    """The whole mixer (conv + SiLU, L2, recurrence, RMSNorm, gate) over a packed two-sequence layer with
    one QK head read by two value heads, conv history and initial states: every partial derivative of
    L = sum dout . o + <dS, S_final> by central differences of the oracle's gdn_prefill."""
    rng = np.random.default_rng(24)
    cu = np.array([0, 3, 8])
    T, hk, hv, d = 8, 1, 2, 4
    C = 2 * hk * d + hv * d
    inp = {"cu_seqlens": cu, "q": rng.standard_normal((T, hk, d)), "k": rng.standard_normal((T, hk, d)),
           "v": rng.standard_normal((T, hv, d)), "alpha": rng.uniform(0.5, 1, (T, hv)),
           "beta": rng.uniform(0.1, 1, (T, hv)), "gate": rng.standard_normal((T, hv, d)),
           "conv_w": 0.5 * rng.standard_normal((C, 4)), "norm_w": 0.2 * rng.standard_normal(d),
           "state_in": 0.3 * rng.standard_normal((2, hv, d, d)), "conv_in": rng.standard_normal((2, 3, C))}
    dout, dS = rng.standard_normal((T, hv, d)), rng.standard_normal((2, hv, d, d))

    def loss(x):
        o, S, _ = O.gdn_prefill(x)
        return float(np.sum(dout * o) + np.sum(dS * S))

    got = O.gdn_prefill_backward(inp, dout, dS)
    h = 1e-6
    for name in ("q", "k", "v", "alpha", "beta", "gate", "conv_w", "norm_w", "state_in", "conv_in"):
        x = inp[name]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = dict(inp), dict(inp)
            xp[name], xm[name] = x.copy(), x.copy()
            xp[name][idx] += h
            xm[name][idx] -= h
            fd[idx] = (loss(xp) - loss(xm)) / (2 * h)
        assert np.allclose(got[name], fd, rtol=1e-5, atol=1e-7), name
