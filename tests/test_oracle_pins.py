"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics, not by itself.

Each test names what it pins. The recurrence is checked against its second statement on the
pages (product form), exact rational brute force, closed-form special cases and invariants; the
conv against numpy.convolve; SiLU/sigmoid against torch; composition order by invariants that a
wrong order would break.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
from workloads import prefill_inputs, decode_inputs


def _rand_chain(rng, L, dk, dv, unit_k=True):
    q = rng.standard_normal((L, dk))
    k = rng.standard_normal((L, dk))
    if unit_k:
        q /= np.linalg.norm(q, axis=1, keepdims=True)
        k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((L, dv))
    alpha = np.exp(-0.1 * np.log1p(np.exp(rng.standard_normal(L))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(L)))
    S0 = 0.1 * rng.standard_normal((dk, dv))
    return q, k, v, alpha, beta, S0


# ---------------------------------------------------------------- recurrence ----------------

@pytest.mark.parametrize("unit_k", [True, False])
def test_error_form_equals_product_form(unit_k):
    """The two statements of the recurrence on the pages (error form, analysis notes §03;
    product form, paper reading §四 4.1) agree in fp64."""
    rng = np.random.default_rng(1)
    q, k, v, a, b, S0 = _rand_chain(rng, 64, 16, 16, unit_k)
    y1, S1 = O.gated_delta_rule(q, k, v, a, b, S0)
    y2, S2 = O.gated_delta_rule_product_form(q, k, v, a, b, S0)
    assert np.max(np.abs(y1 - y2)) < 1e-12 * max(1.0, np.max(np.abs(y2)))
    assert np.max(np.abs(S1 - S2)) < 1e-12 * max(1.0, np.max(np.abs(S2)))


def _frac_mat(a):
    return [[Fraction(x) for x in row] for row in a]


def _mm(A, B):
    return [[sum(A[i][t] * B[t][j] for t in range(len(B))) for j in range(len(B[0]))]
            for i in range(len(A))]


def _add(A, B):
    return [[A[i][j] + B[i][j] for j in range(len(A[0]))] for i in range(len(A))]


def _outer(a, b):
    return [[x * y for y in b] for x in a]


def _scal(c, A):
    return [[c * x for x in row] for row in A]


def _eye(n):
    return [[Fraction(int(i == j)) for j in range(n)] for i in range(n)]


@pytest.mark.parametrize("T", [1, 2, 3, 4])
def test_brute_force_unrolled_exact(T):
    """Exact rational brute force of the unrolled recurrence for T <= 4:
    S_T = prod_{t=T..1} M_t S0 + sum_i prod_{t=T..i+1} M_t beta_i k_i v_i^T,
    M_t = alpha_t (I - beta_t k_t k_t^T), built with explicit d x d matrices; y_t = S_t^T q_t."""
    rng = np.random.default_rng(10 + T)
    dk, dv = 3, 2
    # small dyadic rationals are exact in binary floating point
    q = rng.integers(-4, 5, (T, dk)) / 4.0
    k = rng.integers(-4, 5, (T, dk)) / 4.0
    v = rng.integers(-4, 5, (T, dv)) / 4.0
    alpha = rng.integers(1, 9, T) / 8.0
    beta = rng.integers(0, 9, T) / 8.0
    S0 = rng.integers(-4, 5, (dk, dv)) / 4.0
    Fq, Fk, Fv, FS0 = _frac_mat(q), _frac_mat(k), _frac_mat(v), _frac_mat(S0)
    Fa = [Fraction(x) for x in alpha]
    Fb = [Fraction(x) for x in beta]
    M = [_scal(Fa[t], _add(_eye(dk), _scal(-Fb[t], _outer(Fk[t], Fk[t])))) for t in range(T)]
    y_exact = []
    for tt in range(1, T + 1):          # S after tt tokens, by the unrolled sum
        prod_all = _eye(dk)
        for t in range(0, tt):          # prod_{t=tt..1} M_t = M_tt ... M_1
            prod_all = _mm(M[t], prod_all)
        S = _mm(prod_all, FS0)
        for i in range(tt):
            Pi = _eye(dk)
            for t in range(i + 1, tt):
                Pi = _mm(M[t], Pi)
            S = _add(S, _mm(Pi, _scal(Fb[i], _outer(Fk[i], Fv[i]))))
        y_exact.append([sum(S[r][c] * Fq[tt - 1][r] for r in range(dk)) for c in range(dv)])
    S_exact = np.array([[float(x) for x in row] for row in S])
    y_exact = np.array([[float(x) for x in row] for row in y_exact])
    y, S_or = O.gated_delta_rule(q, k, v, alpha, beta, S0)
    np.testing.assert_allclose(S_or, S_exact, rtol=0, atol=1e-13)
    np.testing.assert_allclose(y, y_exact, rtol=0, atol=1e-13)


def test_alpha_one_beta_zero_identity():
    """alpha = 1, beta = 0 leaves the state bit-identical and reads y_t = S0^T q_t."""
    rng = np.random.default_rng(2)
    q, k, v, _, _, S0 = _rand_chain(rng, 40, 16, 8)
    y, S = O.gated_delta_rule(q, k, v, np.ones(40), np.zeros(40), S0)
    assert np.array_equal(S, S0)
    np.testing.assert_allclose(y, q @ S0, rtol=1e-14, atol=1e-15)


def test_unit_key_full_write_reads_back_value():
    """With unit-norm k and beta = 1 the write makes S_t^T k_t = v_t exactly, for any alpha
    (analysis notes §03: read what k retrieves, write only the residual). Reading with q = k
    returns y_t = v_t."""
    rng = np.random.default_rng(3)
    q, k, v, a, _, S0 = _rand_chain(rng, 64, 16, 16)
    y, _ = O.gated_delta_rule(k, k, v, a, np.ones(64), S0)
    np.testing.assert_allclose(y, v, rtol=0, atol=1e-12)


def test_beta_zero_pure_decay():
    """beta = 0: S_T = (prod alpha) S0 and y_t = (prod_{s<=t} alpha_s) S0^T q_t."""
    rng = np.random.default_rng(4)
    q, k, v, a, _, S0 = _rand_chain(rng, 32, 8, 8)
    y, S = O.gated_delta_rule(q, k, v, a, np.zeros(32), S0)
    np.testing.assert_allclose(S, np.prod(a) * S0, rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(y, np.cumprod(a)[:, None] * (q @ S0), rtol=1e-12, atol=1e-15)


def test_linear_in_state_and_values():
    """For fixed q, k, alpha, beta the map (S0, V) -> (S_T, Y) is linear (superposition)."""
    rng = np.random.default_rng(5)
    q, k, v1, a, b, S01 = _rand_chain(rng, 48, 16, 12)
    v2 = rng.standard_normal(v1.shape)
    S02 = rng.standard_normal(S01.shape)
    c1, c2 = 0.7, -1.3
    y1, S1 = O.gated_delta_rule(q, k, v1, a, b, S01)
    y2, S2 = O.gated_delta_rule(q, k, v2, a, b, S02)
    y3, S3 = O.gated_delta_rule(q, k, c1 * v1 + c2 * v2, a, b, c1 * S01 + c2 * S02)
    np.testing.assert_allclose(y3, c1 * y1 + c2 * y2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(S3, c1 * S1 + c2 * S2, rtol=0, atol=1e-12)


def test_non_expansive_with_zero_values():
    """With V = 0, unit k and beta in [0, 1]: ||S_t||_2 <= alpha_t ||S_{t-1}||_2."""
    rng = np.random.default_rng(6)
    q, k, v, a, b, S = _rand_chain(rng, 64, 16, 16)
    for t in range(64):
        _, S_new = O.gated_delta_rule(q[t:t + 1], k[t:t + 1], np.zeros((1, 16)), a[t:t + 1],
                                      b[t:t + 1], S)
        assert np.linalg.norm(S_new, 2) <= a[t] * np.linalg.norm(S, 2) * (1 + 1e-12) + 1e-15
        S = S_new


def test_idempotent_write():
    """Repeating the same unit (k, v) with alpha = beta = 1 leaves S fixed after the first step."""
    rng = np.random.default_rng(7)
    q, k, v, _, _, S0 = _rand_chain(rng, 5, 8, 8)
    kk = np.repeat(k[:1], 5, axis=0)
    vv = np.repeat(v[:1], 5, axis=0)
    S = S0
    states = []
    for t in range(5):
        _, S = O.gated_delta_rule(q[t:t + 1], kk[t:t + 1], vv[t:t + 1], np.ones(1), np.ones(1), S)
        states.append(S)
    for s in states[1:]:
        np.testing.assert_allclose(s, states[0], rtol=0, atol=1e-13)


# ---------------------------------------------------------------- conv / SiLU / L2 / norm -----

def test_conv_identity_and_shift_taps():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((10, 5))
    hist = rng.standard_normal((3, 5))
    w_id = np.tile([0.0, 0.0, 0.0, 1.0], (5, 1))
    np.testing.assert_array_equal(O.short_conv(x, w_id, hist), x)
    w_sh = np.tile([0.0, 0.0, 1.0, 0.0], (5, 1))
    u = O.short_conv(x, w_sh, hist)
    np.testing.assert_array_equal(u[1:], x[:-1])
    np.testing.assert_array_equal(u[0], hist[-1])


def test_conv_matches_numpy_convolve_and_is_causal():
    rng = np.random.default_rng(9)
    L, C = 37, 6
    x = rng.standard_normal((L, C))
    hist = rng.standard_normal((3, C))
    w = rng.standard_normal((C, 4))
    u = O.short_conv(x, w, hist)
    for c in range(C):
        xx = np.concatenate([hist[:, c], x[:, c]])
        ref = np.convolve(xx, w[c][::-1])[3:L + 3]
        np.testing.assert_allclose(u[:, c], ref, rtol=1e-13, atol=1e-13)
    t0 = 11
    x2 = x.copy()
    x2[t0] += 1.0
    du = np.abs(O.short_conv(x2, w, hist) - u).max(axis=1)
    assert np.all(du[:t0] == 0) and np.all(du[t0 + 4:] == 0) and np.all(du[t0:t0 + 4] > 0)


def test_silu_sigmoid_vs_torch():
    z = np.linspace(-30, 30, 1001)
    zt = torch.from_numpy(z)
    np.testing.assert_allclose(O.silu(z), torch.nn.functional.silu(zt).numpy(), rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(O.sigmoid(z), torch.sigmoid(zt).numpy(), rtol=1e-14, atol=1e-300)
    assert O.silu(np.array(0.0)) == 0.0 and O.sigmoid(np.array(0.0)) == 0.5


def test_l2_unit_norm():
    rng = np.random.default_rng(11)
    a = rng.standard_normal((20, 128)) * 3
    n = np.linalg.norm(O.l2_normalize(a, 1e-6), axis=1)
    np.testing.assert_allclose(n, 1.0, rtol=1e-7)


def test_rmsnorm_unit_mean_square_and_scale_invariance():
    rng = np.random.default_rng(12)
    y = rng.standard_normal((20, 128))
    r = O.zero_centred_rmsnorm(y, np.zeros(128), 1e-6)
    np.testing.assert_allclose(np.mean(r * r, axis=1), 1.0, rtol=1e-5)
    w = 0.02 * rng.standard_normal(128)
    np.testing.assert_allclose(O.zero_centred_rmsnorm(5.0 * y, w, 0.0), O.zero_centred_rmsnorm(y, w, 0.0),
                               rtol=1e-13)


def test_rmsnorm_constant_row_closed_form():
    """No mean subtraction: a constant row y = c * 1 normalises to c / sqrt(c^2 + eps) * (1 + w)
    channel by channel (about sign(c) (1 + w)); a mean-subtracting (LayerNorm-style) norm would map it
    to zero. Closed form written out by hand for c = -3, eps = 1e-6."""
    w = np.linspace(-0.05, 0.05, 16)
    r = O.zero_centred_rmsnorm(np.full((1, 16), -3.0), w, 1e-6)
    np.testing.assert_allclose(r[0], -3.0 / np.sqrt(9.0 + 1e-6) * (1.0 + w), rtol=1e-15)
    assert np.all(r[0] < -0.9)
    # a large common offset plus small noise stays near sign(c) (1 + w) instead of amplifying the noise
    rng = np.random.default_rng(13)
    y = 5.0 + 1e-3 * rng.standard_normal((8, 128))
    r = O.zero_centred_rmsnorm(y, np.zeros(128), 1e-6)
    np.testing.assert_allclose(r, 1.0, atol=1e-3)


def test_rmsnorm_fixed_vector_by_hand():
    """y = (1, 2, 3, 4), w = (0, 0.5, -0.5, 1), eps = 0: mean(y^2) = 30 / 4 = 7.5, so
    r = y / sqrt(7.5) * (1 + w) = (1, 3, 1.5, 8) / sqrt(7.5). (A centred norm gives
    (-1.5, -0.5, 0.5, 1.5) / sqrt(1.25) * (1 + w) instead.)"""
    r = O.zero_centred_rmsnorm(np.array([[1.0, 2.0, 3.0, 4.0]]), np.array([0.0, 0.5, -0.5, 1.0]), 0.0)
    np.testing.assert_allclose(r[0], np.array([1.0, 3.0, 1.5, 8.0]) / np.sqrt(7.5), rtol=1e-15)


# ---------------------------------------------------------------- whole mixer -----------------

def test_rmsnorm_per_head_gain_and_scale_through_the_chain():
    """A per-head gain w[HV][d_v] reaches each value head with its own row, and the readout scale
    multiplies the raw y (flags without NORM) but cancels under the norm up to eps."""
    inp = _small([40], hk=1, hv=3)
    rng = np.random.default_rng(14)
    inp["norm_w"] = torch.from_numpy(0.1 * rng.standard_normal((3, 16)))
    for h in range(3):
        shared = dict(inp)
        shared["norm_w"] = inp["norm_w"][h]
        np.testing.assert_array_equal(O.prefill_chain(inp, 0, h)[0], O.prefill_chain(shared, 0, h)[0])
    f = O.FLAG_CONV | O.FLAG_L2QK
    y1, S1 = O.prefill_chain(inp, 0, 1, flags=f)
    y2, S2 = O.prefill_chain(inp, 0, 1, flags=f, scale=0.5)
    np.testing.assert_allclose(y2, 0.5 * y1, rtol=1e-14, atol=1e-15)
    np.testing.assert_array_equal(S1, S2)
    o1, _ = O.prefill_chain(inp, 0, 1, norm_eps=0.0)
    o2, _ = O.prefill_chain(inp, 0, 1, scale=0.5, norm_eps=0.0)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-14)



def _small(lengths, hk=2, hv=6, d=16, seed=0, **kw):
    inp = prefill_inputs(lengths, n_qk_heads=hk, n_v_heads=hv, d_k=d, d_v=d, io_dtype=torch.float32,
                         seed=seed, **kw)
    return vars(inp)


def test_norm_then_gate_order():
    """Head outputs are normalised, then gated (paper summary, Method): with gain w = 0,
    o / sigmoid(gate) has unit mean square per row; gating first would not."""
    inp = _small([50], hk=1, hv=1)
    inp["norm_w"] = torch.zeros_like(inp["norm_w"])
    o, S = O.prefill_chain(inp, 0, 0, norm_eps=0.0)
    g = O.sigmoid(inp["gate"][:, 0].double().numpy())
    np.testing.assert_allclose(np.mean((o / g) ** 2, axis=1), 1.0, rtol=1e-10)


def test_l2_applies_to_q_k_not_v():
    """Queries and keys are L2-normalised, values are not: without conv, scaling q or k leaves y
    unchanged while scaling v scales y."""
    inp = _small([30], hk=1, hv=1)
    f = O.FLAG_L2QK
    y0, _ = O.prefill_chain(inp, 0, 0, flags=f, l2_eps=0.0)
    for key, factor, expect in (("q", 4.0, 1.0), ("k", 0.5, 1.0), ("v", 2.0, 2.0)):
        inp2 = dict(inp)
        inp2[key] = inp[key] * factor
        y, _ = O.prefill_chain(inp2, 0, 0, flags=f, l2_eps=0.0)
        np.testing.assert_allclose(y, expect * y0, rtol=1e-10, atol=1e-12)


def test_value_head_reads_its_qk_group():
    """Value head h reads QK head floor(h * HK / HV): perturbing QK head 1 leaves value heads 0..2
    unchanged and changes heads 3..5."""
    inp = _small([20], hk=2, hv=6)
    o, S, _ = O.gdn_prefill(inp)
    inp2 = dict(inp)
    q2 = inp["q"].clone()
    q2[:, 1] += 1.0
    inp2["q"] = q2
    o2, S2, _ = O.gdn_prefill(inp2)
    assert np.array_equal(o[:, :3], o2[:, :3])
    assert np.all(np.abs(o[:, 3:] - o2[:, 3:]).max(axis=(0, 2)) > 0)


def test_conv_channel_order_q_k_v():
    """Conv taps are indexed q | k | v by channel: identity taps on all channels reproduce
    SiLU of the raw inputs of the chain's own heads."""
    inp = _small([12], hk=2, hv=4, d=8)
    inp["conv_w"] = torch.tensor([0.0, 0.0, 0.0, 1.0]).repeat(inp["conv_w"].shape[0], 1)
    for h in range(4):
        g = h // 2
        y, S = O.prefill_chain(inp, 0, h, flags=O.FLAG_CONV)
        f = lambda t: O.silu(t.double().numpy())
        y_ref, S_ref = O.gated_delta_rule(f(inp["q"][:, g]), f(inp["k"][:, g]), f(inp["v"][:, h]),
                                          inp["alpha"][:, h].double().numpy(),
                                          inp["beta"][:, h].double().numpy(), np.zeros((8, 8)))
        np.testing.assert_array_equal(y, y_ref)


def test_packed_equals_separate():
    """Sequences packed by cu_seqlens are independent: packed == separate runs, bitwise."""
    lengths = [7, 1, 20, 3]
    inp = _small(lengths, s0_std=0.1, conv_in_std=1.0)
    o, S, c = O.gdn_prefill(inp)
    cu = inp["cu_seqlens"].numpy()
    for n, L in enumerate(lengths):
        s0, s1 = cu[n], cu[n + 1]
        one = {k: v for k, v in inp.items()}
        for key in ("q", "k", "v", "alpha", "beta", "gate"):
            one[key] = inp[key][s0:s1]
        one["state_in"] = inp["state_in"][n:n + 1]
        one["conv_in"] = inp["conv_in"][n:n + 1]
        one["cu_seqlens"] = np.array([0, L])
        o1, S1, c1 = O.gdn_prefill(one)
        assert np.array_equal(o1, o[s0:s1]) and np.array_equal(S1[0], S[n]) and np.array_equal(c1[0], c[n])


def test_empty_sequences_pass_through():
    """A zero-length sequence in a packed batch produces no output rows, keeps its initial state
    and conv cache exactly, and leaves its neighbours as they are without it."""
    lengths = [0, 7, 0, 3, 0]
    inp = _small(lengths, s0_std=0.1, conv_in_std=1.0)
    o, S, c = O.gdn_prefill(inp)
    assert o.shape[0] == sum(lengths)
    for n in (0, 2, 4):
        assert np.array_equal(S[n], inp["state_in"][n].double().numpy())
        assert np.array_equal(c[n], inp["conv_in"][n].double().numpy())
    keep = [1, 3]
    dense = {k: v for k, v in inp.items()}
    dense["state_in"] = inp["state_in"][keep]
    dense["conv_in"] = inp["conv_in"][keep]
    dense["cu_seqlens"] = np.array([0, 7, 10])
    o2, S2, c2 = O.gdn_prefill(dense)
    assert np.array_equal(o2, o) and np.array_equal(S2, S[keep]) and np.array_equal(c2, c[keep])


@pytest.mark.parametrize("T1", [1, 2, 5, 17])
def test_continuation_and_decode(T1):
    """prefill(T1 + T2) == prefill(T1) -> (state, conv tail) -> prefill(T2), bitwise; and the
    last token equals a decode step from the state of the first T-1 tokens."""
    T = 24
    inp = _small([T], s0_std=0.1, conv_in_std=1.0)
    o, S, c = O.gdn_prefill(inp)

    def part(a, b, st, ci):
        p = {k: v for k, v in inp.items()}
        for key in ("q", "k", "v", "alpha", "beta", "gate"):
            p[key] = inp[key][a:b]
        p["cu_seqlens"] = np.array([0, b - a])
        p["state_in"], p["conv_in"] = st, ci
        return O.gdn_prefill(p)

    oa, Sa, ca = part(0, T1, inp["state_in"], inp["conv_in"])
    ob, Sb, cb = part(T1, T, Sa, ca)
    assert np.array_equal(np.concatenate([oa, ob]), o)
    assert np.array_equal(Sb, S) and np.array_equal(cb, c)
    # decode of the last token
    oa, Sa, ca = part(0, T - 1, inp["state_in"], inp["conv_in"])
    step = {key: inp[key][T - 1:T] for key in ("q", "k", "v", "alpha", "beta", "gate")}
    od, Sd, cd = O.gdn_decode(step, Sa, ca, inp["conv_w"], inp["norm_w"])
    assert np.array_equal(od[0], o[T - 1]) and np.array_equal(Sd, S) and np.array_equal(cd, c)


def test_short_sequences_take_history_from_conv_in():
    """A sequence shorter than the conv window reads the rest of its window from conv_in, and
    its conv tail keeps the newest entries of conv_in."""
    inp = _small([1, 2], conv_in_std=1.0)
    o, S, c = O.gdn_prefill(inp)
    ci = inp["conv_in"].double().numpy()
    x0 = torch.cat([inp["q"][0].reshape(-1), inp["k"][0].reshape(-1), inp["v"][0].reshape(-1)]).double().numpy()
    np.testing.assert_array_equal(c[0][:2], ci[0][1:])
    np.testing.assert_array_equal(c[0][2], x0)
    np.testing.assert_array_equal(c[1][0], ci[1][2])


# ------------------------------------------------------------- speculative verify / commit -----

def _drafts(B, K, hk=2, hv=4, d=8, seed=5):
    """K draft tokens for B sequences: the step-major draw of decode_inputs, re-laid out with the
    drafts of sequence b in rows b*K .. b*K+K-1, plus the same steps kept step-major."""
    di = decode_inputs(B, K, n_qk_heads=hk, n_v_heads=hv, d_k=d, d_v=d, io_dtype=torch.float32,
                       seed=seed, state_std=0.1)
    steps = {key: getattr(di, key) for key in ("q", "k", "v", "alpha", "beta", "gate")}
    packed = {key: x.transpose(0, 1).reshape(B * K, *x.shape[2:]) for key, x in steps.items()}
    return di, steps, packed


def _decode_run(di, steps, n_steps):
    """The oracle's one-token decode step applied n_steps times per sequence, cache carried."""
    S, c = di.state, di.conv_state
    outs = []
    for t in range(n_steps):
        step = {key: x[t] for key, x in steps.items()}
        o, S, c = O.gdn_decode(step, S, c, di.conv_w, di.norm_w)
        outs.append(o)
    return outs, S, c


def test_verify_equals_token_by_token_decode():
    """Verifying K drafts in one pass gives, token for token, the outputs of K decode steps, and
    leaves the cache it reads untouched."""
    B, K = 3, 4
    di, steps, packed = _drafts(B, K)
    S0, c0 = di.state.clone(), di.conv_state.clone()
    o = O.gdn_verify(packed, di.state, di.conv_state, di.conv_w, di.norm_w, n_tok=K)
    outs, _, _ = _decode_run(di, steps, K)
    for t in range(K):
        assert np.array_equal(o.reshape(B, K, *o.shape[1:])[:, t], outs[t])
    assert torch.equal(di.state, S0) and torch.equal(di.conv_state, c0)


@pytest.mark.parametrize("n_accept", [[0, 0, 0], [4, 4, 4], [0, 4, 2], [1, 3, 0]])
def test_commit_equals_accepted_decode_steps(n_accept):
    """Committing n of the K drafts leaves exactly the cache of n decode steps (n = 0: the cache
    unchanged), per sequence."""
    B, K = 3, 4
    di, steps, packed = _drafts(B, K)
    S, c = O.gdn_commit(packed, np.array(n_accept), di.state, di.conv_state, di.conv_w, di.norm_w, n_tok=K)
    for b, n in enumerate(n_accept):
        one = {key: x[:, b:b + 1] for key, x in steps.items()}
        sub = type("D", (), {})()
        sub.state, sub.conv_state = di.state[b:b + 1], di.conv_state[b:b + 1]
        sub.conv_w, sub.norm_w = di.conv_w, di.norm_w
        _, Sn, cn = _decode_run(sub, one, n)
        as64 = lambda x: x.double().numpy() if torch.is_tensor(x) else np.asarray(x, dtype=np.float64)
        assert np.array_equal(S[b], as64(Sn)[0]) and np.array_equal(c[b], as64(cn)[0])
    for b, n in enumerate(n_accept):
        if n == 0:
            assert np.array_equal(S[b], di.state[b].double().numpy())


# ------------------------------------------------------------------ projections and gates -------

def test_in_projection_matches_brute_force():
    """q | k | v, z and the gate pre-activations are plain products x W: checked against explicit
    loops on a tiny layer, and the gates against their formula written per element."""
    from workloads import projection_inputs
    p = projection_inputs(3, hidden=5, n_qk_heads=1, n_v_heads=2, d_k=2, d_v=2, io_dtype=torch.float32, seed=2)
    qkv, z, alpha, beta = O.in_projection(p.x, p.w_qkv.T, p.w_z.T, p.w_ab.T, p.a_log, p.dt_bias)
    x = p.x.double().tolist()

    def mm(w):  # x W^T for a weight in the [out][in] layout, by explicit loops
        w = w.double().T.tolist()
        return [[sum(x[t][i] * w[i][j] for i in range(len(w))) for j in range(len(w[0]))] for t in range(len(x))]
    np.testing.assert_allclose(qkv, mm(p.w_qkv), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(z, mm(p.w_z), rtol=1e-13, atol=1e-14)
    ab = mm(p.w_ab)
    import math
    for t in range(3):
        for h in range(2):
            u = ab[t][h] + float(p.dt_bias[h])
            sp = math.log(1.0 + math.exp(u))
            assert abs(alpha[t, h] - math.exp(-math.exp(float(p.a_log[h])) * sp)) < 1e-14
            assert abs(beta[t, h] - 1.0 / (1.0 + math.exp(-ab[t][2 + h]))) < 1e-14


def test_gate_limits():
    """alpha -> 1 when the decay rate exp(A) -> 0 or the pre-activation -> -inf; alpha is
    decreasing in a; beta = 1/2 at b = 0; softplus(0) = ln 2 and softplus(x) ~ x for large x."""
    a = np.array([[-50.0, 0.0, 3.0, 40.0]])
    b = np.array([[0.0, -40.0, 2.0, 40.0]])
    al, be = O.gate_alpha_beta(a, b, np.full(4, -60.0), np.zeros(4))
    np.testing.assert_allclose(al, 1.0, rtol=0, atol=1e-20)
    al, be = O.gate_alpha_beta(a, b, np.zeros(4), np.zeros(4))
    assert al[0, 0] >= 1 - 1e-15 and np.all(np.diff(al[0]) < 0)
    assert abs(al[0, 1] - 0.5) < 1e-15  # exp(-ln 2)
    assert abs(np.log(al[0, 3]) + 40.0) < 1e-12
    assert be[0, 0] == 0.5 and be[0, 1] < 1e-17 and abs(be[0, 3] - 1.0) < 1e-17
    assert abs(O.softplus(0.0) - np.log(2.0)) < 1e-16 and O.softplus(800.0) == 800.0


def test_out_projection_is_a_product():
    o = np.arange(6.0).reshape(2, 3)
    w = np.array([[1.0, 0.0], [0.0, 2.0], [1.0, -1.0]])
    np.testing.assert_array_equal(O.out_projection(o, w), [[2.0, 0.0], [8.0, 3.0]])
