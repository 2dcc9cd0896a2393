"""fp64 CPU oracle of the Gated DeltaNet (GDN) token mixer.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the benchmark's CPU-baseline
leg may import this module. The HIP library never calls it, and it shares no code with the
library: it is the plain, slow definition the GPU results are checked against.

Sources (the pages this follows; all quoted facts are restated, not copied):
  [P2] "Qwen3.8-Flash-Next：架构、效率与技术谱系" (technical-report analysis notes)
       §02 configuration table, GDN row: 48 value heads / 16 QK heads, head dim 128, short conv
       kernel 4, Q/K/V go through the short causal conv.
       §03 Gated DeltaNet, update equations: decay the state by alpha, read the error
       e = v - S~^T k, write S = S~ + beta k e^T, read out y = S^T q; alpha and beta in (0, 1).
       §03 "what Qwen changed": sigmoid output gate (instead of SiLU) and zero-centred RMSNorm.
  [P3] "On the Design of Qwen3.8-Next Architecture … 精读" §四 4.1: product form of the same
       recurrence, S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T, and q/k pass a
       short conv + SiLU + L2 normalisation.
  [P5] "Qwen3.8-Flash-Next" paper summary (hyper.ai, English), Method: learned projections then
       short depthwise causal convolutions; L2-normalised queries and keys; head outputs are
       normalised and then modulated by a sigmoid output gate. Results: four-step speculative
       decoding with multi-token prediction (MTP), mean accepted length about 4.
  [P2] §01 (MTP row: one layer trained for multi-step prediction) and the §04 results table
       (four-step MTP accepted length): drafts of several tokens are checked in one pass.
  [P2] §04 (QSA indexer data flow): 4 query heads and 1 key head; keys average-pooled over 4-token
       micro-blocks, RMS-normalised, then given partial RoPE at the block's start position; block
       score = sum over heads of ReLU(q . k_b), only for blocks already complete; the top 512 blocks
       (2048 tokens) are kept and the incomplete tail block is always added.
  [P1] paper reading "Qwen3.8-Flash-Next" (方法): the normalised residual stream goes through
       learned projections, then the short conv; a data-dependent decay gate sets how long the
       state lives and a write gate scales the delta update.
  [P2] §07 optimizer table: the GDN input is one fused matrix in Megatron made of independent
       operators (q, k, v, ...), the GDN input and output projections are 2-D weights, and the GDN
       alpha / beta parameters are vectors.

Readings where the pages are silent (every one is also listed in the design notes):
  * conv + SiLU on q, k and v; L2 on q and k only.
  * conv tap 3 multiplies the current token, taps 0..2 the three previous ones; no bias; the
    history before a sequence start is ``conv_in`` (zeros when absent).
  * L2: a / sqrt(sum(a^2) + l2_eps);  RMSNorm: y / sqrt(mean(y^2) + norm_eps) * (1 + w).
  * value head h reads QK head floor(h * HK / HV) (contiguous groups).
  * the state is stored [d_k][d_v] (row = key index); y carries an optional ``scale`` (1.0).
  * QSA indexer (what the pages leave open): RMSNorm of the pooled key is m / sqrt(mean(m^2) +
    1e-6) * w; partial RoPE rotates dims d and d + 32 (d < 32) of the first 64 by position * 1e4^(-d/32),
    queries at their token index, compressed keys at 4b; ties in the top-k go to the lower block.
  * projections (the pages give no formula for the gates): q | k | v = x W_qkv, gate logits
    z = x W_z, gate pre-activations [a | b] = x W_ab, then beta = sigmoid(b) and
    alpha = exp(-exp(A_h) * softplus(a + delta_h)) with per-head vectors A, delta; the output
    projection is y = o W_out.

Flags mirror the library's stage switches: CONV (conv + SiLU), L2QK, NORM, GATE.
"""
from __future__ import annotations

import numpy as np

FLAG_CONV = 1
FLAG_L2QK = 2
FLAG_NORM = 4
FLAG_GATE = 8
FLAG_ALL = 15
CONV_WIDTH = 4


def silu(u):
    """SiLU, u * sigmoid(u) ([P3] §四 4.1: SiLU after the short conv)."""
    with np.errstate(over="ignore"):
        return u / (1.0 + np.exp(-u))


def sigmoid(z):
    """Logistic function of the output gate ([P2] §03: the output gate is a sigmoid)."""
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def short_conv(x, w, hist):
    """Causal depthwise conv of width 4 ([P2] §02 GDN row; [P5] Method).

    x: [L, C] raw inputs of one sequence; w: [C, 4] taps; hist: [3, C] the three inputs before
    the sequence start, oldest first. Returns u[t, c] = sum_j w[c, j] * x[t - 3 + j, c].
    """
    L = x.shape[0]
    xx = np.concatenate([hist, x], axis=0)          # xx[t + 3] = x[t]
    u = np.zeros((L, x.shape[1]), dtype=np.float64)
    for j in range(CONV_WIDTH):
        u += w[:, j][None, :] * xx[j:j + L]
    return u


def l2_normalize(a, eps):
    """Row-wise L2 normalisation of queries and keys ([P5] Method; [P3] §四 4.1)."""
    return a / np.sqrt(np.sum(a * a, axis=-1, keepdims=True) + eps)


def gated_delta_rule(q, k, v, alpha, beta, S0, scale=1.0):
    """Gated delta rule, error form ([P2] §03 update equations), one token at a time.

    q, k: [L, d_k]; v: [L, d_v]; alpha, beta: [L]; S0: [d_k, d_v].
    For each t:  S~ = alpha_t S;  e = v_t - S~^T k_t;  S = S~ + beta_t k_t e^T;  y_t = S^T q_t.
    Returns (y [L, d_v], S_final [d_k, d_v]).
    """
    S = np.array(S0, dtype=np.float64, copy=True)
    L, d_v = v.shape
    y = np.empty((L, d_v), dtype=np.float64)
    for t in range(L):
        S_tilde = alpha[t] * S
        e = v[t] - S_tilde.T @ k[t]
        S = S_tilde + beta[t] * np.outer(k[t], e)
        y[t] = scale * (S.T @ q[t])
    return y, S


def gated_delta_rule_product_form(q, k, v, alpha, beta, S0, scale=1.0):
    """The same recurrence in product form ([P3] §四 4.1), kept only to pin the error form:
    S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T;  y_t = S_t^T q_t."""
    S = np.array(S0, dtype=np.float64, copy=True)
    L, d_v = v.shape
    eye = np.eye(k.shape[1])
    y = np.empty((L, d_v), dtype=np.float64)
    for t in range(L):
        S = alpha[t] * (eye - beta[t] * np.outer(k[t], k[t])) @ S + beta[t] * np.outer(k[t], v[t])
        y[t] = scale * (S.T @ q[t])
    return y, S


def gated_delta_rule_backward(q, k, v, alpha, beta, S0, dy, dS_final=None, scale=1.0):
    """Reverse-mode derivatives of gated_delta_rule for one chain: given dL/dy_t (dy [L, d_v]) and
    dL/dS_L (dS_final [d_k, d_v], None = 0), returns (dq, dk, dv, dalpha, dbeta, dS0).

    The forward states are recomputed and kept; the reverse loop takes the statements of the error
    form ([P2] §03 update equations) last to first and applies the chain rule to each:
      y_t = scale S_t^T q_t        ->  dS += scale q_t dy_t^T,  dq_t = scale S_t dy_t
      S_t = S~ + beta_t k_t e^T    ->  dbeta_t = k_t^T dS e,  dk_t = beta_t dS e,  de = beta_t dS^T k_t,
                                       dS~ = dS
      e = v_t - S~^T k_t           ->  dv_t = de,  dS~ -= k_t de^T,  dk_t -= S~ de
      S~ = alpha_t S_{t-1}         ->  dalpha_t = <S_{t-1}, dS~>,  dS_{t-1} = alpha_t dS~
    """
    q, k, v, dy = _f64(q), _f64(k), _f64(v), _f64(dy)
    L, d_v = v.shape
    d_k = k.shape[1]
    states = [np.array(_f64(S0), dtype=np.float64, copy=True)]
    errs = []
    for t in range(L):
        S_tilde = alpha[t] * states[-1]
        e = v[t] - S_tilde.T @ k[t]
        errs.append(e)
        states.append(S_tilde + beta[t] * np.outer(k[t], e))
    dS = np.zeros((d_k, d_v)) if dS_final is None else np.array(_f64(dS_final), dtype=np.float64, copy=True)
    dq, dk, dv = np.zeros((L, d_k)), np.zeros((L, d_k)), np.zeros((L, d_v))
    dalpha, dbeta = np.zeros(L), np.zeros(L)
    for t in range(L - 1, -1, -1):
        S_t, S_prev, e = states[t + 1], states[t], errs[t]
        dS = dS + scale * np.outer(q[t], dy[t])
        dq[t] = scale * (S_t @ dy[t])
        dbeta[t] = k[t] @ dS @ e
        de = beta[t] * (dS.T @ k[t])
        dk[t] = beta[t] * (dS @ e)
        dv[t] = de
        S_tilde = alpha[t] * S_prev
        dS_tilde = dS - np.outer(k[t], de)
        dk[t] -= S_tilde @ de
        dalpha[t] = np.sum(S_prev * dS_tilde)
        dS = alpha[t] * dS_tilde
    return dq, dk, dv, dalpha, dbeta, dS


def recurrence_layer(q, k, v, alpha, beta, S0, cu, *, scale=1.0):
    """The recurrence over a packed layer: q, k [T, HK, d_k], v [T, HV, d_v], alpha, beta [T, HV],
    S0 [N, HV, d_k, d_v] or None; value head h reads QK head floor(h HK / HV). Returns (y [T, HV, d_v],
    S_final [N, HV, d_k, d_v])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    alpha, beta = _f64(alpha), _f64(beta)
    T, HK, d_k = k.shape
    HV, d_v = v.shape[1], v.shape[2]
    cu = np.asarray(cu)
    N = len(cu) - 1
    y = np.zeros((T, HV, d_v))
    S_fin = np.zeros((N, HV, d_k, d_v))
    for n in range(N):
        a, b = int(cu[n]), int(cu[n + 1])
        for h in range(HV):
            g = h * HK // HV
            s0 = np.zeros((d_k, d_v)) if S0 is None else _f64(S0)[n, h]
            y[a:b, h], S_fin[n, h] = gated_delta_rule(q[a:b, g], k[a:b, g], v[a:b, h], alpha[a:b, h],
                                                      beta[a:b, h], s0, scale)
    return y, S_fin


def recurrence_layer_backward(q, k, v, alpha, beta, S0, cu, dy, dS_final=None, *, scale=1.0):
    """Derivatives of recurrence_layer: (dq, dk [T, HK, d_k] -- summed over the value heads that read
    each QK head --, dv [T, HV, d_v], dalpha, dbeta [T, HV], dS0 [N, HV, d_k, d_v])."""
    q, k, v, dy = _f64(q), _f64(k), _f64(v), _f64(dy)
    alpha, beta = _f64(alpha), _f64(beta)
    T, HK, d_k = k.shape
    HV, d_v = v.shape[1], v.shape[2]
    cu = np.asarray(cu)
    N = len(cu) - 1
    dq, dk = np.zeros((T, HK, d_k)), np.zeros((T, HK, d_k))
    dv, da, db = np.zeros((T, HV, d_v)), np.zeros((T, HV)), np.zeros((T, HV))
    dS0 = np.zeros((N, HV, d_k, d_v))
    for n in range(N):
        a, b = int(cu[n]), int(cu[n + 1])
        for h in range(HV):
            g = h * HK // HV
            s0 = np.zeros((d_k, d_v)) if S0 is None else _f64(S0)[n, h]
            dsf = None if dS_final is None else _f64(dS_final)[n, h]
            r = gated_delta_rule_backward(q[a:b, g], k[a:b, g], v[a:b, h], alpha[a:b, h], beta[a:b, h], s0,
                                          dy[a:b, h], dsf, scale)
            dq[a:b, g] += r[0]
            dk[a:b, g] += r[1]
            dv[a:b, h], da[a:b, h], db[a:b, h], dS0[n, h] = r[2], r[3], r[4], r[5]
    return dq, dk, dv, da, db, dS0


def zero_centred_rmsnorm(y, w, eps):
    """RMSNorm over the d_v channels of one head with gain (1 + w) ([P2] §03: zero-centred
    RMSNorm; [P5] Method: head outputs are normalised)."""
    return y / np.sqrt(np.mean(y * y, axis=-1, keepdims=True) + eps) * (1.0 + w)


def _f64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):          # a torch tensor: exact upcast of its values
        a = a.detach().to("cpu").double().numpy()
    return np.asarray(a, dtype=np.float64)


def _head_channels(h, g, hk, hv, dk, dv):
    """Channel index ranges (q | k | v order) of QK head g and value head h."""
    q0 = g * dk
    k0 = hk * dk + g * dk
    v0 = 2 * hk * dk + h * dv
    return slice(q0, q0 + dk), slice(k0, k0 + dk), slice(v0, v0 + dv)


def gdn_chain(xq, xk, xv, wq, wk, wv, hq, hk_, hv_, alpha, beta, gate, norm_w, S0, *,
              flags=FLAG_ALL, scale=1.0, l2_eps=1e-6, norm_eps=1e-6):
    """The whole mixer for one (sequence, value head) chain.

    xq, xk: [L, d_k] raw inputs of the chain's QK head; xv: [L, d_v] raw values;
    wq/wk/wv: their conv taps [·, 4]; hq/hk_/hv_: their conv history [3, ·];
    alpha, beta: [L]; gate: [L, d_v] logits; norm_w: [d_v]; S0: [d_k, d_v].
    Steps: conv + SiLU, L2(q, k), gated delta rule, RMSNorm, sigmoid gate.
    Returns (o [L, d_v], S_final [d_k, d_v]).
    """
    if flags & FLAG_CONV:
        aq = silu(short_conv(xq, wq, hq))
        ak = silu(short_conv(xk, wk, hk_))
        av = silu(short_conv(xv, wv, hv_))
    else:
        aq, ak, av = xq, xk, xv
    if flags & FLAG_L2QK:
        aq = l2_normalize(aq, l2_eps)
        ak = l2_normalize(ak, l2_eps)
    y, S = gated_delta_rule(aq, ak, av, alpha, beta, S0, scale)
    o = y
    if flags & FLAG_NORM:
        o = zero_centred_rmsnorm(o, norm_w, norm_eps)
    if flags & FLAG_GATE:
        o = o * sigmoid(gate)
    return o, S


def gdn_chain_backward(xq, xk, xv, wq, wk, wv, hq, hk_, hv_, alpha, beta, gate, norm_w, S0, do, dS_final=None,
                       *, scale=1.0, l2_eps=1e-6, norm_eps=1e-6):
    """Reverse-mode derivatives of gdn_chain with every step on, for one (sequence, value head) chain:
    given dL/do (do [L, d_v]) and dL/dS_final, returns a dict of the derivatives for xq, xk, xv, wq, wk,
    wv, hq, hk, hv, alpha, beta, gate, norm_w and S0. Each step of the forward is taken last to first:
      o = n * sigmoid(gate)              ->  dn = do * s,  dgate = do * n * s (1 - s)
      n = y / r * (1 + w),  r = sqrt(mean(y^2) + eps)
                                         ->  dw = sum_t dn * y / r,
                                             dy = (1 + w) dn / r - y <(1 + w) dn, y> / (d_v r^3)
      the recurrence                     ->  gated_delta_rule_backward
      a = a0 / sqrt(|a0|^2 + eps)        ->  da0 = (da - a <a, da>) / sqrt(|a0|^2 + eps)
      a0 = silu(u)                       ->  du = da0 * sigmoid(u) (1 + u (1 - sigmoid(u)))
      u[t] = sum_j w[:, j] x[t - 3 + j]  ->  dx[t - 3 + j] += w[:, j] du[t],  dw[:, j] = sum_t du[t] x[t - 3 + j]
    (the history rows are x[-3..-1])."""
    xq, xk, xv, do = _f64(xq), _f64(xk), _f64(xv), _f64(do)
    L = xv.shape[0]
    u = {}
    pre = {}
    act = {}
    for name, x, w, hst in (("q", xq, wq, hq), ("k", xk, wk, hk_), ("v", xv, wv, hv_)):
        u[name] = short_conv(x, w, hst)
        pre[name] = silu(u[name])
    act["q"] = l2_normalize(pre["q"], l2_eps)
    act["k"] = l2_normalize(pre["k"], l2_eps)
    act["v"] = pre["v"]
    y, _ = gated_delta_rule(act["q"], act["k"], act["v"], alpha, beta, S0, scale)
    d_v = y.shape[1]
    r = np.sqrt(np.mean(y * y, axis=1, keepdims=True) + norm_eps)
    n = y / r * (1.0 + norm_w)
    sg = sigmoid(gate)
    dn = do * sg
    out = {"gate": do * n * sg * (1.0 - sg), "norm_w": np.sum(dn * y / r, axis=0)}
    g1 = (1.0 + norm_w) * dn
    dy = g1 / r - y * np.sum(g1 * y, axis=1, keepdims=True) / (d_v * r ** 3)
    dq_a, dk_a, dv_a, out["alpha"], out["beta"], out["S0"] = gated_delta_rule_backward(
        act["q"], act["k"], act["v"], alpha, beta, S0, dy, dS_final, scale)
    dact = {"q": dq_a, "k": dk_a, "v": dv_a}
    for name in ("q", "k"):
        a0 = pre[name]
        inv = 1.0 / np.sqrt(np.sum(a0 * a0, axis=1, keepdims=True) + l2_eps)
        a = a0 * inv
        dact[name] = (dact[name] - a * np.sum(a * dact[name], axis=1, keepdims=True)) * inv
    for name, x, w, hst in (("q", xq, wq, hq), ("k", xk, wk, hk_), ("v", xv, wv, hv_)):
        sgu = sigmoid(u[name])
        du = dact[name] * sgu * (1.0 + u[name] * (1.0 - sgu))
        xx = np.concatenate([_f64(hst), x], axis=0)
        dxx = np.zeros_like(xx)
        dw = np.zeros_like(_f64(w))
        for j in range(CONV_WIDTH):
            dxx[j:j + L] += _f64(w)[:, j][None, :] * du
            dw[:, j] = np.sum(du * xx[j:j + L], axis=0)
        out["x" + name], out["h" + name], out["w" + name] = dxx[CONV_WIDTH - 1:], dxx[:CONV_WIDTH - 1], dw
    return out


def gdn_prefill_backward(inp, dout, dstate_out=None, *, scale=1.0, l2_eps=1e-6, norm_eps=1e-6):
    """Derivatives of gdn_prefill (every step on) for a packed layer, given dL/dout [T, HV, d_v] and dL/dS_final
    [N, HV, d_k, d_v] (None = 0). Returns a dict with q, k [T, HK, d_k], v [T, HV, d_v], alpha, beta [T, HV],
    gate [T, HV, d_v], conv_w [C, 4], norm_w (the shape of inp's norm_w), state_in [N, HV, d_k, d_v] and
    conv_in [N, 3, C]. A QK head's derivatives (its inputs, conv taps and conv history) are the sums over
    the value heads that read it."""
    cu = np.asarray(_f64(inp["cu_seqlens"]), dtype=np.int64)
    q, k, v = _f64(inp["q"]), _f64(inp["k"]), _f64(inp["v"])
    T, hk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    N = len(cu) - 1
    C = 2 * hk * dk + hv * dv
    conv_w = _f64(inp["conv_w"])
    nw_all = _f64(inp["norm_w"])
    st, ci = inp.get("state_in"), inp.get("conv_in")
    do = _f64(dout)
    res = {"q": np.zeros_like(q), "k": np.zeros_like(k), "v": np.zeros_like(v), "alpha": np.zeros((T, hv)),
           "beta": np.zeros((T, hv)), "gate": np.zeros((T, hv, dv)), "conv_w": np.zeros((C, CONV_WIDTH)),
           "norm_w": np.zeros_like(nw_all), "state_in": np.zeros((N, hv, dk, dv)),
           "conv_in": np.zeros((N, CONV_WIDTH - 1, C))}
    for n in range(N):
        s0, s1 = int(cu[n]), int(cu[n + 1])
        ci_n = _f64(ci[n]) if ci is not None else np.zeros((CONV_WIDTH - 1, C))
        for h in range(hv):
            g = (h * hk) // hv
            cq, ck, cv = _head_channels(h, g, hk, hv, dk, dv)
            S0 = _f64(st[n, h]) if st is not None else np.zeros((dk, dv))
            nw = nw_all if nw_all.ndim == 1 else nw_all[h]
            dsf = None if dstate_out is None else _f64(dstate_out)[n, h]
            r = gdn_chain_backward(q[s0:s1, g], k[s0:s1, g], v[s0:s1, h], conv_w[cq], conv_w[ck], conv_w[cv],
                                   ci_n[:, cq], ci_n[:, ck], ci_n[:, cv], _f64(inp["alpha"][s0:s1, h]),
                                   _f64(inp["beta"][s0:s1, h]), _f64(inp["gate"][s0:s1, h]), nw, S0,
                                   do[s0:s1, h], dsf, scale=scale, l2_eps=l2_eps, norm_eps=norm_eps)
            res["q"][s0:s1, g] += r["xq"]
            res["k"][s0:s1, g] += r["xk"]
            res["v"][s0:s1, h] += r["xv"]
            res["alpha"][s0:s1, h] = r["alpha"]
            res["beta"][s0:s1, h] = r["beta"]
            res["gate"][s0:s1, h] = r["gate"]
            res["conv_w"][cq] += r["wq"]
            res["conv_w"][ck] += r["wk"]
            res["conv_w"][cv] += r["wv"]
            if nw_all.ndim == 1:
                res["norm_w"] += r["norm_w"]
            else:
                res["norm_w"][h] += r["norm_w"]
            res["state_in"][n, h] = r["S0"]
            res["conv_in"][n][:, cq] += r["hq"]
            res["conv_in"][n][:, ck] += r["hk"]
            res["conv_in"][n][:, cv] += r["hv"]
    return res


def chain_inputs(inp, n, h, *, state_in=None, conv_in=None):
    """The arguments of gdn_chain for one (sequence n, value head h) chain of a packed prefill, in fp64.

    ``inp`` holds q [T,HK,dk], k [T,HK,dk], v [T,HV,dv], alpha/beta [T,HV], gate [T,HV,dv],
    conv_w [C,4], norm_w [dv] or [HV,dv], cu_seqlens [N+1] and optional state_in
    [N,HV,dk,dv] / conv_in [N,3,C] (arrays or tensors; values are upcast to fp64 exactly).
    Value head h reads QK head floor(h * HK / HV).
    """
    cu = np.asarray(_f64(inp["cu_seqlens"]), dtype=np.int64)
    s0, s1 = int(cu[n]), int(cu[n + 1])
    q, k, v = inp["q"], inp["k"], inp["v"]
    hk, dk = q.shape[1], q.shape[2]
    hv, dv = v.shape[1], v.shape[2]
    g = (h * hk) // hv
    cq, ck, cv = _head_channels(h, g, hk, hv, dk, dv)
    conv_w = _f64(inp["conv_w"])
    st = state_in if state_in is not None else inp.get("state_in")
    ci = conv_in if conv_in is not None else inp.get("conv_in")
    if ci is not None:
        ci_n = _f64(ci[n])
        hq, hk_, hv_ = ci_n[:, cq], ci_n[:, ck], ci_n[:, cv]
    else:
        hq, hk_, hv_ = (np.zeros((CONV_WIDTH - 1, dk)), np.zeros((CONV_WIDTH - 1, dk)),
                        np.zeros((CONV_WIDTH - 1, dv)))
    S0 = _f64(st[n, h]) if st is not None else np.zeros((dk, dv))
    nw = _f64(inp["norm_w"])
    nw = nw if nw.ndim == 1 else nw[h]
    return dict(xq=_f64(q[s0:s1, g]), xk=_f64(k[s0:s1, g]), xv=_f64(v[s0:s1, h]),
                wq=conv_w[cq], wk=conv_w[ck], wv=conv_w[cv], hq=hq, hk_=hk_, hv_=hv_,
                alpha=_f64(inp["alpha"][s0:s1, h]), beta=_f64(inp["beta"][s0:s1, h]),
                gate=_f64(inp["gate"][s0:s1, h]), norm_w=nw, S0=S0)


def prefill_chain(inp, n, h, *, flags=FLAG_ALL, scale=1.0, l2_eps=1e-6, norm_eps=1e-6,
                  state_in=None, conv_in=None):
    """Run one (sequence n, value head h) chain of a packed prefill (inputs as for chain_inputs).
    Returns (o [L, d_v], S_final [d_k, d_v]) for that chain.
    """
    return gdn_chain(**chain_inputs(inp, n, h, state_in=state_in, conv_in=conv_in),
                     flags=flags, scale=scale, l2_eps=l2_eps, norm_eps=norm_eps)


def conv_tail(x_raw, hist):
    """The last 3 raw inputs of a sequence per channel (history first when L < 3)."""
    return np.concatenate([hist, x_raw], axis=0)[-(CONV_WIDTH - 1):]


def gdn_prefill(inp, *, flags=FLAG_ALL, scale=1.0, l2_eps=1e-6, norm_eps=1e-6):
    """Whole packed prefill: every (sequence, value head) chain, then the conv-cache tail.

    Sequences split by ``cu_seqlens`` are independent. Returns (o [T,HV,dv],
    state_out [N,HV,dk,dv], conv_out [N,3,C]) in fp64.
    """
    cu = np.asarray(_f64(inp["cu_seqlens"]), dtype=np.int64)
    N = len(cu) - 1
    q, k, v = inp["q"], inp["k"], inp["v"]
    T, hk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    C = 2 * hk * dk + hv * dv
    o = np.zeros((T, hv, dv))
    S_out = np.zeros((N, hv, dk, dv))
    conv_out = np.zeros((N, CONV_WIDTH - 1, C))
    ci = inp.get("conv_in")
    for n in range(N):
        s0, s1 = int(cu[n]), int(cu[n + 1])
        for h in range(hv):
            o[s0:s1, h], S_out[n, h] = prefill_chain(inp, n, h, flags=flags, scale=scale,
                                                     l2_eps=l2_eps, norm_eps=norm_eps)
        x_raw = np.concatenate([_f64(q[s0:s1]).reshape(s1 - s0, hk * dk),
                                _f64(k[s0:s1]).reshape(s1 - s0, hk * dk),
                                _f64(v[s0:s1]).reshape(s1 - s0, hv * dv)], axis=1)
        hist = _f64(ci[n]) if ci is not None else np.zeros((CONV_WIDTH - 1, C))
        conv_out[n] = conv_tail(x_raw, hist)
    return o, S_out, conv_out


def gdn_decode(step, state, conv_state, conv_w, norm_w, *, flags=FLAG_ALL, scale=1.0,
               l2_eps=1e-6, norm_eps=1e-6):
    """One decode step: the prefill with one token per sequence, state and conv cache carried.

    ``step`` holds q [B,HK,dk], k [B,HK,dk], v [B,HV,dv], alpha/beta [B,HV], gate [B,HV,dv].
    Returns (o [B,HV,dv], new state [B,HV,dk,dv], new conv cache [B,3,C]) in fp64.
    """
    B = step["q"].shape[0]
    inp = dict(step)
    inp.update(cu_seqlens=np.arange(B + 1), conv_w=conv_w, norm_w=norm_w,
               state_in=state, conv_in=conv_state)
    return gdn_prefill(inp, flags=flags, scale=scale, l2_eps=l2_eps, norm_eps=norm_eps)


def _rows(x, rows):
    """Rows ``rows`` of a [T, ...] array or tensor, as fp64."""
    return _f64(x)[np.asarray(rows, dtype=np.int64)]


def gdn_verify(steps, state, conv_state, conv_w, norm_w, *, n_tok, flags=FLAG_ALL, scale=1.0,
               l2_eps=1e-6, norm_eps=1e-6):
    """Speculative verify: each of the B sequences brings K = ``n_tok`` draft tokens (rows
    b*K .. b*K+K-1 of ``steps``), which run through the mixer from the sequence's cached state and
    conv cache. Checking a multi-token draft in one pass is how the four-step MTP decoding of the
    pages ([P5] results, [P2] §01 / §04) uses the layer. The cache itself is not advanced here.

    ``steps`` holds q [B*K,HK,dk], k [B*K,HK,dk], v [B*K,HV,dv], alpha/beta [B*K,HV],
    gate [B*K,HV,dv]. Returns o [B*K,HV,dv] in fp64: by definition the prefill of each draft
    (a sequence of length K) from that cache.
    """
    B = int(np.asarray(_f64(state)).shape[0])
    inp = dict(steps)
    inp.update(cu_seqlens=np.arange(B + 1) * n_tok, conv_w=conv_w, norm_w=norm_w,
               state_in=state, conv_in=conv_state)
    o, _, _ = gdn_prefill(inp, flags=flags, scale=scale, l2_eps=l2_eps, norm_eps=norm_eps)
    return o


def gdn_commit(steps, n_accept, state, conv_state, conv_w, norm_w, *, n_tok, flags=FLAG_ALL,
               scale=1.0, l2_eps=1e-6, norm_eps=1e-6):
    """Speculative commit: the state and conv cache of sequence b after its first ``n_accept[b]``
    draft tokens (0 <= n <= K), i.e. the cache a prefill of only the accepted tokens leaves.
    Returns (state [B,HV,dk,dv], conv cache [B,3,C]) in fp64.
    """
    B = int(np.asarray(_f64(state)).shape[0])
    n = [int(x) for x in np.asarray(n_accept).reshape(-1)]
    assert len(n) == B and all(0 <= x <= n_tok for x in n)
    rows = [b * n_tok + t for b in range(B) for t in range(n[b])]
    inp = {key: _rows(steps[key], rows) for key in ("q", "k", "v", "alpha", "beta", "gate")}
    inp.update(cu_seqlens=np.concatenate([[0], np.cumsum(n)]), conv_w=conv_w, norm_w=norm_w,
               state_in=state, conv_in=conv_state)
    _, S, c = gdn_prefill(inp, flags=flags, scale=scale, l2_eps=l2_eps, norm_eps=norm_eps)
    return S, c


def softplus(x):
    """log(1 + e^x), evaluated without overflow."""
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def gate_alpha_beta(a, b, a_log, dt_bias):
    """Data-dependent decay and write gates of every (token, value head) ([P1] 方法; the formula
    is a reading, the pages give none): alpha = exp(-exp(A_h) softplus(a + delta_h)) in (0, 1],
    beta = sigmoid(b) in (0, 1). a, b: [T, HV]; a_log (A), dt_bias (delta): [HV]."""
    a, b = _f64(a), _f64(b)
    alpha = np.exp(-np.exp(_f64(a_log))[None, :] * softplus(a + _f64(dt_bias)[None, :]))
    return alpha, sigmoid(b)


def in_projection(x, w_qkv, w_z, w_ab, a_log, dt_bias):
    """The layer's input side ([P1] 方法, [P2] §07): the normalised residual stream x [T, hidden]
    through the fused input matrix. Returns (qkv [T, C] in the conv's channel order q | k | v,
    gate logits z [T, HV*dv], alpha [T, HV], beta [T, HV]) in fp64."""
    x = _f64(x)
    qkv = x @ _f64(w_qkv)
    z = x @ _f64(w_z)
    ab = x @ _f64(w_ab)
    hv = ab.shape[1] // 2
    alpha, beta = gate_alpha_beta(ab[:, :hv], ab[:, hv:], a_log, dt_bias)
    return qkv, z, alpha, beta


def out_projection(o, w_out):
    """The mixer output o [T, HV*dv] back to the residual width: o W_out, fp64."""
    return _f64(o) @ _f64(w_out)


# ------------------------------------------------------------------------ QSA compressed indexer ----

QSA_BLOCK = 4        # keys per micro-block ([P2] §04: r = 4)
QSA_TOPK = 512       # blocks kept per query (K = 2048 tokens)
QSA_ROPE_DIMS = 64   # rotated dims of the 128 (a reading: "partial RoPE")
QSA_ROPE_BASE = 1e4


def partial_rope(x, pos, rope_dims=QSA_ROPE_DIMS):
    """Rotate dims (d, d + h), d < h = rope_dims / 2, of x [..., 128] by angle pos * base^(-d/h) (fp64);
    64 rotated dims by default (dims 0..31 paired with 32..63)."""
    x = np.array(_f64(x), dtype=np.float64, copy=True)
    half = rope_dims // 2
    if half == 0:
        return x
    ang = np.asarray(pos, dtype=np.float64)[..., None] * QSA_ROPE_BASE ** (-np.arange(half) / half)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half].copy(), x[..., half:2 * half].copy()
    x[..., :half] = a * c - b * s
    x[..., half:2 * half] = a * s + b * c
    return x


def qsa_compress(k, w, eps=1e-6, rope_dims=QSA_ROPE_DIMS):
    """Compressed keys of the complete micro-blocks of one sequence ([P2] §04): the mean of each 4
    keys, RMS-normalised with gain w, then partial RoPE at the block's first position 4b.
    k [T, 128] -> [floor(T/4), 128] fp64."""
    k = _f64(k)
    nb = k.shape[0] // QSA_BLOCK
    m = k[:nb * QSA_BLOCK].reshape(nb, QSA_BLOCK, k.shape[1]).mean(axis=1)
    m = m / np.sqrt(np.mean(m * m, axis=1, keepdims=True) + eps) * _f64(w)[None, :]
    return partial_rope(m, QSA_BLOCK * np.arange(nb), rope_dims)


def qsa_scores(q, kbar, pos, rope_dims=QSA_ROPE_DIMS):
    """I[i, b] = sum over the 4 heads of ReLU(rope(q_ih, pos_i) . kbar_b) for the blocks complete at
    query i (4b + 3 <= pos_i); -inf elsewhere. q [M, 4, 128], kbar [N, 128], pos [M]."""
    qr = partial_rope(q, np.asarray(pos)[:, None] * np.ones((1, _f64(q).shape[1])), rope_dims)
    sc = np.maximum(np.einsum("mhd,nd->mhn", qr, _f64(kbar)), 0.0).sum(axis=1)
    valid = (QSA_BLOCK * np.arange(sc.shape[1])[None, :] + QSA_BLOCK - 1) <= np.asarray(pos)[:, None]
    return np.where(valid, sc, -np.inf)


def qsa_select(scores, pos, topk=QSA_TOPK):
    """Per query: the top-k complete blocks by score (ties to the lower block), listed in block
    order, and the first token of the incomplete tail block (pos + 1 when the block is complete).
    Returns (list of index arrays, tail_start [M])."""
    out = []
    for row in scores:
        cand = np.nonzero(np.isfinite(row))[0]
        if len(cand) > topk:
            order = sorted(cand, key=lambda b: (-row[b], b))[:topk]
            cand = np.sort(np.array(order))
        out.append(cand.astype(np.int64))
    pos = np.asarray(pos)
    return out, QSA_BLOCK * ((pos + 1) // QSA_BLOCK)
