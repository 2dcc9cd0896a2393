"""GPU parity of the recurrence backward (gdn_recurrence_backward) against the fp64 oracle's
reverse-mode derivatives, element by element as rel-L2 <= 1e-4 per output (fp32 io)."""
import numpy as np
import pytest
import torch

import oracle as O

pytestmark = pytest.mark.gpu

gdn = pytest.importorskip("linear_attention_token_amd.gdn")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

DEV = "cuda:0"
TOL = 1e-4


def _inputs(lens, hk, hv, seed, alpha_lo=0.9, with_state=True):
    g = torch.Generator(device="cpu").manual_seed(seed)
    T = sum(lens)
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32)
    q = torch.randn(T, hk, 128, generator=g)
    q = q / q.norm(dim=-1, keepdim=True)
    k = torch.randn(T, hk, 128, generator=g)
    k = k / k.norm(dim=-1, keepdim=True)
    v = torch.randn(T, hv, 128, generator=g)
    alpha = torch.exp(torch.log(torch.tensor(alpha_lo)) * torch.rand(T, hv, generator=g))
    beta = torch.sigmoid(torch.randn(T, hv, generator=g))
    dy = torch.randn(T, hv, 128, generator=g)
    n = len(lens)
    s0 = 0.05 * torch.randn(n, hv, 128, 128, generator=g) if with_state else None
    dsf = 0.1 * torch.randn(n, hv, 128, 128, generator=g) if with_state else None
    return cu, q, k, v, alpha, beta, dy, s0, dsf


def _rel(a, b):
    a = a.detach().cpu().double().numpy()
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def _run(cfg, cu, q, k, v, alpha, beta, dy, s0, dsf):
    d = lambda t: None if t is None else t.to(DEV).contiguous()
    out = gdn.gdn_recurrence_backward(cfg, d(cu), d(q), d(k), d(v), d(alpha), d(beta), d(dy), state_in=d(s0),
                                      dstate_out=d(dsf))
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("hk,hv,alpha_lo,with_state", [(2, 6, 0.9, True), (2, 2, 0.5, True), (1, 3, 0.5, False)])
def test_backward_matches_oracle(hk, hv, alpha_lo, with_state):
    lens = [1, 5, 70, 0, 130]
    cu, q, k, v, alpha, beta, dy, s0, dsf = _inputs(lens, hk, hv, 31, alpha_lo, with_state)
    cfg = gdn.cfg_for(hk, hv, 128, 128, torch.float32, scale=0.7)
    got = _run(cfg, cu, q, k, v, alpha, beta, dy, s0, dsf)
    ref = O.recurrence_layer_backward(q, k, v, alpha, beta, s0, cu.numpy(), dy, dsf, scale=0.7)
    for name, a, b in zip(("dq", "dk", "dv", "dalpha", "dbeta", "dstate_in"), got, ref):
        assert _rel(a, b) <= TOL, (name, _rel(a, b))


@pytest.mark.parametrize("lens", [[64, 128, 63, 65, 127, 129], [1, 2, 3] * 13 + [0, 200], [3000]])
def test_backward_chunk_boundaries(lens):
    """Sequence lengths at and around the 64-token chunk size, many tiny sequences (a chunk table of
    41 entries, most with one chunk of 1-3 tokens, and an empty one), and one long sequence (47 chunks):
    every output against the oracle."""
    cu, q, k, v, alpha, beta, dy, s0, dsf = _inputs(lens, 1, 2, 33, 0.5, True)
    cfg = gdn.cfg_for(1, 2, 128, 128, torch.float32, scale=0.9)
    got = _run(cfg, cu, q, k, v, alpha, beta, dy, s0, dsf)
    ref = O.recurrence_layer_backward(q, k, v, alpha, beta, s0, cu.numpy(), dy, dsf, scale=0.9)
    for name, a, b in zip(("dq", "dk", "dv", "dalpha", "dbeta", "dstate_in"), got, ref):
        assert _rel(a, b) <= TOL, (name, _rel(a, b))


def test_backward_model_shape_group():
    """16 QK / 48 value heads, one 1024-token sequence: every output of QK group 5 (value heads 15-17)
    against the oracle's chains, summed over the group for dq and dk."""
    lens = [1024]
    cu, q, k, v, alpha, beta, dy, s0, dsf = _inputs(lens, 16, 48, 32)
    cfg = gdn.cfg_for(16, 48, 128, 128, torch.float32)
    dq, dk, dv, da, db, ds0 = _run(cfg, cu, q, k, v, alpha, beta, dy, s0, dsf)
    g = 5
    rq, rk = 0.0, 0.0
    for h in range(3 * g, 3 * g + 3):
        r = O.gated_delta_rule_backward(q[:, g], k[:, g], v[:, h], alpha[:, h].double().numpy(),
                                        beta[:, h].double().numpy(), s0[0, h], dy[:, h], dsf[0, h])
        rq, rk = rq + r[0], rk + r[1]
        for name, a, b in (("dv", dv[:, h], r[2]), ("dalpha", da[:, h], r[3]), ("dbeta", db[:, h], r[4]),
                           ("dstate_in", ds0[0, h], r[5])):
            assert _rel(a, b) <= TOL, (name, h, _rel(a, b))
    assert _rel(dq[:, g], rq) <= TOL and _rel(dk[:, g], rk) <= TOL


@pytest.mark.parametrize("lens,hk,hv,history", [([1, 5, 70, 0, 130], 2, 6, True), ([200], 1, 1, False)])
def test_mixer_backward_matches_oracle(lens, hk, hv, history):
    """gdn_backward (conv + SiLU, L2, recurrence, RMSNorm, gate) against the oracle's derivatives of the whole
    mixer, every output element by element (rel-L2 <= 1e-4)."""
    from workloads import prefill_inputs
    inp = prefill_inputs(lens, n_qk_heads=hk, n_v_heads=hv, d_k=128, d_v=128, io_dtype=torch.float32, seed=41,
                         s0_std=0.05 if history else 0.0, conv_in_std=1.0 if history else 0.0)
    g = torch.Generator(device="cpu").manual_seed(42)
    dout = torch.randn(sum(lens), hv, 128, generator=g)
    dsf = 0.1 * torch.randn(len(lens), hv, 128, 128, generator=g)
    cfg = gdn.cfg_for(hk, hv, 128, 128, torch.float32)
    d = lambda t: None if t is None else t.to(DEV).contiguous()
    si = inp.state_in if history else None
    ci = inp.conv_in if history else None
    got = gdn.gdn_backward(cfg, d(inp.cu_seqlens), d(inp.q), d(inp.k), d(inp.v), d(inp.alpha), d(inp.beta), d(inp.gate),
                           d(inp.conv_w), d(inp.norm_w), d(dout), state_in=d(si), conv_in=d(ci), dstate_out=d(dsf))
    torch.cuda.synchronize()
    ref_in = {"cu_seqlens": inp.cu_seqlens, "q": inp.q, "k": inp.k, "v": inp.v, "alpha": inp.alpha, "beta": inp.beta,
              "gate": inp.gate, "conv_w": inp.conv_w, "norm_w": inp.norm_w, "state_in": si, "conv_in": ci}
    ref = O.gdn_prefill_backward(ref_in, dout, dsf)
    for name in ("q", "k", "v", "alpha", "beta", "gate", "conv_w", "norm_w", "state_in", "conv_in"):
        assert _rel(got[name], ref[name]) <= TOL, (name, _rel(got[name], ref[name]))


def test_mixer_backward_is_reproducible():
    """Two calls on the same inputs give the same bits for every output (sums over tokens run in a fixed
    order)."""
    from workloads import prefill_inputs
    inp = prefill_inputs([300, 77], n_qk_heads=2, n_v_heads=4, d_k=128, d_v=128, io_dtype=torch.float32, seed=43,
                         device=DEV, s0_std=0.05, conv_in_std=1.0)
    dout = torch.randn(377, 4, 128, device=DEV)
    cfg = gdn.cfg_for(2, 4, 128, 128, torch.float32)
    args = (cfg, inp.cu_seqlens, inp.q, inp.k, inp.v, inp.alpha, inp.beta, inp.gate, inp.conv_w, inp.norm_w, dout)
    a = gdn.gdn_backward(*args, state_in=inp.state_in, conv_in=inp.conv_in)
    b = gdn.gdn_backward(*args, state_in=inp.state_in, conv_in=inp.conv_in)
    torch.cuda.synchronize()
    for name in a:
        assert torch.equal(a[name], b[name]), name


def test_mixer_backward_bench_shape_sampled_group():
    """The benchmark's configuration (one 4096-token sequence, 16 QK / 48 value heads): every derivative that
    depends only on QK group 5 (value heads 15-17) against the oracle's chains -- their raw q, k, v inputs,
    alpha, beta, gate, and the conv taps of their channels."""
    from workloads import prefill_inputs
    T, g = 4096, 5
    inp = prefill_inputs([T], n_qk_heads=16, n_v_heads=48, d_k=128, d_v=128, io_dtype=torch.float32, seed=11)
    gg = torch.Generator(device="cpu").manual_seed(12)
    dout = torch.randn(T, 48, 128, generator=gg)
    cfg = gdn.cfg_for(16, 48, 128, 128, torch.float32)
    d = lambda t: t.to(DEV).contiguous()
    got = gdn.gdn_backward(cfg, d(inp.cu_seqlens), d(inp.q), d(inp.k), d(inp.v), d(inp.alpha), d(inp.beta),
                           d(inp.gate), d(inp.conv_w), d(inp.norm_w), d(dout), want_dstate_in=False,
                           want_dconv_in=False)
    torch.cuda.synchronize()
    C = 2 * 16 * 128 + 48 * 128
    cw = inp.conv_w.double().numpy()
    qs, ks = slice(128 * g, 128 * g + 128), slice(2048 + 128 * g, 2048 + 128 * g + 128)
    zeros = np.zeros((3, 128))
    dq = dk = dwq = dwk = 0.0
    for h in range(3 * g, 3 * g + 3):
        vs = slice(4096 + 128 * h, 4096 + 128 * h + 128)
        r = O.gdn_chain_backward(inp.q[:, g], inp.k[:, g], inp.v[:, h], cw[qs], cw[ks], cw[vs], zeros, zeros, zeros,
                                 inp.alpha[:, h].double().numpy(), inp.beta[:, h].double().numpy(),
                                 inp.gate[:, h].double().numpy(), inp.norm_w.double().numpy(), np.zeros((128, 128)),
                                 dout[:, h])
        dq, dk, dwq, dwk = dq + r["xq"], dk + r["xk"], dwq + r["wq"], dwk + r["wk"]
        for name, a, b in (("v", got["v"][:, h], r["xv"]), ("alpha", got["alpha"][:, h], r["alpha"]),
                           ("beta", got["beta"][:, h], r["beta"]), ("gate", got["gate"][:, h], r["gate"]),
                           ("conv_w v", got["conv_w"][vs], r["wv"])):
            assert _rel(a, b) <= TOL, (name, h, _rel(a, b))
    for name, a, b in (("q", got["q"][:, g], dq), ("k", got["k"][:, g], dk), ("conv_w q", got["conv_w"][qs], dwq),
                       ("conv_w k", got["conv_w"][ks], dwk)):
        assert _rel(a, b) <= TOL, (name, _rel(a, b))
    assert got["conv_w"].shape == (C, 4)
