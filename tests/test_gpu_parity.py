"""GPU parity: the HIP library (through the C ABI) against the fp64 oracle, element by element.

Bars: relative L2 <= 1e-4 for fp32 io and <= 1e-2 for bf16 io, on outputs and final states; the
conv tail is a copy and must match exactly. Small cases run the whole oracle; model-shape cases at
full size compare sampled (sequence, value head) chains, which the oracle computes one by one.
"""
import numpy as np
import pytest
import torch

import oracle as O
from workloads import (prefill_inputs, decode_inputs, config_tiny, config_layer, config_long,
                       config_varlen, loguniform_lengths)

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from linear_attention_token_amd import gdn  # noqa: E402  (raises if libgdn.so is missing)
from gdn_testutil import TOL, rel_l2, cfg_of, run_prefill, oracle_prefill, oracle_chain, seq_bounds  # noqa: E402

gdn.load_library()
DEV = "cuda"


def _check_full(inp, flags=gdn.GDN_ALL, tol=None):
    tol = tol if tol is not None else TOL[inp.io_dtype]
    out, st, cv = run_prefill(inp, flags)
    o_ref, s_ref, c_ref = oracle_prefill(inp.to("cpu"), flags=flags)
    e_o, e_s = rel_l2(out, o_ref), rel_l2(st, s_ref)
    print(f"rel_l2 out={e_o:.3e} state={e_s:.3e}", flush=True)
    assert e_o <= tol and e_s <= tol, (e_o, e_s)
    np.testing.assert_array_equal(cv.double().cpu().numpy(), c_ref)
    return out, st, cv


# ------------------------------------------------------------------ fp32 io (sequential path) ---

@pytest.mark.parametrize("flags", [gdn.GDN_CONV | gdn.GDN_L2QK, gdn.GDN_ALL])
def test_tiny_fp32(flags):
    """T=64, one QK head and one value head, d=16, fp32; raw readout and the full layer."""
    _check_full(config_tiny(DEV), flags)


def test_fp32_multihead_varlen_with_history():
    inp = prefill_inputs([37, 64, 1, 130, 2], n_qk_heads=2, n_v_heads=6, d_k=32, d_v=32,
                         io_dtype=torch.float32, seed=3, device=DEV, s0_std=0.1, conv_in_std=1.0)
    _check_full(inp)


def test_fp32_model_dims_short():
    inp = prefill_inputs([70, 9], n_qk_heads=2, n_v_heads=6, d_k=128, d_v=128,
                         io_dtype=torch.float32, seed=4, device=DEV, s0_std=0.02)
    _check_full(inp)


# ------------------------------------------------------------------ bf16 io (chunked path) -------

def test_bf16_chunked_ragged():
    """Several chunks, a ragged tail, sequences shorter than the conv window and one chunk long."""
    inp = prefill_inputs([200, 64, 3, 130, 1], n_qk_heads=2, n_v_heads=6, d_k=128, d_v=128,
                         io_dtype=torch.bfloat16, seed=5, device=DEV, s0_std=0.01, conv_in_std=1.0)
    _check_full(inp)


@pytest.mark.parametrize("io", [torch.float32, torch.bfloat16])
def test_fused_qkv_views_and_empty_sequences(io):
    """q, k, v as column slices of one [T, C] projection output (token row stride C, the usual
    caller layout), in a packed batch with zero-length sequences: identical (bitwise) to contiguous
    copies, within tolerance of the oracle, and empty sequences pass state and conv cache through."""
    lens = [0, 70, 0, 5, 0, 64]
    inp = prefill_inputs(lens, n_qk_heads=2, n_v_heads=6, d_k=128, d_v=128, io_dtype=io, seed=21, device=DEV,
                         s0_std=0.01, conv_in_std=1.0)
    T, hk, hv = inp.q.shape[0], 2, 6
    ref_out, ref_st, ref_cv = run_prefill(inp)
    fused = torch.cat([inp.q.reshape(T, -1), inp.k.reshape(T, -1), inp.v.reshape(T, -1)], dim=1)
    qc = hk * 128
    inp.q = fused[:, :qc].view(T, hk, 128)
    inp.k = fused[:, qc:2 * qc].view(T, hk, 128)
    inp.v = fused[:, 2 * qc:].view(T, hv, 128)
    assert not inp.q.is_contiguous() and inp.q.stride(0) == fused.shape[1]
    out, st, cv = run_prefill(inp)
    assert torch.equal(out, ref_out) and torch.equal(st, ref_st) and torch.equal(cv, ref_cv)
    o_ref, s_ref, c_ref = oracle_prefill(inp.to("cpu"))
    tol = TOL[io]
    assert rel_l2(out, o_ref) <= tol and rel_l2(st, s_ref) <= tol
    np.testing.assert_array_equal(cv.double().cpu().numpy(), c_ref)
    for n, L in enumerate(lens):
        if L == 0:
            assert torch.equal(st[n], inp.state_in[n])
            assert torch.equal(cv[n], inp.conv_in[n])


@pytest.mark.parametrize("hk,hv", [(2, 2), (2, 4), (1, 4), (1, 5), (1, 6)])
def test_bf16_chunked_head_ratios(hk, hv):
    """Value heads per QK head from 1 to 6: the WY kernel batches 1, 2 or 3 of them per block."""
    inp = prefill_inputs([150, 64, 3], n_qk_heads=hk, n_v_heads=hv, d_k=128, d_v=128,
                         io_dtype=torch.bfloat16, seed=11 + hv, device=DEV, s0_std=0.01, conv_in_std=1.0)
    _check_full(inp)


@pytest.mark.parametrize("flags", [gdn.GDN_CONV | gdn.GDN_L2QK, gdn.GDN_L2QK | gdn.GDN_NORM | gdn.GDN_GATE])
def test_bf16_chunked_stage_flags(flags):
    inp = prefill_inputs([150], n_qk_heads=1, n_v_heads=3, d_k=128, d_v=128,
                         io_dtype=torch.bfloat16, seed=6, device=DEV, s0_std=0.01)
    _check_full(inp, flags)


def test_bf16_other_dims_sequential():
    """bf16 io at d=64 runs the fp32 sequential kernel."""
    inp = prefill_inputs([100, 33], n_qk_heads=2, n_v_heads=4, d_k=64, d_v=64,
                         io_dtype=torch.bfloat16, seed=7, device=DEV, s0_std=0.01)
    _check_full(inp)


def test_layer_model_shape_full():
    """One layer at model shape (T=4096, 16/48 heads, d=128, bf16), whole output and all states."""
    _check_full(config_layer(DEV))


def _sampled(inp, chains, flags=gdn.GDN_ALL):
    out, st, cv = run_prefill(inp, flags)
    tol = TOL[inp.io_dtype]
    for n, h in chains:
        s0, s1 = seq_bounds(inp, n)
        o_ref, s_ref = oracle_chain(inp, n, h, flags)
        e_o, e_s = rel_l2(out[s0:s1, h], o_ref), rel_l2(st[n, h], s_ref)
        print(f"seq {n} head {h} len {s1 - s0}: rel_l2 out={e_o:.3e} state={e_s:.3e}", flush=True)
        assert e_o <= tol and e_s <= tol, (n, h, e_o, e_s)
    return out, st, cv


def _sampled_pool(inp, chains, flags=gdn.GDN_ALL):
    """Like _sampled, with the oracle chains spread over a process pool."""
    out, st, cv = run_prefill(inp, flags)
    tol = TOL[inp.io_dtype]
    refs = O.run_chains(vars(inp), chains, flags=flags)
    for (n, h), (o_ref, s_ref) in zip(chains, refs):
        s0, s1 = seq_bounds(inp, n)
        e_o, e_s = rel_l2(out[s0:s1, h], o_ref), rel_l2(st[n, h], s_ref)
        print(f"seq {n} head {h} len {s1 - s0}: rel_l2 out={e_o:.3e} state={e_s:.3e}", flush=True)
        assert e_o <= tol and e_s <= tol, (n, h, e_o, e_s)
    return out, st, cv


def test_varlen_model_shape_sampled():
    """32 packed sequences, lengths log-uniform in [512, 32768], S0 ~ N(0, 0.01): 16 chains, every
    other sequence in order of length (shortest and longest included), heads spread over all 16 QK
    groups."""
    inp = config_varlen(DEV)
    lens = np.diff(inp.cu_seqlens.cpu().numpy())
    order = np.argsort(lens)
    picks = list(order[::2][:15]) + [order[-1]]
    chains = [(int(n), (7 * i + 3 * (i % 2)) % 48) for i, n in enumerate(picks)]
    _, st, _ = _sampled_pool(inp, chains)
    assert torch.isfinite(st).all()


def test_long_prefill_sampled():
    """T = 262144 (native context), B=1, model shape: eight value heads, in eight of the 16 QK groups,
    against the oracle."""
    inp = config_long(DEV)
    _sampled_pool(inp, [(0, h) for h in (0, 7, 13, 20, 26, 33, 39, 46)])


# ------------------------------------------------------------------ invariants -------------------

def test_packed_equals_separate_bitwise():
    lengths = [130, 64, 5, 77]
    inp = prefill_inputs(lengths, n_qk_heads=2, n_v_heads=6, d_k=128, d_v=128,
                         io_dtype=torch.bfloat16, seed=8, device=DEV, s0_std=0.01, conv_in_std=1.0)
    out, st, cv = run_prefill(inp)
    cu = inp.cu_seqlens.cpu().numpy()
    for n, L in enumerate(lengths):
        s0, s1 = cu[n], cu[n + 1]
        one = prefill_inputs([L], n_qk_heads=2, n_v_heads=6, d_k=128, d_v=128, io_dtype=torch.bfloat16,
                             seed=8, device=DEV)
        for key in ("q", "k", "v", "alpha", "beta", "gate"):
            setattr(one, key, getattr(inp, key)[s0:s1].contiguous())
        one.conv_w, one.norm_w = inp.conv_w, inp.norm_w
        one.state_in = inp.state_in[n:n + 1].contiguous()
        one.conv_in = inp.conv_in[n:n + 1].contiguous()
        o1, s1_, c1 = run_prefill(one)
        assert torch.equal(o1, out[s0:s1]) and torch.equal(s1_[0], st[n]) and torch.equal(c1[0], cv[n])


def test_repeat_runs_bitwise():
    inp = prefill_inputs([300, 45], n_qk_heads=2, n_v_heads=6, d_k=128, d_v=128,
                         io_dtype=torch.bfloat16, seed=9, device=DEV, s0_std=0.01)
    a = run_prefill(inp)
    b = run_prefill(inp)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_graph_replay_matches_eager():
    """A prefill captured in a HIP graph and replayed several times, with other GPU work and
    synchronisations between the replays, reproduces the eager result bit for bit each time (the
    library records no memset or host-side work that a graph would freeze)."""
    inp = prefill_inputs([200, 64, 3], n_qk_heads=2, n_v_heads=6, d_k=128, d_v=128,
                         io_dtype=torch.bfloat16, seed=21, device=DEV, s0_std=0.01, conv_in_std=1.0)
    cfg = cfg_of(inp)
    N, T = inp.n_seqs, int(inp.q.shape[0])
    out = torch.empty((T, inp.n_v_heads, inp.d_v), dtype=inp.io_dtype, device=DEV)
    st = torch.empty((N, inp.n_v_heads, inp.d_k, inp.d_v), dtype=torch.float32, device=DEV)
    cv = torch.empty((N, 3, inp.n_channels), dtype=inp.io_dtype, device=DEV)
    ws = torch.empty(gdn.gdn_prefill_workspace(cfg, N, T), dtype=torch.uint8, device=DEV)
    host = inp.cu_seqlens.cpu()

    def step():
        gdn.gdn_prefill(cfg, inp.cu_seqlens, inp.q, inp.k, inp.v, inp.alpha, inp.beta, inp.gate, inp.conv_w,
                        inp.norm_w, state_in=inp.state_in, state_out=st, conv_in=inp.conv_in, conv_out=cv,
                        out=out, workspace=ws, cu_seqlens_host=host)

    step()
    torch.cuda.synchronize()
    ref = (out.clone(), st.clone(), cv.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(3):
        for t in (out, st, cv, ws):
            t.zero_()                    # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]) and torch.equal(st, ref[1]) and torch.equal(cv, ref[2])


def test_alpha_one_beta_zero_keeps_state():
    inp = prefill_inputs([150, 20], n_qk_heads=2, n_v_heads=6, d_k=128, d_v=128,
                         io_dtype=torch.bfloat16, seed=10, device=DEV, alpha_recipe="one",
                         beta_recipe="zero", s0_std=0.05)
    out, st, _ = run_prefill(inp)
    assert torch.equal(st, inp.state_in)
    o_ref, _, _ = oracle_prefill(inp.to("cpu"))
    assert rel_l2(out, o_ref) <= 1e-2


@pytest.mark.parametrize("T1", [1, 64, 100])
def test_continuation(T1):
    """prefill(T1 + T2) == prefill(T1) -> (state, conv tail) -> prefill(T2), within tolerance."""
    T = 230
    inp = prefill_inputs([T], n_qk_heads=2, n_v_heads=6, d_k=128, d_v=128, io_dtype=torch.bfloat16,
                         seed=11, device=DEV, s0_std=0.01, conv_in_std=1.0)
    out, st, cv = run_prefill(inp)

    def part(a, b, s_in, c_in):
        p = prefill_inputs([b - a], n_qk_heads=2, n_v_heads=6, d_k=128, d_v=128, io_dtype=torch.bfloat16,
                           seed=11, device=DEV)
        for key in ("q", "k", "v", "alpha", "beta", "gate"):
            setattr(p, key, getattr(inp, key)[a:b].contiguous())
        p.conv_w, p.norm_w, p.state_in, p.conv_in = inp.conv_w, inp.norm_w, s_in, c_in
        return run_prefill(p)

    oa, sa, ca = part(0, T1, inp.state_in, inp.conv_in)
    ob, sb, cb = part(T1, T, sa, ca)
    assert torch.equal(cb, cv)
    assert rel_l2(torch.cat([oa, ob]), out) <= 1e-2 and rel_l2(sb, st) <= 1e-2


def test_state_in_place_alias():
    inp = prefill_inputs([100, 70], n_qk_heads=2, n_v_heads=6, d_k=128, d_v=128, io_dtype=torch.bfloat16,
                         seed=12, device=DEV, s0_std=0.01, conv_in_std=1.0)
    out, st, cv = run_prefill(inp)
    cfg = gdn.cfg_for(2, 6, 128, 128, torch.bfloat16)
    s_io = inp.state_in.clone()
    c_io = inp.conv_in.clone()
    out2 = gdn.gdn_prefill(cfg, inp.cu_seqlens, inp.q, inp.k, inp.v, inp.alpha, inp.beta, inp.gate, inp.conv_w,
                           inp.norm_w, state_in=s_io, state_out=s_io, conv_in=c_io, conv_out=c_io)
    torch.cuda.synchronize()
    assert torch.equal(out2, out) and torch.equal(s_io, st) and torch.equal(c_io, cv)


# ------------------------------------------------------------------ decode -----------------------

def _decode_steps(di, steps, flags=gdn.GDN_ALL):
    cfg = gdn.cfg_for(di.n_qk_heads, di.n_v_heads, di.d_k, di.d_v, di.io_dtype, flags=flags)
    state = di.state.clone()
    conv = di.conv_state.clone()
    outs = []
    for s in range(steps):
        outs.append(gdn.gdn_decode_step(cfg, di.q[s], di.k[s], di.v[s], di.alpha[s], di.beta[s], di.gate[s],
                                        di.conv_w, di.norm_w, conv, state))
    torch.cuda.synchronize()
    return torch.stack(outs), state, conv


def _oracle_decode_seq(di, b, steps, flags=O.FLAG_ALL, heads=None):
    """Decode of sequence b over `steps` steps == prefill of those tokens from the cached state."""
    inp = dict(q=di.q[:steps, b], k=di.k[:steps, b], v=di.v[:steps, b], alpha=di.alpha[:steps, b],
               beta=di.beta[:steps, b], gate=di.gate[:steps, b], conv_w=di.conv_w, norm_w=di.norm_w,
               cu_seqlens=np.array([0, steps]), state_in=di.state[b:b + 1], conv_in=di.conv_state[b:b + 1])
    res = {}
    for h in (heads if heads is not None else range(di.n_v_heads)):
        res[h] = O.prefill_chain(inp, 0, h, flags=flags)
    return res


@pytest.mark.parametrize("io", [torch.float32, torch.bfloat16])
def test_decode_small(io):
    di = decode_inputs(4, 5, n_qk_heads=1, n_v_heads=1, d_k=16, d_v=16, io_dtype=io, device=DEV,
                       alpha_recipe="softplus", state_std=0.1)
    outs, st, cv = _decode_steps(di, 5)
    tol = TOL[io]
    for b in range(4):
        ref = _oracle_decode_seq(di, b, 5)
        o_ref, s_ref = ref[0]
        assert rel_l2(outs[:, b, 0], o_ref) <= tol and rel_l2(st[b, 0], s_ref) <= tol
    # conv cache: the last 3 raw inputs
    x_last = torch.cat([di.q[2:5].reshape(3, 4, -1), di.k[2:5].reshape(3, 4, -1), di.v[2:5].reshape(3, 4, -1)], -1)
    assert torch.equal(cv, x_last.transpose(0, 1))


@pytest.mark.parametrize("io", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("hk,hv,flags", [(1, 1, gdn.GDN_ALL), (2, 4, gdn.GDN_ALL), (1, 5, gdn.GDN_ALL),
                                         (1, 1, gdn.GDN_CONV | gdn.GDN_L2QK), (2, 4, gdn.GDN_CONV | gdn.GDN_L2QK),
                                         (1, 5, gdn.GDN_L2QK), (2, 4, gdn.GDN_L2QK), (1, 64, gdn.GDN_ALL)])
def test_decode_d128_head_ratios(io, hk, hv, flags):
    """Head size 128 (the dedicated decode kernel): value heads per QK head 1, 2, 5 (the v channels
    of a group span more than one load pass of the block) and 64 (the largest ratio, the most
    LDS), the flag subsets the kernel branches on, fp32 and bf16 io; the conv cache ends as the
    last three raw inputs."""
    B, steps = 3, 4
    di = decode_inputs(B, steps, n_qk_heads=hk, n_v_heads=hv, d_k=128, d_v=128, io_dtype=io, device=DEV,
                       seed=29 + hv, state_std=0.05)
    outs, st, cv = _decode_steps(di, steps, flags=flags)
    tol = TOL[io]
    for b in range(B):
        ref = _oracle_decode_seq(di, b, steps, flags=flags)
        for h, (o_ref, s_ref) in ref.items():
            e_o, e_s = rel_l2(outs[:, b, h], o_ref), rel_l2(st[b, h], s_ref)
            assert e_o <= tol and e_s <= tol, (b, h, e_o, e_s)
    if flags & gdn.GDN_CONV:
        x_last = torch.cat([di.q[steps - 3:steps].reshape(3, B, -1), di.k[steps - 3:steps].reshape(3, B, -1),
                            di.v[steps - 3:steps].reshape(3, B, -1)], -1)
        assert torch.equal(cv, x_last.transpose(0, 1))


def test_decode_model_shape_fp32_every_head():
    """One fp32 step at B=256, model shape: every value head of a sample of sequences to 1e-4, so a
    single wrong element of the 128x128 state of any head fails."""
    di = decode_inputs(256, 1, n_qk_heads=16, n_v_heads=48, d_k=128, d_v=128, io_dtype=torch.float32,
                       device=DEV, seed=5)
    outs, st, _ = _decode_steps(di, 1)
    for b in range(0, 256, 5):
        ref = _oracle_decode_seq(di, b, 1)
        for h, (o_ref, s_ref) in ref.items():
            e_o, e_s = rel_l2(outs[:, b, h], o_ref), rel_l2(st[b, h], s_ref)
            assert e_o <= 1e-4 and e_s <= 1e-4, (b, h, e_o, e_s)
            assert np.max(np.abs(st[b, h].double().cpu().numpy() - s_ref)) <= 1e-5 * np.max(np.abs(s_ref))


def _decode_start_from_prefill(n_distinct=4, T=1024, seed=61):
    """Decode starting caches as the decode workload specifies them: the final fp32 states and conv
    tails of 1024-token prefills with the layer's input distributions, computed by the oracle (so no
    oracle input comes from the GPU path). Returns (state [n, 48, 128, 128] fp32, conv [n, 3, C] bf16)."""
    inp = prefill_inputs([T] * n_distinct, n_qk_heads=16, n_v_heads=48, d_k=128, d_v=128,
                         io_dtype=torch.bfloat16, seed=seed)
    res = O.run_chains(vars(inp), [(n, h) for n in range(n_distinct) for h in range(48)])
    S = np.stack([r[1] for r in res]).reshape(n_distinct, 48, 128, 128)
    x_raw = torch.cat([inp.q.reshape(n_distinct * T, -1), inp.k.reshape(n_distinct * T, -1),
                       inp.v.reshape(n_distinct * T, -1)], 1).reshape(n_distinct, T, -1)
    tails = np.stack([O.conv_tail(x_raw[n].double().numpy(), np.zeros((3, x_raw.shape[2])))
                      for n in range(n_distinct)])
    return torch.from_numpy(S).float(), torch.from_numpy(tails).to(torch.bfloat16)


def _as_packed(di, steps, rows=None):
    """The first `steps` decode steps of the sequences `rows` as a packed prefill input (one sequence
    per decode row, its steps as tokens), for the oracle's chains."""
    rows = list(range(di.batch)) if rows is None else list(rows)
    pk = lambda x: x[:steps, rows].transpose(0, 1).reshape(len(rows) * steps, *x.shape[2:]).cpu()
    return dict(q=pk(di.q), k=pk(di.k), v=pk(di.v), alpha=pk(di.alpha), beta=pk(di.beta), gate=pk(di.gate),
                conv_w=di.conv_w.cpu(), norm_w=di.norm_w.cpu(), cu_seqlens=np.arange(len(rows) + 1) * steps,
                state_in=di.state[rows].cpu(), conv_in=di.conv_state[rows].cpu())


def test_decode_model_shape():
    """The decode workload: B=256 at model shape, bf16, starting from the states and conv tails that
    1024-token prefills leave (four oracle prefills, sequence b starting from prefill b % 4, each with
    its own decode inputs). All 256 sequences x 48 heads over the first 8 steps, and 4 sequences x 48
    heads over 1000 steps, against the oracle."""
    S4, C4 = _decode_start_from_prefill()
    di = decode_inputs(256, 1000, n_qk_heads=16, n_v_heads=48, d_k=128, d_v=128, io_dtype=torch.bfloat16,
                       device=DEV)
    di.state = S4.to(DEV)[torch.arange(256) % 4].contiguous()
    di.conv_state = C4.to(DEV)[torch.arange(256) % 4].contiguous()
    outs8, st8, _ = _decode_steps(di, 8)
    ref = O.run_chains(_as_packed(di, 8), [(b, h) for b in range(256) for h in range(48)])
    o_ref = np.stack([r[0] for r in ref]).reshape(256, 48, 8, 128).transpose(2, 0, 1, 3)
    s_ref = np.stack([r[1] for r in ref]).reshape(256, 48, 128, 128)
    e_o, e_s = rel_l2(outs8, o_ref), rel_l2(st8, s_ref)
    worst = max(max(rel_l2(outs8[:, b], o_ref[:, b]), rel_l2(st8[b], s_ref[b])) for b in range(256))
    print(f"8 steps, all 256 sequences: rel_l2 out={e_o:.3e} state={e_s:.3e}; worst sequence {worst:.3e}",
          flush=True)
    assert e_o <= 1e-2 and e_s <= 1e-2 and worst <= 1e-2
    outs, st, _ = _decode_steps(di, 1000)
    pick = (0, 85, 170, 255)
    ref = O.run_chains(_as_packed(di, 1000, pick), [(i, h) for i in range(4) for h in range(48)])
    for i, b in enumerate(pick):
        o_ref = np.stack([ref[48 * i + h][0] for h in range(48)], axis=1)
        s_ref = np.stack([ref[48 * i + h][1] for h in range(48)], axis=0)
        e_o, e_s = rel_l2(outs[:, b], o_ref), rel_l2(st[b], s_ref)
        print(f"1000 steps seq {b}: rel_l2 out={e_o:.3e} state={e_s:.3e}", flush=True)
        assert e_o <= 1e-2 and e_s <= 1e-2


def test_decode_equals_prefill_last_token():
    """prefill(T) and prefill(T-1) + decode_step agree on the last output and the final state."""
    T = 97
    inp = prefill_inputs([T], n_qk_heads=2, n_v_heads=6, d_k=128, d_v=128, io_dtype=torch.bfloat16,
                         seed=13, device=DEV, s0_std=0.01)
    out, st, cv = run_prefill(inp)
    head = prefill_inputs([T - 1], n_qk_heads=2, n_v_heads=6, d_k=128, d_v=128, io_dtype=torch.bfloat16,
                          seed=13, device=DEV)
    for key in ("q", "k", "v", "alpha", "beta", "gate"):
        setattr(head, key, getattr(inp, key)[:T - 1].contiguous())
    head.conv_w, head.norm_w, head.state_in = inp.conv_w, inp.norm_w, inp.state_in
    _, sh, ch = run_prefill(head)
    cfg = gdn.cfg_for(2, 6, 128, 128, torch.bfloat16)
    od = gdn.gdn_decode_step(cfg, inp.q[T - 1:], inp.k[T - 1:], inp.v[T - 1:], inp.alpha[T - 1:], inp.beta[T - 1:],
                             inp.gate[T - 1:], inp.conv_w, inp.norm_w, ch, sh)
    torch.cuda.synchronize()
    assert rel_l2(od[0], out[T - 1]) <= 1e-2 and rel_l2(sh, st) <= 1e-2
    assert torch.equal(ch, cv)


# ------------------------------------------------------------- speculative verify / commit -------

def _drafts(B, K, io, hk=2, hv=6, seed=31):
    """K draft tokens for B sequences (decode_inputs' step-major draw), with the drafts of
    sequence b as rows b*K .. b*K+K-1."""
    di = decode_inputs(B, K, n_qk_heads=hk, n_v_heads=hv, d_k=128, d_v=128, io_dtype=io, seed=seed,
                       device=DEV, state_std=0.02)
    packed = {key: getattr(di, key).transpose(0, 1).reshape(B * K, *getattr(di, key).shape[2:]).contiguous()
              for key in ("q", "k", "v", "alpha", "beta", "gate")}
    return di, packed


def _verify(cfg, K, di, p, state=None, conv=None):
    return gdn.gdn_verify(cfg, K, p["q"], p["k"], p["v"], p["alpha"], p["beta"], p["gate"], di.conv_w,
                          di.norm_w, di.conv_state if conv is None else conv, di.state if state is None else state)


@pytest.mark.parametrize("io", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("K", [1, 4, 5, 8])
def test_verify_commit(io, K):
    """Verify = the prefill of each K-token draft from the cache (which it leaves unchanged);
    commit(n) = the cache after the first n drafts, per sequence (n = 0 leaves it untouched)."""
    B = 5
    di, p = _drafts(B, K, io)
    cfg = gdn.cfg_for(2, 6, 128, 128, io)
    S0, c0 = di.state.clone(), di.conv_state.clone()
    print(f"verify io={io} K={K}", flush=True)
    out, log = _verify(cfg, K, di, p)
    torch.cuda.synchronize()
    assert torch.equal(di.state, S0) and torch.equal(di.conv_state, c0)
    cpu = {key: x.cpu() for key, x in p.items()}
    o_ref = O.gdn_verify(cpu, S0.cpu(), c0.cpu(), di.conv_w.cpu(), di.norm_w.cpu(), n_tok=K)
    e_o = rel_l2(out, o_ref)
    n_acc = [0, K, K // 2, 1, K - 1]
    print(f"commit n={n_acc}", flush=True)
    gdn.gdn_commit(cfg, K, torch.tensor(n_acc, dtype=torch.int32, device=DEV), log, di.conv_state, di.state)
    torch.cuda.synchronize()
    S_ref, c_ref = O.gdn_commit(cpu, np.array(n_acc), S0.cpu(), c0.cpu(), di.conv_w.cpu(), di.norm_w.cpu(), n_tok=K)
    e_s = rel_l2(di.state, S_ref)
    print(f"rel_l2 out={e_o:.3e} state={e_s:.3e}", flush=True)
    assert e_o <= TOL[io] and e_s <= TOL[io], (e_o, e_s)
    np.testing.assert_array_equal(di.conv_state.double().cpu().numpy(), c_ref)
    for b, n in enumerate(n_acc):
        if n == 0:
            assert torch.equal(di.state[b], S0[b]) and torch.equal(di.conv_state[b], c0[b])


@pytest.mark.parametrize("io", [torch.float32, torch.bfloat16])
def test_commit_then_verify_continues(io):
    """After committing 2 of 5 drafts, verifying the other 3 from the committed cache reproduces the
    first verify's outputs for them (to fp32 rounding, then the io rounding): the committed cache is
    the one verify's outputs assumed."""
    B, K, n = 4, 5, 2
    di, p = _drafts(B, K, io, seed=33)
    cfg = gdn.cfg_for(2, 6, 128, 128, io)
    out, log = _verify(cfg, K, di, p)
    gdn.gdn_commit(cfg, K, torch.full((B,), n, dtype=torch.int32, device=DEV), log, di.conv_state, di.state)
    rest = {key: x.reshape(B, K, *x.shape[1:])[:, n:].reshape(B * (K - n), *x.shape[1:]).contiguous()
            for key, x in p.items()}
    out2, _ = _verify(cfg, K - n, di, rest)
    torch.cuda.synchronize()
    tail = out.reshape(B, K, *out.shape[1:])[:, n:].reshape(B * (K - n), *out.shape[1:])
    err = rel_l2(out2, tail.double().cpu().numpy())
    print(f"continuation rel_l2 {err:.3e}", flush=True)
    assert err <= (1e-5 if io == torch.float32 else 4e-3)


def test_verify_commit_model_shape():
    """B = 256 sequences, 4-token drafts, 16 QK / 48 value heads, bf16: every 16th sequence against the
    oracle (outputs and committed states), accepted lengths 0..4."""
    B, K = 256, 4
    di, p = _drafts(B, K, torch.bfloat16, hk=16, hv=48, seed=35)
    cfg = gdn.cfg_for(16, 48, 128, 128, torch.bfloat16)
    S0, c0 = di.state.clone(), di.conv_state.clone()
    out, log = _verify(cfg, K, di, p)
    n_acc = torch.arange(B, dtype=torch.int32, device=DEV) % (K + 1)
    gdn.gdn_commit(cfg, K, n_acc, log, di.conv_state, di.state)
    torch.cuda.synchronize()
    pick = list(range(0, B, 16))
    rows = [b * K + t for b in pick for t in range(K)]
    cpu = {key: x[rows].cpu() for key, x in p.items()}
    o_ref = O.gdn_verify(cpu, S0[pick].cpu(), c0[pick].cpu(), di.conv_w.cpu(), di.norm_w.cpu(), n_tok=K)
    S_ref, c_ref = O.gdn_commit(cpu, n_acc[pick].cpu().numpy(), S0[pick].cpu(), c0[pick].cpu(), di.conv_w.cpu(),
                                di.norm_w.cpu(), n_tok=K)
    e_o, e_s = rel_l2(out[rows], o_ref), rel_l2(di.state[pick], S_ref)
    print(f"rel_l2 out={e_o:.3e} state={e_s:.3e}", flush=True)
    assert e_o <= TOL[torch.bfloat16] and e_s <= TOL[torch.bfloat16]
    np.testing.assert_array_equal(di.conv_state[pick].double().cpu().numpy(), c_ref)


# ------------------------------------------------------------------ projections around the mixer ---

def _proj(T, hidden, hk, hv, seed=41):
    from workloads import projection_inputs
    return projection_inputs(T, hidden=hidden, n_qk_heads=hk, n_v_heads=hv, d_k=128, d_v=128, seed=seed, device=DEV)


@pytest.mark.parametrize("T,hidden,hk,hv", [(200, 256, 2, 6), (512, 2560, 16, 48), (1, 64, 1, 3)])
def test_in_proj(T, hidden, hk, hv):
    """q | k | v and gate logits (bf16 GEMM outputs) and alpha, beta (fp32 gate pre-activations and
    formula) against the oracle's products of the same bf16 values."""
    p = _proj(T, hidden, hk, hv)
    cfg = gdn.cfg_for(hk, hv, 128, 128, torch.bfloat16)
    qkv, z, al, be = gdn.gdn_in_proj(cfg, p.x, p.w_qkv, p.w_z, p.w_ab, p.a_log, p.dt_bias)
    torch.cuda.synchronize()
    r_qkv, r_z, r_al, r_be = O.in_projection(p.x.cpu(), p.w_qkv.cpu().T, p.w_z.cpu().T, p.w_ab.cpu().T,
                                             p.a_log.cpu(), p.dt_bias.cpu())
    errs = (rel_l2(qkv, r_qkv), rel_l2(z.reshape(T, -1), r_z), rel_l2(al, r_al), rel_l2(be, r_be))
    print("rel_l2 qkv %.3e z %.3e alpha %.3e beta %.3e" % errs, flush=True)
    assert errs[0] <= TOL[torch.bfloat16] and errs[1] <= TOL[torch.bfloat16]
    assert errs[2] <= 1e-4 and errs[3] <= 1e-4


def test_out_proj():
    T, hidden = 300, 512
    p = _proj(T, hidden, 2, 6, seed=43)
    cfg = gdn.cfg_for(2, 6, 128, 128, torch.bfloat16)
    o = torch.randn((T, 6, 128), generator=torch.Generator(device=DEV).manual_seed(3), device=DEV).to(torch.bfloat16)
    y = gdn.gdn_out_proj(cfg, o, p.w_out)
    torch.cuda.synchronize()
    err = rel_l2(y, O.out_projection(o.cpu().reshape(T, -1), p.w_out.cpu().T))
    print(f"rel_l2 y {err:.3e}", flush=True)
    assert err <= TOL[torch.bfloat16]


def test_layer_end_to_end():
    """x -> input projection -> mixer (prefill, two packed sequences) -> output projection, against the
    oracle: its projections, with the projected activations rounded to bf16 as the GPU path stores
    them, its mixer, and its output projection."""
    T, hidden, hk, hv = 160, 256, 2, 6
    p = _proj(T, hidden, hk, hv, seed=45)
    cfg = gdn.cfg_for(hk, hv, 128, 128, torch.bfloat16)
    g = torch.Generator(device=DEV).manual_seed(7)
    conv_w = (torch.randn((2 * hk * 128 + hv * 128, 4), generator=g, device=DEV) * 0.5)
    norm_w = torch.randn((128,), generator=g, device=DEV) * 0.02
    cu = torch.tensor([0, 100, T], dtype=torch.int32, device=DEV)
    qkv, z, al, be = gdn.gdn_in_proj(cfg, p.x, p.w_qkv, p.w_z, p.w_ab, p.a_log, p.dt_bias)
    q, k, v = gdn.qkv_views(cfg, qkv)
    o = gdn.gdn_prefill(cfg, cu, q, k, v, al, be, z, conv_w, norm_w, cu_seqlens_host=cu.cpu())
    y = gdn.gdn_out_proj(cfg, o, p.w_out)
    torch.cuda.synchronize()
    r_qkv, r_z, r_al, r_be = O.in_projection(p.x.cpu(), p.w_qkv.cpu().T, p.w_z.cpu().T, p.w_ab.cpu().T,
                                             p.a_log.cpu(), p.dt_bias.cpu())
    bf = lambda a: torch.from_numpy(a).to(torch.bfloat16)
    qc = hk * 128
    inp = dict(q=bf(r_qkv[:, :qc]).reshape(T, hk, 128), k=bf(r_qkv[:, qc:2 * qc]).reshape(T, hk, 128),
               v=bf(r_qkv[:, 2 * qc:]).reshape(T, hv, 128), alpha=r_al, beta=r_be, gate=bf(r_z).reshape(T, hv, 128),
               conv_w=conv_w.cpu(), norm_w=norm_w.cpu(), cu_seqlens=cu.cpu().numpy())
    r_o, _, _ = O.gdn_prefill(inp)
    r_y = O.out_projection(r_o.reshape(T, -1), p.w_out.cpu().T)
    err = rel_l2(y, r_y)
    print(f"rel_l2 layer {err:.3e}", flush=True)
    assert err <= TOL[torch.bfloat16]
