"""GPU parity of the QSA indexer (compression, block scores, top-k selection) against the fp64 oracle.

Compressed keys are compared element by element (rel-L2 1e-2 for bf16 storage, 1e-4 for fp32).
The selection is an integer result decided by floating point, so it is checked for what is unique:
list structure (ascending, complete blocks only, count min(topk, blocks), -1 padding, tail start)
exactly, and the chosen set against the oracle's fp64 scores S within an error bound E on the
kernel's scores. The kernel scores stored keys (rounded to the io dtype: |dk| <= 2^-8 |k| for bf16)
against rotated queries (fp32, and rounded to bf16 for the prefill's bf16 MFMA: another 2^-8), with
fp32 accumulation, so per query and block
    |s_kernel - S| <= sum_h sum_d |q_hd| |kbar_d| * c,   c = 2^-7 + 2e-5 (bf16), 2e-5 (fp32)
(ReLU is 1-Lipschitz). A valid selection then has min over chosen (S + E) >= max over the others
(S - E); where the oracle's k-th and (k+1)-th scores are further apart than that, the chosen set
is exactly the oracle's.
"""
import numpy as np
import pytest
import torch

import oracle as O
from workloads import IndexerInputs, indexer_inputs

pytestmark = pytest.mark.gpu

qsa = pytest.importorskip("linear_attention_token_amd.qsa")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

DEV = "cuda:0"
TOL_KBAR = {torch.bfloat16: 1e-2, torch.float32: 1e-4}
C_SCORE = {torch.bfloat16: 2.0 ** -7 + 2e-5, torch.float32: 2e-5}


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _rel(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def _check_rows(dtype, q_rows, pos, kb_or, sel, n_sel, tail, topk):
    """q_rows [M, 4, 128] (io values as fp64), pos [M] positions, kb_or [N, 128] the oracle's compressed
    keys of the rows' sequence; sel/n_sel/tail the kernel's outputs for those rows (numpy)."""
    M = len(pos)
    S = O.qsa_scores(q_rows, kb_or, pos) if kb_or.shape[0] else np.full((M, 0), -np.inf)
    qr = np.stack([O.partial_rope(q_rows[:, h], pos.astype(np.float64)) for h in range(4)], axis=1)
    E = C_SCORE[dtype] * np.einsum("mhd,nd->mn", np.abs(qr), np.abs(kb_or)) + 1e-30
    exact = compared = 0
    for i in range(M):
        nb = (pos[i] + 1) // 4
        cnt = min(topk, nb)
        assert n_sel[i] == cnt, (i, pos[i], n_sel[i], cnt)
        assert tail[i] == 4 * ((pos[i] + 1) // 4)
        row = sel[i]
        assert np.all(row[cnt:] == -1)
        chosen = row[:cnt]
        assert np.all(np.diff(chosen) > 0) and (cnt == 0 or (chosen[0] >= 0 and chosen[-1] < nb))
        if cnt == nb:
            continue
        s, e = S[i, :nb], E[i, :nb]
        mask = np.zeros(nb, bool)
        mask[chosen] = True
        lo = np.min(s[mask] + e[mask])
        hi = np.max(s[~mask] - e[~mask])
        assert lo >= hi, (i, pos[i], lo, hi)
        ref, _ = O.qsa_select(S[i:i + 1, :nb], pos[i:i + 1], topk=topk)
        exact += np.array_equal(ref[0], chosen)
        compared += 1
    return exact, compared


def _compress(cfg, x, cap, pending=True):
    n = x.cu_seqlens.numel() - 1
    io = x.k.dtype
    kbar = torch.full((n, cap, 128), 7.0, dtype=io, device=DEV)
    pend = torch.full((n, 3, 128), 7.0, dtype=io, device=DEV) if pending else None
    qsa.qsa_compress(cfg, x.cu_seqlens, x.k, x.norm_w, kbar, pend, cu_seqlens_host=x.cu_seqlens.cpu())
    return kbar, pend


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_compress_matches_oracle(dtype):
    lens = [0, 3, 4, 7, 130, 1029, 0, 2]
    x = indexer_inputs(lens, io_dtype=dtype, seed=11, device=DEV)
    cfg = qsa.cfg_for(dtype)
    cap = max(lens) // 4 + 5
    kbar, pend = _compress(cfg, x, cap)
    torch.cuda.synchronize()
    cu = x.cu_seqlens.cpu().numpy()
    k, w = _np(x.k), _np(x.norm_w)
    kb, pd = _np(kbar), _np(pend)
    for n, L in enumerate(lens):
        nb = L // 4
        ref = O.qsa_compress(k[cu[n]:cu[n + 1]], w)
        if nb:
            assert _rel(kb[n, :nb], ref) <= TOL_KBAR[dtype]
            assert np.max(np.abs(kb[n, :nb] - ref)) <= 40 * TOL_KBAR[dtype] * np.sqrt(np.mean(ref ** 2))
        assert np.all(kb[n, nb:] == 7.0), "blocks past the sequence must stay untouched"
        r = L % 4
        assert np.array_equal(pd[n, :r], k[cu[n] + L - r:cu[n + 1]])
        assert np.all(pd[n, r:] == 7.0)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("topk", [16, 512])
def test_prefill_select(dtype, topk):
    lens = [1, 3, 4, 5, 64, 257, 2051, 0, 3000]
    x = indexer_inputs(lens, io_dtype=dtype, seed=12, device=DEV)
    cfg = qsa.cfg_for(dtype, topk=topk)
    cap = max(lens) // 4 + 3
    kbar, _ = _compress(cfg, x, cap, pending=False)
    sel, n_sel, tail = qsa.qsa_select(cfg, x.cu_seqlens, x.q, kbar)
    torch.cuda.synchronize()
    cu = x.cu_seqlens.cpu().numpy()
    k, w, q = _np(x.k), _np(x.norm_w), _np(x.q)
    sel, n_sel, tail = sel.cpu().numpy(), n_sel.cpu().numpy(), tail.cpu().numpy()
    exact = compared = 0
    for n, L in enumerate(lens):
        if L == 0:
            continue
        s0, s1 = cu[n], cu[n + 1]
        kb = O.qsa_compress(k[s0:s1], w)
        e, c = _check_rows(dtype, q[s0:s1], np.arange(L), kb, sel[s0:s1], n_sel[s0:s1], tail[s0:s1], topk)
        exact, compared = exact + e, compared + c
    assert compared > 0
    if dtype == torch.float32:  # fp32 scores differ from fp64 by ~1e-6: ties within that are rare
        assert exact >= 0.95 * compared, (exact, compared)


def test_select_in_row_groups_equals_one_pass():
    """A workspace smaller than all rows runs the tokens in groups; the result is the same bits."""
    lens = [700, 1300]
    x = indexer_inputs(lens, io_dtype=torch.bfloat16, seed=13, device=DEV)
    cfg = qsa.cfg_for(torch.bfloat16, topk=32)
    cap = 400
    kbar, _ = _compress(cfg, x, cap, pending=False)
    full = qsa.qsa_select(cfg, x.cu_seqlens, x.q, kbar)
    ws = torch.empty(qsa.qsa_workspace(cfg, 97, cap), dtype=torch.uint8, device=DEV)
    part = qsa.qsa_select(cfg, x.cu_seqlens, x.q, kbar, workspace=ws)
    torch.cuda.synchronize()
    for a, b in zip(full, part):
        assert torch.equal(a, b)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_decode_appends_and_selects(dtype):
    """Prefill-compress a prefix per sequence, then decode 6 tokens one by one: blocks completed by the
    decode appends equal the oracle's compression of the whole sequence, pending keys are the raw
    tail, and each step's selection is valid for its query."""
    prefix = [0, 1, 2, 3, 4, 9, 1022, 2047]
    steps = 6
    B = len(prefix)
    full_lens = [p + steps for p in prefix]
    x = indexer_inputs(full_lens, io_dtype=dtype, seed=14, device=DEV)
    cfg = qsa.cfg_for(dtype, topk=64)
    cap = max(full_lens) // 4 + 2
    cu = x.cu_seqlens.cpu().numpy()
    idx_prefix = np.concatenate([np.arange(cu[b], cu[b] + prefix[b]) for b in range(B)]).astype(np.int64)
    cu_p = torch.tensor([0] + list(np.cumsum(prefix)), dtype=torch.int32, device=DEV)
    sub = IndexerInputs(cu_p, None, x.k[torch.as_tensor(idx_prefix, device=DEV)].contiguous(), x.norm_w)
    kbar, pend = _compress(cfg, sub, cap)
    k, w, q = _np(x.k), _np(x.norm_w), _np(x.q)
    for st in range(steps):
        rows = torch.as_tensor([cu[b] + prefix[b] + st for b in range(B)], device=DEV)
        n_tok = torch.tensor([prefix[b] + st + 1 for b in range(B)], dtype=torch.int32, device=DEV)
        sel, n_sel, tail = qsa.qsa_decode(cfg, n_tok, x.q[rows].contiguous(), x.k[rows].contiguous(), x.norm_w,
                                          pend, kbar)
        torch.cuda.synchronize()
        sel, n_sel, tail = sel.cpu().numpy(), n_sel.cpu().numpy(), tail.cpu().numpy()
        kb_all, pd = _np(kbar), _np(pend)
        for b in range(B):
            L = prefix[b] + st + 1
            kb = O.qsa_compress(k[cu[b]:cu[b] + L], w)
            if L // 4:
                assert _rel(kb_all[b, :L // 4], kb) <= TOL_KBAR[dtype]
            r = L % 4
            assert np.array_equal(pd[b, :r], k[cu[b] + L - r:cu[b] + L])
            _check_rows(dtype, q[cu[b] + L - 1:cu[b] + L], np.array([L - 1]), kb, sel[b:b + 1], n_sel[b:b + 1],
                        tail[b:b + 1], cfg.topk)


def test_decode_empty_sequences():
    """n_tok < 1 appends nothing and selects nothing (n_sel 0, all -1, tail 0)."""
    dtype = torch.bfloat16
    cfg = qsa.cfg_for(dtype)
    B, cap = 3, 16
    kbar = torch.full((B, cap, 128), 7.0, dtype=dtype, device=DEV)
    pend = torch.full((B, 3, 128), 7.0, dtype=dtype, device=DEV)
    q = torch.randn(B, 4, 128, device=DEV).to(dtype)
    k = torch.randn(B, 128, device=DEV).to(dtype)
    sel, n_sel, tail = qsa.qsa_decode(cfg, torch.tensor([0, -5, 0], dtype=torch.int32, device=DEV), q, k,
                                      torch.ones(128, device=DEV), pend, kbar)
    torch.cuda.synchronize()
    assert torch.all(n_sel == 0) and torch.all(tail == 0) and torch.all(sel == -1)
    assert torch.all(kbar == 7.0) and torch.all(pend == 7.0)


@pytest.mark.parametrize("dtype,n_tok", [(torch.bfloat16, [1 << 20, 700001]), (torch.float32, [70001, 140000])])
def test_decode_one_million_tokens(dtype, n_tok):
    """Model shape at the pages' longest context: two sequences at about 1M tokens (256K blocks, 16
    segments of the select, then the merge), top-512, compressed by a prefill and one decode append; and
    fp32 io at 70K / 140K tokens (2 and 3 segments)."""
    B = len(n_tok)
    x = indexer_inputs(n_tok, io_dtype=dtype, seed=15, device=DEV)
    cfg = qsa.cfg_for(dtype)
    cap = max(n_tok) // 4
    cu = x.cu_seqlens.cpu().numpy()
    keep = torch.cat([torch.arange(cu[b], cu[b + 1] - 1, device=DEV) for b in range(B)])
    cu_p = torch.tensor([0, n_tok[0] - 1, n_tok[0] + n_tok[1] - 2], dtype=torch.int32, device=DEV)
    sub = IndexerInputs(cu_p, None, x.k[keep].contiguous(), x.norm_w)
    kbar, pend = _compress(cfg, sub, cap)
    del sub
    last = torch.as_tensor([cu[b + 1] - 1 for b in range(B)], device=DEV)
    sel, n_sel, tail = qsa.qsa_decode(cfg, torch.tensor(n_tok, dtype=torch.int32, device=DEV),
                                      x.q[last].contiguous(), x.k[last].contiguous(), x.norm_w, pend, kbar)
    torch.cuda.synchronize()
    k, w = _np(x.k), _np(x.norm_w)
    kb_all = kbar.float().cpu().numpy()
    sel, n_sel, tail = sel.cpu().numpy(), n_sel.cpu().numpy(), tail.cpu().numpy()
    for b in range(B):
        L = n_tok[b]
        kb = O.qsa_compress(k[cu[b]:cu[b] + L], w)
        assert _rel(kb_all[b, :L // 4].astype(np.float64), kb) <= TOL_KBAR[dtype]
        qrow = _np(x.q[int(last[b])].unsqueeze(0))
        _check_rows(dtype, qrow, np.array([L - 1]), kb, sel[b:b + 1], n_sel[b:b + 1], tail[b:b + 1], cfg.topk)
    assert n_sel.tolist() == [512, 512]


@pytest.mark.parametrize("T,topk", [(20000, 512), (66000, 512), (66000, 509)])
def test_prefill_select_long_rows(T, topk):
    """One long sequence, sampled rows (including the last ones) against the oracle. 20000 tokens:
    caches of 5000 blocks take the 512-thread select, with 4, 8 or 16 scores per thread by row length
    (rows 8191 / 8195 and 16383 / 16387 sit on either side of 2048 and 4096 blocks); 66000: tokens past
    65536 see more than 16384 blocks (two select segments and the merge), and a top-k that is not a
    multiple of 4 takes the merge's 4-byte candidate reads."""
    dtype = torch.bfloat16
    x = indexer_inputs([T], io_dtype=dtype, seed=16, device=DEV)
    cfg = qsa.cfg_for(dtype, topk=topk)
    kbar, _ = _compress(cfg, x, T // 4, pending=False)
    sel, n_sel, tail = qsa.qsa_select(cfg, x.cu_seqlens, x.q, kbar)
    torch.cuda.synchronize()
    rows = np.concatenate([np.arange(T - 6, T), np.random.default_rng(0).integers(0, T, 10),
                           [3, 2050, T - 4461, 8191, 8195, 16383, 16387]])
    kb = O.qsa_compress(_np(x.k), _np(x.norm_w))
    r_t = torch.as_tensor(rows, device=DEV)
    _check_rows(dtype, _np(x.q[r_t]), rows, kb, sel[r_t].cpu().numpy(), n_sel[r_t].cpu().numpy(),
                tail[r_t].cpu().numpy(), cfg.topk)


@pytest.mark.parametrize("case", ["zero_scores", "equal_scores", "two_levels"])
def test_select_ties_exact(case):
    """Scores with exact ties, where the selection is fully determined: ties go to the lower block.
    zero_scores: q = 0, so every score is ReLU(0) = 0 -> blocks 0..k-1. equal_scores: no rotation
    (rope_dims 0) and one repeated key, q along it -> one positive score everywhere -> blocks 0..k-1.
    two_levels: even blocks hold key a, odd blocks key b, with q.a > q.b > 0 -> the first k even
    blocks. Checked for a prefill (one segment) and a decode row of 17500 blocks (two segments and
    the merge)."""
    dtype = torch.bfloat16
    k_top = 512
    cfg = qsa.cfg_for(dtype, topk=k_top, rope_dims=0 if case != "zero_scores" else 64)
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    a = torch.randn(128, generator=g, device=DEV)
    b = torch.randn(128, generator=g, device=DEV)
    b = b - (b @ a) / (a @ a) * a  # orthogonal to a
    for T in (4 * 1500, 70000):
        nblk = T // 4
        if case == "two_levels":
            blk = torch.where(torch.arange(nblk, device=DEV) % 2 == 0, 0, 1)
            keys = torch.stack([a, a + 0.5 * b])[blk]           # q.a > q.(a + b/2) > 0 for q = a + small
            k = keys.repeat_interleave(4, 0)
        else:
            k = a.expand(T, 128)
        k = k.to(dtype).contiguous()
        if case == "zero_scores":
            q = torch.zeros(1, 4, 128, dtype=dtype, device=DEV)
        else:
            q = (a - 0.1 * b).to(dtype).expand(1, 4, 128).contiguous()
        want = np.arange(k_top) if case != "two_levels" else 2 * np.arange(k_top)
        # decode row: the cache holds T - 1 keys, the T-th completes the last block
        kbar = torch.zeros((1, nblk, 128), dtype=dtype, device=DEV)
        pend = torch.zeros((1, 3, 128), dtype=dtype, device=DEV)
        cu = torch.tensor([0, T - 1], dtype=torch.int32, device=DEV)
        qsa.qsa_compress(cfg, cu, k[:T - 1].contiguous(), torch.ones(128, device=DEV), kbar, pend)
        sel, n_sel, _ = qsa.qsa_decode(cfg, torch.tensor([T], dtype=torch.int32, device=DEV), q,
                                       k[T - 1:].contiguous(), torch.ones(128, device=DEV), pend, kbar)
        torch.cuda.synchronize()
        assert int(n_sel[0]) == k_top
        assert np.array_equal(sel[0].cpu().numpy(), want), (case, T)
        if T <= 6000:  # prefill: the last token's row sees the same blocks
            cu2 = torch.tensor([0, T], dtype=torch.int32, device=DEV)
            sel2, _, _ = qsa.qsa_select(cfg, cu2, q.expand(T, 4, 128).contiguous(), kbar)
            torch.cuda.synchronize()
            assert np.array_equal(sel2[T - 1].cpu().numpy(), want), (case, "prefill")


@pytest.mark.parametrize("rope_dims", [128, 16])
def test_other_rope_widths(rope_dims):
    """qsa_cfg.rope_dims other than 64: compressed keys (fp32) and selections against the oracle."""
    dtype = torch.float32
    lens = [300, 45]
    x = indexer_inputs(lens, io_dtype=dtype, seed=17, device=DEV)
    cfg = qsa.cfg_for(dtype, topk=16, rope_dims=rope_dims)
    cap = 80
    kbar, _ = _compress(cfg, x, cap, pending=False)
    sel, n_sel, tail = qsa.qsa_select(cfg, x.cu_seqlens, x.q, kbar)
    torch.cuda.synchronize()
    cu = x.cu_seqlens.cpu().numpy()
    k, w, q, kb_all = _np(x.k), _np(x.norm_w), _np(x.q), _np(kbar)
    sel, n_sel, tail = sel.cpu().numpy(), n_sel.cpu().numpy(), tail.cpu().numpy()
    for n, L in enumerate(lens):
        s0 = cu[n]
        kb = O.qsa_compress(k[s0:s0 + L], w, rope_dims=rope_dims)
        assert _rel(kb_all[n, :L // 4], kb) <= TOL_KBAR[dtype]
        S = O.qsa_scores(q[s0:s0 + L], kb, np.arange(L), rope_dims=rope_dims)
        qr = np.stack([O.partial_rope(q[s0:s0 + L, h], np.arange(L, dtype=np.float64), rope_dims) for h in range(4)], 1)
        E = C_SCORE[dtype] * np.einsum("mhd,nd->mn", np.abs(qr), np.abs(kb)) + 1e-30
        for i in range(L):
            nb = (i + 1) // 4
            chosen = sel[s0 + i, :n_sel[s0 + i]]
            assert n_sel[s0 + i] == min(16, nb) and np.all(np.diff(chosen) > 0)
            rest = np.setdiff1d(np.arange(nb), chosen)
            if len(rest):
                assert np.min(S[i, chosen] + E[i, chosen]) >= np.max(S[i, rest] - E[i, rest])


def test_decode_graph_replay_matches_eager():
    """qsa_decode captured once in a HIP graph (workspace and outputs allocated beforehand) and replayed
    over four steps, with eager work and synchronisations in between: each replay equals an eager call
    on copies of the same caches."""
    dtype = torch.bfloat16
    cfg = qsa.cfg_for(dtype, topk=32)
    B, cap = 4, 600
    x = indexer_inputs([2000] * B, io_dtype=dtype, seed=18, device=DEV)
    kbar, pend = _compress(cfg, IndexerInputs(x.cu_seqlens, None, x.k, x.norm_w), cap)
    n_tok = torch.full((B,), 2001, dtype=torch.int32, device=DEV)
    q = torch.randn(B, 4, 128, device=DEV).to(dtype)
    k = torch.randn(B, 128, device=DEV).to(dtype)
    ws = torch.empty(qsa.qsa_workspace(cfg, B, cap), dtype=torch.uint8, device=DEV)
    outs = (torch.empty((B, 32), dtype=torch.int32, device=DEV), torch.empty(B, dtype=torch.int32, device=DEV),
            torch.empty(B, dtype=torch.int32, device=DEV))
    kb_g, pd_g = kbar.clone(), pend.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        qsa.qsa_decode(cfg, n_tok, q, k, x.norm_w, pd_g, kb_g, *outs, workspace=ws)  # warm-up on the side stream
    torch.cuda.current_stream().wait_stream(s)
    kb_g.copy_(kbar)
    pd_g.copy_(pend)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        qsa.qsa_decode(cfg, n_tok, q, k, x.norm_w, pd_g, kb_g, *outs, workspace=ws)
    kb_e, pd_e = kbar.clone(), pend.clone()
    kb_g.copy_(kbar)
    pd_g.copy_(pend)
    for step in range(4):
        n_tok.add_(1)
        q.normal_()
        k.normal_()
        graph.replay()
        torch.cuda.synchronize()
        ref = qsa.qsa_decode(cfg, n_tok, q, k, x.norm_w, pd_e, kb_e)
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(a, b), step
        assert torch.equal(kb_g, kb_e) and torch.equal(pd_g, pd_e), step
