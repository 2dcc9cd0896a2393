#!/usr/bin/env python3
"""Benchmark of the GDN token mixer on one MI355X.

Headline: prefill tokens/s of one GDN layer at model shape (B=1, T=4096, 16 QK / 48 value heads,
d=128, bf16 io, fp32 state). A step is one gdn_prefill call over that batch: conv + SiLU + L2,
WY transform, state propagation, output + RMSNorm + gate, conv tail. The decode step (B=256, one
token each, state streamed in place) and the speculative step (B=256, a 5-token draft each:
gdn_verify of all of it, then gdn_commit of the accepted tokens) are timed in the same run and
reported beside it.

The headline times K eager steps between two events on the library's stream. Per-kernel times
come from HIP events the library records on the same stream around each stage, in a second pass of
the same K steps right after (recording them inside the headline loop would add host work between
launches); the dominant kernel's algorithmic bytes (or flops) per launch divided by its mean
duration gives the roofline fraction. The fp64 CPU oracle is timed on the host as a baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
MFMA_FP32_PEAK_TFLOPS = 157.3   # MI355X dense fp32 MFMA

# Shape of the layer (16 QK heads, 48 value heads, d = 128, chunk 64).
HK, HV, D, CH = 16, 48, 128, 64


def stage_model(T: int, n_seqs: int):
    """Algorithmic bytes and flops of each prefill stage for T tokens (bf16 io, model shape).

    Bytes: each stage's inputs read once and outputs written once. Flops: dense-tile MFMA work
    (2 per multiply-add) of the stage's contractions.
    """
    nc = -(-T // CH)  # chunks (B=1 here: ceil(T / 64))
    per_tok = {
        # raw q/k/v in (20480 B) + normalised q/k/v out (20480 B)
        "conv_silu_l2": dict(bytes=40960 * T + 10240 * 16, flops=0.0, bound="hbm"),
        # k^, v^, alpha, beta in; U, Wk (bf16 64x128 per chunk and value head), G, K^T out
        "wy_or_sequential": dict(bytes=(4096 + 12288 + 384) * T + nc * (HV * (2 * 64 * 128 * 2 + 64 * 4) + HK * 128 * 64 * 2),
                                 flops=nc * HV * 3 * 2 * 64 * 64 * 128, bound="hbm"),
        # Wk, U, K^T, G in; chunk-start states (bf16 128x128) and W (bf16 128x64) out; final states
        "state": dict(bytes=nc * (HV * (2 * 64 * 128 * 2 + 64 * 4) + HK * 128 * 64 * 2)
                      + nc * HV * (128 * 128 * 2 + 128 * 64 * 2) + n_seqs * HV * 128 * 128 * 4,
                      flops=nc * HV * 2 * 2 * 64 * 128 * 128, bound="hbm"),
        # q^, k^, G, chunk states, W, gate in; o out
        "output_norm_gate": dict(bytes=(8192 + 12288 + 12288) * T + nc * HV * (128 * 128 * 2 + 128 * 64 * 2 + 64 * 4),
                                 flops=nc * HV * (2 * 64 * 64 * 128 + 2 * 64 * 128 * 128 + 2 * 64 * 64 * 128),
                                 bound="hbm"),
        "conv_tail": dict(bytes=n_seqs * 3 * 10240 * 2 * 2, flops=0.0, bound="hbm"),
        "chunk_table": dict(bytes=nc * 16, flops=0.0, bound="hbm"),
    }
    return per_tok


def path_bytes(lengths, state_in: bool, hk=HK, hv=HV, dk=D, dv=D, elem=2) -> float:
    """Compulsory bytes of a whole packed prefill: raw q/k/v, gate logits and output in the io dtype,
    alpha/beta fp32, the fp32 states (written; read too when given) and the conv tails written
    (45,440 B per token at the model shape in bf16, plus 3 MiB per sequence per state direction)."""
    T, N = sum(lengths), len(lengths)
    C = 2 * hk * dk + hv * dv
    per_tok = (C + 2 * hv * dv) * elem + hv * 8
    return float(per_tok * T + N * hv * dk * dv * 4 * (2 if state_in else 1) + N * 3 * C * elem)


def path_flops(lengths, hv=HV, dk=D, dv=D) -> float:
    """Dense-tile MFMA flops of the chunked algorithm per (64-token chunk, value head): Gram, U and Wk
    (3 x 2 C^2 d), the two state products (2 x 2 C d^2), Q K^T (2 C^2 d), Q S (2 C d^2) and P W
    (2 C^2 d) -- 8.65 MFLOP per token at the model shape; a sequence's last chunk counts in full."""
    nc = sum(-(-L // CH) for L in lengths)
    per_chunk_head = (3 * 2 * CH * CH * dk + 2 * 2 * CH * dk * dv + 2 * CH * CH * dk + 2 * CH * dk * dv
                      + 2 * CH * CH * dv)
    return float(nc * hv * per_chunk_head)


def path_roofline(lengths, state_in, ms, **shape):
    """The step against both compulsory bounds: HBM (path_bytes at 8 TB/s) and bf16 MFMA (path_flops
    at 2.5 PFLOP/s); `frac` is against the binding one, `frac_of_mfma_bound` the MFMA fraction alone."""
    pb = path_bytes(lengths, state_in, **shape)
    pf = path_flops(lengths, **{k: v for k, v in shape.items() if k in ("hv", "dk", "dv")})
    t_hbm, t_mfma = pb / (HBM_PEAK_GBPS * 1e9), pf / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    s = ms * 1e-3
    return dict(bytes=pb, flops=pf, hbm_bound_us=round(t_hbm * 1e6, 2), mfma_bound_us=round(t_mfma * 1e6, 2),
                bound="hbm" if t_hbm >= t_mfma else "mfma", frac=round(max(t_hbm, t_mfma) / s, 4),
                frac_of_hbm_bound=round(t_hbm / s, 4), frac_of_mfma_bound=round(t_mfma / s, 4),
                achieved_GBps=round(pb / s / 1e9, 1), achieved_TFLOPs=round(pf / s / 1e12, 2))


def decode_bytes(B: int) -> float:
    """Per decode step: state read + write, conv cache read + write, q/k/v, gate, o, alpha/beta."""
    return float(B * (HV * 128 * 128 * 4 * 2 + 3 * 10240 * 2 * 2 + 10240 * 2 + HV * 128 * 2 * 2 + HV * 8))


def verify_bytes(B: int, K: int) -> float:
    """Per speculative verify of K tokens: state read, conv cache read, raw q/k/v, gate, o and
    alpha/beta of the K tokens, and the log (k^ per QK head, e per value head in fp32, alpha/beta,
    raw inputs)."""
    C = 2 * HK * 128 + HV * 128
    per_tok = C * 2 + HV * 128 * 2 * 2 + HV * 8 + (HK + HV) * 128 * 4 + HV * 8 + C * 2
    return float(B * (HV * 128 * 128 * 4 + 3 * C * 2 + K * per_tok))


def commit_bytes(B: int, K: int) -> float:
    """Per commit of all K tokens: state read + write, the log's k^, e and alpha/beta of the K
    tokens, the 3 newest raw rows and the conv cache written."""
    C = 2 * HK * 128 + HV * 128
    return float(B * (HV * 128 * 128 * 4 * 2 + K * ((HK + HV) * 128 * 4 + HV * 8) + 3 * C * 2 * 2))


KERNEL_DIR = os.path.join(ROOT, "linear_attention_token_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def kernel_source_hash(src: str) -> str:
    """sha256 over a kernel's source file and the two headers every kernel includes."""
    h = hashlib.sha256()
    for f in (src, "gdn_device.h", "gdn_internal.h"):
        with open(os.path.join(KERNEL_DIR, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


STAGE_SOURCE = {"conv_silu_l2": "k_conv.hip", "wy_or_sequential": "k_wy.hip", "state": "k_state.hip",
                "output_norm_gate": "k_out.hip", "conv_tail": "k_conv.hip", "decode": "k_decode.hip",
                "verify": "k_mtp.hip", "commit": "k_mtp.hip"}


def measured_traffic(stage: str, grid_tag: str):
    """HBM bytes per launch of a stage from the committed counter summary (FETCH_SIZE and WRITE_SIZE
    scaled by a plain copy's readings), or None when absent, taken at another launch shape, or taken
    on a different kernel source than the one built now."""
    try:
        with open(TRAFFIC_FILE) as fh:
            k = json.load(fh)["kernels"][stage]
    except (OSError, KeyError, ValueError):
        return None
    if k.get("workload") != grid_tag or k.get("source_sha256") != kernel_source_hash(STAGE_SOURCE[stage]):
        return None
    return round(float(k["traffic_bytes"]))


MFMA_FILE = os.path.join(ROOT, "profiles", "mfma_counters.json")


def measured_mfma(stage: str, grid_tag: str):
    """MFMA busy fraction of a stage's kernel from the committed counter summary
    (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x 1024 SIMDs), or None when absent, taken at another
    launch shape, or on a different kernel source than the one built now."""
    try:
        with open(MFMA_FILE) as fh:
            k = json.load(fh)["kernels"][stage]
    except (OSError, KeyError, ValueError):
        return None
    if k.get("workload") != grid_tag or k.get("source_sha256") != kernel_source_hash(STAGE_SOURCE[stage]):
        return None
    return k.get("mfma_busy")


def prefill_step(gdn, inp, dev, with_state=True):
    """One gdn_prefill call over `inp` with preallocated outputs and workspace (state_out and conv_out
    written; state_in/conv_in as the workload gives them)."""
    import torch
    io = inp.io_dtype
    N, T = inp.n_seqs, int(inp.q.shape[0])
    cfg = gdn.cfg_for(inp.n_qk_heads, inp.n_v_heads, inp.d_k, inp.d_v, io)
    out = torch.empty((T, inp.n_v_heads, inp.d_v), dtype=io, device=dev)
    st = torch.empty((N, inp.n_v_heads, inp.d_k, inp.d_v), dtype=torch.float32, device=dev) if with_state else None
    cv = torch.empty((N, 3, inp.n_channels), dtype=io, device=dev)
    ws = torch.empty(max(1, gdn.gdn_prefill_workspace(cfg, N, T)), dtype=torch.uint8, device=dev)
    cu_host = inp.cu_seqlens.cpu()

    def step():
        gdn.gdn_prefill(cfg, inp.cu_seqlens, inp.q, inp.k, inp.v, inp.alpha, inp.beta, inp.gate, inp.conv_w,
                        inp.norm_w, state_in=inp.state_in, state_out=st, conv_in=inp.conv_in, conv_out=cv, out=out,
                        workspace=ws, cu_seqlens_host=cu_host)

    return step, (out, st, cv, ws)


def step_distribution(step, n, stream):
    """Per-step times (ms) from one event between consecutive steps: median, p10, p90, mean."""
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i in range(n):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    t = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(n))
    q = lambda f: t[min(n - 1, int(round(f * (n - 1))))]
    return dict(median=round(q(0.5), 5), p10=round(q(0.1), 5), p90=round(q(0.9), 5), mean=round(sum(t) / n, 5), n=n)


def stage_times(gdn, step, n, stream):
    """Per-stage mean times (ms) from the library's stage events, in a separate eager pass."""
    import ctypes
    import torch
    nev = gdn.N_STAGES + 1
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(n)]
    for row in evs:
        for e in row:
            e.record(stream)
    torch.cuda.synchronize()
    handles = [(ctypes.c_void_p * nev)(*[e.cuda_event for e in row]) for row in evs]
    for i in range(n):
        gdn.gdn_set_stage_events(handles[i])
        step()
    torch.cuda.synchronize()
    gdn.gdn_set_stage_events(None)
    return {name: sum(evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(n)) / n
            for j, name in enumerate(gdn.STAGE_NAMES)}


def config_legs(args, gdn, dev, stream):
    """The other prefill workloads, each timed over repeated calls (median, p10, p90) with its path
    roofline: the tiny fp32 case (token-sequential fp32 path, launch-bound), the 262,144-token prefill
    and the 32-sequence variable-length pack with initial states."""
    import torch
    from workloads import config_tiny, config_long, config_varlen
    legs = {}
    specs = [
        ("tiny", lambda: config_tiny(dev), 200,
         "B=1, T=64, 1 QK / 1 value head, d=16, fp32 io (token-sequential fp32 path), full layer"),
        ("long", lambda: config_long(dev, T=args.long_tokens), args.long_reps,
         f"B=1, T={args.long_tokens}, 16 QK / 48 value heads, d=128, bf16 io, fp32 state, full layer"),
        ("varlen", lambda: config_varlen(dev), args.long_reps,
         "32 sequences, lengths log-uniform in [512, 32768] (seed 0), S0 ~ N(0, 0.01), 16 QK / 48 value heads, "
         "d=128, bf16 io, fp32 state, full layer"),
    ]
    for name, make, reps, desc in specs:
        inp = make()
        lengths = [int(x) for x in torch.diff(inp.cu_seqlens.cpu()).tolist()]
        step, bufs = prefill_step(gdn, inp, dev)
        for _ in range(min(3, reps)):
            step()
        torch.cuda.synchronize()
        d = step_distribution(step, reps, stream)
        shape = dict(hk=inp.n_qk_heads, hv=inp.n_v_heads, dk=inp.d_k, dv=inp.d_v,
                     elem=2 if inp.io_dtype == torch.bfloat16 else 4)
        T = sum(lengths)
        legs[name] = dict(workload=desc, tokens=T, sequences=len(lengths), ms_per_call=d,
                          tokens_per_s=round(T / (d["median"] * 1e-3), 1),
                          path_roofline=path_roofline(lengths, inp.state_in is not None, d["median"], **shape))
        if name != "tiny":
            legs[name]["stage_ms"] = {k: round(v, 4) for k, v in stage_times(gdn, step, min(3, reps), stream).items()}
        del inp, bufs, step
        torch.cuda.empty_cache()
    legs["tiny"]["note"] = "launch-bound: the MFMA and HBM bounds of 64 tokens are far below one launch"
    return legs


def cpu_baseline(prefill_tokens: int, decode_batch: int):
    """The fp64 oracle as it stands, on the host's cores (a process pool over independent (sequence,
    value head) chains, one thread each): a prefill of the one-layer workload's first `prefill_tokens`
    tokens, all 48 value heads, and one decode step of `decode_batch` sequences (every (sequence, value
    head) chain with one token)."""
    import oracle as O
    from workloads import config_layer, decode_inputs
    workers = O.default_workers()
    inp = config_layer("cpu", T=prefill_tokens)
    d = vars(inp)
    O.prefill_chain(d, 0, 0)          # first-call warm-up in this process
    t0 = time.perf_counter()
    O.run_chains(d, [(0, h) for h in range(HV)], workers=workers)
    dt = time.perf_counter() - t0
    di = decode_inputs(decode_batch, 1, n_qk_heads=HK, n_v_heads=HV, d_k=D, d_v=D, seed=2)
    pk = lambda x: x[0]
    step = dict(q=pk(di.q), k=pk(di.k), v=pk(di.v), alpha=pk(di.alpha), beta=pk(di.beta), gate=pk(di.gate),
                conv_w=di.conv_w, norm_w=di.norm_w, cu_seqlens=list(range(decode_batch + 1)),
                state_in=di.state, conv_in=di.conv_state)
    t1 = time.perf_counter()
    O.run_chains(step, [(b, h) for b in range(decode_batch) for h in range(HV)], workers=workers)
    dd = time.perf_counter() - t1
    return dict(value=round(prefill_tokens / dt, 1), unit="tokens/s", cores=workers, kind="oracle",
                cpu_model=O.cpu_model(), host_cores=O.host_cores(),
                decode_us_per_step=round(dd * 1e6, 1),
                sample=f"fp64 numpy oracle (conv + SiLU + L2 + per-token recurrence + RMSNorm + gate) over a pool of "
                       f"{workers} single-thread processes: prefill of the first {prefill_tokens} tokens of the "
                       f"one-layer workload (B=1, all 48 value heads; 4096 is all of it) in {dt:.1f} s wall, "
                       f"scaled to tokens/s; one "
                       f"decode step at B={decode_batch} (all {decode_batch * HV} chains, one token each) in "
                       f"{dd:.1f} s wall")


# Multiply-adds per (64-token chunk, value head) of the chunked backward, by product (M x N x K):
# the forward recomputed (K K^T, Q K^T, U, Wk, the forward substitution of (I + A)^-1, the two state
# products of the forward chunk pass, and y = gQ S + P W for the norm and gate backward), then the backward
# (P^T dY, gQ^T dY, the two products of the reverse chunk pass, W dS'^T, dY S^T, dW S^T, dY W^T, dQK K,
# dQK^T Q, dT's two, T^T dW, T^T dWk, dA's two and the two K terms of dA).
CBWD_FMA_PER_CHUNK = (4 * 64 * 64 * 128 + 64 ** 3 // 6 + 2 * 64 * 128 * 128        # forward: WY and pass
                      + 64 * 128 * 128 + 64 * 128 * 64                              # forward: y
                      + 64 * 128 * 64 + 128 * 128 * 64 + 2 * 64 * 128 * 128         # backward pass and addends
                      + 3 * 64 * 128 * 128 + 64 * 64 * 128 + 2 * 64 * 128 * 64        # dK~, X, dWk, dP, dQ, dK
                      + 2 * 64 * 64 * 128 + 2 * 64 * 128 * 64 + 2 * 64 * 64 * 64      # dT, dbV, dbgK, dA
                      + 2 * 64 * 128 * 64)                                          # dK from dA


def backward_leg(args, dev, stream):
    """Backward of the whole mixer (conv + SiLU, L2, recurrence, RMSNorm, gate) at model shape (16 QK / 48
    value heads, d = 128, fp32), one sequence. The recurrence's part is the chunked form: per 64-token
    chunk and value head the WY factors are recomputed, the two chunk passes carry the state and its
    derivative across chunks, and the rest is chunk-parallel fp32 products, so the leg is priced against
    the fp32 MFMA peak on the products' multiply-adds (the HBM figure, inputs and outputs only, is given
    beside it)."""
    import torch
    from linear_attention_token_amd import gdn
    from workloads import prefill_inputs

    T = args.bwd_tokens
    inp = prefill_inputs([T], n_qk_heads=HK, n_v_heads=HV, d_k=D, d_v=D, io_dtype=torch.float32, seed=11,
                         device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(12)
    dout = torch.randn(T, HV, D, generator=g, device=dev)
    cfg = gdn.cfg_for(HK, HV, D, D, torch.float32)
    ws = torch.empty(gdn.gdn_backward_workspace(cfg, 1, T), dtype=torch.uint8, device=dev)

    def step():
        gdn.gdn_backward(cfg, inp.cu_seqlens, inp.q, inp.k, inp.v, inp.alpha, inp.beta, inp.gate, inp.conv_w,
                         inp.norm_w, dout, workspace=ws)

    step()
    torch.cuda.synchronize()
    n = 5
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    C = 2 * HK * D + HV * D
    # inputs (q, k, v, alpha, beta, gate, dout) read once, their derivatives written once, fp32
    io_bytes = 2 * 4 * T * (C + 2 * HV + HV * D + HV * D // 2)
    gb = io_bytes / (ms * 1e-3) / 1e9
    flops = 2 * CBWD_FMA_PER_CHUNK * (-(-T // CH)) * HV
    tf = flops / (ms * 1e-3) / 1e12
    ws_bytes = ws.numel()
    del ws
    torch.cuda.empty_cache()
    return {
        "workload": f"mixer backward, B=1, T={T}, 16 QK / 48 value heads, d=128, fp32, every step on: derivatives "
                    f"for q, k, v, alpha, beta, gate, conv weights and norm gain from dout",
        "ms_per_call": round(ms, 3), "tokens_per_s": round(T / (ms * 1e-3), 1), "workspace_bytes": ws_bytes,
        "roofline": dict(bound="mfma", achieved=round(tf, 2), peak=MFMA_FP32_PEAK_TFLOPS, unit="TFLOP/s",
                         frac=round(tf / MFMA_FP32_PEAK_TFLOPS, 4), algorithmic_flops=flops,
                         hbm_GBps_inputs_outputs=round(gb, 1), hbm_frac_inputs_outputs=round(gb / HBM_PEAK_GBPS, 4),
                         note="flops: the chunked form's fp32 products (forward recomputed, y included) per 64-token "
                              "chunk and value head; the chunk states and factors kept in the workspace are "
                              "not counted as HBM bytes"),
    }


def indexer_leg(args, dev, stream):
    """QSA compressed indexer: a decode step of B sequences at a long context (append the token's key,
    score every complete block, keep the top 512) and a prefill of one sequence (compress, then
    select for every token). Decode streams the compressed-key cache once per step, so it is priced
    against HBM; the prefill's block scores are a dense contraction on bf16 MFMA over a cache that
    stays in L2, so they are priced against the bf16 MFMA peak."""
    import torch
    from linear_attention_token_amd import qsa
    from workloads import indexer_inputs

    cfg = qsa.cfg_for(torch.bfloat16)
    B, N, S = args.qsa_batch, args.qsa_context, args.qsa_steps
    cap = N // 4

    def timed(fn, n):
        for _ in range(min(args.warmup, n, 5)):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    # decode: caches of N - 1 tokens per sequence, then the N-th token (it completes block N/4 - 1)
    kbar = torch.empty((B, cap, 128), dtype=torch.bfloat16, device=dev)
    pend = torch.empty((B, 3, 128), dtype=torch.bfloat16, device=dev)
    for b in range(B):
        x = indexer_inputs([N - 1], io_dtype=torch.bfloat16, seed=100 + b, device=dev, queries=False)
        qsa.qsa_compress(cfg, x.cu_seqlens, x.k, x.norm_w, kbar[b:b + 1], pend[b:b + 1])
        del x
    xs = indexer_inputs([B], io_dtype=torch.bfloat16, seed=99, device=dev)
    n_tok = torch.full((B,), N, dtype=torch.int32, device=dev)
    ws = torch.empty(qsa.qsa_workspace(cfg, B, cap), dtype=torch.uint8, device=dev)
    sel = torch.empty((B, cfg.topk), dtype=torch.int32, device=dev)
    nsel = torch.empty((B,), dtype=torch.int32, device=dev)
    tail = torch.empty((B,), dtype=torch.int32, device=dev)

    def dec():
        qsa.qsa_decode(cfg, n_tok, xs.q, xs.k, xs.norm_w, pend, kbar, sel, nsel, tail, workspace=ws)

    us_dec = timed(dec, S)
    nb = N // 4
    dec_bytes = B * (nb * 128 * 2 + 4 * 128 * 2 + 4 * 128 * 2 + cfg.topk * 4)
    gb = dec_bytes / (us_dec * 1e-6) / 1e9
    del kbar, ws
    torch.cuda.empty_cache()

    # prefill: one sequence of T tokens
    T = args.qsa_prefill
    xp = indexer_inputs([T], io_dtype=torch.bfloat16, seed=7, device=dev)
    capp = T // 4
    kb = torch.empty((1, capp, 128), dtype=torch.bfloat16, device=dev)
    wsp = torch.empty(qsa.qsa_workspace(cfg, T, capp), dtype=torch.uint8, device=dev)
    ps, pn, pt = (torch.empty((T, cfg.topk), dtype=torch.int32, device=dev),
                  torch.empty((T,), dtype=torch.int32, device=dev), torch.empty((T,), dtype=torch.int32, device=dev))

    def pre():
        qsa.qsa_compress(cfg, xp.cu_seqlens, xp.k, xp.norm_w, kb)
        qsa.qsa_select(cfg, xp.cu_seqlens, xp.q, kb, ps, pn, pt, workspace=wsp)

    us_pre = timed(pre, max(3, S // 10))
    pairs = sum((i + 1) // 4 for i in range(T))  # (token, complete block) scores
    flops = pairs * 4 * 128 * 2
    tf = flops / (us_pre * 1e-6) / 1e12
    del wsp
    torch.cuda.empty_cache()
    return {
        "workload": f"QSA indexer (4 query heads, 1 key head, d=128, blocks of 4, top-512, bf16 io): decode step of "
                    f"B={B} sequences at {N} tokens (append + score {nb} blocks + select), prefill of one "
                    f"{T}-token sequence (compress + select for every token)",
        "us_decode_step": round(us_dec, 2),
        "roofline_decode": dict(bound="hbm", achieved=round(gb, 1), peak=HBM_PEAK_GBPS, unit="GB/s",
                                frac=round(gb / HBM_PEAK_GBPS, 4), algorithmic_bytes=dec_bytes,
                                note="whole qsa_decode call: compressed-key cache read once"),
        "ms_prefill": round(us_pre / 1e3, 3), "prefill_tokens_per_s": round(T / (us_pre * 1e-6), 1),
        "roofline_prefill": dict(bound="mfma", achieved=round(tf, 2), peak=MFMA_BF16_PEAK_TFLOPS, unit="TFLOP/s",
                                 frac=round(tf / MFMA_BF16_PEAK_TFLOPS, 4), algorithmic_flops=flops,
                                 note="whole compress + select call over the block-score flops (bf16 MFMA)"),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--tokens", type=int, default=4096, help="prefill length (one sequence)")
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--decode-batch", type=int, default=256)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--spec-tokens", type=int, default=5,
                    help="tokens per speculative verify: the last sampled token + 4 MTP drafts")
    ap.add_argument("--spec-steps", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the reference timing of one captured HIP graph replayed per step")
    ap.add_argument("--cpu-tokens", type=int, default=4096,
                    help="tokens of the oracle's prefill (4096: the whole one-layer workload)")
    ap.add_argument("--long-tokens", type=int, default=262144, help="tokens of the long prefill workload")
    ap.add_argument("--long-reps", type=int, default=10, help="timed calls of the long and varlen workloads")
    ap.add_argument("--no-configs", action="store_true", help="skip the tiny, long and varlen prefill workloads")
    ap.add_argument("--hidden", type=int, default=2560, help="residual width of the layer leg")
    ap.add_argument("--qsa-context", type=int, default=1 << 20, help="tokens per sequence of the indexer decode")
    ap.add_argument("--qsa-batch", type=int, default=8, help="sequences of the indexer decode")
    ap.add_argument("--qsa-prefill", type=int, default=32768, help="tokens of the indexer prefill (one sequence)")
    ap.add_argument("--qsa-steps", type=int, default=50)
    ap.add_argument("--bwd-tokens", type=int, default=4096, help="tokens of the recurrence backward (one sequence)")
    ap.add_argument("--only", choices=["all", "prefill", "configs", "decode", "speculative", "layer", "indexer",
                                       "backward", "copy"],
                    default="all",
                    help="run one part only (for profilers); 'copy' times a plain 1 GiB device copy, the "
                         "reference kernel for scaling HBM byte counters")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the GDN mixer path here has no multi-GPU code "
              "(sequences and heads would shard without communication). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from linear_attention_token_amd import gdn
    from workloads import config_layer, decode_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    gdn.load_library()
    stream = torch.cuda.current_stream()

    if args.only == "copy":
        nbytes = 1 << 30
        src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).normal_()
        dst = torch.empty_like(src)
        for _ in range(args.warmup):
            dst.copy_(src)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            dst.copy_(src)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "ms_per_copy": round(ms, 4),
                          "GBps_read_plus_write": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}), flush=True)
        return

    cfg = gdn.cfg_for(HK, HV, D, D, torch.bfloat16)
    result = {}
    if args.only in ("all", "prefill"):
        # ---------------- headline prefill: one layer, B=1, T tokens ---------------------------------
        T = args.tokens
        inp = config_layer(dev, T=T)
        step, bufs = prefill_step(gdn, inp, dev)

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()

        # headline: K eager steps bracketed by events, no stage events inside
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t_wall = time.perf_counter()
        start.record(stream)
        for _ in range(args.steps):
            step()
        end.record(stream)
        torch.cuda.synchronize()
        t_wall = time.perf_counter() - t_wall
        ms_step = start.elapsed_time(end) / args.steps
        dist = step_distribution(step, args.steps, stream)

        # the same steps replayed from one captured HIP graph, for reference
        ms_step_graph = None
        if not args.no_graph:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                step()
            graph.replay()
            torch.cuda.synchronize()
            start.record(stream)
            for _ in range(args.steps):
                graph.replay()
            end.record(stream)
            torch.cuda.synchronize()
            ms_step_graph = start.elapsed_time(end) / args.steps

        stage_ms = stage_times(gdn, step, args.steps, stream)
        model = stage_model(T, 1)
        kernels = {}
        # the chunk table is built by the conv launch and the conv-cache tail by the output launch's
        # extra blocks: neither is a kernel of its own here, so their bytes count with those launches
        folded = {"chunk_table": "conv_silu_l2", "conv_tail": "output_norm_gate"}
        for name, ms in stage_ms.items():
            m = model[name]
            if name in folded or ms <= 0.0005 or m["bytes"] == 0:
                continue
            own = m["bytes"] + sum(model[f]["bytes"] for f, host in folded.items() if host == name)
            kernels[name] = dict(ms_per_launch=round(ms, 5), own_bytes=own,
                                 own_GBps=round(own / (ms * 1e-3) / 1e9, 1),
                                 own_frac_of_hbm=round(own / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                                 traffic=measured_traffic(name, f"prefill T={T}"),
                                 mfma_busy=measured_mfma(name, f"prefill T={T}"))
        path = path_roofline([T], False, ms_step)
        traffic = [k["traffic"] for k in kernels.values()]
        roof = dict(bound="hbm", achieved=path["achieved_GBps"], peak=HBM_PEAK_GBPS, unit="GB/s",
                    frac=round(path["achieved_GBps"] / HBM_PEAK_GBPS, 4),
                    traffic=(sum(traffic) if traffic and all(t is not None for t in traffic) else None),
                    kernel="whole prefill step (conv, WY, state and output kernels)",
                    ms_per_launch=round(ms_step, 5), algorithmic_bytes=path["bytes"],
                    algorithmic_flops=path["flops"], frac_of_mfma_bound=path["frac_of_mfma_bound"],
                    note="algorithmic bytes = compulsory traffic of the step (raw q/k/v, gate, o, alpha/beta, "
                         "final states, conv tails); traffic = counter-measured HBM bytes summed over the "
                         "step's kernels")

        result.update({
            "metric": "GDN prefill tokens/s/GPU (48 v-heads, d=128) + decode step us at B=256; % roofline",
            "value": round(T / (ms_step * 1e-3), 1),
            "unit": "tokens/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": round(ms_step, 5),
            "ms_per_step_graph_replay": round(ms_step_graph, 5) if ms_step_graph is not None else None,
            "ms_per_step_distribution": dist,
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": f"GDN layer prefill, B=1, T={T}, 16 QK / 48 value heads, d=128, chunk 64, "
                                   f"bf16 io, fp32 state, conv4+SiLU+L2+RMSNorm+sigmoid gate",
                       "batch": 1, "seq_len": T},
            "roofline": roof,
            "path_roofline": path,
            "stage_ms": {k: round(v, 5) for k, v in stage_ms.items()},
            "kernels": kernels,
            "wall_s": round(t_wall, 4),
        })
        del inp, bufs
        torch.cuda.empty_cache()

    if args.only in ("all", "prefill", "configs") and not args.no_configs:
        result["configs"] = config_legs(args, gdn, dev, stream)

    if args.only in ("all", "decode") and not args.no_decode:
        # ---------------- decode: B sequences, one token each ------------------------------------
        B, S = args.decode_batch, args.decode_steps
        di = decode_inputs(B, S, n_qk_heads=HK, n_v_heads=HV, d_k=D, d_v=D, io_dtype=torch.bfloat16,
                           device=dev)
        # starting states: the final state and conv tail of a 1024-token prefill of each sequence
        pre = config_layer(dev, T=1024 * B, seed=1)
        pre.cu_seqlens = (torch.arange(B + 1, dtype=torch.int32) * 1024).to(dev)
        st = torch.empty((B, HV, D, D), dtype=torch.float32, device=dev)
        cst = torch.empty((B, 3, 2 * HK * D + HV * D), dtype=torch.bfloat16, device=dev)
        gdn.gdn_prefill(cfg, pre.cu_seqlens, pre.q, pre.k, pre.v, pre.alpha, pre.beta, pre.gate, pre.conv_w,
                        pre.norm_w, state_out=st, conv_out=cst)
        del pre
        dout = torch.empty((B, HV, D), dtype=torch.bfloat16, device=dev)

        def dstep(i):
            gdn.gdn_decode_step(cfg, di.q[i], di.k[i], di.v[i], di.alpha[i], di.beta[i], di.gate[i],
                                di.conv_w, di.norm_w, cst, st, out=dout)

        for i in range(min(args.warmup, S)):
            dstep(i)
        torch.cuda.synchronize()
        d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        d0.record(stream)
        for i in range(S):
            dstep(i)
        d1.record(stream)
        torch.cuda.synchronize()
        us = d0.elapsed_time(d1) * 1e3 / S
        it = iter(range(S))
        ddist = step_distribution(lambda: dstep(next(it)), S, stream)
        db = decode_bytes(B)
        gbps = db / (us * 1e-6) / 1e9
        result["decode"] = {
            "workload": f"decode step, B={B} sequences x 1 token, 16 QK / 48 value heads, d=128, bf16 io, "
                        f"fp32 state in place, {S} consecutive steps",
            "us_per_step": round(us, 2),
            "us_per_step_median": round(ddist["median"] * 1e3, 2),
            "us_per_step_p10_p90": [round(ddist["p10"] * 1e3, 2), round(ddist["p90"] * 1e3, 2)],
            "roofline": dict(bound="hbm", achieved=round(gbps, 1), peak=HBM_PEAK_GBPS, unit="GB/s",
                             frac=round(gbps / HBM_PEAK_GBPS, 4),
                             traffic=measured_traffic("decode", f"decode B={B}"), kernel="decode",
                             algorithmic_bytes=db),
        }

    if args.only in ("all", "layer"):
        # ------------- the whole layer: input projection + gates, mixer, output projection ------------
        from workloads import projection_inputs
        T, Hd = 4096, args.hidden
        pj = projection_inputs(T, hidden=Hd, n_qk_heads=HK, n_v_heads=HV, d_k=D, d_v=D, device=dev, seed=5)
        lay = config_layer(dev, T=T)
        C = 2 * HK * D + HV * D
        qkv = torch.empty((T, C), dtype=torch.bfloat16, device=dev)
        zg = torch.empty((T, HV, D), dtype=torch.bfloat16, device=dev)
        al = torch.empty((T, HV), dtype=torch.float32, device=dev)
        be = torch.empty((T, HV), dtype=torch.float32, device=dev)
        lo = torch.empty((T, HV, D), dtype=torch.bfloat16, device=dev)
        ly = torch.empty((T, Hd), dtype=torch.bfloat16, device=dev)
        pws = torch.empty(gdn.gdn_proj_workspace(), dtype=torch.uint8, device=dev)
        lws = torch.empty(gdn.gdn_prefill_workspace(cfg, 1, T), dtype=torch.uint8, device=dev)
        lst = torch.empty((1, HV, D, D), dtype=torch.float32, device=dev)
        lq, lk, lv = gdn.qkv_views(cfg, qkv)
        cuh = lay.cu_seqlens.cpu()

        def in_proj():
            gdn.gdn_in_proj(cfg, pj.x, pj.w_qkv, pj.w_z, pj.w_ab, pj.a_log, pj.dt_bias, qkv=qkv, z=zg, alpha=al,
                            beta=be, workspace=pws)

        def mixer():
            gdn.gdn_prefill(cfg, lay.cu_seqlens, lq, lk, lv, al, be, zg, lay.conv_w, lay.norm_w, state_out=lst,
                            out=lo, workspace=lws, cu_seqlens_host=cuh)

        def out_proj():
            gdn.gdn_out_proj(cfg, lo, pj.w_out, y=ly, workspace=pws)

        def timed_n(fn, n):
            for _ in range(min(args.warmup, n)):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(n):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / n  # ms

        n = args.steps
        ms_in, ms_mix, ms_out = timed_n(in_proj, n), timed_n(mixer, n), timed_n(out_proj, n)
        ms_layer = timed_n(lambda: (in_proj(), mixer(), out_proj()), n)
        f_in = 2.0 * T * Hd * (C + HV * D + 2 * HV)
        f_out = 2.0 * T * HV * D * Hd

        def mroof(fl, ms):
            tf = fl / (ms * 1e-3) / 1e12
            return dict(bound="mfma", achieved=round(tf, 1), peak=MFMA_BF16_PEAK_TFLOPS, unit="TFLOP/s",
                        frac=round(tf / MFMA_BF16_PEAK_TFLOPS, 4), algorithmic_flops=fl)

        result["layer"] = {
            "workload": f"one GDN layer, B=1, T={T}, hidden {Hd}: input projection (q|k|v, gate logits, "
                        f"alpha/beta) + mixer (16 QK / 48 value heads, d=128) + output projection, bf16, "
                        f"synthetic weights",
            "ms_per_step": round(ms_layer, 5), "tokens_per_s": round(T / (ms_layer * 1e-3), 1),
            "ms_in_proj": round(ms_in, 5), "ms_mixer": round(ms_mix, 5), "ms_out_proj": round(ms_out, 5),
            "roofline_in_proj": mroof(f_in, ms_in), "roofline_out_proj": mroof(f_out, ms_out),
        }

    if args.only in ("all", "speculative") and not args.no_decode:
        # ------------- speculative decoding: B sequences, K-token drafts, verify + commit -----------
        B, K, S = args.decode_batch, args.spec_tokens, args.spec_steps
        sp = decode_inputs(B, K, n_qk_heads=HK, n_v_heads=HV, d_k=D, d_v=D, io_dtype=torch.bfloat16,
                           device=dev, seed=3)
        pk = {key: getattr(sp, key).transpose(0, 1).reshape(B * K, *getattr(sp, key).shape[2:]).contiguous()
              for key in ("q", "k", "v", "alpha", "beta", "gate")}
        sst, scs = sp.state, sp.conv_state
        sout = torch.empty((B * K, HV, D), dtype=torch.bfloat16, device=dev)
        slog = torch.empty(gdn.gdn_verify_log_bytes(cfg, B, K), dtype=torch.uint8, device=dev)
        nacc = torch.full((B,), K, dtype=torch.int32, device=dev)

        def verify():
            gdn.gdn_verify(cfg, K, pk["q"], pk["k"], pk["v"], pk["alpha"], pk["beta"], pk["gate"], sp.conv_w,
                           sp.norm_w, scs, sst, out=sout, log=slog)

        def commit():
            gdn.gdn_commit(cfg, K, nacc, slog, scs, sst)

        def timed(fn):
            for _ in range(min(args.warmup, S)):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(S):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / S

        us_v = timed(verify)
        us_c = timed(commit)
        us_s = timed(lambda: (verify(), commit()))
        vb, cb = verify_bytes(B, K), commit_bytes(B, K)
        acc = 4.06  # mean accepted length of four-step MTP speculation on the pages

        def roof(nbytes, us, kernel):
            gb = nbytes / (us * 1e-6) / 1e9
            return dict(bound="hbm", achieved=round(gb, 1), peak=HBM_PEAK_GBPS, unit="GB/s",
                        frac=round(gb / HBM_PEAK_GBPS, 4), traffic=measured_traffic(kernel, f"{kernel} B={B} K={K}"),
                        kernel=kernel, algorithmic_bytes=nbytes)

        result["speculative"] = {
            "workload": f"speculative decode step, B={B} sequences x {K}-token drafts (last sampled token + "
                        f"{K - 1} MTP drafts), 16 QK / 48 value heads, d=128, bf16 io, fp32 state; verify of all "
                        f"tokens, then commit of all of them",
            "us_verify": round(us_v, 2), "us_commit": round(us_c, 2), "us_per_step": round(us_s, 2),
            "mean_accepted_tokens": acc, "us_per_accepted_token": round(us_s / acc, 2),
            "roofline_verify": roof(vb, us_v, "verify"), "roofline_commit": roof(cb, us_c, "commit"),
        }

    if args.only in ("all", "indexer"):
        result["indexer"] = indexer_leg(args, dev, stream)

    if args.only in ("all", "backward"):
        result["backward"] = backward_leg(args, dev, stream)

    if not args.no_cpu_baseline and args.only == "all":
        result["cpu_baseline"] = cpu_baseline(args.cpu_tokens, args.decode_batch)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
