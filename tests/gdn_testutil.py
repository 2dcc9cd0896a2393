"""Helpers for the GPU parity tests: run the library through the C ABI, compare with the oracle."""
import numpy as np
import torch

import oracle as O
from linear_attention_token_amd import gdn

TOL = {torch.bfloat16: 1e-2, torch.float32: 1e-4}   # relative L2 on outputs and final states


def rel_l2(x, ref) -> float:
    """||x - ref||_2 / ||ref||_2 over the whole array, in fp64 (absolute error if ref is 0)."""
    x = x.detach().to("cpu").double().numpy() if hasattr(x, "detach") else np.asarray(x, np.float64)
    ref = ref.detach().to("cpu").double().numpy() if hasattr(ref, "detach") else np.asarray(ref, np.float64)
    num = np.linalg.norm((x - ref).ravel())
    den = np.linalg.norm(ref.ravel())
    return float(num / den) if den > 0 else float(num)


def cfg_of(inp, flags=gdn.GDN_ALL, **kw):
    return gdn.cfg_for(inp.n_qk_heads, inp.n_v_heads, inp.d_k, inp.d_v, inp.io_dtype, flags=flags, **kw)


def run_prefill(inp, flags=gdn.GDN_ALL, want_state=True, want_conv=True, workspace=None, **kw):
    """Runs gdn_prefill on inputs already on the GPU. Returns (out, state_out, conv_out)."""
    cfg = cfg_of(inp, flags, **kw)
    dev = inp.q.device
    N = inp.n_seqs
    state_out = torch.full((N, inp.n_v_heads, inp.d_k, inp.d_v), float("nan"), device=dev) if want_state else None
    conv_out = torch.zeros((N, 3, inp.n_channels), dtype=inp.io_dtype, device=dev) if want_conv else None
    out = gdn.gdn_prefill(cfg, inp.cu_seqlens, inp.q, inp.k, inp.v, inp.alpha, inp.beta, inp.gate,
                          inp.conv_w, inp.norm_w, state_in=inp.state_in, state_out=state_out,
                          conv_in=inp.conv_in, conv_out=conv_out, workspace=workspace,
                          cu_seqlens_host=inp.cu_seqlens.cpu())
    torch.cuda.synchronize()
    return out, state_out, conv_out


def oracle_prefill(inp, flags=O.FLAG_ALL):
    return O.gdn_prefill(vars(inp), flags=flags)


def oracle_chain(inp, n, h, flags=O.FLAG_ALL):
    return O.prefill_chain(vars(inp), n, h, flags=flags)


def seq_bounds(inp, n):
    cu = inp.cu_seqlens.cpu().numpy()
    return int(cu[n]), int(cu[n + 1])
