"""GPU test of the allocation-free prefill (gdn_prefill_static): through the C ABI, its outputs,
final states and conv tails equal gdn_prefill's with a workspace (the same kernels on the same
inputs: bitwise) and the oracle's within the io tolerance, on two calls in a row, the second
smaller than the first (the static scratch keeps the first call's contents, which the kernels do
not depend on); a problem that needs more scratch than the library holds is refused.
"""
import numpy as np
import pytest
import torch

import oracle as O
from workloads import prefill_inputs

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from linear_attention_token_amd import gdn  # noqa: E402  (raises if libgdn.so is missing)
from gdn_testutil import TOL, rel_l2  # noqa: E402

gdn.load_library()
DEV = "cuda"


def _both(inp):
    cfg = gdn.cfg_for(inp.n_qk_heads, inp.n_v_heads, inp.d_k, inp.d_v, inp.io_dtype)
    N, T = inp.n_seqs, int(inp.q.shape[0])
    res = []
    for static in (False, True):
        st = torch.full((N, inp.n_v_heads, inp.d_k, inp.d_v), float("nan"), device=DEV)
        cv = torch.zeros((N, 3, inp.n_channels), dtype=inp.io_dtype, device=DEV)
        out = torch.full((T, inp.n_v_heads, inp.d_v), float("nan"), dtype=inp.io_dtype, device=DEV)
        fn = gdn.gdn_prefill_static if static else gdn.gdn_prefill
        print(f"{'static' if static else 'workspace'} prefill T={T} N={N} io={inp.io_dtype}", flush=True)
        fn(cfg, inp.cu_seqlens, inp.q, inp.k, inp.v, inp.alpha, inp.beta, inp.gate, inp.conv_w, inp.norm_w,
           state_in=inp.state_in, state_out=st, conv_in=inp.conv_in, conv_out=cv, out=out,
           cu_seqlens_host=inp.cu_seqlens.cpu())
        torch.cuda.synchronize()
        res.append((out, st, cv))
    return res


@pytest.mark.parametrize("io", [torch.bfloat16, torch.float32])
def test_static_prefill_equals_workspace_prefill_twice(io):
    big = prefill_inputs([700, 64, 236], n_qk_heads=16, n_v_heads=48, d_k=128, d_v=128, io_dtype=io, seed=71,
                         device=DEV, s0_std=0.01, conv_in_std=1.0)
    small = prefill_inputs([130, 2], n_qk_heads=16, n_v_heads=48, d_k=128, d_v=128, io_dtype=io, seed=72,
                           device=DEV, s0_std=0.01, conv_in_std=1.0)
    cfg = gdn.cfg_for(16, 48, 128, 128, io)
    assert gdn.gdn_prefill_workspace(cfg, 3, 1000) <= gdn.GDN_STATIC_WORKSPACE_BYTES
    for inp, chains in ((big, [(0, 0), (1, 17), (2, 47)]), (small, [(0, 5), (1, 46)])):
        (o_ws, s_ws, c_ws), (o_st, s_st, c_st) = _both(inp)
        assert torch.equal(o_st, o_ws) and torch.equal(s_st, s_ws) and torch.equal(c_st, c_ws)
        cpu = vars(inp.to("cpu"))
        cu = inp.cu_seqlens.cpu().numpy()
        for n, h in chains:
            o_ref, s_ref = O.prefill_chain(cpu, n, h)
            e_o, e_s = rel_l2(o_st[cu[n]:cu[n + 1], h], o_ref), rel_l2(s_st[n, h], s_ref)
            print(f"seq {n} head {h}: rel_l2 out={e_o:.3e} state={e_s:.3e}", flush=True)
            assert e_o <= TOL[io] and e_s <= TOL[io]
        x_raw = torch.cat([cpu["q"].reshape(cpu["q"].shape[0], -1), cpu["k"].reshape(cpu["k"].shape[0], -1),
                           cpu["v"].reshape(cpu["v"].shape[0], -1)], 1).double().numpy()
        for n in range(inp.n_seqs):
            tail = O.conv_tail(x_raw[cu[n]:cu[n + 1]], cpu["conv_in"][n].double().numpy())
            np.testing.assert_array_equal(c_st[n].double().cpu().numpy(), tail)


def test_static_prefill_refuses_oversized_problem():
    inp = prefill_inputs([4096], n_qk_heads=16, n_v_heads=48, d_k=128, d_v=128, io_dtype=torch.bfloat16, seed=73,
                         device=DEV)
    cfg = gdn.cfg_for(16, 48, 128, 128, torch.bfloat16)
    out = torch.zeros((4096, 48, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(gdn.GdnError, match="GDN_E_WORKSPACE"):
        gdn.gdn_prefill_static(cfg, inp.cu_seqlens, inp.q, inp.k, inp.v, inp.alpha, inp.beta, inp.gate, inp.conv_w,
                               inp.norm_w, out=out)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(out)) == 0
