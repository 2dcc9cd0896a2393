"""GPU parity for options the C ABI accepts beyond the default layer: a per-head norm gain
(norm_head_stride = d_v), a readout scale other than 1, and calls without the optional gate logits
(gate = NULL with GDN_GATE off), on the chunked bf16 path, the token-sequential fp32 path and both
decode kernels, each against the fp64 oracle (rel-L2 <= 1e-2 bf16 io, <= 1e-4 fp32 io).
"""
import numpy as np
import pytest
import torch

import oracle as O
from workloads import prefill_inputs, decode_inputs

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from linear_attention_token_amd import gdn  # noqa: E402  (raises if libgdn.so is missing)
from gdn_testutil import TOL, rel_l2  # noqa: E402

gdn.load_library()
DEV = "cuda"
NO_GATE = gdn.GDN_CONV | gdn.GDN_L2QK | gdn.GDN_NORM


def _per_head_gain(hv, dv, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return 0.1 * torch.randn((hv, dv), generator=g, device=DEV)


def _prefill_case(inp, flags, per_head, scale, with_gate=True):
    hv, dv = inp.n_v_heads, inp.d_v
    if per_head:
        inp.norm_w = _per_head_gain(hv, dv, 77)
    cfg = gdn.cfg_for(inp.n_qk_heads, hv, inp.d_k, dv, inp.io_dtype, flags=flags, scale=scale,
                      norm_head_stride=dv if per_head else 0)
    N = inp.n_seqs
    st = torch.full((N, hv, inp.d_k, dv), float("nan"), device=DEV)
    cv = torch.zeros((N, 3, inp.n_channels), dtype=inp.io_dtype, device=DEV)
    print(f"prefill io={inp.io_dtype} d={dv} flags={flags} per_head={per_head} scale={scale} "
          f"gate={with_gate}", flush=True)
    out = gdn.gdn_prefill(cfg, inp.cu_seqlens, inp.q, inp.k, inp.v, inp.alpha, inp.beta,
                          inp.gate if with_gate else None, inp.conv_w, inp.norm_w, state_in=inp.state_in,
                          state_out=st, conv_in=inp.conv_in, conv_out=cv, cu_seqlens_host=inp.cu_seqlens.cpu())
    torch.cuda.synchronize()
    o_ref, s_ref, c_ref = O.gdn_prefill(vars(inp.to("cpu")), flags=flags, scale=scale)
    e_o, e_s = rel_l2(out, o_ref), rel_l2(st, s_ref)
    print(f"rel_l2 out={e_o:.3e} state={e_s:.3e}", flush=True)
    tol = TOL[inp.io_dtype]
    assert e_o <= tol and e_s <= tol, (e_o, e_s)
    np.testing.assert_array_equal(cv.double().cpu().numpy(), c_ref)


@pytest.mark.parametrize("io,d", [(torch.bfloat16, 128), (torch.float32, 128), (torch.bfloat16, 64),
                                  (torch.float32, 32)])
@pytest.mark.parametrize("flags", [gdn.GDN_ALL, gdn.GDN_CONV | gdn.GDN_L2QK | gdn.GDN_GATE])
@pytest.mark.parametrize("per_head,scale", [(True, 1.0), (False, 0.5), (True, 0.5)])
def test_prefill_gain_and_scale(io, d, flags, per_head, scale):
    """bf16 at d=128 runs the chunked MFMA path, the rest the token-sequential fp32 path: each with
    a per-head gain [HV][d_v] and/or scale 0.5, with the norm on (the scale then cancels up to eps)
    and off (the raw y is scaled, then gated)."""
    inp = prefill_inputs([150, 64, 3], n_qk_heads=2, n_v_heads=6, d_k=d, d_v=d, io_dtype=io, seed=51, device=DEV,
                         s0_std=0.02, conv_in_std=1.0)
    _prefill_case(inp, flags, per_head, scale)


@pytest.mark.parametrize("io,d", [(torch.bfloat16, 128), (torch.float32, 128), (torch.bfloat16, 64)])
def test_prefill_without_gate_logits(io, d):
    """GDN_GATE off and gate = NULL: no kernel reads the absent logits."""
    inp = prefill_inputs([130, 5], n_qk_heads=1, n_v_heads=3, d_k=d, d_v=d, io_dtype=io, seed=52, device=DEV,
                         s0_std=0.02)
    _prefill_case(inp, NO_GATE, False, 1.0, with_gate=False)


def _decode_case(B, steps, hk, hv, d, io, flags, per_head, scale, with_gate=True, seed=53):
    di = decode_inputs(B, steps, n_qk_heads=hk, n_v_heads=hv, d_k=d, d_v=d, io_dtype=io, device=DEV, seed=seed,
                       state_std=0.05)
    norm_w = _per_head_gain(hv, d, 78) if per_head else di.norm_w
    cfg = gdn.cfg_for(hk, hv, d, d, io, flags=flags, scale=scale, norm_head_stride=d if per_head else 0)
    state, conv = di.state.clone(), di.conv_state.clone()
    print(f"decode B={B} hk={hk} hv={hv} d={d} io={io} flags={flags} per_head={per_head} scale={scale} "
          f"gate={with_gate}", flush=True)
    outs = []
    for s in range(steps):
        outs.append(gdn.gdn_decode_step(cfg, di.q[s], di.k[s], di.v[s], di.alpha[s], di.beta[s],
                                        di.gate[s] if with_gate else None, di.conv_w, norm_w, conv, state))
    torch.cuda.synchronize()
    outs = torch.stack(outs)
    tol = TOL[io]
    for b in range(B):
        inp = dict(q=di.q[:, b], k=di.k[:, b], v=di.v[:, b], alpha=di.alpha[:, b], beta=di.beta[:, b],
                   gate=di.gate[:, b], conv_w=di.conv_w, norm_w=norm_w, cu_seqlens=np.array([0, steps]),
                   state_in=di.state[b:b + 1], conv_in=di.conv_state[b:b + 1])
        for h in range(hv):
            o_ref, s_ref = O.prefill_chain(inp, 0, h, flags=flags, scale=scale)
            e_o, e_s = rel_l2(outs[:, b, h], o_ref), rel_l2(state[b, h], s_ref)
            assert e_o <= tol and e_s <= tol, (b, h, e_o, e_s)
    x_last = torch.cat([di.q[steps - 3:steps].reshape(3, B, -1), di.k[steps - 3:steps].reshape(3, B, -1),
                        di.v[steps - 3:steps].reshape(3, B, -1)], -1)
    assert torch.equal(conv, x_last.transpose(0, 1))


@pytest.mark.parametrize("io", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("per_head,scale", [(True, 1.0), (False, 0.5), (True, 0.5)])
def test_decode_gain_and_scale(io, d, per_head, scale):
    """Head size 128 (the dedicated decode kernel) and 64 (the general one): per-head gains and a
    readout scale, with the norm on and off."""
    for flags in (gdn.GDN_ALL, gdn.GDN_CONV | gdn.GDN_L2QK | gdn.GDN_GATE):
        _decode_case(3, 4, 2, 6, d, io, flags, per_head, scale)


@pytest.mark.parametrize("io", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [128, 64])
def test_decode_without_gate_logits(io, d):
    """GDN_GATE off and gate = NULL at both decode kernels: the logits are never read."""
    _decode_case(3, 4, 2, 6, d, io, NO_GATE, False, 1.0, with_gate=False)
