"""Seeded synthetic workloads at the shapes of the Qwen3.8-Flash-Next GDN layer.

Layer shape (analysis notes "Qwen3.8-Flash-Next：架构、效率与技术谱系", §02 configuration table,
GDN row): 16 QK heads, 48 value heads, head dim 128, short causal conv of width 4 on Q/K/V.

Everything here is drawing random numbers; nothing computes the mixer. Tensors are drawn with
``torch.Generator(device).manual_seed(seed)`` in this fixed order:

    x_q, x_k, x_v, conv_w, alpha source, beta source, gate, norm gain w, S0, conv_in

bf16 tensors are drawn in fp32 and rounded to nearest even by ``Tensor.to(torch.bfloat16)``.
Packed sequence lengths come from ``numpy.random.default_rng(seed)`` before any tensor is drawn.
``N(mu, s)`` means standard deviation ``s``.

Decay alpha, two recipes:
  * ``"softplus"``: alpha = exp(-0.1 * softplus(z)), z ~ N(0, 1)      (tiny correctness case)
  * ``"loguniform"``: ln(alpha) ~ U(ln 0.9, ln 0.999)                   (model-shape cases)
Write strength: beta = sigmoid(z), z ~ N(0, 1).
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np
import torch

CONV_WIDTH = 4


@dataclass
class PrefillInputs:
    """Inputs of one packed prefill call. All tensors live on one device."""
    n_qk_heads: int
    n_v_heads: int
    d_k: int
    d_v: int
    io_dtype: torch.dtype
    cu_seqlens: torch.Tensor        # int32 [N+1]
    q: torch.Tensor                 # io [T, HK, d_k]   raw, before conv
    k: torch.Tensor                 # io [T, HK, d_k]
    v: torch.Tensor                 # io [T, HV, d_v]
    alpha: torch.Tensor             # f32 [T, HV]
    beta: torch.Tensor              # f32 [T, HV]
    gate: torch.Tensor              # io [T, HV, d_v]  sigmoid-gate logits
    conv_w: torch.Tensor            # f32 [C_tot, 4]   channel order q | k | v
    norm_w: torch.Tensor            # f32 [d_v]        zero-centred gain (multiplier 1 + w)
    state_in: Optional[torch.Tensor]  # f32 [N, HV, d_k, d_v] or None (zeros)
    conv_in: Optional[torch.Tensor]   # io [N, 3, C_tot] or None (zeros)

    @property
    def n_seqs(self) -> int:
        return int(self.cu_seqlens.numel()) - 1

    @property
    def total_tokens(self) -> int:
        return int(self.q.shape[0])

    @property
    def n_channels(self) -> int:
        return 2 * self.n_qk_heads * self.d_k + self.n_v_heads * self.d_v

    def to(self, device) -> "PrefillInputs":
        def mv(t):
            return None if t is None else t.to(device)
        return PrefillInputs(self.n_qk_heads, self.n_v_heads, self.d_k, self.d_v, self.io_dtype,
                             mv(self.cu_seqlens), mv(self.q), mv(self.k), mv(self.v), mv(self.alpha),
                             mv(self.beta), mv(self.gate), mv(self.conv_w), mv(self.norm_w),
                             mv(self.state_in), mv(self.conv_in))


@dataclass
class DecodeInputs:
    """Inputs of ``n_steps`` consecutive decode steps for ``batch`` sequences."""
    n_qk_heads: int
    n_v_heads: int
    d_k: int
    d_v: int
    io_dtype: torch.dtype
    q: torch.Tensor                 # io [S, B, HK, d_k]  one raw token per sequence per step
    k: torch.Tensor                 # io [S, B, HK, d_k]
    v: torch.Tensor                 # io [S, B, HV, d_v]
    alpha: torch.Tensor             # f32 [S, B, HV]
    beta: torch.Tensor              # f32 [S, B, HV]
    gate: torch.Tensor              # io [S, B, HV, d_v]
    conv_w: torch.Tensor            # f32 [C_tot, 4]
    norm_w: torch.Tensor            # f32 [d_v]
    state: torch.Tensor             # f32 [B, HV, d_k, d_v]  state before the first step
    conv_state: torch.Tensor        # io [B, 3, C_tot]       last 3 raw inputs per channel

    @property
    def batch(self) -> int:
        return int(self.state.shape[0])

    @property
    def n_steps(self) -> int:
        return int(self.q.shape[0])


def loguniform_lengths(seed: int, n: int, lo: int, hi: int) -> list[int]:
    """L = round(exp(U(ln lo, ln hi))), clipped to [lo, hi]."""
    rng = np.random.default_rng(seed)
    u = rng.uniform(math.log(lo), math.log(hi), size=n)
    return [int(min(hi, max(lo, round(math.exp(x))))) for x in u]


def _normal(g, shape, std, device):
    t = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    return t * std if std != 1.0 else t


def _alpha(g, shape, recipe, device):
    if recipe == "softplus":
        z = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
        return torch.exp(-0.1 * torch.nn.functional.softplus(z))
    if recipe == "loguniform":
        u = torch.rand(*shape, generator=g, device=device, dtype=torch.float32)
        lo, hi = math.log(0.9), math.log(0.999)
        return torch.exp(lo + (hi - lo) * u)
    if recipe == "one":
        return torch.ones(*shape, device=device, dtype=torch.float32)
    raise ValueError(f"unknown alpha recipe {recipe!r}")


def _beta(g, shape, recipe, device):
    if recipe == "sigmoid":
        return torch.sigmoid(torch.randn(*shape, generator=g, device=device, dtype=torch.float32))
    if recipe == "zero":
        return torch.zeros(*shape, device=device, dtype=torch.float32)
    if recipe == "one":
        return torch.ones(*shape, device=device, dtype=torch.float32)
    raise ValueError(f"unknown beta recipe {recipe!r}")


def prefill_inputs(lengths: Sequence[int], *, n_qk_heads: int, n_v_heads: int, d_k: int, d_v: int,
                   io_dtype: torch.dtype = torch.bfloat16, seed: int = 0, device="cpu",
                   alpha_recipe: str = "loguniform", beta_recipe: str = "sigmoid",
                   conv_std: float = 0.5, gain_std: float = 0.02, s0_std: Optional[float] = None,
                   conv_in_std: Optional[float] = None) -> PrefillInputs:
    """Draw one packed prefill workload (see the module docstring for the order and recipes)."""
    lengths = [int(x) for x in lengths]
    T = sum(lengths)
    N = len(lengths)
    hk, hv = n_qk_heads, n_v_heads
    C = 2 * hk * d_k + hv * d_v
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x_q = _normal(g, (T, hk, d_k), 1.0, device).to(io_dtype)
    x_k = _normal(g, (T, hk, d_k), 1.0, device).to(io_dtype)
    x_v = _normal(g, (T, hv, d_v), 1.0, device).to(io_dtype)
    conv_w = _normal(g, (C, CONV_WIDTH), conv_std, device)
    alpha = _alpha(g, (T, hv), alpha_recipe, device)
    beta = _beta(g, (T, hv), beta_recipe, device)
    gate = _normal(g, (T, hv, d_v), 1.0, device).to(io_dtype)
    norm_w = _normal(g, (d_v,), gain_std, device)
    state_in = None
    if s0_std is not None:
        state_in = _normal(g, (N, hv, d_k, d_v), s0_std, device)
    conv_in = None
    if conv_in_std is not None:
        conv_in = _normal(g, (N, CONV_WIDTH - 1, C), conv_in_std, device).to(io_dtype)
    cu = torch.zeros(N + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    return PrefillInputs(hk, hv, d_k, d_v, io_dtype, cu.to(device), x_q, x_k, x_v, alpha, beta,
                         gate, conv_w, norm_w, state_in, conv_in)


def decode_inputs(batch: int, n_steps: int, *, n_qk_heads: int, n_v_heads: int, d_k: int, d_v: int,
                  io_dtype: torch.dtype = torch.bfloat16, seed: int = 0, device="cpu",
                  alpha_recipe: str = "loguniform", state_std: float = 0.05,
                  conv_state_std: float = 1.0) -> DecodeInputs:
    """Draw ``n_steps`` decode steps for ``batch`` sequences.

    The starting state is drawn i.i.d. N(0, state_std) and the conv cache N(0, conv_state_std)
    (raw inputs are N(0, 1)); a caller that wants the state a real prefill leaves behind runs a
    prefill and passes its outputs instead.
    """
    hk, hv = n_qk_heads, n_v_heads
    C = 2 * hk * d_k + hv * d_v
    S, B = n_steps, batch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x_q = _normal(g, (S, B, hk, d_k), 1.0, device).to(io_dtype)
    x_k = _normal(g, (S, B, hk, d_k), 1.0, device).to(io_dtype)
    x_v = _normal(g, (S, B, hv, d_v), 1.0, device).to(io_dtype)
    conv_w = _normal(g, (C, CONV_WIDTH), 0.5, device)
    alpha = _alpha(g, (S, B, hv), alpha_recipe, device)
    beta = _beta(g, (S, B, hv), "sigmoid", device)
    gate = _normal(g, (S, B, hv, d_v), 1.0, device).to(io_dtype)
    norm_w = _normal(g, (d_v,), 0.02, device)
    state = _normal(g, (B, hv, d_k, d_v), state_std, device)
    conv_state = _normal(g, (B, CONV_WIDTH - 1, C), conv_state_std, device).to(io_dtype)
    return DecodeInputs(hk, hv, d_k, d_v, io_dtype, x_q, x_k, x_v, alpha, beta, gate, conv_w,
                        norm_w, state, conv_state)


@dataclass
class ProjectionInputs:
    """The layer's projections around the mixer, weights in the linear-layer layout [out][in]:
    x [T, hidden] (normalised residual stream, io dtype), w_qkv [C, hidden] (q | k | v rows in conv
    channel order), w_z [HV*dv, hidden] (gate logits), w_ab [2*HV, hidden] (decay / write gate
    pre-activations), a_log, dt_bias [HV] fp32 (the per-head gate vectors), w_out [hidden, HV*dv]."""
    x: torch.Tensor
    w_qkv: torch.Tensor
    w_z: torch.Tensor
    w_ab: torch.Tensor
    a_log: torch.Tensor
    dt_bias: torch.Tensor
    w_out: torch.Tensor


def projection_inputs(T: int, *, hidden: int, n_qk_heads: int, n_v_heads: int, d_k: int, d_v: int,
                      io_dtype: torch.dtype = torch.bfloat16, seed: int = 0, device="cpu") -> ProjectionInputs:
    """x ~ N(0, 1); weights ~ N(0, 1/fan_in) so projected values are ~N(0, 1); exp(A) ~ U(0.5, 2)
    and delta ~ U(-5, -2), which put alpha mostly in [0.9, 0.999] like the layer workloads."""
    C = 2 * n_qk_heads * d_k + n_v_heads * d_v
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    s_in, s_out = hidden ** -0.5, (n_v_heads * d_v) ** -0.5
    x = _normal(g, (T, hidden), 1.0, device).to(io_dtype)
    w_qkv = _normal(g, (C, hidden), s_in, device).to(io_dtype)
    w_z = _normal(g, (n_v_heads * d_v, hidden), s_in, device).to(io_dtype)
    w_ab = _normal(g, (2 * n_v_heads, hidden), s_in, device).to(io_dtype)
    a_log = torch.log(torch.rand((n_v_heads,), generator=g, device=device) * 1.5 + 0.5)
    dt_bias = torch.rand((n_v_heads,), generator=g, device=device) * 3.0 - 5.0
    w_out = _normal(g, (hidden, n_v_heads * d_v), s_out, device).to(io_dtype)
    return ProjectionInputs(x, w_qkv, w_z, w_ab, a_log, dt_bias, w_out)


@dataclass
class IndexerInputs:
    """Inputs of the QSA compressed indexer (analysis notes §02 configuration table, QSA indexer row:
    4 query heads and one shared key head of dim 128): q [T, 4, 128] and k [T, 128] in the io dtype,
    the RMSNorm gain norm_w [128] fp32, and the packing cu_seqlens int32 [N+1]."""
    cu_seqlens: torch.Tensor
    q: torch.Tensor
    k: torch.Tensor
    norm_w: torch.Tensor


def indexer_inputs(lengths: Sequence[int], *, io_dtype: torch.dtype = torch.bfloat16, seed: int = 0,
                   device="cpu", queries: bool = True) -> IndexerInputs:
    """q, k ~ N(0, 1) per element (the scale of a projection of the normalised residual stream);
    norm_w ~ U(0.5, 1.5). Drawn in the order q, k, norm_w; with queries=False (a key cache only)
    q is None and the draws start at k."""
    T = int(sum(lengths))
    cu = torch.tensor([0] + list(np.cumsum(lengths)), dtype=torch.int32, device=device)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    q = _normal(g, (T, 4, 128), 1.0, device).to(io_dtype) if queries else None
    k = _normal(g, (T, 128), 1.0, device).to(io_dtype)
    norm_w = torch.rand((128,), generator=g, device=device) + 0.5
    return IndexerInputs(cu, q, k, norm_w)


# --- the five workloads (tiny correctness case, one layer, long prefill, varlen, decode) -----

MODEL_HEADS = dict(n_qk_heads=16, n_v_heads=48, d_k=128, d_v=128)


def config_tiny(device="cpu", seed: int = 0) -> PrefillInputs:
    """B=1, T=64, one QK head, one value head, d=16, fp32; alpha = exp(-0.1 softplus(z))."""
    return prefill_inputs([64], n_qk_heads=1, n_v_heads=1, d_k=16, d_v=16, io_dtype=torch.float32,
                          seed=seed, device=device, alpha_recipe="softplus")


def config_layer(device="cpu", seed: int = 0, T: int = 4096) -> PrefillInputs:
    """One layer at model shape: B=1, T=4096, 16/48 heads, d=128, bf16 I/O, zero initial state."""
    return prefill_inputs([T], **MODEL_HEADS, io_dtype=torch.bfloat16, seed=seed, device=device)


def config_long(device="cpu", seed: int = 0, T: int = 262144) -> PrefillInputs:
    """Long prefill at the native context: B=1, T=262144, model shape, bf16 I/O."""
    return prefill_inputs([T], **MODEL_HEADS, io_dtype=torch.bfloat16, seed=seed, device=device)


def config_varlen(device="cpu", seed: int = 0, n: int = 32, lo: int = 512,
                  hi: int = 32768) -> PrefillInputs:
    """32 packed sequences, lengths log-uniform in [512, 32768], S0 ~ N(0, 0.01), conv_in = 0."""
    lengths = loguniform_lengths(seed, n, lo, hi)
    return prefill_inputs(lengths, **MODEL_HEADS, io_dtype=torch.bfloat16, seed=seed,
                          device=device, s0_std=0.01)


def config_decode(device="cpu", seed: int = 0, batch: int = 256, n_steps: int = 1000) -> DecodeInputs:
    """Batched decode at model shape: 256 sequences, one new token each, for n_steps steps."""
    return decode_inputs(batch, n_steps, **MODEL_HEADS, io_dtype=torch.bfloat16, seed=seed,
                         device=device)
