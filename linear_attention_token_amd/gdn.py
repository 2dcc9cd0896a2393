"""Thin ctypes binding of libgdn.so (include/gdn.h), same entry-point names.

Argument marshalling only: tensors become device pointers and strides, the current torch stream
becomes the hipStream_t, outputs and the prefill workspace are allocated with torch. Every step of
the mixer runs in the library's HIP kernels. There is no fallback: without the built library or a
GPU these functions raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdn.so")

GDN_BF16, GDN_F32 = 0, 1
GDN_CONV, GDN_L2QK, GDN_NORM, GDN_GATE, GDN_ALL = 1, 2, 4, 8, 15
STATUS = {0: "GDN_OK", 1: "GDN_E_NULL", 2: "GDN_E_SHAPE", 3: "GDN_E_DTYPE", 4: "GDN_E_ALIGN",
          5: "GDN_E_WORKSPACE", 6: "GDN_E_UNSUPPORTED", 7: "GDN_E_HIP", 8: "GDN_E_VALUE"}
EXPORTS = ("gdn_cfg_default", "gdn_prefill_workspace", "gdn_prefill", "gdn_prefill_static", "gdn_decode_step",
           "gdn_verify_log_bytes", "gdn_verify", "gdn_commit",
           "gdn_proj_workspace", "gdn_in_proj", "gdn_out_proj",
           "gdn_recurrence_backward_workspace", "gdn_recurrence_backward", "gdn_backward_workspace", "gdn_backward",
           "gdn_set_stage_events", "gdn_status_string", "gdn_last_error", "gdn_abi_version")
N_STAGES = 6
STAGE_NAMES = ("chunk_table", "conv_silu_l2", "wy_or_sequential", "state", "output_norm_gate", "conv_tail")


class GdnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class gdn_cfg(ctypes.Structure):
    _fields_ = [("n_qk_heads", ctypes.c_int32), ("n_v_heads", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32), ("conv_width", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("flags", ctypes.c_uint32), ("scale", ctypes.c_float),
                ("l2_eps", ctypes.c_float), ("norm_eps", ctypes.c_float),
                ("norm_head_stride", ctypes.c_int32)]


_lib = None
_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def load_library(path: str = LIB_PATH):
    """Loads libgdn.so once and declares the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    lib.gdn_cfg_default.argtypes = [ctypes.POINTER(gdn_cfg)]
    lib.gdn_cfg_default.restype = None
    lib.gdn_prefill_workspace.argtypes = [ctypes.POINTER(gdn_cfg), ctypes.c_int32, _I64,
                                          ctypes.POINTER(ctypes.c_size_t)]
    lib.gdn_prefill_workspace.restype = ctypes.c_int
    lib.gdn_prefill.argtypes = [ctypes.POINTER(gdn_cfg), ctypes.c_int32, _I64, _P, _P, _P, _P, _P,
                                _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                ctypes.c_size_t, _P]
    lib.gdn_prefill.restype = ctypes.c_int
    lib.gdn_prefill_static.argtypes = [ctypes.POINTER(gdn_cfg), ctypes.c_int32, _I64, _P, _P, _P, _P, _P,
                                       _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]
    lib.gdn_prefill_static.restype = ctypes.c_int
    lib.gdn_decode_step.argtypes = [ctypes.POINTER(gdn_cfg), ctypes.c_int32, _P, _P, _P, _I64, _I64,
                                    _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P]
    lib.gdn_decode_step.restype = ctypes.c_int
    lib.gdn_verify_log_bytes.argtypes = [ctypes.POINTER(gdn_cfg), ctypes.c_int32, ctypes.c_int32,
                                         ctypes.POINTER(ctypes.c_size_t)]
    lib.gdn_verify_log_bytes.restype = ctypes.c_int
    lib.gdn_verify.argtypes = [ctypes.POINTER(gdn_cfg), ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _I64, _I64,
                               _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.gdn_verify.restype = ctypes.c_int
    lib.gdn_commit.argtypes = [ctypes.POINTER(gdn_cfg), ctypes.c_int32, ctypes.c_int32, _P, _P, ctypes.c_size_t,
                               _P, _P, _P]
    lib.gdn_commit.restype = ctypes.c_int
    lib.gdn_proj_workspace.argtypes = [ctypes.POINTER(ctypes.c_size_t)]
    lib.gdn_proj_workspace.restype = ctypes.c_int
    lib.gdn_in_proj.argtypes = [ctypes.POINTER(gdn_cfg), ctypes.c_int32, _I64, _P, _I64, _P, _P, _P, _P, _P, _P, _P,
                                _P, _P, _P, ctypes.c_size_t, _P]
    lib.gdn_in_proj.restype = ctypes.c_int
    lib.gdn_out_proj.argtypes = [ctypes.POINTER(gdn_cfg), ctypes.c_int32, _I64, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.gdn_out_proj.restype = ctypes.c_int
    lib.gdn_status_string.argtypes = [ctypes.c_int]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_last_error.argtypes = []
    lib.gdn_last_error.restype = ctypes.c_char_p
    lib.gdn_set_stage_events.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int32]
    lib.gdn_set_stage_events.restype = ctypes.c_int
    lib.gdn_abi_version.argtypes = []
    lib.gdn_abi_version.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise GdnError(status, load_library().gdn_last_error().decode())


def gdn_cfg_default(**overrides) -> gdn_cfg:
    """The library's default configuration (model shape, bf16, all stages), then ``overrides``."""
    cfg = gdn_cfg()
    load_library().gdn_cfg_default(ctypes.byref(cfg))
    for k, v in overrides.items():
        setattr(cfg, k, v)
    return cfg


def gdn_abi_version() -> int:
    return load_library().gdn_abi_version()


_stage_events = None  # the array the library points at, kept alive while it is set


def gdn_set_stage_events(events) -> None:
    """Records raw hipEvent_t handles around each prefill stage (None switches it off).

    ``events`` is a ctypes array of N_STAGES + 1 handles (or a sequence of integer handles, copied
    into one); the array stays referenced here until the next call, since the library keeps its
    address. The events themselves must outlive the prefills that record them."""
    global _stage_events
    lib = load_library()
    if events is None:
        _check(lib.gdn_set_stage_events(None, 0))
        _stage_events = None
        return
    if not isinstance(events, ctypes.Array):
        events = (ctypes.c_void_p * len(events))(*events)
    _check(lib.gdn_set_stage_events(events, len(events)))
    _stage_events = events


def gdn_prefill_workspace(cfg: gdn_cfg, n_seqs: int, total_tokens: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().gdn_prefill_workspace(ctypes.byref(cfg), n_seqs, total_tokens, ctypes.byref(n)))
    return int(n.value)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("gdn tensors must be on the GPU")
    return t.data_ptr()


def _row_stride(t: torch.Tensor, inner: int) -> int:
    """Token row stride of a [rows, heads, dim] view whose (heads, dim) block is contiguous."""
    if t.dim() != 3 or t.stride(2) != 1 or t.stride(1) != t.shape[2]:
        raise ValueError("q/k/v need contiguous (heads, dim) blocks per token")
    return t.stride(0) if t.shape[0] > 0 else inner


def _expect(t, shape, dtype, name, optional=False):
    """Host-side check that a buffer has exactly the shape, dtype and layout the kernels index."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name}: expected {tuple(shape)} {dtype}, got {tuple(t.shape)} {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_common(cfg, T, io, alpha, beta, gate, conv_w, norm_w, out):
    hv, dv = cfg.n_v_heads, cfg.d_v
    C = 2 * cfg.n_qk_heads * cfg.d_k + hv * dv
    _expect(alpha, (T, hv), torch.float32, "alpha")
    _expect(beta, (T, hv), torch.float32, "beta")
    _expect(gate, (T, hv, dv), io, "gate", optional=not (cfg.flags & GDN_GATE))
    _expect(conv_w, (C, 4), torch.float32, "conv_w", optional=not (cfg.flags & GDN_CONV))
    if cfg.flags & GDN_NORM:
        shape = (dv,) if cfg.norm_head_stride == 0 else (hv, dv)
        _expect(norm_w, shape, torch.float32, "norm_w")
    _expect(out, (T, hv, dv), io, "out")
    return C


def _check_qkv(cfg, q, k, v, io):
    T = int(q.shape[0])
    for t, name, heads, d in ((q, "q", cfg.n_qk_heads, cfg.d_k), (k, "k", cfg.n_qk_heads, cfg.d_k),
                              (v, "v", cfg.n_v_heads, cfg.d_v)):
        if t.dim() != 3 or tuple(t.shape) != (T, heads, d) or t.dtype != io:
            raise ValueError(f"{name}: expected ({T}, {heads}, {d}) {io}, got {tuple(t.shape)} {t.dtype}")
    return T


def _io_dtype(cfg):
    return torch.bfloat16 if cfg.io_dtype == GDN_BF16 else torch.float32


def _stream(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _prefill(cfg, cu_seqlens, q, k, v, alpha, beta, gate, conv_w, norm_w, state_in, state_out, conv_in, conv_out,
             out, workspace, cu_seqlens_host, stream, static):
    lib = load_library()
    io = _io_dtype(cfg)
    n_seqs = int(cu_seqlens.numel()) - 1
    T = _check_qkv(cfg, q, k, v, io)
    if out is None:
        out = torch.empty((T, cfg.n_v_heads, cfg.d_v), dtype=io, device=q.device)
    C = _check_common(cfg, T, io, alpha, beta, gate, conv_w, norm_w, out)
    _expect(cu_seqlens, (n_seqs + 1,), torch.int32, "cu_seqlens")
    sshape = (n_seqs, cfg.n_v_heads, cfg.d_k, cfg.d_v)
    _expect(state_in, sshape, torch.float32, "state_in", optional=True)
    _expect(state_out, sshape, torch.float32, "state_out", optional=True)
    _expect(conv_in, (n_seqs, 3, C), io, "conv_in", optional=True)
    _expect(conv_out, (n_seqs, 3, C), io, "conv_out", optional=True)
    if not static:
        need = gdn_prefill_workspace(cfg, n_seqs, T)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        if workspace.dtype != torch.uint8 or workspace.numel() < need:
            raise ValueError(f"workspace needs {need} uint8 elements")
    host = None
    if cu_seqlens_host is not None:
        host = cu_seqlens_host.to(torch.int32).contiguous()
    args = [ctypes.byref(cfg), n_seqs, T, _ptr(cu_seqlens), host.data_ptr() if host is not None else None,
            _ptr(q), _ptr(k), _ptr(v), _row_stride(q, cfg.n_qk_heads * cfg.d_k),
            _row_stride(k, cfg.n_qk_heads * cfg.d_k), _row_stride(v, cfg.n_v_heads * cfg.d_v),
            _ptr(alpha), _ptr(beta), _ptr(gate), _ptr(conv_w), _ptr(norm_w),
            _ptr(state_in), _ptr(state_out), _ptr(conv_in), _ptr(conv_out), _ptr(out)]
    if static:
        st = lib.gdn_prefill_static(*args, _stream(stream))
    else:
        st = lib.gdn_prefill(*args, _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st)
    return out


def gdn_prefill(cfg: gdn_cfg, cu_seqlens: torch.Tensor, q, k, v, alpha, beta, gate, conv_w, norm_w,
                state_in=None, state_out=None, conv_in=None, conv_out=None, out=None, workspace=None,
                cu_seqlens_host: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Packed prefill; returns ``out`` [T, HV, d_v] (allocated when not given).

    Writes ``state_out`` / ``conv_out`` when given. ``workspace`` (uint8, >= gdn_prefill_workspace
    bytes) is allocated when not given.
    """
    return _prefill(cfg, cu_seqlens, q, k, v, alpha, beta, gate, conv_w, norm_w, state_in, state_out, conv_in,
                    conv_out, out, workspace, cu_seqlens_host, stream, static=False)


def gdn_prefill_static(cfg: gdn_cfg, cu_seqlens: torch.Tensor, q, k, v, alpha, beta, gate, conv_w, norm_w,
                       state_in=None, state_out=None, conv_in=None, conv_out=None, out=None,
                       cu_seqlens_host: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """gdn_prefill on the library's static scratch (no workspace): the call itself allocates nothing
    when ``out`` is given. Problems whose workspace exceeds GDN_STATIC_WORKSPACE_BYTES raise
    GDN_E_WORKSPACE; overlapping calls on one GPU race."""
    return _prefill(cfg, cu_seqlens, q, k, v, alpha, beta, gate, conv_w, norm_w, state_in, state_out, conv_in,
                    conv_out, out, None, cu_seqlens_host, stream, static=True)


GDN_STATIC_WORKSPACE_BYTES = 128 << 20


def gdn_decode_step(cfg: gdn_cfg, q, k, v, alpha, beta, gate, conv_w, norm_w, conv_state, state,
                    out=None, stream=None) -> torch.Tensor:
    """One decode step for B sequences; updates ``state`` and ``conv_state`` in place."""
    lib = load_library()
    io = _io_dtype(cfg)
    B = _check_qkv(cfg, q, k, v, io)
    if out is None:
        out = torch.empty((B, cfg.n_v_heads, cfg.d_v), dtype=io, device=q.device)
    C = _check_common(cfg, B, io, alpha, beta, gate, conv_w, norm_w, out)
    _expect(state, (B, cfg.n_v_heads, cfg.d_k, cfg.d_v), torch.float32, "state")
    _expect(conv_state, (B, 3, C), io, "conv_state", optional=not (cfg.flags & GDN_CONV))
    st = lib.gdn_decode_step(ctypes.byref(cfg), B, _ptr(q), _ptr(k), _ptr(v),
                             _row_stride(q, cfg.n_qk_heads * cfg.d_k), _row_stride(k, cfg.n_qk_heads * cfg.d_k),
                             _row_stride(v, cfg.n_v_heads * cfg.d_v), _ptr(alpha), _ptr(beta), _ptr(gate),
                             _ptr(conv_w), _ptr(norm_w), _ptr(conv_state), _ptr(state), _ptr(out),
                             _stream(stream))
    _check(st)
    return out


def gdn_verify_log_bytes(cfg: gdn_cfg, batch: int, n_tok: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().gdn_verify_log_bytes(ctypes.byref(cfg), batch, n_tok, ctypes.byref(n)))
    return int(n.value)


def gdn_verify(cfg: gdn_cfg, n_tok: int, q, k, v, alpha, beta, gate, conv_w, norm_w, conv_state, state,
               out=None, log=None, stream=None):
    """Speculative verify of ``n_tok`` draft tokens per sequence (rows b*K .. b*K+K-1 of q, k, v,
    alpha, beta, gate). Reads ``state`` and ``conv_state`` without changing them; returns
    (out [B*K, HV, d_v], log), allocating either when not given."""
    lib = load_library()
    io = _io_dtype(cfg)
    T = _check_qkv(cfg, q, k, v, io)
    if n_tok < 1 or T % n_tok:
        raise ValueError(f"{T} token rows are not a whole number of {n_tok}-token drafts")
    B = T // n_tok
    if out is None:
        out = torch.empty((T, cfg.n_v_heads, cfg.d_v), dtype=io, device=q.device)
    C = _check_common(cfg, T, io, alpha, beta, gate, conv_w, norm_w, out)
    _expect(state, (B, cfg.n_v_heads, cfg.d_k, cfg.d_v), torch.float32, "state")
    _expect(conv_state, (B, 3, C), io, "conv_state", optional=not (cfg.flags & GDN_CONV))
    need = gdn_verify_log_bytes(cfg, B, n_tok)
    if log is None:
        log = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if log.dtype != torch.uint8 or log.numel() < need:
        raise ValueError(f"log needs {need} uint8 elements")
    st = lib.gdn_verify(ctypes.byref(cfg), B, n_tok, _ptr(q), _ptr(k), _ptr(v),
                        _row_stride(q, cfg.n_qk_heads * cfg.d_k), _row_stride(k, cfg.n_qk_heads * cfg.d_k),
                        _row_stride(v, cfg.n_v_heads * cfg.d_v), _ptr(alpha), _ptr(beta), _ptr(gate),
                        _ptr(conv_w), _ptr(norm_w), _ptr(conv_state), _ptr(state), _ptr(out),
                        _ptr(log), log.numel(), _stream(stream))
    _check(st)
    return out, log


def gdn_commit(cfg: gdn_cfg, n_tok: int, n_accept, log, conv_state, state, stream=None) -> None:
    """Advances ``state`` and ``conv_state`` in place by the first ``n_accept[b]`` drafts of the
    verify that filled ``log`` (``n_accept``: int32 [B] on the GPU)."""
    lib = load_library()
    io = _io_dtype(cfg)
    B = int(n_accept.numel())
    C = 2 * cfg.n_qk_heads * cfg.d_k + cfg.n_v_heads * cfg.d_v
    _expect(n_accept, (B,), torch.int32, "n_accept")
    _expect(state, (B, cfg.n_v_heads, cfg.d_k, cfg.d_v), torch.float32, "state")
    _expect(conv_state, (B, 3, C), io, "conv_state", optional=not (cfg.flags & GDN_CONV))
    if log.dtype != torch.uint8:
        raise ValueError("log must be the uint8 buffer gdn_verify filled")
    st = lib.gdn_commit(ctypes.byref(cfg), B, n_tok, _ptr(n_accept), _ptr(log), log.numel(), _ptr(conv_state),
                        _ptr(state), _stream(stream))
    _check(st)


def gdn_proj_workspace() -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().gdn_proj_workspace(ctypes.byref(n)))
    return int(n.value)


def _proj_ws(workspace, device):
    need = gdn_proj_workspace()
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    if workspace.dtype != torch.uint8 or workspace.numel() < need:
        raise ValueError(f"workspace needs {need} uint8 elements")
    return workspace


def gdn_in_proj(cfg: gdn_cfg, x, w_qkv, w_z, w_ab, a_log, dt_bias, qkv=None, z=None, alpha=None, beta=None,
                workspace=None, stream=None):
    """Input projection of x [T, hidden] (bf16; rows may be strided): returns (qkv [T, C_tot],
    z [T, HV, d_v], alpha [T, HV], beta [T, HV]), allocating outputs that are not given."""
    lib = load_library()
    if x.dim() != 2 or x.stride(1) != 1 or x.dtype != torch.bfloat16:
        raise ValueError("x must be a bf16 [T, hidden] matrix with contiguous rows")
    T, H = int(x.shape[0]), int(x.shape[1])
    hv, dv = cfg.n_v_heads, cfg.d_v
    C = 2 * cfg.n_qk_heads * cfg.d_k + hv * dv
    _expect(w_qkv, (C, H), torch.bfloat16, "w_qkv")
    _expect(w_z, (hv * dv, H), torch.bfloat16, "w_z")
    _expect(w_ab, (2 * hv, H), torch.bfloat16, "w_ab")
    _expect(a_log, (hv,), torch.float32, "a_log")
    _expect(dt_bias, (hv,), torch.float32, "dt_bias")
    dev = x.device
    qkv = torch.empty((T, C), dtype=torch.bfloat16, device=dev) if qkv is None else qkv
    z = torch.empty((T, hv, dv), dtype=torch.bfloat16, device=dev) if z is None else z
    alpha = torch.empty((T, hv), dtype=torch.float32, device=dev) if alpha is None else alpha
    beta = torch.empty((T, hv), dtype=torch.float32, device=dev) if beta is None else beta
    _expect(qkv, (T, C), torch.bfloat16, "qkv")
    _expect(z, (T, hv, dv), torch.bfloat16, "z")
    _expect(alpha, (T, hv), torch.float32, "alpha")
    _expect(beta, (T, hv), torch.float32, "beta")
    workspace = _proj_ws(workspace, dev)
    st = lib.gdn_in_proj(ctypes.byref(cfg), H, T, _ptr(x), x.stride(0) if T > 0 else H, _ptr(w_qkv), _ptr(w_z),
                         _ptr(w_ab), _ptr(a_log), _ptr(dt_bias), _ptr(qkv), _ptr(z), _ptr(alpha), _ptr(beta),
                         _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st)
    return qkv, z, alpha, beta


def qkv_views(cfg: gdn_cfg, qkv):
    """q, k, v as [T, heads, dim] views of a [T, C_tot] input-projection output."""
    T = qkv.shape[0]
    qc = cfg.n_qk_heads * cfg.d_k
    return (qkv[:, :qc].view(T, cfg.n_qk_heads, cfg.d_k), qkv[:, qc:2 * qc].view(T, cfg.n_qk_heads, cfg.d_k),
            qkv[:, 2 * qc:].view(T, cfg.n_v_heads, cfg.d_v))


def gdn_out_proj(cfg: gdn_cfg, o, w_out, y=None, workspace=None, stream=None) -> torch.Tensor:
    """Output projection of the mixer output o [T, HV, d_v] (or [T, HV*d_v]); returns y [T, hidden]."""
    lib = load_library()
    T = int(o.shape[0])
    vz = cfg.n_v_heads * cfg.d_v
    o2 = o.reshape(T, vz)
    _expect(o2, (T, vz), torch.bfloat16, "o")
    if w_out.dim() != 2 or w_out.shape[1] != vz:
        raise ValueError(f"w_out: expected (hidden, {vz})")
    H = int(w_out.shape[0])
    _expect(w_out, (H, vz), torch.bfloat16, "w_out")
    y = torch.empty((T, H), dtype=torch.bfloat16, device=o.device) if y is None else y
    _expect(y, (T, H), torch.bfloat16, "y")
    workspace = _proj_ws(workspace, o.device)
    _check(lib.gdn_out_proj(ctypes.byref(cfg), H, T, _ptr(o2), _ptr(w_out), _ptr(y), _ptr(workspace),
                            workspace.numel(), _stream(stream)))
    return y


def _declare_bwd(lib):
    if getattr(lib, "_bwd_declared", False):
        return
    C = ctypes.POINTER(gdn_cfg)
    lib.gdn_recurrence_backward_workspace.argtypes = [C, ctypes.c_int32, _I64, ctypes.POINTER(ctypes.c_size_t)]
    lib.gdn_recurrence_backward.argtypes = [C, ctypes.c_int32, _I64] + [_P] * 16 + [ctypes.c_size_t, _P]
    lib.gdn_recurrence_backward_workspace.restype = ctypes.c_int
    lib.gdn_recurrence_backward.restype = ctypes.c_int
    lib.gdn_backward_workspace.argtypes = [C, ctypes.c_int32, _I64, ctypes.POINTER(ctypes.c_size_t)]
    lib.gdn_backward.argtypes = [C, ctypes.c_int32, _I64] + [_P] * 24 + [ctypes.c_size_t, _P]
    lib.gdn_backward_workspace.restype = ctypes.c_int
    lib.gdn_backward.restype = ctypes.c_int
    lib._bwd_declared = True


def gdn_recurrence_backward_workspace(cfg: gdn_cfg, n_seqs: int, total_tokens: int) -> int:
    lib = load_library()
    _declare_bwd(lib)
    n = ctypes.c_size_t()
    _check(lib.gdn_recurrence_backward_workspace(ctypes.byref(cfg), n_seqs, total_tokens, ctypes.byref(n)))
    return n.value


def gdn_recurrence_backward(cfg: gdn_cfg, cu_seqlens, q, k, v, alpha, beta, dy, state_in=None, dstate_out=None,
                            want_dstate_in: bool = True, workspace=None, stream=None):
    """Derivatives of the recurrence (fp32, d = 128): returns (dq, dk, dv, dalpha, dbeta, dstate_in or None)."""
    lib = load_library()
    _declare_bwd(lib)
    n = int(cu_seqlens.numel()) - 1
    T = int(q.shape[0])
    hk, hv, d = cfg.n_qk_heads, cfg.n_v_heads, cfg.d_k
    f = torch.float32
    _expect(cu_seqlens, (n + 1,), torch.int32, "cu_seqlens")
    for t, shape, name in ((q, (T, hk, d), "q"), (k, (T, hk, d), "k"), (v, (T, hv, d), "v"), (alpha, (T, hv), "alpha"),
                           (beta, (T, hv), "beta"), (dy, (T, hv, d), "dy")):
        _expect(t, shape, f, name)
    _expect(state_in, (n, hv, d, d), f, "state_in", optional=True)
    _expect(dstate_out, (n, hv, d, d), f, "dstate_out", optional=True)
    dev = q.device
    dq, dk = torch.empty((T, hk, d), dtype=f, device=dev), torch.empty((T, hk, d), dtype=f, device=dev)
    dv = torch.empty((T, hv, d), dtype=f, device=dev)
    da, db = torch.empty((T, hv), dtype=f, device=dev), torch.empty((T, hv), dtype=f, device=dev)
    ds0 = torch.empty((n, hv, d, d), dtype=f, device=dev) if want_dstate_in else None
    if workspace is None:
        workspace = torch.empty(max(gdn_recurrence_backward_workspace(cfg, n, T), 1), dtype=torch.uint8, device=dev)
    _check(lib.gdn_recurrence_backward(ctypes.byref(cfg), n, T, _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v),
                                       _ptr(alpha), _ptr(beta), _ptr(state_in), _ptr(dy), _ptr(dstate_out),
                                       _ptr(dq), _ptr(dk), _ptr(dv), _ptr(da), _ptr(db), _ptr(ds0),
                                       _ptr(workspace), workspace.numel(), _stream(stream)))
    return dq, dk, dv, da, db, ds0


def gdn_backward_workspace(cfg: gdn_cfg, n_seqs: int, total_tokens: int) -> int:
    lib = load_library()
    _declare_bwd(lib)
    n = ctypes.c_size_t()
    _check(lib.gdn_backward_workspace(ctypes.byref(cfg), n_seqs, total_tokens, ctypes.byref(n)))
    return n.value


def gdn_backward(cfg: gdn_cfg, cu_seqlens, q, k, v, alpha, beta, gate, conv_w, norm_w, dout, state_in=None,
                 conv_in=None, dstate_out=None, want_dstate_in=True, want_dconv_in=True, workspace=None,
                 stream=None) -> dict:
    """Derivatives of the whole mixer (fp32, d = 128, every step on) for every input of gdn_prefill; returns a
    dict keyed like the inputs (q, k, v, alpha, beta, gate, conv_w, norm_w, state_in, conv_in)."""
    lib = load_library()
    _declare_bwd(lib)
    n = int(cu_seqlens.numel()) - 1
    T = int(q.shape[0])
    hk, hv, d = cfg.n_qk_heads, cfg.n_v_heads, cfg.d_k
    C = 2 * hk * d + hv * d
    f = torch.float32
    _expect(cu_seqlens, (n + 1,), torch.int32, "cu_seqlens")
    for t, shape, name in ((q, (T, hk, d), "q"), (k, (T, hk, d), "k"), (v, (T, hv, d), "v"), (alpha, (T, hv), "alpha"),
                           (beta, (T, hv), "beta"), (gate, (T, hv, d), "gate"), (conv_w, (C, 4), "conv_w"),
                           (norm_w, (d,), "norm_w"), (dout, (T, hv, d), "dout")):
        _expect(t, shape, f, name)
    _expect(state_in, (n, hv, d, d), f, "state_in", optional=True)
    _expect(conv_in, (n, 3, C), f, "conv_in", optional=True)
    _expect(dstate_out, (n, hv, d, d), f, "dstate_out", optional=True)
    dev = q.device
    e = lambda *shape: torch.empty(shape, dtype=f, device=dev)
    out = {"q": e(T, hk, d), "k": e(T, hk, d), "v": e(T, hv, d), "alpha": e(T, hv), "beta": e(T, hv),
           "gate": e(T, hv, d), "conv_w": e(C, 4), "norm_w": e(d),
           "state_in": e(n, hv, d, d) if want_dstate_in else None, "conv_in": e(n, 3, C) if want_dconv_in else None}
    if workspace is None:
        workspace = torch.empty(max(gdn_backward_workspace(cfg, n, T), 1), dtype=torch.uint8, device=dev)
    _check(lib.gdn_backward(ctypes.byref(cfg), n, T, _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                            _ptr(beta), _ptr(gate), _ptr(conv_w), _ptr(norm_w), _ptr(state_in), _ptr(conv_in),
                            _ptr(dout), _ptr(dstate_out), _ptr(out["q"]), _ptr(out["k"]), _ptr(out["v"]),
                            _ptr(out["alpha"]), _ptr(out["beta"]), _ptr(out["gate"]), _ptr(out["conv_w"]),
                            _ptr(out["norm_w"]), _ptr(out["state_in"]), _ptr(out["conv_in"]), _ptr(workspace),
                            workspace.numel(), _stream(stream)))
    return out


def cfg_for(n_qk_heads: int, n_v_heads: int, d_k: int, d_v: int, dtype: torch.dtype,
            flags: int = GDN_ALL, **kw) -> gdn_cfg:
    """Configuration for a shape and io dtype."""
    io = GDN_BF16 if dtype == torch.bfloat16 else GDN_F32
    return gdn_cfg_default(n_qk_heads=n_qk_heads, n_v_heads=n_v_heads, d_k=d_k, d_v=d_v, io_dtype=io,
                           flags=flags, **kw)
