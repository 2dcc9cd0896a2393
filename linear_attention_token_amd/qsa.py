"""Thin ctypes binding of the QSA indexer entry points of libgdn.so (include/qsa.h), same names.

Argument marshalling only: tensors become device pointers and strides, outputs and workspaces are
allocated with torch, and every step (compression, scores, selection) runs in the library's HIP
kernels. Without the built library or a GPU these functions raise.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import gdn as _g

EXPORTS = ("qsa_cfg_default", "qsa_compress", "qsa_workspace", "qsa_select", "qsa_decode")
D = 128          # head dim of the indexer queries and keys
HEADS = 4        # indexer query heads
BLOCK = 4        # keys per micro-block


class qsa_cfg(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("d", ctypes.c_int32), ("block", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("rope_dims", ctypes.c_int32), ("io_dtype", ctypes.c_int32),
                ("rope_base", ctypes.c_float), ("norm_eps", ctypes.c_float)]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_declared = False


def _lib():
    global _declared
    lib = _g.load_library()
    if not _declared:
        C = ctypes.POINTER(qsa_cfg)
        lib.qsa_cfg_default.argtypes = [C]
        lib.qsa_cfg_default.restype = None
        lib.qsa_compress.argtypes = [C, _I32, _I64, _P, _P, _P, _I64, _P, _P, _I64, _P, _P]
        lib.qsa_workspace.argtypes = [C, _I64, _I64, ctypes.POINTER(ctypes.c_size_t)]
        lib.qsa_select.argtypes = [C, _I32, _I64, _P, _P, _I64, _P, _I64, _P, _P, _P, _P, ctypes.c_size_t, _P]
        lib.qsa_decode.argtypes = [C, _I32, _P, _P, _I64, _P, _I64, _P, _P, _P, _I64, _P, _P, _P, _P,
                                   ctypes.c_size_t, _P]
        for f in ("qsa_compress", "qsa_workspace", "qsa_select", "qsa_decode"):
            getattr(lib, f).restype = ctypes.c_int
        _declared = True
    return lib


def qsa_cfg_default(**overrides) -> qsa_cfg:
    """The library's defaults (4 heads of 128, blocks of 4, top 512, 64 rotated dims, bf16)."""
    c = qsa_cfg()
    _lib().qsa_cfg_default(ctypes.byref(c))
    for k, v in overrides.items():
        setattr(c, k, v)
    return c


def cfg_for(dtype: torch.dtype, **kw) -> qsa_cfg:
    return qsa_cfg_default(io_dtype=_g.GDN_BF16 if dtype == torch.bfloat16 else _g.GDN_F32, **kw)


def _io(cfg):
    return torch.bfloat16 if cfg.io_dtype == _g.GDN_BF16 else torch.float32


def qsa_workspace(cfg: qsa_cfg, rows: int, cap_blocks: int) -> int:
    n = ctypes.c_size_t()
    _g._check(_lib().qsa_workspace(ctypes.byref(cfg), rows, cap_blocks, ctypes.byref(n)))
    return n.value


def _ws(cfg, rows, cap, workspace, device):
    if workspace is None:
        workspace = torch.empty(max(qsa_workspace(cfg, rows, cap), 1), dtype=torch.uint8, device=device)
    return workspace


def _rows2(t, width, name, io):
    """A [rows, width] (or [rows, ..., ] whose trailing dims flatten to width) view with unit inner stride."""
    t2 = t.reshape(t.shape[0], -1) if t.dim() != 2 else t
    if t2.shape[1] != width or t2.dtype != io or (t2.shape[0] > 0 and t2.stride(1) != 1):
        raise ValueError(f"{name}: expected rows of {width} contiguous {io}, got {tuple(t.shape)} {t.dtype}")
    return t2, (t2.stride(0) if t2.shape[0] > 0 else width)


def qsa_compress(cfg: qsa_cfg, cu_seqlens: torch.Tensor, k, norm_w, kbar, pending=None,
                 cu_seqlens_host=None, stream=None) -> None:
    """Compressed keys of the packed sequences into kbar [n_seqs, cap, 128] (and the tail keys into
    pending [n_seqs, 3, 128] when given). k is [T, 128]."""
    lib = _lib()
    io = _io(cfg)
    n_seqs = int(cu_seqlens.numel()) - 1
    k2, ld_k = _rows2(k, D, "k", io)
    T = int(k2.shape[0])
    if kbar.dim() != 3 or kbar.shape[0] != n_seqs or kbar.shape[2] != D:
        raise ValueError(f"kbar: expected ({n_seqs}, cap, {D})")
    _g._expect(kbar, tuple(kbar.shape), io, "kbar")
    _g._expect(norm_w, (D,), torch.float32, "norm_w")
    _g._expect(pending, (n_seqs, 3, D), io, "pending", optional=True)
    _g._expect(cu_seqlens, (n_seqs + 1,), torch.int32, "cu_seqlens")
    host = None
    if cu_seqlens_host is not None:
        host = torch.as_tensor(cu_seqlens_host, dtype=torch.int32).cpu().contiguous()
    _g._check(lib.qsa_compress(ctypes.byref(cfg), n_seqs, T, _g._ptr(cu_seqlens),
                               host.data_ptr() if host is not None else None, _g._ptr(k2), ld_k,
                               _g._ptr(norm_w), _g._ptr(kbar), int(kbar.shape[1]), _g._ptr(pending),
                               _g._stream(stream)))


def _outs(cfg, rows, device, sel, n_sel, tail):
    sel = torch.empty((rows, cfg.topk), dtype=torch.int32, device=device) if sel is None else sel
    n_sel = torch.empty((rows,), dtype=torch.int32, device=device) if n_sel is None else n_sel
    tail = torch.empty((rows,), dtype=torch.int32, device=device) if tail is None else tail
    _g._expect(sel, (rows, cfg.topk), torch.int32, "sel")
    _g._expect(n_sel, (rows,), torch.int32, "n_sel")
    _g._expect(tail, (rows,), torch.int32, "tail")
    return sel, n_sel, tail


def qsa_select(cfg: qsa_cfg, cu_seqlens: torch.Tensor, q, kbar, sel=None, n_sel=None, tail=None,
               workspace=None, stream=None):
    """Top-k blocks of every token of a packed prefill. q is [T, 4, 128] (or [T, 512]); returns
    (sel [T, topk], n_sel [T], tail [T])."""
    lib = _lib()
    io = _io(cfg)
    n_seqs = int(cu_seqlens.numel()) - 1
    q2, ld_q = _rows2(q, HEADS * D, "q", io)
    T = int(q2.shape[0])
    if kbar.dim() != 3 or kbar.shape[0] != n_seqs or kbar.shape[2] != D:
        raise ValueError(f"kbar: expected ({n_seqs}, cap, {D})")
    _g._expect(kbar, tuple(kbar.shape), io, "kbar")
    _g._expect(cu_seqlens, (n_seqs + 1,), torch.int32, "cu_seqlens")
    cap = int(kbar.shape[1])
    sel, n_sel, tail = _outs(cfg, T, q.device, sel, n_sel, tail)
    workspace = _ws(cfg, T, cap, workspace, q.device)
    _g._check(lib.qsa_select(ctypes.byref(cfg), n_seqs, T, _g._ptr(cu_seqlens), _g._ptr(q2), ld_q, _g._ptr(kbar),
                             cap, _g._ptr(sel), _g._ptr(n_sel), _g._ptr(tail), _g._ptr(workspace),
                             workspace.numel(), _g._stream(stream)))
    return sel, n_sel, tail


def qsa_decode(cfg: qsa_cfg, n_tok: torch.Tensor, q, k, norm_w, pending, kbar, sel=None, n_sel=None,
               tail=None, workspace=None, stream=None):
    """One decode step: k [B, 128] joins each sequence's pending block (compressed into kbar
    [B, cap, 128] when it completes one), then q [B, 4, 128] selects. Returns (sel, n_sel, tail)."""
    lib = _lib()
    io = _io(cfg)
    B = int(n_tok.numel())
    q2, ld_q = _rows2(q, HEADS * D, "q", io)
    k2, ld_k = _rows2(k, D, "k", io)
    if q2.shape[0] != B or k2.shape[0] != B:
        raise ValueError("q, k and n_tok must have one row per sequence")
    _g._expect(n_tok, (B,), torch.int32, "n_tok")
    _g._expect(norm_w, (D,), torch.float32, "norm_w")
    _g._expect(pending, (B, 3, D), io, "pending")
    if kbar.dim() != 3 or kbar.shape[0] != B or kbar.shape[2] != D:
        raise ValueError(f"kbar: expected ({B}, cap, {D})")
    _g._expect(kbar, tuple(kbar.shape), io, "kbar")
    cap = int(kbar.shape[1])
    sel, n_sel, tail = _outs(cfg, B, q.device, sel, n_sel, tail)
    workspace = _ws(cfg, B, cap, workspace, q.device)
    _g._check(lib.qsa_decode(ctypes.byref(cfg), B, _g._ptr(n_tok), _g._ptr(q2), ld_q, _g._ptr(k2), ld_k,
                             _g._ptr(norm_w), _g._ptr(pending), _g._ptr(kbar), cap, _g._ptr(sel), _g._ptr(n_sel),
                             _g._ptr(tail), _g._ptr(workspace), workspace.numel(), _g._stream(stream)))
    return sel, n_sel, tail
