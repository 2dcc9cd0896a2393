"""Host-only tests of the C ABI: the library loads without a GPU, exports every function the header
declares, sizes workspaces, and rejects bad arguments before any HIP call (so these run on CPU).
Every gdn_prefill / gdn_decode_step call here is invalid on purpose and must return early."""
import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("gdn.h", "qsa.h")]

gdn = pytest.importorskip("linear_attention_token_amd.gdn")
qsa = pytest.importorskip("linear_attention_token_amd.qsa")

if not os.path.exists(gdn.LIB_PATH):
    pytest.skip("libgdn.so not built (run __graft_entry__.build())", allow_module_level=True)

lib = gdn.load_library()
A = 0x100000           # a fake, 16-byte aligned "device" address; never dereferenced
T_, N_ = 128, 1


def header_functions():
    funcs = set()
    for h in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))):
        txt = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        funcs |= set(re.findall(r"\b((?:gdn|qsa)_[a-z_0-9]+)\s*\(", txt))
    return sorted(funcs)


def test_exports_every_declared_function():
    funcs = header_functions()
    assert set(funcs) == set(gdn.EXPORTS) | set(qsa.EXPORTS)
    for f in funcs:
        assert hasattr(lib, f), f"libgdn.so does not export {f}"


def header_arity():
    """Parameter count of every function the headers declare."""
    arity = {}
    for h in HEADERS:
        txt = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        for name, params in re.findall(r"\b((?:gdn|qsa)_[a-z_0-9]+)\s*\(([^;{]*?)\)\s*;", txt, flags=re.S):
            ps = [p for p in params.split(",") if p.strip() and p.strip() != "void"]
            arity[name] = len(ps)
    return arity


def test_bindings_declare_every_argument():
    """Each ctypes declaration lists exactly the header's parameters: an argument missing from argtypes
    would still be passed, as a C int, truncating a pointer such as the stream handle."""
    gdn._declare_bwd(lib)
    qsa._lib()
    arity = header_arity()
    assert set(arity) == set(header_functions())
    for name, n in arity.items():
        at = getattr(lib, name).argtypes
        assert at is not None and len(at) == n, (name, None if at is None else len(at), n)


def test_abi_version_and_defaults():
    assert lib.gdn_abi_version() == 1
    c = gdn.gdn_cfg_default()
    assert (c.n_qk_heads, c.n_v_heads, c.d_k, c.d_v, c.conv_width) == (16, 48, 128, 128, 4)
    assert c.io_dtype == gdn.GDN_BF16 and c.flags == gdn.GDN_ALL and c.norm_head_stride == 0
    assert abs(c.scale - 1.0) < 1e-9 and abs(c.l2_eps - 1e-6) < 1e-12 and abs(c.norm_eps - 1e-6) < 1e-12
    for s in range(9):
        assert lib.gdn_status_string(s).decode().startswith(gdn.STATUS[s])


def test_workspace_sizes():
    c = gdn.gdn_cfg_default()
    small = gdn.gdn_prefill_workspace(c, 1, 4096)
    big = gdn.gdn_prefill_workspace(c, 1, 8192)
    assert 0 < small < big
    # chunk bound floor(T/64) + N: the chunked path holds at least U, Wk, chunk states and W
    nc = 4096 // 64 + 1
    assert small >= nc * 48 * (2 * 64 * 128 * 2 + 128 * 128 * 2 + 128 * 64 * 2)
    # more sequences for the same tokens can only need more chunks
    assert gdn.gdn_prefill_workspace(c, 32, 4096) >= small
    f = gdn.gdn_cfg_default(io_dtype=gdn.GDN_F32, n_qk_heads=1, n_v_heads=1, d_k=16, d_v=16)
    assert gdn.gdn_prefill_workspace(f, 1, 64) >= 3 * 64 * 16 * 4
    assert gdn.gdn_prefill_workspace(c, 0, 0) >= 0


def test_oversized_calls_are_refused():
    # grids of the chunked kernels would pass 2^32 work-items: refused up front, before any launch
    c = gdn.gdn_cfg_default()
    nbytes = ctypes.c_size_t(0)
    _err(lib.gdn_prefill_workspace(ctypes.byref(c), 1, 1 << 30, ctypes.byref(nbytes)), 6)
    _err(_prefill(c, n_seqs=1, T=1 << 30), 6)
    assert gdn.gdn_prefill_workspace(c, 1, 1 << 24) > 0  # 16M tokens still fit


def _prefill(cfg, n_seqs=N_, T=T_, cu=A, cu_host=None, q=A, k=A, v=A, ld_q=2048, ld_k=2048, ld_v=6144,
             alpha=A, beta=A, gate=A, conv_w=A, norm_w=A, state_in=None, state_out=None, conv_in=None,
             conv_out=None, out=A, ws=A, ws_bytes=1 << 40):
    ch = None
    if cu_host is not None:
        ch = (ctypes.c_int32 * len(cu_host))(*cu_host)
    return lib.gdn_prefill(ctypes.byref(cfg), n_seqs, T, cu, ch, q, k, v, ld_q, ld_k, ld_v, alpha, beta,
                           gate, conv_w, norm_w, state_in, state_out, conv_in, conv_out, out, ws, ws_bytes,
                           None)


def _err(st, code):
    assert st == code, (gdn.STATUS.get(st), lib.gdn_last_error().decode())
    assert len(lib.gdn_last_error()) > 0


def test_prefill_rejects_bad_config():
    _err(lib.gdn_prefill(None, 1, 128, A, None, A, A, A, 2048, 2048, 6144, A, A, A, A, A, None, None,
                         None, None, A, A, 1 << 40, None), 1)
    _err(_prefill(gdn.gdn_cfg_default(n_v_heads=47)), 2)              # HV % HK != 0
    _err(_prefill(gdn.gdn_cfg_default(d_k=48)), 6)                    # unsupported dim
    _err(_prefill(gdn.gdn_cfg_default(d_v=256)), 6)
    _err(_prefill(gdn.gdn_cfg_default(conv_width=3)), 6)
    _err(_prefill(gdn.gdn_cfg_default(io_dtype=7)), 3)
    _err(_prefill(gdn.gdn_cfg_default(flags=16)), 8)
    _err(_prefill(gdn.gdn_cfg_default(l2_eps=-1.0)), 8)
    _err(_prefill(gdn.gdn_cfg_default(norm_eps=float("nan"))), 8)
    _err(_prefill(gdn.gdn_cfg_default(norm_head_stride=7)), 2)
    _err(_prefill(gdn.gdn_cfg_default(n_qk_heads=0)), 2)


def test_prefill_rejects_bad_arguments():
    c = gdn.gdn_cfg_default()
    _err(_prefill(c, n_seqs=-1), 2)
    _err(_prefill(c, n_seqs=0, T=5), 2)
    _err(_prefill(c, cu=None), 1)
    _err(_prefill(c, q=None), 1)
    _err(_prefill(c, alpha=None), 1)
    _err(_prefill(c, out=None), 1)
    _err(_prefill(c, gate=None), 1)                                   # GDN_GATE needs gate
    _err(_prefill(c, norm_w=None), 1)                                 # GDN_NORM needs norm_w
    _err(_prefill(c, conv_w=None), 1)                                 # GDN_CONV needs conv_w
    _err(_prefill(c, ld_q=1024), 2)                                   # stride below a token row
    _err(_prefill(c, ld_v=6148), 4)                                   # stride not 16-byte
    _err(_prefill(c, q=A + 2), 4)                                     # misaligned pointer
    _err(_prefill(c, state_out=A + 4), 4)
    _err(_prefill(c, ws=None, ws_bytes=0), 5)
    need = gdn.gdn_prefill_workspace(c, N_, T_)
    _err(_prefill(c, ws_bytes=need - 1), 5)
    _err(_prefill(c, ws=A + 16), 4)                                   # workspace 256-byte aligned
    _err(_prefill(c, cu_host=[1, T_]), 2)                             # cu[0] != 0
    _err(_prefill(c, n_seqs=2, cu_host=[0, 100, 90]), 2)              # decreasing
    _err(_prefill(c, cu_host=[0, T_ - 1]), 2)                         # cu[N] != T
    _err(_prefill(c, conv_in=A, conv_out=A + 256), 8)                 # partial overlap


def _prefill_static(cfg, n_seqs=N_, T=T_, cu=A, q=A, k=A, v=A, ld_q=2048, ld_k=2048, ld_v=6144, alpha=A,
                    beta=A, gate=A, conv_w=A, norm_w=A, out=A):
    return lib.gdn_prefill_static(ctypes.byref(cfg), n_seqs, T, cu, None, q, k, v, ld_q, ld_k, ld_v, alpha, beta,
                                  gate, conv_w, norm_w, None, None, None, None, out, None)


def test_static_prefill_validates_before_any_hip_call():
    """The allocation-free prefill refuses, with no HIP call (no GPU here), a problem whose workspace
    exceeds its static scratch, and every argument gdn_prefill refuses."""
    c = gdn.gdn_cfg_default()
    assert gdn.gdn_prefill_workspace(c, 1, 4096) > gdn.GDN_STATIC_WORKSPACE_BYTES
    _err(_prefill_static(c, T=4096), 5)
    assert "static scratch" in lib.gdn_last_error().decode()
    assert gdn.gdn_prefill_workspace(c, 1, 1024) <= gdn.GDN_STATIC_WORKSPACE_BYTES
    _err(_prefill_static(gdn.gdn_cfg_default(n_v_heads=47)), 2)
    _err(_prefill_static(c, q=None), 1)
    _err(_prefill_static(c, ld_v=6148), 4)
    _err(_prefill_static(c, out=A + 2), 4)
    _err(_prefill_static(c, n_seqs=0, T=5), 2)
    with open(HEADERS[0]) as f:
        m = re.search(r"#define GDN_STATIC_WORKSPACE_BYTES \(\(size_t\)(\d+) << (\d+)\)", f.read())
    assert m and int(m.group(1)) << int(m.group(2)) == gdn.GDN_STATIC_WORKSPACE_BYTES


def test_flags_relax_required_pointers():
    """With GATE/NORM/CONV off those tensors may be NULL; the call then fails only on what is
    still wrong (here: a workspace that is too small), proving the NULLs were accepted."""
    c = gdn.gdn_cfg_default(flags=gdn.GDN_L2QK)
    _err(_prefill(c, gate=None, norm_w=None, conv_w=None, ws_bytes=16), 5)


def _decode(cfg, B=4, q=A, k=A, v=A, alpha=A, beta=A, gate=A, conv_w=A, norm_w=A, conv_state=A,
            state=A, out=A, ld=(2048, 2048, 6144)):
    return lib.gdn_decode_step(ctypes.byref(cfg), B, q, k, v, ld[0], ld[1], ld[2], alpha, beta, gate,
                               conv_w, norm_w, conv_state, state, out, None)


def test_decode_rejects_bad_arguments():
    c = gdn.gdn_cfg_default()
    _err(_decode(c, B=-1), 2)
    _err(_decode(c, state=None), 1)
    _err(_decode(c, conv_state=None), 1)
    _err(_decode(c, gate=None), 1)
    _err(_decode(c, out=None), 1)
    _err(_decode(c, state=A + 8), 4)
    _err(_decode(c, ld=(2048, 2000, 6144)), 2)
    _err(_decode(gdn.gdn_cfg_default(d_k=100)), 6)
    _err(_decode(gdn.gdn_cfg_default(n_v_heads=40)), 2)


def test_verify_log_sizes():
    c = gdn.gdn_cfg_default()
    n = gdn.gdn_verify_log_bytes(c, 256, 4)
    # per token: k^ of 16 QK heads and e of 48 value heads in fp32, alpha/beta, raw inputs (bf16)
    rows = 256 * 4
    assert n >= rows * (16 * 128 * 4 + 48 * 128 * 4 + 48 * 8 + 10240 * 2)
    assert n < rows * (16 * 128 * 4 + 48 * 128 * 4 + 48 * 8 + 10240 * 2) + 4 * 256
    assert gdn.gdn_verify_log_bytes(c, 256, 5) > n
    assert gdn.gdn_verify_log_bytes(c, 0, 4) == 0


def _verify(cfg, B=4, K=4, q=A, k=A, v=A, alpha=A, beta=A, gate=A, conv_w=A, norm_w=A, conv_state=A,
            state=A, out=A, log=A, log_bytes=1 << 40, ld=(2048, 2048, 6144)):
    return lib.gdn_verify(ctypes.byref(cfg), B, K, q, k, v, ld[0], ld[1], ld[2], alpha, beta, gate, conv_w,
                          norm_w, conv_state, state, out, log, log_bytes, None)


def _commit(cfg, B=4, K=4, n_accept=A, log=A, log_bytes=1 << 40, conv_state=A, state=A):
    return lib.gdn_commit(ctypes.byref(cfg), B, K, n_accept, log, log_bytes, conv_state, state, None)


def test_verify_and_commit_reject_bad_arguments():
    c = gdn.gdn_cfg_default()
    nbytes = ctypes.c_size_t(0)
    _err(lib.gdn_verify_log_bytes(ctypes.byref(c), 4, 0, ctypes.byref(nbytes)), 2)
    _err(lib.gdn_verify_log_bytes(ctypes.byref(c), 4, 9, ctypes.byref(nbytes)), 6)
    _err(lib.gdn_verify_log_bytes(ctypes.byref(c), 4, 4, None), 1)
    for call in (_verify, _commit):
        _err(call(c, B=-1), 2)
        _err(call(c, K=0), 2)
        _err(call(c, K=9), 6)
        _err(call(gdn.gdn_cfg_default(d_k=64, d_v=64)), 6)        # only d = 128
        _err(call(gdn.gdn_cfg_default(n_qk_heads=8, n_v_heads=48)), 6)  # HV/HK = 6 > 4
        _err(call(c, log=None), 1)
        _err(call(c, log=A + 128), 4)                              # log 256-byte aligned
        _err(call(c, log_bytes=1024), 5)
        _err(call(c, state=None), 1)
        _err(call(c, state=A + 8), 4)
        _err(call(c, conv_state=None), 1)
    _err(_verify(c, out=None), 1)
    _err(_verify(c, gate=None), 1)
    _err(_verify(c, ld=(2048, 2000, 6144)), 2)
    _err(_commit(c, n_accept=None), 1)
    _err(_commit(c, n_accept=A + 2), 4)
    # with the conv off the conv cache may be absent; an empty batch does nothing
    off = gdn.gdn_cfg_default(flags=gdn.GDN_L2QK | gdn.GDN_NORM | gdn.GDN_GATE)
    assert _verify(off, B=0, conv_state=None) == 0
    assert _commit(off, B=0, conv_state=None) == 0


def test_projections_reject_bad_arguments():
    c = gdn.gdn_cfg_default()
    n = ctypes.c_size_t(0)
    n.value = 7
    assert lib.gdn_proj_workspace(ctypes.byref(n)) == 0 and n.value == 0   # the kernels need no scratch
    _err(lib.gdn_proj_workspace(None), 1)

    def inp(cfg=c, H=2560, T=64, x=A, ld=2560, wq=A, wz=A, wab=A, al=A, dt=A, qkv=A, z=A, alpha=A, beta=A,
            ws=A, wsb=1 << 30):
        return lib.gdn_in_proj(ctypes.byref(cfg), H, T, x, ld, wq, wz, wab, al, dt, qkv, z, alpha, beta, ws, wsb, None)

    def outp(cfg=c, H=2560, T=64, o=A, w=A, y=A, ws=A, wsb=1 << 30):
        return lib.gdn_out_proj(ctypes.byref(cfg), H, T, o, w, y, ws, wsb, None)

    for call in (inp, outp):
        _err(call(cfg=gdn.gdn_cfg_default(io_dtype=gdn.GDN_F32)), 6)
        _err(call(H=100), 2)                     # hidden % 32
        _err(call(T=-1), 2)
        _err(call(ws=None, wsb=0, T=-1), 2)      # no workspace is needed; the next problem is reported
    _err(inp(x=None), 1)
    _err(inp(beta=None), 1)
    _err(inp(ld=2000), 2)
    _err(inp(ld=2564), 2)                        # rows must stay 16-byte aligned
    _err(inp(qkv=A + 8), 4)
    _err(inp(alpha=A + 2), 4)
    _err(outp(o=None), 1)
    _err(outp(y=A + 8), 4)
    assert inp(T=0, x=None, qkv=None) == 0 and outp(T=0, o=None) == 0


def test_qsa_defaults_and_workspace():
    c = qsa.qsa_cfg_default()
    assert (c.n_heads, c.d, c.block, c.topk, c.rope_dims, c.io_dtype) == (4, 128, 4, 512, 64, gdn.GDN_BF16)
    assert abs(c.rope_base - 1e4) < 1e-3 and abs(c.norm_eps - 1e-6) < 1e-12
    one = qsa.qsa_workspace(c, 1, 1 << 18)
    many = qsa.qsa_workspace(c, 8, 1 << 18)
    assert one >= (1 << 18) * 4 + 2048 and many >= 8 * (1 << 18) * 4
    # 256K blocks = 16 select segments: each row also keeps 16 x 512 (key, block) candidates
    assert many >= 8 * ((1 << 18) * 4 + 16 * 512 * 8)
    assert qsa.qsa_workspace(c, 0, 0) >= 0


def test_qsa_reject_bad_arguments():
    c = qsa.qsa_cfg_default()
    cu = (ctypes.c_int32 * 3)(0, 40, 100)
    n = ctypes.c_size_t(0)
    L = qsa._lib()
    _err(L.qsa_workspace(ctypes.byref(qsa.qsa_cfg_default(n_heads=8)), 1, 16, ctypes.byref(n)), 6)
    _err(L.qsa_workspace(ctypes.byref(qsa.qsa_cfg_default(topk=0)), 1, 16, ctypes.byref(n)), 6)
    _err(L.qsa_workspace(ctypes.byref(qsa.qsa_cfg_default(rope_dims=40)), 1, 16, ctypes.byref(n)), 6)
    _err(L.qsa_workspace(ctypes.byref(qsa.qsa_cfg_default(io_dtype=5)), 1, 16, ctypes.byref(n)), 3)
    _err(L.qsa_workspace(ctypes.byref(qsa.qsa_cfg_default(norm_eps=-1.0)), 1, 16, ctypes.byref(n)), 8)
    _err(L.qsa_workspace(ctypes.byref(c), 1, 16384 * 32 + 1, ctypes.byref(n)), 6)   # beyond 2M tokens at top-512
    assert L.qsa_workspace(ctypes.byref(c), 1, 16384 * 32, ctypes.byref(n)) == 0

    def comp(cfg=c, N=2, T=100, cud=A, cuh=cu, k=A, ld=128, w=A, kb=A, cap=64, pend=A):
        return L.qsa_compress(ctypes.byref(cfg), N, T, cud, ctypes.cast(cuh, ctypes.c_void_p) if cuh else None,
                              k, ld, w, kb, cap, pend, None)

    _err(comp(cap=10), 2)            # sequence 1 has 15 blocks
    _err(comp(cuh=(ctypes.c_int32 * 3)(0, 50, 40)), 2)
    _err(comp(k=None), 1)
    _err(comp(cud=None), 1)
    _err(comp(ld=100), 2)
    _err(comp(ld=132), 4)
    _err(comp(kb=A + 8), 4)
    _err(comp(N=70000), 6)
    assert comp(N=0, T=0) == 0 and comp(T=0, cuh=(ctypes.c_int32 * 3)(0, 0, 0)) == 0

    def sel(cfg=c, N=2, T=100, cud=A, q=A, ld=512, kb=A, cap=64, s=A, ns=A, tl=A, ws=A, wsb=1 << 30):
        return L.qsa_select(ctypes.byref(cfg), N, T, cud, q, ld, kb, cap, s, ns, tl, ws, wsb, None)

    _err(sel(q=None), 1)
    _err(sel(cud=None), 1)
    _err(sel(ld=256), 2)
    _err(sel(ws=None), 5)
    _err(sel(wsb=100), 5)
    _err(sel(ws=A + 16), 4)
    _err(sel(ns=A + 2), 4)
    assert sel(T=0, q=None) == 0

    def dec(cfg=c, B=2, nt=A, q=A, ldq=512, k=A, ldk=128, w=A, pend=A, kb=A, cap=64, s=A, ns=A, tl=A, ws=A,
            wsb=1 << 30):
        return L.qsa_decode(ctypes.byref(cfg), B, nt, q, ldq, k, ldk, w, pend, kb, cap, s, ns, tl, ws, wsb, None)

    _err(dec(nt=None), 1)
    _err(dec(pend=None), 1)
    _err(dec(B=-1), 2)
    _err(dec(ldk=64), 2)
    _err(dec(wsb=64), 5)
    _err(dec(cap=-1), 2)
    assert dec(B=0, q=None, k=None) == 0


def test_recurrence_backward_rejects_bad_arguments():
    f32 = gdn.gdn_cfg_default(io_dtype=gdn.GDN_F32)
    gdn._declare_bwd(lib)
    n = ctypes.c_size_t(0)
    assert lib.gdn_recurrence_backward_workspace(ctypes.byref(f32), 1, 4096, ctypes.byref(n)) == 0
    # the state at each 64-token chunk boundary and its derivative are kept, not one state per token
    assert 2 * 65 * 48 * 128 * 128 * 4 <= n.value < 4096 * 48 * 128 * 128 * 4 // 4
    _err(lib.gdn_recurrence_backward_workspace(ctypes.byref(gdn.gdn_cfg_default()), 1, 64, ctypes.byref(n)), 6)
    _err(lib.gdn_recurrence_backward_workspace(
        ctypes.byref(gdn.gdn_cfg_default(io_dtype=gdn.GDN_F32, d_k=64, d_v=64)), 1, 64, ctypes.byref(n)), 6)

    def bwd(cfg=f32, N=1, T=64, cu=A, q=A, dy=A, dq=A, ws=A, wsb=1 << 40, da=A):
        return lib.gdn_recurrence_backward(ctypes.byref(cfg), N, T, cu, q, A, A, A, A, None, dy, None, dq, A, A, da,
                                           A, None, ws, wsb, None)

    _err(bwd(dy=None), 1)
    _err(bwd(cu=None), 1)
    _err(bwd(wsb=1024), 5)
    _err(bwd(ws=A + 16), 4)
    _err(bwd(q=A + 4), 4)
    _err(bwd(da=A + 2), 4)
    _err(bwd(N=0), 2)
    assert bwd(N=0, T=0) == 0


def test_mixer_backward_rejects_bad_arguments():
    f32 = gdn.gdn_cfg_default(io_dtype=gdn.GDN_F32)
    gdn._declare_bwd(lib)
    n = ctypes.c_size_t(0)
    assert lib.gdn_backward_workspace(ctypes.byref(f32), 1, 4096, ctypes.byref(n)) == 0
    assert 2 * 65 * 48 * 128 * 128 * 4 <= n.value < 4096 * 48 * 128 * 128 * 4 // 2
    _err(lib.gdn_backward_workspace(ctypes.byref(gdn.gdn_cfg_default(io_dtype=gdn.GDN_F32, flags=gdn.GDN_CONV)),
                                    1, 64, ctypes.byref(n)), 6)
    _err(lib.gdn_backward_workspace(ctypes.byref(gdn.gdn_cfg_default(io_dtype=gdn.GDN_F32, norm_head_stride=128)),
                                    1, 64, ctypes.byref(n)), 6)
    _err(lib.gdn_backward_workspace(ctypes.byref(gdn.gdn_cfg_default()), 1, 64, ctypes.byref(n)), 6)

    def bwd(N=1, T=64, cu=A, q=A, dout=A, dconv_w=A, ws=A, wsb=1 << 40, gate=A):
        return lib.gdn_backward(ctypes.byref(f32), N, T, cu, q, A, A, A, A, gate, A, A, None, None, dout, None,
                                A, A, A, A, A, A, dconv_w, A, None, None, ws, wsb, None)

    _err(bwd(dout=None), 1)
    _err(bwd(gate=None), 1)
    _err(bwd(dconv_w=None), 1)
    _err(bwd(wsb=4096), 5)
    _err(bwd(q=A + 8), 4)
    assert bwd(N=0, T=0) == 0
