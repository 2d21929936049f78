"""Host-side checks of the C ABI: the library loads, exports every function
the header declares, and rejects invalid arguments before any GPU work.

Nothing here launches a kernel; all calls return from host validation."""

import ctypes
import os
import re

import pytest

import block_sparse_attention_plan_amd as bsa

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(REPO, "include", "bsa.h")

OK, INVALID, UNSUPPORTED, MISALIGNED, MISMATCH, TOO_SMALL = 0, -1, -2, -3, -4, -5


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bsa.library_path()):
        pytest.fail("libbsa.so is not built (python -m block_sparse_attention_plan_amd.build)")
    return bsa.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while", "sizeof")))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("bsa_plan", "bsa_forward", "topk_sparse_attn", "bsa_plan_buffer_bytes",
              "bsa_plan_sections", "bsa_plan_nnz", "bsa_status_string", "bsa_last_error"):
        assert n in names


def test_library_exports_every_declared_function(lib):
    for n in declared_functions():
        assert hasattr(lib, n), f"libbsa.so does not export {n}"


def test_plan_buffer_sizes(lib):
    assert lib.bsa_plan_buffer_bytes(0, 4, 4) == 0
    assert lib.bsa_plan_buffer_bytes(4, -1, 4) == 0
    assert lib.bsa_plan_buffer_bytes(1 << 11, 1 << 10, 1 << 10) == 0  # 2^31 tiles
    H, Mb, Nb = 32, 256, 256
    n = lib.bsa_plan_buffer_bytes(H, Mb, Nb)
    offs = (ctypes.c_size_t * 4)()
    assert lib.bsa_plan_sections(H, Mb, Nb, offs) == OK
    o = list(offs)
    assert o[0] == 0 and all(x % 256 == 0 for x in o) and o == sorted(o)
    assert o[1] >= (H * Mb + 1) * 4 and o[3] >= o[2] + 4
    assert n >= o[3] + H * Mb * Nb * 4 and n % 256 == 0
    assert lib.bsa_plan_sections(H, 0, Nb, offs) == INVALID


def _plan_struct(H=2, Mb=4, Nb=4, buf=0x100000, nbytes=None, lib=None):
    p = bsa._PlanT()
    p.H, p.Mb, p.Nb = H, Mb, Nb
    p.dev_buf = buf
    p.dev_bytes = nbytes if nbytes is not None else lib.bsa_plan_buffer_bytes(H, Mb, Nb)
    return p


def test_bsa_plan_validation(lib):
    P = ctypes.byref(bsa._PlanT())
    fake = ctypes.c_void_p(0x10000)
    n = lib.bsa_plan_buffer_bytes(2, 4, 4)
    assert lib.bsa_plan(None, 2, 4, 4, fake, n, P, None) == INVALID
    assert lib.bsa_plan(fake, 2, 4, 4, None, n, P, None) == INVALID
    assert lib.bsa_plan(fake, 2, 4, 4, fake, n, None, None) == INVALID
    assert lib.bsa_plan(fake, 0, 4, 4, fake, n, P, None) == INVALID
    assert lib.bsa_plan(fake, 2, 4, 20000, fake, 1 << 30, P, None) == UNSUPPORTED
    assert lib.bsa_plan(fake, 2, 4, 4, ctypes.c_void_p(0x10010), n, P, None) == MISALIGNED
    assert lib.bsa_plan(fake, 2, 4, 4, fake, n - 1, P, None) == TOO_SMALL
    assert b"buffer" in lib.bsa_last_error()


def test_bsa_forward_validation(lib):
    f = ctypes.c_void_p(0x10000)
    p = _plan_struct(lib=lib)
    P = ctypes.byref(p)
    args = dict(B=1, H=2, Sq=64, Sk=64, bs=16, d=32, dtype=0, scale=0.5)

    def call(q=f, k=f, v=f, plan=P, out=f, lse=None, **kw):
        a = dict(args, **kw)
        return lib.bsa_forward(q, k, v, plan, a["B"], a["H"], a["Sq"], a["Sk"], a["bs"], a["d"],
                               a["dtype"], a["scale"], out, lse, None)

    assert call(q=None) == INVALID
    assert call(out=None) == INVALID
    assert call(plan=None) == INVALID
    assert call(B=0) == INVALID
    assert call(H=3) == MISMATCH
    assert call(Sq=128) == MISMATCH
    assert call(Sk=32) == MISMATCH
    assert call(scale=0.0) == INVALID
    assert call(scale=float("nan")) == INVALID
    assert call(scale=-1.0) == INVALID
    assert call(dtype=7) == INVALID
    assert call(d=48) == UNSUPPORTED
    assert call(bs=8, Sq=32, Sk=32) == UNSUPPORTED
    assert call(q=ctypes.c_void_p(0x10008)) == MISALIGNED
    assert call(lse=ctypes.c_void_p(0x10002)) == MISALIGNED
    small = _plan_struct(nbytes=64, lib=lib)
    assert call(plan=ctypes.byref(small)) == TOO_SMALL
    nobuf = _plan_struct(buf=0, lib=lib)
    assert call(plan=ctypes.byref(nobuf)) == INVALID


def test_bsa_forward_ex_validation(lib):
    """Option checks of bsa_forward_ex; every call here fails before a launch."""
    f = ctypes.c_void_p(0x10000)
    p = _plan_struct(lib=lib)
    P = ctypes.byref(p)

    def call(sink=None, soft_cap=0.0, causal=0, kv_heads=0, opts=True, **kw):
        a = dict(B=1, H=2, Sq=64, Sk=64, bs=16, d=32, dtype=0, scale=0.5)
        a.update(kw)
        o = bsa._FwdOptsT(sink, soft_cap, causal, kv_heads)
        return lib.bsa_forward_ex(f, f, f, P, a["B"], a["H"], a["Sq"], a["Sk"], a["bs"],
                                  a["d"], a["dtype"], a["scale"],
                                  ctypes.byref(o) if opts else None, f, None, None)

    assert call(kv_heads=3) == INVALID          # does not divide H = 2
    assert call(kv_heads=-1) == INVALID
    assert call(kv_heads=4) == INVALID
    assert call(soft_cap=-1.0) == INVALID
    assert call(soft_cap=float("inf")) == INVALID
    assert call(soft_cap=float("nan")) == INVALID
    assert call(soft_cap=1e-44) == INVALID      # 2*scale*log2(e)/cap overflows fp32
    assert call(sink=0x10002) == MISALIGNED
    # segment ids come in pairs and are 4-byte aligned
    def call_seg(qs, ks):
        o = bsa._FwdOptsT(None, 0.0, 0, 0, qs, ks)
        return lib.bsa_forward_ex(f, f, f, P, 1, 2, 64, 64, 16, 32, 0, 0.5, ctypes.byref(o), f,
                                  None, None)
    assert call_seg(0x10000, None) == INVALID
    assert call_seg(None, 0x10000) == INVALID
    assert call_seg(0x10002, 0x10000) == MISALIGNED
    # the plain checks still run first with options present
    assert call(kv_heads=1, H=3) == MISMATCH
    assert call(opts=False, d=48) == UNSUPPORTED
    assert call(causal=1, bs=8, Sq=32, Sk=32) == UNSUPPORTED


def test_topk_validation(lib):
    f = ctypes.c_void_p(0x10000)

    def call(q=f, kv=f, idx=f, sink=None, B=1, M=4, N=16, H=8, d=512, topk=8, scale=0.1, out=f):
        return lib.topk_sparse_attn(q, kv, idx, sink, B, M, N, H, d, topk, scale, out, None)

    assert call(q=None) == INVALID
    assert call(idx=None) == INVALID
    assert call(topk=0) == INVALID
    assert call(N=-1) == INVALID
    assert call(scale=float("inf")) == INVALID
    assert call(H=64 * 65535 + 1) == UNSUPPORTED  # head groups of 64 exceed the grid's y range
    assert call(d=192) == UNSUPPORTED
    assert call(kv=ctypes.c_void_p(0x10004)) == MISALIGNED
    assert call(sink=ctypes.c_void_p(0x10001)) == MISALIGNED
    # one batch of kv may span at most 4 GiB - 1 KiB (row offsets of -1 slots wrap past it)
    assert call(N=(1 << 22), d=512) == UNSUPPORTED      # 4 GiB
    assert call(N=(1 << 23) - 1, d=256) == UNSUPPORTED  # 4 GiB - 512 B


def test_backward_noalloc_validation(lib):
    """The entry point without a workspace validates like bsa_backward and
    refuses problems beyond its static scratch (2^21 query rows), all before
    any HIP call."""
    assert lib.bsa_backward_noalloc_max_rows() == 1 << 21
    f = ctypes.c_void_p(0x10000)

    def planned(H, Sq, bs):
        nb = -(-Sq // bs)
        p = _plan_struct(H=H, Mb=nb, Nb=nb, lib=lib)
        pc = bsa._PlanColsT()
        pc.H, pc.Hkv, pc.Mb, pc.Nb = H, H, nb, nb
        pc.dev_buf = 0x200000
        pc.dev_bytes = lib.bsa_plan_cols_buffer_bytes(H, H, nb, nb)
        return p, pc

    def call(B=1, H=2, Sq=64, bs=16, d=32, dq=f, lse=f, scale=0.5):
        p, pc = planned(H, Sq, bs)
        return lib.bsa_backward_noalloc(f, f, f, f, f, lse, ctypes.byref(p), ctypes.byref(pc), B,
                                        H, Sq, Sq, bs, d, 0, scale, None, dq, f, f, None, None)

    assert call(dq=None) == INVALID
    assert call(lse=None) == INVALID
    assert call(scale=0.0) == INVALID
    assert call(d=48) == UNSUPPORTED
    assert call(dq=ctypes.c_void_p(0x10008)) == MISALIGNED
    # one query row past the limit, as several batch items of 32 heads
    assert call(B=65, H=32, Sq=1024, bs=128, d=128) == UNSUPPORTED
    assert "static scratch" in lib.bsa_last_error().decode()


def test_status_strings(lib):
    for code in (OK, INVALID, UNSUPPORTED, MISALIGNED, MISMATCH, TOO_SMALL, -6):
        s = lib.bsa_status_string(code)
        assert s and s != b"unknown status"
    assert lib.bsa_status_string(42) == b"unknown status"


def test_python_binding_rejects_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        bsa.bsa_plan(torch.ones((1, 2, 2), dtype=torch.int32))
