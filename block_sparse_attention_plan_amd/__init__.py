"""Block-sparse attention forward for AMD Instinct MI355X (gfx950).

Thin Python binding of ``libbsa.so`` (C ABI in ``include/bsa.h``).  The
functions below only check and marshal arguments; every step of the
computation runs in the library's HIP kernels.  PyTorch supplies device
memory and the current stream.  There is no CPU fallback: if the library is
missing, every call raises.

    bsa_plan(layout)                      -> Plan   (per-row CSR of live tiles)
    bsa_forward(q, k, v, plan, scale, *, attn_sink, soft_cap, causal)
                                          -> (out, lse)
    bsa_plan_cols(layout, kv_heads)       -> PlanCols (per-column CSR, backward)
    bsa_backward(q, k, v, out, dout, lse, plan, plan_cols, scale, *, options)
                                          -> (dq, dk, dv, dsink)
    bsa_backward_noalloc(..., dq=, dk=, dv=, dsink=)  (no allocation; static scratch)
    bsa_layout_adaptive(q, k, bs, tau, causal, keep_diagonal) -> (layout, scores)
    topk_sparse_attn(q, kv, idx, attn_sink, scale) -> out
    bsa_plan_check(plan, plan_cols)       consistency of plan contents (raises)
    set_debug(on)                         check plans before every call
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "BsaError",
    "Plan",
    "bsa_plan",
    "plan_buffer",
    "bsa_plan_nnz",
    "bsa_forward",
    "PlanCols",
    "bsa_plan_cols",
    "bsa_backward",
    "bsa_backward_noalloc",
    "bsa_layout_adaptive",
    "topk_sparse_attn",
    "bsa_plan_check",
    "set_debug",
    "library_path",
    "load_library",
]

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG_DIR, "libbsa.so")
_lib = None

BSA_BF16 = 0
BSA_F32 = 1


class BsaError(RuntimeError):
    """A libbsa call returned a non-zero status."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


class _PlanT(ctypes.Structure):
    _fields_ = [
        ("H", ctypes.c_int32),
        ("Mb", ctypes.c_int32),
        ("Nb", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("dev_buf", ctypes.c_void_p),
        ("dev_bytes", ctypes.c_size_t),
    ]


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libbsa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"libbsa.so not found at {_LIB_PATH}; build it with "
            "`python -m block_sparse_attention_plan_amd.build`")
    # torch is imported first so that its HIP runtime (same soname) is the one
    # the library binds to; streams and pointers then belong to one runtime.
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    lib.bsa_plan_buffer_bytes.argtypes = [i32, i32, i32]
    lib.bsa_plan_buffer_bytes.restype = ctypes.c_size_t
    lib.bsa_plan_sections.argtypes = [i32, i32, i32, ctypes.POINTER(ctypes.c_size_t)]
    lib.bsa_plan_sections.restype = ctypes.c_int
    lib.bsa_plan_pair_sections.argtypes = [i32, i32, i32, ctypes.POINTER(ctypes.c_size_t)]
    lib.bsa_plan_pair_sections.restype = ctypes.c_int
    lib.bsa_plan.argtypes = [vp, i32, i32, i32, vp, ctypes.c_size_t, ctypes.POINTER(_PlanT), vp]
    lib.bsa_plan.restype = ctypes.c_int
    lib.bsa_plan_nnz.argtypes = [ctypes.POINTER(_PlanT), ctypes.POINTER(ctypes.c_int64), vp]
    lib.bsa_plan_nnz.restype = ctypes.c_int
    lib.bsa_forward.argtypes = [vp, vp, vp, ctypes.POINTER(_PlanT), i32, i32, i32, i32, i32, i32,
                                ctypes.c_int, f32, vp, vp, vp]
    lib.bsa_forward.restype = ctypes.c_int
    lib.bsa_forward_ex.argtypes = [vp, vp, vp, ctypes.POINTER(_PlanT), i32, i32, i32, i32, i32,
                                   i32, i32, f32, ctypes.POINTER(_FwdOptsT), vp, vp, vp]
    lib.bsa_forward_ex.restype = ctypes.c_int
    lib.bsa_plan_cols_buffer_bytes.argtypes = [i32, i32, i32, i32]
    lib.bsa_plan_cols_buffer_bytes.restype = ctypes.c_size_t
    lib.bsa_plan_cols_sections.argtypes = [i32, i32, i32, i32, ctypes.POINTER(ctypes.c_size_t)]
    lib.bsa_plan_cols_sections.restype = ctypes.c_int
    lib.bsa_plan_cols.argtypes = [vp, i32, i32, i32, i32, vp, ctypes.c_size_t,
                                  ctypes.POINTER(_PlanColsT), vp]
    lib.bsa_plan_cols.restype = ctypes.c_int
    lib.bsa_backward_workspace_bytes.argtypes = [i32, i32, i32]
    lib.bsa_backward_workspace_bytes.restype = ctypes.c_size_t
    lib.bsa_backward.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.POINTER(_PlanT),
                                 ctypes.POINTER(_PlanColsT), i32, i32, i32, i32, i32, i32, i32,
                                 f32, ctypes.POINTER(_FwdOptsT), vp, ctypes.c_size_t, vp, vp, vp,
                                 vp, vp]
    lib.bsa_backward.restype = ctypes.c_int
    lib.bsa_backward_noalloc_max_rows.argtypes = []
    lib.bsa_backward_noalloc_max_rows.restype = ctypes.c_size_t
    lib.bsa_backward_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.POINTER(_PlanT),
                                         ctypes.POINTER(_PlanColsT), i32, i32, i32, i32, i32, i32,
                                         i32, f32, ctypes.POINTER(_FwdOptsT), vp, vp, vp, vp, vp]
    lib.bsa_backward_noalloc.restype = ctypes.c_int
    lib.bsa_layout_adaptive_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.bsa_layout_adaptive_workspace_bytes.restype = ctypes.c_size_t
    lib.bsa_layout_adaptive.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, i32, i32,
                                        vp, ctypes.c_size_t, vp, vp, vp]
    lib.bsa_layout_adaptive.restype = ctypes.c_int
    lib.topk_sparse_attn.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, vp, vp]
    lib.topk_sparse_attn.restype = ctypes.c_int
    lib.bsa_plan_check.argtypes = [ctypes.POINTER(_PlanT), ctypes.POINTER(_PlanColsT), vp]
    lib.bsa_plan_check.restype = ctypes.c_int
    lib.bsa_plan_check_host.argtypes = [vp, ctypes.c_size_t, vp, ctypes.c_size_t, i32, i32, i32,
                                        i32]
    lib.bsa_plan_check_host.restype = ctypes.c_int
    lib.bsa_set_debug.argtypes = [ctypes.c_int]
    lib.bsa_set_debug.restype = ctypes.c_int
    lib.bsa_status_string.argtypes = [ctypes.c_int]
    lib.bsa_status_string.restype = ctypes.c_char_p
    lib.bsa_last_error.argtypes = []
    lib.bsa_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        lib = load_library()
        msg = lib.bsa_last_error().decode(errors="replace") or lib.bsa_status_string(status).decode()
        raise BsaError(status, msg)


def _stream(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _require_gpu(name: str, t: torch.Tensor) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


class _FwdOptsT(ctypes.Structure):
    _fields_ = [
        ("attn_sink", ctypes.c_void_p),
        ("soft_cap", ctypes.c_float),
        ("causal", ctypes.c_int32),
        ("kv_heads", ctypes.c_int32),
        ("q_segment_ids", ctypes.c_void_p),
        ("kv_segment_ids", ctypes.c_void_p),
    ]


def _segment_args(q_segment_ids, kv_segment_ids, B, Sq, Sk):
    if (q_segment_ids is None) != (kv_segment_ids is None):
        raise ValueError("segment ids come in pairs (queries and keys)")
    if q_segment_ids is None:
        return 0, 0
    for name, t, S in (("q_segment_ids", q_segment_ids, Sq), ("kv_segment_ids", kv_segment_ids, Sk)):
        _require_gpu(name, t)
        if t.dtype != torch.int32 or tuple(t.shape) != (B, S):
            raise ValueError(f"{name} must be int32 [B, {S}]")
    return q_segment_ids.data_ptr(), kv_segment_ids.data_ptr()


class _PlanColsT(ctypes.Structure):
    _fields_ = [
        ("H", ctypes.c_int32),
        ("Hkv", ctypes.c_int32),
        ("Mb", ctypes.c_int32),
        ("Nb", ctypes.c_int32),
        ("dev_buf", ctypes.c_void_p),
        ("dev_bytes", ctypes.c_size_t),
    ]


class Plan:
    """A built plan: owns its device buffer (a uint8 tensor)."""

    def __init__(self, buf: torch.Tensor, raw: _PlanT, H: int, Mb: int, Nb: int):
        self.buf = buf
        self._raw = raw
        self.H, self.Mb, self.Nb = H, Mb, Nb
        offs = (ctypes.c_size_t * 4)()
        _check(load_library().bsa_plan_sections(H, Mb, Nb, offs))
        self._offs = [int(o) for o in offs]
        _check(load_library().bsa_plan_pair_sections(H, Mb, Nb, offs))
        self._offs += [int(o) for o in offs]
        self.Mp = (Mb + 1) // 2

    def _section(self, i: int, count: int) -> torch.Tensor:
        off = self._offs[i]
        return self.buf[off:off + 4 * count].view(torch.int32)

    @property
    def row_ptr(self) -> torch.Tensor:
        return self._section(0, self.H * self.Mb + 1)

    @property
    def row_order(self) -> torch.Tensor:
        return self._section(1, self.H * self.Mb)

    @property
    def nnz_total_dev(self) -> torch.Tensor:
        return self._section(2, 1)

    def col_idx(self, nnz_total: Optional[int] = None) -> torch.Tensor:
        n = self.nnz() if nnz_total is None else nnz_total
        return self._section(3, n)

    def nnz(self) -> int:
        return bsa_plan_nnz(self)

    # Pairs of neighbouring block rows (2p, 2p+1): the union of their live
    # columns, each entry n | mask << 24 (bit 24: row 2p lists n, bit 25: row
    # 2p+1 does), and the flag that makes the forward use them.
    @property
    def pair_ptr(self) -> torch.Tensor:
        return self._section(4, self.H * self.Mp + 1)

    @property
    def pair_order(self) -> torch.Tensor:
        return self._section(5, self.H * self.Mp)

    @property
    def pair_info(self) -> torch.Tensor:
        """int32 [2]: pair_total, use_pairs."""
        return self._section(6, 2)

    def pair_cols(self, pair_total: Optional[int] = None) -> torch.Tensor:
        n = int(self.pair_info[0].item()) if pair_total is None else pair_total
        return self._section(7, n)


def plan_buffer(layout_shape, device) -> torch.Tensor:
    """Allocate a 256-byte aligned plan buffer for a layout of this shape."""
    H, Mb, Nb = (int(x) for x in layout_shape)
    nbytes = load_library().bsa_plan_buffer_bytes(H, Mb, Nb)
    if nbytes == 0:
        raise ValueError(f"invalid layout shape {tuple(layout_shape)}")
    buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    shift = (-buf.data_ptr()) % 256
    return buf[shift:shift + nbytes]


def bsa_plan(layout: torch.Tensor, buf: Optional[torch.Tensor] = None) -> Plan:
    """Build the per-row CSR plan of an int32 layout [H, Mb, Nb] on the GPU.

    ``buf`` optionally supplies a buffer from plan_buffer() to reuse."""
    _require_gpu("layout", layout)
    if layout.dtype != torch.int32 or layout.dim() != 3:
        raise ValueError("layout must be an int32 tensor [H, Mb, Nb]")
    lib = load_library()
    H, Mb, Nb = (int(x) for x in layout.shape)
    nbytes = lib.bsa_plan_buffer_bytes(H, Mb, Nb)
    if buf is None:
        buf = plan_buffer(layout.shape, layout.device)
    elif buf.dtype != torch.uint8 or buf.numel() < nbytes or buf.device != layout.device:
        raise ValueError("buf must be a uint8 plan buffer from plan_buffer() for this shape")
    raw = _PlanT()
    _check(lib.bsa_plan(ctypes.c_void_p(layout.data_ptr()), H, Mb, Nb,
                        ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.byref(raw),
                        _stream(layout)))
    return Plan(buf, raw, H, Mb, Nb)


def bsa_plan_nnz(plan: Plan) -> int:
    """Number of live tiles of a plan (synchronises the current stream)."""
    out = ctypes.c_int64(0)
    _check(load_library().bsa_plan_nnz(ctypes.byref(plan._raw), ctypes.byref(out),
                                       _stream(plan.buf)))
    return int(out.value)


def _block_size(Sq: int, Sk: int, plan, bs: Optional[int]) -> int:
    if bs is None:
        if Sq % plan.Mb:
            raise ValueError("Sq is not a multiple of the layout's block rows: pass bs")
        bs = Sq // plan.Mb
    bs = int(bs)
    if bs <= 0 or -(-Sq // bs) != plan.Mb or -(-Sk // bs) != plan.Nb:
        raise ValueError(f"bs={bs}: the layout's {plan.Mb} x {plan.Nb} blocks do not cover "
                         f"Sq={Sq}, Sk={Sk}")
    return bs


def bsa_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, plan: Plan,
                scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                lse: Optional[torch.Tensor] = None, want_lse: bool = True, *,
                attn_sink: Optional[torch.Tensor] = None, soft_cap: Optional[float] = None,
                causal: bool = False, bs: Optional[int] = None,
                q_segment_ids: Optional[torch.Tensor] = None,
                kv_segment_ids: Optional[torch.Tensor] = None
                ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Block-sparse attention forward.

    q: [B, H, Sq, d], k/v: [B, Hkv, Sk, d] with H % Hkv == 0 (query head h
    reads K/V head h // (H // Hkv)), bf16 or fp32, with Sq = Mb*bs and
    Sk = Nb*bs for the plan's layout.  Returns (out [B, H, Sq, d] of q's dtype,
    lse [B, H, Sq] fp32 or None).  scale defaults to 1/sqrt(d).  attn_sink
    (fp32 [H]) adds exp(attn_sink[h]) to each softmax denominator; soft_cap
    caps the scaled scores to soft_cap * tanh(s / soft_cap); causal also masks
    key tokens after the query token.  bs (default Sq / Mb) must be given when
    a length is not a multiple of the block size: the plan's layout then
    covers ceil(S / bs) blocks and the last block is cut at the sequence end.
    q_segment_ids / kv_segment_ids (int32 [B, Sq] / [B, Sk]) restrict every
    query to the keys of its own segment (packed sequences).
    """
    for name, t in (("q", q), ("k", k), ("v", v)):
        _require_gpu(name, t)
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, S, d]")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q, k, v must share dtype bf16 or fp32")
    B, H, Sq, d = (int(x) for x in q.shape)
    Hkv = int(k.shape[1])
    if (tuple(k.shape) != tuple(v.shape) or k.shape[0] != B or k.shape[3] != d or Hkv < 1
            or H % Hkv != 0):
        raise ValueError("k and v must be [B, Hkv, Sk, d] matching q, with Hkv dividing H")
    if attn_sink is not None:
        _require_gpu("attn_sink", attn_sink)
        if attn_sink.dtype != torch.float32 or tuple(attn_sink.shape) != (H,):
            raise ValueError("attn_sink must be fp32 [H]")
    if soft_cap is not None and not (math.isfinite(soft_cap) and soft_cap > 0):
        raise ValueError("soft_cap must be finite and > 0")
    Sk = int(k.shape[2])
    bs = _block_size(Sq, Sk, plan, bs)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    else:
        _require_gpu("out", out)
        if out.shape != q.shape or out.dtype != q.dtype:
            raise ValueError("out must match q")
    if want_lse and lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _require_gpu("lse", lse)
        if tuple(lse.shape) != (B, H, Sq) or lse.dtype != torch.float32:
            raise ValueError("lse must be fp32 [B, H, Sq]")
    dtype = BSA_BF16 if q.dtype == torch.bfloat16 else BSA_F32
    lse_ptr = ctypes.c_void_p(lse.data_ptr() if lse is not None else 0)
    qsp, ksp = _segment_args(q_segment_ids, kv_segment_ids, B, Sq, Sk)
    if attn_sink is None and soft_cap is None and not causal and Hkv == H and not qsp:
        _check(load_library().bsa_forward(
            ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
            ctypes.c_void_p(v.data_ptr()), ctypes.byref(plan._raw), B, H, Sq, Sk, bs, d, dtype,
            float(scale), ctypes.c_void_p(out.data_ptr()), lse_ptr, _stream(q)))
        return out, lse
    opts = _FwdOptsT(ctypes.c_void_p(attn_sink.data_ptr() if attn_sink is not None else 0),
                     float(soft_cap or 0.0), 1 if causal else 0, Hkv, ctypes.c_void_p(qsp),
                     ctypes.c_void_p(ksp))
    _check(load_library().bsa_forward_ex(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
        ctypes.c_void_p(v.data_ptr()), ctypes.byref(plan._raw), B, H, Sq, Sk, bs, d, dtype,
        float(scale), ctypes.byref(opts), ctypes.c_void_p(out.data_ptr()), lse_ptr, _stream(q)))
    return out, lse


class PlanCols:
    """A built column plan (backward): owns its device buffer."""

    def __init__(self, buf: torch.Tensor, raw: _PlanColsT, H: int, Hkv: int, Mb: int, Nb: int):
        self.buf = buf
        self._raw = raw
        self.H, self.Hkv, self.Mb, self.Nb = H, Hkv, Mb, Nb
        offs = (ctypes.c_size_t * 4)()
        _check(load_library().bsa_plan_cols_sections(H, Hkv, Mb, Nb, offs))
        self._offs = [int(o) for o in offs]

    def _section(self, i: int, count: int) -> torch.Tensor:
        off = self._offs[i]
        return self.buf[off:off + 4 * count].view(torch.int32)

    @property
    def col_ptr(self) -> torch.Tensor:
        return self._section(0, self.H * self.Nb + 1)

    @property
    def col_order(self) -> torch.Tensor:
        return self._section(1, self.Hkv * self.Nb)

    @property
    def nnz_total_dev(self) -> torch.Tensor:
        return self._section(2, 1)

    def row_idx(self, nnz_total: int) -> torch.Tensor:
        return self._section(3, nnz_total)


def bsa_plan_cols(layout: torch.Tensor, kv_heads: Optional[int] = None,
                  buf: Optional[torch.Tensor] = None) -> PlanCols:
    """Build the column plan (for the backward) of an int32 layout [H, Mb, Nb]
    whose query heads share kv_heads K/V heads (default: H)."""
    _require_gpu("layout", layout)
    if layout.dtype != torch.int32 or layout.dim() != 3:
        raise ValueError("layout must be an int32 tensor [H, Mb, Nb]")
    lib = load_library()
    H, Mb, Nb = (int(x) for x in layout.shape)
    Hkv = H if kv_heads is None else int(kv_heads)
    nbytes = lib.bsa_plan_cols_buffer_bytes(H, Hkv, Mb, Nb)
    if nbytes == 0:
        raise ValueError(f"invalid layout shape {tuple(layout.shape)} for kv_heads={Hkv}")
    if buf is None:
        raw_buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=layout.device)
        shift = (-raw_buf.data_ptr()) % 256
        buf = raw_buf[shift:shift + nbytes]
    elif buf.dtype != torch.uint8 or buf.numel() < nbytes or buf.device != layout.device:
        raise ValueError("buf must be a 256-byte aligned uint8 buffer of enough bytes")
    raw = _PlanColsT()
    _check(lib.bsa_plan_cols(ctypes.c_void_p(layout.data_ptr()), H, Hkv, Mb, Nb,
                             ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.byref(raw),
                             _stream(layout)))
    return PlanCols(buf, raw, H, Hkv, Mb, Nb)


def bsa_plan_check(plan: Optional[Plan] = None, plan_cols: Optional[PlanCols] = None) -> None:
    """Check the contents of a plan and/or a column plan (and, given both,
    that one is the other's transpose); raises BsaError (status
    BSA_ERR_BAD_PLAN = -7) naming the first inconsistency.  Synchronises the
    current stream."""
    if plan is None and plan_cols is None:
        raise ValueError("give a plan, a column plan or both")
    buf = plan.buf if plan is not None else plan_cols.buf
    _check(load_library().bsa_plan_check(
        ctypes.byref(plan._raw) if plan is not None else None,
        ctypes.byref(plan_cols._raw) if plan_cols is not None else None, _stream(buf)))


def set_debug(on: bool) -> bool:
    """Debug mode: every call that reads a plan checks it first (as
    bsa_plan_check) and refuses an inconsistent one.  Returns the previous
    setting.  The environment variable BSA_DEBUG sets the initial value."""
    return bool(load_library().bsa_set_debug(1 if on else 0))


def _backward_args(q, k, v, out, dout, lse, plan, scale, attn_sink, soft_cap, causal, dq, dk,
                   dv, dsink, bs, q_segment_ids, kv_segment_ids):
    """Checks of a backward call; returns the sizes, the outputs (allocated
    where not given) and the marshalled options."""
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout), ("lse", lse)):
        _require_gpu(name, t)
    if not (q.dtype == k.dtype == v.dtype == out.dtype == dout.dtype) or \
            q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q, k, v, out, dout must share dtype bf16 or fp32")
    B, H, Sq, d = (int(x) for x in q.shape)
    Hkv, Sk = int(k.shape[1]), int(k.shape[2])
    if tuple(k.shape) != tuple(v.shape) or k.shape[0] != B or k.shape[3] != d or H % Hkv:
        raise ValueError("k and v must be [B, Hkv, Sk, d] matching q, with Hkv dividing H")
    if tuple(out.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape):
        raise ValueError("out and dout must match q")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, Sq):
        raise ValueError("lse must be fp32 [B, H, Sq]")
    bs = _block_size(Sq, Sk, plan, bs)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if attn_sink is not None:
        _require_gpu("attn_sink", attn_sink)
        if attn_sink.dtype != torch.float32 or tuple(attn_sink.shape) != (H,):
            raise ValueError("attn_sink must be fp32 [H]")
    if soft_cap is not None and not (math.isfinite(soft_cap) and soft_cap > 0):
        raise ValueError("soft_cap must be finite and > 0")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _require_gpu(name, t)
        if t.shape != like.shape or t.dtype != like.dtype:
            raise ValueError(f"{name} must match {'q' if like is q else 'k'}")
    if attn_sink is None:
        dsink = None
    elif dsink is None:
        dsink = torch.empty(H, dtype=torch.float32, device=q.device)
    else:
        _require_gpu("dsink", dsink)
        if dsink.dtype != torch.float32 or tuple(dsink.shape) != (H,):
            raise ValueError("dsink must be fp32 [H]")
    qsp, ksp = _segment_args(q_segment_ids, kv_segment_ids, B, Sq, Sk)
    opts = _FwdOptsT(ctypes.c_void_p(attn_sink.data_ptr() if attn_sink is not None else 0),
                     float(soft_cap or 0.0), 1 if causal else 0, Hkv, ctypes.c_void_p(qsp),
                     ctypes.c_void_p(ksp))
    dtype = BSA_BF16 if q.dtype == torch.bfloat16 else BSA_F32
    return (B, H, Sq, Sk, bs, d, float(scale), dtype), (dq, dk, dv, dsink), opts


def _ptr(t: Optional[torch.Tensor]) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr() if t is not None else 0)


def bsa_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                 dout: torch.Tensor, lse: torch.Tensor, plan: Plan, plan_cols: PlanCols,
                 scale: Optional[float] = None, *, attn_sink: Optional[torch.Tensor] = None,
                 soft_cap: Optional[float] = None, causal: bool = False,
                 dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
                 dv: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None, bs: Optional[int] = None,
                 q_segment_ids: Optional[torch.Tensor] = None,
                 kv_segment_ids: Optional[torch.Tensor] = None,
                 dsink: Optional[torch.Tensor] = None):
    """Gradients of bsa_forward for the upstream gradient dout.

    q, k, v, scale and the options must be those of the forward call that
    produced out and lse.  Returns (dq, dk, dv, dsink): dq like q, dk and dv
    like k, dsink fp32 [H] (None without a sink).  bf16 or fp32 I/O.
    """
    sizes, (dq, dk, dv, dsink), opts = _backward_args(
        q, k, v, out, dout, lse, plan, scale, attn_sink, soft_cap, causal, dq, dk, dv, dsink, bs,
        q_segment_ids, kv_segment_ids)
    B, H, Sq, Sk, bs, d, scale, dtype = sizes
    lib = load_library()
    wbytes = lib.bsa_backward_workspace_bytes(B, H, Sq)
    if workspace is None:
        workspace = torch.empty(wbytes // 4, dtype=torch.float32, device=q.device)
    elif workspace.numel() * workspace.element_size() < wbytes:
        raise ValueError("workspace too small")
    _check(lib.bsa_backward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse),
        ctypes.byref(plan._raw), ctypes.byref(plan_cols._raw), B, H, Sq, Sk, bs, d, dtype,
        scale, ctypes.byref(opts), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dsink), _stream(q)))
    return dq, dk, dv, dsink


def bsa_backward_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                         dout: torch.Tensor, lse: torch.Tensor, plan: Plan, plan_cols: PlanCols,
                         scale: Optional[float] = None, *, dq: torch.Tensor, dk: torch.Tensor,
                         dv: torch.Tensor, dsink: Optional[torch.Tensor] = None,
                         attn_sink: Optional[torch.Tensor] = None,
                         soft_cap: Optional[float] = None, causal: bool = False,
                         bs: Optional[int] = None, q_segment_ids: Optional[torch.Tensor] = None,
                         kv_segment_ids: Optional[torch.Tensor] = None):
    """bsa_backward for callers that cannot allocate: the outputs dq, dk, dv
    (and dsink with a sink) are the caller's, and the library's per-row
    scratch lives in a static device array (at most
    bsa_backward_noalloc_max_rows() query rows, B*H*Sq).  Calls that overlap
    on one GPU share that array and race.  Returns (dq, dk, dv, dsink)."""
    if attn_sink is not None and dsink is None:
        raise ValueError("bsa_backward_noalloc: pass dsink (fp32 [H]) with attn_sink")
    sizes, (dq, dk, dv, dsink), opts = _backward_args(
        q, k, v, out, dout, lse, plan, scale, attn_sink, soft_cap, causal, dq, dk, dv, dsink, bs,
        q_segment_ids, kv_segment_ids)
    B, H, Sq, Sk, bs, d, scale, dtype = sizes
    lib = load_library()
    _check(lib.bsa_backward_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse),
        ctypes.byref(plan._raw), ctypes.byref(plan_cols._raw), B, H, Sq, Sk, bs, d, dtype,
        scale, ctypes.byref(opts), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dsink), _stream(q)))
    return dq, dk, dv, dsink


def bsa_layout_adaptive(q: torch.Tensor, k: torch.Tensor, bs: int, tau: float, *,
                        causal: bool = False, keep_diagonal: bool = True,
                        want_scores: bool = False, workspace: Optional[torch.Tensor] = None):
    """Content-adaptive block layout of one batch item.

    q: [H, Sq, d], k: [Hkv, Sk, d] (bf16 or fp32, same dtype).  Returns
    (layout int32 [H, Sq/bs, Sk/bs], scores fp32 of the same shape or None):
    a block pair is live when the cosine similarity of its block-mean query
    and key reaches tau.
    """
    for name, t in (("q", q), ("k", k)):
        _require_gpu(name, t)
        if t.dim() != 3:
            raise ValueError(f"{name} must be [heads, S, d]")
    if q.dtype != k.dtype or q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q and k must share dtype bf16 or fp32")
    H, Sq, d = (int(x) for x in q.shape)
    Hkv, Sk = int(k.shape[0]), int(k.shape[1])
    if int(k.shape[2]) != d or H % Hkv:
        raise ValueError("k must be [Hkv, Sk, d] with Hkv dividing H")
    if Sq % bs or Sk % bs:
        raise ValueError("Sq and Sk must be multiples of bs")
    lib = load_library()
    Mb, Nb = Sq // bs, Sk // bs
    wbytes = lib.bsa_layout_adaptive_workspace_bytes(H, Hkv, Mb, Nb, d)
    if workspace is None:
        workspace = torch.empty(max(wbytes // 4, 1), dtype=torch.float32, device=q.device)
    layout = torch.empty((H, Mb, Nb), dtype=torch.int32, device=q.device)
    scores = torch.empty((H, Mb, Nb), dtype=torch.float32, device=q.device) if want_scores else None
    _check(lib.bsa_layout_adaptive(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()), H, Hkv, Sq, Sk, int(bs), d,
        BSA_BF16 if q.dtype == torch.bfloat16 else BSA_F32, float(tau), 1 if causal else 0,
        1 if keep_diagonal else 0, ctypes.c_void_p(workspace.data_ptr()),
        workspace.numel() * workspace.element_size(), ctypes.c_void_p(layout.data_ptr()),
        ctypes.c_void_p(scores.data_ptr() if scores is not None else 0), _stream(q)))
    return layout, scores


def topk_sparse_attn(q: torch.Tensor, kv: torch.Tensor, idx: torch.Tensor,
                     attn_sink: Optional[torch.Tensor], scale: Optional[float] = None,
                     out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Top-k gathered sparse attention with a per-head sink.

    q: bf16 [B, M, H, d]; kv: bf16 [B, N, d]; idx: int32 [B, M, topk] (-1 =
    unused slot); attn_sink: fp32 [H] or None.  Returns bf16 [B, M, H, d].
    scale defaults to 1/sqrt(d).
    """
    for name, t in (("q", q), ("kv", kv), ("idx", idx)):
        _require_gpu(name, t)
    if q.dtype != torch.bfloat16 or kv.dtype != torch.bfloat16:
        raise ValueError("q and kv must be bf16")
    if idx.dtype != torch.int32:
        raise ValueError("idx must be int32")
    if q.dim() != 4 or kv.dim() != 3 or idx.dim() != 3:
        raise ValueError("expected q [B,M,H,d], kv [B,N,d], idx [B,M,topk]")
    B, M, H, d = (int(x) for x in q.shape)
    N = int(kv.shape[1])
    topk = int(idx.shape[2])
    if kv.shape[0] != B or kv.shape[2] != d or idx.shape[0] != B or idx.shape[1] != M:
        raise ValueError("q, kv, idx shapes disagree")
    if attn_sink is not None:
        _require_gpu("attn_sink", attn_sink)
        if attn_sink.dtype != torch.float32 or tuple(attn_sink.shape) != (H,):
            raise ValueError("attn_sink must be fp32 [H]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    else:
        _require_gpu("out", out)
        if out.shape != q.shape or out.dtype != q.dtype:
            raise ValueError("out must match q")
    _check(load_library().topk_sparse_attn(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(kv.data_ptr()),
        ctypes.c_void_p(idx.data_ptr()),
        ctypes.c_void_p(attn_sink.data_ptr() if attn_sink is not None else 0),
        B, M, N, H, d, topk, float(scale), ctypes.c_void_p(out.data_ptr()), _stream(q)))
    return out
