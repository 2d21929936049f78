"""Reference oracle for block-sparse attention forward and the top-k gathered variant.

TEST INFRASTRUCTURE ONLY.  This module is a plain, slow, obviously correct CPU
implementation in float64 NumPy of what the GPU library computes.  It exists to
check the GPU path and to serve as the CPU baseline in the benchmark.  Only the
test suite, the package smoke check and the benchmark's CPU-baseline leg may
import it; the library itself never does, and this module imports nothing from
the library.  Callers hand it plain arrays (the same values the GPU consumes,
upcast exactly to float64).

Sources (web pages; cite by title and section):

* "Block Sparse Attention Techniques" (next.gr tutorial), section 1 "Scaled
  Dot-Product Attention" -- attention is softmax(Q K^T / sqrt(d_k)) V with rows
  of the softmax summing to one; section "Case Study: Longformer's Dilated
  Attention" -- entries outside the pattern take the value -infinity before the
  softmax; section 3.2 "Implementation with Sparse Matrix Formats" -- only the
  non-zero blocks are stored, together with their indices (the CSR plan).
* "Implementation: DeepSpeed Sparse Attention Utils" (leeroopedia), "I/O
  Contract" -- the layout is an int tensor [heads x blocks_m x blocks_n] in which
  a non-zero entry means the block is computed; the layout has no batch axis.
* "Block-Sparse Attention" (Language AI Handbook), "Block Structure" -- each
  b x b block pair is a dense piece of work; its create_block_sparse_mask example
  expands a block pattern into a token-level boolean mask.
* "ejkernel: BlockSparseAttention" (ejkernel operations page), the operation's
  arguments -- ``softmax_aux`` (values added to the scores for attention sinks),
  ``logits_soft_cap`` (tanh capping of the logits, Gemma-2 style), ``causal``
  (causal masking) and ``kv_num_heads`` for keys and values (grouped heads).
* DeepSeek-V4.1 "Sparse attention / Weighted row sum" page, code excerpt of
  sparse_attn_kernel and sparse_attn -- per query position the top-k KV rows are
  gathered by index (the same rows for every head, -1 marks an unused slot),
  scores are scaled, one softmax runs over all gathered rows, each head's sink
  logit adds one term to the softmax denominator (it is not scaled and takes no
  part in the running maximum), and a position whose slots are all -1 yields an
  all-zero output.

Readings where the pages are silent (each is listed in the design notes):

* A query row whose block row holds no live tile has out = 0 and lse = -inf.
* lse is the natural logarithm of the softmax denominator, sum_j exp(s_ij).
* Causality lives in the layout unless ``causal`` is set; then, in addition,
  key position j is masked for query position i whenever j > i (positions
  counted from 0 in both sequences).
* The soft cap maps the scaled score s to cap * tanh(s / cap), before masking.
* A block-sparse sink is one logit per query head that adds exp(sink_h) to the
  denominator, like the top-k sink (not scaled, not capped); lse includes it,
  so a row with no live key then has out = 0 and lse = sink_h.
* With kv_heads = H / g, query head h reads key/value head h // g (groups of
  g consecutive query heads share one K/V head).
* Sequence lengths are multiples of the block size.
* An absent sink (None) is the same as a sink of -infinity.
* Duplicate top-k indices count once per occurrence.

Arithmetic: every function works in float64.  The top-k function subtracts
max(max_t s_t, sink) before exponentiating; that shift cancels exactly in the
quotient and only guards float64 against overflow.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "PlanRef",
    "plan",
    "token_mask",
    "attention_dense_masked",
    "attention_live_tiles",
    "topk_attention",
]


# --------------------------------------------------------------------------
# Plan: layout -> per-row CSR of live block columns, rows ordered by nnz
# --------------------------------------------------------------------------

@dataclass
class PlanRef:
    """Per-row CSR of a block layout.

    Row r = h * Mb + m.  ``row_ptr[r]:row_ptr[r+1]`` delimits the live block
    columns of row r in ``col_idx`` (ascending n).  ``row_order`` lists all rows,
    head by head (head-major), and inside each head by nnz descending with ties
    broken by m ascending.
    """

    H: int
    Mb: int
    Nb: int
    row_ptr: np.ndarray  # int32 [H*Mb+1]
    col_idx: np.ndarray  # int32 [nnz_total]
    row_order: np.ndarray  # int32 [H*Mb]
    nnz_total: int


def plan(layout: np.ndarray) -> PlanRef:
    """CSR plan of a block layout [H, Mb, Nb]; non-zero means live.

    The layout semantics follow the DeepSpeed utils page ("I/O Contract": a
    [heads x blocks_m x blocks_n] int tensor, 1 = compute the block); storing
    only live blocks with their indices is the CSR format of the next.gr
    tutorial, section 3.2.  The ordering by nnz is the load-balance order the
    library promises: within each head, heaviest rows first, ties by m.
    """
    lay = np.asarray(layout)
    if lay.ndim != 3:
        raise ValueError("layout must be [H, Mb, Nb]")
    H, Mb, Nb = lay.shape
    live = lay != 0
    nnz = live.reshape(H * Mb, Nb).sum(axis=1).astype(np.int64)
    row_ptr = np.zeros(H * Mb + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(nnz)
    # np.nonzero on a C-ordered [rows, Nb] array walks rows in order and columns
    # ascending inside each row -- exactly the CSR column order.
    _, cols = np.nonzero(live.reshape(H * Mb, Nb))
    order = []
    for h in range(H):
        m = np.arange(Mb)
        key_nnz = nnz[h * Mb:(h + 1) * Mb]
        # lexsort sorts by the last key first: primary -nnz, secondary m.
        perm = np.lexsort((m, -key_nnz))
        order.append(h * Mb + perm)
    row_order = np.concatenate(order) if order else np.zeros(0, np.int64)
    return PlanRef(
        H=H, Mb=Mb, Nb=Nb,
        row_ptr=row_ptr.astype(np.int32),
        col_idx=cols.astype(np.int32),
        row_order=row_order.astype(np.int32),
        nnz_total=int(row_ptr[-1]),
    )


# --------------------------------------------------------------------------
# Block-sparse attention forward
# --------------------------------------------------------------------------

def token_mask(layout: np.ndarray, bs: int) -> np.ndarray:
    """Expand a block layout [H, Mb, Nb] into a token mask [H, Mb*bs, Nb*bs].

    Every token of query block m sees every token of key block n iff
    layout[h, m, n] != 0 -- the block-to-token expansion of the Language AI
    Handbook's create_block_sparse_mask example.
    """
    live = (np.asarray(layout) != 0)
    return np.repeat(np.repeat(live, bs, axis=1), bs, axis=2)


def _as64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _kv_head(H: int, Hkv: int):
    """Map query head -> key/value head for grouped heads (h // (H / Hkv))."""
    if Hkv <= 0 or H % Hkv:
        raise ValueError("the number of query heads must be a multiple of the K/V heads")
    g = H // Hkv
    return lambda h: h // g


def _cap(s: np.ndarray, soft_cap: Optional[float]) -> np.ndarray:
    return s if not soft_cap else soft_cap * np.tanh(s / soft_cap)


def attention_dense_masked(q, k, v, layout, bs: int, scale: float, *, sink=None,
                           soft_cap: Optional[float] = None, causal: bool = False
                           ) -> Tuple[np.ndarray, np.ndarray]:
    """Dense definition with non-live tiles masked to -inf.

    q: [B, H, Sq, d]; k, v: [B, Hkv, Sk, d] with H a multiple of Hkv; layout
    [H, Sq/bs, Sk/bs].  Returns out [B, H, Sq, d] and lse [B, H, Sq] (natural
    log).

    Scores s = scale * q k^T (next.gr tutorial, "Scaled Dot-Product Attention"),
    optionally capped to soft_cap * tanh(s / soft_cap), entries outside the
    layout (and, when causal, above the diagonal) set to -inf (its Longformer
    formula), then one softmax across the whole key axis of each row -- whose
    denominator also holds exp(sink_h) when a sink is given -- and a product
    with v.  Rows with no live key give out = 0 and lse = -inf (sink_h with a
    sink).
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, H, Sq, d = q.shape
    Sk = k.shape[2]
    kvh = _kv_head(H, k.shape[1])
    k = k[:, [kvh(h) for h in range(H)]]
    v = v[:, [kvh(h) for h in range(H)]]
    mask = token_mask(layout, bs)
    if mask.shape != (H, Sq, Sk):
        raise ValueError("layout does not match q/k shapes")
    if causal:
        mask = mask & (np.arange(Sk)[None, None, :] <= np.arange(Sq)[None, :, None])
    s = _cap(scale * np.matmul(q, np.swapaxes(k, -1, -2)), soft_cap)
    s = np.where(mask[None], s, -np.inf)
    row_max = s.max(axis=-1, keepdims=True)
    sk = None if sink is None else _as64(sink)[None, :, None, None]
    if sk is not None:
        row_max = np.maximum(row_max, sk)
    has_live = np.isfinite(row_max)
    shift = np.where(has_live, row_max, 0.0)
    e = np.exp(s - shift)  # exp(-inf) == 0 exactly
    den = e.sum(axis=-1, keepdims=True)
    if sk is not None:
        den = den + np.exp(sk - shift)
    with np.errstate(invalid="ignore", divide="ignore"):
        p = np.where(has_live, e / np.where(has_live, den, 1.0), 0.0)
        lse = np.where(has_live[..., 0], shift[..., 0] + np.log(np.where(has_live, den, 1.0))[..., 0],
                       -np.inf)
    out = np.matmul(p, v)
    return out, lse


def attention_live_tiles(q, k, v, layout, bs: int, scale: float,
                         row_blocks: Optional[Iterable[Tuple[int, int, int]]] = None, *,
                         sink=None, soft_cap: Optional[float] = None, causal: bool = False
                         ) -> Tuple[np.ndarray, np.ndarray]:
    """Same definition evaluated over the live tiles of each row only.

    Because exp(-inf) is exactly zero, dropping the masked keys leaves the
    softmax of every row unchanged; this form touches n*k*b score entries
    instead of n^2 (Language AI Handbook, "Block Structure").  The options have
    the meaning given in attention_dense_masked.

    ``row_blocks`` optionally restricts the work to a list of (b, h, m) query
    blocks; rows not computed are left as NaN in the returned arrays.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, H, Sq, d = q.shape
    kvh = _kv_head(H, k.shape[1])
    lay = np.asarray(layout) != 0
    Mb = Sq // bs
    if lay.shape[0] != H or lay.shape[1] != Mb or lay.shape[2] * bs != k.shape[2]:
        raise ValueError("layout does not match q/k shapes")
    sk = None if sink is None else _as64(sink)
    out = np.full((B, H, Sq, v.shape[3]), np.nan)
    lse = np.full((B, H, Sq), np.nan)
    if row_blocks is None:
        row_blocks = [(b, h, m) for b in range(B) for h in range(H) for m in range(Mb)]
    offs = np.arange(bs)
    for (b, h, m) in row_blocks:
        rows = slice(m * bs, (m + 1) * bs)
        cols = np.flatnonzero(lay[h, m])
        tok = (cols[:, None] * bs + offs[None, :]).reshape(-1)
        s = _cap(scale * (q[b, h, rows] @ k[b, kvh(h), tok].T), soft_cap)   # [bs, T]
        if causal:
            qpos = m * bs + offs
            s = np.where(tok[None, :] <= qpos[:, None], s, -np.inf)
        mx = s.max(axis=1) if tok.size else np.full(bs, -np.inf)
        if sk is not None:
            mx = np.maximum(mx, sk[h])
        live = np.isfinite(mx)
        shift = np.where(live, mx, 0.0)
        e = np.exp(s - shift[:, None])
        den = e.sum(axis=1)
        if sk is not None:
            den = den + np.exp(sk[h] - shift)
        with np.errstate(invalid="ignore", divide="ignore"):
            o = (e @ v[b, kvh(h), tok]) / np.where(live, den, 1.0)[:, None]
            out[b, h, rows] = np.where(live[:, None], o, 0.0)
            lse[b, h, rows] = np.where(live, shift + np.log(np.where(live, den, 1.0)), -np.inf)
    return out, lse


# --------------------------------------------------------------------------
# Top-k gathered sparse attention with a per-head sink
# --------------------------------------------------------------------------

def topk_attention(q, kv, idx, sink, scale: float,
                   positions: Optional[Sequence[Tuple[int, int]]] = None) -> np.ndarray:
    """Top-k gathered attention with an optional per-head sink.

    q: [B, M, H, d]; kv: [B, N, d] (one row set, used as keys and as values, the
    same for every head); idx: [B, M, topk] int with -1 for an unused slot;
    sink: [H] or None.  Returns out [B, M, H, d].

    DeepSeek-V4.1 "Weighted row sum" page: for each (batch, position) gather the
    listed rows, score every head's query against them with the given scale,
    take one softmax across all gathered rows whose denominator also holds
    exp(sink_h) (sink not scaled), and sum the rows with those weights.  Slots
    equal to -1 contribute nothing; when none is valid the output is zero.

    ``positions`` optionally restricts the work to a list of (b, m); others are
    left as NaN.
    """
    q, kv = _as64(q), _as64(kv)
    idx = np.asarray(idx)
    B, M, H, d = q.shape
    N = kv.shape[1]
    if idx.shape[:2] != (B, M):
        raise ValueError("idx must be [B, M, topk]")
    bad = (idx != -1) & ((idx < 0) | (idx >= N))
    if bad.any():
        raise ValueError("indices must be -1 or in [0, N)")
    sink64 = None if sink is None else _as64(sink)
    out = np.full((B, M, H, kv.shape[2]), np.nan)
    if positions is None:
        positions = [(b, m) for b in range(B) for m in range(M)]
    for (b, m) in positions:
        sel = idx[b, m][idx[b, m] != -1]
        rows = kv[b, sel]                       # explicit gather [T, d]
        s = scale * (q[b, m] @ rows.T)          # [H, T]
        if sel.size:
            top = s.max(axis=1)
        else:
            top = np.full(H, -np.inf)
        if sink64 is not None:
            top = np.maximum(top, sink64)
        if not np.all(np.isfinite(top)):
            # no valid slot and no sink: every weight is zero
            out[b, m] = 0.0
            continue
        e = np.exp(s - top[:, None])
        den = e.sum(axis=1)
        if sink64 is not None:
            den = den + np.exp(sink64 - top)
        out[b, m] = (e @ rows) / den[:, None]
    return out
