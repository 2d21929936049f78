"""Reference oracle for block-sparse attention (forward and backward) and the top-k gathered variant.

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
* Segment ids (the ejkernel operation's q_segment_ids [batch, seq_len] and
  kv_segment_ids [batch, kv_len], "to handle multiple sequences"): query
  token i may attend key token j only when their ids are equal, on top of
  every other mask; they come in pairs.
* Sequence lengths need not be multiples of the block size: as in the
  Language AI Handbook's create_block_sparse_mask (ceil(len / bs) blocks, the
  last block ending at the sequence end), a layout [H, ceil(Sq/bs),
  ceil(Sk/bs)] covers the sequences and its token mask is cut to [Sq, Sk].
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
    "PlanPairsRef",
    "plan_pairs",
    "token_mask",
    "attention_dense_masked",
    "attention_live_tiles",
    "PlanColsRef",
    "plan_columns",
    "attention_backward_dense",
    "attention_backward_live_tiles",
    "adaptive_layout",
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


@dataclass
class PlanPairsRef:
    """Pairs of neighbouring block rows with the union of their live columns.

    Pair q = h * Mp + p (Mp = ceil(Mb / 2)) joins block rows 2p and 2p + 1 of
    head h (only row 2p when Mb is odd and p is the last pair).
    ``pair_ptr[q]:pair_ptr[q+1]`` delimits in ``pair_cols`` the columns live in
    either row, ascending; each entry is n + 2^24 * mask, where bit 0 of mask
    says that row 2p lists column n and bit 1 that row 2p + 1 does.
    ``pair_order`` lists all pairs head by head, inside each head by union
    size descending, ties by p ascending.  ``use_pairs`` is 1 when the unions
    hold at most three quarters of the live tiles (4 * pair_total <= 3 *
    nnz_total), i.e. when streaming each pair's union once saves at least a
    quarter of the tile loads; 0 otherwise.
    """

    H: int
    Mb: int
    Nb: int
    pair_ptr: np.ndarray    # int32 [H*Mp+1]
    pair_cols: np.ndarray   # int32 [pair_total]
    pair_order: np.ndarray  # int32 [H*Mp]
    pair_total: int
    use_pairs: int


def plan_pairs(layout: np.ndarray) -> PlanPairsRef:
    """Pair plan of a block layout [H, Mb, Nb] (see PlanPairsRef).

    Neighbouring block rows of local, global and strided patterns (the
    DeepSpeed utils page's local/strided/BigBird layouts; the next.gr
    tutorial, section 3.2, on local windows and strided patterns) list
    nearly the same columns; a tile two rows both need is then loaded once
    for both.  The pair plan is a schedule of the same live tiles: decoding it
    gives back the layout exactly.
    """
    lay = np.asarray(layout)
    if lay.ndim != 3:
        raise ValueError("layout must be [H, Mb, Nb]")
    H, Mb, Nb = lay.shape
    if Nb >= (1 << 24):
        raise ValueError("column indices must fit below bit 24")
    Mp = (Mb + 1) // 2
    live = np.zeros((H, 2 * Mp, Nb), dtype=bool)
    live[:, :Mb] = lay != 0
    first, second = live[:, 0::2], live[:, 1::2]            # rows 2p and 2p+1, [H, Mp, Nb]
    union = (first | second).reshape(H * Mp, Nb)
    cnt = union.sum(axis=1).astype(np.int64)
    pair_ptr = np.zeros(H * Mp + 1, dtype=np.int64)
    pair_ptr[1:] = np.cumsum(cnt)
    q, n = np.nonzero(union)                               # n ascending inside each pair
    mask = first.reshape(H * Mp, Nb)[q, n].astype(np.int64) + \
        2 * second.reshape(H * Mp, Nb)[q, n].astype(np.int64)
    cols = n.astype(np.int64) + (mask << 24)
    order = []
    for h in range(H):
        p = np.arange(Mp)
        order.append(h * Mp + np.lexsort((p, -cnt[h * Mp:(h + 1) * Mp])))
    pair_order = np.concatenate(order) if order else np.zeros(0, np.int64)
    pair_total = int(pair_ptr[-1])
    nnz_total = int((lay != 0).sum())
    return PlanPairsRef(H=H, Mb=Mb, Nb=Nb, pair_ptr=pair_ptr.astype(np.int32),
                        pair_cols=cols.astype(np.int32), pair_order=pair_order.astype(np.int32),
                        pair_total=pair_total, use_pairs=int(4 * pair_total <= 3 * nnz_total))


# --------------------------------------------------------------------------
# Block-sparse attention forward
# --------------------------------------------------------------------------

def token_mask(layout: np.ndarray, bs: int, Sq: Optional[int] = None,
               Sk: Optional[int] = None) -> np.ndarray:
    """Expand a block layout [H, Mb, Nb] into a token mask [H, Sq, Sk]
    (default Sq = Mb*bs, Sk = Nb*bs; shorter lengths cut the last block).

    Every token of query block m sees every token of key block n iff
    layout[h, m, n] != 0 -- the block-to-token expansion of the Language AI
    Handbook's create_block_sparse_mask example, whose last block ends at the
    sequence end.
    """
    live = (np.asarray(layout) != 0)
    Mb, Nb = live.shape[1], live.shape[2]
    Sq = Mb * bs if Sq is None else Sq
    Sk = Nb * bs if Sk is None else Sk
    if _nblocks(Sq, bs) != Mb or _nblocks(Sk, bs) != Nb:
        raise ValueError("layout does not cover the sequence lengths")
    return np.repeat(np.repeat(live, bs, axis=1), bs, axis=2)[:, :Sq, :Sk]


def _nblocks(S: int, bs: int) -> int:
    """Blocks covering S tokens: ceil(S / bs) (the last one may be partial)."""
    return (S + bs - 1) // bs


def _as64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _kv_head(H: int, Hkv: int):
    """Map query head -> key/value head for grouped heads (h // (H / Hkv))."""
    if Hkv <= 0 or H % Hkv:
        raise ValueError("the number of query heads must be a multiple of the K/V heads")
    g = H // Hkv
    return lambda h: h // g


def _segments(q_segment_ids, kv_segment_ids, B, Sq, Sk):
    """Per-batch [B, Sq, Sk] mask of equal segment ids, or None."""
    if q_segment_ids is None and kv_segment_ids is None:
        return None
    if q_segment_ids is None or kv_segment_ids is None:
        raise ValueError("segment ids come in pairs (queries and keys)")
    qs = np.asarray(q_segment_ids)
    ks = np.asarray(kv_segment_ids)
    if qs.shape != (B, Sq) or ks.shape != (B, Sk):
        raise ValueError("segment ids must be [B, Sq] and [B, Sk]")
    return qs[:, :, None] == ks[:, None, :]


def _cap(s: np.ndarray, soft_cap: Optional[float]) -> np.ndarray:
    return s if not soft_cap else soft_cap * np.tanh(s / soft_cap)


def attention_dense_masked(q, k, v, layout, bs: int, scale: float, *, sink=None,
                           soft_cap: Optional[float] = None, causal: bool = False,
                           q_segment_ids=None, kv_segment_ids=None
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
    mask = token_mask(layout, bs, Sq, Sk)
    if mask.shape != (H, Sq, Sk):
        raise ValueError("layout does not match q/k shapes")
    if causal:
        mask = mask & (np.arange(Sk)[None, None, :] <= np.arange(Sq)[None, :, None])
    s = _cap(scale * np.matmul(q, np.swapaxes(k, -1, -2)), soft_cap)
    seg = _segments(q_segment_ids, kv_segment_ids, B, Sq, Sk)
    full = mask[None] if seg is None else mask[None] & seg[:, None]
    s = np.where(full, s, -np.inf)
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
                         sink=None, soft_cap: Optional[float] = None, causal: bool = False,
                         q_segment_ids=None, kv_segment_ids=None
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
    Sk = k.shape[2]
    Mb = _nblocks(Sq, bs)
    if lay.shape[0] != H or lay.shape[1] != Mb or lay.shape[2] != _nblocks(Sk, bs):
        raise ValueError("layout does not match q/k shapes")
    sk = None if sink is None else _as64(sink)
    seg = _segments(q_segment_ids, kv_segment_ids, B, Sq, Sk)
    out = np.full((B, H, Sq, v.shape[3]), np.nan)
    lse = np.full((B, H, Sq), np.nan)
    if row_blocks is None:
        row_blocks = [(b, h, m) for b in range(B) for h in range(H) for m in range(Mb)]
    offs = np.arange(bs)
    for (b, h, m) in row_blocks:
        rows = slice(m * bs, min((m + 1) * bs, Sq))
        nr = rows.stop - rows.start
        cols = np.flatnonzero(lay[h, m])
        tok = (cols[:, None] * bs + offs[None, :]).reshape(-1)
        tok = tok[tok < Sk]                                   # the last key block may be cut
        s = _cap(scale * (q[b, h, rows] @ k[b, kvh(h), tok].T), soft_cap)   # [nr, T]
        if causal:
            qpos = m * bs + offs[:nr]
            s = np.where(tok[None, :] <= qpos[:, None], s, -np.inf)
        if seg is not None:
            s = np.where(seg[b][rows][:, tok], s, -np.inf)
        mx = s.max(axis=1) if tok.size else np.full(nr, -np.inf)
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
# Backward: gradients of the block-sparse forward
# --------------------------------------------------------------------------
#
# The next.gr tutorial ("Gradient Propagation in Block Sparse Attention", and
# the block-structured Jacobian under "Mathematical Formulation") fixes only
# that gradients flow through the live blocks of the pattern: the gradient of
# query block i sums over the blocks attending to it, and the Jacobian of an
# output row with respect to an input row is zero outside the row's
# neighbourhood.  The pages print no formula for the softmax step, so the
# oracle is the chain rule of the forward definition above written out.  With
# c_ij the (capped) scaled score, Z_i = sum_j exp(c_ij) + exp(sink_h),
# P_ij = exp(c_ij) / Z_i and out_i = sum_j P_ij v_j, an upstream gradient dO
# gives
#   dv_j    = sum_i P_ij dO_i
#   dP_ij   = dO_i . v_j,      D_i = sum_j P_ij dP_ij = dO_i . out_i
#   dc_ij   = P_ij (dP_ij - D_i)
#   ds_ij   = dc_ij (1 - tanh^2(s_ij / cap))      (dc_ij without a cap)
#   dq_i    = scale sum_j ds_ij k_j,   dk_j = scale sum_i ds_ij q_i
#   dsink_h = -sum_i exp(sink_h) / Z_i * D_i       (over every batch item and row)
# with masked entries contributing nothing (P_ij = 0 there) and, under grouped
# heads, dk and dv of a K/V head summed over the query heads that read it.


@dataclass
class PlanColsRef:
    """Per-column CSR (the transposed plan) of a block layout, for the
    backward's key-block work items.

    Column c = h * Nb + n.  ``col_ptr[c]:col_ptr[c+1]`` delimits the query
    blocks m with (h, m, n) live, ascending, in ``row_idx``.  ``col_order``
    lists the key-block work items w = kvh * Nb + n (one per K/V head and key
    block), K/V head by K/V head, and inside each K/V head by the number of
    live tiles the item visits -- summed over the query heads of its group --
    descending, ties by n ascending.
    """

    H: int
    Hkv: int
    Mb: int
    Nb: int
    col_ptr: np.ndarray    # int32 [H*Nb+1]
    row_idx: np.ndarray    # int32 [nnz_total]
    col_order: np.ndarray  # int32 [Hkv*Nb]
    nnz_total: int


def plan_columns(layout: np.ndarray, kv_heads: Optional[int] = None) -> PlanColsRef:
    """Transposed CSR of a block layout [H, Mb, Nb] and the order of the
    backward's key-block work items (see PlanColsRef)."""
    lay = np.asarray(layout)
    if lay.ndim != 3:
        raise ValueError("layout must be [H, Mb, Nb]")
    H, Mb, Nb = lay.shape
    Hkv = H if kv_heads is None else kv_heads
    if Hkv <= 0 or H % Hkv:
        raise ValueError("kv_heads must divide H")
    g = H // Hkv
    live_t = np.swapaxes(lay != 0, 1, 2)                     # [H, Nb, Mb]
    cnt = live_t.reshape(H * Nb, Mb).sum(axis=1).astype(np.int64)
    col_ptr = np.zeros(H * Nb + 1, dtype=np.int64)
    col_ptr[1:] = np.cumsum(cnt)
    _, rows = np.nonzero(live_t.reshape(H * Nb, Mb))         # m ascending per column
    order = []
    for kvh in range(Hkv):
        work = cnt.reshape(H, Nb)[kvh * g:(kvh + 1) * g].sum(axis=0)
        n = np.arange(Nb)
        order.append(kvh * Nb + np.lexsort((n, -work)))
    col_order = np.concatenate(order) if order else np.zeros(0, np.int64)
    return PlanColsRef(H=H, Hkv=Hkv, Mb=Mb, Nb=Nb, col_ptr=col_ptr.astype(np.int32),
                       row_idx=rows.astype(np.int32), col_order=col_order.astype(np.int32),
                       nnz_total=int(col_ptr[-1]))


def _cap_slope(s: np.ndarray, soft_cap: Optional[float]) -> np.ndarray:
    """d cap(s) / d s = 1 - tanh^2(s / cap) (1 without a cap)."""
    if not soft_cap:
        return np.ones_like(s)
    t = np.tanh(s / soft_cap)
    return 1.0 - t * t


def attention_backward_dense(q, k, v, dout, layout, bs: int, scale: float, *, sink=None,
                             soft_cap: Optional[float] = None, causal: bool = False,
                             q_segment_ids=None, kv_segment_ids=None):
    """Gradients of attention_dense_masked's ``out`` for the upstream gradient
    ``dout`` [B, H, Sq, d]: returns dq [B, H, Sq, d], dk and dv [B, Hkv, Sk, d],
    and dsink [H] (None without a sink).  Dense S x S form of the formulas
    above; the options mean what they mean in the forward."""
    q, k, v, dout = _as64(q), _as64(k), _as64(v), _as64(dout)
    B, H, Sq, d = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    kvh = _kv_head(H, Hkv)
    heads = [kvh(h) for h in range(H)]
    kx, vx = k[:, heads], v[:, heads]                        # per query head
    mask = token_mask(layout, bs, Sq, Sk)
    if mask.shape != (H, Sq, Sk):
        raise ValueError("layout does not match q/k shapes")
    if causal:
        mask = mask & (np.arange(Sk)[None, None, :] <= np.arange(Sq)[None, :, None])
    seg = _segments(q_segment_ids, kv_segment_ids, B, Sq, Sk)
    mask = mask[None] if seg is None else mask[None] & seg[:, None]    # [B or 1, H, Sq, Sk]
    s = scale * np.matmul(q, np.swapaxes(kx, -1, -2))        # scaled, uncapped
    out, lse = attention_dense_masked(q, k, v, layout, bs, scale, sink=sink,
                                      soft_cap=soft_cap, causal=causal,
                                      q_segment_ids=q_segment_ids, kv_segment_ids=kv_segment_ids)
    live_row = np.isfinite(lse)[..., None]
    c = np.where(mask, _cap(s, soft_cap), -np.inf)
    with np.errstate(invalid="ignore"):
        p = np.where(live_row & mask, np.exp(c - np.where(live_row, lse[..., None], 0.0)), 0.0)
    dv_x = np.matmul(np.swapaxes(p, -1, -2), dout)           # [B, H, Sk, d]
    dp = np.matmul(dout, np.swapaxes(vx, -1, -2))            # [B, H, Sq, Sk]
    D = (dout * out).sum(axis=-1, keepdims=True)             # [B, H, Sq, 1]
    ds = p * (dp - D) * _cap_slope(s, soft_cap)
    dq = scale * np.matmul(ds, kx)
    dk_x = scale * np.matmul(np.swapaxes(ds, -1, -2), q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(H):
        dk[:, heads[h]] += dk_x[:, h]
        dv[:, heads[h]] += dv_x[:, h]
    dsink = None
    if sink is not None:
        sk = _as64(sink)
        with np.errstate(invalid="ignore"):
            w = np.where(np.isfinite(lse), np.exp(sk[None, :, None] - np.where(np.isfinite(lse), lse, 0.0)), 0.0)
        dsink = -(w * D[..., 0]).sum(axis=(0, 2))
    return dq, dk, dv, dsink


def attention_backward_live_tiles(q, k, v, dout, layout, bs: int, scale: float, *,
                                  row_blocks=None, col_blocks=None, sink=None,
                                  soft_cap: Optional[float] = None, causal: bool = False,
                                  q_segment_ids=None, kv_segment_ids=None):
    """The same gradients over live tiles only, for sampled blocks.

    ``row_blocks`` lists (b, h, m) query blocks whose dq rows are computed;
    ``col_blocks`` lists (b, kvh, n) key blocks whose dk and dv rows are
    computed (summing the query heads of the K/V head's group).  Entries not
    computed are NaN.  dsink is returned only when both lists are None (then
    every block is computed).  Each needed query row's out and lse come from
    attention_live_tiles.
    """
    q, k, v, dout = _as64(q), _as64(k), _as64(v), _as64(dout)
    B, H, Sq, d = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    kvh = _kv_head(H, Hkv)
    g = H // Hkv
    lay = np.asarray(layout) != 0
    Mb, Nb = _nblocks(Sq, bs), _nblocks(Sk, bs)
    if lay.shape != (H, Mb, Nb):
        raise ValueError("layout does not match q/k shapes")
    full = row_blocks is None and col_blocks is None
    if row_blocks is None:
        row_blocks = [(b, h, m) for b in range(B) for h in range(H) for m in range(Mb)]
    if col_blocks is None:
        col_blocks = [(b, j, n) for b in range(B) for j in range(Hkv) for n in range(Nb)]
    need = set(row_blocks)
    for (b, j, n) in col_blocks:
        for h in range(j * g, (j + 1) * g):
            need.update((b, h, int(m)) for m in np.flatnonzero(lay[h, :, n]))
    need = sorted(need)
    out, lse = attention_live_tiles(q, k, v, layout, bs, scale, row_blocks=need, sink=sink,
                                    soft_cap=soft_cap, causal=causal,
                                    q_segment_ids=q_segment_ids, kv_segment_ids=kv_segment_ids)
    seg = _segments(q_segment_ids, kv_segment_ids, B, Sq, Sk)
    D = (dout * out).sum(axis=-1)                            # NaN where not computed

    def rows_of(m):
        return slice(m * bs, min((m + 1) * bs, Sq))

    def keys_of(n):
        return slice(n * bs, min((n + 1) * bs, Sk))

    def tile_terms(b, h, m, n):
        """P, dS of tile (m, n) of head h: [queries, keys] of the tile (the
        last block row / column may be cut short)."""
        rows, keys = rows_of(m), keys_of(n)
        s = scale * (q[b, h, rows] @ k[b, kvh(h), keys].T)
        c = _cap(s, soft_cap)
        if causal:
            qpos = np.arange(rows.start, rows.stop)
            kpos = np.arange(keys.start, keys.stop)
            c = np.where(kpos[None, :] <= qpos[:, None], c, -np.inf)
        if seg is not None:
            c = np.where(seg[b][rows, keys], c, -np.inf)
        lr = lse[b, h, rows][:, None]
        live = np.isfinite(lr)
        with np.errstate(invalid="ignore"):
            p = np.where(live, np.exp(c - np.where(live, lr, 0.0)), 0.0)
        dp = dout[b, h, rows] @ v[b, kvh(h), keys].T
        ds = p * (dp - D[b, h, rows][:, None]) * _cap_slope(s, soft_cap)
        return p, ds

    dq = np.full(q.shape, np.nan)
    for (b, h, m) in row_blocks:
        rows = rows_of(m)
        acc = np.zeros((rows.stop - rows.start, d))
        for n in np.flatnonzero(lay[h, m]):
            _, ds = tile_terms(b, h, m, int(n))
            acc += scale * ds @ k[b, kvh(h), keys_of(int(n))]
        dq[b, h, rows] = acc
    dk = np.full(k.shape, np.nan)
    dv = np.full(v.shape, np.nan)
    for (b, j, n) in col_blocks:
        keys = keys_of(n)
        ak = np.zeros((keys.stop - keys.start, d))
        av = np.zeros((keys.stop - keys.start, v.shape[3]))
        for h in range(j * g, (j + 1) * g):
            for m in np.flatnonzero(lay[h, :, n]):
                p, ds = tile_terms(b, h, int(m), n)
                rows = rows_of(int(m))
                av += p.T @ dout[b, h, rows]
                ak += scale * ds.T @ q[b, h, rows]
        dk[b, j, keys] = ak
        dv[b, j, keys] = av
    dsink = None
    if full and sink is not None:
        sk = _as64(sink)
        with np.errstate(invalid="ignore"):
            w = np.where(np.isfinite(lse), np.exp(sk[None, :, None] - np.where(np.isfinite(lse), lse, 0.0)), 0.0)
        dsink = -(w * D).sum(axis=(0, 2))
    return dq, dk, dv, dsink


# --------------------------------------------------------------------------
# Content-adaptive block layout
# --------------------------------------------------------------------------

def adaptive_layout(q, k, bs: int, tau: float, *, causal: bool = False,
                    keep_diagonal: bool = True):
    """Block layout chosen from the content of q and k.

    The next.gr tutorial ("Fixed vs. Adaptive Block Sparsity") marks a pair
    live when sim(Q_i, K_j) >= tau, naming cosine similarity as the metric;
    the Language AI Handbook ("Block Structure" discussion of choosing which
    blocks to attend) scores the candidates at a coarser granularity than
    tokens.  Reading used here: Q_i and K_j are the mean of the query rows of
    block i and of the key rows of block j (mean pooling over the block's
    tokens), sim is their cosine similarity (0 when either mean is the zero
    vector), and a block pair is live when sim >= tau.  With ``causal`` only
    pairs with j <= i may be live; with ``keep_diagonal`` the pairs j == i
    are always live, so that every block row keeps a tile.

    q: [H, Sq, d], k: [Hkv, Sk, d] (one batch item; query head h reads K/V
    head h // (H / Hkv)).  Returns (layout int32 [H, Sq/bs, Sk/bs], sim).
    """
    q, k = _as64(q), _as64(k)
    H, Sq, d = q.shape
    Hkv, Sk, _ = k.shape
    kvh = _kv_head(H, Hkv)
    Mb, Nb = Sq // bs, Sk // bs
    if Mb * bs != Sq or Nb * bs != Sk:
        raise ValueError("sequence lengths must be multiples of the block size")
    qbar = q.reshape(H, Mb, bs, d).mean(axis=2)
    kbar = k.reshape(Hkv, Nb, bs, d).mean(axis=2)

    def unit(x):
        nrm = np.linalg.norm(x, axis=-1, keepdims=True)
        return np.where(nrm > 0, x / np.where(nrm > 0, nrm, 1.0), 0.0)

    qh, kh = unit(qbar), unit(kbar)
    sim = np.stack([qh[h] @ kh[kvh(h)].T for h in range(H)])        # [H, Mb, Nb]
    live = sim >= tau
    m = np.arange(Mb)[:, None]
    n = np.arange(Nb)[None, :]
    if causal:
        live &= (n <= m)[None]
    if keep_diagonal:
        live |= (n == m)[None]
    return live.astype(np.int32), sim


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
