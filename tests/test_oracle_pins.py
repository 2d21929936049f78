"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each test checks the oracle through a route that does not repeat its own
code: a library routine (torch's scaled_dot_product_attention, softmax,
logsumexp), a closed form, an invariant, a printed number, or element-by-
element brute force with Python floats.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import bsa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")


def rnd(shape, seed, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


def token_mask_by_lookup(layout, bs):
    """Token mask built by index lookup (i // bs, j // bs), independent of the
    oracle's repeat-based expansion."""
    H, Mb, Nb = layout.shape
    mask = np.zeros((H, Mb * bs, Nb * bs), dtype=bool)
    for h in range(H):
        for i in range(Mb * bs):
            for j in range(Nb * bs):
                mask[h, i, j] = layout[h, i // bs, j // bs] != 0
    return mask


# ---------------------------------------------------------------- block sparse

def test_all_ones_layout_is_dense_attention():
    """All tiles live: the method reduces to dense scaled dot-product
    attention (next.gr tutorial, section 1)."""
    B, H, S, d, bs, scale = 2, 3, 48, 8, 16, 0.37
    q, k, v = rnd((B, H, S, d), 1), rnd((B, H, S, d), 2), rnd((B, H, S, d), 3)
    lay = np.ones((H, S // bs, S // bs), np.int32)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale).numpy()
    ref_lse = torch.logsumexp(scale * tq @ tk.transpose(-1, -2), dim=-1).numpy()
    for fn in (O.attention_dense_masked, O.attention_live_tiles):
        out, lse = fn(q, k, v, lay, bs, scale)
        assert np.abs(out - ref).max() < 1e-12
        assert np.abs(lse - ref_lse).max() < 1e-12


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_masked_layout_matches_sdpa_with_boolean_mask(seed):
    """-inf outside the pattern before one row-wide softmax (next.gr,
    Longformer formula): torch's SDPA with a boolean mask computes exactly
    that.  Every block row keeps at least one live tile here."""
    rng = np.random.default_rng(100 + seed)
    B, H, bs, d, Mb, Nb = 1, 2, 8, 4, 4, 6
    lay = (rng.random((H, Mb, Nb)) < 0.4).astype(np.int32)
    lay[:, np.arange(Mb), rng.integers(0, Nb, Mb)] = 1
    q, k, v = rnd((B, H, Mb * bs, d), seed), rnd((B, H, Nb * bs, d), seed + 10), rnd((B, H, Nb * bs, d), seed + 20)
    mask = torch.from_numpy(token_mask_by_lookup(lay, bs))
    scale = 0.5
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask[None], scale=scale)
    s = (scale * tq @ tk.transpose(-1, -2)).masked_fill(~mask[None], -math.inf)
    ref_lse = torch.logsumexp(s, dim=-1)
    for fn in (O.attention_dense_masked, O.attention_live_tiles):
        out, lse = fn(q, k, v, lay, bs, scale)
        assert np.abs(out - ref.numpy()).max() < 1e-12
        assert np.abs(lse - ref_lse.numpy()).max() < 1e-12


def test_softmax_rows_sum_to_one_and_masked_weights_are_zero():
    """With V = identity the output row is the softmax row itself: it sums to
    one (next.gr, section 1) and is exactly zero on masked keys."""
    H, bs, Mb, Nb = 2, 4, 3, 5
    rng = np.random.default_rng(7)
    lay = (rng.random((H, Mb, Nb)) < 0.5).astype(np.int32)
    lay[:, :, 0] = 1
    S, Sk = Mb * bs, Nb * bs
    q, k = rnd((1, H, S, 6), 8), rnd((1, H, Sk, 6), 9)
    v = np.broadcast_to(np.eye(Sk), (1, H, Sk, Sk)).copy()
    mask = token_mask_by_lookup(lay, bs)
    for fn in (O.attention_dense_masked, O.attention_live_tiles):
        p, _ = fn(q, k, v, lay, bs, 0.8)
        assert np.all(p >= 0)
        assert np.abs(p.sum(-1) - 1).max() < 1e-12
        assert np.all(p[0][~mask] == 0)


def test_empty_block_row_gives_zero_output_and_neg_inf_lse():
    """A row with no live block: all-zero output (the finite-floor
    convention of the DeepSeek kernel) and lse = -inf."""
    H, bs, Mb = 2, 8, 4
    lay = np.ones((H, Mb, Mb), np.int32)
    lay[0, 2, :] = 0
    lay[1] = 0
    q, k, v = rnd((1, H, Mb * bs, 4), 1), rnd((1, H, Mb * bs, 4), 2), rnd((1, H, Mb * bs, 4), 3)
    for fn in (O.attention_dense_masked, O.attention_live_tiles):
        out, lse = fn(q, k, v, lay, bs, 0.5)
        assert np.all(out[0, 0, 2 * bs:3 * bs] == 0) and np.all(np.isneginf(lse[0, 0, 2 * bs:3 * bs]))
        assert np.all(out[0, 1] == 0) and np.all(np.isneginf(lse[0, 1]))
        assert np.all(np.isfinite(out)) and np.isfinite(lse[0, 0, :2 * bs]).all()


def test_zero_query_gives_mean_of_live_values():
    """Closed form: q = 0 makes every live score 0, so the output is the mean
    of v over the live key tokens and lse = ln(number of live keys)."""
    H, bs, Mb, Nb, d = 3, 4, 5, 6, 3
    rng = np.random.default_rng(3)
    lay = (rng.random((H, Mb, Nb)) < 0.5).astype(np.int32)
    lay[:, :, 1] = 1
    q = np.zeros((2, H, Mb * bs, d))
    k, v = rnd((2, H, Nb * bs, d), 4), rnd((2, H, Nb * bs, d), 5)
    for fn in (O.attention_dense_masked, O.attention_live_tiles):
        out, lse = fn(q, k, v, lay, bs, 0.9)
        for b in range(2):
            for h in range(H):
                for m in range(Mb):
                    cols = [n for n in range(Nb) if lay[h, m, n]]
                    vv = np.concatenate([v[b, h, n * bs:(n + 1) * bs] for n in cols])
                    rows = slice(m * bs, (m + 1) * bs)
                    assert np.abs(out[b, h, rows] - vv.mean(0)).max() < 1e-12
                    assert np.abs(lse[b, h, rows] - math.log(len(cols) * bs)).max() < 1e-12


def test_block_diagonal_is_independent_dense_attention_per_block():
    """Block-diagonal layout (next.gr section 3.2; Language AI Handbook
    'diagonal' pattern): each block attends only to itself."""
    H, bs, nb, d = 2, 8, 4, 5
    lay = np.broadcast_to(np.eye(nb, dtype=np.int32), (H, nb, nb)).copy()
    q, k, v = rnd((1, H, nb * bs, d), 11), rnd((1, H, nb * bs, d), 12), rnd((1, H, nb * bs, d), 13)
    out, _ = O.attention_live_tiles(q, k, v, lay, bs, 0.4)
    for m in range(nb):
        sl = slice(m * bs, (m + 1) * bs)
        ref = torch.nn.functional.scaled_dot_product_attention(
            *(torch.from_numpy(x[:, :, sl]) for x in (q, k, v)), scale=0.4).numpy()
        assert np.abs(out[:, :, sl] - ref).max() < 1e-12


def brute_force_bsa(q, k, v, lay, bs, scale):
    """Element-by-element definition with Python floats."""
    B, H, S, d = q.shape
    Sk = k.shape[2]
    out = [[[[0.0] * d for _ in range(S)] for _ in range(H)] for _ in range(B)]
    lse = [[[0.0] * S for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            for i in range(S):
                live = [j for j in range(Sk) if lay[h][i // bs][j // bs]]
                if not live:
                    lse[b][h][i] = -math.inf
                    continue
                s = {}
                for j in live:
                    acc = 0.0
                    for t in range(d):
                        acc += float(q[b, h, i, t]) * float(k[b, h, j, t])
                    s[j] = scale * acc
                mx = max(s.values())
                den = sum(math.exp(s[j] - mx) for j in live)
                for t in range(d):
                    out[b][h][i][t] = sum(math.exp(s[j] - mx) * float(v[b, h, j, t]) for j in live) / den
                lse[b][h][i] = mx + math.log(den)
    return np.array(out), np.array(lse)


@pytest.mark.parametrize("seed", [0, 1])
def test_brute_force_tiny(seed):
    rng = np.random.default_rng(seed)
    B, H, S, bs, d = 1, 2, 32, 8, 4
    lay = (rng.random((H, S // bs, S // bs)) < 0.45).astype(np.int32)
    lay[0, 1, :] = 0  # one empty block row
    q, k, v = rnd((B, H, S, d), seed + 1), rnd((B, H, S, d), seed + 2), rnd((B, H, S, d), seed + 3)
    ref_out, ref_lse = brute_force_bsa(q, k, v, lay, bs, 0.6)
    for fn in (O.attention_dense_masked, O.attention_live_tiles):
        out, lse = fn(q, k, v, lay, bs, 0.6)
        assert np.abs(out - ref_out).max() < 1e-12
        fin = np.isfinite(ref_lse)
        assert np.array_equal(fin, np.isfinite(lse))
        assert np.abs(lse[fin] - ref_lse[fin]).max() < 1e-12


@pytest.mark.parametrize("seed", range(4))
def test_live_tile_mode_equals_dense_masked_mode(seed):
    rng = np.random.default_rng(50 + seed)
    H, bs, Mb, Nb, d = 3, 8, 5, 7, 6
    lay = (rng.random((H, Mb, Nb)) < 0.3).astype(np.int32)
    q, k, v = rnd((2, H, Mb * bs, d), seed), rnd((2, H, Nb * bs, d), seed + 5), rnd((2, H, Nb * bs, d), seed + 9)
    o1, l1 = O.attention_dense_masked(q, k, v, lay, bs, 0.3)
    o2, l2 = O.attention_live_tiles(q, k, v, lay, bs, 0.3)
    assert np.abs(o1 - o2).max() < 1e-12
    assert np.array_equal(np.isneginf(l1), np.isneginf(l2))
    fin = np.isfinite(l1)
    assert np.abs(l1[fin] - l2[fin]).max() < 1e-12


def test_live_tile_mode_row_subset():
    rng = np.random.default_rng(5)
    H, bs, nb, d = 2, 8, 4, 4
    lay = (rng.random((H, nb, nb)) < 0.5).astype(np.int32)
    q, k, v = rnd((1, H, nb * bs, d), 1), rnd((1, H, nb * bs, d), 2), rnd((1, H, nb * bs, d), 3)
    full, full_lse = O.attention_live_tiles(q, k, v, lay, bs, 0.5)
    part, part_lse = O.attention_live_tiles(q, k, v, lay, bs, 0.5, row_blocks=[(0, 1, 2)])
    sl = slice(2 * bs, 3 * bs)
    assert np.array_equal(part[0, 1, sl], full[0, 1, sl])
    assert np.isnan(part[0, 0]).all()


# ---------------------------------------------------------------------- top-k

def test_topk_equals_block_sparse_on_live_tile_indices():
    """Cross-variant identity: top-k over exactly the tokens of a query's live
    tiles (rows shared by all heads, no sink) equals block-sparse attention
    with k = v = kv for every head."""
    rng = np.random.default_rng(21)
    B, H, S, bs, d = 2, 3, 64, 16, 8
    nb = S // bs
    one = (rng.random((nb, nb)) < 0.5).astype(np.int32)
    one[np.arange(nb), np.arange(nb)] = 1
    lay = np.broadcast_to(one, (H, nb, nb)).copy()
    kv = rnd((B, S, d), 22)
    qbs = rnd((B, H, S, d), 23)
    kk = np.broadcast_to(kv[:, None], (B, H, S, d)).copy()
    ref, _ = O.attention_live_tiles(qbs, kk, kk, lay, bs, 0.45)
    topk = nb * bs
    idx = -np.ones((B, S, topk), dtype=np.int64)
    for b in range(B):
        for i in range(S):
            toks = [j for j in range(S) if one[i // bs, j // bs]]
            perm = rng.permutation(len(toks))
            idx[b, i, :len(toks)] = np.array(toks)[perm]
    qtk = np.transpose(qbs, (0, 2, 1, 3))
    out = O.topk_attention(qtk, kv, idx, None, 0.45)
    assert np.abs(np.transpose(out, (0, 2, 1, 3)) - ref).max() < 1e-12


def test_topk_zero_query_closed_form_with_unscaled_sink():
    """q = 0: every score is 0 regardless of scale, so out = sum of the
    gathered rows / (T + exp(sink_h)); the sink enters unscaled."""
    B, M, H, d, N = 1, 3, 4, 5, 9
    kv = rnd((B, N, d), 1)
    sink = np.array([-1.0, 0.0, 0.7, 2.5])
    idx = np.array([[[0, 3, 3, -1, 8], [-1, -1, -1, -1, -1], [2, 5, 1, 7, 4]]])
    q = np.zeros((B, M, H, d))
    out = O.topk_attention(q, kv, idx, sink, scale=0.25)
    for m in range(M):
        sel = [t for t in idx[0, m] if t != -1]
        for h in range(H):
            exp = sum(kv[0, t] for t in sel) / (len(sel) + math.exp(sink[h])) if sel else np.zeros(d)
            assert np.abs(out[0, m, h] - exp).max() < 1e-12


def test_topk_all_invalid_slots_give_zero():
    q, kv = rnd((1, 2, 3, 4), 1), rnd((1, 6, 4), 2)
    idx = -np.ones((1, 2, 5), dtype=np.int64)
    for sink in (None, np.array([0.5, -2.0, 9.0])):
        out = O.topk_attention(q, kv, idx, sink, 0.5)
        assert np.all(out == 0)


def test_topk_without_sink_is_softmax_of_gathered_rows():
    """No sink: plain softmax over the gathered rows (torch.softmax), and a
    sink of -inf or a huge negative sink changes nothing."""
    B, M, H, d, N = 1, 2, 3, 6, 10
    q, kv = rnd((B, M, H, d), 3), rnd((B, N, d), 4)
    idx = np.array([[[1, 4, 9, -1, 2], [0, -1, 7, 5, 3]]])
    out = O.topk_attention(q, kv, idx, None, 0.4)
    for m in range(M):
        sel = [t for t in idx[0, m] if t != -1]
        rows = torch.from_numpy(kv[0, sel])
        w = torch.softmax(0.4 * torch.from_numpy(q[0, m]) @ rows.T, dim=-1)
        assert np.abs(out[0, m] - (w @ rows).numpy()).max() < 1e-12
    for s in (np.full(H, -np.inf), np.full(H, -1e300)):
        assert np.abs(O.topk_attention(q, kv, idx, s, 0.4) - out).max() < 1e-12


def test_topk_sink_only_lowers_total_weight():
    """With kv = identity rows the output is the weight vector: the sink
    leaves a total real weight strictly between 0 and 1 that falls as the
    sink grows, and a huge sink drives the output to zero."""
    N = d = 6
    kv = np.eye(N)[None]
    q = rnd((1, 1, 2, d), 5)
    idx = np.array([[[0, 1, 2, 3, 4, 5]]])
    prev = None
    for sv in (-3.0, 0.0, 1.0, 4.0):
        w = O.topk_attention(q, kv, idx, np.array([sv, sv]), 0.7)[0, 0]
        tot = w.sum(-1)
        assert np.all(tot > 0) and np.all(tot < 1)
        if prev is not None:
            assert np.all(tot < prev)
        prev = tot
    w = O.topk_attention(q, kv, idx, np.array([1e4, 1e4]), 0.7)
    assert np.abs(w).max() == 0.0


def test_topk_duplicates_count_twice_and_order_is_irrelevant():
    B, M, H, d, N = 1, 1, 2, 4, 8
    q, kv = rnd((B, M, H, d), 6), rnd((B, N, d), 7)
    sink = np.array([0.3, -0.4])
    a = O.topk_attention(q, kv, np.array([[[2, 5, 5, 1]]]), sink, 0.5)
    b = O.topk_attention(q, kv, np.array([[[5, 1, 2, 5]]]), sink, 0.5)
    assert np.abs(a - b).max() < 1e-14
    # duplicate == doubled weight of that row: q=0 closed form
    z = O.topk_attention(np.zeros_like(q), kv, np.array([[[3, 3, 6]]]), sink, 0.5)
    for h in range(H):
        exp = (2 * kv[0, 3] + kv[0, 6]) / (3 + math.exp(sink[h]))
        assert np.abs(z[0, 0, h] - exp).max() < 1e-12


def brute_force_topk(q, kv, idx, sink, scale):
    B, M, H, d = q.shape
    out = np.zeros((B, M, H, d))
    for b in range(B):
        for m in range(M):
            sel = [int(t) for t in idx[b, m] if t != -1]
            for h in range(H):
                s = [scale * sum(float(q[b, m, h, c]) * float(kv[b, t, c]) for c in range(d)) for t in sel]
                terms = s + ([float(sink[h])] if sink is not None else [])
                if not terms:
                    continue
                mx = max(terms)
                den = sum(math.exp(x - mx) for x in terms)
                for c in range(d):
                    out[b, m, h, c] = sum(math.exp(s[i] - mx) * float(kv[b, t, c]) for i, t in enumerate(sel)) / den
    return out


@pytest.mark.parametrize("with_sink", [True, False])
def test_topk_brute_force_tiny(with_sink):
    rng = np.random.default_rng(11)
    B, M, H, d, N, topk = 2, 3, 3, 4, 12, 7
    q, kv = rnd((B, M, H, d), 1), rnd((B, N, d), 2)
    idx = np.stack([np.stack([rng.choice(N, topk, replace=False) for _ in range(M)]) for _ in range(B)])
    idx[rng.random(idx.shape) < 0.3] = -1
    idx[1, 2] = -1
    sink = rnd((H,), 3) if with_sink else None
    assert np.abs(O.topk_attention(q, kv, idx, sink, 0.35) - brute_force_topk(q, kv, idx, sink, 0.35)).max() < 1e-12


def test_topk_rejects_out_of_range_indices():
    q, kv = rnd((1, 1, 1, 2), 1), rnd((1, 4, 2), 2)
    for bad in (-2, 4):
        with pytest.raises(ValueError):
            O.topk_attention(q, kv, np.array([[[0, bad]]]), None, 1.0)


# ----------------------------------------------------------------------- plan

def brute_force_plan(lay):
    H, Mb, Nb = lay.shape
    row_ptr, cols, nnz = [0], [], []
    for h in range(H):
        for m in range(Mb):
            c = [n for n in range(Nb) if lay[h][m][n] != 0]
            cols += c
            nnz.append(len(c))
            row_ptr.append(row_ptr[-1] + len(c))
    order = []
    for h in range(H):
        rows = list(range(Mb))
        # selection by repeated maximum: heaviest remaining row, lowest m first
        while rows:
            best = rows[0]
            for m in rows[1:]:
                if nnz[h * Mb + m] > nnz[h * Mb + best]:
                    best = m
            rows.remove(best)
            order.append(h * Mb + best)
    return row_ptr, cols, order


@pytest.mark.parametrize("seed", range(6))
def test_plan_matches_brute_force_and_invariants(seed):
    rng = np.random.default_rng(seed)
    H, Mb, Nb = int(rng.integers(1, 4)), int(rng.integers(1, 9)), int(rng.integers(1, 70))
    lay = (rng.random((H, Mb, Nb)) < rng.random()).astype(np.int32) * rng.integers(1, 5, (H, Mb, Nb))
    if seed == 0:
        lay[:] = 0
    p = O.plan(lay)
    rp, cols, order = brute_force_plan(lay)
    assert p.row_ptr.tolist() == rp and p.col_idx.tolist() == cols and p.row_order.tolist() == order
    assert p.nnz_total == int((lay != 0).sum())
    assert p.row_ptr.dtype == np.int32 and p.col_idx.dtype == np.int32 and p.row_order.dtype == np.int32
    # CSR round trip reproduces the live set exactly
    back = np.zeros((H * Mb, Nb), bool)
    for r in range(H * Mb):
        c = p.col_idx[p.row_ptr[r]:p.row_ptr[r + 1]]
        assert np.all(np.diff(c) > 0)
        back[r, c] = True
    assert np.array_equal(back.reshape(H, Mb, Nb), lay != 0)
    # order: a permutation, head-major, nnz non-increasing, ties by m
    assert sorted(p.row_order.tolist()) == list(range(H * Mb))
    nnz = np.diff(p.row_ptr)
    for h in range(H):
        seg = p.row_order[h * Mb:(h + 1) * Mb]
        assert np.all(seg // Mb == h)
        key = [(-nnz[r], r % Mb) for r in seg]
        assert key == sorted(key)


def brute_force_pairs(lay):
    """Pair plan from the brute-force row lists: a two-pointer merge of the
    sorted column lists of rows 2p and 2p+1, the order by repeated selection
    of the largest union."""
    H, Mb, Nb = lay.shape
    rp, cols, _ = brute_force_plan(lay)
    row = lambda h, m: cols[rp[h * Mb + m]:rp[h * Mb + m + 1]]  # noqa: E731
    Mp = (Mb + 1) // 2
    ptr, out, cnt = [0], [], []
    for h in range(H):
        for p in range(Mp):
            a = row(h, 2 * p)
            b = row(h, 2 * p + 1) if 2 * p + 1 < Mb else []
            i = j = 0
            merged = []
            while i < len(a) or j < len(b):
                if j == len(b) or (i < len(a) and a[i] < b[j]):
                    merged.append(a[i] | (1 << 24))
                    i += 1
                elif i == len(a) or b[j] < a[i]:
                    merged.append(b[j] | (2 << 24))
                    j += 1
                else:
                    merged.append(a[i] | (3 << 24))
                    i += 1
                    j += 1
            out += merged
            cnt.append(len(merged))
            ptr.append(ptr[-1] + len(merged))
    order = []
    for h in range(H):
        left = list(range(Mp))
        while left:
            best = left[0]
            for p in left[1:]:
                if cnt[h * Mp + p] > cnt[h * Mp + best]:
                    best = p
            left.remove(best)
            order.append(h * Mp + best)
    return ptr, out, order


@pytest.mark.parametrize("seed", range(8))
def test_plan_pairs_matches_brute_force_and_round_trips(seed):
    rng = np.random.default_rng(100 + seed)
    H, Mb, Nb = int(rng.integers(1, 4)), int(rng.integers(1, 10)), int(rng.integers(1, 70))
    lay = (rng.random((H, Mb, Nb)) < rng.random()).astype(np.int32) * rng.integers(1, 5, (H, Mb, Nb))
    if seed == 0:
        lay[:] = 0
    if seed == 1:  # rows 2p+1 copy rows 2p: every shared column carries mask 3
        lay[:, 1::2] = lay[:, 0:Mb - Mb % 2:2]
    pp = O.plan_pairs(lay)
    ptr, cols, order = brute_force_pairs(lay)
    assert pp.pair_ptr.tolist() == ptr and pp.pair_cols.tolist() == cols
    assert pp.pair_order.tolist() == order
    assert pp.pair_total == len(cols)
    nnz = int((lay != 0).sum())
    assert pp.use_pairs == int(4 * len(cols) <= 3 * nnz)
    assert pp.pair_ptr.dtype == np.int32 and pp.pair_cols.dtype == np.int32
    # decoding the pairs gives back the live set exactly
    Mp = (Mb + 1) // 2
    back = np.zeros((H, 2 * Mp, Nb), bool)
    for q in range(H * Mp):
        h, p = divmod(q, Mp)
        ent = pp.pair_cols[pp.pair_ptr[q]:pp.pair_ptr[q + 1]]
        n, mask = ent & 0xFFFFFF, ent >> 24
        assert np.all(np.diff(n) > 0) and np.all((mask >= 1) & (mask <= 3))
        back[h, 2 * p, n[(mask & 1) != 0]] = True
        back[h, 2 * p + 1, n[(mask & 2) != 0]] = True
    assert not back[:, Mb:].any()
    assert np.array_equal(back[:, :Mb], lay != 0)


def test_plan_pairs_of_the_page_layouts():
    """A band |i - j| <= w shares all but two columns between neighbouring
    rows (union of rows 2p, 2p+1 = 2w + 2 inside the grid), so the pairs hold
    about half the tiles; identical rows pair to exactly half; a diagonal
    layout shares nothing (the union is the sum) and is not paired."""
    nb, w = 64, 4
    i, j = np.meshgrid(np.arange(nb), np.arange(nb), indexing="ij")
    band = (np.abs(i - j) <= w).astype(np.int32)[None]
    pp = O.plan_pairs(band)
    inner = [pp.pair_ptr[p + 1] - pp.pair_ptr[p] for p in range(3, nb // 2 - 3)]
    assert all(c == 2 * w + 2 for c in inner)
    assert pp.use_pairs == 1
    same = np.repeat((np.random.default_rng(3).random((2, 8, 40)) < 0.3).astype(np.int32), 2, axis=1)
    pp = O.plan_pairs(same)
    assert 2 * pp.pair_total == int(same.sum()) and pp.use_pairs == 1
    assert np.all((pp.pair_cols >> 24) == 3)
    diag = np.eye(16, dtype=np.int32)[None]
    pp = O.plan_pairs(diag)
    assert pp.pair_total == 16 and pp.use_pairs == 0


def load_golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_page_block_diagonal_entry_count():
    g = load_golden()["block_diagonal_entries"]
    nb = g["seq_len"] // g["block"]
    p = O.plan(np.eye(nb, dtype=np.int32)[None])
    assert p.nnz_total * g["block"] ** 2 == g["block_diagonal_entries"]
    assert nb * nb * g["block"] ** 2 == g["dense_entries"]
    assert g["dense_entries"] // g["block_diagonal_entries"] == g["reduction"]


def test_page_block_diagonal_flop_reduction():
    g = load_golden()["block_diagonal_flop_reduction"]
    nb = g["seq_len"] // g["block"]
    p = O.plan(np.eye(nb, dtype=np.int32)[None])
    assert (nb * nb) // p.nnz_total == g["reduction"]


def test_page_two_blocks_per_row_reduction():
    g = load_golden()["gpt3_two_blocks_per_row"]
    nb = g["seq_len"] // g["block"]
    lay = np.zeros((1, nb, nb), np.int32)
    lay[0, np.arange(nb), np.arange(nb)] = 1
    lay[0, np.arange(nb), (np.arange(nb) + 1) % nb] = 1
    p = O.plan(lay)
    assert np.all(np.diff(p.row_ptr) == g["blocks_per_row"])
    assert g["seq_len"] ** 2 // (p.nnz_total * g["block"] ** 2) == g["reduction"]


def test_page_toy_block_sparse_pair_count():
    g = load_golden()["toy_block_sparse_pairs"]
    nb = g["seq_len"] // g["block"]
    per_row = int(nb * (1 - g["sparsity"]))
    lay = np.zeros((1, nb, nb), np.int32)
    for m in range(nb):
        lay[0, m, (m * 7) % nb: (m * 7) % nb + per_row] = 1
    p = O.plan(lay)
    assert p.nnz_total * g["block"] ** 2 == g["block_sparse_pairs"]


def test_band_layout_count_closed_form():
    """Local band |i-j| <= w on nb blocks (the DeepSpeed utils page's local
    attention example: 8 heads, 64 blocks, bandwidth 4) has
    nb(2w+1) - w(w+1) live tiles per head: 556, i.e. 86.43% sparse."""
    nb, w = 64, 4
    i, j = np.meshgrid(np.arange(nb), np.arange(nb), indexing="ij")
    lay = np.broadcast_to((np.abs(i - j) <= w).astype(np.int32), (8, nb, nb)).copy()
    p = O.plan(lay)
    assert p.nnz_total == 8 * (nb * (2 * w + 1) - w * (w + 1)) == 8 * 556
    assert round(100 * (1 - 556 / nb ** 2), 2) == 86.43


# ------------------------------------------- forward options (sink, cap, causal, GQA)

BOTH = (O.attention_dense_masked, O.attention_live_tiles)


def test_causal_full_layout_is_causal_sdpa():
    """causal with every tile live is torch's causal scaled dot-product
    attention; so is causal with the lower-triangular block layout, since the
    tiles above the diagonal are fully masked anyway."""
    B, H, S, d, bs, scale = 2, 2, 48, 8, 16, 0.41
    q, k, v = rnd((B, H, S, d), 61), rnd((B, H, S, d), 62), rnd((B, H, S, d), 63)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale).numpy()
    full = np.ones((H, S // bs, S // bs), np.int32)
    lower = np.tril(full)
    for fn in BOTH:
        for lay in (full, lower):
            out, lse = fn(q, k, v, lay, bs, scale, causal=True)
            np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    # row 0 of every head sees only key 0: its output is v[.., 0, :]
    out, lse = O.attention_live_tiles(q, k, v, lower, bs, scale, causal=True)
    np.testing.assert_allclose(out[:, :, 0], v[:, :, 0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse[:, :, 0], scale * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]),
                               rtol=1e-12, atol=1e-12)


def test_causal_masks_tiles_above_the_diagonal():
    """A block row whose only live tiles lie above the diagonal has no
    visible key under causal: zeros and -inf, as for an empty row."""
    B, H, S, d, bs = 1, 1, 32, 4, 8
    q, k, v = rnd((B, H, S, d), 64), rnd((B, H, S, d), 65), rnd((B, H, S, d), 66)
    lay = np.zeros((H, 4, 4), np.int32)
    lay[0, 1, 2:] = 1            # strictly above the diagonal
    lay[0, 2, :3] = 1
    for fn in BOTH:
        out, lse = fn(q, k, v, lay, bs, 0.5, causal=True)
        assert np.all(out[0, 0, bs:2 * bs] == 0) and np.all(np.isneginf(lse[0, 0, bs:2 * bs]))
        assert np.all(np.isfinite(lse[0, 0, 2 * bs:3 * bs]))


def test_grouped_heads_match_repeated_heads_and_sdpa():
    """kv_heads = H / g: query head h reads K/V head h // g.  Equal to the
    ungrouped oracle with every K/V head repeated g times in a row, and to
    torch's scaled dot-product attention with enable_gqa."""
    B, H, Hkv, S, d, bs, scale = 1, 6, 2, 32, 8, 8, 0.3
    q, k, v = rnd((B, H, S, d), 67), rnd((B, Hkv, S, d), 68), rnd((B, Hkv, S, d), 69)
    lay = np.ones((H, S // bs, S // bs), np.int32)
    kr, vr = np.repeat(k, H // Hkv, axis=1), np.repeat(v, H // Hkv, axis=1)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale, enable_gqa=True).numpy()
    for fn in BOTH:
        out, lse = fn(q, k, v, lay, bs, scale)
        rep, rep_lse = fn(q, kr, vr, lay, bs, scale)
        np.testing.assert_allclose(out, rep, rtol=0, atol=0)
        np.testing.assert_allclose(lse, rep_lse, rtol=0, atol=0)
        np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    with pytest.raises(ValueError):
        O.attention_live_tiles(q, rnd((B, 4, S, d), 1), rnd((B, 4, S, d), 2), lay, bs, scale)


def test_sink_closed_form_with_zero_queries():
    """q = 0 makes every visible score 0: out = (sum of visible v) /
    (n + e^sink) and lse = ln(n + e^sink); the sink only lowers the total
    weight on the real keys (DeepSeek-V4.1 sink term)."""
    B, H, S, d, bs = 1, 3, 32, 4, 8
    q = np.zeros((B, H, S, d))
    k, v = rnd((B, H, S, d), 70), rnd((B, H, S, d), 71)
    rng = np.random.default_rng(72)
    lay = (rng.random((H, 4, 4)) < 0.5).astype(np.int32)
    lay[:, :, 0] = 1
    sink = np.array([-1.0, 0.5, 3.0])
    mask = token_mask_by_lookup(lay, bs)
    n = mask.sum(-1)                                     # [H, S]
    vsum = np.einsum("hij,bhjd->bhid", mask.astype(float), v)
    ref = vsum / (n + np.exp(sink)[:, None])[None, :, :, None]
    for fn in BOTH:
        out, lse = fn(q, k, v, lay, bs, 0.7, sink=sink)
        np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse[0], np.log(n + np.exp(sink)[:, None]), rtol=1e-12)


def test_sink_limits():
    """A sink of -1e9 is no sink; with a sink, a row without a visible key
    has out = 0 and lse = sink_h."""
    B, H, S, d, bs = 2, 2, 24, 4, 8
    q, k, v = rnd((B, H, S, d), 73), rnd((B, H, S, d), 74), rnd((B, H, S, d), 75)
    lay = np.ones((H, 3, 3), np.int32)
    lay[1, 2, :] = 0
    sink = np.array([0.25, -0.75])
    for fn in BOTH:
        base, base_lse = fn(q, k, v, lay, bs, 0.6)
        off, off_lse = fn(q, k, v, lay, bs, 0.6, sink=np.full(H, -1e9))
        np.testing.assert_allclose(off, base, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(off_lse[np.isfinite(base_lse)], base_lse[np.isfinite(base_lse)], rtol=1e-12)
        out, lse = fn(q, k, v, lay, bs, 0.6, sink=sink)
        assert np.all(out[:, 1, 2 * bs:] == 0)
        np.testing.assert_allclose(lse[:, 1, 2 * bs:], -0.75)
        live = np.isfinite(base_lse)
        assert np.all(lse[live] > base_lse[live])        # the denominator only grows


def test_soft_cap_limits():
    """A huge cap changes nothing; with scores driven to +-infinity the capped
    logits saturate at +-cap, so two visible keys get weights
    e^(+-cap) / (e^cap + e^-cap) (tanh capping, Gemma-2 style)."""
    B, H, S, d, bs = 1, 2, 16, 4, 8
    q, k, v = rnd((B, H, S, d), 76), rnd((B, H, S, d), 77), rnd((B, H, S, d), 78)
    lay = np.ones((H, 2, 2), np.int32)
    for fn in BOTH:
        a, la = fn(q, k, v, lay, bs, 0.5)
        b_, lb = fn(q, k, v, lay, bs, 0.5, soft_cap=1e8)
        np.testing.assert_allclose(b_, a, rtol=1e-10, atol=1e-10)
        np.testing.assert_allclose(lb, la, rtol=1e-10)
    # saturation: one query row, two keys with scores +-1e6
    q1 = np.zeros((1, 1, 2, 2)); q1[..., 0] = 1.0
    k1 = np.zeros((1, 1, 2, 2)); k1[0, 0, 0, 0] = 1e6; k1[0, 0, 1, 0] = -1e6
    v1 = np.array([[[[1.0, 0.0], [0.0, 1.0]]]])
    lay1 = np.ones((1, 1, 1), np.int32)
    cap = 1.5
    for fn in BOTH:
        out, lse = fn(q1, k1, v1, lay1, 2, 0.5, soft_cap=cap)   # capping after scaling
        w = np.exp(cap) / (np.exp(cap) + np.exp(-cap))
        np.testing.assert_allclose(out[0, 0, 0], [w, 1 - w], rtol=1e-12)
        np.testing.assert_allclose(lse[0, 0, 0], np.log(np.exp(cap) + np.exp(-cap)), rtol=1e-12)
        assert np.all(np.abs(lse) <= cap + np.log(2) + 1e-12)


def test_options_dense_and_live_tile_forms_agree():
    """All options together on random layouts, grouped heads and a ragged
    block grid: the dense and the live-tile forms give the same result."""
    B, H, Hkv, bs, d = 2, 4, 2, 8, 6
    Mb, Nb = 5, 5
    rng = np.random.default_rng(79)
    q = rnd((B, H, Mb * bs, d), 80)
    k, v = rnd((B, Hkv, Nb * bs, d), 81), rnd((B, Hkv, Nb * bs, d), 82)
    lay = (rng.random((H, Mb, Nb)) < 0.5).astype(np.int32)
    lay[0, 2] = 0
    sink = rnd((H,), 83)
    kw = dict(sink=sink, soft_cap=2.5, causal=True)
    a, la = O.attention_dense_masked(q, k, v, lay, bs, 0.45, **kw)
    b_, lb = O.attention_live_tiles(q, k, v, lay, bs, 0.45, **kw)
    np.testing.assert_allclose(b_, a, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lb, la, rtol=1e-12)


# ------------------------------------------------ ragged sequence lengths

@pytest.mark.parametrize("Sq,Sk,causal", [(37, 53, False), (64, 70, True), (17, 16, False),
                                         (5, 29, True)])
def test_ragged_lengths_match_sdpa(Sq, Sk, causal):
    """Lengths that are not multiples of bs: the layout covers ceil(S/bs)
    blocks and the last block is cut at the sequence end (Language AI
    Handbook, create_block_sparse_mask).  Both oracle forms equal SDPA with a
    mask built by index lookup on the cut sequences."""
    import torch
    bs, B, H, d = 8, 2, 3, 16
    Mb, Nb = -(-Sq // bs), -(-Sk // bs)
    rng = np.random.default_rng(Sq * 100 + Sk)
    q = rng.standard_normal((B, H, Sq, d))
    k = rng.standard_normal((B, H, Sk, d))
    v = rng.standard_normal((B, H, Sk, d))
    lay = (rng.random((H, Mb, Nb)) < 0.6).astype(np.int32)
    lay[:, :, 0] = 1
    scale = 0.3
    m = np.stack([lay[h][np.arange(Sq)[:, None] // bs, np.arange(Sk)[None, :] // bs] != 0
                  for h in range(H)])
    if causal:
        m &= np.arange(Sk)[None, None, :] <= np.arange(Sq)[None, :, None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=torch.from_numpy(m)[None], scale=scale).numpy()
    o1, l1 = O.attention_dense_masked(q, k, v, lay, bs, scale, causal=causal)
    o2, l2 = O.attention_live_tiles(q, k, v, lay, bs, scale, causal=causal)
    assert o1.shape == (B, H, Sq, d)
    assert np.abs(o1 - ref).max() <= 1e-12 and np.abs(o2 - ref).max() <= 1e-12
    assert np.abs(l1 - l2).max() <= 1e-12
    # a layout that does not cover the lengths is rejected
    with pytest.raises(ValueError):
        O.attention_dense_masked(q, k, v, lay[:, :, :Nb - 1] if Nb > 1 else lay[:, :0], bs, scale)


# ------------------------------------------------------------- segment ids

@pytest.mark.parametrize("causal", [False, True])
def test_segments_equal_separate_sequences(causal):
    """Packed sequences: with a full layout and segment ids, every segment's
    output equals attention over that segment alone (torch SDPA, fp64), and
    the live-tile form agrees."""
    import torch
    bs, H, d = 8, 2, 16
    lens = [[13, 20, 7], [25, 15]]          # two batch items, 40 tokens each
    S = 40
    rng = np.random.default_rng(21)
    q = rng.standard_normal((2, H, S, d))
    k = rng.standard_normal((2, H, S, d))
    v = rng.standard_normal((2, H, S, d))
    seg = np.zeros((2, S), np.int32)
    for b, ls in enumerate(lens):
        seg[b] = np.repeat(np.arange(len(ls)), ls)
    nb = -(-S // bs)
    lay = np.ones((H, nb, nb), np.int32)
    out, lse = O.attention_dense_masked(q, k, v, lay, bs, 0.25, causal=causal,
                                        q_segment_ids=seg, kv_segment_ids=seg)
    o2, l2 = O.attention_live_tiles(q, k, v, lay, bs, 0.25, causal=causal,
                                    q_segment_ids=seg, kv_segment_ids=seg)
    assert np.abs(out - o2).max() <= 1e-12 and np.abs(lse - l2).max() <= 1e-12
    for b, ls in enumerate(lens):
        start = 0
        for L in ls:
            sl = slice(start, start + L)
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q[b:b + 1, :, sl]), torch.from_numpy(k[b:b + 1, :, sl]),
                torch.from_numpy(v[b:b + 1, :, sl]), scale=0.25, is_causal=causal).numpy()
            assert np.abs(out[b:b + 1, :, sl] - ref).max() <= 1e-12
            start += L


def test_segments_with_every_option_live_tiles_agree():
    rng = np.random.default_rng(22)
    B, H, Hkv, bs, Sq, Sk, d = 2, 4, 2, 4, 21, 27, 8
    q = rng.standard_normal((B, H, Sq, d))
    k = rng.standard_normal((B, Hkv, Sk, d))
    v = rng.standard_normal((B, Hkv, Sk, d))
    qs = np.sort(rng.integers(0, 3, (B, Sq)), axis=1)
    ks = np.sort(rng.integers(0, 3, (B, Sk)), axis=1)
    lay = (rng.random((H, -(-Sq // bs), -(-Sk // bs))) < 0.6).astype(np.int32)
    kw = dict(sink=rng.standard_normal(H), soft_cap=1.5, causal=True, q_segment_ids=qs,
              kv_segment_ids=ks)
    o1, l1 = O.attention_dense_masked(q, k, v, lay, bs, 0.4, **kw)
    o2, l2 = O.attention_live_tiles(q, k, v, lay, bs, 0.4, **kw)
    assert np.abs(o1 - o2).max() <= 1e-12 and np.abs(l1 - l2).max() <= 1e-12
    with pytest.raises(ValueError):
        O.attention_dense_masked(q, k, v, lay, bs, 0.4, q_segment_ids=qs)
