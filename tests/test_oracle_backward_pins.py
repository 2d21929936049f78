"""Pins of the backward oracle against things other than itself.

* Central finite differences of the forward oracle (float64): every entry of
  dq, dk, dv and dsink, for each option alone and together, grouped heads
  included.  A dropped term, a wrong sign or a transposed operand in any of
  the backward formulas moves some entry far outside the difference quotient.
* torch autograd of torch's scaled_dot_product_attention in float64 with a
  boolean mask (and enable_gqa for grouped heads): an independent derivation
  of the same gradients.
* Invariants: a shift of every key row leaves every softmax unchanged (so the
  key gradients of a K/V head sum to zero without sink or cap); a shift of
  every value row moves each output row by the shift (so the value gradients
  sum to the upstream gradients of the rows with a live key); sum q.dq equals
  sum k.dk; zero upstream gradient gives zero gradients.
* The transposed plan against a brute-force construction.
"""

import numpy as np
import pytest
import torch

from oracle import bsa_oracle as O


def _inputs(seed, B=1, H=2, Hkv=2, bs=2, Mb=2, Nb=3, d=3, p=0.6, std=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, Mb * bs, d)) * std
    k = rng.standard_normal((B, Hkv, Nb * bs, d)) * std
    v = rng.standard_normal((B, Hkv, Nb * bs, d))
    dout = rng.standard_normal((B, H, Mb * bs, d))
    lay = (rng.random((H, Mb, Nb)) < p).astype(np.int32)
    sink = rng.standard_normal(H)
    return q, k, v, dout, lay, bs, sink


def _loss(q, k, v, dout, lay, bs, scale, **kw):
    out, _ = O.attention_dense_masked(q, k, v, lay, bs, scale, **kw)
    return float((out * dout).sum())


def _fd(f, x, h=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = x[i]
        x[i] = old + h
        fp = f()
        x[i] = old - h
        fm = f()
        x[i] = old
        g[i] = (fp - fm) / (2 * h)
    return g


OPTION_SETS = [
    dict(),
    dict(sink=True),
    dict(soft_cap=0.8),
    dict(causal=True),
    dict(Hkv=1),
    dict(sink=True, soft_cap=0.8, causal=True, Hkv=1),
]


@pytest.mark.parametrize("opts", OPTION_SETS, ids=lambda o: "+".join(o) or "plain")
def test_backward_matches_finite_differences(opts):
    Hkv = opts.get("Hkv", 2)
    q, k, v, dout, lay, bs, sink = _inputs(11, Hkv=Hkv, std=1.5)
    lay[1, 0, :] = 0                     # a block row with no live tile
    lay[0, 0, 2] = 1                     # a tile above the diagonal
    kw = {}
    if opts.get("sink"):
        kw["sink"] = sink
    if "soft_cap" in opts:
        kw["soft_cap"] = opts["soft_cap"]
    if opts.get("causal"):
        kw["causal"] = True
    scale = 0.7
    dq, dk, dv, dsink = O.attention_backward_dense(q, k, v, dout, lay, bs, scale, **kw)
    f = lambda: _loss(q, k, v, dout, lay, bs, scale, **kw)  # noqa: E731
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = _fd(f, x)
        assert np.abs(num - g).max() <= 1e-7 * max(1.0, np.abs(num).max()), name
    if "sink" in kw:
        s = kw["sink"]
        num = _fd(f, s)
        assert np.abs(num - dsink).max() <= 1e-7
    else:
        assert dsink is None
    # live-tile form gives the same values
    lt = O.attention_backward_live_tiles(q, k, v, dout, lay, bs, scale, **kw)
    for a, b in zip((dq, dk, dv), lt[:3]):
        assert np.abs(a - b).max() <= 1e-12
    if dsink is not None:
        assert np.abs(dsink - lt[3]).max() <= 1e-12


@pytest.mark.parametrize("Hkv", [4, 2, 1])
def test_backward_matches_torch_autograd_sdpa(Hkv):
    B, H, bs, Mb, Nb, d = 2, 4, 4, 3, 5, 8
    q, k, v, dout, lay, bs, _ = _inputs(5, B=B, H=H, Hkv=Hkv, bs=bs, Mb=Mb, Nb=Nb, d=d, p=0.5)
    lay[:, :, 0] = 1                     # every row has a live key (SDPA has no empty rows)
    scale = 0.35
    dq, dk, dv, _ = O.attention_backward_dense(q, k, v, dout, lay, bs, scale)
    # boolean token mask built by index arithmetic, not by the oracle's helper
    tq = np.arange(Mb * bs)[:, None] // bs
    tk = np.arange(Nb * bs)[None, :] // bs
    mask = torch.from_numpy(np.stack([lay[h][tq, tk] != 0 for h in range(H)]))
    tq_, tk_, tv_ = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(
        tq_, tk_, tv_, attn_mask=mask[None], scale=scale, enable_gqa=(Hkv != H))
    out.backward(torch.from_numpy(dout))
    for a, b in ((dq, tq_.grad), (dk, tk_.grad), (dv, tv_.grad)):
        assert np.abs(a - b.numpy()).max() <= 1e-12


def test_backward_sink_and_cap_match_torch_autograd():
    """Autograd through a forward built from torch ops: the sink as one more
    logit column of the softmax (dropped afterwards), the cap as tanh."""
    B, H, bs, Mb, Nb, d = 1, 3, 4, 3, 4, 8
    q, k, v, dout, lay, bs, sink = _inputs(7, B=B, H=H, Hkv=H, bs=bs, Mb=Mb, Nb=Nb, d=d, p=0.5,
                                           std=2.0)
    lay[:, :, 1] = 1
    scale, cap = 0.5, 1.3
    dq, dk, dv, dsink = O.attention_backward_dense(q, k, v, dout, lay, bs, scale, sink=sink,
                                                   soft_cap=cap)
    tq = np.arange(Mb * bs)[:, None] // bs
    tk = np.arange(Nb * bs)[None, :] // bs
    mask = torch.from_numpy(np.stack([lay[h][tq, tk] != 0 for h in range(H)]))[None]
    tq_, tk_, tv_, ts_ = (torch.tensor(x, requires_grad=True) for x in (q, k, v, sink))
    s = cap * torch.tanh(scale * tq_ @ tk_.transpose(-1, -2) / cap)
    s = s.masked_fill(~mask, float("-inf"))
    col = ts_[None, :, None, None].expand(B, H, Mb * bs, 1)
    w = torch.softmax(torch.cat([s, col], dim=-1), dim=-1)[..., :-1]
    out = w @ tv_
    out.backward(torch.from_numpy(dout))
    for a, b in ((dq, tq_.grad), (dk, tk_.grad), (dv, tv_.grad), (dsink, ts_.grad)):
        assert np.abs(a - b.numpy()).max() <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_backward_shift_invariances(causal):
    q, k, v, dout, lay, bs, _ = _inputs(3, B=2, H=4, Hkv=2, bs=4, Mb=3, Nb=3, d=5, p=0.5)
    lay[2, 1, :] = 0
    dq, dk, dv, _ = O.attention_backward_dense(q, k, v, dout, lay, bs, 0.4, causal=causal)
    # keys: every softmax is unchanged by a common shift of the key rows
    assert np.abs(dk.sum(axis=2)).max() <= 1e-12
    # values: each row with a live key moves by the shift
    _, lse = O.attention_dense_masked(q, k, v, lay, bs, 0.4, causal=causal)
    live = np.isfinite(lse)[..., None]
    want = np.where(live, dout, 0.0).reshape(2, 2, 2, -1, 5).sum(axis=(2, 3))   # groups of 2
    assert np.abs(dv.sum(axis=2) - want).max() <= 1e-12
    # sum q.dq = sum k.dk (both are scale * sum ds_ij q_i.k_j)
    assert abs((q * dq).sum() - (k * dk).sum()) <= 1e-12 * max(1.0, abs((q * dq).sum()))


def test_backward_zero_upstream_gradient():
    q, k, v, dout, lay, bs, sink = _inputs(4)
    g = O.attention_backward_dense(q, k, v, np.zeros_like(dout), lay, bs, 0.5, sink=sink,
                                   soft_cap=2.0, causal=True)
    for x in g:
        assert np.all(x == 0)


def test_plan_columns_brute_force():
    rng = np.random.default_rng(2)
    for (H, Hkv, Mb, Nb) in ((4, 2, 5, 7), (3, 3, 1, 4), (6, 1, 9, 2), (2, 2, 3, 3)):
        lay = (rng.random((H, Mb, Nb)) < 0.4).astype(np.int32)
        lay[0, :, 0] = 0
        pc = O.plan_columns(lay, Hkv)
        g = H // Hkv
        ptr = 0
        for h in range(H):
            for n in range(Nb):
                ms = [m for m in range(Mb) if lay[h, m, n] != 0]
                assert pc.col_ptr[h * Nb + n] == ptr
                assert list(pc.row_idx[ptr:ptr + len(ms)]) == ms
                ptr += len(ms)
        assert pc.col_ptr[-1] == ptr == pc.nnz_total
        # order: selection of the heaviest remaining item, ties by n
        for j in range(Hkv):
            work = {n: sum(int(lay[h, m, n] != 0) for h in range(j * g, (j + 1) * g)
                           for m in range(Mb)) for n in range(Nb)}
            seq = []
            while work:
                best = max(work, key=lambda n: (work[n], -n))
                seq.append(j * Nb + best)
                del work[best]
            assert list(pc.col_order[j * Nb:(j + 1) * Nb]) == seq


@pytest.mark.parametrize("Sq,Sk", [(7, 9), (6, 5)])
def test_backward_ragged_matches_finite_differences(Sq, Sk):
    """Cut last blocks (bs = 4): the dense and live-tile backward agree with
    central differences of the forward oracle."""
    bs, d, H = 4, 3, 2
    rng = np.random.default_rng(Sq + 10 * Sk)
    Mb, Nb = -(-Sq // bs), -(-Sk // bs)
    q = rng.standard_normal((1, H, Sq, d))
    k = rng.standard_normal((1, 1, Sk, d))
    v = rng.standard_normal((1, 1, Sk, d))
    dout = rng.standard_normal((1, H, Sq, d))
    lay = (rng.random((H, Mb, Nb)) < 0.7).astype(np.int32)
    lay[:, :, Nb - 1] = 1
    kw = dict(causal=True, sink=rng.standard_normal(H), soft_cap=1.1)
    dq, dk, dv, ds = O.attention_backward_dense(q, k, v, dout, lay, bs, 0.6, **kw)
    f = lambda: _loss(q, k, v, dout, lay, bs, 0.6, **kw)  # noqa: E731
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = _fd(f, x)
        assert np.abs(num - g).max() <= 1e-7 * max(1.0, np.abs(num).max())
    lt = O.attention_backward_live_tiles(q, k, v, dout, lay, bs, 0.6, **kw)
    for a, b in zip((dq, dk, dv, ds), lt):
        assert np.abs(a - b).max() <= 1e-12


def test_backward_segments_match_finite_differences():
    rng = np.random.default_rng(31)
    B, H, bs, Sq, Sk, d = 2, 2, 2, 5, 6, 3
    q = rng.standard_normal((B, H, Sq, d))
    k = rng.standard_normal((B, 1, Sk, d))
    v = rng.standard_normal((B, 1, Sk, d))
    dout = rng.standard_normal((B, H, Sq, d))
    lay = (rng.random((H, 3, 3)) < 0.8).astype(np.int32)
    qs = np.array([[0, 0, 1, 1, 1], [0, 1, 1, 2, 2]])
    ks = np.array([[0, 0, 0, 1, 1, 1], [0, 1, 1, 1, 2, 2]])
    kw = dict(causal=True, sink=rng.standard_normal(H), q_segment_ids=qs, kv_segment_ids=ks)
    dq, dk, dv, ds = O.attention_backward_dense(q, k, v, dout, lay, bs, 0.6, **kw)
    f = lambda: _loss(q, k, v, dout, lay, bs, 0.6, **kw)  # noqa: E731
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = _fd(f, x)
        assert np.abs(num - g).max() <= 1e-7 * max(1.0, np.abs(num).max())
    lt = O.attention_backward_live_tiles(q, k, v, dout, lay, bs, 0.6, **kw)
    for a, b in zip((dq, dk, dv, ds), lt):
        assert np.abs(a - b).max() <= 1e-12
