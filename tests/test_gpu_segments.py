"""GPU parity of segment ids (packed sequences) against the fp64 oracle.

Sequences of random lengths are packed back to back; a query attends only
the keys of its own segment, on top of the layout (and the causal mask and
cut last blocks where given).  Forward on every kernel family -- bf16 with
bs >= 64 then runs the register-staged kernel -- and the backward, with the
whole-block tolerances.
"""

import numpy as np
import pytest
import torch

import block_sparse_attention_plan_amd as bsa
from block_sparse_attention_plan_amd import workloads as W
from oracle import bsa_oracle as O

from test_gpu_backward import check_plan_cols, compare_grad
from test_gpu_parity import bf16_rounded, check_plan, compare, compare_lse, say, to64

pytestmark = pytest.mark.gpu

FWD = [(16, 64, "bf16", 160, 160), (16, 32, "f32", 100, 93), (32, 64, "bf16", 256, 256),
       (64, 128, "f32", 320, 320), (64, 128, "bf16", 300, 300), (128, 128, "bf16", 512, 512),
       (128, 64, "bf16", 500, 450), (64, 64, "bf16", 250, 256), (128, 32, "bf16", 384, 300)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("bs,d,dtype,Sq,Sk", FWD)
def test_forward_segments(gpu, bs, d, dtype, Sq, Sk, causal):
    H, B = 2, 2
    Mb, Nb = -(-Sq // bs), -(-Sk // bs)
    rng = np.random.default_rng(bs * 7 + d + Sq)
    lay = (rng.random((H, Mb, Nb)) < 0.7).astype(np.int32)
    lay[:, np.arange(min(Mb, Nb)), np.arange(min(Mb, Nb))] = 1
    x = W.make_bsa("segments", B=B, H=H, S=Sq, Sk=Sk, bs=bs, d=d, dtype=dtype, layout="given",
                   layout_array=lay, seed=Sq + d)
    qs = W.packed_segment_ids(B, Sq, 5, 90, seed=Sq)
    ks = qs if Sq == Sk else W.packed_segment_ids(B, Sk, 5, 90, seed=Sq)
    say(f"[segments] forward bs={bs} d={d} {dtype} Sq={Sq} Sk={Sk} causal={causal}")
    plan, _ = check_plan(gpu, lay)
    out, lse = bsa.bsa_forward(x.q.to(gpu), x.k.to(gpu), x.v.to(gpu), plan, x.scale, bs=bs,
                               causal=causal, q_segment_ids=qs.to(gpu),
                               kv_segment_ids=ks.to(gpu))
    torch.cuda.synchronize()
    kw = dict(causal=causal, q_segment_ids=qs.numpy(), kv_segment_ids=ks.numpy())
    ref, ref_lse = O.attention_live_tiles(to64(x.q), to64(x.k), to64(x.v), lay, bs, x.scale, **kw)
    compare(to64(out), ref, f"segments bs={bs} d={d} {dtype}")
    if dtype == "f32":
        _, ref_lse = O.attention_live_tiles(bf16_rounded(x.q), bf16_rounded(x.k),
                                            bf16_rounded(x.v), lay, bs, x.scale, **kw)
    compare_lse(lse.cpu().numpy(), ref_lse, f"segments bs={bs} d={d}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("bs,d,S", [(16, 64, 120), (32, 64, 250), (64, 128, 256), (128, 128, 400)])
def test_backward_segments(gpu, bs, d, S, causal):
    H, Hkv, B = 4, 2, 2
    nb = -(-S // bs)
    rng = np.random.default_rng(bs + S)
    lay = (rng.random((H, nb, nb)) < 0.7).astype(np.int32)
    lay[:, np.arange(nb), np.arange(nb)] = 1
    x = W.make_bsa("segments_bwd", B=B, H=H, S=S, bs=bs, d=d, dtype="bf16", layout="given",
                   layout_array=lay, seed=S + 3, Hkv=Hkv, sink_mean=1.0)
    seg = W.packed_segment_ids(B, S, 5, 120, seed=S + 1)
    dout = W.upstream_gradient(x.q.shape, seed=S + 2)
    say(f"[segments] backward bs={bs} d={d} S={S} causal={causal}")
    plan, _ = check_plan(gpu, lay)
    pc = check_plan_cols(gpu, lay, Hkv)
    q, k, v, sink, sg = x.q.to(gpu), x.k.to(gpu), x.v.to(gpu), x.sink.to(gpu), seg.to(gpu)
    kw = dict(attn_sink=sink, causal=causal, bs=bs, q_segment_ids=sg, kv_segment_ids=sg)
    out, lse = bsa.bsa_forward(q, k, v, plan, x.scale, **kw)
    dq, dk, dv, dsink = bsa.bsa_backward(q, k, v, out, dout.to(gpu), lse, plan, pc, x.scale, **kw)
    torch.cuda.synchronize()
    sk64 = x.sink.numpy().astype(np.float64)
    okw = dict(sink=sk64, causal=causal, q_segment_ids=seg.numpy(), kv_segment_ids=seg.numpy())
    rq, rk, rv, rs = O.attention_backward_dense(to64(x.q), to64(x.k), to64(x.v), to64(dout), lay,
                                                bs, x.scale, **okw)
    compare_grad(to64(dq), rq, f"dq segments bs={bs}")
    compare_grad(to64(dk), rk, f"dk segments bs={bs}")
    compare_grad(to64(dv), rv, f"dv segments bs={bs}")
    o64, l64 = O.attention_dense_masked(to64(x.q), to64(x.k), to64(x.v), lay, bs, x.scale, **okw)
    w = np.exp(sk64[None, :, None] - l64)
    bound = 2.0 * 2.0 ** -9 * (w * np.abs(to64(dout) * o64).sum(-1)).sum(axis=(0, 2))
    assert np.all(np.abs(dsink.cpu().numpy() - rs) <= bound + 1e-6)


@pytest.mark.parametrize("bs,d,lengths", [(128, 128, (256, 384, 128, 256)),
                                          (64, 128, (64, 320, 192, 448)),
                                          (64, 64, (128, 64, 64, 256, 512))])
def test_forward_segments_equal_reduced_layout(gpu, bs, d, lengths):
    """Segments that start and end on block boundaries mask exactly the tiles
    between different segments, so the forward with segment ids (which drops
    the tiles whose keys all lie in other segments) equals the forward
    without them on the layout with those tiles removed.  At bs = 64 the
    reduced layout's neighbouring rows share tiles, so its forward runs in the
    paired form (64-key pieces instead of 32), whose bf16 weights and rescale
    points differ: there the two agree to the rounding of the bf16 output and
    weights (2^-8 absolute plus 2^-7 relative), and both meet the oracle."""
    S = sum(lengths)
    H, nb = 2, S // bs
    seg = np.repeat(np.arange(len(lengths), dtype=np.int32), lengths)[None]     # [1, S]
    rng = np.random.default_rng(S + bs)
    lay = (rng.random((H, nb, nb)) < 0.6).astype(np.int32)
    lay[:, np.arange(nb), np.arange(nb)] = 1
    blk = seg[0, ::bs]
    reduced = lay * (blk[:, None] == blk[None, :])[None].astype(np.int32)
    x = W.make_bsa("segments_reduced", B=1, H=H, S=S, bs=bs, d=d, dtype="bf16",
                   layout="given", layout_array=lay, seed=S)
    say(f"[segments] reduced layout bs={bs} d={d} lengths={lengths}")
    q, k, v = x.q.to(gpu), x.k.to(gpu), x.v.to(gpu)
    sg = torch.from_numpy(seg).to(gpu)
    plan, _ = check_plan(gpu, lay)
    plan_r, _ = check_plan(gpu, reduced)
    out, lse = bsa.bsa_forward(q, k, v, plan, x.scale, bs=bs, q_segment_ids=sg, kv_segment_ids=sg)
    out_r, lse_r = bsa.bsa_forward(q, k, v, plan_r, x.scale, bs=bs)
    torch.cuda.synchronize()
    diff = (out.float() - out_r.float()).abs().max().item()
    say(f"  segment ids vs reduced layout: max |diff| {diff:.3e}")
    assert torch.allclose(out.float(), out_r.float(), atol=2 ** -8, rtol=2 ** -7 if bs == 64 else 0)
    assert torch.allclose(lse, lse_r, atol=1e-5, rtol=0)
    ref, _ = O.attention_live_tiles(to64(x.q), to64(x.k), to64(x.v), reduced, bs, x.scale)
    compare(to64(out), ref, f"segments reduced bs={bs} d={d}")


def _segment_case(gpu, lay, bs, d, Sq, Sk, qs, ks, seed, causal=False, sink=False, what=""):
    """Forward with segment ids against the oracle, outputs and lse."""
    B, H = qs.shape[0], lay.shape[0]
    x = W.make_bsa("segments_filter", B=B, H=H, S=Sq, Sk=Sk, bs=bs, d=d, dtype="bf16",
                   layout="given", layout_array=lay, seed=seed,
                   sink_mean=1.0 if sink else None)
    plan, _ = check_plan(gpu, lay)
    kw = dict(bs=bs, causal=causal, q_segment_ids=qs.to(gpu), kv_segment_ids=ks.to(gpu))
    if sink:
        kw["attn_sink"] = x.sink.to(gpu)
    out, lse = bsa.bsa_forward(x.q.to(gpu), x.k.to(gpu), x.v.to(gpu), plan, x.scale, **kw)
    torch.cuda.synchronize()
    okw = dict(causal=causal, q_segment_ids=qs.numpy(), kv_segment_ids=ks.numpy())
    if sink:
        okw["sink"] = x.sink.numpy().astype(np.float64)
    ref, ref_lse = O.attention_live_tiles(to64(x.q), to64(x.k), to64(x.v), lay, bs, x.scale, **okw)
    compare(to64(out), ref, what)
    compare_lse(lse.cpu().numpy(), ref_lse, what)
    return out, lse, ref, ref_lse


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("bs,d,S", [(128, 128, 512), (128, 64, 500), (64, 128, 448), (64, 64, 390)])
def test_forward_segments_unordered_ids(gpu, bs, d, S, causal):
    """Ids drawn per token from {0, 1, 2} (not contiguous runs): the id ranges
    of every query block and key tile overlap, so no tile is dropped and every
    piece mixes ids -- each score's mask comes from the key ids read one by
    one.  S not a multiple of bs puts keys past the end into mixed pieces."""
    H, B = 2, 2
    nb = -(-S // bs)
    rng = np.random.default_rng(S + bs + d)
    lay = (rng.random((H, nb, nb)) < 0.6).astype(np.int32)
    lay[:, np.arange(nb), np.arange(nb)] = 1
    ids = torch.from_numpy(rng.integers(0, 3, size=(B, S)).astype(np.int32))
    say(f"[segments] unordered ids bs={bs} d={d} S={S} causal={causal}")
    _segment_case(gpu, lay, bs, d, S, S, ids, ids, seed=S + 1, causal=causal,
                  what=f"unordered ids bs={bs} d={d}")


@pytest.mark.parametrize("sink", [False, True])
@pytest.mark.parametrize("bs,d", [(128, 128), (64, 64)])
def test_forward_segments_rows_without_same_segment_tiles(gpu, bs, d, sink):
    """Block-aligned segments of two blocks each; in every head, block rows
    3 and 6 list only tiles of other segments.  Their tiles are all dropped
    before the pipeline: the rows come out as zeros with lse -inf (the sink
    logit with a sink), as the oracle's fully masked rows do; the other rows
    keep their same-segment tiles and mixed layouts."""
    H, B, nb = 2, 2, 8
    S = nb * bs
    rng = np.random.default_rng(bs + d + sink)
    lay = (rng.random((H, nb, nb)) < 0.6).astype(np.int32)
    lay[:, np.arange(nb), np.arange(nb)] = 1
    blk_seg = np.arange(nb) // 2
    for m in (3, 6):
        other = blk_seg != blk_seg[m]
        lay[:, m, :] = 0
        lay[:, m, other] = 1
    seg = torch.from_numpy(np.repeat(np.repeat(blk_seg, bs)[None], B, 0).astype(np.int32))
    say(f"[segments] rows without same-segment tiles bs={bs} d={d} sink={sink}")
    out, lse, ref, ref_lse = _segment_case(gpu, lay, bs, d, S, S, seg, seg, seed=S + 2,
                                           sink=sink, what=f"dropped rows bs={bs} d={d}")
    rows = np.concatenate([np.arange(3 * bs, 4 * bs), np.arange(6 * bs, 7 * bs)])
    assert torch.count_nonzero(out[:, :, rows]).item() == 0
    if not sink:
        assert np.isneginf(lse.cpu().numpy()[:, :, rows]).all()


@pytest.mark.parametrize("bs,d", [(64, 64), (128, 32)])
def test_forward_segments_long_row_unfiltered(gpu, bs, d):
    """One block row with more live tiles (520) than the filter's list holds:
    the row walks the plan's list unfiltered, and every piece's mask comes
    from its key ids read one by one."""
    H, B, nb = 1, 1, 520
    Sq, Sk = bs, nb * bs - 5
    lay = np.ones((H, 1, nb), np.int32)
    qs = torch.from_numpy(np.full((B, Sq), 3, np.int32))
    ks = W.packed_segment_ids(B, Sk, 50, 4000, seed=nb)
    say(f"[segments] long row, {nb} tiles, bs={bs} d={d}")
    _segment_case(gpu, lay, bs, d, Sq, Sk, qs, ks, seed=nb + bs, what=f"long row bs={bs} d={d}")


@pytest.mark.parametrize("ids", ["packed", "unordered"])
@pytest.mark.parametrize("bs,d,S,lo,hi", [(32, 64, 1024, 60, 300), (64, 128, 1536, 100, 600),
                                          (128, 64, 2560, 300, 1200)])
def test_backward_segments_long_lists(gpu, bs, d, S, lo, hi, ids):
    """Rows and columns of more than 16 live tiles, so the bs >= 32 kernels
    test their tiles' segment ranges in several batches of 16; with packed
    sequences most tiles are skipped (disjoint id ranges), with ids drawn
    per token from {0, 1, 2} none are.  Two query heads share each K/V head
    and there is a sink; every gradient against the oracle."""
    H, Hkv, B = 2, 1, 1
    nb = S // bs
    rng = np.random.default_rng(S + bs)
    lay = (rng.random((H, nb, nb)) < 0.8).astype(np.int32)
    lay[:, np.arange(nb), np.arange(nb)] = 1
    x = W.make_bsa("segments_bwd_long", B=B, H=H, S=S, bs=bs, d=d, dtype="bf16", layout="given",
                   layout_array=lay, seed=S + 5, Hkv=Hkv, sink_mean=1.0)
    if ids == "packed":
        seg = W.packed_segment_ids(B, S, lo, hi, seed=S + 6)
    else:
        seg = torch.from_numpy(rng.integers(0, 3, size=(B, S)).astype(np.int32))
    dout = W.upstream_gradient(x.q.shape, seed=S + 7)
    say(f"[segments] backward long lists bs={bs} d={d} S={S} ids={ids}")
    plan, _ = check_plan(gpu, lay)
    pc = check_plan_cols(gpu, lay, Hkv)
    q, k, v, sink, sg = x.q.to(gpu), x.k.to(gpu), x.v.to(gpu), x.sink.to(gpu), seg.to(gpu)
    kw = dict(attn_sink=sink, bs=bs, q_segment_ids=sg, kv_segment_ids=sg)
    out, lse = bsa.bsa_forward(q, k, v, plan, x.scale, **kw)
    dq, dk, dv, _ = bsa.bsa_backward(q, k, v, out, dout.to(gpu), lse, plan, pc, x.scale, **kw)
    torch.cuda.synchronize()
    okw = dict(sink=x.sink.numpy().astype(np.float64), q_segment_ids=seg.numpy(),
               kv_segment_ids=seg.numpy())
    rq, rk, rv, _ = O.attention_backward_dense(to64(x.q), to64(x.k), to64(x.v), to64(dout), lay,
                                               bs, x.scale, **okw)
    compare_grad(to64(dq), rq, f"dq long lists bs={bs} {ids}")
    compare_grad(to64(dk), rk, f"dk long lists bs={bs} {ids}")
    compare_grad(to64(dv), rv, f"dv long lists bs={bs} {ids}")
