"""Seeded randomized parity sweep of the forward, the backward and the top-k
gathered attention.

Each case draws every free choice at once from a fixed seed: kernel family
(block size, head dim, dtype), batch, query heads and a dividing number of
K/V heads, query and key lengths (whole or cut last blocks), layout density
with forced empty and full rows, and each option on or off (sink logit, tanh
cap, causal mask, packed-sequence segment ids).  The combinations the
hand-picked tests do not name are where a kernel's instance selection or an
option's interaction with a cut block can go wrong.  Every case is checked
against the fp64 oracle with the tolerances of the whole-block tests; the
case's parameters are printed before it runs.  The top-k cases draw head
size, head count (1..64), batch, positions, table size, top-k, the share of
-1 slots, the sink, repeated indices and entries outside [0, N).
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

FAMILIES = [(bs, d) for bs in (16, 32, 64, 128) for d in (32, 64, 128)]


def draw_case(seed: int, max_blocks: int):
    r = np.random.default_rng(seed)
    bs, d = FAMILIES[r.integers(len(FAMILIES))]
    dtype = "bf16" if r.random() < 0.7 else "f32"
    B = int(r.integers(1, 4))
    H = int(r.choice([1, 2, 3, 4, 6]))
    Hkv = int(r.choice([h for h in range(1, H + 1) if H % h == 0]))
    Mb = int(r.integers(1, max_blocks + 1))
    Nb = int(r.integers(1, max_blocks + 1))
    Sq = Mb * bs - (int(r.integers(0, bs)) if r.random() < 0.5 else 0)
    Sk = Nb * bs - (int(r.integers(0, bs)) if r.random() < 0.5 else 0)
    p = float(r.choice([0.1, 0.3, 0.6, 0.9]))
    lay = (r.random((H, Mb, Nb)) < p).astype(np.int32)
    if H > 1 and Mb > 1:
        lay[1, int(r.integers(Mb)), :] = 0          # a row with no live tile
    lay[0, int(r.integers(Mb)), :] = 1              # a full row
    opts = dict(sink=bool(r.random() < 0.5), cap=bool(r.random() < 0.35),
                causal=bool(r.random() < 0.5), seg=bool(r.random() < 0.35))
    return dict(bs=bs, d=d, dtype=dtype, B=B, H=H, Hkv=Hkv, Sq=Sq, Sk=Sk, lay=lay, **opts)


def build(c, seed):
    x = W.make_bsa("sweep", B=c["B"], H=c["H"], S=c["Sq"], Sk=c["Sk"], bs=c["bs"], d=c["d"],
                   dtype=c["dtype"], layout="given", layout_array=c["lay"], seed=seed,
                   Hkv=c["Hkv"], sink_mean=1.0 if c["sink"] else None)
    qs = ks = None
    if c["seg"]:
        qs = W.packed_segment_ids(c["B"], c["Sq"], 3, 70, seed=seed + 1)
        ks = qs if c["Sq"] == c["Sk"] else W.packed_segment_ids(c["B"], c["Sk"], 3, 70,
                                                                 seed=seed + 2)
    return x, qs, ks


def describe(c):
    on = [k for k in ("sink", "cap", "causal", "seg") if c[k]]
    return (f"bs={c['bs']} d={c['d']} {c['dtype']} B={c['B']} H={c['H']} Hkv={c['Hkv']} "
            f"Sq={c['Sq']} Sk={c['Sk']} density={c['lay'].mean():.2f} opts={'+'.join(on) or '-'}")


def oracle_kw(c, x, qs, ks):
    return dict(sink=None if x.sink is None else x.sink.numpy().astype(np.float64),
                soft_cap=2.5 if c["cap"] else None, causal=c["causal"],
                q_segment_ids=None if qs is None else qs.numpy(),
                kv_segment_ids=None if ks is None else ks.numpy())


def kernel_kw(c, x, qs, ks, gpu):
    return dict(attn_sink=None if x.sink is None else x.sink.to(gpu),
                soft_cap=2.5 if c["cap"] else None, causal=c["causal"], bs=c["bs"],
                q_segment_ids=None if qs is None else qs.to(gpu),
                kv_segment_ids=None if ks is None else ks.to(gpu))


FWD_SEEDS = list(range(9000, 9096))
BWD_SEEDS = list(range(9500, 9540))


@pytest.mark.parametrize("seed", FWD_SEEDS)
def test_forward_sweep(gpu, seed):
    c = draw_case(seed, max_blocks=6)
    say(f"[sweep] forward seed={seed} {describe(c)}")
    x, qs, ks = build(c, seed)
    plan, _ = check_plan(gpu, c["lay"])
    out, lse = bsa.bsa_forward(x.q.to(gpu), x.k.to(gpu), x.v.to(gpu), plan, x.scale,
                               **kernel_kw(c, x, qs, ks, gpu))
    torch.cuda.synchronize()
    kw = oracle_kw(c, x, qs, ks)
    ref, ref_lse = O.attention_live_tiles(to64(x.q), to64(x.k), to64(x.v), c["lay"], c["bs"],
                                          x.scale, **kw)
    compare(to64(out), ref, f"sweep {seed}")
    if c["dtype"] == "f32":
        _, ref_lse = O.attention_live_tiles(bf16_rounded(x.q), bf16_rounded(x.k),
                                            bf16_rounded(x.v), c["lay"], c["bs"], x.scale, **kw)
    compare_lse(lse.cpu().numpy(), ref_lse, f"sweep {seed}")


@pytest.mark.parametrize("seed", BWD_SEEDS)
def test_backward_sweep(gpu, seed):
    c = draw_case(seed, max_blocks=4)
    say(f"[sweep] backward seed={seed} {describe(c)}")
    x, qs, ks = build(c, seed)
    dout = W.upstream_gradient(x.q.shape, seed=seed + 3)
    if c["dtype"] == "f32":
        dout = dout.float()
    plan, _ = check_plan(gpu, c["lay"])
    pc = check_plan_cols(gpu, c["lay"], c["Hkv"])
    q, k, v = x.q.to(gpu), x.k.to(gpu), x.v.to(gpu)
    kw = kernel_kw(c, x, qs, ks, gpu)
    out, lse = bsa.bsa_forward(q, k, v, plan, x.scale, **kw)
    dq, dk, dv, dsink = bsa.bsa_backward(q, k, v, out, dout.to(gpu), lse, plan, pc, x.scale,
                                         **kw)
    torch.cuda.synchronize()
    okw = oracle_kw(c, x, qs, ks)
    rq, rk, rv, rs = O.attention_backward_dense(to64(x.q), to64(x.k), to64(x.v), to64(dout),
                                                c["lay"], c["bs"], x.scale, **okw)
    compare_grad(to64(dq), rq, f"dq sweep {seed}")
    compare_grad(to64(dk), rk, f"dk sweep {seed}")
    compare_grad(to64(dv), rv, f"dv sweep {seed}")
    if c["sink"]:
        # the bound of the whole-block backward tests: rounding of the output
        # inside D_i, twice 2^-9 of the summed magnitudes
        o64, l64 = O.attention_dense_masked(to64(x.q), to64(x.k), to64(x.v), c["lay"], c["bs"],
                                            x.scale, **okw)
        w = np.exp(okw["sink"][None, :, None] - l64)
        bound = 2.0 * 2.0 ** -9 * (w * np.abs(to64(dout) * o64).sum(-1)).sum(axis=(0, 2))
        assert np.all(np.abs(dsink.cpu().numpy() - rs) <= bound + 1e-6)
    else:
        assert dsink is None


TOPK_SEEDS = list(range(9700, 9736))


def draw_topk_case(seed: int):
    r = np.random.default_rng(seed)
    d = int(r.choice([128, 256, 512]))
    H = int(r.integers(1, 65))
    B, M = int(r.integers(1, 3)), int(r.integers(1, 6))
    N = int(r.integers(1, 600))
    topk = int(r.integers(1, N + 1))
    drop = float(r.choice([0.0, 0.1, 0.5, 0.95]))
    with_sink = bool(r.random() < 0.6)
    dups = bool(r.random() < 0.3)       # indices drawn with replacement
    wild = bool(r.random() < 0.3)       # some entries outside [0, N) other than -1
    return dict(d=d, H=H, B=B, M=M, N=N, topk=topk, drop=drop, with_sink=with_sink, dups=dups,
                wild=wild)


@pytest.mark.parametrize("seed", TOPK_SEEDS)
def test_topk_sweep(gpu, seed):
    c = draw_topk_case(seed)
    say(f"[sweep] topk seed={seed} {c}")
    t = W.make_topk("sweep_topk", B=c["B"], M=c["M"], H=c["H"], d=c["d"], N=c["N"],
                    topk=c["topk"], seed=seed, drop=0.0, with_sink=c["with_sink"])
    r = np.random.default_rng(seed + 1)
    if c["dups"]:
        idx = r.integers(0, c["N"], size=(c["B"], c["M"], c["topk"])).astype(np.int32)
    else:
        idx = t.idx.numpy().copy()
    idx[r.random(idx.shape) < c["drop"]] = -1
    if c["wild"]:
        wild = r.random(idx.shape) < 0.1
        idx[wild] = r.choice([-7, c["N"], c["N"] + 3, 2 ** 31 - 1], size=int(wild.sum()))
    sink = t.sink.to(gpu) if c["with_sink"] else None
    out = bsa.topk_sparse_attn(t.q.to(gpu), t.kv.to(gpu), torch.from_numpy(idx).to(gpu), sink,
                               t.scale)
    torch.cuda.synchronize()
    ref_idx = idx.copy()
    ref_idx[(ref_idx < 0) | (ref_idx >= c["N"])] = -1
    ref = O.topk_attention(to64(t.q), to64(t.kv), ref_idx,
                           t.sink.numpy() if c["with_sink"] else None, t.scale)
    compare(to64(out), ref, f"topk sweep {seed}")
    empty = (ref_idx < 0).all(axis=-1)       # positions without a valid slot give zeros
    assert torch.all(out.cpu()[torch.from_numpy(empty)] == 0)


TOPK_WIDE_SEEDS = list(range(9800, 9820))


def draw_topk_wide_case(seed: int):
    """Tables of 2 to 35 index ranges (N up to 70,000 rows) and lists of up
    to 2048 slots, so the compacted list groups indices by range."""
    r = np.random.default_rng(seed)
    d = int(r.choice([128, 256, 512]))
    return dict(d=d, H=int(r.integers(1, 21)), B=int(r.integers(1, 3)), M=int(r.integers(1, 5)),
                N=int(r.integers(2049, 70001)), topk=int(r.integers(1, 2049)),
                drop=float(r.choice([0.0, 0.1, 0.5])), with_sink=bool(r.random() < 0.6),
                dups=bool(r.random() < 0.3), wild=bool(r.random() < 0.3))


@pytest.mark.parametrize("seed", TOPK_WIDE_SEEDS)
def test_topk_wide_sweep(gpu, seed):
    c = draw_topk_wide_case(seed)
    say(f"[sweep] topk wide seed={seed} {c}")
    t = W.make_topk("sweep_topk_wide", B=c["B"], M=c["M"], H=c["H"], d=c["d"], N=c["N"],
                    topk=c["topk"], seed=seed, drop=0.0, with_sink=c["with_sink"])
    r = np.random.default_rng(seed + 1)
    if c["dups"]:
        idx = r.integers(0, c["N"], size=(c["B"], c["M"], c["topk"])).astype(np.int32)
    else:
        idx = t.idx.numpy().copy()
    idx[r.random(idx.shape) < c["drop"]] = -1
    if c["wild"]:
        wild = r.random(idx.shape) < 0.1
        idx[wild] = r.choice([-7, c["N"], c["N"] + 3, 2 ** 31 - 1], size=int(wild.sum()))
    sink = t.sink.to(gpu) if c["with_sink"] else None
    ig = torch.from_numpy(idx).to(gpu)
    q, kv = t.q.to(gpu), t.kv.to(gpu)
    out = bsa.topk_sparse_attn(q, kv, ig, sink, t.scale)
    out2 = bsa.topk_sparse_attn(q, kv, ig, sink, t.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "top-k is not deterministic"
    ref_idx = idx.copy()
    ref_idx[(ref_idx < 0) | (ref_idx >= c["N"])] = -1
    ref = O.topk_attention(to64(t.q), to64(t.kv), ref_idx,
                           t.sink.numpy() if c["with_sink"] else None, t.scale)
    compare(to64(out), ref, f"topk wide sweep {seed}")
