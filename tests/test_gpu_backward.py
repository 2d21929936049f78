"""GPU parity of the backward (bsa_plan_cols, bsa_backward) against the fp64
oracle.

Column plans must match bit for bit.  Gradients are compared with the
oracle's gradients of the exact function at the same bf16 inputs; the GPU
backward is fed the GPU forward's own out and lse, as a training step would.
Tolerance (derived from the arithmetic): the kernels round P and dS to bf16
(relative 2^-9 each) before their products and round the result to bf16
(2^-9), with fp32 accumulation; the rounding errors are independent, so each
gradient entry carries an error of a few 2^-9 of the magnitude of the terms
summed into it.  We require max |err| <= 2^-6 * max |ref| and
mean |err| <= 2^-7 * mean |ref| for dq, dk and dv.  dsink_h sums
exp(sink_h - lse_i) D_i over every row, where D_i = dO_i . out_i uses the
forward's bf16 output, each of whose entries carries up to 2^-9 relative
rounding; its error is therefore at most
2^-9 * sum_i exp(sink_h - lse_i) sum_d |dO_id out_id|, and we allow twice that.
"""

import zlib

import numpy as np
import pytest
import torch

import block_sparse_attention_plan_amd as bsa
from block_sparse_attention_plan_amd import workloads as W
from oracle import bsa_oracle as O

from test_gpu_parity import _sample_row_blocks, check_plan, say, to64

pytestmark = pytest.mark.gpu

MAX_REL = 2.0 ** -6
MEAN_REL = 2.0 ** -7


def compare_grad(gpu: np.ndarray, ref: np.ndarray, what: str):
    assert np.isfinite(gpu).all(), f"{what}: non-finite gradient"
    err = np.abs(gpu - ref)
    scale_max = np.abs(ref).max()
    scale_mean = np.abs(ref).mean()
    say(f"  {what}: max_abs={err.max():.3e} (ref max {scale_max:.3e}) "
        f"mean_abs={err.mean():.3e} (ref mean {scale_mean:.3e})")
    assert err.max() <= MAX_REL * scale_max + 1e-6, what
    assert err.mean() <= MEAN_REL * scale_mean + 1e-7, what


def check_plan_cols(dev, layout: np.ndarray, Hkv: int):
    ref = O.plan_columns(layout, Hkv)
    pc = bsa.bsa_plan_cols(torch.from_numpy(np.ascontiguousarray(layout, dtype=np.int32)).to(dev),
                           Hkv)
    nnz = int(pc.nnz_total_dev.item())
    assert nnz == ref.nnz_total
    assert torch.equal(pc.col_ptr.cpu(), torch.from_numpy(ref.col_ptr))
    assert torch.equal(pc.col_order.cpu(), torch.from_numpy(ref.col_order))
    assert torch.equal(pc.row_idx(nnz).cpu(), torch.from_numpy(ref.row_idx))
    return pc


@pytest.mark.parametrize("case", [
    ("empty", (2, 2, 3, 5), 0.0), ("full", (4, 2, 4, 4), 1.0), ("one_row", (3, 3, 1, 70), 0.5),
    ("tall", (2, 1, 300, 40), 0.15), ("wide", (4, 4, 5, 200), 0.2), ("ragged", (8, 2, 33, 65), 0.4),
    ("mqa", (16, 1, 64, 64), 0.1)])
def test_plan_cols_random_layouts(gpu, case):
    name, (H, Hkv, Mb, Nb), p = case
    say(f"[plan_cols] {name} H={H} Hkv={Hkv} Mb={Mb} Nb={Nb} p={p}")
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    lay = (rng.random((H, Mb, Nb)) < p).astype(np.int32) * rng.integers(1, 4, (H, Mb, Nb)).astype(np.int32)
    check_plan_cols(gpu, lay, Hkv)


OPTION_SETS = {
    "plain": dict(),
    "sink": dict(sink_mean=1.0),
    "cap": dict(soft_cap=2.0),
    "causal": dict(causal=True),
    "gqa": dict(Hkv=2),
    "all": dict(sink_mean=1.0, soft_cap=2.0, causal=True, Hkv=2),
}
BWD_CASES = [(16, 32), (16, 128), (32, 32), (32, 128), (64, 64), (64, 128), (128, 32),
             (128, 128)]


def _forward_backward(gpu, x, opts, plan, pc, dout):
    q, k, v = (t.to(gpu) for t in (x.q, x.k, x.v))
    sink = x.sink.to(gpu) if x.sink is not None else None
    kw = dict(attn_sink=sink, soft_cap=opts.get("soft_cap"), causal=opts.get("causal", False))
    out, lse = bsa.bsa_forward(q, k, v, plan, x.scale, **kw)
    g = bsa.bsa_backward(q, k, v, out, dout.to(gpu), lse, plan, pc, x.scale, **kw)
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("opt_name", list(OPTION_SETS))
@pytest.mark.parametrize("bs,d", BWD_CASES)
def test_backward_small(gpu, bs, d, opt_name):
    """Several tiles per row and column, a block row with no live tile, a
    key block column with no live tile, a non-square grid; every gradient
    entry is checked."""
    opts = OPTION_SETS[opt_name]
    Mb, Nb, H, B = 5, 7, 4, 2
    Hkv = opts.get("Hkv", H)
    rng = np.random.default_rng(bs * 1000 + d + 11)
    lay = (rng.random((H, Mb, Nb)) < 0.45).astype(np.int32)
    lay[0, 3, :] = 0            # a block row with no live tile
    lay[:, :, 5] = 0            # a key block no query head reads
    lay[1, 0, :5] = 1
    lay[2, :, 6] = 1
    x = W.make_bsa("bwd", B=B, H=H, S=Mb * bs, Sk=Nb * bs, bs=bs, d=d, dtype="bf16",
                   layout="given", layout_array=lay, seed=bs + d + 5, Hkv=Hkv,
                   sink_mean=opts.get("sink_mean"))
    dout = W.upstream_gradient(x.q.shape, seed=bs * 7 + d)
    say(f"[backward] {opt_name} bs={bs} d={d} H={H} Hkv={Hkv}")
    plan, _ = check_plan(gpu, lay)
    pc = check_plan_cols(gpu, lay, Hkv)
    dq, dk, dv, dsink = _forward_backward(gpu, x, opts, plan, pc, dout)
    sink = None if x.sink is None else x.sink.numpy().astype(np.float64)
    rq, rk, rv, rs = O.attention_backward_dense(
        to64(x.q), to64(x.k), to64(x.v), to64(dout), lay, bs, x.scale, sink=sink,
        soft_cap=opts.get("soft_cap"), causal=opts.get("causal", False))
    compare_grad(to64(dq), rq, f"dq {opt_name} bs={bs} d={d}")
    compare_grad(to64(dk), rk, f"dk {opt_name} bs={bs} d={d}")
    compare_grad(to64(dv), rv, f"dv {opt_name} bs={bs} d={d}")
    assert torch.all(dq[:, 0, 3 * bs:4 * bs] == 0)
    assert torch.all(dk[:, :, 5 * bs:6 * bs] == 0) and torch.all(dv[:, :, 5 * bs:6 * bs] == 0)
    if rs is not None:
        out, lse = O.attention_dense_masked(
            to64(x.q), to64(x.k), to64(x.v), lay, bs, x.scale, sink=sink,
            soft_cap=opts.get("soft_cap"), causal=opts.get("causal", False))
        w = np.exp(sink[None, :, None] - lse)                       # [B, H, Sq]
        bound = 2.0 * 2.0 ** -9 * (w * np.abs(to64(dout) * out).sum(-1)).sum(axis=(0, 2))
        err = np.abs(dsink.cpu().numpy() - rs)
        say(f"  dsink: err {np.array2string(err, precision=2)} bound "
            f"{np.array2string(bound, precision=2)} (ref {np.abs(rs).max():.3e})")
        assert np.all(err <= bound + 1e-6)
    else:
        assert dsink is None


@pytest.mark.parametrize("causal", [False, True])
def test_backward_full_workload(gpu, causal):
    """The 32-head, 32768-token, bs-128 causal workload: sampled query blocks
    for dq and sampled key blocks for dk and dv against the oracle; two
    launches bit-identical.  With the element causal mask as well (the
    instances that mask the diagonal tiles only): every sampled block row
    and key block column holds its diagonal tile."""
    name = "causal_bernoulli_h32_s32768_bs128_d128"
    say(f"[backward] full {name} causal={causal}: generating inputs")
    x = W.make_workload(name)
    dout = W.upstream_gradient(x.q.shape, seed=41)
    plan, _ = check_plan(gpu, x.layout)
    H = x.layout.shape[0]
    pc = check_plan_cols(gpu, x.layout, H)
    say(f"[backward] full {name}: launching")
    g1 = _forward_backward(gpu, x, {"causal": causal}, plan, pc, dout)
    g2 = _forward_backward(gpu, x, {"causal": causal}, plan, pc, dout)
    for a, b in zip(g1[:3], g2[:3]):
        assert torch.equal(a, b), "backward is not deterministic"
    dq, dk, dv, _ = g1
    rng = np.random.default_rng(2)
    rows = _sample_row_blocks(x.layout, 1, 12, rng)
    Nb = x.layout.shape[2]
    cols = sorted({(0, int(rng.integers(H)), int(rng.integers(Nb))) for _ in range(8)}
                  | {(0, 0, 0), (0, H - 1, Nb - 1)})
    say(f"[backward] full {name}: oracle on {len(rows)} row blocks, {len(cols)} key blocks")
    rq, rk, rv, _ = O.attention_backward_live_tiles(
        to64(x.q), to64(x.k), to64(x.v), to64(dout), x.layout, x.bs, x.scale,
        row_blocks=rows, col_blocks=cols, causal=causal)
    bs = x.bs
    compare_grad(np.concatenate([to64(dq[b, h, m * bs:(m + 1) * bs]) for b, h, m in rows]),
                 np.concatenate([rq[b, h, m * bs:(m + 1) * bs] for b, h, m in rows]), "dq full")
    compare_grad(np.concatenate([to64(dk[b, j, n * bs:(n + 1) * bs]) for b, j, n in cols]),
                 np.concatenate([rk[b, j, n * bs:(n + 1) * bs] for b, j, n in cols]), "dk full")
    compare_grad(np.concatenate([to64(dv[b, j, n * bs:(n + 1) * bs]) for b, j, n in cols]),
                 np.concatenate([rv[b, j, n * bs:(n + 1) * bs] for b, j, n in cols]), "dv full")


@pytest.mark.parametrize("opt_name", ["plain", "all"])
@pytest.mark.parametrize("bs,d,Sq,Sk", [(32, 32, 160, 224), (64, 128, 320, 256),
                                        (128, 64, 256, 384), (64, 64, 250, 190),
                                        (16, 32, 96, 80), (16, 64, 75, 90)])
def test_backward_f32(gpu, bs, d, Sq, Sk, opt_name):
    """fp32 I/O: tiles are rounded to bf16 on load (as in the forward) and the
    gradients come back in fp32; compared with the oracle's gradients at the
    fp32 inputs, cut last blocks included."""
    opts = OPTION_SETS[opt_name]
    H, B = 4, 2
    Hkv = opts.get("Hkv", H)
    Mb, Nb = -(-Sq // bs), -(-Sk // bs)
    rng = np.random.default_rng(bs + d + Sq)
    lay = (rng.random((H, Mb, Nb)) < 0.5).astype(np.int32)
    lay[:, :, 0] = 1
    x = W.make_bsa("bwd_f32", B=B, H=H, S=Sq, Sk=Sk, bs=bs, d=d, dtype="f32", layout="given",
                   layout_array=lay, seed=Sq + Sk, Hkv=Hkv, sink_mean=opts.get("sink_mean"))
    dout = torch.from_numpy(np.random.default_rng(Sq).standard_normal(x.q.shape).astype(np.float32))
    say(f"[backward] f32 {opt_name} bs={bs} d={d} Sq={Sq} Sk={Sk}")
    plan, _ = check_plan(gpu, lay)
    pc = check_plan_cols(gpu, lay, Hkv)
    q, k, v = (t.to(gpu) for t in (x.q, x.k, x.v))
    sink = x.sink.to(gpu) if x.sink is not None else None
    kw = dict(attn_sink=sink, soft_cap=opts.get("soft_cap"), causal=opts.get("causal", False),
              bs=bs)
    out, lse = bsa.bsa_forward(q, k, v, plan, x.scale, **kw)
    dq, dk, dv, dsink = bsa.bsa_backward(q, k, v, out, dout.to(gpu), lse, plan, pc, x.scale, **kw)
    torch.cuda.synchronize()
    assert dq.dtype == torch.float32 and dk.dtype == torch.float32
    sk64 = None if x.sink is None else x.sink.numpy().astype(np.float64)
    rq, rk, rv, rs = O.attention_backward_dense(
        to64(x.q), to64(x.k), to64(x.v), to64(dout), lay, bs, x.scale, sink=sk64,
        soft_cap=opts.get("soft_cap"), causal=opts.get("causal", False))
    compare_grad(to64(dq), rq, f"dq f32 {opt_name} bs={bs} d={d}")
    compare_grad(to64(dk), rk, f"dk f32 {opt_name} bs={bs} d={d}")
    compare_grad(to64(dv), rv, f"dv f32 {opt_name} bs={bs} d={d}")


def test_backward_band_f32_config(gpu):
    """The fp32 band workload (B1 H2 S256 bs16 d32, layout |m - n| <= 1):
    every gradient entry against the oracle's dense gradients."""
    name = "band1_h2_s256_bs16_d32_f32"
    x = W.make_workload(name)
    dout = torch.from_numpy(np.random.default_rng(3).standard_normal(x.q.shape).astype(np.float32))
    say(f"[backward] {name}")
    plan, _ = check_plan(gpu, x.layout)
    pc = check_plan_cols(gpu, x.layout, x.layout.shape[0])
    q, k, v = (t.to(gpu) for t in (x.q, x.k, x.v))
    out, lse = bsa.bsa_forward(q, k, v, plan, x.scale)
    dq, dk, dv, _ = bsa.bsa_backward(q, k, v, out, dout.to(gpu), lse, plan, pc, x.scale)
    torch.cuda.synchronize()
    rq, rk, rv, _ = O.attention_backward_dense(to64(x.q), to64(x.k), to64(x.v), to64(dout),
                                               x.layout, x.bs, x.scale)
    compare_grad(to64(dq), rq, f"dq {name}")
    compare_grad(to64(dk), rk, f"dk {name}")
    compare_grad(to64(dv), rv, f"dv {name}")
