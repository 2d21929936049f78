"""GPU parity for sequence lengths that are not multiples of the block size.

The layout covers ceil(S / bs) blocks and the last block row / column is cut
at the sequence end (Language AI Handbook, create_block_sparse_mask).  Every
kernel family of the forward and the backward is run on cut lengths, with and
without the causal mask and a sink, against the fp64 oracle (same tolerances
as the whole-block tests), and outputs are written into views of larger
buffers whose remainder holds a sentinel that must survive: nothing is read
into the result or written past a sequence end.
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

SENTINEL = 12345.0


def padded(shape, dtype, dev):
    """A tensor of `shape` at the start of a buffer twice its size; the rest
    holds SENTINEL."""
    n = int(np.prod(shape))
    buf = torch.full((2 * n,), SENTINEL, dtype=dtype, device=dev)
    return buf, buf[:n].view(shape)


def sentinel_intact(buf, n):
    return bool(torch.all(buf[n:] == SENTINEL))


CASES = [  # bs, d, dtype, Sq, Sk
    (16, 64, "bf16", 5 * 16 - 3, 7 * 16 - 9),
    (16, 32, "f32", 33, 50),
    (32, 64, "bf16", 3 * 32 - 1, 4 * 32 - 20),
    (64, 128, "f32", 2 * 64 + 5, 3 * 64 - 63),
    (64, 128, "bf16", 4 * 64 - 17, 4 * 64 - 17),
    (128, 128, "bf16", 3 * 128 - 100, 5 * 128 - 1),
    (128, 64, "bf16", 130, 129),
]


@pytest.mark.parametrize("causal,sink", [(False, False), (True, True)])
@pytest.mark.parametrize("bs,d,dtype,Sq,Sk", CASES)
def test_forward_ragged(gpu, bs, d, dtype, Sq, Sk, causal, sink):
    H, B = 3, 2
    Mb, Nb = -(-Sq // bs), -(-Sk // bs)
    rng = np.random.default_rng(bs + d + Sq + Sk)
    lay = (rng.random((H, Mb, Nb)) < 0.5).astype(np.int32)
    lay[:, :, 0] = 1
    lay[:, :, Nb - 1] = 1                  # the cut last key block is always visited
    lay[0, Mb - 1, :] = 1                  # and the cut last query block sees everything
    x = W.make_bsa("ragged", B=B, H=H, S=Sq, Sk=Sk, bs=bs, d=d, dtype=dtype, layout="given",
                   layout_array=lay, seed=bs + Sq, sink_mean=1.0 if sink else None)
    say(f"[ragged] forward bs={bs} d={d} {dtype} Sq={Sq} Sk={Sk} causal={causal} sink={sink}")
    plan, _ = check_plan(gpu, lay)
    tdt = x.q.dtype
    obuf, out = padded((B, H, Sq, d), tdt, gpu)
    lbuf, lse = padded((B, H, Sq), torch.float32, gpu)
    s_ = x.sink.to(gpu) if sink else None
    bsa.bsa_forward(x.q.to(gpu), x.k.to(gpu), x.v.to(gpu), plan, x.scale, out=out, lse=lse,
                    attn_sink=s_, causal=causal, bs=bs)
    torch.cuda.synchronize()
    assert sentinel_intact(obuf, out.numel()) and sentinel_intact(lbuf, lse.numel())
    sk_ = None if not sink else x.sink.numpy().astype(np.float64)
    ref, ref_lse = O.attention_live_tiles(to64(x.q), to64(x.k), to64(x.v), lay, bs, x.scale,
                                          sink=sk_, causal=causal)
    compare(to64(out), ref, f"ragged bs={bs} d={d} {dtype}")
    if dtype == "f32":
        _, ref_lse = O.attention_live_tiles(bf16_rounded(x.q), bf16_rounded(x.k),
                                            bf16_rounded(x.v), lay, bs, x.scale, sink=sk_,
                                            causal=causal)
    compare_lse(lse.cpu().numpy(), ref_lse, f"ragged bs={bs} d={d}")


@pytest.mark.parametrize("causal,cap", [(False, None), (True, None), (True, 2.0)])
@pytest.mark.parametrize("bs,d,Sq,Sk", [(32, 64, 3 * 32 - 5, 4 * 32 - 31), (64, 128, 200, 150),
                                        (128, 128, 3 * 128 - 1, 2 * 128 + 3), (128, 32, 129, 300),
                                        (16, 32, 3 * 16 - 7, 5 * 16 + 1)])
def test_backward_ragged(gpu, bs, d, Sq, Sk, causal, cap):
    H, Hkv, B = 4, 2, 2
    Mb, Nb = -(-Sq // bs), -(-Sk // bs)
    rng = np.random.default_rng(bs * 3 + Sq + Sk)
    lay = (rng.random((H, Mb, Nb)) < 0.5).astype(np.int32)
    lay[:, :, Nb - 1] = 1
    lay[:, Mb - 1, 0] = 1
    x = W.make_bsa("ragged_bwd", B=B, H=H, S=Sq, Sk=Sk, bs=bs, d=d, dtype="bf16",
                   layout="given", layout_array=lay, seed=Sq + 7, Hkv=Hkv, sink_mean=1.0)
    dout = W.upstream_gradient(x.q.shape, seed=Sk)
    say(f"[ragged] backward bs={bs} d={d} Sq={Sq} Sk={Sk} causal={causal} cap={cap}")
    plan, _ = check_plan(gpu, lay)
    pc = check_plan_cols(gpu, lay, Hkv)
    q, k, v, sink = x.q.to(gpu), x.k.to(gpu), x.v.to(gpu), x.sink.to(gpu)
    out, lse = bsa.bsa_forward(q, k, v, plan, x.scale, attn_sink=sink, causal=causal, bs=bs,
                               soft_cap=cap)
    qb, dq = padded(tuple(q.shape), torch.bfloat16, gpu)
    kb, dk = padded(tuple(k.shape), torch.bfloat16, gpu)
    vb, dv = padded(tuple(v.shape), torch.bfloat16, gpu)
    _, _, _, dsink = bsa.bsa_backward(q, k, v, out, dout.to(gpu), lse, plan, pc, x.scale,
                                      attn_sink=sink, causal=causal, dq=dq, dk=dk, dv=dv, bs=bs,
                                      soft_cap=cap)
    torch.cuda.synchronize()
    for buf, t in ((qb, dq), (kb, dk), (vb, dv)):
        assert sentinel_intact(buf, t.numel())
    rq, rk, rv, rs = O.attention_backward_dense(
        to64(x.q), to64(x.k), to64(x.v), to64(dout), lay, bs, x.scale,
        sink=x.sink.numpy().astype(np.float64), causal=causal, soft_cap=cap)
    compare_grad(to64(dq), rq, f"dq ragged bs={bs}")
    compare_grad(to64(dk), rk, f"dk ragged bs={bs}")
    compare_grad(to64(dv), rv, f"dv ragged bs={bs}")
    # dsink: the bound derived for the whole-block backward tests (rounding
    # of the bf16 output inside D_i, twice 2^-9 of the summed magnitudes)
    sk64 = x.sink.numpy().astype(np.float64)
    o64, l64 = O.attention_dense_masked(to64(x.q), to64(x.k), to64(x.v), lay, bs, x.scale,
                                        sink=sk64, causal=causal, soft_cap=cap)
    w = np.exp(sk64[None, :, None] - l64)
    bound = 2.0 * 2.0 ** -9 * (w * np.abs(to64(dout) * o64).sum(-1)).sum(axis=(0, 2))
    assert np.all(np.abs(dsink.cpu().numpy() - rs) <= bound + 1e-6)
