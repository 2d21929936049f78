"""GPU parity of the forward's optional terms against the fp64 oracle.

The options are those of the ejkernel BlockSparseAttention operation: a
per-head sink logit in the softmax denominator, a tanh cap on the scaled
scores, a causal mask on top of the layout and grouped K/V heads.  Each is
checked alone and all together on every kernel family (bs 16; bs 32; bs >= 64
fp32; bs >= 64 bf16 with tile copies), with rows that the causal mask empties
completely, rows with no live tile and a non-square block grid; then all of
them at once on the 32-head, 32768-token, bs-128 causal workload, on every
row, with two launches bit-identical.  Tolerances as in the plain
parity tests.
"""

import numpy as np
import pytest
import torch

import block_sparse_attention_plan_amd as bsa
from block_sparse_attention_plan_amd import workloads as W
from oracle import bsa_oracle as O

import parity_full as PF
from test_gpu_parity import (bf16_rounded, check_full, check_plan, compare, compare_lse, say,
                             to64)

pytestmark = pytest.mark.gpu

OPTION_SETS = {
    "sink": dict(sink_mean=3.0),
    "cap": dict(soft_cap=2.0),
    "causal": dict(causal=True),
    "gqa": dict(Hkv=2),
    "mqa_causal": dict(Hkv=1, causal=True),
    "all": dict(sink_mean=3.0, soft_cap=2.0, causal=True, Hkv=2),
}

KERNEL_CASES = [(16, 32, "f32"), (16, 64, "bf16"), (32, 64, "f32"), (32, 128, "bf16"),
                (64, 64, "f32"), (64, 32, "bf16"), (64, 128, "bf16"), (128, 32, "bf16"),
                (128, 128, "bf16")]


def _run(gpu, x, plan, opts, Hkv):
    sink = x.sink.to(gpu) if x.sink is not None else None
    q, k, v = (t.to(gpu) for t in (x.q, x.k, x.v))
    assert k.shape[1] == Hkv
    out, lse = bsa.bsa_forward(q, k, v, plan, x.scale, attn_sink=sink,
                               soft_cap=opts.get("soft_cap"), causal=opts.get("causal", False))
    return out, lse


def _oracle(x, opts, rows=None, rounded=False):
    conv = bf16_rounded if rounded else to64
    sink = None if x.sink is None else x.sink.numpy().astype(np.float64)
    return O.attention_live_tiles(conv(x.q), conv(x.k), conv(x.v), x.layout, x.bs, x.scale,
                                  row_blocks=rows, sink=sink, soft_cap=opts.get("soft_cap"),
                                  causal=opts.get("causal", False))


@pytest.mark.parametrize("opt_name", list(OPTION_SETS))
@pytest.mark.parametrize("bs,d,dtype", KERNEL_CASES)
def test_forward_options_small(gpu, bs, d, dtype, opt_name):
    opts = OPTION_SETS[opt_name]
    Mb, Nb, H, B = 5, 7, 4, 2
    Hkv = opts.get("Hkv", H)
    rng = np.random.default_rng(bs * 1000 + d + 7)
    lay = (rng.random((H, Mb, Nb)) < 0.45).astype(np.int32)
    lay[0, 3, :] = 0                        # no live tile
    lay[1, 0, :] = 1                        # full row: causal keeps its first tile only
    lay[2, :, 6] = 1                        # a column above the diagonal of every row
    lay[3, 1, :] = 0
    lay[3, 1, 4] = 1                        # only a tile that the causal mask empties
    x = W.make_bsa("options", B=B, H=H, S=Mb * bs, Sk=Nb * bs, bs=bs, d=d, dtype=dtype,
                   layout="given", layout_array=lay, seed=bs + d + 1, Hkv=Hkv,
                   sink_mean=opts.get("sink_mean"))
    say(f"[options] {opt_name} bs={bs} d={d} {dtype} H={H} Hkv={Hkv}")
    plan, _ = check_plan(gpu, lay)
    out, lse = _run(gpu, x, plan, opts, Hkv)
    torch.cuda.synchronize()
    ref, ref_lse = _oracle(x, opts)
    compare(to64(out), ref, f"{opt_name} bs={bs} d={d} {dtype}")
    if dtype == "f32":
        _, ref_lse = _oracle(x, opts, rounded=True)
    compare_lse(lse.cpu().numpy(), ref_lse, f"{opt_name} bs={bs} d={d}")
    # rows without a live key: zero output, lse = sink (or -inf); a row with
    # no live tile takes the sink logit as it is, a row the causal mask
    # empties goes through the log2-domain fold (rounding only)
    empty_rows = [(0, slice(3 * bs, 4 * bs), 0.0)]
    if opts.get("causal"):
        empty_rows.append((3, slice(1 * bs, 2 * bs), 1e-5))
    for h, rs, tol in empty_rows:
        assert torch.all(out[:, h, rs] == 0)
        got = lse[:, h, rs].cpu().numpy()
        if x.sink is None:
            assert np.all(np.isneginf(got))
        else:
            assert np.all(np.abs(got - float(x.sink[h])) <= tol * abs(float(x.sink[h])))


def test_forward_options_cap_saturates(gpu):
    """Raw scores far beyond the cap: the capped scores crowd at +-cap, so the
    weights of a row differ by at most a factor exp(2 cap); without the cap
    the softmax would be close to one-hot."""
    bs, d, Mb = 64, 64, 3
    lay = np.ones((2, Mb, Mb), np.int32)
    x = W.make_bsa("cap_saturation", B=1, H=2, S=Mb * bs, bs=bs, d=d, dtype="bf16",
                   layout="given", layout_array=lay, seed=11, std=4.0)
    say("[options] cap saturation bs=64 d=64 std=4 cap=0.5")
    plan, _ = check_plan(gpu, lay)
    out, lse = _run(gpu, x, plan, dict(soft_cap=0.5), 2)
    torch.cuda.synchronize()
    ref, ref_lse = _oracle(x, dict(soft_cap=0.5))
    compare(to64(out), ref, "cap saturation", bf16_out_rounding=True)
    compare_lse(lse.cpu().numpy(), ref_lse, "cap saturation")


def test_forward_options_full_workload(gpu):
    """All options at the full 32-head, 32768-token, bs-128 causal workload
    (eight K/V heads); the oracle checks every row."""
    name = "causal_bernoulli_h32_s32768_bs128_d128"
    opts = dict(sink_mean=3.0, soft_cap=1.0, causal=True, Hkv=8)
    say(f"[options] full {name} {opts}: generating inputs")
    x = W.make_workload(name, Hkv=8, sink_mean=3.0)
    plan, _ = check_plan(gpu, x.layout)
    say(f"[options] full {name}: launching")
    out, lse = _run(gpu, x, plan, opts, 8)
    out2, lse2 = _run(gpu, x, plan, opts, 8)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2), "forward is not deterministic"
    say(f"[options] full {name}: oracle on every row")
    agg = PF.bsa_full(x.q, x.k, x.v, x.layout, x.bs, x.scale, out, lse, sink=x.sink,
                      soft_cap=1.0, causal=True)
    check_full(agg, f"{name} options")
