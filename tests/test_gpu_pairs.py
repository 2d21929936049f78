"""GPU parity of the paired forward: work items that cover two neighbouring
block rows and load each tile the two rows share once (bf16, bs = 64, plain
scores; the plan's use-pairs flag set).

Layouts are local windows with global and strided columns, the patterns whose
neighbouring rows repeat their columns, with the cases the pairing meets: an
odd number of block rows (the last pair has one row), a row with no live
tile beside a row with many, a pair with no live tile at all, several heads
and batch items, grouped K/V heads and a sink.  Every row of out and lse is
checked against the oracle with the tolerances of the other parity tests.
"""

import numpy as np
import pytest
import torch

import block_sparse_attention_plan_amd as bsa
from block_sparse_attention_plan_amd import workloads as W
from oracle import bsa_oracle as O

from test_gpu_parity import check_plan, compare, compare_lse, say, to64

pytestmark = pytest.mark.gpu


def shared_layout(H, Mb, Nb, seed):
    """Causal window of radius 2, two global columns, a per-head stride of 3;
    row 3 of head 0 empty (its partner, row 2, is not), rows 4 and 5 of the
    last head empty (a whole pair)."""
    lay = np.zeros((H, Mb, Nb), np.int32)
    for h in range(H):
        for m in range(Mb):
            for n in range(Nb):
                if n <= m and (m - n <= 2 or n < 2 or n % 3 == h % 3):
                    lay[h, m, n] = 1
    lay[0, 3, :] = 0
    if Mb > 5:
        lay[H - 1, 4:6, :] = 0
    rng = np.random.default_rng(seed)
    lay[rng.random(lay.shape) < 0.05] = 0  # a few holes, so the rows differ
    return lay


CASES = [
    # d, B, H, Hkv, Mb, sink
    (128, 2, 3, 3, 7, False),
    (128, 1, 4, 2, 8, True),
    (64, 2, 2, 1, 9, True),
    (32, 1, 5, 5, 6, False),
]


@pytest.mark.parametrize("d,B,H,Hkv,Mb,with_sink", CASES)
def test_paired_forward(gpu, d, B, H, Hkv, Mb, with_sink):
    bs = 64
    lay = shared_layout(H, Mb, Mb, seed=d + Mb)
    pref = O.plan_pairs(lay)
    assert pref.use_pairs == 1, "test layout must select the paired form"
    x = W.make_bsa("pairs", B=B, H=H, S=Mb * bs, bs=bs, d=d, dtype="bf16", layout="given",
                   layout_array=lay, seed=3 * d + Mb, Hkv=Hkv,
                   sink_mean=1.0 if with_sink else None)
    say(f"[pairs] d={d} B={B} H={H} Hkv={Hkv} Mb={Mb} sink={with_sink} "
        f"({pref.pair_total} pair entries for {int(lay.sum())} tiles)")
    plan, _ = check_plan(gpu, lay)
    q, k, v = x.q.to(gpu), x.k.to(gpu), x.v.to(gpu)
    sink = x.sink.to(gpu) if with_sink else None
    out, lse = bsa.bsa_forward(q, k, v, plan, x.scale, attn_sink=sink)
    out2, lse2 = bsa.bsa_forward(q, k, v, plan, x.scale, attn_sink=sink)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    ref, ref_lse = O.attention_live_tiles(to64(x.q), to64(x.k), to64(x.v), lay, bs, x.scale,
                                          sink=None if sink is None else to64(x.sink))
    compare(to64(out), ref, f"pairs d={d}")
    compare_lse(lse.cpu().numpy(), ref_lse, f"pairs d={d}")
    if not with_sink:
        assert torch.all(out[:, 0, 3 * bs:4 * bs] == 0)          # the empty row of head 0
        assert torch.all(torch.isneginf(lse[:, 0, 3 * bs:4 * bs]))


def test_paired_layout_with_score_options_uses_rows(gpu):
    """With a causal mask the forward keeps its per-row form even when the
    layout would pair; the result is unchanged against the oracle."""
    bs, d, H, Mb = 64, 128, 2, 6
    lay = shared_layout(H, Mb, Mb, seed=5)
    x = W.make_bsa("pairs_causal", B=1, H=H, S=Mb * bs, bs=bs, d=d, dtype="bf16",
                   layout="given", layout_array=lay, seed=17)
    say("[pairs] layout that pairs, with causal and a cap: per-row kernels")
    plan, _ = check_plan(gpu, lay)
    out, lse = bsa.bsa_forward(x.q.to(gpu), x.k.to(gpu), x.v.to(gpu), plan, x.scale,
                               causal=True, soft_cap=3.0)
    torch.cuda.synchronize()
    ref, ref_lse = O.attention_live_tiles(to64(x.q), to64(x.k), to64(x.v), lay, bs, x.scale,
                                          causal=True, soft_cap=3.0)
    compare(to64(out), ref, "pairs layout, causal + cap")
    compare_lse(lse.cpu().numpy(), ref_lse, "pairs layout, causal + cap")
