"""The full-size parity helper (parity_full) on the CPU.

It splits the oracle by (batch item, head) or by runs of positions and farms
the slices out to worker processes.  Here it is fed the oracle's own result
for the whole tensor, so it must report agreement to fp32 rounding; a
mistake planted in one output element (on the CPU) must come back as the
maximum error, attributed to its slice.
"""

import numpy as np
import torch

from block_sparse_attention_plan_amd import workloads as W
from oracle import bsa_oracle as O

import parity_full as PF


def _f64(t):
    return t.float().numpy().astype(np.float64)


def test_bsa_full_matches_whole_tensor_oracle_and_finds_a_planted_error():
    rng = np.random.default_rng(5)
    H, Mb, bs = 4, 6, 32
    lay = (rng.random((H, Mb, Mb)) < 0.5).astype(np.int32)
    lay[2, 4, :] = 0  # an empty block row: lse = -inf there
    x = W.make_bsa("pf_host", B=2, H=H, S=Mb * bs, bs=bs, d=32, dtype="bf16", layout="given",
                   layout_array=lay, seed=3, Hkv=2, sink_mean=1.0)
    kw = dict(sink=_f64(x.sink), soft_cap=3.0, causal=True)
    ref, ref_lse = O.attention_live_tiles(_f64(x.q), _f64(x.k), _f64(x.v), lay, bs, x.scale, **kw)
    out = torch.from_numpy(ref.astype(np.float32))
    lse = torch.from_numpy(ref_lse.astype(np.float32))
    agg = PF.bsa_full(x.q, x.k, x.v, lay, bs, x.scale, out, lse, sink=x.sink, soft_cap=3.0,
                      causal=True)
    assert agg["slices"] == 2 * H
    assert agg["finite"] and agg["lse_pattern"]
    assert agg["max"] < 1e-6 and agg["lse_max"] < 1e-5
    out[1, 3, 17, 5] += 0.25
    lse[0, 1, 40] += 0.01
    agg = PF.bsa_full(x.q, x.k, x.v, lay, bs, x.scale, out, lse, sink=x.sink, soft_cap=3.0,
                      causal=True)
    assert abs(agg["max"] - 0.25) < 1e-6 and agg["worst"] == (1, 3)
    assert abs(agg["lse_max"] - 0.01) < 1e-5
    # without the options the same output no longer matches
    agg = PF.bsa_full(x.q, x.k, x.v, lay, bs, x.scale, out, lse)
    assert agg["max"] > 0.01


def test_topk_full_matches_whole_tensor_oracle_and_finds_a_planted_error():
    x = W.make_topk("pf_topk", B=2, M=10, H=5, d=128, N=40, topk=20, seed=4, drop=0.2)
    ref = O.topk_attention(_f64(x.q), _f64(x.kv), x.idx.numpy(), x.sink.numpy(), x.scale)
    out = torch.from_numpy(ref.astype(np.float32))
    agg = PF.topk_full(x.q, x.kv, x.idx, x.sink, x.scale, out, positions_per_task=3)
    assert agg["slices"] == 2 * 4 and agg["finite"]
    assert agg["max"] < 1e-6
    out[1, 7, 2, 100] -= 0.5
    agg = PF.topk_full(x.q, x.kv, x.idx, x.sink, x.scale, out, positions_per_task=3)
    assert abs(agg["max"] - 0.5) < 1e-6 and agg["worst"] == (1, 6)
