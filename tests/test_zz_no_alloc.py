"""bsa_backward_noalloc (no workspace, no allocation; static device scratch)
against bsa_backward (caller's workspace) through the C ABI.

Both run the same kernels, and the backward uses no atomics, so the two must
agree bit for bit.  Two calls in a row, the second on a smaller problem, so
the second call meets the first one's values in the shared scratch (nothing
there needs to start at zero).  Outputs are preallocated and passed in, as a
caller that cannot allocate would.
"""

import numpy as np
import pytest
import torch

import block_sparse_attention_plan_amd as bsa
from block_sparse_attention_plan_amd import workloads as W

from test_gpu_parity import say

pytestmark = pytest.mark.gpu

CASES = [
    # name, B, H, Hkv, S, bs, d, dtype, options
    ("large", 2, 8, 4, 1024, 64, 128, "bf16", dict(sink_mean=1.0, soft_cap=5.0, causal=True)),
    ("small", 1, 2, 2, 192, 32, 64, "bf16", dict()),
]


def _run_pair(gpu, name, B, H, Hkv, S, bs, d, dtype, opts):
    nb = S // bs
    rng = np.random.default_rng(nb * 7 + d)
    lay = (rng.random((H, nb, nb)) < 0.4).astype(np.int32)
    lay[:, np.arange(nb), np.arange(nb)] = 1
    x = W.make_bsa(f"noalloc_{name}", B=B, H=H, S=S, bs=bs, d=d, dtype=dtype, layout="given",
                   layout_array=lay, seed=nb + d, Hkv=Hkv, sink_mean=opts.get("sink_mean"))
    say(f"[noalloc] {name}: B={B} H={H} Hkv={Hkv} S={S} bs={bs} d={d} {opts}")
    q, k, v = x.q.to(gpu), x.k.to(gpu), x.v.to(gpu)
    layout = torch.from_numpy(lay).to(gpu)
    plan = bsa.bsa_plan(layout)
    pc = bsa.bsa_plan_cols(layout, kv_heads=Hkv)
    kw = dict(attn_sink=x.sink.to(gpu) if x.sink is not None else None,
              soft_cap=opts.get("soft_cap"), causal=opts.get("causal", False))
    out, lse = bsa.bsa_forward(q, k, v, plan, x.scale, **kw)
    dout = W.upstream_gradient(x.q.shape, seed=nb + 3).to(gpu)
    ref = bsa.bsa_backward(q, k, v, out, dout, lse, plan, pc, x.scale, **kw)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dsink = torch.empty(H, dtype=torch.float32, device=gpu) if x.sink is not None else None
    got = bsa.bsa_backward_noalloc(q, k, v, out, dout, lse, plan, pc, x.scale, dq=dq, dk=dk,
                                   dv=dv, dsink=dsink, **kw)
    torch.cuda.synchronize()
    assert got[0] is dq and got[1] is dk and got[2] is dv
    for what, a, b in zip(("dq", "dk", "dv", "dsink"), got, ref):
        if b is None:
            assert a is None
            continue
        assert torch.isfinite(a.float()).all(), what
        assert torch.equal(a, b), f"{name}: {what} differs from bsa_backward"
    say(f"  {name}: dq, dk, dv{', dsink' if dsink is not None else ''} bit-identical")


def test_noalloc_matches_backward_two_calls_second_smaller(gpu):
    for case in CASES:
        _run_pair(gpu, *case)


def test_noalloc_rejects_rows_beyond_scratch(gpu):
    """A problem with more query rows than the static scratch holds is refused with a clear
    error (host-side check; nothing is launched)."""
    lib = bsa.load_library()
    max_rows = lib.bsa_backward_noalloc_max_rows()
    # 33 batch items of one head, 65536 tokens, bs 128: 2,162,688 query rows;
    # a one-column layout keeps the plans small, and k and v hold one block
    B, H, S, bs, d = 33, 1, 65536, 128, 32
    assert B * H * S > max_rows
    q = torch.zeros((B, H, S, d), dtype=torch.bfloat16, device=gpu)
    lse = torch.zeros((B, H, S), dtype=torch.float32, device=gpu)
    layout = torch.ones((H, S // bs, 1), dtype=torch.int32, device=gpu)
    k = torch.zeros((B, H, bs, d), dtype=torch.bfloat16, device=gpu)
    plan = bsa.bsa_plan(layout)
    pc = bsa.bsa_plan_cols(layout)
    torch.cuda.synchronize()
    say(f"[noalloc] {B * H * S} query rows against a limit of {max_rows}")
    with pytest.raises(bsa.BsaError, match="static scratch"):
        bsa.bsa_backward_noalloc(q, k, k, q, q, lse, plan, pc, dq=torch.empty_like(q),
                                 dk=torch.empty_like(k), dv=torch.empty_like(k))
