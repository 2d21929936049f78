"""GPU parity of the top-k gathered attention at head sizes 128 and 256 (the
page's kernel takes d as a parameter) against the fp64 oracle, with the same
cases as the d = 512 tests: sinks, -1 slots, out-of-range entries, head
counts that are not multiples of 16, and a position with no valid slot; and
head counts above 64 at every head size."""

import numpy as np
import pytest
import torch

import block_sparse_attention_plan_amd as bsa
from block_sparse_attention_plan_amd import workloads as W
from oracle import bsa_oracle as O

from test_gpu_parity import compare, say, to64

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("H,topk,N,with_sink,drop", [
    (64, 200, 300, True, 0.05), (16, 65, 80, True, 0.3), (5, 1, 10, True, 0.0),
    (1, 130, 500, False, 0.1), (37, 127, 127, True, 0.5)])
def test_topk_head_dims(gpu, d, H, topk, N, with_sink, drop):
    t = W.make_topk("topk_dims", B=2, M=6, H=H, d=d, N=N, topk=topk, seed=H + topk + d,
                    drop=drop, with_sink=with_sink)
    idx = t.idx.clone()
    idx[0, 0, :] = -1                      # a position with no valid slot
    if topk > 2:
        idx[1, 1, 0] = N + 5               # out of range acts as missing
        idx[1, 1, 1] = -7
    say(f"[topk] d={d} H={H} topk={topk} N={N} sink={with_sink} drop={drop}")
    sink = t.sink.to(gpu) if with_sink else None
    out = bsa.topk_sparse_attn(t.q.to(gpu), t.kv.to(gpu), idx.to(gpu), sink, t.scale)
    torch.cuda.synchronize()
    ref_idx = idx.numpy().copy()
    ref_idx[(ref_idx < 0) | (ref_idx >= N)] = -1
    ref = O.topk_attention(to64(t.q), to64(t.kv), ref_idx,
                           t.sink.numpy() if with_sink else None, t.scale)
    compare(to64(out), ref, f"topk d={d} H={H}")
    assert torch.all(out[0, 0] == 0)


@pytest.mark.parametrize("d", [128, 256, 512])
@pytest.mark.parametrize("H,with_sink", [(65, True), (96, False), (128, True), (200, True)])
def test_topk_many_heads(gpu, d, H, with_sink):
    """More than 64 heads: the heads are served in groups of 64 (the last
    group partial), each group gathering the position's rows itself.  Every
    head of every position against the oracle, including a position with no
    valid slot and the sink of heads past the first group."""
    t = W.make_topk("topk_heads", B=2, M=5, H=H, d=d, N=150, topk=90, seed=H + d, drop=0.1,
                    with_sink=with_sink)
    idx = t.idx.clone()
    idx[0, 3] = -1
    say(f"[topk] many heads d={d} H={H} sink={with_sink}")
    sink = t.sink.to(gpu) if with_sink else None
    out = bsa.topk_sparse_attn(t.q.to(gpu), t.kv.to(gpu), idx.to(gpu), sink, t.scale)
    torch.cuda.synchronize()
    ref = O.topk_attention(to64(t.q), to64(t.kv), idx.numpy(),
                           t.sink.numpy() if with_sink else None, t.scale)
    compare(to64(out), ref, f"topk d={d} H={H}")
    assert torch.all(out[0, 3] == 0)


@pytest.mark.parametrize("d", [128, 256, 512])
@pytest.mark.parametrize("topk", [2048, 2049, 3000])
def test_topk_long_lists(gpu, d, topk):
    """Lists of up to 2048 slots have their valid indices compacted in LDS
    before chunks are formed; longer lists are read in place.  Both forms
    against the oracle, with -1 and out-of-range slots, a position whose only
    valid slots are its last three, and a position with none."""
    N = 4096
    t = W.make_topk("topk_long", B=1, M=4, H=20, d=d, N=N, topk=topk, seed=topk + d, drop=0.2,
                    with_sink=True)
    idx = t.idx.clone()
    idx[0, 1, :] = -1
    idx[0, 1, -3:] = torch.tensor([5, 17, N - 1], dtype=idx.dtype)
    idx[0, 2, :] = -1
    idx[0, 3, ::7] = N + 11
    say(f"[topk] long list d={d} topk={topk}")
    out = bsa.topk_sparse_attn(t.q.to(gpu), t.kv.to(gpu), idx.to(gpu), t.sink.to(gpu), t.scale)
    torch.cuda.synchronize()
    ref_idx = idx.numpy().copy()
    ref_idx[(ref_idx < 0) | (ref_idx >= N)] = -1
    ref = O.topk_attention(to64(t.q), to64(t.kv), ref_idx, t.sink.numpy(), t.scale)
    compare(to64(out), ref, f"topk long d={d} topk={topk}")
    assert torch.all(out[0, 2] == 0)


@pytest.mark.parametrize("d,N", [(128, 8193), (128, 65536), (128, 70000), (256, 4097),
                                 (256, 40000), (512, 2049), (512, 16384), (512, 20000)])
def test_topk_index_ranges(gpu, d, N):
    """The compacted list groups valid indices by table range (about 2 MiB of
    rows each, at most eight ranges, wider ones past that): two ranges with a
    last range of one row, exactly eight, and tables that widen the ranges.
    Positions with indices in descending order, all in the last range, and
    -1 / out-of-range slots, over two batch items (two tables); every output
    against the oracle, and two launches bit for bit."""
    t = W.make_topk("topk_ranges", B=2, M=4, H=20, d=d, N=N, topk=600, seed=N + d, drop=0.1,
                    with_sink=True)
    idx = t.idx.clone()
    idx[0, 1] = torch.sort(idx[0, 1], descending=True).values
    idx[0, 2, :] = torch.arange(N - 600, N, dtype=idx.dtype).flip(0)
    idx[0, 2, ::5] = N
    idx[0, 3, ::9] = -3
    idx[1, 0] = torch.sort(idx[1, 0]).values   # second batch item: its own table
    say(f"[topk] index ranges d={d} N={N}")
    q, kv, ig, sink = t.q.to(gpu), t.kv.to(gpu), idx.to(gpu), t.sink.to(gpu)
    out = bsa.topk_sparse_attn(q, kv, ig, sink, t.scale)
    out2 = bsa.topk_sparse_attn(q, kv, ig, sink, t.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "top-k is not deterministic"
    ref_idx = idx.numpy().copy()
    ref_idx[(ref_idx < 0) | (ref_idx >= N)] = -1
    ref = O.topk_attention(to64(t.q), to64(t.kv), ref_idx, t.sink.numpy(), t.scale)
    compare(to64(out), ref, f"topk ranges d={d} N={N}")
