"""GPU parity: libbsa (through the C ABI) against the fp64 CPU oracle.

Plans must match bit for bit.  Attention outputs must be within max-abs
1.5e-2 and mean-abs 2e-3 of the oracle (bf16 I/O, fp32 accumulation), lse
within 1e-3 where finite and exactly -inf for rows without a live tile.
Inputs are the seeded synthetic workloads; at full size every output row
(and every top-k position) is checked, the oracle running per head (per run
of positions) in a pool of host processes.
"""

import sys
import zlib

import numpy as np
import pytest
import torch

import block_sparse_attention_plan_amd as bsa
from block_sparse_attention_plan_amd import workloads as W
from oracle import bsa_oracle as O

import parity_full as PF

pytestmark = pytest.mark.gpu

MAX_ABS = 1.5e-2
MEAN_ABS = 2e-3
LSE_ABS = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_plan(dev, layout: np.ndarray):
    """The GPU plan against the oracle's, bit for bit: rows, and the pairs of
    neighbouring rows with their use flag."""
    ref = O.plan(layout)
    p = bsa.bsa_plan(torch.from_numpy(np.ascontiguousarray(layout, dtype=np.int32)).to(dev))
    nnz = p.nnz()
    assert nnz == ref.nnz_total
    assert torch.equal(p.row_ptr.cpu(), torch.from_numpy(ref.row_ptr))
    assert torch.equal(p.row_order.cpu(), torch.from_numpy(ref.row_order))
    assert torch.equal(p.col_idx(nnz).cpu(), torch.from_numpy(ref.col_idx))
    pref = O.plan_pairs(layout)
    info = p.pair_info.cpu().tolist()
    assert info == [pref.pair_total, pref.use_pairs]
    assert torch.equal(p.pair_ptr.cpu(), torch.from_numpy(pref.pair_ptr))
    assert torch.equal(p.pair_order.cpu(), torch.from_numpy(pref.pair_order))
    assert torch.equal(p.pair_cols(pref.pair_total).cpu(), torch.from_numpy(pref.pair_cols))
    return p, ref


def compare(out_gpu: np.ndarray, out_ref: np.ndarray, what: str, bf16_out_rounding: bool = False):
    """Output tolerance: max-abs 1.5e-2, mean-abs 2e-3.  With
    bf16_out_rounding the max-abs bound also allows the rounding of the bf16
    output itself (2^-8 |ref|), which exceeds 1.5e-2 once |out| >= 4 --
    outputs that large only arise when a test pushes the softmax towards
    one-hot."""
    assert np.isfinite(out_gpu).all(), f"{what}: non-finite output"
    err = np.abs(out_gpu - out_ref)
    say(f"  {what}: max_abs={err.max():.3e} mean_abs={err.mean():.3e}")
    bound = MAX_ABS + (np.abs(out_ref) * 2.0 ** -8 if bf16_out_rounding else 0.0)
    assert np.all(err <= bound), what
    assert err.mean() <= MEAN_ABS, what


def bf16_rounded(t: torch.Tensor) -> np.ndarray:
    """fp32 inputs as the kernel multiplies them: rounded to bf16 on load."""
    return to64(t.to(torch.bfloat16))


def compare_lse(lse_gpu: np.ndarray, lse_ref: np.ndarray, what: str):
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse_gpu), empty), f"{what}: -inf pattern differs"
    fin = ~empty
    if fin.any():
        err = np.abs(lse_gpu[fin] - lse_ref[fin]).max()
        say(f"  {what}: lse max_abs={err:.3e}")
        assert err <= LSE_ABS


# ------------------------------------------------------------------ planner

@pytest.mark.parametrize("case", [
    ("empty", (2, 3, 5), 0.0), ("full", (1, 4, 4), 1.0), ("one_col", (3, 70, 1), 0.5),
    ("wide", (2, 5, 200), 0.2), ("tall", (2, 300, 40), 0.15), ("ragged", (4, 33, 65), 0.4),
    ("square", (8, 64, 64), 0.1)])
def test_plan_random_layouts(gpu, case):
    name, (H, Mb, Nb), p = case
    say(f"[plan] {name} H={H} Mb={Mb} Nb={Nb} p={p}")
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    lay = (rng.random((H, Mb, Nb)) < p).astype(np.int32) * rng.integers(1, 4, (H, Mb, Nb)).astype(np.int32)
    check_plan(gpu, lay)


@pytest.mark.parametrize("name", [n for n, s in W.WORKLOADS.items() if s["kind"] == "bsa"])
def test_plan_workload_layouts(gpu, name):
    spec = W.WORKLOADS[name]
    nb = spec["S"] // spec["bs"]
    H = spec["H"]
    say(f"[plan] workload {name} H={H} nb={nb}")
    if spec["layout"] == "band":
        lay = W.band_layout(H, nb, spec["w"])
    elif spec["layout"] == "causal_lgs":
        lay = W.causal_lgs_layout(H, nb, spec["window"], spec["n_global"], spec["stride"])
    else:
        lay = W.causal_bernoulli_layout(H, nb, spec["p"], np.random.default_rng(spec["seed"]))
    check_plan(gpu, lay)


# ------------------------------------------------------- block-sparse forward

SMALL_CASES = []
for bs_ in (16, 32, 64, 128):
    for d_ in (32, 64, 128):
        SMALL_CASES.append((bs_, d_, "bf16"))
SMALL_CASES += [(16, 32, "f32"), (64, 128, "f32"), (128, 64, "f32")]


@pytest.mark.parametrize("bs,d,dtype", SMALL_CASES)
def test_forward_small_all_rows(gpu, bs, d, dtype):
    """Several tiles per row with ragged per-row counts, an empty block row,
    a non-square block grid; every output row is checked."""
    Mb, Nb, H, B = 5, 7, 3, 2
    rng = np.random.default_rng(bs * 1000 + d)
    lay = (rng.random((H, Mb, Nb)) < 0.45).astype(np.int32)
    lay[0, 3, :] = 0          # empty block row
    lay[1, 0, :] = 1          # full row
    lay[2, :, 6] = 1
    x = W.make_bsa("small", B=B, H=H, S=Mb * bs, Sk=Nb * bs, bs=bs, d=d, dtype=dtype,
                   layout="given", layout_array=lay, seed=bs + d)
    say(f"[forward] small bs={bs} d={d} {dtype}")
    plan, _ = check_plan(gpu, lay)
    q, k, v = (t.to(gpu) for t in (x.q, x.k, x.v))
    out, lse = bsa.bsa_forward(q, k, v, plan, x.scale)
    torch.cuda.synchronize()
    ref, ref_lse = O.attention_live_tiles(to64(x.q), to64(x.k), to64(x.v), lay, bs, x.scale)
    compare(to64(out), ref, f"bs={bs} d={d} {dtype}")
    if dtype == "f32":
        # lse is compared with the oracle on the bf16-rounded values the
        # kernel multiplies (fp32 I/O rounds tiles to bf16 on load).
        _, ref_lse = O.attention_live_tiles(bf16_rounded(x.q), bf16_rounded(x.k),
                                            bf16_rounded(x.v), lay, bs, x.scale)
    compare_lse(lse.cpu().numpy(), ref_lse, f"bs={bs} d={d}")
    assert torch.all(out[0, 0, 3 * bs:4 * bs] == 0)


def test_forward_all_empty_layout(gpu):
    lay = np.zeros((2, 3, 3), np.int32)
    x = W.make_bsa("empty", B=1, H=2, S=48, bs=16, d=32, dtype="bf16", layout="given",
                   layout_array=lay, seed=9)
    say("[forward] all-empty layout")
    plan, _ = check_plan(gpu, lay)
    out, lse = bsa.bsa_forward(x.q.to(gpu), x.k.to(gpu), x.v.to(gpu), plan)
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


def _sample_row_blocks(layout, B, k, rng):
    """k row blocks (b, h, m), always including the heaviest and the lightest."""
    H, Mb, _ = layout.shape
    nnz = (layout != 0).sum(-1)
    picks = set()
    for b in range(B):
        h, m = np.unravel_index(np.argmax(nnz), nnz.shape)
        picks.add((b, int(h), int(m)))
        h, m = np.unravel_index(np.argmin(nnz), nnz.shape)
        picks.add((b, int(h), int(m)))
    while len(picks) < k:
        picks.add((int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(Mb))))
    return sorted(picks)


def check_full(agg, what: str, with_lse: bool = True):
    """Aggregate statistics of parity_full against the output bounds."""
    line = (f"{what}: all {agg['slices']} slices: max_abs={agg['max']:.3e} "
            f"mean_abs={agg['mean']:.3e} (worst slice {agg['worst']})"
            + (f", lse max_abs={agg['lse_max']:.3e}" if with_lse else ""))
    say("  " + line)
    PF.REPORT.append(line)
    assert agg["finite"], f"{what}: non-finite output"
    assert agg["max"] <= MAX_ABS, what
    assert agg["mean"] <= MEAN_ABS, what
    if with_lse:
        assert agg["lse_pattern"], f"{what}: -inf pattern of lse differs"
        assert agg["lse_max"] <= LSE_ABS, what


@pytest.mark.parametrize("name", [n for n, s in W.WORKLOADS.items() if s["kind"] == "bsa"])
def test_forward_full_workloads(gpu, name):
    """Full-size workloads in the launch configuration the benchmark times;
    the oracle checks every output row and every lse.  Two runs must agree bit
    for bit."""
    say(f"[forward] full workload {name}: generating inputs")
    x = W.make_workload(name)
    B = x.q.shape[0]
    plan, _ = check_plan(gpu, x.layout)
    q, k, v = (t.to(gpu) for t in (x.q, x.k, x.v))
    say(f"[forward] full workload {name}: launching")
    out, lse = bsa.bsa_forward(q, k, v, plan, x.scale)
    out2, lse2 = bsa.bsa_forward(q, k, v, plan, x.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2), "forward is not deterministic"
    nrows = B * x.layout.shape[0] * x.layout.shape[1]
    if nrows <= 1024:
        ref, ref_lse = O.attention_live_tiles(to64(x.q), to64(x.k), to64(x.v), x.layout, x.bs,
                                              x.scale)
        compare(to64(out), ref, name)
        if x.q.dtype == torch.float32:
            _, ref_lse = O.attention_live_tiles(bf16_rounded(x.q), bf16_rounded(x.k),
                                                bf16_rounded(x.v), x.layout, x.bs, x.scale)
        compare_lse(lse.cpu().numpy(), ref_lse, name)
    else:
        say(f"[forward] full workload {name}: oracle on every row")
        agg = PF.bsa_full(x.q, x.k, x.v, x.layout, x.bs, x.scale, out, lse)
        check_full(agg, name)


# ------------------------------------------------------------------- top-k

TOPK_CASES = [
    # H, topk, N, with_sink, drop
    (64, 200, 300, True, 0.05),
    (64, 64, 100, False, 0.0),
    (16, 65, 80, True, 0.3),
    (5, 1, 10, True, 0.0),
    (1, 130, 500, False, 0.1),
    (37, 127, 127, True, 0.5),
]


@pytest.mark.parametrize("H,topk,N,with_sink,drop", TOPK_CASES)
def test_topk_small(gpu, H, topk, N, with_sink, drop):
    say(f"[topk] small H={H} topk={topk} N={N} sink={with_sink} drop={drop}")
    x = W.make_topk("topk_small", B=2, M=6, H=H, d=512, N=N, topk=topk, seed=H + topk,
                    drop=drop, with_sink=with_sink)
    idx = x.idx.clone()
    idx[1, 4] = -1            # a position with no valid slot
    out = bsa.topk_sparse_attn(x.q.to(gpu), x.kv.to(gpu), idx.to(gpu),
                               x.sink.to(gpu) if x.sink is not None else None, x.scale)
    torch.cuda.synchronize()
    ref = O.topk_attention(to64(x.q), to64(x.kv), idx.numpy(),
                           x.sink.numpy() if x.sink is not None else None, x.scale)
    compare(to64(out), ref, f"topk H={H} topk={topk}")
    assert torch.all(out[1, 4] == 0)


def test_topk_full_workload(gpu):
    name = "topk2048_m4096_h64_d512_n8192"
    say(f"[topk] full workload {name}: generating inputs")
    x = W.make_workload(name)
    q, kv, idx, sink = x.q.to(gpu), x.kv.to(gpu), x.idx.to(gpu), x.sink.to(gpu)
    say(f"[topk] full workload {name}: launching")
    out = bsa.topk_sparse_attn(q, kv, idx, sink, x.scale)
    out2 = bsa.topk_sparse_attn(q, kv, idx, sink, x.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "top-k is not deterministic"
    say(f"[topk] full workload {name}: oracle on every position")
    agg = PF.topk_full(x.q, x.kv, x.idx, x.sink, x.scale, out)
    check_full(agg, name, with_lse=False)


@pytest.mark.parametrize("bs,d", [(16, 64), (32, 64), (64, 128), (128, 128)])
def test_forward_growing_scores(gpu, bs, d):
    """Scores that grow by large factors from tile to tile, in both directions
    of the row, so the running maximum is raised (and O rescaled) many times."""
    Mb, Nb, H = 2, 6, 2
    lay = np.ones((H, Mb, Nb), np.int32)
    lay[1, 1, ::2] = 0
    x = W.make_bsa("grow", B=1, H=H, S=Mb * bs, Sk=Nb * bs, bs=bs, d=d, dtype="bf16",
                   layout="given", layout_array=lay, seed=bs + 3 * d)
    ramp = torch.repeat_interleave(torch.tensor([1.0, 6.0, 0.5, 14.0, 2.0, 30.0]), bs)
    k = (x.k.float() * ramp[None, None, :, None]).to(torch.bfloat16)
    say(f"[forward] growing scores bs={bs} d={d}")
    plan, _ = check_plan(gpu, lay)
    out, lse = bsa.bsa_forward(x.q.to(gpu), k.to(gpu), x.v.to(gpu), plan, x.scale)
    torch.cuda.synchronize()
    ref, ref_lse = O.attention_live_tiles(to64(x.q), to64(k), to64(x.v), lay, bs, x.scale)
    compare(to64(out), ref, f"grow bs={bs} d={d}", bf16_out_rounding=True)
    fin = np.isfinite(ref_lse)
    err = np.abs(lse.cpu().numpy()[fin] - ref_lse[fin]) / np.maximum(1.0, np.abs(ref_lse[fin]))
    say(f"  lse rel err {err.max():.2e}")
    assert err.max() <= 1e-3


# ------------------------------------------------------------- edge cases

def test_plan_widest_row(gpu):
    """Block rows as wide as the planner accepts (16384 columns), a few ragged
    densities, one row empty and one full."""
    H, Mb, Nb = 2, 3, 16384
    rng = np.random.default_rng(11)
    lay = (rng.random((H, Mb, Nb)) < np.array([0.001, 0.3, 0.9])[None, :, None]).astype(np.int32)
    lay[0, 0, :] = 0
    lay[1, 2, :] = 1
    say(f"[plan] widest rows H={H} Mb={Mb} Nb={Nb}")
    check_plan(gpu, lay)


def test_topk_out_of_range_indices_act_as_missing(gpu):
    """Entries outside [0, N) other than -1 are documented to contribute
    nothing, exactly as -1 does: the result equals the oracle's on the same
    input with those entries replaced by -1."""
    x = W.make_topk("topk_oob", B=1, M=5, H=24, d=512, N=90, topk=70, seed=21, drop=0.1)
    idx = x.idx.clone()
    idx[0, 0, 3] = 90            # == N
    idx[0, 1, 0] = 1 << 30
    idx[0, 2, 69] = -7
    idx[0, 3, :40] = -2          # a leading run of bad entries
    say("[topk] out-of-range entries")
    out = bsa.topk_sparse_attn(x.q.to(gpu), x.kv.to(gpu), idx.to(gpu), x.sink.to(gpu), x.scale)
    torch.cuda.synchronize()
    clean = idx.numpy().copy()
    clean[(clean < 0) | (clean >= 90)] = -1
    ref = O.topk_attention(to64(x.q), to64(x.kv), clean, x.sink.numpy(), x.scale)
    compare(to64(out), ref, "topk out-of-range entries")


def test_topk_duplicates_and_late_valid_slots(gpu):
    """Repeated rows count once per slot; a position whose first chunks hold
    no valid slot starts its running max from a later chunk."""
    x = W.make_topk("topk_dup", B=2, M=4, H=64, d=512, N=50, topk=50, seed=22, drop=0.0)  # q, kv, sink
    rng = np.random.default_rng(23)
    idx = torch.from_numpy(rng.integers(0, 50, (2, 4, 160)).astype(np.int32))  # with repeats
    idx[0, 1, :130] = -1         # only the last chunk holds valid slots
    idx[1, 2, :] = 7             # one row, 160 times
    say("[topk] duplicates and late valid slots")
    out = bsa.topk_sparse_attn(x.q.to(gpu), x.kv.to(gpu), idx.to(gpu), x.sink.to(gpu), x.scale)
    torch.cuda.synchronize()
    ref = O.topk_attention(to64(x.q), to64(x.kv), idx.numpy(), x.sink.numpy(), x.scale)
    compare(to64(out), ref, "topk duplicates")


@pytest.mark.parametrize("name", ["causal_lgs_b2_h16_s16384_bs64_d128",
                                  "causal_bernoulli_h32_s32768_bs128_d128"])
def test_forward_repeatable(gpu, name):
    """Five launches on the full workload give bit-identical out and lse.  A
    copy read before it has landed shows up here as a few differing row
    groups, not as a tolerance failure."""
    x = W.make_workload(name)
    q, k, v = x.q.to(gpu), x.k.to(gpu), x.v.to(gpu)
    plan = bsa.bsa_plan(torch.from_numpy(x.layout).to(gpu))
    say(f"[forward] repeatability {name}")
    out0, lse0 = bsa.bsa_forward(q, k, v, plan, x.scale)
    for _ in range(4):
        out, lse = bsa.bsa_forward(q, k, v, plan, x.scale)
        torch.cuda.synchronize()
        assert torch.equal(out, out0) and torch.equal(lse, lse0)
