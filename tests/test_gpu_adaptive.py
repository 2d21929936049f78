"""GPU parity of the content-adaptive layout (bsa_layout_adaptive) against
the fp64 oracle.

Scores are cosine similarities of fp32 block sums: against the fp64 oracle
on the same (bf16 or fp32) inputs they agree to 1e-5 absolute (sums of at
most 128 * 128 products of magnitude ~1 carry fp32 errors near 1e-6 of
their size).  A layout entry is a threshold decision, so it must match the
oracle's wherever the oracle's score is more than 1e-5 from tau; closer
entries may fall either way but must agree with the GPU's own score.
"""

import numpy as np
import pytest
import torch

import block_sparse_attention_plan_amd as bsa
from block_sparse_attention_plan_amd import workloads as W
from oracle import bsa_oracle as O

from test_gpu_parity import check_plan, compare, compare_lse, say, to64

pytestmark = pytest.mark.gpu

SCORE_ABS = 1e-5


def check_layout(gpu_layout, gpu_scores, q, k, bs, tau, causal, keep):
    ref, sim = O.adaptive_layout(to64(q), to64(k), bs, tau, causal=causal, keep_diagonal=keep)
    sc = gpu_scores.cpu().numpy().astype(np.float64)
    err = np.abs(sc - sim).max()
    say(f"  scores max_abs={err:.2e}; density {ref.mean():.3f}")
    assert err <= SCORE_ABS
    lay = gpu_layout.cpu().numpy()
    sure = np.abs(sim - tau) > SCORE_ABS
    assert np.array_equal(lay[sure], ref[sure])
    # near-threshold entries: consistent with the GPU's own score and the rules
    Mb, Nb = lay.shape[1], lay.shape[2]
    m = np.arange(Mb)[:, None]
    n = np.arange(Nb)[None, :]
    own = (sc >= tau)
    if causal:
        own &= (n <= m)[None]
    if keep:
        own |= (n == m)[None]
    assert np.array_equal(lay, own.astype(np.int32))
    return ref


@pytest.mark.parametrize("bs,d,dtype", [(16, 32, "bf16"), (32, 64, "bf16"), (64, 128, "bf16"),
                                        (128, 128, "bf16"), (64, 64, "f32"), (128, 32, "f32")])
@pytest.mark.parametrize("causal,keep", [(False, False), (True, True)])
def test_adaptive_random(gpu, bs, d, dtype, causal, keep):
    H, Hkv, Mb, Nb = 4, 2, 7, 9
    rng = np.random.default_rng(bs + d)
    q = torch.from_numpy(rng.standard_normal((H, Mb * bs, d)).astype(np.float32))
    k = torch.from_numpy(rng.standard_normal((Hkv, Nb * bs, d)).astype(np.float32))
    if dtype == "bf16":
        q, k = q.to(torch.bfloat16), k.to(torch.bfloat16)
    tau = 0.05
    say(f"[adaptive] random bs={bs} d={d} {dtype} causal={causal} keep={keep}")
    lay, sc = bsa.bsa_layout_adaptive(q.to(gpu), k.to(gpu), bs, tau, causal=causal,
                                      keep_diagonal=keep, want_scores=True)
    torch.cuda.synchronize()
    check_layout(lay, sc, q, k, bs, tau, causal, keep)


def test_adaptive_causal_without_scores(gpu):
    """Causal layout asked for without scores (tiles above the diagonal take
    a shortcut) equals the one computed with scores."""
    H, bs, d, S = 3, 16, 64, 16 * 150
    rng = np.random.default_rng(5)
    q = torch.from_numpy(rng.standard_normal((H, S, d)).astype(np.float32)).to(torch.bfloat16)
    k = torch.from_numpy(rng.standard_normal((H, S, d)).astype(np.float32)).to(torch.bfloat16)
    say("[adaptive] causal without scores, 150 x 150 blocks")
    a, sc = bsa.bsa_layout_adaptive(q.to(gpu), k.to(gpu), bs, 0.05, causal=True, want_scores=True)
    b, none = bsa.bsa_layout_adaptive(q.to(gpu), k.to(gpu), bs, 0.05, causal=True)
    torch.cuda.synchronize()
    assert none is None and torch.equal(a, b)
    check_layout(b, sc, q, k, bs, 0.05, True, True)


def test_adaptive_zero_blocks(gpu):
    """A zero block scores 0 against everything (no division by zero)."""
    q = torch.zeros((1, 64, 32), dtype=torch.bfloat16)
    k = torch.randn((1, 64, 32)).to(torch.bfloat16)
    lay, sc = bsa.bsa_layout_adaptive(q.to(gpu), k.to(gpu), 32, -0.5, keep_diagonal=False,
                                      want_scores=True)
    torch.cuda.synchronize()
    assert torch.all(sc == 0) and torch.all(lay == 1)


def test_adaptive_topics_full_size_and_pipeline(gpu):
    """32 heads (8 K/V heads), 32768 tokens, bs 128, d 128, topic-structured
    blocks: the layout matches the oracle, repeats bit for bit, and its plan
    and forward pass parity on sampled rows."""
    H, Hkv, S, d, bs = 32, 8, 32768, 128, 128
    q, k, tq, tk = W.make_topic_qk(H, Hkv, S, d, bs, n_topics=16, noise=2.0, seed=12)
    say("[adaptive] topics full size")
    qg, kg = q.to(gpu), k.to(gpu)
    lay, sc = bsa.bsa_layout_adaptive(qg, kg, bs, 0.5, causal=True, want_scores=True)
    lay2, sc2 = bsa.bsa_layout_adaptive(qg, kg, bs, 0.5, causal=True, want_scores=True)
    torch.cuda.synchronize()
    assert torch.equal(lay, lay2) and torch.equal(sc, sc2)
    ref = check_layout(lay, sc, q, k, bs, 0.5, True, True)
    # the layout found the topics: same-topic causal pairs are live, others mostly not
    same = (tq[:, :, None] == np.repeat(tk, H // Hkv, axis=0)[:, None, :])
    below = np.tril(np.ones(same.shape[1:], bool), -1)[None]     # causal, off the diagonal
    live = ref.astype(bool)
    say(f"  live|same-topic {live[same & below].mean():.3f}, "
        f"live|other {live[~same & below].mean():.3f}")
    assert live[same & below].mean() > 0.99 and live[~same & below].mean() < 0.01
    # plan + forward on the adaptive layout (first 2 heads, 4096 tokens), with
    # N(0, 1) attention inputs (the topic vectors only choose the layout)
    h2, s2 = 2, 4096
    sub = lay[:h2, :s2 // bs, :s2 // bs].contiguous()
    plan, _ = check_plan(gpu, sub.cpu().numpy())
    x = W.make_bsa("adaptive_pipeline", B=1, H=h2, S=s2, bs=bs, d=d, dtype="bf16",
                   layout="given", layout_array=sub.cpu().numpy(), seed=13)
    qs, ks, vs = x.q, x.k, x.v
    out, lse = bsa.bsa_forward(qs.to(gpu), ks.to(gpu), vs.to(gpu), plan)
    torch.cuda.synchronize()
    r_out, r_lse = O.attention_live_tiles(to64(qs), to64(ks), to64(vs), sub.cpu().numpy(), bs,
                                          1.0 / np.sqrt(d))
    compare(to64(out), r_out, "forward on the adaptive layout")
    compare_lse(lse.cpu().numpy(), r_lse, "forward on the adaptive layout")
