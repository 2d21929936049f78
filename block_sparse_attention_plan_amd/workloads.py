"""Seeded synthetic inputs for block-sparse and top-k attention.

This module only draws inputs: random tensors, block layouts and index lists.
It holds none of the attention arithmetic, so the GPU path and the CPU
reference can both consume its output without sharing any of the method.

Every workload is drawn from ``numpy.random.default_rng(seed)`` (PCG64) in a
fixed order -- q, k, v (or kv), then the layout's random draws or the top-k
indices, then the -1 slot mask, then the sink -- as float32 normals scaled by
the stated standard deviation and rounded to bf16 (round to nearest even)
unless the workload is fp32.

Layout families (block level; "live" = non-zero):
  band              |i - j| <= w                       (local attention band)
  causal_lgs        j <= i and (i - j <= window or j < n_global or i < n_global
                    or j % stride == h % stride)        (local + global + strided)
  causal_bernoulli  (j < i and u_hij < p) or j == i,  u ~ U[0, 1) per head
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np
import torch

__all__ = [
    "BsaInputs",
    "TopkInputs",
    "WORKLOADS",
    "band_layout",
    "causal_lgs_layout",
    "causal_bernoulli_layout",
    "make_bsa",
    "make_topk",
    "make_workload",
]


@dataclass
class BsaInputs:
    name: str
    q: torch.Tensor          # CPU [B, H, S, d], bf16 or fp32
    k: torch.Tensor          # CPU [B, Hkv, Sk, d]
    v: torch.Tensor
    layout: np.ndarray       # int32 [H, Mb, Nb]
    bs: int
    scale: float
    seed: int
    params: Dict = field(default_factory=dict)
    sink: Optional[torch.Tensor] = None  # CPU fp32 [H] or None


@dataclass
class TopkInputs:
    name: str
    q: torch.Tensor          # CPU bf16 [B, M, H, d]
    kv: torch.Tensor         # CPU bf16 [B, N, d]
    idx: torch.Tensor        # CPU int32 [B, M, topk]
    sink: Optional[torch.Tensor]  # CPU fp32 [H] or None
    scale: float
    seed: int
    params: Dict = field(default_factory=dict)


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _tensor(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(x)
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f32":
        return t.contiguous()
    raise ValueError(dtype)


def band_layout(H: int, nb: int, w: int) -> np.ndarray:
    i = np.arange(nb)[:, None]
    j = np.arange(nb)[None, :]
    one = (np.abs(i - j) <= w).astype(np.int32)
    return np.ascontiguousarray(np.broadcast_to(one, (H, nb, nb)))


def causal_lgs_layout(H: int, nb: int, window: int = 4, n_global: int = 2,
                      stride: int = 8) -> np.ndarray:
    i = np.arange(nb)[None, :, None]
    j = np.arange(nb)[None, None, :]
    h = np.arange(H)[:, None, None]
    live = (j <= i) & ((i - j <= window) | (j < n_global) | (i < n_global)
                       | ((j % stride) == (h % stride)))
    return live.astype(np.int32)


def causal_bernoulli_layout(H: int, nb: int, p: float, rng: np.random.Generator) -> np.ndarray:
    u = rng.random((H, nb, nb))
    i = np.arange(nb)[None, :, None]
    j = np.arange(nb)[None, None, :]
    live = ((j < i) & (u < p)) | (j == i)
    return live.astype(np.int32)


def make_bsa(name: str, B: int, H: int, S: int, bs: int, d: int, dtype: str, layout: str,
             seed: int, std: float = 1.0, Sk: Optional[int] = None, Hkv: Optional[int] = None,
             sink_mean: Optional[float] = None, **kw) -> BsaInputs:
    """Draw q, k, v and a layout.  ``layout`` names a family above, or
    ``"given"`` with ``kw['layout_array']``.  ``Hkv`` (default H) is the
    number of K/V heads; with ``sink_mean`` a per-head sink logit
    N(sink_mean, 1) is drawn last, so the other draws do not depend on it."""
    Sk = S if Sk is None else Sk
    Hkv = H if Hkv is None else Hkv
    if (S % bs or Sk % bs) and layout not in ("given", "random"):
        raise ValueError("the named layout families need lengths that are multiples of bs")
    if Hkv < 1 or H % Hkv:
        raise ValueError("Hkv must divide H")
    rng = np.random.default_rng(seed)
    q = _tensor(_normal(rng, (B, H, S, d), std), dtype)
    k = _tensor(_normal(rng, (B, Hkv, Sk, d), std), dtype)
    v = _tensor(_normal(rng, (B, Hkv, Sk, d), std), dtype)
    mb, nb = -(-S // bs), -(-Sk // bs)     # the last block may be cut
    if layout == "band":
        if mb != nb:
            raise ValueError("band layout needs a square block grid")
        lay = band_layout(H, nb, kw.get("w", 1))
    elif layout == "causal_lgs":
        lay = causal_lgs_layout(H, nb, kw.get("window", 4), kw.get("n_global", 2),
                                kw.get("stride", 8))
    elif layout == "causal_bernoulli":
        lay = causal_bernoulli_layout(H, nb, kw.get("p", 0.1), rng)
    elif layout == "random":
        lay = (rng.random((H, mb, nb)) < kw.get("p", 0.3)).astype(np.int32)
    elif layout == "given":
        lay = np.ascontiguousarray(kw["layout_array"], dtype=np.int32)
    else:
        raise ValueError(layout)
    if lay.shape != (H, mb, nb):
        raise ValueError("layout shape mismatch")
    sink = None
    if sink_mean is not None:
        sink = torch.from_numpy((rng.standard_normal(H) + sink_mean).astype(np.float32))
    params = dict(B=B, H=H, Hkv=Hkv, S=S, Sk=Sk, bs=bs, d=d, dtype=dtype, layout=layout,
                  std=std, sink_mean=sink_mean,
                  **{k2: v2 for k2, v2 in kw.items() if k2 != "layout_array"})
    return BsaInputs(name=name, q=q, k=k, v=v, layout=lay, bs=bs, scale=1.0 / np.sqrt(d),
                     seed=seed, params=params, sink=sink)


def upstream_gradient(shape, seed: int, std: float = 1.0) -> torch.Tensor:
    """An upstream gradient dO of the given shape: bf16 N(0, std^2) on the CPU."""
    rng = np.random.default_rng(seed)
    return _tensor(_normal(rng, tuple(int(x) for x in shape), std), "bf16")


def make_topic_qk(H: int, Hkv: int, S: int, d: int, bs: int, n_topics: int, noise: float,
                  seed: int, dtype: str = "bf16"):
    """Queries and keys whose blocks each carry a topic: every token of block
    m of head h is topic_vector[h, t(h, m)] plus N(0, noise^2) noise, the
    topics drawn uniformly per (head, block).  Returns CPU q [H, S, d],
    k [Hkv, S, d] and the topic ids (q topics [H, S/bs], k topics
    [Hkv, S/bs]); blocks that share a topic have similar means."""
    rng = np.random.default_rng(seed)
    nb = S // bs
    basis = rng.standard_normal((max(H, Hkv), n_topics, d)).astype(np.float32)
    tq = rng.integers(0, n_topics, (H, nb))
    tk = rng.integers(0, n_topics, (Hkv, nb))
    g = H // Hkv
    q = np.empty((H, S, d), np.float32)
    k = np.empty((Hkv, S, d), np.float32)
    for h in range(H):
        q[h] = np.repeat(basis[h // g][tq[h]], bs, axis=0)
    for j in range(Hkv):
        k[j] = np.repeat(basis[j][tk[j]], bs, axis=0)
    q += _normal(rng, q.shape, noise)
    k += _normal(rng, k.shape, noise)
    return _tensor(q, dtype), _tensor(k, dtype), tq, tk


def packed_segment_ids(B: int, S: int, min_len: int, max_len: int, seed: int) -> torch.Tensor:
    """Segment ids of sequences packed back to back: per batch item, lengths
    drawn uniformly from [min_len, max_len] until S tokens are filled (the
    last one cut), ids 0, 1, 2, ... in order.  int32 [B, S] on the CPU."""
    rng = np.random.default_rng(seed)
    ids = np.empty((B, S), np.int32)
    for b in range(B):
        pos, sid = 0, 0
        while pos < S:
            L = int(rng.integers(min_len, max_len + 1))
            ids[b, pos:pos + L] = sid
            pos += L
            sid += 1
    return torch.from_numpy(ids)


def sink_logits(H: int, mean: float, seed: int) -> torch.Tensor:
    """Per-head sink logits N(mean, 1), fp32 [H] on the CPU."""
    rng = np.random.default_rng(seed)
    return torch.from_numpy((rng.standard_normal(H) + mean).astype(np.float32))


def make_topk(name: str, B: int, M: int, H: int, d: int, N: int, topk: int, seed: int,
              drop: float = 0.05, with_sink: bool = True, std: float = 1.0) -> TopkInputs:
    """Draw q, kv, per-position indices (without replacement, then each slot
    independently set to -1 with probability ``drop``) and the per-head sink."""
    if topk > N:
        raise ValueError("topk must not exceed N")
    rng = np.random.default_rng(seed)
    q = _tensor(_normal(rng, (B, M, H, d), std), "bf16")
    kv = _tensor(_normal(rng, (B, N, d), std), "bf16")
    idx = np.empty((B, M, topk), dtype=np.int32)
    for b in range(B):
        for m in range(M):
            idx[b, m] = rng.choice(N, size=topk, replace=False)
    if drop > 0:
        idx[rng.random((B, M, topk)) < drop] = -1
    sink = torch.from_numpy(rng.standard_normal(H).astype(np.float32)) if with_sink else None
    params = dict(B=B, M=M, H=H, d=d, N=N, topk=topk, drop=drop, with_sink=with_sink, std=std)
    return TopkInputs(name=name, q=q, kv=kv, idx=torch.from_numpy(idx), sink=sink,
                      scale=1.0 / np.sqrt(d), seed=seed, params=params)


# The five standard workloads, each named by what it is.
WORKLOADS = {
    "band1_h2_s256_bs16_d32_f32": dict(
        kind="bsa", B=1, H=2, S=256, bs=16, d=32, dtype="f32", layout="band", w=1, seed=1),
    "band4_h8_s4096_bs64_d64": dict(
        kind="bsa", B=1, H=8, S=4096, bs=64, d=64, dtype="bf16", layout="band", w=4, seed=2),
    "causal_lgs_b2_h16_s16384_bs64_d128": dict(
        kind="bsa", B=2, H=16, S=16384, bs=64, d=128, dtype="bf16", layout="causal_lgs",
        window=4, n_global=2, stride=8, seed=3),
    "causal_bernoulli_h32_s32768_bs128_d128": dict(
        kind="bsa", B=1, H=32, S=32768, bs=128, d=128, dtype="bf16", layout="causal_bernoulli",
        p=0.10, std=0.5, seed=4),
    "topk2048_m4096_h64_d512_n8192": dict(
        kind="topk", B=1, M=4096, H=64, d=512, N=8192, topk=2048, drop=0.05, seed=5),
}


def make_workload(name: str, **overrides):
    """Draw one of WORKLOADS (optionally with sizes overridden, e.g. a
    smaller S or H for a quick case of the same family)."""
    spec = dict(WORKLOADS[name])
    spec.update(overrides)
    kind = spec.pop("kind")
    if kind == "bsa":
        return make_bsa(name, **spec)
    return make_topk(name, **spec)
