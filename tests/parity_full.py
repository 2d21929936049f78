"""Full-size parity helpers: every output of a large workload against the oracle.

The oracle runs one (batch item, head) of a block-sparse workload, or one run
of query positions of a top-k workload, at a time, in a pool of worker
processes started fresh (spawn), so that no worker inherits the GPU context of
the test process.  Inputs and GPU results reach the workers through .npy files
in a temporary directory, memory-mapped (bf16 tensors as their raw 16-bit
words, widened exactly to float64 in the worker).  Each worker compares its
slice and returns error statistics only, so no full-size float64 result ever
crosses a process boundary.

Heads (and batch items) are independent in the definition -- every softmax
runs over one query row of one head -- so the oracle evaluated on one head's
slice with that head's layout is the oracle of the whole tensor restricted to
that head.
"""

from __future__ import annotations

import multiprocessing as mp
import os
import tempfile
from concurrent.futures import ProcessPoolExecutor
from typing import Dict, List, Optional, Tuple

import numpy as np

from oracle import bsa_oracle as O

# One line per full-size check that ran (printed in the run's summary).
REPORT: List[str] = []

# Worker processes: at most 12, within the host cores this process may use.
MAX_WORKERS = 12


def n_workers() -> int:
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count() or 1
    return max(1, min(MAX_WORKERS, cores))


def save(tmp: str, name: str, t: torch.Tensor) -> None:
    """Store a CPU or GPU tensor as .npy; bf16 as raw uint16 words."""
    import torch  # the workers never need it

    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        a = t.view(torch.int16).numpy().view(np.uint16)
    else:
        a = t.numpy()
    np.save(os.path.join(tmp, name + ".npy"), a, allow_pickle=False)


def _load(tmp: str, name: str):
    return np.load(os.path.join(tmp, name + ".npy"), mmap_mode="r", allow_pickle=False)


def _f64(a: np.ndarray) -> np.ndarray:
    """bf16 words (uint16) or fp32 -> float64, exactly."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _stats(err: np.ndarray) -> Tuple[float, float, int]:
    return float(err.max(initial=0.0)), float(err.sum()), int(err.size)


def _bsa_task(args) -> Dict:
    tmp, b, h, kvh, bs, scale, layout_h, has_lse, opts = args
    q = _f64(_load(tmp, "q")[b, h])[None, None]
    k = _f64(_load(tmp, "k")[b, kvh])[None, None]
    v = _f64(_load(tmp, "v")[b, kvh])[None, None]
    ref, ref_lse = O.attention_live_tiles(q, k, v, layout_h, bs, scale, **opts)
    out = _f64(_load(tmp, "out")[b, h])
    err = np.abs(out - ref[0, 0])
    res = {"bh": (b, h), "finite": bool(np.isfinite(out).all())}
    res["max"], res["sum"], res["n"] = _stats(err)
    if has_lse:
        lse = np.asarray(_load(tmp, "lse")[b, h], dtype=np.float64)
        rl = ref_lse[0, 0]
        empty = np.isneginf(rl)
        res["lse_pattern"] = bool(np.array_equal(np.isneginf(lse), empty))
        fin = ~empty
        res["lse_max"] = float(np.abs(lse[fin] - rl[fin]).max(initial=0.0))
    return res


def _topk_task(args) -> Dict:
    tmp, b, m0, m1, scale, has_sink = args
    q = _f64(_load(tmp, "q")[b, m0:m1])[None]
    kv = _f64(_load(tmp, "kv")[b])[None]
    idx = np.asarray(_load(tmp, "idx")[b, m0:m1])[None]
    sink = np.asarray(_load(tmp, "sink"), dtype=np.float64) if has_sink else None
    ref = O.topk_attention(q, kv, idx, sink, scale)
    out = _f64(_load(tmp, "out")[b, m0:m1])
    err = np.abs(out - ref[0])
    res = {"bm": (b, m0), "finite": bool(np.isfinite(out).all())}
    res["max"], res["sum"], res["n"] = _stats(err)
    return res


# One BLAS thread per worker: the parallelism is the pool's.
_ONE_THREAD = {v: "1" for v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS",
                                "BLIS_NUM_THREADS", "NUMEXPR_NUM_THREADS")}


def _run(fn, tasks: List) -> List[Dict]:
    ctx = mp.get_context("spawn")
    saved = {v: os.environ.get(v) for v in _ONE_THREAD}
    os.environ.update(_ONE_THREAD)  # inherited by the workers spawned below
    try:
        with ProcessPoolExecutor(max_workers=n_workers(), mp_context=ctx) as ex:
            return list(ex.map(fn, tasks, chunksize=1))
    finally:
        for v, old in saved.items():
            if old is None:
                os.environ.pop(v, None)
            else:
                os.environ[v] = old


def bsa_full(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, layout: np.ndarray, bs: int,
             scale: float, out: torch.Tensor, lse: Optional[torch.Tensor], *,
             sink: Optional[torch.Tensor] = None, soft_cap: Optional[float] = None,
             causal: bool = False) -> Dict:
    """Oracle of every (b, h) of a block-sparse forward against the GPU's
    out [B, H, Sq, d] and lse [B, H, Sq].  k and v may have fewer heads than
    q (grouped heads); sink, soft_cap and causal are the oracle's options.
    Returns the aggregate statistics: max and mean abs error of out, max abs
    lse error where finite, and whether the -inf pattern of lse and the
    finiteness of out hold everywhere."""
    B, H = q.shape[0], q.shape[1]
    g = H // k.shape[1]
    sink64 = None if sink is None else sink.detach().cpu().double().numpy()

    def opts(h):
        return dict(sink=None if sink64 is None else sink64[h:h + 1], soft_cap=soft_cap,
                    causal=causal)

    with tempfile.TemporaryDirectory(prefix="bsa_full_") as tmp:
        for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
            save(tmp, name, t)
        if lse is not None:
            save(tmp, "lse", lse)
        tasks = [(tmp, b, h, h // g, bs, scale, np.ascontiguousarray(layout[h:h + 1]),
                  lse is not None, opts(h)) for b in range(B) for h in range(H)]
        res = _run(_bsa_task, tasks)
    agg = {
        "max": max(r["max"] for r in res),
        "mean": sum(r["sum"] for r in res) / sum(r["n"] for r in res),
        "finite": all(r["finite"] for r in res),
        "worst": max(res, key=lambda r: r["max"])["bh"],
        "slices": len(res),
    }
    if lse is not None:
        agg["lse_max"] = max(r["lse_max"] for r in res)
        agg["lse_pattern"] = all(r["lse_pattern"] for r in res)
    return agg


def topk_full(q: torch.Tensor, kv: torch.Tensor, idx: torch.Tensor, sink: Optional[torch.Tensor],
              scale: float, out: torch.Tensor, positions_per_task: int = 64) -> Dict:
    """Oracle of every (b, position) of a top-k forward against the GPU's out
    [B, M, H, d]; same statistics as bsa_full (without lse)."""
    B, M = q.shape[0], q.shape[1]
    with tempfile.TemporaryDirectory(prefix="topk_full_") as tmp:
        for name, t in (("q", q), ("kv", kv), ("idx", idx), ("out", out)):
            save(tmp, name, t)
        if sink is not None:
            save(tmp, "sink", sink)
        tasks = [(tmp, b, m0, min(M, m0 + positions_per_task), scale, sink is not None)
                 for b in range(B) for m0 in range(0, M, positions_per_task)]
        res = _run(_topk_task, tasks)
    return {
        "max": max(r["max"] for r in res),
        "mean": sum(r["sum"] for r in res) / sum(r["n"] for r in res),
        "finite": all(r["finite"] for r in res),
        "worst": max(res, key=lambda r: r["max"])["bm"],
        "slices": len(res),
    }
