#!/usr/bin/env python3
"""Throughput of the block-sparse attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  bsa_plan          layout -> per-row CSR   (causal Bernoulli layout, 32 heads,
                                             256 x 256 blocks)
  bsa_forward       block-sparse attention  (B1 H32 S32768 bs128 d128, bf16)
  topk_sparse_attn  top-k gathered attention with sink
                                            (M4096 H64 d512 N8192 top-k 2048)
Inputs are drawn once, copied to the GPU, and stay resident; W untimed warm-up
steps precede K timed steps, bracketed by device synchronisation.  HIP events
recorded on the launch stream between the three calls give each kernel's
average duration.

Prints ONE JSON line.  `value` = live-tile FLOPs of the step (4*b^2*d per live
tile per head per batch item + 4*d*H per valid top-k index) / step time.

After the timed steps, the forward with all of its optional terms (causal
mask, per-head sink, tanh logit cap 50, eight K/V heads shared by the 32
query heads) is timed on the same workload and reported beside the plain
forward under kernels.bsa_forward_options; it is not part of `value`.  Then
the backward of the plain forward (column plan + bsa_backward for a random
upstream gradient) is timed the same way, under kernels.bsa_backward, with
its FLOPs counted as the 10*b^2*d per live tile of the five tile products a
backward needs (the kernels execute 14: S and dP are recomputed once more).
Last, the content-adaptive layout producer runs on the same q and k (block
means, cosine scores, threshold) under kernels.bsa_layout_adaptive, reported
against HBM bandwidth for the q and k bytes it must read.  Then two more
forms of the hot path on the same inputs: the forward over packed sequences
(segment ids, sequence lengths uniform in [1024, 8192]) under
kernels.bsa_forward_segments, and the top-k
kernel at head size 256 (same indices and sink, fresh q and kv) under
kernels.topk_sparse_attn_d256, and the forward over S - 77 tokens with the
same layout (every last block cut) under kernels.bsa_forward_ragged, its
rate counted on whole tiles.  Last, the second block-sparse workload
(causal local + global + strided, B2 H16 S16384 bs64 d128) is planned and
its forward timed warm, under kernels.bsa_forward_lgs, and both block-sparse
workloads are timed cold: before each timed launch a 1 GiB fill evicts L2
and the Infinity Cache, and events bracket the forward alone.  Per-launch
times of the step's kernels give p10 / median / p90 beside the averages.

Flags: --gpus N (only 1 is supported), --steps K, --warmup W,
--no-cpu-baseline (skip the oracle timing), --cpu-seconds S (oracle sample
budget per kernel), --copy-calibration (also run one plain elementwise copy
of 1 GiB, for HBM counter scaling under a profiler), --option-steps N (launches
of the forward with options; 0 skips that leg), --backward-steps N (calls of
the backward; 0 skips that leg), --adaptive-steps N (calls of the adaptive
layout producer; 0 skips that leg), --variant-steps N (calls of each of the three
forms above; 0 skips them), --config-steps N (launches of each cold-cache leg;
0 skips them and the second workload), --config-warm-steps N (warm launches of
the second workload, after 5 warm-up launches).

--summarize-counters FETCH_CSV WRITE_CSV (no GPU needed) turns the counter
files of two `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs of
`bench.py --copy-calibration` into profiles/hbm_traffic.json: HBM bytes per
launch of each kernel, scaled by what the same counters read for the copy.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

REPO = os.path.dirname(os.path.abspath(__file__))
FWD_WORKLOAD = "causal_bernoulli_h32_s32768_bs128_d128"
LGS_WORKLOAD = "causal_lgs_b2_h16_s16384_bs64_d128"
FLUSH_BYTES = 1 << 30          # > the 256 MB Infinity Cache and 8 x 4 MB of L2
TOPK_WORKLOAD = "topk2048_m4096_h64_d512_n8192"
METRIC = "effective TFLOP/s on live tiles and % of bf16 MFMA peak, 1×MI355X"
PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA, TFLOP/s
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, GB/s
TRAFFIC_FILE = os.path.join(REPO, "profiles", "hbm_traffic.json")
KERNEL_SOURCES = {
    "bsa_forward": os.path.join(REPO, "block_sparse_attention_plan_amd", "csrc", "forward.hip"),
    "topk_sparse_attn": os.path.join(REPO, "block_sparse_attention_plan_amd", "csrc", "topk.hip"),
}
KERNEL_SOURCES["bsa_forward_options"] = KERNEL_SOURCES["bsa_forward"]
KERNEL_SOURCES["bsa_forward_lgs"] = KERNEL_SOURCES["bsa_forward"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(path: str) -> str:
    h = hashlib.sha256()
    for p in (path, os.path.join(os.path.dirname(path), "bsa_device.h")):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch from the committed counter summary, or None when
    absent or taken on a different version of the kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    ent = data.get(kernel)
    if not ent or ent.get("source_sha") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return ent.get("bytes_per_launch")


def same_segment_tiles(layout: np.ndarray, seg: np.ndarray, bs: int) -> int:
    """Live tiles (over the batch) whose query and key blocks can share a
    segment: the id ranges of the two blocks overlap.  For packed sequences
    (ids non-decreasing along a row) these are exactly the tiles with a
    same-segment (query, key) pair; the others are wholly masked."""
    B, S = seg.shape
    nb = -(-S // bs)
    pad = np.concatenate([seg, np.repeat(seg[:, -1:], nb * bs - S, axis=1)], axis=1)
    blocks = pad.reshape(B, nb, bs)
    lo, hi = blocks.min(-1), blocks.max(-1)
    total = 0
    for b in range(B):
        overlap = (hi[b][None, :] >= lo[b][:, None]) & (lo[b][None, :] <= hi[b][:, None])
        total += int((layout.astype(bool) & overlap[None, :layout.shape[1], :layout.shape[2]]).sum())
    return total


def percentiles(ms) -> dict:
    """p10 / median / p90 of per-launch times (ms)."""
    a = np.asarray(ms, dtype=np.float64)
    return {"p10_ms": round(float(np.percentile(a, 10)), 5),
            "median_ms": round(float(np.median(a)), 5),
            "p90_ms": round(float(np.percentile(a, 90)), 5)}


def bsa_counts(layout: np.ndarray, B: int, bs: int, d: int, elem: int = 2):
    """Live tiles, algorithmic FLOPs and bytes of one block-sparse forward."""
    H, Mb, Nb = layout.shape
    tiles = int((layout != 0).sum())
    flops = 4.0 * bs * bs * d * tiles * B
    q_o = 2.0 * B * H * Mb * bs * d * elem          # read q, write out
    kv = 2.0 * bs * d * elem * tiles * B            # live K and V tiles
    lse = 4.0 * B * H * Mb * bs
    return tiles * B, flops, q_o + kv + lse


def topk_counts(idx: np.ndarray, H: int, d: int):
    """Valid indices, algorithmic FLOPs and bytes of one top-k forward."""
    B, M, topk = idx.shape
    valid = int((idx >= 0).sum())
    flops = 4.0 * d * H * valid
    nbytes = valid * d * 2.0 + B * M * (2.0 * H * d * 2 + topk * 4)
    return valid, flops, nbytes


def cpu_baseline(fwd, topk_in, budget_s: float):
    """Time the oracle, as it stands, on a bounded sample of the same step."""
    from oracle import bsa_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    B, H, S, d = fwd.q.shape
    bs = fwd.bs
    q64, k64, v64 = (t.float().numpy().astype(np.float64) for t in (fwd.q, fwd.k, fwd.v))
    nnz = (fwd.layout != 0).sum(-1)
    rng = np.random.default_rng(0)
    all_rows = [(b, h, m) for b in range(B) for h in range(H) for m in range(S // bs)]
    order = rng.permutation(len(all_rows))
    flops_f, t_f, n_rows = 0.0, 0.0, 0
    t_plan0 = time.perf_counter()
    O.plan(fwd.layout)
    t_plan = time.perf_counter() - t_plan0
    chunk = 16
    i = 0
    while t_f < budget_s and i < len(order):
        rows = [all_rows[j] for j in order[i:i + chunk]]
        i += chunk
        t0 = time.perf_counter()
        O.attention_live_tiles(q64, k64, v64, fwd.layout, bs, fwd.scale, row_blocks=rows)
        t_f += time.perf_counter() - t0
        flops_f += sum(4.0 * bs * bs * d * nnz[h, m] for _, h, m in rows)
        n_rows += len(rows)
    qk64, kv64 = (t.float().numpy().astype(np.float64) for t in (topk_in.q, topk_in.kv))
    idx = topk_in.idx.numpy()
    sink = topk_in.sink.numpy() if topk_in.sink is not None else None
    Bq, M, Hq, dq = topk_in.q.shape
    pos_all = rng.permutation(Bq * M)
    flops_t, t_t, n_pos = 0.0, 0.0, 0
    i = 0
    while t_t < budget_s and i < len(pos_all):
        pos = [(int(p) // M, int(p) % M) for p in pos_all[i:i + 4]]
        i += 4
        t0 = time.perf_counter()
        O.topk_attention(qk64, kv64, idx, sink, topk_in.scale, positions=pos)
        t_t += time.perf_counter() - t0
        flops_t += sum(4.0 * dq * Hq * int((idx[b, m] >= 0).sum()) for b, m in pos)
        n_pos += len(pos)
    total_t = t_plan + t_f + t_t
    value = (flops_f + flops_t) / (t_f + t_t) / 1e12
    return {
        "value": value,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"fp64 NumPy oracle on {n_rows} random row blocks of {FWD_WORKLOAD} "
                   f"({t_f:.1f} s) and {n_pos} random positions of {TOPK_WORKLOAD} "
                   f"({t_t:.1f} s), plus the full plan ({t_plan:.2f} s); value = sampled "
                   f"live-tile FLOPs / sampled time"),
        "seconds": round(total_t, 2),
        "host_cores_visible": len(os.sched_getaffinity(0)),
    }


CALIBRATION_BYTES = float(1 << 30)   # read and written by the calibration copy
# Kernel-name tests on mangled names: the copy-staged forward for bs 128, d 128
# (one wave per row group, tiles in two pieces) with its five flags (MASK,
# segment ids, pairs, the plain-copy option form, the cap compiled into that
# form) all `false` (Lb0E) for the plain step; the plain-copy option form with
# the cap (last two flags Lb1E), which serves the forward with every option on
# whole blocks; the pair form (third flag Lb1E), which serves the bs-64
# workload whose neighbouring rows share tiles; and the d-512 top-k instance.
KERNEL_MATCH = {
    "bsa_forward": lambda n: "bsa_fwd_dma_kernelILi128ELi128ELi1ELi2ELb0ELb0ELb0ELb0ELb0EE" in n,
    "bsa_forward_options": lambda n: "bsa_fwd_dma_kernelILi128ELi128ELi1ELi2ELb0ELb0ELb0ELb1ELb1EE" in n,
    "bsa_forward_lgs": lambda n: "bsa_fwd_dma_kernelILi128ELi128ELi1ELi2ELb0ELb0ELb1ELb0ELb0EE" in n,
    # the instance for topk <= 2048 (valid slots compacted first)
    "topk_sparse_attn": lambda n: "topk_kernel" in n and ("<512, true>" in n or "ILi512ELb1EE" in n),
}


def _counter_means(path: str, counter: str):
    """Mean value (KiB) of `counter` per dispatch, by kernel name."""
    import csv
    acc = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            acc.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def summarize_counters(fetch_csv: str, write_csv: str, out_path: str = TRAFFIC_FILE) -> dict:
    """HBM bytes per launch from FETCH_SIZE / WRITE_SIZE counter runs, each
    scaled so that the calibration copy reads and writes exactly 1 GiB."""
    fetch = _counter_means(fetch_csv, "FETCH_SIZE")
    write = _counter_means(write_csv, "WRITE_SIZE")
    cal_f = [v for k, v in fetch.items() if "neg_kernel" in k]
    cal_w = [v for k, v in write.items() if "neg_kernel" in k]
    if not cal_f or not cal_w:
        raise SystemExit("summarize-counters: calibration copy (neg_kernel) not found in the counter files")
    f_scale = CALIBRATION_BYTES / (cal_f[0] * 1024.0)
    w_scale = CALIBRATION_BYTES / (cal_w[0] * 1024.0)
    out = {"_calibration": {"kernel": "elementwise neg over 1 GiB fp32 (reads 1 GiB, writes 1 GiB)",
                            "fetch_kib": cal_f[0], "write_kib": cal_w[0],
                            "fetch_scale": f_scale, "write_scale": w_scale}}
    for kernel, match in KERNEL_MATCH.items():
        fk = [v for k, v in fetch.items() if match(k)]
        wk = [v for k, v in write.items() if match(k)]
        if not fk or not wk:
            continue
        rd, wr = fk[0] * 1024.0 * f_scale, wk[0] * 1024.0 * w_scale
        out[kernel] = {"fetch_kib": fk[0], "write_kib": wk[0], "read_bytes": rd, "write_bytes": wr,
                       "bytes_per_launch": rd + wr,
                       "source_sha": source_hash(KERNEL_SOURCES[kernel])}
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    return out


def main(argv=None) -> int:
    if argv is None:
        argv = sys.argv[1:]
    if argv and argv[0] == "--summarize-counters":
        if len(argv) != 3:
            print("usage: bench.py --summarize-counters FETCH_CSV WRITE_CSV", file=sys.stderr)
            return 2
        print(json.dumps(summarize_counters(argv[1], argv[2]), indent=1))
        return 0
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--option-steps", type=int, default=20)
    ap.add_argument("--backward-steps", type=int, default=10)
    ap.add_argument("--adaptive-steps", type=int, default=20)
    ap.add_argument("--variant-steps", type=int, default=30)
    ap.add_argument("--config-steps", type=int, default=20)
    ap.add_argument("--config-warm-steps", type=int, default=100)
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py: this library runs on one GPU; --gpus {args.gpus} is not supported "
              "(the path shards by heads or query blocks with no exchange, see the design notes)",
              file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("bench.py: --steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    import torch
    import block_sparse_attention_plan_amd as bsa
    from block_sparse_attention_plan_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    bsa.load_library()

    log(f"[bench] drawing {FWD_WORKLOAD}")
    fwd = W.make_workload(FWD_WORKLOAD)
    log(f"[bench] drawing {TOPK_WORKLOAD}")
    tk = W.make_workload(TOPK_WORKLOAD)
    B, H, S, d = (int(x) for x in fwd.q.shape)
    tiles, f_flops, f_bytes = bsa_counts(fwd.layout, B, fwd.bs, d)
    Bq, M, Hq, dq = (int(x) for x in tk.q.shape)
    valid, t_flops, t_bytes = topk_counts(tk.idx.numpy(), Hq, dq)

    layout = torch.from_numpy(fwd.layout).to(dev)
    q, k, v = (t.to(dev) for t in (fwd.q, fwd.k, fwd.v))
    out = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    tq, tkv, tidx, tsink = tk.q.to(dev), tk.kv.to(dev), tk.idx.to(dev), tk.sink.to(dev)
    tout = torch.empty_like(tq)
    pbuf = bsa.plan_buffer(layout.shape, dev)
    torch.cuda.synchronize()

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        plan = bsa.bsa_plan(layout, buf=pbuf)
        if ev is not None:
            ev[1].record()
        bsa.bsa_forward(q, k, v, plan, fwd.scale, out=out, lse=lse)
        if ev is not None:
            ev[2].record()
        bsa.topk_sparse_attn(tq, tkv, tidx, tsink, tk.scale, out=tout)
        if ev is not None:
            ev[3].record()

    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_plan = sum(e[0].elapsed_time(e[1]) for e in events) / args.steps
    t_fwd = sum(e[1].elapsed_time(e[2]) for e in events) / args.steps
    t_topk = sum(e[2].elapsed_time(e[3]) for e in events) / args.steps
    t_step_ev = sum(e[0].elapsed_time(e[3]) for e in events) / args.steps
    pct_fwd = percentiles([e[1].elapsed_time(e[2]) for e in events])
    pct_topk = percentiles([e[2].elapsed_time(e[3]) for e in events])
    ms_per_step = wall * 1e3 / args.steps

    opt_leg = None
    if args.option_steps > 0:
        # same q and layout; K/V = the first 8 heads of k, v, shared by groups of 4
        hkv = 8
        k8, v8 = k[:, :hkv].contiguous(), v[:, :hkv].contiguous()
        sink = W.sink_logits(H, 3.0, 6).to(dev)
        plan = bsa.bsa_plan(layout, buf=pbuf)
        kw = dict(out=out, lse=lse, attn_sink=sink, soft_cap=50.0, causal=True)
        for _ in range(3):
            bsa.bsa_forward(q, k8, v8, plan, fwd.scale, **kw)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.option_steps):
            bsa.bsa_forward(q, k8, v8, plan, fwd.scale, **kw)
        e1.record()
        torch.cuda.synchronize()
        t_opt = e0.elapsed_time(e1) / args.option_steps
        opt_tflops = f_flops / (t_opt * 1e-3) / 1e12
        opt_leg = {"avg_ms": round(t_opt, 5), "launches": args.option_steps,
                   "options": {"causal": True, "attn_sink": "N(3,1) per head", "soft_cap": 50.0,
                               "kv_heads": hkv},
                   "tflops": round(opt_tflops, 2),
                   "pct_bf16_peak": round(100 * opt_tflops / PEAK_BF16_TFLOPS, 2),
                   "traffic": measured_traffic("bsa_forward_options")}
        log(f"[bench] forward with options: {t_opt:.4f} ms")

    bwd_leg = None
    if args.backward_steps > 0:
        dout = W.upstream_gradient(fwd.q.shape, seed=41).to(dev)
        plan = bsa.bsa_plan(layout, buf=pbuf)
        bsa.bsa_forward(q, k, v, plan, fwd.scale, out=out, lse=lse)
        g_q, g_k, g_v = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(bsa.load_library().bsa_backward_workspace_bytes(B, H, S) // 4,
                         dtype=torch.float32, device=dev)

        def bwd():
            pc = bsa.bsa_plan_cols(layout)
            bsa.bsa_backward(q, k, v, out, dout, lse, plan, pc, fwd.scale, dq=g_q, dk=g_k,
                             dv=g_v, workspace=ws)
        for _ in range(2):
            bwd()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.backward_steps):
            bwd()
        e1.record()
        torch.cuda.synchronize()
        t_bwd = e0.elapsed_time(e1) / args.backward_steps
        b_flops = 2.5 * f_flops
        b_tflops = b_flops / (t_bwd * 1e-3) / 1e12
        bwd_leg = {"avg_ms": round(t_bwd, 5), "calls": args.backward_steps,
                   "includes": "bsa_plan_cols + bsa_backward (D/lse pass, dq kernel, dk/dv kernel)",
                   "flops": b_flops, "tflops": round(b_tflops, 2),
                   "pct_bf16_peak": round(100 * b_tflops / PEAK_BF16_TFLOPS, 2)}
        log(f"[bench] backward: {t_bwd:.4f} ms")

    ad_leg = None
    if args.adaptive_steps > 0:
        q0, k0 = q[0], k[0]
        ad_ws = torch.empty(bsa.load_library().bsa_layout_adaptive_workspace_bytes(
            H, H, S // fwd.bs, S // fwd.bs, d) // 4, dtype=torch.float32, device=dev)
        for _ in range(3):
            bsa.bsa_layout_adaptive(q0, k0, fwd.bs, 0.1, causal=True, workspace=ad_ws)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.adaptive_steps):
            bsa.bsa_layout_adaptive(q0, k0, fwd.bs, 0.1, causal=True, workspace=ad_ws)
        e1.record()
        torch.cuda.synchronize()
        t_ad = e0.elapsed_time(e1) / args.adaptive_steps
        ad_bytes = float(q0.numel() + k0.numel()) * q0.element_size()
        ad_gbs = ad_bytes / (t_ad * 1e-3) / 1e9
        ad_leg = {"avg_ms": round(t_ad, 5), "calls": args.adaptive_steps,
                  "config": f"H{H} S{S} bs{fwd.bs} d{d} bf16, tau 0.1, causal",
                  "algorithmic_bytes": ad_bytes, "algorithmic_gbs": round(ad_gbs, 1),
                  "pct_hbm_peak": round(100 * ad_gbs / PEAK_HBM_GBS, 2)}
        log(f"[bench] adaptive layout: {t_ad:.4f} ms")

    def timed(fn, n):
        for _ in range(5):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    seg_leg = d256_leg = rag_leg = None
    if args.variant_steps > 0:
        seg = W.packed_segment_ids(B, S, 1024, 8192, seed=7).to(dev)
        plan = bsa.bsa_plan(layout, buf=pbuf)
        t_seg = timed(lambda: bsa.bsa_forward(q, k, v, plan, fwd.scale, out=out, lse=lse,
                                              q_segment_ids=seg, kv_segment_ids=seg),
                      args.variant_steps)
        same = same_segment_tiles(fwd.layout, seg.cpu().numpy(), fwd.bs)
        share = same / (int(fwd.layout.sum()) * B)
        # the kernel drops the other tiles before its pipeline, so the rate
        # is taken over the tiles that hold a same-segment pair
        seg_tf = f_flops * share / (t_seg * 1e-3) / 1e12
        seg_leg = {"avg_ms": round(t_seg, 5), "calls": args.variant_steps,
                   "segments": "packed, lengths uniform in [1024, 8192]",
                   "tflops_on_same_segment_tiles": round(seg_tf, 2),
                   "pct_bf16_peak": round(100 * seg_tf / PEAK_BF16_TFLOPS, 2),
                   "live_tiles_with_same_segment_keys": same,
                   "share_of_live_tiles": round(share, 4)}
        log(f"[bench] forward with segment ids: {t_seg:.4f} ms")
        rng = np.random.default_rng(8)
        q256 = torch.from_numpy(rng.standard_normal((Bq, M, Hq, 256), dtype=np.float32)).to(
            torch.bfloat16).to(dev)
        kv256 = torch.from_numpy(rng.standard_normal((Bq, int(tk.kv.shape[1]), 256),
                                                     dtype=np.float32)).to(torch.bfloat16).to(dev)
        o256 = torch.empty_like(q256)
        t_256 = timed(lambda: bsa.topk_sparse_attn(q256, kv256, tidx, tsink, 1.0 / 16.0, out=o256),
                      args.variant_steps)
        _, f256, b256 = topk_counts(tk.idx.numpy(), Hq, 256)
        d256_leg = {"avg_ms": round(t_256, 5), "calls": args.variant_steps,
                    "tflops": round(f256 / (t_256 * 1e-3) / 1e12, 2),
                    "algorithmic_gbs": round(b256 / (t_256 * 1e-3) / 1e9, 1),
                    "pct_hbm_peak": round(100 * b256 / (t_256 * 1e-3) / 1e9 / PEAK_HBM_GBS, 2)}
        log(f"[bench] top-k at d 256: {t_256:.4f} ms")
        # lengths that are not a multiple of bs: the same layout over
        # S' = S - 77 tokens, so every block row and column ends in a cut block
        S_r = S - 77
        qr, kr, vr = (t[:, :, :S_r].contiguous() for t in (q, k, v))
        out_r = torch.empty_like(qr)
        lse_r = torch.empty((B, H, S_r), dtype=torch.float32, device=dev)
        plan = bsa.bsa_plan(layout, buf=pbuf)
        t_rag = timed(lambda: bsa.bsa_forward(qr, kr, vr, plan, fwd.scale, out=out_r, lse=lse_r,
                                              bs=fwd.bs),
                      args.variant_steps)
        rag_tf = f_flops / (t_rag * 1e-3) / 1e12
        rag_leg = {"avg_ms": round(t_rag, 5), "calls": args.variant_steps,
                   "seq_len": S_r, "tflops_on_whole_tiles": round(rag_tf, 2),
                   "pct_bf16_peak": round(100 * rag_tf / PEAK_BF16_TFLOPS, 2)}
        log(f"[bench] forward with cut last blocks (S = {S_r}): {t_rag:.4f} ms")
        del qr, kr, vr, out_r, lse_r

    def timed_cold(fn, n, flush):
        """Per-launch ms of fn with L2 and the Infinity Cache evicted before each."""
        fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n)]
        torch.cuda.synchronize()
        for a, b in ev:
            flush.zero_()
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in ev]

    lgs_leg = cold_legs = None
    if args.config_steps > 0:
        flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
        plan = bsa.bsa_plan(layout, buf=pbuf)
        c4 = timed_cold(lambda: bsa.bsa_forward(q, k, v, plan, fwd.scale, out=out, lse=lse),
                        args.config_steps, flush)
        log(f"[bench] drawing {LGS_WORKLOAD}")
        lw = W.make_workload(LGS_WORKLOAD)
        lB, lH, lS, ld = (int(x) for x in lw.q.shape)
        l_tiles, l_flops, l_bytes = bsa_counts(lw.layout, lB, lw.bs, ld)
        l_layout = torch.from_numpy(lw.layout).to(dev)
        lq, lk, lv = (t.to(dev) for t in (lw.q, lw.k, lw.v))
        l_out = torch.empty_like(lq)
        l_lse = torch.empty((lB, lH, lS), dtype=torch.float32, device=dev)
        l_plan = bsa.bsa_plan(l_layout)
        fn = lambda: bsa.bsa_forward(lq, lk, lv, l_plan, lw.scale, out=l_out, lse=l_lse)  # noqa: E731
        for _ in range(5):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(max(1, args.config_warm_steps))]
        torch.cuda.synchronize()
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        warm = [a.elapsed_time(b) for a, b in ev]
        c3 = timed_cold(fn, args.config_steps, flush)
        del flush
        t_l = sum(warm) / len(warm)
        l_tf = l_flops / (t_l * 1e-3) / 1e12
        lgs_leg = {"workload": LGS_WORKLOAD, "avg_ms": round(t_l, 5), **percentiles(warm),
                   "launches": len(warm), "live_tiles": l_tiles, "flops": l_flops,
                   "tflops": round(l_tf, 2), "pct_bf16_peak": round(100 * l_tf / PEAK_BF16_TFLOPS, 2),
                   "algorithmic_bytes": l_bytes,
                   "algorithmic_gbs": round(l_bytes / (t_l * 1e-3) / 1e9, 1),
                   "traffic": measured_traffic("bsa_forward_lgs")}
        log(f"[bench] {LGS_WORKLOAD} forward: {t_l:.4f} ms")
        cold_legs = {}
        for name, ms, fl in ((FWD_WORKLOAD, c4, f_flops), (LGS_WORKLOAD, c3, l_flops)):
            t_c = sum(ms) / len(ms)
            cold_legs[name] = {"avg_ms": round(t_c, 5), **percentiles(ms), "launches": len(ms),
                               "tflops": round(fl / (t_c * 1e-3) / 1e12, 2),
                               "pct_bf16_peak": round(100 * fl / (t_c * 1e-3) / 1e12
                                                      / PEAK_BF16_TFLOPS, 2),
                               "flush": "1 GiB fill before each launch"}
            log(f"[bench] {name} forward, cold caches: {t_c:.4f} ms")

    if args.copy_calibration:
        # one full-grid elementwise kernel that reads 1 GiB and writes 1 GiB
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log("[bench] copy calibration: elementwise neg over 1 GiB issued")

    fwd_tflops = f_flops / (t_fwd * 1e-3) / 1e12
    topk_tflops = t_flops / (t_topk * 1e-3) / 1e12
    topk_gbs = t_bytes / (t_topk * 1e-3) / 1e9
    fwd_gbs = f_bytes / (t_fwd * 1e-3) / 1e9
    kernels = {
        "bsa_plan": {"avg_ms": round(t_plan, 5)},
        "bsa_forward": {
            "avg_ms": round(t_fwd, 5), **pct_fwd, "live_tiles": tiles, "flops": f_flops,
            "tflops": round(fwd_tflops, 2), "pct_bf16_peak": round(100 * fwd_tflops / PEAK_BF16_TFLOPS, 2),
            "algorithmic_bytes": f_bytes, "algorithmic_gbs": round(fwd_gbs, 1)},
        "topk_sparse_attn": {
            "avg_ms": round(t_topk, 5), **pct_topk, "valid_indices": valid, "flops": t_flops,
            "tflops": round(topk_tflops, 2), "pct_bf16_peak": round(100 * topk_tflops / PEAK_BF16_TFLOPS, 2),
            "algorithmic_bytes": t_bytes, "algorithmic_gbs": round(topk_gbs, 1),
            "pct_hbm_peak": round(100 * topk_gbs / PEAK_HBM_GBS, 2)},
    }
    if opt_leg is not None:
        kernels["bsa_forward_options"] = opt_leg
    if bwd_leg is not None:
        kernels["bsa_backward"] = bwd_leg
    if ad_leg is not None:
        kernels["bsa_layout_adaptive"] = ad_leg
    if seg_leg is not None:
        kernels["bsa_forward_segments"] = seg_leg
    if d256_leg is not None:
        kernels["topk_sparse_attn_d256"] = d256_leg
    if rag_leg is not None:
        kernels["bsa_forward_ragged"] = rag_leg
    if lgs_leg is not None:
        kernels["bsa_forward_lgs"] = lgs_leg
    if cold_legs is not None:
        kernels["bsa_forward_cold"] = cold_legs
    # Rooflines.  Both kernels are bound by their matrix cores: the forward
    # streams each K/V tile once per block row that lists it (bs FLOP per
    # streamed byte; about half of those bytes are L2 hits), and the top-k
    # kernel's gathered rows come from an 8 MiB table held in L2 and the
    # Infinity Cache, so its algorithmic bytes per second (each gathered row
    # counted once per position) can exceed the HBM peak and do not bind it.
    # The measured fabric traffic (FETCH_SIZE + WRITE_SIZE counters, when
    # taken on this source) gives its HBM fraction.  `roofline` is the
    # dominant kernel's MFMA fraction; both kernels' figures sit under
    # `by_kernel`.
    def mfma_roof(kernel, tflops, t_ms, alg_bytes):
        traffic = measured_traffic(kernel)
        r = {"kernel": kernel, "bound": "mfma", "achieved": round(tflops, 2),
             "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
             "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
             "avg_ms": round(t_ms, 5),
             "algorithmic_gbs": round(alg_bytes / (t_ms * 1e-3) / 1e9, 1)}
        if traffic is not None:
            hbm = traffic / (t_ms * 1e-3) / 1e9
            r["measured_hbm_gbs"] = round(hbm, 1)
            r["measured_hbm_frac"] = round(hbm / PEAK_HBM_GBS, 4)
        return r

    fwd_roof = mfma_roof("bsa_forward", fwd_tflops, t_fwd, f_bytes)
    topk_roof = mfma_roof("topk_sparse_attn", topk_tflops, t_topk, t_bytes)
    topk_roof["algorithmic_gbs_note"] = ("gathered rows counted once per position; served mostly "
                                         "from L2 and the Infinity Cache, not an HBM rate")
    roof = dict(topk_roof if t_topk > t_fwd else fwd_roof)
    roof["by_kernel"] = {"bsa_forward": fwd_roof, "topk_sparse_attn": topk_roof}
    value = (f_flops + t_flops) / (ms_per_step * 1e-3) / 1e12
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{FWD_WORKLOAD} + {TOPK_WORKLOAD}",
            "block_sparse": {"B": B, "H": H, "S": S, "bs": fwd.bs, "d": d,
                             "layout": "causal Bernoulli(0.10) + diagonal", "live_tiles": tiles},
            "topk": {"B": Bq, "M": M, "H": Hq, "d": dq, "N": int(tk.kv.shape[1]),
                     "topk": int(tk.idx.shape[2]), "valid_indices": valid, "sink": True},
            "event_ms_per_step": round(t_step_ev, 4),
            "pct_bf16_peak_step": round(100 * value / PEAK_BF16_TFLOPS, 2),
        },
        "roofline": roof,
        "kernels": kernels,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log(f"[bench] timing the CPU oracle (about {2 * args.cpu_seconds:.0f} s)")
        result["cpu_baseline"] = cpu_baseline(fwd, tk, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
