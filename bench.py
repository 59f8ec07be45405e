"""Benchmark: forward + backward of one context-parallel rank's share of ring attention.

Workload: the 64K share — B=1, Hq=32, Hkv=8, d=128, total S=65536 split into CP=8
contiguous chunks of 8192, rank 7 (8 ring steps, the diagonal chunk causal), bf16
inputs ~ N(0,1) (synthetic, seeded), fp32 accumulation.  One step = the whole ring
forward (8 fwd steps, 7 merges, final bf16 conversion) + the whole ring backward
(delta preprocess, 8 bwd steps, including zeroing the gradient accumulators), with
all inputs resident in HBM.

Throughput counts ALGORITHMIC flops on live (unmasked) pairs only: 4*Hq*d per pair
forward (QK^T and PV) and 10*Hq*d backward (QK^T recomputed, dP, dV, dK, dQ).

Prints ONE JSON line (rank 0).  --gpus N with N > 1 exits: the benchmark measures
one GPU's share of the ring.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "causal ring-attn fwd+bwd TFLOP/s and % MFMA peak, 8K local Q × 64K ctx bf16"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (published)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "ring_bwd_step_64k_cp8_r7_traffic.txt")


def kernel_source_hash() -> str:
    """sha256 over the HIP sources and headers of the library (name + contents)."""
    import glob
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "context_long_sequence_amd", "csrc")
    for path in sorted(glob.glob(os.path.join(csrc, "*.hip")) + glob.glob(os.path.join(csrc, "*.h"))):
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None when
    the summary is missing or was taken on different kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            kv = dict(line.strip().split("=", 1) for line in f if "=" in line and not line.startswith("#"))
    except OSError:
        return None
    if kv.get("source_sha256") != kernel_source_hash():
        return None
    v = kv.get(f"{kernel}.hbm_bytes_per_launch")
    return float(v) if v else None


def live_pairs_causal(C: int, rank: int) -> int:
    """Causal pairs of rank `rank` with contiguous chunks of C: rank*C^2 + C(C+1)/2."""
    return rank * C * C + C * (C + 1) // 2


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing on host cores")
    p.add_argument("--no-extras", action="store_true", help="skip the packed/8K/workspace side measurements")
    p.add_argument("--profile-copy", action="store_true",
                   help="also run one plain 1 GiB device copy (calibrates HBM byte counters)")
    p.add_argument("--only", choices=["fwd", "bwd", "all"], default="all",
                   help="restrict the timed loop (for profiling a single kernel family)")
    return p.parse_args()


class Timer:
    """Per-entry-point HIP event timing on the stream the kernels are launched on."""

    def __init__(self, torch, enabled=True):
        self.torch = torch
        self.enabled = enabled
        self.events = {}
        self.pending = None

    def begin(self):
        if self.enabled:
            e = self.torch.cuda.Event(enable_timing=True)
            e.record()
            self.pending = e

    def hook(self, name, _i):
        if not self.enabled:
            return
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.events.setdefault(name, []).append((self.pending, e))
        self.pending = e

    def mean_ms(self, name):
        pairs = self.events.get(name, [])
        if not pairs:
            return None
        return sum(a.elapsed_time(b) for a, b in pairs) / len(pairs)

    def total_ms(self, name):
        return sum(a.elapsed_time(b) for a, b in self.events.get(name, []))

    def count(self, name):
        return len(self.events.get(name, []))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the ring (one rank); --gpus {args.gpus} is not "
              "supported: run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import context_long_sequence_amd as ra
    from synthetic import LLAMA3_8K_FWD, METRIC_CONFIG, PACKED16K_FWD, make_workload

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    ra.load()
    dev = torch.device("cuda:0")
    cfg = METRIC_CONFIG
    C, r, CP = cfg.C, cfg.rank, cfg.CP
    pairs = live_pairs_causal(C, r)
    f_fwd = 4.0 * cfg.Hq * cfg.d * pairs
    f_bwd = 10.0 * cfg.Hq * cfg.d * pairs

    wl = make_workload(cfg, q_chunks=[r])

    def t(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(torch.bfloat16)

    q = t(wl.q_local)
    ks = [t(k) for k in wl.k_chunks]
    vs = [t(v) for v in wl.v_chunks]
    do = t(wl.do)
    del wl
    o = torch.empty_like(q)
    lse = torch.empty((1, cfg.Hq, C), dtype=torch.float32, device=dev)
    # dQ and the per-chunk dK/dV accumulators as views of one buffer, cleared by one fill
    grads = flat_grads(torch, dev, q.shape, [k.shape for k in ks])
    dq, dks, dvs = grads["dq"], grads["dk_chunks"], grads["dv_chunks"]
    torch.cuda.synchronize()
    base_alloc = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    ws = ra.RingWorkspace(1, C, cfg.Hq, cfg.d, dev, backward=True)

    def step(timer=None):
        hook = timer.hook if timer else None
        if timer:
            timer.begin()
        if args.only in ("fwd", "all"):
            ra.ring_forward(q, ks, vs, r, CP, causal=True, out=o, lse=lse, workspace=ws, step_hook=hook)
        if args.only in ("bwd", "all"):
            grads["flat"].zero_()
            if hook:
                hook("zero_grads", 0)
            ra.ring_backward(q, ks, vs, o, lse, do, r, CP, causal=True, dq=dq, dk_chunks=dks, dv_chunks=dvs,
                             delta=ws.delta, step_hook=hook)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    workspace_peak = torch.cuda.max_memory_allocated() - base_alloc

    # Timed region: K whole steps (events around each step give the median as well).
    timer = Timer(torch)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    marks[0].record()
    for i in range(args.steps):
        step(timer)
        marks[i + 1].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    step_ms = [marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)]

    flops = {"all": f_fwd + f_bwd, "fwd": f_fwd, "bwd": f_bwd}[args.only]
    value = flops / (ms_per_step * 1e-3) / 1e12

    t_fwd_step = timer.mean_ms("fwd_step")
    t_merge = timer.mean_ms("merge")
    t_bwd_step = timer.mean_ms("bwd_step")
    t_pre = timer.mean_ms("bwd_preprocess")
    per_step_ms = {}
    for name in ("fwd_step", "merge", "zero_grads", "bwd_preprocess", "bwd_step"):
        if timer.count(name):
            per_step_ms[name] = timer.total_ms(name) / args.steps

    # Dominant entry point by time.
    roofline = None
    merge_bytes = 3 * (C * cfg.Hq * cfg.d * 4) + 3 * (cfg.Hq * C * 4)
    if per_step_ms:
        dom = max(("fwd_step", "bwd_step"), key=lambda n: per_step_ms.get(n, 0.0))
        if dom == "bwd_step" and t_bwd_step:
            achieved = f_bwd / CP / (t_bwd_step * 1e-3) / 1e12
            roofline = {"kernel": "ring_attn_bwd_step (dK/dV kernel + dQ kernel)", "bound": "mfma",
                        "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                        "traffic": measured_traffic("ring_attn_bwd_step"),
                        "avg_launch_ms": round(t_bwd_step, 4), "flop_per_launch": f_bwd / CP}
        elif t_fwd_step:
            achieved = f_fwd / CP / (t_fwd_step * 1e-3) / 1e12
            roofline = {"kernel": "ring_attn_fwd_step", "bound": "mfma",
                        "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                        "traffic": measured_traffic("ring_attn_fwd_step"),
                        "avg_launch_ms": round(t_fwd_step, 4), "flop_per_launch": f_fwd / CP}

    extra = {
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "live_pairs": pairs,
        "algorithmic_flop": {"fwd": f_fwd, "bwd": f_bwd},
        "per_step_ms": {k: round(v, 4) for k, v in per_step_ms.items()},
        "timer_ms": {"host_wall_per_step": round(ms_per_step, 4),
                     "event_median_per_step": round(float(np.median(step_ms)), 4),
                     "event_min_per_step": round(min(step_ms), 4)},
    }
    if t_fwd_step and args.only in ("fwd", "all"):
        # steps 1..7 fold their partial into the running result inside the step's own
        # launch (ring_attn_fwd_step_merge); "merge" is only the final conversion, if any
        fwd_ms = per_step_ms["fwd_step"] + per_step_ms.get("merge", 0.0)
        extra["fwd_tflops"] = round(f_fwd / (fwd_ms * 1e-3) / 1e12, 2)
        # the merge entry point on its own, at the share's shape (the unfused path)
        t_merge = time_lse_merge(torch, ra, dev, C, cfg.Hq, cfg.d)
        extra["merge"] = {"bytes_per_call": merge_bytes, "avg_us": round(t_merge * 1e3, 2),
                          "GB_per_s": round(merge_bytes / (t_merge * 1e-3) / 1e9, 1),
                          "frac_of_hbm_peak": round(merge_bytes / (t_merge * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    if t_bwd_step and args.only in ("bwd", "all"):
        bwd_ms = per_step_ms["bwd_step"] + per_step_ms.get("bwd_preprocess", 0.0)
        extra["bwd_tflops"] = round(f_bwd / (bwd_ms * 1e-3) / 1e12, 2)
        if t_pre:
            pre_bytes = 2 * C * cfg.Hq * cfg.d * 2 + cfg.Hq * C * 4
            extra["bwd_preprocess_GB_per_s"] = round(pre_bytes / (t_pre * 1e-3) / 1e9, 1)
    extra["workspace"] = {"peak_bytes": int(workspace_peak), "ring_workspace_bytes": ws.nbytes(),
                          "score_matrix_avoided_bytes": C * cfg.S * cfg.Hq * 4}

    if not args.no_extras:
        # Cold caches: before each of 3 steps, 1 GiB is written (more than the 4 MiB L2
        # per XCD and the 256 MiB Infinity Cache), then the step is timed alone.
        flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        cold = []
        for _ in range(3):
            flush.fill_(1.0)
            a_ev, b_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_ev.record()
            step()
            b_ev.record()
            torch.cuda.synchronize()
            cold.append(a_ev.elapsed_time(b_ev))
        del flush
        cold_ms = float(np.median(cold))
        extra["cache_flushed"] = {"ms_per_step_median": round(cold_ms, 4),
                                  "tflops": round(flops / (cold_ms * 1e-3) / 1e12, 2), "steps": len(cold)}
        extra.update(side_measurements(torch, ra, np, dev, LLAMA3_8K_FWD, PACKED16K_FWD, make_workload))
        zz = extra["zigzag_64k_cp8"]
        # the ring runs at the pace of its slowest rank: contiguous rank 7 (this line's
        # step) against the slower of zigzag ranks 0 and 7 (all ranks have equal work)
        if args.only == "all":
            zz["critical_path_speedup_vs_contiguous"] = round(
                ms_per_step / max(zz["rank0"]["ms"], zz[f"rank{zz['cp'] - 1}"]["ms"]), 3)

    if args.profile_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        extra["copy_calibration_bytes"] = {"read": src.numel() * 4, "write": dst.numel() * 4}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg)

    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded i.i.d. N(0,1) Q/K/V/dO rounded to bf16 (no dataset)",
        "config": {"workload": "64K-context causal ring-attention share, rank 7 of CP=8, fwd+bwd"
                               + ("" if args.only == "all" else f" ({args.only} only)"),
                   "global_batch": 1, "seq_len": cfg.S, "local_q": C, "cp": CP, "rank": r,
                   "heads_q": cfg.Hq, "heads_kv": cfg.Hkv, "head_dim": cfg.d, "parallelism": "cp8 (one rank)"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


def time_lse_merge(torch, ra, dev, C, Hq, d, reps=20):
    """Mean time (ms) of one lse_merge call (running and step results of the share's
    shape, both live) on the current stream, from events around `reps` calls."""
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    o_acc = torch.randn((1, C, Hq, d), generator=g, device=dev)
    o_step = torch.randn((1, C, Hq, d), generator=g, device=dev)
    lse_acc = torch.randn((1, Hq, C), generator=g, device=dev) + 5.0
    lse_step = torch.randn((1, Hq, C), generator=g, device=dev) + 5.0
    ra.lse_merge(o_acc, lse_acc, o_step, lse_step)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        ra.lse_merge(o_acc, lse_acc, o_step, lse_step)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def packed_live_pairs(lengths, C, rank):
    """Causal same-sample pairs of rank `rank`'s queries, from the packed sample lengths:
    a query at global index i inside sample [s0, s1) sees the i - s0 + 1 keys s0..i."""
    total = 0
    s0 = 0
    lo, hi = rank * C, (rank + 1) * C
    for n in lengths:
        s1 = s0 + int(n)
        a, b = max(s0, lo), min(s1, hi)
        if a < b:
            # sum_{i=a}^{b-1} (i - s0 + 1)
            total += (b - a) * (a - s0 + 1 + b - s0) // 2
        s0 = s1
    return total


def flat_grads(torch, dev, q_shape, kv_shapes):
    """fp32 dQ [q_shape] and dK/dV [kv_shapes[c]] per chunk as contiguous views of one
    buffer ("flat"), so that one fill clears them all."""
    n_q = math.prod(q_shape)
    n_kv = [math.prod(s) for s in kv_shapes]
    flat = torch.empty(n_q + 2 * sum(n_kv), dtype=torch.float32, device=dev)
    out = {"flat": flat, "dq": flat[:n_q].view(q_shape), "dk_chunks": [], "dv_chunks": []}
    off = n_q
    for name in ("dk_chunks", "dv_chunks"):
        for s, n in zip(kv_shapes, n_kv):
            out[name].append(flat[off:off + n].view(s))
            off += n
    return out


def packed_executed_pairs(np, seg_row, C, rank, cp, qblock=64, ktile=32):
    """(query, key) pairs the packed forward computes per query head: for every block
    of `qblock` local queries and every chunk, the key tiles of `ktile` keys from the
    first to the last that shares a sample with the block, within the causal range
    (the forward kernel's tile range on packed rows).  seg_row: the row's segment ids."""
    total = 0
    for c in range(cp):
        for q0 in range(0, C, qblock):
            q_last = min(q0 + qblock, C) - 1
            n_keys = max(0, min(C, rank * C + q_last - c * C + 1))
            n_tiles = (n_keys + ktile - 1) // ktile
            if n_tiles == 0:
                continue
            lo, hi = seg_row[rank * C + q0], seg_row[rank * C + q_last]
            starts = c * C + np.arange(n_tiles) * ktile
            ends = c * C + np.minimum(np.arange(1, n_tiles + 1) * ktile, C) - 1
            live = (seg_row[ends] >= lo) & (seg_row[starts] <= hi)
            idx = np.nonzero(live)[0]
            if idx.size:
                total += qblock * ktile * int(idx[-1] - idx[0] + 1)
    return total


def side_measurements(torch, ra, np, dev, LLAMA3_8K_FWD, PACKED16K_FWD, make_workload):
    """Forward TFLOP/s of the 8K and packed-16K shares, the segment-id kernel time, the
    load-balanced (zigzag) 64K forward+backward of ranks 0 and 7, the 64K ring with
    overlapped receives, the head-sharded and gathered-KV 64K shares, and the peak workspace of one forward+backward at S = 16K..128K
    (CP=8, rank 7)."""
    out = {}

    def ev_ms(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    def bf(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(torch.bfloat16)

    def grad_buffers(q, ks):
        """fp32 dQ and per-chunk dK/dV accumulators, allocated once (views of one buffer)."""
        return flat_grads(torch, dev, q.shape, [k.shape for k in ks])

    def zeroed(gb):
        """Clears the accumulators (part of each timed backward, as in the main step)."""
        gb["flat"].zero_()
        return {k: gb[k] for k in ("dq", "dk_chunks", "dv_chunks")}

    # 8K Llama-3-8B-shaped share (rank 3 of 4), forward
    c2 = LLAMA3_8K_FWD
    wl = make_workload(c2, q_chunks=[c2.rank])
    q, ks, vs = bf(wl.q_local), [bf(k) for k in wl.k_chunks], [bf(v) for v in wl.v_chunks]
    ws = ra.RingWorkspace(1, c2.C, c2.Hq, c2.d, dev)
    ms = ev_ms(lambda: ra.ring_forward(q, ks, vs, c2.rank, c2.CP, causal=True, workspace=ws), reps=20)
    pairs = live_pairs_causal(c2.C, c2.rank)
    out["fwd_8k_cp4_r3"] = {"ms": round(ms, 4), "tflops": round(4.0 * c2.Hq * c2.d * pairs / (ms * 1e-3) / 1e12, 2)}
    # the same share's backward (dO ~ N(0,1)), from the forward's O and LSE
    o2 = torch.empty_like(q)
    l2 = torch.empty((1, c2.Hq, c2.C), dtype=torch.float32, device=dev)
    ws = ra.RingWorkspace(1, c2.C, c2.Hq, c2.d, dev, backward=True)
    ra.ring_forward(q, ks, vs, c2.rank, c2.CP, causal=True, workspace=ws, out=o2, lse=l2)
    do2 = torch.randn(q.shape, generator=torch.Generator(device=dev).manual_seed(5), device=dev).to(torch.bfloat16)
    g2 = grad_buffers(q, ks)
    bms = ev_ms(lambda: ra.ring_backward(q, ks, vs, o2, l2, do2, c2.rank, c2.CP, causal=True, delta=ws.delta,
                                         **zeroed(g2)), reps=20)
    out["bwd_8k_cp4_r3"] = {"ms": round(bms, 4),
                            "tflops": round(10.0 * c2.Hq * c2.d * pairs / (bms * 1e-3) / 1e12, 2)}
    del o2, l2, do2

    # packed 16K share (rank 2 of 4): segment ids + forward + backward
    c4 = PACKED16K_FWD.with_(backward=True)
    wl = make_workload(c4, q_chunks=[c4.rank])
    q, ks, vs = bf(wl.q_local), [bf(k) for k in wl.k_chunks], [bf(v) for v in wl.v_chunks]
    do = bf(wl.do)
    pos = torch.from_numpy(wl.position_ids).to(dev)
    seg = torch.empty_like(pos)
    seg_ms = ev_ms(lambda: ra.segment_mask_from_pos(pos, seg), reps=20)
    ws = ra.RingWorkspace(1, c4.C, c4.Hq, c4.d, dev, backward=True)
    o4 = torch.empty_like(q)
    l4 = torch.empty((1, c4.Hq, c4.C), dtype=torch.float32, device=dev)
    fms = ev_ms(lambda: ra.ring_forward(q, ks, vs, c4.rank, c4.CP, causal=True, seg_ids=seg, workspace=ws,
                                         out=o4, lse=l4), reps=20)
    g4 = grad_buffers(q, ks)
    bms = ev_ms(lambda: ra.ring_backward(q, ks, vs, o4, l4, do, c4.rank, c4.CP, causal=True, seg_ids=seg,
                                         delta=ws.delta, **zeroed(g4)), reps=20)
    pairs4 = packed_live_pairs(wl.lengths, c4.C, c4.rank)
    exec4 = packed_executed_pairs(np, seg[0].cpu().numpy(), c4.C, c4.rank, c4.CP)
    out["packed_16k_cp4_r2"] = {
        "live_pairs": pairs4, "frac_of_causal_pairs": round(pairs4 / live_pairs_causal(c4.C, c4.rank), 4),
        "fwd_executed_pairs": exec4, "live_frac_of_executed": round(pairs4 / exec4, 4),
        "segment_ids_us": round(seg_ms * 1e3, 2),
        "fwd_ms": round(fms, 4), "fwd_tflops": round(4.0 * c4.Hq * c4.d * pairs4 / (fms * 1e-3) / 1e12, 2),
        "bwd_ms": round(bms, 4), "bwd_tflops": round(10.0 * c4.Hq * c4.d * pairs4 / (bms * 1e-3) / 1e12, 2)}
    del q, ks, vs, do, ws, o4, l4

    # load-balanced (zigzag) layout at the 64K shape: ranks 0 and 7, forward + backward
    S, cp, Hq, Hkv, d = 65536, 8, 32, 8, 128
    h = S // (2 * cp)
    g = torch.Generator(device=dev)
    g.manual_seed(1234)
    zq = torch.randn((1, 2 * h, Hq, d), generator=g, device=dev).to(torch.bfloat16)
    zk = [torch.randn((1, 2 * h, Hkv, d), generator=g, device=dev).to(torch.bfloat16) for _ in range(cp)]
    zv = [torch.randn((1, 2 * h, Hkv, d), generator=g, device=dev).to(torch.bfloat16) for _ in range(cp)]
    zdo = torch.randn((1, 2 * h, Hq, d), generator=g, device=dev).to(torch.bfloat16)
    zo = torch.empty_like(zq)
    zl = torch.empty((2, Hq, h), dtype=torch.float32, device=dev)
    zdq = torch.zeros((1, 2 * h, Hq, d), dtype=torch.float32, device=dev)
    zdk = [torch.zeros((1, 2 * h, Hkv, d), dtype=torch.float32, device=dev) for _ in range(cp)]
    zdv = [torch.zeros((1, 2 * h, Hkv, d), dtype=torch.float32, device=dev) for _ in range(cp)]
    zws = ra.ZigzagWorkspace(h, Hq, d, dev, backward=True)
    pairs_z = 2 * cp * h * h + h  # visible pairs of every rank in this layout
    zz = {"seq_len": S, "cp": cp, "live_pairs_per_rank": pairs_z}
    for r in (0, cp - 1):
        def fb(r=r):
            ra.ring_forward_zigzag(zq, zk, zv, r, cp, causal=True, out=zo, lse=zl, workspace=zws)
            ra.ring_backward_zigzag(zq, zk, zv, zo, zl, zdo, r, cp, causal=True, dq=zdq, dk_ranks=zdk, dv_ranks=zdv,
                                    workspace=zws)
        ms = ev_ms(fb, reps=3)
        zz[f"rank{r}"] = {"ms": round(ms, 3), "tflops": round(14.0 * Hq * d * pairs_z / (ms * 1e-3) / 1e12, 2)}
    out["zigzag_64k_cp8"] = zz
    del zq, zk, zv, zdo, zo, zl, zdq, zdk, zdv, zws
    torch.cuda.empty_cache()

    # overlapped receives at the 64K shape (rank 7 of 8): chunks resident, received on a
    # second stream into two slots while the previous step computes, or received on the
    # compute stream (serialized); the transfer is a device-to-device copy standing for
    # the peer's send
    C, cp, Hq, Hkv, d = 8192, 8, 32, 8, 128
    g = torch.Generator(device=dev)
    g.manual_seed(4321)
    oq = torch.randn((1, C, Hq, d), generator=g, device=dev).to(torch.bfloat16)
    okc = [torch.randn((1, C, Hkv, d), generator=g, device=dev).to(torch.bfloat16) for _ in range(cp)]
    ovc = [torch.randn((1, C, Hkv, d), generator=g, device=dev).to(torch.bfloat16) for _ in range(cp)]
    odo = torch.randn((1, C, Hq, d), generator=g, device=dev).to(torch.bfloat16)
    oo = torch.empty_like(oq)
    ol = torch.empty((1, Hq, C), dtype=torch.float32, device=dev)
    odq = torch.zeros((1, C, Hq, d), dtype=torch.float32, device=dev)
    odk = [torch.zeros((1, C, Hkv, d), dtype=torch.float32, device=dev) for _ in range(cp)]
    odv = [torch.zeros((1, C, Hkv, d), dtype=torch.float32, device=dev) for _ in range(cp)]
    ows = ra.RingWorkspace(1, C, Hq, d, dev, backward=True)
    osl = ra.RingSlots(okc[0], ovc[0], backward=True)
    cur = torch.cuda.current_stream()
    comm = torch.cuda.Stream(dev)

    def resident():
        ra.ring_forward(oq, okc, ovc, 7, cp, causal=True, out=oo, lse=ol, workspace=ows)
        ra.ring_backward(oq, okc, ovc, oo, ol, odo, 7, cp, causal=True, dq=odq, dk_chunks=odk, dv_chunks=odv,
                         delta=ows.delta)

    def received(comm_stream):
        ra.ring_forward_overlapped(oq, okc, ovc, 7, cp, causal=True, out=oo, lse=ol, workspace=ows, slots=osl,
                                   stream=cur, comm_stream=comm_stream)
        ra.ring_backward_overlapped(oq, okc, ovc, oo, ol, odo, 7, cp, causal=True, dq=odq, dk_chunks=odk,
                                    dv_chunks=odv, delta=ows.delta, slots=osl, stream=cur, comm_stream=comm_stream)

    t_res = ev_ms(resident, reps=3)
    t_ovl = ev_ms(lambda: received(comm), reps=3)
    t_ser = ev_ms(lambda: received(cur), reps=3)
    per_step_bytes = 2 * C * Hkv * d * 2 + 2 * (2 * C * Hkv * d * 4)  # fwd K+V in; bwd K+V+dK+dV in, dK+dV out
    out["overlapped_ring_64k_cp8_r7"] = {
        "resident_ms": round(t_res, 3), "overlapped_ms": round(t_ovl, 3), "serialized_ms": round(t_ser, 3),
        "received_bytes_per_step_fwd_plus_bwd": per_step_bytes,
        "transfer_hidden_frac": round((t_ser - t_ovl) / (t_ser - t_res), 3) if t_ser > t_res else None}
    del oq, okc, ovc, odo, oo, ol, odq, odk, odv, ows, osl
    torch.cuda.empty_cache()

    # the same 64K attention, other shares: head-sharded (Ulysses: 4 of 32 query heads and
    # 1 of 8 KV heads over all 65536 tokens) and gathered-KV (rank 7's chunk against the
    # gathered row, gather and gradient scatter included)
    S, cp, d = 65536, 8, 128
    C = S // cp
    g = torch.Generator(device=dev)
    g.manual_seed(999)
    uq = torch.randn((1, S, 4, d), generator=g, device=dev).to(torch.bfloat16)
    uk = torch.randn((1, S, 1, d), generator=g, device=dev).to(torch.bfloat16)
    uv = torch.randn((1, S, 1, d), generator=g, device=dev).to(torch.bfloat16)
    udo = torch.randn((1, S, 4, d), generator=g, device=dev).to(torch.bfloat16)
    uo, ul = torch.empty_like(uq), torch.empty((1, 4, S), dtype=torch.float32, device=dev)
    uo32 = torch.empty((1, S, 4, d), dtype=torch.float32, device=dev)
    udq = torch.zeros((1, S, 4, d), dtype=torch.float32, device=dev)
    udk = torch.zeros((1, S, 1, d), dtype=torch.float32, device=dev)
    udv = torch.zeros_like(udk)
    udelta = torch.empty((1, 4, S), dtype=torch.float32, device=dev)

    def uly():
        ra.ulysses_forward(uq, uk, uv, causal=True, out=uo, lse=ul, o_f32=uo32)
        ra.ulysses_backward(uq, uk, uv, uo, ul, udo, causal=True, dq=udq, dk=udk, dv=udv, delta=udelta)

    ums = ev_ms(uly, reps=3)
    upairs = S * (S + 1) // 2
    out["ulysses_64k_h4_of_32"] = {"ms": round(ums, 3), "tflops": round(14.0 * 4 * d * upairs / (ums * 1e-3) / 1e12, 2)}
    del uq, uk, uv, udo, uo, ul, uo32, udq, udk, udv, udelta

    gq = torch.randn((1, C, 32, d), generator=g, device=dev).to(torch.bfloat16)
    gks = [torch.randn((1, C, 8, d), generator=g, device=dev).to(torch.bfloat16) for _ in range(cp)]
    gvs = [torch.randn((1, C, 8, d), generator=g, device=dev).to(torch.bfloat16) for _ in range(cp)]
    gdo = torch.randn((1, C, 32, d), generator=g, device=dev).to(torch.bfloat16)
    gk_all = torch.empty((1, S, 8, d), dtype=torch.bfloat16, device=dev)
    gv_all = torch.empty_like(gk_all)
    go, gl = torch.empty_like(gq), torch.empty((1, 32, C), dtype=torch.float32, device=dev)
    go32 = torch.empty((1, C, 32, d), dtype=torch.float32, device=dev)
    gdq = torch.zeros((1, C, 32, d), dtype=torch.float32, device=dev)
    gdk_all = torch.zeros((1, S, 8, d), dtype=torch.float32, device=dev)
    gdv_all = torch.zeros_like(gdk_all)
    gdks = [torch.empty((1, C, 8, d), dtype=torch.float32, device=dev) for _ in range(cp)]
    gdvs = [torch.empty((1, C, 8, d), dtype=torch.float32, device=dev) for _ in range(cp)]
    gdelta = torch.empty((1, 32, C), dtype=torch.float32, device=dev)

    def gat():
        ra.gather_kv(gks, gvs, gk_all, gv_all)
        ra.gathered_forward(gq, gk_all, gv_all, cp - 1, causal=True, out=go, lse=gl, o_f32=go32)
        ra.gathered_backward(gq, gk_all, gv_all, go, gl, gdo, cp - 1, causal=True, dq=gdq, dk_all=gdk_all,
                             dv_all=gdv_all, delta=gdelta)
        ra.scatter_dkv(gdk_all, gdv_all, gdks, gdvs)

    gms = ev_ms(gat, reps=3)
    gpairs = live_pairs_causal(C, cp - 1)
    out["gathered_kv_64k_cp8_r7"] = {"ms": round(gms, 3),
                                     "tflops": round(14.0 * 32 * d * gpairs / (gms * 1e-3) / 1e12, 2)}
    del gq, gks, gvs, gdo, gk_all, gv_all, go, gl, go32, gdq, gdk_all, gdv_all, gdks, gdvs, gdelta
    torch.cuda.empty_cache()

    # workspace sweep: peak bytes beyond inputs/outputs for one fwd+bwd, CP=8, rank 7
    sweep = []
    for S in (16384, 32768, 65536, 131072):
        C = S // 8
        g = torch.Generator(device=dev)
        g.manual_seed(S)
        qs = torch.randn((1, C, 32, 128), generator=g, device=dev).to(torch.bfloat16)
        kk = [torch.randn((1, C, 8, 128), generator=g, device=dev).to(torch.bfloat16) for _ in range(8)]
        vv = [torch.randn((1, C, 8, 128), generator=g, device=dev).to(torch.bfloat16) for _ in range(8)]
        dd = torch.randn((1, C, 32, 128), generator=g, device=dev).to(torch.bfloat16)
        oo = torch.empty_like(qs)
        ll = torch.empty((1, 32, C), dtype=torch.float32, device=dev)
        dq = torch.zeros((1, C, 32, 128), dtype=torch.float32, device=dev)
        dk = [torch.zeros((1, C, 8, 128), dtype=torch.float32, device=dev) for _ in range(8)]
        dv = [torch.zeros((1, C, 8, 128), dtype=torch.float32, device=dev) for _ in range(8)]
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        ra.ring_forward(qs, kk, vv, 7, 8, causal=True, out=oo, lse=ll)
        ra.ring_backward(qs, kk, vv, oo, ll, dd, 7, 8, causal=True, dq=dq, dk_chunks=dk, dv_chunks=dv)
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated() - base
        sweep.append({"S": S, "workspace_bytes": int(peak), "bytes_per_token": round(peak / S, 1),
                      "score_matrix_bytes_avoided": C * S * 32 * 4})
        del qs, kk, vv, dd, oo, ll, dq, dk, dv
        torch.cuda.empty_cache()
    out["workspace_sweep_cp8_r7"] = sweep
    return out


def cpu_baseline(cfg, wl=None):
    """The fp64 oracle, as it stands, timed on the host cores (one query head per
    worker thread, single-threaded BLAS per worker; heads are independent).

    `value`: forward + backward of a bounded sample of the benchmark's workload, the
    last R query rows of the 64K share (each sees all 65536 keys), all 32 heads, in
    the metric's unit on the sample's algorithmic flops.  `per_config_s`: wall time of
    the oracle on each of the five workloads at full size (ring forward, plus the
    ring backward for the 8K backward workload); the 64K forward and the benchmark's
    64K forward + backward are extrapolated from the sample by live pairs (each row
    of the sample sees at least as many keys as an average row) and labelled so."""
    import numpy as np

    import oracle
    from oracle import parallel as opar
    from synthetic import CONFIGS, LLAMA3_8K_BWD, LLAMA3_8K_FWD, PACKED16K_FWD, TINY_RING, make_workload

    workers = opar.host_cores()
    per_cfg = {}

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    # tiny fp32 ring (one head): the plain call
    w1 = make_workload(TINY_RING, q_chunks=[TINY_RING.rank])
    per_cfg[TINY_RING.name] = round(timed(lambda: oracle.ring_forward(
        w1.q_local, w1.k_chunks, w1.v_chunks, TINY_RING.rank, TINY_RING.CP, TINY_RING.scale, True)), 3)
    # 8K forward and packed 16K forward: the ring forward per head
    for c in (LLAMA3_8K_FWD, PACKED16K_FWD):
        w = make_workload(c, q_chunks=[c.rank])
        seg = oracle.segment_ids(w.position_ids) if c.packed else None
        per_cfg[c.name] = round(timed(lambda: opar.ring_forward_heads(
            w.q_local, w.k_chunks, w.v_chunks, c.rank, c.CP, c.scale, True, seg, workers=workers)), 3)
    # 8K backward: ring forward (for O, LSE) + ring backward
    c5 = LLAMA3_8K_BWD
    w5 = make_workload(c5, q_chunks=[c5.rank])

    def fb5():
        o, lse = opar.ring_forward_heads(w5.q_local, w5.k_chunks, w5.v_chunks, c5.rank, c5.CP, c5.scale, True,
                                         workers=workers)
        opar.ring_backward_heads(w5.q_local, w5.k_chunks, w5.v_chunks, o, lse, w5.do, c5.rank, c5.CP, c5.scale,
                                 True, workers=workers)

    per_cfg[c5.name] = round(timed(fb5), 3)

    # the bounded sample of the benchmark's 64K workload
    if wl is None:
        wl = make_workload(cfg, q_chunks=[cfg.rank])
    C, r = cfg.C, cfg.rank
    R = 512
    rows = np.arange(C - R, C)
    q_rows = wl.q_local[:, rows]
    do_rows = wl.do[:, rows]
    k_full, v_full = wl.k_full(), wl.v_full()
    q_idx = r * C + rows
    k_idx = np.arange(cfg.S)
    res = {}

    def fwd():
        res["o"], res["lse"] = opar.attention_full_heads(q_rows, k_full, v_full, q_idx, k_idx, cfg.scale, True,
                                                         workers=workers)

    def bwd():
        delta = oracle.bwd_delta(res["o"], do_rows)
        opar.attention_bwd_full_heads(q_rows, k_full, v_full, do_rows, res["lse"], delta, q_idx, k_idx, cfg.scale,
                                      True, workers=workers)

    t_f = timed(fwd)
    t_b = timed(bwd)
    dt = t_f + t_b
    pairs = int(np.sum(q_idx + 1))
    flops = 14.0 * cfg.Hq * cfg.d * pairs
    all_pairs = live_pairs_causal(C, r)
    c3 = CONFIGS["ctx64k_cp8_r7_fwd"]
    per_cfg[c3.name + " (extrapolated from the sample)"] = round(t_f * all_pairs / pairs, 1)
    per_cfg[cfg.name + " (extrapolated from the sample)"] = round(dt * all_pairs / pairs, 1)
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(workers), "kind": "oracle",
            "affinity_cores": opar.affinity_cores(), "blas": opar.blas_info(),
            "per_config_s": per_cfg,
            "sample": f"fp64 numpy oracle fwd+bwd of the last {R} query rows of the 64K share "
                      f"(rank 7, all {cfg.Hq} heads, {cfg.S} keys each): {pairs} live pairs, "
                      f"{flops:.3e} algorithmic flop in {dt:.1f} s (fwd {t_f:.1f} s, bwd {t_b:.1f} s) on "
                      f"{workers} worker threads, one query head each, single-threaded {opar.blas_info()} BLAS"}


if __name__ == "__main__":
    main()
