"""Benchmark: useful causal attention TFLOP/s of one CP rank's share on one GPU.

Default workload: text L=65536, P=8 (16 chunks of 4096), rank 3, GQA 32/8
heads, head_dim 128, bf16 Q/K/V ~ N(0,1), batch 1. One step is one call of
cp_attn_rank_fwd: host plan + upload, V relayout, attention over all P ring
steps (the Q gather fused into the kernel's Q loads), LSE merge. Inputs are
resident in HBM before timing starts.

Prints one JSON line. ``roofline`` covers the dominant kernel (the per-step
attention): achieved = useful FLOPs per launch / its average duration, timed
with HIP events recorded by the library on the launch stream.
``cpu_baseline`` times the fp64 oracle on a bounded sample of the same
rank's rows on this host's cores (worker processes, spawned before the GPU
is touched), and, on the default workload, the literal form of the oracle
(whole sequence, then select) beside its rows-only form on workload 2.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0
METRIC = "useful causal attn TFLOP/s per CP-rank share (1 GPU) + % of bf16 MFMA peak"
PMC_FILE = os.path.join(ROOT, "profiles", "attn_bf16_text64k_rank3_pmc.json")
ATTN_SRC = os.path.join(ROOT, "context_parallelism_amd", "csrc", "attn_bf16.hip")


def hip_runtime():
    """The HIP runtime library already loaded in this process (torch's)."""
    for line in open("/proc/self/maps"):
        path = line.split()[-1]
        if "libamdhip64.so" in path:
            lib = ctypes.CDLL(path)
            lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
            return lib
    raise RuntimeError("libamdhip64 is not loaded")


def traffic_from_profile():
    """HBM bytes per attention launch from the committed rocprofv3 counters,
    or None if they were taken on a different version of the kernel."""
    if not os.path.exists(PMC_FILE):
        return None
    doc = json.load(open(PMC_FILE))
    sha = hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest()
    if doc.get("attn_bf16_sha256") != sha:
        return None
    return doc.get("hbm_bytes_per_launch")


def cpu_baseline(w, q, k, v, n_img, cu, target_s: float, split: str = "head_tail"):
    """The fp64 oracle, as it stands, on a bounded sample of the rank's rows,
    its (KV group, 256-row block) tasks spread over worker processes (one per
    core of this process's affinity set, at most 16; BLAS one thread each).
    Must run before this process touches the GPU: the workers are spawned.
    A small calibration pass sizes the sample to about ``target_s`` seconds."""
    import numpy as np

    import oracle
    from oracle.pool import default_workers, rank_attention_pooled

    workers = default_workers()
    index, _ = oracle.partition_index(w.seq_len, n_img, cu, w.cp_size, w.rank, split)
    R = len(index)

    def run(n):
        rows = np.unique(np.linspace(0, R - 1, n).astype(np.int64))
        st = {}
        rank_attention_pooled(q, k, v, n_img, cu, w.cp_size, w.rank, local_rows=rows, split=split,
                              workers=workers, row_chunk=256, executor="process", stats=st)
        return rows, st["wall_s"]

    n0 = min(R, 32 * workers)
    rows, dt = run(n0)
    if dt < target_s / 2 and n0 < R:
        rows, dt = run(min(R, int(n0 * target_s / max(dt, 1e-3))))
    # a real row at position p of its sample sees p + 1 keys; pads see none
    ids = index[rows].astype(np.int64)
    ids = ids[ids >= 0]
    starts = w.cu_seqlens.astype(np.int64)
    pairs = int(np.sum(ids - starts[np.searchsorted(starts, ids, side="right") - 1] + 1))
    flops = 4.0 * w.head_dim * w.heads * pairs
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(workers), "kind": "oracle",
            "sample": f"{len(rows)} of {R} rank-local rows (evenly spaced), all {w.heads} heads, "
                      f"{pairs} useful pairs/head, {dt:.1f} s on {workers} worker processes "
                      f"(affinity set of this process, at most 16; one BLAS thread each), fp64 numpy, "
                      f"rows-only form"}


def cpu_literal_workload2(target_workers=None):
    """The literal oracle -- whole-sequence causal attention, then the rank's
    rows selected -- on workload 2 (text 8192, P=4, rank 0, 16 heads), one
    head per worker process, timed beside its rows-only form."""
    import numpy as np

    import oracle
    import workloads
    from oracle.pool import default_workers, rank_attention_pooled

    w = workloads.get(2)
    q, k, v = workloads.make_inputs(w)
    workers = target_workers or default_workers()
    res = {}
    for form, literal in (("literal", True), ("rows_only", False)):
        st = {}
        rank_attention_pooled(q, k, v, None, None, w.cp_size, 0, literal=literal, workers=workers,
                              executor="process", stats=st)
        res[form] = st["wall_s"]
    _, pairs = oracle.pair_counts(w.seq_len, None, None, w.cp_size, 0)
    useful = 4.0 * w.head_dim * w.heads * pairs
    L = w.seq_len
    full = 4.0 * w.head_dim * w.heads * L * (L + 1) // 2
    return {"workload": w.name, "cores": int(workers),
            "literal_s": round(res["literal"], 2), "rows_only_s": round(res["rows_only"], 2),
            "literal_useful_TFLOPs": round(useful / res["literal"] / 1e12, 4),
            "literal_computed_TFLOPs": round(full / res["literal"] / 1e12, 4),
            "rows_only_TFLOPs": round(useful / res["rows_only"] / 1e12, 4),
            "note": "literal computes all 8192 rows (4x the rank's useful work) before selecting the rank's 2048"}


def timed_calls(ra, hip, steps, warmup):
    """Median per-call and attention-stage times (ms) of `steps` calls, HIP events."""
    import numpy as np
    import torch

    evs = []
    for _ in range(steps):
        row = []
        for _ in range(6):
            e = ctypes.c_void_p()
            assert hip.hipEventCreate(ctypes.byref(e)) == 0
            row.append(e.value)
        evs.append(row)
    for _ in range(warmup):
        ra()
    torch.cuda.synchronize()
    for i in range(steps):
        ra(evs[i])
    torch.cuda.synchronize()

    def el(a, b):
        ms = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
        return ms.value
    call = np.median([el(e[0], e[5]) for e in evs])
    attn = np.median([el(e[3], e[4]) for e in evs])
    for row in evs:
        for e in row:
            hip.hipEventDestroy(ctypes.c_void_p(e))
    return float(call), float(attn)


def compare_splits(w, args):
    """Every rank share of one workload under head-tail pairing and under the
    plain contiguous split, same kernels. The CP step waits for its slowest
    rank, so the figure of merit is the maximum over ranks."""
    import torch

    import context_parallelism_amd as cp
    import workloads

    dev = torch.device("cuda:0")
    q, k, v = workloads.make_inputs(w)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    n_img = w.n_img_array if any(w.n_img) else None
    cu = w.cu_seqlens if w.n_samples > 1 else None
    hip = hip_runtime()
    res = {}
    for split in ("head_tail", "contiguous"):
        rows = []
        for r in range(w.cp_size):
            ra = cp.RankAttention(qd, kd, vd, cp_size=w.cp_size, cp_rank=r, n_img=n_img, cu_seqlens=cu,
                                  split=split)
            _, pairs = cp.pair_counts(w.seq_len, n_img, cu, cp_size=w.cp_size, cp_rank=r, split=split)
            call, attn = timed_calls(ra, hip, args.steps, args.warmup)
            rows.append({"rank": r, "pairs_per_head": pairs, "call_ms": round(call, 4),
                         "attention_ms": round(attn, 4)})
            del ra
            print(f"{split} rank {r}: {pairs} pairs/head, call {call:.4f} ms", file=sys.stderr, flush=True)
        calls = [x["call_ms"] for x in rows]
        res[split] = {"ranks": rows, "max_call_ms": max(calls), "mean_call_ms": round(sum(calls) / len(calls), 4),
                      "max_over_mean": round(max(calls) / (sum(calls) / len(calls)), 4)}
    useful = 4.0 * w.head_dim * w.heads * sum(x["pairs_per_head"] for x in res["head_tail"]["ranks"])
    line = {"mode": "compare_splits", "workload": w.name, "cp_size": w.cp_size, "steps": args.steps,
            "warmup": args.warmup, "splits": res,
            "job_step_ms": {s: res[s]["max_call_ms"] for s in res},
            "job_useful_TFLOPs_per_gpu": {s: round(useful / w.cp_size / (res[s]["max_call_ms"] * 1e-3) / 1e12, 2)
                                          for s in res},
            "head_tail_speedup": round(res["contiguous"]["max_call_ms"] / res["head_tail"]["max_call_ms"], 4)}
    print(json.dumps(line), flush=True)


def compare_ulysses(w, args):
    """One GPU's attention share of the same CP job in two layouts: the ring
    (head-tail rank share, all heads, P steps) and Ulysses (after the
    all-to-all over heads: every token, heads/P query and kv_heads/P KV
    heads, one causal pass, no steps). Both hold the same useful work for a
    single-sample text workload. The all-to-all itself is not run (one GPU)."""
    import torch

    import context_parallelism_amd as cp
    import workloads

    P = w.cp_size
    if w.n_samples != 1 or any(w.n_img) or w.heads % P or w.kv_heads % P:
        raise SystemExit("--ulysses needs a single-sample text workload whose head counts P divides")
    dev = torch.device("cuda:0")
    q, k, v = workloads.make_inputs(w)
    hip = hip_runtime()
    res = {}
    # ring: the headline rank share
    ra = cp.RankAttention(q.to(dev), k.to(dev), v.to(dev), cp_size=P, cp_rank=w.rank)
    _, pairs = cp.pair_counts(w.seq_len, cp_size=P, cp_rank=w.rank)
    call, attn = timed_calls(ra, hip, args.steps, args.warmup)
    useful = 4.0 * w.head_dim * w.heads * pairs
    res["ring"] = {"heads": w.heads, "kv_heads": w.kv_heads, "rows": ra.R, "useful_flop": useful,
                   "call_ms": round(call, 4), "attention_ms": round(attn, 4),
                   "TFLOPs": round(useful / (call * 1e-3) / 1e12, 2)}
    del ra
    # Ulysses: heads [0, H/P) with their KV heads [0, Hkv/P) -- same head map
    hq, hk = w.heads // P, w.kv_heads // P
    qu = q[:, :hq].contiguous().to(dev)
    ku, vu = k[:, :hk].contiguous().to(dev), v[:, :hk].contiguous().to(dev)
    ru = cp.RankAttention(qu, ku, vu, cp_size=1, cp_rank=0)
    _, pairs_u = cp.pair_counts(w.seq_len, cp_size=1, cp_rank=0)
    call, attn = timed_calls(ru, hip, args.steps, args.warmup)
    useful_u = 4.0 * w.head_dim * hq * pairs_u
    res["ulysses"] = {"heads": hq, "kv_heads": hk, "rows": ru.R, "useful_flop": useful_u,
                      "call_ms": round(call, 4), "attention_ms": round(attn, 4),
                      "TFLOPs": round(useful_u / (call * 1e-3) / 1e12, 2)}
    line = {"mode": "compare_ulysses", "workload": w.name, "cp_size": P, "steps": args.steps,
            "warmup": args.warmup, "shares": res,
            "ring_over_ulysses_time": round(res["ring"]["call_ms"] / res["ulysses"]["call_ms"], 4)}
    print(json.dumps(line), flush=True)


def bench_backward(w, args):
    """cp_attn_rank_bwd on the rank share: delta, transposes, dQ and dK/dV.
    Useful FLOPs follow the usual backward count of five products per
    (query, key) pair -- QK^T, dO V^T, P^T dO, dS^T Q, dS K -- i.e. 2.5x the
    forward's (the kernels recompute QK^T and dO V^T once more: 7 products)."""
    import numpy as np
    import torch

    import context_parallelism_amd as cp
    import workloads

    if w.dtype != "bf16" or w.head_dim != 128:
        raise SystemExit("--backward: bf16 with head_dim 128 only")
    dev = torch.device("cuda:0")
    q, k, v = workloads.make_inputs(w)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    n_img = w.n_img_array if any(w.n_img) else None
    cu = w.cu_seqlens if w.n_samples > 1 else None
    out, lse = cp.rank_fwd(qd, kd, vd, cp_size=w.cp_size, cp_rank=w.rank, n_img=n_img, cu_seqlens=cu,
                           split=args.split)
    g = torch.Generator(device="cpu").manual_seed(w.seed + 7)
    dout = torch.randn(out.shape, generator=g).to(torch.bfloat16).to(dev)
    bw = cp.RankAttentionBackward(qd, kd, vd, cp_size=w.cp_size, cp_rank=w.rank, n_img=n_img,
                                  cu_seqlens=cu, split=args.split)
    for _ in range(args.warmup):
        bw(out, lse, dout)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        a.record()
        bw(out, lse, dout)
        b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = np.array([a.elapsed_time(b) for a, b in evs])
    _, pairs = cp.pair_counts(w.seq_len, n_img, cu, cp_size=w.cp_size, cp_rank=w.rank, split=args.split)
    useful = 2.5 * 4.0 * w.head_dim * w.heads * pairs
    med = float(np.median(ms))
    line = {"mode": "backward", "metric": "useful causal attn backward TFLOP/s per CP-rank share (1 GPU)",
            "value": round(useful / (med * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "ms_median": round(med, 4),
            "ms_p10": round(float(np.percentile(ms, 10)), 4), "ms_p90": round(float(np.percentile(ms, 90)), 4),
            "wall_ms_per_call": round(wall / args.steps * 1e3, 4), "useful_flop": useful,
            "pct_of_peak": round(100.0 * useful / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
            "config": {"workload": w.name, "cp_rank": w.rank, "split": args.split, "rank_rows": bw.R}}
    print(json.dumps(line), flush=True)


def bench_hbm(w, args):
    """A2 (gather) and A5 (merge) are HBM-bound; report GB/s of algorithmic
    bytes against the 8 TB/s peak and against a plain device copy of about
    the same size timed in the same process. A 512 MiB fill before each
    timed call evicts the 256 MB MALL, so no call finds its inputs (or the
    previous call's output) in cache."""
    import numpy as np
    import torch

    import context_parallelism_amd as cp

    dev = torch.device("cuda:0")
    n_img = w.n_img_array if any(w.n_img) else None
    cu = w.cu_seqlens if w.n_samples > 1 else None
    index, _ = cp.partition_index(w.seq_len, n_img, cu, cp_size=w.cp_size, cp_rank=w.rank)
    R, H, D, P = len(index), w.heads, w.head_dim, w.cp_size
    esize = 2 if w.dtype == "bf16" else 4
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    g = torch.Generator(device="cpu").manual_seed(w.seed)
    q = torch.randn((w.seq_len, H, D), generator=g).to(dt).to(dev)
    part = torch.randn((P, R, H, D), generator=g).to(dev)
    plse = torch.randn((P, H, R), generator=g).to(dev)
    mask = np.full(R, (1 << P) - 1, dtype=np.uint64).astype(np.uint32)

    # between timed calls, a 512 MiB fill evicts the 256 MB MALL (last-level
    # cache), so every call reads its inputs from HBM
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    def time_ms(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for a, b in evs:
            flush.fill_(1)
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in evs]))

    gather_bytes = 2 * R * H * D * esize
    merge_bytes = P * R * H * (D + 1) * 4 + R * H * (D * esize + 4)
    # buffers made once; the timed calls are the C-ABI calls alone
    idx_d = torch.as_tensor(index).to(dev)
    qr = torch.empty((R, H, D), dtype=dt, device=dev)
    mask_d = torch.as_tensor(mask.view(np.int32)).to(dev)
    out = torch.empty((R, H, D), dtype=dt, device=dev)
    lse = torch.empty((H, R), dtype=torch.float32, device=dev)
    code = cp.CP_DTYPE_BF16 if w.dtype == "bf16" else cp.CP_DTYPE_F32
    stream = torch.cuda.current_stream().cuda_stream

    def gather():
        cp.check(cp.cp_gather_rows(q.data_ptr(), code, w.seq_len, H * D, idx_d.data_ptr(), R, qr.data_ptr(),
                                   stream), "cp_gather_rows")

    def merge():
        cp.check(cp.cp_lse_merge(part.data_ptr(), plse.data_ptr(), mask_d.data_ptr(), P, R, H, D, code,
                                 out.data_ptr(), lse.data_ptr(), stream), "cp_lse_merge")
    t_gather = time_ms(gather)
    t_merge = time_ms(merge)
    src = torch.empty(merge_bytes // 2 // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    t_copy = time_ms(lambda: dst.copy_(src))
    copy_bytes = 2 * src.numel() * 4

    def rate(b, t):
        return round(b / (t * 1e-3) / 1e9, 1)
    copy_gbps = rate(copy_bytes, t_copy)
    line = {"mode": "hbm", "unit": "GB/s", "peak_GBps": 8000.0, "cache": "MALL flushed before every timed call",
            "gather": {"kernel": "gather_rows_kernel", "bytes": gather_bytes, "ms": round(t_gather, 4),
                       "GBps": rate(gather_bytes, t_gather),
                       "frac_of_copy": round(rate(gather_bytes, t_gather) / copy_gbps, 3)},
            "merge": {"kernel": "lse_merge_kernel", "bytes": merge_bytes, "ms": round(t_merge, 4),
                      "GBps": rate(merge_bytes, t_merge), "steps_per_row": P,
                      "frac_of_copy": round(rate(merge_bytes, t_merge) / copy_gbps, 3)},
            "copy": {"bytes": copy_bytes, "ms": round(t_copy, 4), "GBps": copy_gbps},
            "config": {"workload": w.name, "cp_rank": w.rank, "rank_rows": R}}
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=4, help="synthetic workload number (1-5)")
    ap.add_argument("--rank", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="CPU-baseline budget: the oracle sample is sized to take about this long")
    ap.add_argument("--split", choices=["head_tail", "contiguous"], default="head_tail",
                    help="text split over the CP group (contiguous: the plain P-way split)")
    ap.add_argument("--compare-splits", action="store_true",
                    help="instead of the headline line: time every rank share under both splits "
                         "and print one JSON line with the per-rank times (the CP step waits for "
                         "the slowest rank)")
    ap.add_argument("--ulysses", action="store_true",
                    help="instead of the headline line: one GPU's share under Ulysses (all-to-all "
                         "over heads: full-sequence causal attention on heads/P and kv_heads/P) next "
                         "to the ring rank share of the same workload; one JSON line")
    ap.add_argument("--backward", action="store_true",
                    help="instead of the headline line: time cp_attn_rank_bwd (gradients of the rank "
                         "share) on the workload; one JSON line")
    ap.add_argument("--hbm", action="store_true",
                    help="instead of the headline line: the HBM-bound steps on the workload's shape -- "
                         "the Q gather (cp_gather_rows) and the LSE merge (cp_lse_merge, every row with "
                         "all P steps) -- in GB/s against the 8 TB/s peak and a device copy; one JSON line")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="instead of the attention, run --steps plain device copies of this many MiB "
                         "(the reference kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one CP rank's share on one GPU; --gpus {args.gpus} is not supported "
              "(no multi-GPU path is built in this library)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import context_parallelism_amd as cp
    import workloads

    if args.copy_mib:
        n = args.copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": args.warmup + args.steps}), flush=True)
        return

    w = workloads.get(args.workload)
    if args.compare_splits:
        compare_splits(w, args)
        return
    if args.ulysses:
        compare_ulysses(w, args)
        return
    if args.backward:
        bench_backward(w, args)
        return
    if args.hbm:
        bench_hbm(w, args)
        return
    rank = w.rank if args.rank is None else args.rank
    if rank != w.rank:
        import dataclasses
        w = dataclasses.replace(w, ranks=(rank,))
    q, k, v = workloads.make_inputs(w)
    n_img = w.n_img_array if any(w.n_img) else None
    cu = w.cu_seqlens if w.n_samples > 1 else None
    # the CPU baseline first: its worker processes are spawned, which this
    # process does before it touches the GPU
    cpu = None
    if not args.no_cpu_baseline:
        print("cpu baseline (fp64 oracle, worker processes) ...", file=sys.stderr, flush=True)
        try:
            cpu = cpu_baseline(w, q, k, v, n_img, cu, args.cpu_seconds, args.split)
            if args.workload == 4:
                cpu["literal_vs_rows_only"] = cpu_literal_workload2()
        except Exception as e:  # the baseline is reported, never the product: keep the GPU line
            cpu = {"error": f"{type(e).__name__}: {e}"}
        print(f"cpu baseline: {json.dumps(cpu)}", file=sys.stderr, flush=True)
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    ra = cp.RankAttention(qd, kd, vd, cp_size=w.cp_size, cp_rank=rank, n_img=n_img, cu_seqlens=cu,
                          split=args.split)
    _, pairs = cp.pair_counts(w.seq_len, n_img, cu, cp_size=w.cp_size, cp_rank=rank, split=args.split)
    useful = 4.0 * w.head_dim * w.heads * pairs

    hip = hip_runtime()
    K = args.steps

    def make_events(n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert hip.hipEventCreate(ctypes.byref(e)) == 0
            out.append(e.value)
        return out

    def elapsed(a, b):
        ms = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
        return ms.value

    # timed steps: only the attention kernel's two boundaries are recorded
    # (events 3 and 4), so the step carries no empty-stage event records
    kern = [make_events(2) for _ in range(K)]
    for _ in range(args.warmup):
        ra()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ra([None, None, None, kern[i][0], kern[i][1], None])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    attn = np.array([elapsed(a, b) for a, b in kern])
    # stage breakdown: a separate, untimed pass with all six boundaries
    events = [make_events(6) for _ in range(K)]
    for i in range(K):
        ra(events[i])
    torch.cuda.synchronize()
    stage = np.array([[elapsed(e[j], e[j + 1]) for j in range(5)] for e in events])  # ms
    call = np.array([elapsed(e[0], e[5]) for e in events])
    for evs in events + kern:
        for e in evs:
            hip.hipEventDestroy(ctypes.c_void_p(e))

    ms_per_step = wall / K * 1e3
    value = useful / (wall / K) / 1e12
    attn_ms = float(attn.mean())
    achieved = useful / (attn_ms * 1e-3) / 1e12
    R = ra.R
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic: Q/K/V ~ N(0,1) drawn from numpy default_rng(%d), rounded to %s" % (w.seed, w.dtype),
        "config": {"workload": w.name, "seq_len": w.seq_len, "cp_size": w.cp_size, "cp_rank": rank,
                   "split": args.split,
                   "heads": w.heads, "kv_heads": w.kv_heads, "head_dim": w.head_dim,
                   "n_img": list(w.n_img), "samples": w.n_samples, "rank_rows": R,
                   "useful_pairs_per_head": pairs, "useful_flop": useful},
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "stages_ms": {"note": "separate untimed pass with all six stage events; the Q gather is part of "
                              "the attention kernel's Q loads and V is read in place",
                      "plan_upload": round(float(stage[:, 0].mean()), 4),
                      "attention": round(attn_ms, 4),
                      "merge": round(float(stage[:, 4].mean()), 4),
                      "call_median": round(float(np.median(call)), 4),
                      "call_p10": round(float(np.percentile(call, 10)), 4),
                      "call_p90": round(float(np.percentile(call, 90)), 4)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_from_profile(),
                     "kernel": ("attn_rank_bf16_d128_kernel (all ring steps of a row tile per workgroup, one online softmax across them)" if w.head_dim == 128 else "attn_step_bf16_kernel (per-step attention, all ring steps, one launch)")
                               },
    }
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
