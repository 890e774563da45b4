#!/usr/bin/env python3
"""Forward throughput of Reformer shared-QK LSH attention on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload text64k]

One step is one whole forward (hash, sort, gather, chunked attention, unsort
and combine) over one batch of seeded synthetic inputs already resident in
HBM. Prints ONE JSON line: tokens/s (batch * seq_len / seconds per forward),
the roofline of the dominant kernel (per-stage HIP events recorded by the
library on the launch stream during the timed region), and the fp64 oracle
timed on the host cores over a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "LSH-attn fwd tokens/sec at L=64K, 4 rounds; % MFMA / HBM roofline"

# MI355X published peaks
PEAK = {
    "hbm_GBps": 8000.0,
    "mfma_bf16_TFLOPs": 2500.0,
    "mfma_fp16_TFLOPs": 2500.0,
    "fp32_vector_TFLOPs": 157.3,
    "fp64_vector_TFLOPs": 78.6,
}


def esize(dt: str) -> int:
    return 2 if dt == "bf16" else 4


def algorithmic_units(w, out_dtype: str, round_bytes: int = 2):
    """Per-launch algorithmic work of each stage's kernel (what the method
    must compute or move, not what an implementation happens to move).
    N = B*H*L token-heads, R rounds, d head dim, nb buckets, m chunk length;
    round_bytes = bytes per element of the per-round outputs kept between the
    attention and the combine (2 for fp16, 4 with the fp32 option)."""
    N = w.batch * w.heads * w.seq_len
    R, d, nb, m = w.n_rounds, w.head_dim, w.n_buckets, w.chunk_len
    e, eo, ro = esize(w.dtype), esize(out_dtype), round_bytes
    return {
        # projection x.R for every token-head and round: nb/2 MACs of length d
        "hash": {"flops": N * R * d * nb, "bytes": N * d * e + N * R * 2},
        # read bucket ids twice (count, scatter), write the permutation
        "sort": {"bytes": N * R * (2 + 2 + 4)},
        # read two rows, write two rows per (round, slot), plus the perm read
        "gather": {"bytes": N * R * (4 * d * e + 4)},
        # QK^T and PV over the 2m-key window of every query-round; rows read
        # through the permutation, per-round output row and lse written
        "attend": {"flops": N * R * 4 * d * 2 * m,
                   "bytes": N * R * (2 * d * e + 4 + d * ro + 4)},
        # R per-round rows and lse read, one output row written
        "combine": {"bytes": N * R * (d * ro + 4) + N * d * eo},
    }


# How each stage's kernel is bound in the current implementation, and the peak
# it is measured against.
KERNEL_BOUND = {
    "hash": ("mfma", "mfma_fp16_TFLOPs"),       # fp16 MFMA projection (+ rare fp64 re-score)
    "sort": ("hbm", "hbm_GBps"),
    "gather": ("hbm", "hbm_GBps"),
    "attend": ("mfma", "mfma_bf16_TFLOPs"),     # bf16 MFMA QK^T and PV
    "combine": ("hbm", "hbm_GBps"),
}


def roofline(stage: str, units: dict, ms: float, traffic=None):
    bound, peak_key = KERNEL_BOUND[stage]
    u = units[stage]
    if peak_key == "hbm_GBps":
        achieved = u["bytes"] / (ms * 1e-3) / 1e9
        unit = "GB/s"
    else:
        achieved = u["flops"] / (ms * 1e-3) / 1e12
        unit = "TFLOP/s"
    peak = PEAK[peak_key]
    return {"kernel": stage, "bound": bound, "achieved": round(achieved, 3), "peak": peak,
            "unit": unit, "frac": round(achieved / peak, 5), "traffic": traffic,
            "algorithmic_bytes": u.get("bytes"), "algorithmic_flops": u.get("flops")}


def cpu_baseline(w, inp, heads: int):
    """The fp64 oracle as it stands, on batch 0 and the first `heads` heads at
    full sequence length, all rounds; scaled to tokens/s of the whole workload."""
    import numpy as np

    import oracle

    threads = len(os.sched_getaffinity(0))
    env_threads = os.environ.get("OMP_NUM_THREADS")
    if env_threads:
        threads = min(threads, int(env_threads))
    sub = w.with_(batch=1, heads=heads)
    c = oracle.config(sub)
    qk = np.ascontiguousarray(inp.qk[:1, :heads], dtype=np.float64)
    v = np.ascontiguousarray(inp.v[:1, :heads], dtype=np.float64)
    rot = None if inp.rotations is None else inp.rotations.astype(np.float64)
    oracle.build(force=False)
    t0 = time.perf_counter()
    oracle.forward(c, qk, v, rot)
    t = time.perf_counter() - t0
    frac = heads / (w.batch * w.heads)
    value = w.batch * w.seq_len * frac / t
    used = min(threads, heads * w.n_rounds)
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(value, 3), "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": f"batch 0, heads 0..{heads - 1} of {w.heads}, full L={w.seq_len}, "
                      f"all {w.n_rounds} rounds ({frac:.4f} of the workload), fp64 oracle "
                      f"forward in {t:.2f} s; OpenMP over (head, round) segments",
            "seconds": round(t, 3), "cpu_model": model, "threads_available": threads}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="text64k")
    ap.add_argument("--out-dtype", default=None, choices=[None, "bf16", "fp32"])
    ap.add_argument("--separate-gather", action="store_true")
    ap.add_argument("--fp32-round-outputs", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=0,
                    help="heads in the oracle sample (0: as many as rounds fit the cores)")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="HBM bytes per launch measured with rocprofv3 counters")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}); the path shards over (batch, head) with no exchange, so more GPUs "
              "are not part of this benchmark.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import lsh_attention_hash_amd as lat
    import workloads

    w = workloads.get(args.workload)
    out_dtype = args.out_dtype or w.dtype
    inp = workloads.make_inputs(w)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if w.dtype == "bf16":
        qk = torch.from_numpy(inp.qk_bits.view(np.int16)).to(dev).view(torch.bfloat16)
        v = torch.from_numpy(inp.v_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        qk = torch.from_numpy(inp.qk).to(dev)
        v = torch.from_numpy(inp.v).to(dev)
    rot = None if inp.rotations is None else torch.from_numpy(inp.rotations).to(dev)
    tdt = {"bf16": torch.bfloat16, "fp32": torch.float32}
    op = lat.LSHAttention(w.batch, w.heads, w.seq_len, w.head_dim, w.n_buckets, w.n_rounds,
                          w.chunk_len, w.causal, dtype=tdt[w.dtype], out_dtype=tdt[out_dtype],
                          separate_gather=args.separate_gather,
                          fp32_round_outputs=args.fp32_round_outputs)
    out = torch.empty((w.batch, w.heads, w.seq_len, w.head_dim), dtype=tdt[out_dtype],
                      device=dev)
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        op(qk, v, rot, out=out)
    torch.cuda.synchronize()

    op.set_timing(args.steps)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        op(qk, v, rot, out=out)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end) / args.steps
    stage_ms, n_timed = op.get_timing()
    stage_avg = {k: v_ / max(n_timed, 1) for k, v_ in stage_ms.items()}
    stats = op.stats()

    fp16_rounds = w.dtype == "bf16" and w.chunk_len == 64 and not args.fp32_round_outputs
    units = algorithmic_units(w, out_dtype, 2 if fp16_rounds else 4)
    if not args.separate_gather:
        stage_avg.pop("gather")   # rows are read through the permutation inside attend
    dominant = max(stage_avg, key=stage_avg.get)
    traffic = None
    if os.path.exists(args.traffic_json):
        try:
            with open(args.traffic_json) as f:
                tj = json.load(f)
            entry = tj.get(args.workload, {}).get(dominant)
            if entry and entry.get("source_hash") == kernel_source_hash(dominant):
                traffic = entry.get("bytes_per_launch")
        except (OSError, ValueError):
            traffic = None
    rl = roofline(dominant, units, stage_avg[dominant], traffic)
    per_stage = {k: {"ms": round(stage_avg[k], 5)} for k in stage_avg}
    for k in per_stage:
        if stage_avg[k] > 0:
            r = roofline(k, units, stage_avg[k])
            per_stage[k].update({"achieved": r["achieved"], "unit": r["unit"],
                                 "frac": r["frac"], "bound": r["bound"]})

    tokens = w.batch * w.seq_len
    res = {
        "metric": METRIC,
        "value": round(tokens / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads,
                   "seq_len": w.seq_len, "head_dim": w.head_dim, "n_buckets": w.n_buckets,
                   "n_rounds": w.n_rounds, "chunk_len": w.chunk_len, "causal": w.causal,
                   "qk_v_dtype": w.dtype, "out_dtype": out_dtype,
                   "inputs": f"{w.kind} seeded (qk {1000 + w.seed_base}, v {2000 + w.seed_base},"
                             f" R {3000 + w.seed_base})",
                   "separate_gather": bool(args.separate_gather),
                   "round_outputs": "fp16" if fp16_rounds else "fp32"},
        "roofline": rl,
        "stages": per_stage,
        "token_heads_per_s": round(w.batch * w.heads * w.seq_len / (ms * 1e-3), 1),
        "hash_stats": stats,
        "wall_s_timed": round(wall, 4),
    }
    if not args.no_cpu_baseline:
        heads = args.cpu_heads or max(1, min(w.heads, len(os.sched_getaffinity(0)) // w.n_rounds))
        res["cpu_baseline"] = cpu_baseline(w, inp, heads)
    op.close()
    print(json.dumps(res), flush=True)


def kernel_source_hash(stage: str) -> str:
    """Hash of the source file of a stage's kernel; counter-derived traffic is
    only reported while the kernel source is unchanged."""
    import hashlib
    fname = {"hash": "hash.hip", "sort": "sort.hip", "gather": "gather.hip",
             "attend": "attend.hip", "combine": "combine.hip"}[stage]
    path = os.path.join(ROOT, "lsh_attention_hash_amd", "csrc", fname)
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


if __name__ == "__main__":
    main()
