#!/usr/bin/env python3
"""Forward throughput of Reformer shared-QK LSH attention on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload text64k] [--backward]

One step is one whole forward (hash, sort, gather, chunked attention, unsort
and combine) over one batch of seeded synthetic inputs already resident in
HBM. Prints ONE JSON line: tokens/s (batch * seq_len / seconds per forward),
the roofline of the dominant kernel (per-stage HIP events recorded by the
library on the launch stream during the timed region), and the fp64 oracle
timed on the host cores over a bounded sample of the same workload.

With --backward, one step is one backward (gradients of qk and v for a seeded
dout, at the permutation of one forward of the same inputs), with the same
line layout: tokens/s of backwards, the dominant backward kernel's roofline,
and the oracle's backward on a bounded sample.

With --ffn, one step is the chunked feed-forward half of the reversible block
over the workload's B * L rows (d_model = H * d, d_ff = 4 d_model, chunks of
--ffn-chunk rows), with its two matrix-core layers' roofline.
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
METRIC_BWD = "LSH-attn bwd tokens/sec at L=64K, 4 rounds; % MFMA / HBM roofline"


def metric_name(w, direction: str) -> str:
    """The headline metric for the 64K-token, 4-round workload; the same
    metric at the other workloads' length and round count."""
    if w.seq_len == 65536 and w.n_rounds == 4:
        return METRIC if direction == "fwd" else METRIC_BWD
    L = f"{w.seq_len // 1024}K" if w.seq_len % 1024 == 0 else str(w.seq_len)
    return f"LSH-attn {direction} tokens/sec at L={L}, {w.n_rounds} rounds; % MFMA / HBM roofline"
METRIC_FFN = "chunked feed-forward tokens/sec at L=64K; % MFMA roofline"

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


def algorithmic_units(w, out_dtype: str, round_bytes: int = 2, stats=None, window_chunks=2,
                      model_dim=None):
    """Per-launch algorithmic work of each stage (what the method must compute
    or move, not what an implementation happens to move).
    N = B*H*L token-heads, R rounds, d head dim, nb buckets, m chunk length;
    round_bytes = bytes per element of the per-round outputs kept between the
    attention and the combine (2 for fp16, 4 with the fp32 option); stats =
    the re-scoring counts of the forward (rows re-scored on two columns, rows
    re-scored on all columns)."""
    N = w.batch * w.heads * w.seq_len
    R, d, nb, m = w.n_rounds, w.head_dim, w.n_buckets, w.chunk_len
    e, eo, ro = esize(w.dtype), esize(out_dtype), round_bytes
    half = max(nb // 2, 1)
    n_a = (stats or {}).get("n_exact_rescored", 0)
    n_b = (stats or {}).get("n_full_fallback", 0)
    return {
        # qk read for the two norm bounds of its fp16 form and the key norms;
        # rotation copies (fp16, fp32)
        "hash_prep": {"bytes": N * d * e + N * 12 + R * d * half * (4 + 2 + 4)},
        # projection x.R for every token-head and round: nb/2 MACs of length d;
        # reads the rows (converted to fp16 in registers) and norm bounds once,
        # writes the bucket ids
        "hash": {"flops": N * R * d * nb, "bytes": N * d * e + N * 8 + N * R * 2},
        # exact fp64 dot products of the re-scored rows
        "hash_rescore": {"flops64": 2 * d * (2 * n_a + half * n_b),
                         "bytes": (n_a + n_b) * d * e + 2 * n_a * d * 4},
        # read bucket ids twice (count, scatter), write the permutation
        "sort": {"bytes": N * R * (2 + 2 + 4)},
        # read two rows, write two rows per (round, slot), plus the perm read
        "gather": {"bytes": N * R * (4 * d * e + 4)},
        # QK^T and PV over the 2m-key window of every query-round; rows read
        # through the permutation, per-round output row and lse written
        "attend": {"flops": N * R * 4 * d * window_chunks * m,
                   "bytes": N * R * (2 * d * e + 4 + d * ro + 4)},
        # R per-round rows and lse read, one output row written
        "combine": {"bytes": N * R * (d * ro + 4) + N * d * eo},
        # forward from x: x [B*L, K] times the two weights [H*d, K]; x and the
        # weights read once, qk and v written, with the hash's norm bounds
        # and the key norms of qk (K = model_dim)
        "project": {"flops": 2 * w.batch * w.seq_len * (model_dim or 0) * 2 * w.heads * d,
                    "bytes": w.batch * w.seq_len * (model_dim or 0) * e
                    + 2 * w.heads * d * (model_dim or 0) * e + 2 * N * d * e + N * 12},
    }


def backward_units(w, out_dtype: str, grad_row_bytes: int = 2, window_chunks: int = 2,
                   split_rows: bool = False):
    """Per-launch algorithmic work of each backward stage (matrix-core path:
    bf16 inputs, per-round gradient rows of grad_row_bytes per element: fp16
    by default, fp32 with --fp32-round-outputs). N token-heads, R rounds, d, m
    as above; a round's window is window_chunks * m keys per query (3 with the
    look-ahead reading). Rows are read through the permutation once per
    (round, slot); the per-round gradients are rows at original positions.
    split_rows: the look-ahead and de-duplicated readings' products write dq
    and dkhat as separate fp32 rows (three per round, not two), which the
    reduction reads back with the round's lse and weight."""
    N = w.batch * w.heads * w.seq_len
    R, d, m = w.n_rounds, w.head_dim, w.chunk_len
    e, eo, g = esize(w.dtype), esize(out_dtype), grad_row_bytes
    nrows = 3 if split_rows else 2
    return {
        # attention at the permutation (as the forward's) with dout read per
        # query-round; per query-round lse and dout . o_r written; key norms
        "recompute": {"flops": N * R * 4 * d * window_chunks * m,
                      "bytes": N * R * (3 * d * e + 4 + 4 + 4) + N * (d * e + 4)},
        # lse and dout . o_r read and the round weight written per round; dout . out
        # and the self-only weight written per token-head
        "rows": {"bytes": N * R * (4 + 4 + 4) + N * (4 + 4)},
        # per (round, slot), over the window of each query: S, dP once, then
        # dQ, dkhat and dv; qk, v, dout rows, perm, lse, weight, dout . out and
        # key norm read once; the per-round gradient rows written
        "products": {"flops": N * R * 5 * 2 * d * window_chunks * m,
                     "bytes": N * R * (3 * d * e + 5 * 4 + nrows * d * g)},
        # R rounds of gradient rows (and, split, lse and weight) read; dqk and
        # dv written (dout is read only for rows with a self-only round)
        "reduce": {"bytes": N * R * (nrows * d * g + (8 if split_rows else 0)) + N * 4
                   + N * 2 * d * eo},
    }


# The matrix-core peak each stage's contraction runs at (fp16 projection,
# bf16 attention); HBM for the rest; fp64 vector for the exact re-scoring.
MFMA_PEAK = {"hash": "mfma_fp16_TFLOPs", "attend": "mfma_bf16_TFLOPs", "project": "mfma_bf16_TFLOPs",
             "recompute": "mfma_bf16_TFLOPs", "products": "mfma_bf16_TFLOPs",
             "ffn_up": "mfma_bf16_TFLOPs", "ffn_down": "mfma_bf16_TFLOPs"}


def stage_bound(stage: str, u: dict):
    """The resource that bounds a stage at its algorithmic work: the larger of
    flops / matrix peak and bytes / HBM peak."""
    if "flops64" in u:
        return "alu", "fp64_vector_TFLOPs"
    if "flops" in u:
        t_f = u["flops"] / (PEAK[MFMA_PEAK[stage]] * 1e12)
        t_b = u["bytes"] / (PEAK["hbm_GBps"] * 1e9)
        if t_f >= t_b:
            return "mfma", MFMA_PEAK[stage]
    return "hbm", "hbm_GBps"


def roofline(stage: str, units: dict, ms: float, traffic=None):
    u = units[stage]
    bound, peak_key = stage_bound(stage, u)
    if peak_key == "hbm_GBps":
        achieved = u["bytes"] / (ms * 1e-3) / 1e9
        unit = "GB/s"
    elif peak_key == "fp64_vector_TFLOPs":
        achieved = u["flops64"] / (ms * 1e-3) / 1e12
        unit = "TFLOP/s"
    else:
        achieved = u["flops"] / (ms * 1e-3) / 1e12
        unit = "TFLOP/s"
    peak = PEAK[peak_key]
    kernels = {**STAGE_KERNEL, **BWD_STAGE_KERNEL, **FFN_STAGE_KERNEL}
    return {"kernel": kernels.get(stage, stage),
            "stage": stage, "bound": bound,
            "achieved": round(achieved, 3), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 5), "traffic": traffic,
            "algorithmic_bytes": u.get("bytes"),
            "algorithmic_flops": u.get("flops", u.get("flops64"))}


def both_fractions(stage: str, units: dict, ms: float):
    """A stage's algorithmic bytes against the HBM peak and, where it has a
    matrix-core contraction, its flops against that matrix peak."""
    u = units[stage]
    out = {}
    if u.get("bytes"):
        out["hbm_frac"] = round(u["bytes"] / (ms * 1e-3) / 1e9 / PEAK["hbm_GBps"], 5)
    if u.get("flops") and stage in MFMA_PEAK:
        out["mfma_frac"] = round(u["flops"] / (ms * 1e-3) / 1e12 / PEAK[MFMA_PEAK[stage]], 5)
    return out


# Stages that are exactly one kernel launch (name as rocprofv3 reports it),
# and the source files each stage's kernels are built from.
STAGE_KERNEL = {"hash": "k_hash_mfma", "attend": "k_attend_mfma", "combine": "k_combine",
                "project": "k_proj"}  # k_proj_pp (d = 128, even heads) or k_proj_mfma
FFN_STAGE_KERNEL = {"ffn_up": "k_ffn_mfma<true, 256>", "ffn_down": "k_ffn_mfma<false, 256>"}
BWD_STAGE_KERNEL = {"rows": "k_bwd_rows_dot", "products": "k_bwd_fused_mfma",
                    "reduce": "k_bwd_reduce_sum"}
STAGE_SOURCES = {
    "hash_prep": ["hash_mfma.hip", "hash_x16.h"], "hash": ["hash_mfma.hip", "hash.hip", "hash_x16.h"],
    "hash_rescore": ["hash_mfma.hip"], "sort": ["sort.hip"], "gather": ["gather.hip"],
    "attend": ["attend_mfma.hip", "attend.hip"], "combine": ["combine.hip"],
    "project": ["project.hip", "hash_x16.h", "gemm_core.h"],
    "recompute": ["attend_mfma.hip", "backward.hip"], "rows": ["backward.hip"],
    "products": ["backward_mfma.hip", "rows_lds.h"], "reduce": ["backward.hip"],
    "ffn_up": ["ffn.hip", "gemm_core.h"], "ffn_down": ["ffn.hip", "gemm_core.h"],
}


def _oracle_threads():
    threads = len(os.sched_getaffinity(0))
    env_threads = os.environ.get("OMP_NUM_THREADS")
    if env_threads:
        threads = min(threads, int(env_threads))
    return threads


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def cpu_sample(w, pairs: int):
    """The first `pairs` (batch, head) pairs in batch-major order, as whole
    batches when pairs >= heads (pairs rounded down to a multiple of heads),
    else the first heads of batch 0: (batches, heads) of the sample."""
    if pairs >= w.heads:
        return min(w.batch, pairs // w.heads), w.heads
    return 1, max(1, pairs)


def cpu_baseline(w, inp, target_s: float = 10.0, pairs: int = 0):
    """The fp64 oracle as it stands, timed on a bounded sample of the workload
    (whole (batch, head) pairs at full sequence length, all rounds): a pilot
    on one pair sizes the sample to about target_s seconds (or `pairs` pairs),
    repeated when even the whole workload takes less; scaled to tokens/s.
    Returns (the record, the oracle's result on the sample, (batches, heads))."""
    import numpy as np

    import oracle

    threads = _oracle_threads()
    rot = None if inp.rotations is None else inp.rotations.astype(np.float64)
    oracle.build(force=False)

    def run(nb, nh):
        c = oracle.config(w.with_(batch=nb, heads=nh))
        qk = np.ascontiguousarray(inp.qk[:nb, :nh], dtype=np.float64)
        v = np.ascontiguousarray(inp.v[:nb, :nh], dtype=np.float64)
        t0 = time.perf_counter()
        ref = oracle.forward(c, qk, v, rot)
        return time.perf_counter() - t0, ref

    all_pairs = w.batch * w.heads
    if pairs:
        nb, nh = cpu_sample(w, pairs)
        t, ref = run(nb, nh)
    else:
        # grow the sample (the oracle runs its segments in parallel, so the
        # time is not proportional to the pairs) until it takes a third of
        # the target or is the whole workload; it starts with enough pairs
        # for a segment per thread
        pairs, t1 = min(all_pairs, max(1, -(-threads // w.n_rounds))), 0.0
        while True:
            nb, nh = cpu_sample(w, pairs)
            t, ref = run(nb, nh)
            t1 = t1 or t
            if t >= target_s / 3 or nb * nh == all_pairs:
                break
            pairs = min(all_pairs, max(pairs + 1, int(pairs * target_s / max(t, 1e-3))))
    n_pairs = nb * nh
    repeats = 1
    if n_pairs == all_pairs and t < target_s / 3:
        repeats = max(1, min(100, int(target_s / max(t, 1e-6))))
        t = 0.0
        for _ in range(repeats):
            dt, ref = run(nb, nh)
            t += dt
    frac = n_pairs / all_pairs
    value = w.batch * w.seq_len * frac * repeats / t
    used = min(threads, n_pairs * w.n_rounds)
    return {"value": round(value, 3), "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": f"{nb} batch(es) x {nh} head(s) of {w.batch} x {w.heads}, full "
                      f"L={w.seq_len}, all {w.n_rounds} rounds ({frac:.4f} of the workload)"
                      + (f", {repeats} times" if repeats > 1 else "")
                      + f": fp64 oracle forward in {t:.2f} s (sample grown from one (batch, "
                      f"head) pair per {w.n_rounds} threads, a segment per thread, towards "
                      f"{target_s:.0f} s); OpenMP over (batch, head, round) segments",
            "seconds": round(t, 3), "cpu_model": _cpu_model(), "threads_available": threads}, \
        ref, (nb, nh)


def parity_summary(w, inp, gpu, ref, sample):
    """What the timed configuration's results are, against the oracle: bucket
    ids of every head and round against the oracle's hash (mismatches and
    near-ties, oracle top-two margin < 1e-5), and the outputs and logsumexps
    of the cpu_baseline sample (its first `sample` = (batches, heads)) against
    the oracle's forward on them. gpu: out [B,H,L,d], lse [B,H,R,L], buckets
    [B,H,R,L] (numpy)."""
    nb, heads = sample
    import numpy as np

    import oracle

    res = {}
    if w.n_buckets > 1:
        t0 = time.perf_counter()
        bk, mg = oracle.hash(oracle.config(w), inp.qk, inp.rotations)
        res["bucket_ids_compared"] = int(bk.size)
        res["bucket_mismatches"] = int(np.sum(bk != gpu["buckets"]))
        res["near_ties"] = int(np.sum(mg < 1e-5))
        res["near_tie_mismatches"] = int(np.sum((bk != gpu["buckets"]) & (mg < 1e-5)))
        res["oracle_hash_s"] = round(time.perf_counter() - t0, 2)
    out = gpu["out"][:nb, :heads].astype(np.float64)
    res["out_rows_compared"] = int(nb * heads * w.seq_len)
    res["out_max_abs_err"] = float(np.abs(out - ref["out"]).max())
    lg = gpu["lse"][:nb, :heads].astype(np.float64)
    keep = ref["lse"] != oracle.SELF_LOGIT
    res["lse_max_abs_err"] = float(np.abs(lg - ref["lse"])[keep].max()) if keep.any() else 0.0
    res["self_only_flags_equal"] = bool(np.array_equal(lg == oracle.SELF_LOGIT, ~keep))
    res["perm_equal_sample"] = bool(np.array_equal(gpu["perm"][:nb, :heads], ref["perm"]))
    res["out_tolerance"] = 2e-2 if w.dtype == "bf16" else 1e-5
    return res


def settle(step, ms: float):
    """Run forwards for at least `ms` milliseconds of wall time before the
    warm-up steps: the first tens of milliseconds of sustained work run at
    lower clocks (measured: 20 timed forwards after 5 warm-ups take ~7% longer
    than after ~100 ms of work). Returns the record the JSON line declares."""
    import torch
    if ms <= 0:
        return {"forwards": 0, "ms": 0.0}
    n = 0
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            step()
        n += 8
        torch.cuda.synchronize()
    return {"forwards": n, "ms": round((time.perf_counter() - t0) * 1e3, 1),
            "why": "untimed forwards before the warm-up steps so that the timed ones run at "
                   "the clocks of sustained work, not the ramp at the start of the process"}


def calibration_copy(mib: int, dev):
    """After the timed region: copy `mib` MiB device to device three times (the
    reference dispatch for scaling FETCH_SIZE / WRITE_SIZE)."""
    if mib <= 0:
        return
    import torch
    src = torch.empty(mib << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def cpu_baseline_backward(w, inp, heads: int):
    """The fp64 oracle's backward as it stands, on batch 0 and the first
    `heads` heads at full sequence length, all rounds, at the oracle forward's
    permutation (not timed); scaled to tokens/s of the whole workload."""
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
    dout = np.random.default_rng(5).standard_normal(qk.shape)
    oracle.build(force=False)
    perm = oracle.forward(c, qk, v, rot)["perm"]
    t0 = time.perf_counter()
    oracle.backward(c, qk, v, perm, dout)
    t = time.perf_counter() - t0
    frac = heads / (w.batch * w.heads)
    return {"value": round(w.batch * w.seq_len * frac / t, 3), "unit": "tokens/s",
            "cores": min(threads, heads), "kind": "oracle",
            "sample": f"batch 0, heads 0..{heads - 1} of {w.heads}, full L={w.seq_len}, "
                      f"all {w.n_rounds} rounds ({frac:.4f} of the workload), fp64 oracle "
                      f"backward in {t:.2f} s (its forward's permutation made first, not "
                      f"timed); OpenMP over (batch, head)",
            "seconds": round(t, 3), "threads_available": threads}


def main_backward(args, w, inp, op_kw, variants=()):
    """The --backward line (see the module docstring); with --variants, the
    backward of those readings (the same-bucket mask takes the forward's
    bucket ids)."""
    import numpy as np
    import torch

    import lsh_attention_hash_amd as lat

    dev = torch.device("cuda", 0)
    tdt = {"bf16": torch.bfloat16, "fp32": torch.float32}
    if w.dtype == "bf16":
        qk = torch.from_numpy(inp.qk_bits.view(np.int16)).to(dev).view(torch.bfloat16)
        v = torch.from_numpy(inp.v_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        qk = torch.from_numpy(inp.qk).to(dev)
        v = torch.from_numpy(inp.v).to(dev)
    rot = None if inp.rotations is None else torch.from_numpy(inp.rotations).to(dev)
    op = lat.LSHAttention(w.batch, w.heads, w.seq_len, w.head_dim, w.n_buckets, w.n_rounds,
                          w.chunk_len, w.causal, dtype=tdt[w.dtype], backward=True, **op_kw,
                          **{x: True for x in variants})
    sb = "same_bucket" in variants
    _, ex = op(qk, v, rot, return_perm=True, return_buckets=sb)
    perm = ex["perm"]
    bk = ex["buckets"] if sb else None
    g = torch.Generator(device="cpu").manual_seed(5)
    dout = torch.randn((w.batch, w.heads, w.seq_len, w.head_dim), generator=g).to(
        tdt[w.dtype]).to(dev)
    dqk = torch.empty_like(qk)
    dv = torch.empty_like(v)
    stream = torch.cuda.current_stream()
    settled = settle(lambda: op.backward(qk, v, perm, dout, dqk, dv, buckets=bk), args.settle_ms)
    for _ in range(args.warmup):
        op.backward(qk, v, perm, dout, dqk, dv, buckets=bk)
    torch.cuda.synchronize()
    op.set_timing(args.steps)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        op.backward(qk, v, perm, dout, dqk, dv, buckets=bk)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end) / args.steps
    stage_ms, n_timed = op.get_backward_timing()
    stage_avg = {k: v_ / max(n_timed, 1) for k, v_ in stage_ms.items()}
    op.close()
    calibration_copy(args.calib_copy_mib, dev)

    # the look-ahead and de-duplicated readings: their own recomputation form
    # and product kernels, fp32 per-round rows of dq, dkhat and dv
    split = bool(set(variants) & {"look_ahead", "dedup"})
    units = backward_units(w, w.dtype, 4 if (args.fp32_round_outputs or split) else 2,
                           3 if "look_ahead" in variants else 2, split)
    single = {k: v_ for k, v_ in stage_avg.items() if k in BWD_STAGE_KERNEL}
    dominant = max(single, key=single.get)
    traffic = None
    if os.path.exists(args.traffic_json) and not variants:
        try:
            with open(args.traffic_json) as f:
                entry = json.load(f).get(args.workload + ":backward", {}).get(dominant)
            if entry and entry.get("source_hash") == kernel_source_hash(dominant):
                traffic = entry.get("bytes_per_launch")
        except (OSError, ValueError):
            traffic = None
    rl = roofline(dominant, units, stage_avg[dominant], traffic)
    if split and dominant == "products":
        rl["kernel"] = "k_bwd_var_dq + k_bwd_var_dkv"
    elif split and dominant == "reduce":
        rl["kernel"] = "k_bwd_reduce"
    per_stage = {}
    for k, t in stage_avg.items():
        per_stage[k] = {"ms": round(t, 5)}
        if t > 0:
            r = roofline(k, units, t)
            per_stage[k].update({"achieved": r["achieved"], "unit": r["unit"],
                                 "frac": r["frac"], "bound": r["bound"]})
            per_stage[k].update(both_fractions(k, units, t))
    tokens = w.batch * w.seq_len
    res = {
        "metric": metric_name(w, "bwd"),
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
        "config": {"workload": w.name, "pass": "backward", "batch": w.batch, "heads": w.heads,
                   "seq_len": w.seq_len, "head_dim": w.head_dim, "n_buckets": w.n_buckets,
                   "n_rounds": w.n_rounds, "chunk_len": w.chunk_len, "causal": w.causal,
                   "qk_v_dtype": w.dtype,
                   "inputs": f"{w.kind} seeded (qk {1000 + w.seed_base}, v {2000 + w.seed_base},"
                             f" R {3000 + w.seed_base}); dout torch seed 5, standard normal",
                   "per_round_gradients": "fp32" if (args.fp32_round_outputs or split) else "fp16",
                   "variants": list(variants)},
        "roofline": rl,
        "stages": per_stage,
        "settle": settled,
        "wall_s_timed": round(wall, 4),
    }
    if not args.no_cpu_baseline and not variants:
        heads = args.cpu_heads or max(1, min(w.heads, len(os.sched_getaffinity(0)) // 4))
        res["cpu_baseline"] = cpu_baseline_backward(w, inp, heads)
    print(json.dumps(res), flush=True)


def ffn_units(rows: int, d_model: int, d_ff: int, es: int):
    """Algorithmic work of each feed-forward layer over `rows` rows: 2 rows
    d_model d_ff flops, and the bytes each reads and writes once (its input
    rows, weight, bias, output rows; the second layer also the residual)."""
    flops = 2.0 * rows * d_model * d_ff
    return {"ffn_up": {"flops": flops,
                       "bytes": es * (rows * d_model + d_ff * d_model + d_ff + rows * d_ff)},
            "ffn_down": {"flops": flops,
                         "bytes": es * (rows * d_ff + d_model * d_ff + d_model
                                        + 2 * rows * d_model)}}


def cpu_baseline_ffn(fi, n_rows: int):
    """The fp64 oracle's feed-forward as it stands on the first n_rows rows
    (one chunk), scaled to rows/s."""
    import oracle

    threads = len(os.sched_getaffinity(0))
    env_threads = os.environ.get("OMP_NUM_THREADS")
    if env_threads:
        threads = min(threads, int(env_threads))
    oracle.build(force=False)
    t0 = time.perf_counter()
    oracle.ffn(fi.y1[:n_rows], fi.w1, fi.b1, fi.w2, fi.b2, x2=fi.x2[:n_rows])
    t = time.perf_counter() - t0
    return {"value": round(n_rows / t, 3), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"the first {n_rows} of {fi.rows} rows (d_model {fi.d_model}, d_ff "
                      f"{fi.d_ff}, with the residual) through the fp64 oracle's feed-forward "
                      f"in {t:.2f} s; OpenMP over rows",
            "seconds": round(t, 3), "threads_available": threads}


def main_ffn(args, w):
    """The --ffn line (see the module docstring)."""
    import numpy as np
    import torch

    import lsh_attention_hash_amd as lat
    import workloads

    dev = torch.device("cuda", 0)
    rows, d_model = w.batch * w.seq_len, w.heads * w.head_dim
    d_ff = 4 * d_model
    fi = workloads.make_ffn_inputs(rows, d_model, d_ff, w.dtype)
    tdt = {"bf16": torch.bfloat16, "fp32": torch.float32}[w.dtype]
    if w.dtype == "bf16":
        t = {k: torch.from_numpy(b.view(np.int16)).to(dev).view(torch.bfloat16)
             for k, b in fi.bits.items()}
    else:
        t = {k: torch.from_numpy(getattr(fi, k)).to(dev) for k in fi.bits}
    op = lat.ChunkedFeedForward(rows, d_model, d_ff, args.ffn_chunk, dtype=tdt)
    y2 = torch.empty((rows, d_model), dtype=tdt, device=dev)
    call = lambda: op(t["y1"], t["w1"], t["b1"], t["w2"], t["b2"], x2=t["x2"], out=y2)
    stream = torch.cuda.current_stream()
    settled = settle(call, args.settle_ms)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    op.set_timing(args.steps)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        call()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end) / args.steps
    stage_ms, n_timed, n_chunks = op.get_timing()
    ws_bytes = op.workspace_bytes()
    op.close()
    calibration_copy(args.calib_copy_mib, dev)

    chunk = min(args.ffn_chunk or rows, rows)
    per_call = n_chunks / max(n_timed, 1)
    # per launch: one chunk's rows (the last chunk may be shorter: averaged)
    units = ffn_units(rows / per_call, d_model, d_ff, esize(w.dtype))
    stage_avg = {k: v_ / max(n_chunks, 1) for k, v_ in stage_ms.items()}  # ms per launch
    dominant = max(stage_avg, key=stage_avg.get)
    traffic = None
    if os.path.exists(args.traffic_json):
        try:
            with open(args.traffic_json) as f:
                entry = json.load(f).get(args.workload + ":ffn", {}).get(dominant)
            if entry and entry.get("source_hash") == kernel_source_hash(dominant):
                traffic = entry.get("bytes_per_launch")
        except (OSError, ValueError):
            traffic = None
    rl = roofline(dominant, units, stage_avg[dominant], traffic)
    per_stage = {}
    for k, t_ in stage_avg.items():
        r = roofline(k, units, t_)
        per_stage[k] = {"ms_per_launch": round(t_, 5), "launches_per_step": per_call,
                        "achieved": r["achieved"], "unit": r["unit"], "frac": r["frac"]}
    res = {
        "metric": METRIC_FFN,
        "value": round(rows / (ms * 1e-3), 1),
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
        "config": {"workload": w.name, "pass": "chunked feed-forward", "rows": rows,
                   "d_model": d_model, "d_ff": d_ff, "chunk_rows": chunk,
                   "hidden_buffer_bytes": ws_bytes, "residual": True,
                   "inputs": "seeded normal y1, x2; weights N(0, 1/fan_in); biases N(0, 0.01)"},
        "roofline": rl,
        "stages": per_stage,
        "settle": settled,
        "wall_s_timed": round(wall, 4),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_ffn(fi, args.ffn_cpu_rows)
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="text64k")
    ap.add_argument("--out-dtype", default=None, choices=[None, "bf16", "fp32"])
    ap.add_argument("--separate-gather", action="store_true")
    ap.add_argument("--fp32-round-outputs", action="store_true")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward instead of the forward (its own JSON line)")
    ap.add_argument("--from-x", action="store_true",
                    help="time the forward from a layer input x [B, L, H*d] with the shared-QK "
                         "and value projections (lsh_attn_forward_x); model_dim = H * d")
    ap.add_argument("--variants", default="",
                    help="comma list of variant readings for the forward (or, with "
                         "--backward, the backward): look_ahead, same_bucket, norm_queries, "
                         "dedup (default: none)")
    ap.add_argument("--ffn", action="store_true",
                    help="time the chunked feed-forward (d_model = H * d, d_ff = 4 d_model) "
                         "over the workload's B * L rows instead of the attention")
    ap.add_argument("--ffn-chunk", type=int, default=16384,
                    help="rows per feed-forward chunk (0: all rows at once)")
    ap.add_argument("--ffn-cpu-rows", type=int, default=32768,
                    help="rows in the oracle's feed-forward sample")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle's timing and the parity summary")
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="untimed forwards for this many milliseconds before the warm-up "
                         "steps (declared in the JSON line as 'settle')")
    ap.add_argument("--cpu-heads", type=int, default=0,
                    help="(batch, head) pairs in the oracle sample (0: sized to --cpu-seconds)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="oracle time the sample is sized to (a one-pair pilot estimates it)")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="HBM bytes per launch measured with rocprofv3 counters")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after the timed region, copy this many MiB device to device "
                         "(the reference kernel for scaling FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU work: read two rocprofv3 --pmc output folders (FETCH_SIZE, "
                         "WRITE_SIZE) of a run with --calib-copy-mib and write --traffic-json")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(args)
        return

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
    if args.ffn:
        torch.cuda.set_device(torch.device("cuda", 0))
        main_ffn(args, w)
        return
    out_dtype = args.out_dtype or w.dtype
    variants = [x for x in args.variants.split(",") if x]
    for x in variants:
        if x not in ("look_ahead", "same_bucket", "norm_queries", "dedup"):
            raise SystemExit(f"unknown variant {x!r}")
    inp = workloads.make_inputs(w)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.backward:
        main_backward(args, w, inp, {"separate_gather": args.separate_gather,
                                     "fp32_round_outputs": args.fp32_round_outputs}, variants)
        return
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
                          fp32_round_outputs=args.fp32_round_outputs,
                          **{x: True for x in variants})
    out = torch.empty((w.batch, w.heads, w.seq_len, w.head_dim), dtype=tdt[out_dtype],
                      device=dev)
    stream = torch.cuda.current_stream()
    model_dim = w.heads * w.head_dim
    if args.from_x:
        li = workloads.make_layer_inputs(w, model_dim)
        if w.dtype == "bf16":
            tens = lambda bits: torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
            x, wq, wv = tens(li.x_bits), tens(li.w_qk_bits), tens(li.w_v_bits)
        else:
            x, wq, wv = (torch.from_numpy(a).to(dev) for a in (li.x, li.w_qk, li.w_v))
        rot = None if li.rotations is None else torch.from_numpy(li.rotations).to(dev)
        step = lambda: op.forward_x(x, wq, wv, rot, qk=qk, v=v, out=out)
    else:
        step = lambda: op(qk, v, rot, out=out)

    settled = settle(step, args.settle_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    op.set_timing(args.steps)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end) / args.steps
    stage_ms, n_timed = op.get_timing()
    stage_avg = {k: v_ / max(n_timed, 1) for k, v_ in stage_ms.items()}
    stats = op.stats()

    calibration_copy(args.calib_copy_mib, dev)

    fp16_rounds = w.dtype == "bf16" and w.chunk_len == 64 and not args.fp32_round_outputs
    units = algorithmic_units(w, out_dtype, 2 if fp16_rounds else 4, stats,
                              3 if "look_ahead" in variants else 2, model_dim)
    if not args.from_x:
        stage_avg.pop("project")  # no projection in the forward from qk and v
    if not args.separate_gather:
        stage_avg.pop("gather")   # rows are read through the permutation inside attend
    # the dominant kernel: the slowest stage that is one kernel launch
    single = {k: v_ for k, v_ in stage_avg.items() if k in STAGE_KERNEL}
    dominant = max(single, key=single.get)
    traffic = None
    if os.path.exists(args.traffic_json) and not variants:
        try:
            with open(args.traffic_json) as f:
                tj = json.load(f)
            entry = tj.get(args.workload, {}).get(dominant)
            if entry and entry.get("source_hash") == kernel_source_hash(dominant):
                traffic = entry.get("bytes_per_launch")
        except (OSError, ValueError):
            traffic = None
    rl = roofline(dominant, units, stage_avg[dominant], traffic)
    plain = w.dtype != "bf16" or w.chunk_len != 64 or w.head_dim not in (64, 128)
    if dominant == "attend" and plain:
        rl["kernel"] = "k_attend_simple"  # fp32 rows or other chunk lengths
    elif dominant == "hash" and (w.dtype != "bf16" or w.head_dim not in (64, 128)):
        rl["kernel"] = "k_hash_exact"
    elif variants and dominant == "attend" and set(variants) & {"look_ahead", "dedup"}:
        rl["kernel"] = "k_attend_var"  # the look-ahead and de-duplication readings' own kernel
    elif dominant == "project":
        rl["kernel"] = ("k_proj_pp" if w.head_dim == 128 and w.heads % 2 == 0 else
                        "k_proj_mfma")
    per_stage = {k: {"ms": round(stage_avg[k], 5)} for k in stage_avg}
    for k in per_stage:
        if stage_avg[k] > 0:
            r = roofline(k, units, stage_avg[k])
            per_stage[k].update({"achieved": r["achieved"], "unit": r["unit"],
                                 "frac": r["frac"], "bound": r["bound"]})
            per_stage[k].update(both_fractions(k, units, stage_avg[k]))

    tokens = w.batch * w.seq_len
    res = {
        "metric": metric_name(w, "fwd"),
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
                   "variants": variants,
                   "from_x": bool(args.from_x),
                   "model_dim": model_dim if args.from_x else None,
                   "round_outputs": "fp16" if fp16_rounds else "fp32"},
        "roofline": rl,
        "stages": per_stage,
        "token_heads_per_s": round(w.batch * w.heads * w.seq_len / (ms * 1e-3), 1),
        "hash_stats": stats,
        "settle": settled,
        "wall_s_timed": round(wall, 4),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"], ref, sample = cpu_baseline(w, inp, args.cpu_seconds, args.cpu_heads)
        if not args.from_x and not variants:
            # the results of the timed configuration: one more forward, untimed
            out, ex = op(qk, v, rot, out=out, return_lse=True, return_buckets=True,
                         return_perm=True)
            torch.cuda.synchronize()
            gpu = {"out": out.float().cpu().numpy(), "lse": ex["lse"].cpu().numpy(),
                   "buckets": ex["buckets"].cpu().numpy(), "perm": ex["perm"].cpu().numpy()}
            res["parity"] = parity_summary(w, inp, gpu, ref, sample)
    op.close()
    print(json.dumps(res), flush=True)


def kernel_source_hash(stage: str) -> str:
    """Hash of the source files of a stage's kernels, the shared headers and the
    build script (compiler flags); counter-derived traffic is only reported
    while they are unchanged."""
    import hashlib
    h = hashlib.sha256()
    for fname in STAGE_SOURCES[stage] + ["internal.h", "dtype.h"]:
        with open(os.path.join(ROOT, "lsh_attention_hash_amd", "csrc", fname), "rb") as f:
            h.update(f.read())
    with open(os.path.join(ROOT, "lsh_attention_hash_amd", "build.py"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def _pmc_dispatches(folder: str, counter: str):
    """(kernel name, value) of one counter for every dispatch in a rocprofv3
    --pmc output folder (csv)."""
    import csv
    import glob
    rows = []
    for path in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return rows


def write_traffic(args):
    """HBM bytes per launch of the single-kernel stages from FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), each scaled by what the same counter reads
    for the calibration copy of known size (--calib-copy-mib of the profiled
    run: each copy dispatch reads and writes exactly that many bytes)."""
    import statistics
    fetch = _pmc_dispatches(args.write_traffic[0], "FETCH_SIZE")
    write = _pmc_dispatches(args.write_traffic[1], "WRITE_SIZE")
    if args.calib_copy_mib <= 0:
        raise SystemExit("--write-traffic needs --calib-copy-mib of the profiled run")
    known_kib = float(args.calib_copy_mib * 1024)

    def calib(rows):
        # copy dispatches of the calibration size (other copies in the run are small)
        vals = [v for k, v in rows if "copy" in k.lower() and v >= known_kib / 8]
        if not vals:
            raise SystemExit("calibration copy dispatches not found in the counters")
        return "copy", known_kib / statistics.median(vals)

    def mean_of(rows, kname):
        vals = [v for k, v in rows if kname in k]
        return sum(vals) / len(vals) if vals else None

    cf_name, cf = calib(fetch)
    cw_name, cw = calib(write)
    out = {}
    if os.path.exists(args.traffic_json):
        with open(args.traffic_json) as f:
            out = json.load(f)
    key = args.workload + (":backward" if args.backward else ":ffn" if args.ffn else "")
    entry = out.setdefault(key, {})
    kernels = BWD_STAGE_KERNEL if args.backward else FFN_STAGE_KERNEL if args.ffn else STAGE_KERNEL
    for stage, kname in kernels.items():
        f_kib, w_kib = mean_of(fetch, kname), mean_of(write, kname)
        if f_kib is None or w_kib is None:
            continue
        entry[stage] = {
            "bytes_per_launch": round(f_kib * 1024 * cf + w_kib * 1024 * cw),
            "fetch_kib": round(f_kib, 1), "write_kib": round(w_kib, 1),
            "fetch_scale": round(cf, 4), "write_scale": round(cw, 4),
            "calibration": f"{args.calib_copy_mib} MiB device copy (__amd_rocclr_copyBuffer)",
            "source_hash": kernel_source_hash(stage),
        }
    with open(args.traffic_json, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
    print(json.dumps(entry, indent=1))


if __name__ == "__main__":
    main()
