"""The variant readings on the GPU (flags through the C ABI) against the fp64
oracle with the same variant, on the GPU's buckets: look-ahead window,
same-bucket mask, unit-normalised queries, de-duplicated union over rounds,
alone and combined. Buckets and permutations are unaffected by the variants
and are checked as in the default reading. Each case prints what it is first.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
import lsh_attention_hash_amd as lat
from parity import (OUT_TOL, _cmp_lse, check_buckets, lse_tol, out_tol, sample_rows,
                    scaled_inputs, to_device)

pytestmark = pytest.mark.gpu

LA, SB, NQ, DD = oracle.LOOK_AHEAD, oracle.SAME_BUCKET, oracle.NORM_QUERIES, oracle.DEDUP
ALL = LA | SB | NQ | DD


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lat.load_library()


def W(name, **kw):
    return workloads.get(name).with_(**kw)


def _kw(variant):
    return {"look_ahead": bool(variant & LA), "same_bucket": bool(variant & SB),
            "norm_queries": bool(variant & NQ), "dedup": bool(variant & DD)}


def _name(variant):
    parts = [n for b, n in ((LA, "la"), (SB, "sb"), (NQ, "nq"), (DD, "dd")) if variant & b]
    return "+".join(parts) or "default"


def _run(w, variant, inp=None):
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    if inp is None:
        inp = workloads.make_inputs(w)
    qk, v, rot = to_device(inp)
    op = lat.LSHAttention(w.batch, w.heads, w.seq_len, w.head_dim, w.n_buckets, w.n_rounds,
                          w.chunk_len, w.causal, dtype=dt, **_kw(variant))
    try:
        out, ex = op(qk, v, rot, return_lse=True, return_buckets=True, return_perm=True)
        torch.cuda.synchronize()
        res = {"out": out.float().cpu().numpy().astype(np.float64),
               "lse": ex["lse"].cpu().numpy(), "buckets": ex["buckets"].cpu().numpy(),
               "perm": ex["perm"].cpu().numpy()}
    finally:
        op.close()
    return inp, res


CASES = [
    (W("tiny"), LA), (W("tiny"), SB), (W("tiny"), NQ), (W("tiny"), DD),
    (W("tiny", n_rounds=3, causal=True), ALL),
    (W("c4k", batch=1, heads=2, seq_len=1024, n_buckets=16, n_rounds=2), LA),
    (W("c4k", batch=1, heads=2, seq_len=1024, n_buckets=16, n_rounds=2), SB),
    (W("c4k", batch=1, heads=2, seq_len=1024, n_buckets=16, n_rounds=2), NQ),
    (W("c4k", batch=1, heads=2, seq_len=1024, n_buckets=16, n_rounds=3), DD),
    (W("text64k", batch=1, heads=1, seq_len=2048, n_buckets=32, n_rounds=4), ALL),
    (W("text64k", batch=1, heads=1, seq_len=2048, n_buckets=32, n_rounds=4, causal=False),
     LA | DD),
    (W("skewed", batch=1, heads=2, seq_len=2048, n_buckets=32, n_rounds=3), SB | DD),
    # plain kernel at its limits: the largest window (3 chunks of 256) and a
    # chunk length that leaves partial query and key blocks
    (W("tiny", chunk_len=256, n_rounds=2), LA),
    (W("tiny", seq_len=1200, head_dim=128, chunk_len=40, n_rounds=2, causal=True), ALL),
]


@pytest.mark.parametrize("w,variant", CASES,
                         ids=[f"{w.name}-{w.dtype}-L{w.seq_len}d{w.head_dim}R{w.n_rounds}"
                              f"{'c' if w.causal else 'n'}-{_name(v)}" for w, v in CASES])
def test_variant_parity(w, variant):
    _say(f"[variant {_name(variant)}] {w}")
    inp, gpu = _run(w, variant)
    check_buckets(w, inp, gpu["buckets"])
    c = oracle.config(w, variant=variant)
    ref = oracle.forward(c, inp.qk, inp.v, inp.rotations, buckets_override=gpu["buckets"])
    np.testing.assert_array_equal(ref["perm"], gpu["perm"])
    err = np.abs(gpu["out"] - ref["out"])
    _say(f"  out max err {err.max():.3g}")
    assert err.max() <= OUT_TOL[w.dtype], f"out max err {err.max()}"
    _cmp_lse(w, gpu["lse"], ref["lse"], lse_tol(w, inp.qk))


SCALED = [
    # qk x 2^7: the Cauchy-Schwarz shift exceeds the kernel's limit, so the
    # variant kernel takes the true row maximum (unit queries keep it small)
    (W("text64k", batch=1, heads=1, seq_len=2048, n_buckets=32, n_rounds=4), LA | SB | DD),
    (W("c4k", batch=1, heads=2, seq_len=1024, n_buckets=16, n_rounds=3, causal=False), LA | DD),
    (W("c4k", batch=1, heads=2, seq_len=1024, n_buckets=16, n_rounds=2), NQ),
]


@pytest.mark.parametrize("w,variant", SCALED,
                         ids=[f"{w.name}-L{w.seq_len}d{w.head_dim}R{w.n_rounds}"
                              f"{'c' if w.causal else 'n'}-{_name(v)}-qk2^7" for w, v in SCALED])
def test_variant_parity_large_qk(w, variant):
    inp = scaled_inputs(workloads.make_inputs(w), 7, 0)
    _say(f"[variant {_name(variant)}, qk x 2^7] {w}")
    inp, gpu = _run(w, variant, inp)
    check_buckets(w, inp, gpu["buckets"])
    c = oracle.config(w, variant=variant)
    ref = oracle.forward(c, inp.qk, inp.v, inp.rotations, buckets_override=gpu["buckets"])
    np.testing.assert_array_equal(ref["perm"], gpu["perm"])
    err = np.abs(gpu["out"] - ref["out"])
    tol = out_tol(w, inp, scaled_qk=True)
    _say(f"  out max err {err.max():.3g} (bound {tol:.3g})")
    assert err.max() <= tol
    _cmp_lse(w, gpu["lse"], ref["lse"], lse_tol(w, inp.qk))


def test_variants_full_size_sampled_rows():
    """Text-64K at full size with every variant on: every bucket id against
    the oracle's hash, and 256 sampled rows of every head (the chunk ends
    among them) against the oracle's variant attention."""
    w = workloads.get("text64k")
    _say(f"[variant all, full size] {w}")
    inp, gpu = _run(w, ALL)
    n, ties, _ = check_buckets(w, inp, gpu["buckets"])
    rows = sample_rows(w, per_head=256, seed=7)
    N = w.batch * w.heads * w.seq_len
    c = oracle.config(w, variant=ALL)
    out_r, lse_r = oracle.attend_rows(c, inp.qk, inp.v, gpu["perm"], rows, gpu["buckets"])
    err = np.abs(gpu["out"].reshape(N, w.head_dim)[rows] - out_r)
    _say(f"  buckets {n} ties {ties} rows {rows.size} out max err {err.max():.3g}")
    assert err.max() <= OUT_TOL[w.dtype]
    bh, i = rows // w.seq_len, rows % w.seq_len
    tol = lse_tol(w, inp.qk).reshape(w.batch * w.heads, w.seq_len)[bh, i][:, None]
    _cmp_lse(w, gpu["lse"].reshape(w.batch * w.heads, w.n_rounds, w.seq_len)[bh, :, i], lse_r,
             tol)


