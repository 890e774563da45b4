"""Backward (dqk, dv) of the HIP path vs the fp64 oracle's backward, through
the C ABI, at the GPU forward's permutations. Inputs are seeded; dout is drawn
from its own seed and rounded to the input dtype, and the oracle takes the
exact values the GPU sees. Each case prints what it is before it runs.

Tolerance: the gradients come back in the input dtype. For bf16 that
rounding alone is up to 2^-8 of each value (the unit roundoff of an 8-bit
significand); the rest (fp32 sums, the recomputed attention's bf16 products,
and on the matrix-core path the per-round gradient rows held in fp16, 2^-11
of each row value, unless LSH_ATTN_FLAG_FP32_ROUND_OUTPUTS keeps them in fp32)
is bounded by a small fraction of the largest gradient. So
|g - g_ref| <= 2^-8 |g_ref| + 1e-2 max|g_ref| per element for bf16, and
1e-4 max|g_ref| for fp32.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
import lsh_attention_hash_amd as lat
from parity import to_device

pytestmark = pytest.mark.gpu


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


def _dout(w, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((w.batch, w.heads, w.seq_len, w.head_dim)).astype(np.float32)
    if w.dtype == "bf16":
        t = torch.from_numpy(x).to(torch.bfloat16)
        return t, t.to(torch.float64).numpy()
    t = torch.from_numpy(x)
    return t, x.astype(np.float64)


def _check(name, g, ref, bf16):
    err = np.abs(g - ref)
    scale = np.abs(ref).max()
    if bf16:
        bound = 2.0 ** -8 * np.abs(ref) + 1e-2 * scale
    else:
        bound = 1e-4 * scale + 0 * ref
    worst = float((err / np.maximum(bound, 1e-30)).max())
    _say(f"  {name}: max err {err.max():.3g} (max |ref| {scale:.3g}), worst err/bound {worst:.3g}")
    assert (err <= bound).all(), f"{name} outside tolerance"


BWD = [
    W("tiny"),
    W("c4k", batch=1, heads=2, seq_len=1024, n_buckets=16, n_rounds=2, causal=True),
    W("c4k", batch=1, heads=2, seq_len=1024, n_buckets=16, n_rounds=3, causal=False),
    W("text64k", batch=1, heads=2, seq_len=2048, n_buckets=32, n_rounds=4, causal=True),
    W("text64k", batch=1, heads=1, seq_len=1024, n_buckets=16, n_rounds=1, causal=False),
    W("skewed", batch=1, heads=2, seq_len=2048, n_buckets=32, n_rounds=2),
    W("c4k", batch=1, heads=1, seq_len=64, n_buckets=4, n_rounds=2, causal=True),  # one chunk
    # 20 chunks: a full range of 16 and a short last one
    W("text64k", batch=1, heads=2, seq_len=1280, n_buckets=16, n_rounds=3, causal=False),
    W("image12k", batch=2, heads=1, seq_len=3072, n_buckets=32, n_rounds=2),
    # a round count without a specialised reduction
    W("image12k", batch=1, heads=1, seq_len=1024, n_buckets=16, n_rounds=5),
]


@pytest.mark.parametrize("w", BWD, ids=lambda w: f"{w.name}-{w.dtype}-H{w.heads}L{w.seq_len}"
                         f"d{w.head_dim}nb{w.n_buckets}R{w.n_rounds}{'c' if w.causal else 'n'}")
def test_backward_parity(w, fp32_rows=False):
    _say(f"[backward] {w} fp32 round rows={fp32_rows}")
    inp = workloads.make_inputs(w)
    dev = torch.device("cuda", 0)
    qk, v, rot = to_device(inp, dev)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    op = lat.LSHAttention(w.batch, w.heads, w.seq_len, w.head_dim, w.n_buckets, w.n_rounds,
                          w.chunk_len, w.causal, dtype=dt, backward=True,
                          fp32_round_outputs=fp32_rows)
    try:
        _, ex = op(qk, v, rot, return_perm=True)
        dout_t, dout = _dout(w, 9000 + w.seq_len + w.n_rounds)
        dqk, dv = op.backward(qk, v, ex["perm"], dout_t.to(dev))
        torch.cuda.synchronize()
        perm = ex["perm"].cpu().numpy()
        dqk = dqk.to(torch.float64).cpu().numpy()
        dv = dv.to(torch.float64).cpu().numpy()
    finally:
        op.close()
    c = oracle.config(w)
    rq, rv = oracle.backward(c, inp.qk, inp.v, perm, dout)
    _check("dqk", dqk, rq, w.dtype == "bf16")
    _check("dv", dv, rv, w.dtype == "bf16")


def test_backward_needs_the_flag():
    w = W("c4k", batch=1, heads=1, seq_len=256, n_buckets=4, n_rounds=1, causal=True)
    inp = workloads.make_inputs(w)
    dev = torch.device("cuda", 0)
    qk, v, rot = to_device(inp, dev)
    op = lat.LSHAttention(w.batch, w.heads, w.seq_len, w.head_dim, w.n_buckets, w.n_rounds,
                          w.chunk_len, w.causal)
    try:
        _, ex = op(qk, v, rot, return_perm=True)
        with pytest.raises(lat.LSHAttnError) as e:
            op.backward(qk, v, ex["perm"], torch.zeros_like(qk))
        assert e.value.status == 2  # UNSUPPORTED
    finally:
        op.close()


def test_backward_deterministic():
    w = W("skewed", batch=1, heads=2, seq_len=2048, n_buckets=32, n_rounds=2)
    inp = workloads.make_inputs(w)
    dev = torch.device("cuda", 0)
    qk, v, rot = to_device(inp, dev)
    op = lat.LSHAttention(w.batch, w.heads, w.seq_len, w.head_dim, w.n_buckets, w.n_rounds,
                          w.chunk_len, w.causal, backward=True)
    try:
        _, ex = op(qk, v, rot, return_perm=True)
        dout = _dout(w, 77)[0].to(dev)
        a = op.backward(qk, v, ex["perm"], dout)
        b = op.backward(qk, v, ex["perm"], dout)
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    finally:
        op.close()


def test_backward_full_size_sampled_heads():
    """Text-64K at full size, in the bench's configuration; the oracle's
    backward is computed for two of the (batch, head) pairs (each pair's
    gradients depend only on its own rows) at the GPU forward's permutation."""
    w = workloads.get("text64k")
    _say(f"[backward full size] {w}")
    inp = workloads.make_inputs(w)
    dev = torch.device("cuda", 0)
    qk, v, rot = to_device(inp, dev)
    op = lat.LSHAttention(w.batch, w.heads, w.seq_len, w.head_dim, w.n_buckets, w.n_rounds,
                          w.chunk_len, w.causal, backward=True)
    try:
        _, ex = op(qk, v, rot, return_perm=True)
        dout_t, dout = _dout(w, 4242)
        dqk, dv = op.backward(qk, v, ex["perm"], dout_t.to(dev))
        torch.cuda.synchronize()
        perm = ex["perm"].cpu().numpy().reshape(w.batch, w.heads, w.n_rounds, w.seq_len)
        dqk = dqk.to(torch.float64).cpu().numpy()
        dv = dv.to(torch.float64).cpu().numpy()
    finally:
        op.close()
    heads = [0, w.heads - 1]
    sub = w.with_(batch=1, heads=len(heads))
    c = oracle.config(sub)
    rq, rv = oracle.backward(c, np.ascontiguousarray(inp.qk[:1, heads]),
                             np.ascontiguousarray(inp.v[:1, heads]),
                             np.ascontiguousarray(perm[:1, heads]),
                             np.ascontiguousarray(dout[:1, heads]))
    _check("dqk", dqk[:1, heads], rq, True)
    _check("dv", dv[:1, heads], rv, True)


@pytest.mark.parametrize("causal", [True, False])
def test_backward_parity_fp32_round_rows(causal):
    """The per-round gradient rows kept in fp32 (LSH_ATTN_FLAG_FP32_ROUND_OUTPUTS)
    instead of the default fp16: the same parity."""
    test_backward_parity(W("text64k", batch=1, heads=2, seq_len=2048, n_buckets=32, n_rounds=4,
                           causal=causal), fp32_rows=True)


def test_backward_gradient_rows_at_the_fp16_limit():
    """The per-round gradient rows are fp16 by default: with dout x 2^16 some
    pass +-65504, which the library counts (the rows are clamped there); with
    fp32 rows the same backward matches the oracle and counts nothing."""
    w = W("c4k", batch=1, heads=2, seq_len=1024, n_buckets=16, n_rounds=2, causal=True)
    _say(f"[backward fp16 limit] {w}")
    inp = workloads.make_inputs(w)
    dev = torch.device("cuda", 0)
    qk, v, rot = to_device(inp, dev)
    dout_t, dout = _dout(w, 31)
    dout_t = dout_t * 2.0 ** 16
    dout = dout * 2.0 ** 16
    res = {}
    for fp32_rows in (False, True):
        op = lat.LSHAttention(w.batch, w.heads, w.seq_len, w.head_dim, w.n_buckets, w.n_rounds,
                              w.chunk_len, w.causal, backward=True, fp32_round_outputs=fp32_rows)
        try:
            _, ex = op(qk, v, rot, return_perm=True)
            op.stats()  # restart the limit counters
            dqk, dv = op.backward(qk, v, ex["perm"], dout_t.to(dev))
            torch.cuda.synchronize()
            res[fp32_rows] = (ex["perm"].cpu().numpy(), dqk.to(torch.float64).cpu().numpy(),
                              dv.to(torch.float64).cpu().numpy(),
                              op.stats()["n_grad_rows_at_fp16_limit"])
        finally:
            op.close()
    _say(f"  fp16 rows: {res[False][3]} pieces at the limit; fp32 rows: {res[True][3]}")
    assert res[False][3] > 0 and res[True][3] == 0
    perm, dqk, dv, _ = res[True]
    rq, rv = oracle.backward(oracle.config(w), inp.qk, inp.v, perm, dout)
    _check("dqk", dqk, rq, True)
    _check("dv", dv, rv, True)
