"""Backward (dqk, dv) of the HIP path vs the fp64 oracle's backward, through
the C ABI, at the GPU forward's permutations. Inputs are seeded; dout is drawn
from its own seed and rounded to the input dtype, and the oracle takes the
exact values the GPU sees. Each case prints what it is before it runs.

Tolerance, derived from the arithmetic of the matrix-core backward (bf16
inputs). With u = 2^-8 the unit roundoff of bf16 and m the oracle's term
magnitudes (oracle.backward_magnitudes: per element, the sum over rounds and
window pairs of upper bounds of the absolute values of the terms, |dS| <= A
with A = wP (|dout.v| + |dout.out| + 2E)):
  * dv_j = sum_i bf16(wP_ij) dout_i in fp32: u per term (the rounding of wP),
    fp32 sums (<= 2m 2^-24 relative), the per-round row stored in fp16
    (2^-11 of its terms), the result rounded to bf16 (u |dv|):
        |dv - dv_ref| <= u |dv_ref| + (u + 2^-11 + 2^-14) m_dv;
  * dS = wP (dout.v - dout.out) rounded to bf16 (u |dS|), dout.out taken from
    the recomputed per-round rows, whose weights are bf16-rounded P normalised
    by their own sum (at most 2u relative, i.e. <= 2u E of dout.out, <= u A
    after the factor wP), then dq = sum_j dS k/(sqrt(d)|k|) and
    dkhat = sum_i dS q/sqrt(d) in fp32, the normalisation's Jacobian per
    round, fp16 rows and the bf16 result:
        |dqk - dqk_ref| <= u |dqk_ref| + (2u + 2^-11 + 2^-14) m_dqk.
For fp32 inputs (plain kernels: every step in fp32, sums of at most 2 chunk
lengths of terms over head_dim products), the same form with
u = 2^-24 and (4 chunk_len + 2 head_dim) 2^-24 in place of the bracket.
The fp16 per-round rows also have an absolute floor: below 2^-14 fp16 is
subnormal with spacing 2^-24, so each round's value may be off by 2^-25
whatever its size; n_rounds 2^-25 is added for them (not with fp32 rows).
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


def _bound(name, ref, mag, w, fp32_rows=False):
    """The derived per-element bound (module docstring); mag: the oracle's
    term magnitudes of this gradient."""
    if w.dtype == "bf16":
        u = 2.0 ** -8
        c = (2 * u if name == "dqk" else u) + 2.0 ** -11 + 2.0 ** -14
        # fp16 per-round rows: below 2^-14 the spacing is 2^-24, so each
        # round's value may be off by up to 2^-25 whatever its size
        floor = 0.0 if fp32_rows else w.n_rounds * 2.0 ** -25
    else:
        u = 2.0 ** -24
        c = (4 * w.chunk_len + 2 * w.head_dim) * 2.0 ** -24
        floor = 0.0
    return u * np.abs(ref) + c * mag + floor + 1e-30


def _check(name, g, ref, w, mag, fp32_rows=False):
    err = np.abs(g - ref)
    bound = _bound(name, ref, mag, w, fp32_rows)
    worst = float((err / bound).max())
    _say(f"  {name}: max err {err.max():.3g} (max |ref| {np.abs(ref).max():.3g}), "
         f"worst err/bound {worst:.3g}")
    assert (err <= bound).all(), f"{name} outside the derived bound (worst ratio {worst:.3g})"


def _check_both(w, c, qk, v, perm, dout, dqk, dv, fp32_rows=False):
    rq, rv = oracle.backward(c, qk, v, perm, dout)
    mq, mv = oracle.backward_magnitudes(c, qk, v, perm, dout)
    _check("dqk", dqk, rq, w, mq, fp32_rows)
    _check("dv", dv, rv, w, mv, fp32_rows)


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
    _check_both(w, oracle.config(w), inp.qk, inp.v, perm, dout, dqk, dv, fp32_rows)


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
    _check_both(sub, oracle.config(sub), np.ascontiguousarray(inp.qk[:1, heads]),
                np.ascontiguousarray(inp.v[:1, heads]), np.ascontiguousarray(perm[:1, heads]),
                np.ascontiguousarray(dout[:1, heads]), dqk[:1, heads], dv[:1, heads])


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
    _check_both(w, oracle.config(w), inp.qk, inp.v, perm, dout, dqk, dv, fp32_rows=True)


# ---------------------------------------------------------------------------
# Variant readings. Unit queries and the same-bucket mask run on the matrix
# cores for bf16 and chunk length 64, as the default reading does, and take its
# bound (the extra 1/|q| factor is one fp32 rounding, next to the bf16
# roundings the bound counts; the query's term of the magnitudes goes through
# the normalisation as its gradient does). The look-ahead and de-duplicated
# readings, and every fp32 or other-chunk shape, run on the plain kernels:
# every step in fp32 from the inputs' exact values, over windows of up to
# three chunks, so the fp32 form of the bound holds with
# (6 chunk_len + 2 head_dim) 2^-24 for the bracket, plus the rounding of the
# result to the input dtype (u |ref|).

_VFLAGS = {"look_ahead": oracle.LOOK_AHEAD, "same_bucket": oracle.SAME_BUCKET,
           "norm_queries": oracle.NORM_QUERIES, "dedup": oracle.DEDUP}
_ALLV = dict(look_ahead=True, same_bucket=True, norm_queries=True, dedup=True)

VAR_BWD = [
    (W("c4k", batch=1, heads=2, seq_len=512, n_buckets=8, n_rounds=2, causal=True),
     dict(look_ahead=True)),
    (W("c4k", batch=1, heads=2, seq_len=512, n_buckets=8, n_rounds=2, causal=False),
     dict(same_bucket=True)),
    (W("text64k", batch=1, heads=2, seq_len=512, n_buckets=8, n_rounds=2, causal=True),
     dict(norm_queries=True)),
    (W("c4k", batch=1, heads=2, seq_len=1024, n_buckets=8, n_rounds=2, causal=True),
     dict(norm_queries=True)),
    (W("text64k", batch=1, heads=2, seq_len=2048, n_buckets=16, n_rounds=4, causal=True),
     dict(norm_queries=True, same_bucket=True)),
    (W("c4k", batch=1, heads=2, seq_len=1280, n_buckets=8, n_rounds=3, causal=False),
     dict(norm_queries=True, same_bucket=True)),
    (W("c4k", batch=1, heads=2, seq_len=512, n_buckets=8, n_rounds=3, causal=True),
     dict(dedup=True)),
    (W("c4k", batch=1, heads=1, seq_len=512, n_buckets=8, n_rounds=3, causal=False),
     dict(look_ahead=True, dedup=True)),
    (W("text64k", batch=1, heads=2, seq_len=640, n_buckets=8, n_rounds=3, causal=True), _ALLV),
    (W("text64k", batch=1, heads=2, seq_len=1280, n_buckets=16, n_rounds=2, causal=True),
     dict(look_ahead=True)),
    (W("text64k", batch=1, heads=1, seq_len=1024, n_buckets=8, n_rounds=4, causal=False),
     dict(dedup=True, same_bucket=True)),
    # one chunk: the look-ahead window is the chunk itself
    (W("c4k", batch=1, heads=2, seq_len=64, n_buckets=4, n_rounds=2, causal=True),
     dict(look_ahead=True)),
    # two chunks, 8 rounds: the most the matrix-core de-duplication takes
    (W("text64k", batch=1, heads=1, seq_len=128, n_buckets=4, n_rounds=8, causal=False),
     dict(look_ahead=True, dedup=True)),
    (W("image12k", batch=2, heads=1, seq_len=768, n_buckets=8, n_rounds=2, causal=True),
     dict(look_ahead=True, same_bucket=True, norm_queries=True)),
    (W("tiny", n_rounds=2), _ALLV),  # fp32
    # 9 rounds: de-duplication past the matrix-core kernel's 8, plain kernels at bf16
    (W("c4k", batch=1, heads=1, seq_len=256, n_buckets=4, n_rounds=9, causal=True),
     dict(dedup=True)),
    # chunk length 40, 1200 positions: a ragged window count
    (W("c4k", batch=1, heads=1, seq_len=1200, chunk_len=40, n_buckets=8, n_rounds=2,
       causal=False), _ALLV),
]


def _bound_plain(ref, mag, w):
    u = 2.0 ** -8 if w.dtype == "bf16" else 2.0 ** -24
    c = (6 * w.chunk_len + 2 * w.head_dim) * 2.0 ** -24
    return u * np.abs(ref) + c * mag + 1e-30


def _bound_variant_mfma(name, ref, mag, w):
    """Look-ahead and de-duplication at bf16, chunk 64: the recomputation
    runs on the variant matrix-core kernel, reduced to dout . o_r per query,
    and the products on their own matrix-core kernels with fp32 per-round
    rows. The recomputed lse is an fp32 sum of unrounded exponentials
    (fp32-level error), but o_r weights the values by bf16(p_j) normalised by
    their own sum: each normalised weight is within 2u/(1-u) of P_ij, so
    |od_r' - od_r| <= 2u/(1-u) sum_j P_ij |dout . v_j| and |cq' - cq| <=
    2u/(1-u) E_i; in dS that is at most wP 2u/(1-u) E_i <= u/(1-u) A_ij. The
    products round wP and dS to bf16 (u of each term), and sum in fp32:
        |dv - dv_ref|   <= u |dv_ref|  + (u + c_fp32) m_dv,
        |dqk - dqk_ref| <= u |dqk_ref| + (u + u/(1-u) + c_fp32) m_dqk,
    with c_fp32 = (6 chunk_len + 2 head_dim) 2^-24, the plain path's constant
    for its fp32 logits, exponentials and sums."""
    u = 2.0 ** -8
    c = u + (6 * w.chunk_len + 2 * w.head_dim) * 2.0 ** -24
    if name == "dqk":
        c += u / (1 - u)
    return u * np.abs(ref) + c * mag + 1e-30


@pytest.mark.parametrize("w,kw", VAR_BWD,
                         ids=[f"{w.name}-{w.dtype}-H{w.heads}L{w.seq_len}m{w.chunk_len}"
                              f"R{w.n_rounds}{'c' if w.causal else 'n'}-" + "+".join(kw)
                              for w, kw in VAR_BWD])
def test_variant_backward_parity(w, kw):
    _say(f"[backward variant] {w} {sorted(kw)}")
    _variant_backward_check(w, kw, workloads.make_inputs(w))


@pytest.mark.parametrize("kw", [dict(norm_queries=True, same_bucket=True),
                                dict(norm_queries=True, look_ahead=True)],
                         ids=["nq+sb-matrix-cores", "nq+la-variant-kernel"])
def test_variant_backward_zero_rows(kw):
    """Zero qk rows: a zero key or unit query is 0, every logit with it is 0,
    and the normalisation passes no gradient to the row."""
    w = W("c4k", batch=1, heads=2, seq_len=512, n_buckets=8, n_rounds=2, causal=True)
    _say(f"[backward variant zero rows] {w} {sorted(kw)}")
    inp = workloads.make_inputs(w)
    inp.qk[:, :, ::7] = 0.0
    inp.qk_bits[:, :, ::7] = 0
    _variant_backward_check(w, kw, inp)


def _variant_backward_check(w, kw, inp):
    dev = torch.device("cuda", 0)
    qk, v, rot = to_device(inp, dev)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    op = lat.LSHAttention(w.batch, w.heads, w.seq_len, w.head_dim, w.n_buckets, w.n_rounds,
                          w.chunk_len, w.causal, dtype=dt, backward=True, **kw)
    try:
        _, ex = op(qk, v, rot, return_perm=True, return_buckets=True)
        dout_t, dout = _dout(w, 7100 + w.seq_len + w.n_rounds)
        sb = kw.get("same_bucket", False)
        dqk, dv = op.backward(qk, v, ex["perm"], dout_t.to(dev),
                              buckets=ex["buckets"] if sb else None)
        torch.cuda.synchronize()
        perm = ex["perm"].cpu().numpy()
        bk = ex["buckets"].cpu().numpy()
        dqk = dqk.to(torch.float64).cpu().numpy()
        dv = dv.to(torch.float64).cpu().numpy()
    finally:
        op.close()
    variant = sum(_VFLAGS[k] for k, on in kw.items() if on)
    c = oracle.config(w, variant=variant)
    rq, rv = oracle.backward(c, inp.qk, inp.v, perm, dout, buckets=bk)
    mq, mv = oracle.backward_magnitudes(c, inp.qk, inp.v, perm, dout, buckets=bk)
    # which kernels ran: the default kernel's matrix-core recomputation and
    # fused products (its readings), the variant kernels' (look-ahead,
    # de-duplication), or plain kernels throughout
    mfma_shape = w.dtype == "bf16" and w.chunk_len == 64 and w.head_dim in (64, 128)
    la_dd = kw.get("look_ahead", False) or kw.get("dedup", False)
    mfma = mfma_shape and not la_dd
    var_dot = mfma_shape and la_dd and (not kw.get("dedup") or w.n_rounds <= 8)
    for name, g, ref, mag in (("dqk", dqk, rq, mq), ("dv", dv, rv, mv)):
        err = np.abs(g - ref)
        if mfma:
            bound = _bound(name, ref, mag, w)
        elif var_dot:
            bound = _bound_variant_mfma(name, ref, mag, w)
        else:
            bound = _bound_plain(ref, mag, w)
        worst = float((err / bound).max())
        _say(f"  {name}: max err {err.max():.3g} (max |ref| {np.abs(ref).max():.3g}), "
             f"worst err/bound {worst:.3g}")
        assert (err <= bound).all(), f"{name} outside the bound (worst ratio {worst:.3g})"


def test_same_bucket_backward_needs_the_buckets():
    w = W("c4k", batch=1, heads=1, seq_len=256, n_buckets=4, n_rounds=1, causal=True)
    _say(f"[backward same-bucket without buckets] {w}")
    inp = workloads.make_inputs(w)
    dev = torch.device("cuda", 0)
    qk, v, rot = to_device(inp, dev)
    op = lat.LSHAttention(w.batch, w.heads, w.seq_len, w.head_dim, w.n_buckets, w.n_rounds,
                          w.chunk_len, w.causal, backward=True, same_bucket=True)
    try:
        _, ex = op(qk, v, rot, return_perm=True)
        with pytest.raises(lat.LSHAttnError) as e:
            op.backward(qk, v, ex["perm"], torch.zeros_like(qk))
        assert e.value.status == 1  # INVALID_ARG
    finally:
        op.close()
