"""HIP path vs the fp64 oracle, through the C ABI, on seeded inputs.

Every case is compared with the oracle's own forward element by element:
bucket ids and permutations bit-exact everywhere (near-ties included and
counted), every output and logsumexp within its tolerance. That holds for the
full-size workloads too (every head, every round, every position), in the
launch configuration the bench times. Each case prints what it is before it
runs.
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
import lsh_attention_hash_amd as lat
from parity import (OUT_TOL, check_buckets, check_forward, check_outputs_full, check_perm,
                    make_op, run_gpu, scaled_inputs, to_device)

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


SMALL = [
    # several sort tiles with a ragged tail (L = 64 * 37), ragged hash tiles
    W("c4k", batch=1, heads=2, seq_len=2368, n_buckets=96, n_rounds=3, causal=True),
    W("c4k", batch=2, heads=1, seq_len=2368, n_buckets=96, n_rounds=3, causal=False),
    W("c4k", batch=1, heads=3, seq_len=1024, n_buckets=2, n_rounds=2, causal=True),
    W("c4k", batch=1, heads=2, seq_len=1024, n_buckets=6, n_rounds=1, causal=False),
    W("text64k", batch=1, heads=2, seq_len=1536, n_buckets=64, n_rounds=2, causal=True),
    W("text64k", batch=1, heads=1, seq_len=4096, n_buckets=128, n_rounds=1, causal=False),
    W("skewed", batch=1, heads=2, seq_len=2048, n_buckets=32, n_rounds=2),
    W("image12k", batch=2, heads=2, seq_len=768, n_buckets=12, n_rounds=4),
    W("c4k", batch=1, heads=1, seq_len=64, n_buckets=4, n_rounds=2, causal=True),   # one chunk
    W("c4k", batch=1, heads=2, seq_len=512, n_buckets=1024, n_rounds=1, causal=False),  # nb > L
    # a round count the combination has no specialisation for (groups of 4 + 1)
    W("image12k", batch=1, heads=2, seq_len=1024, n_buckets=16, n_rounds=5, causal=True),
    # bucket ids beyond one LDS window of the sort's histograms
    W("c4k", batch=1, heads=1, seq_len=4096, n_buckets=8192, n_rounds=2, causal=True),
    W("c4k", batch=1, heads=1, seq_len=1024, n_buckets=65536, n_rounds=1, causal=False),  # max nb
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: f"{w.name}-B{w.batch}H{w.heads}L{w.seq_len}"
                         f"d{w.head_dim}nb{w.n_buckets}R{w.n_rounds}{'c' if w.causal else 'n'}")
def test_small_full_parity(w):
    _say(f"[small] {w}")
    inp = workloads.make_inputs(w)
    gpu = run_gpu(w, inp)
    r = check_forward(w, inp, gpu)
    _say(f"  buckets {r['buckets']} ties {r['ties']} out err {r['out_err']:.3g} "
         f"lse err {r['lse_err']:.3g}")


def test_tiny_fp32_full_parity():
    w = workloads.get("tiny")
    _say(f"[tiny] {w}")
    inp = workloads.make_inputs(w)
    gpu = run_gpu(w, inp)
    r = check_forward(w, inp, gpu)
    assert r["out_err"] <= 1e-5
    _say(f"  out err {r['out_err']:.3g} lse err {r['lse_err']:.3g}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_one_bucket_one_chunk_is_full_attention(causal, d):
    """n_buckets = 1 and one chunk covering the sequence: the path reduces to
    full shared-QK softmax attention with the self-mask."""
    w = W("c4k", batch=2, heads=2, seq_len=128, head_dim=d, n_buckets=1, n_rounds=2,
          chunk_len=128, causal=causal)
    _say(f"[nb=1] {w}")
    inp = workloads.make_inputs(w)
    gpu = run_gpu(w, inp)
    assert np.all(gpu["buckets"] == 0)
    np.testing.assert_array_equal(gpu["perm"], np.broadcast_to(np.arange(w.seq_len),
                                                               gpu["perm"].shape))
    check_outputs_full(w, inp, gpu)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_odd_chunk_length(causal, d):
    """A chunk length of 40 (the plain kernel): query blocks of 16, 16 and 8,
    and key blocks that end inside the window."""
    w = W("c4k", batch=1, heads=2, seq_len=1200, head_dim=d, n_buckets=16, n_rounds=2,
          chunk_len=40, causal=causal)
    _say(f"[chunk 40] {w}")
    inp = workloads.make_inputs(w)
    gpu = run_gpu(w, inp)
    r = check_forward(w, inp, gpu)
    _say(f"  out err {r['out_err']:.3g} lse err {r['lse_err']:.3g}")


def test_out_dtype_fp32_and_separate_gather():
    w = W("c4k", batch=1, heads=2, seq_len=2048, n_buckets=32, n_rounds=2, causal=True)
    _say(f"[out fp32 / separate gather] {w}")
    inp = workloads.make_inputs(w)
    a = run_gpu(w, inp, out_dtype=torch.float32)
    check_outputs_full(w, inp, a)
    b = run_gpu(w, inp, out_dtype=torch.float32, separate_gather=True)
    for k in ("out", "lse", "buckets", "perm"):
        np.testing.assert_array_equal(a[k], b[k])


@pytest.mark.parametrize("causal", [False, True])
def test_fp32_round_outputs(causal):
    """Per-round outputs kept in fp32 instead of fp16: both within tolerance."""
    w = W("text64k", batch=1, heads=2, seq_len=2048, n_buckets=32, n_rounds=3, causal=causal)
    _say(f"[fp32 round outputs] {w}")
    inp = workloads.make_inputs(w)
    a = run_gpu(w, inp, out_dtype=torch.float32, fp32_round_outputs=True)
    e32, _ = check_outputs_full(w, inp, a)
    b = run_gpu(w, inp, out_dtype=torch.float32)
    e16, _ = check_outputs_full(w, inp, b)
    np.testing.assert_array_equal(a["lse"], b["lse"])
    _say(f"  out err fp32 round outputs {e32:.3g}, fp16 {e16:.3g}")


def test_deterministic():
    w = W("skewed", batch=1, heads=2, seq_len=4096, n_buckets=64, n_rounds=4)
    _say(f"[determinism] {w}")
    inp = workloads.make_inputs(w)
    op = make_op(w)
    qk, v, rot = to_device(inp)
    o1, e1 = op(qk, v, rot, return_lse=True, return_perm=True)
    o2, e2 = op(qk, v, rot, return_lse=True, return_perm=True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(e1["lse"], e2["lse"]) and torch.equal(e1["perm"], e2["perm"])


def test_zero_vectors_and_constant_rows():
    """Zero qk rows: every projection is 0 (bucket 0 by the lowest-index rule,
    margin 0 so it counts as a tie) and a zero key has logit 0."""
    w = W("c4k", batch=1, heads=1, seq_len=512, n_buckets=16, n_rounds=2, causal=True)
    _say(f"[zero rows] {w}")
    inp = workloads.make_inputs(w)
    inp.qk[0, 0, ::7] = 0.0
    inp.qk_bits[0, 0, ::7] = 0
    gpu = run_gpu(w, inp)
    assert np.all(gpu["buckets"][0, 0, :, ::7] == 0)
    check_buckets(w, inp, gpu["buckets"])
    check_outputs_full(w, inp, gpu)


FULL = ["c4k", "text64k", "image12k", "skewed"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_parity(name):
    """The workload at full size, compared over every element with the
    oracle's whole forward (tens of seconds of fp64 on the host threads)."""
    w = workloads.get(name)
    _say(f"[full] {w}")
    inp = workloads.make_inputs(w)
    gpu = run_gpu(w, inp)
    r = check_forward(w, inp, gpu)
    _say(f"  buckets {r['buckets']} ties {r['ties']} out err {r['out_err']:.3g} "
         f"lse err {r['lse_err']:.3g} stats {gpu['stats']}")


def test_forward_rejects_null_and_misaligned_pointers():
    w = W("c4k", batch=1, heads=1, seq_len=256, n_buckets=8, n_rounds=1)
    op = make_op(w)
    inp = workloads.make_inputs(w)
    qk, v, rot = to_device(inp)
    out = torch.empty_like(qk)
    lib = op.lib
    P = ctypes.c_void_p
    s = P(torch.cuda.current_stream().cuda_stream)
    assert lib.lsh_attn_forward(op.handle, None, P(v.data_ptr()), P(rot.data_ptr()),
                                P(out.data_ptr()), None, None, None, s) == 1
    assert lib.lsh_attn_forward(op.handle, P(qk.data_ptr()), P(v.data_ptr()), None,
                                P(out.data_ptr()), None, None, None, s) == 1
    assert lib.lsh_attn_forward(op.handle, P(qk.data_ptr() + 2), P(v.data_ptr()),
                                P(rot.data_ptr()), P(out.data_ptr()), None, None, None, s) == 1
    assert op.workspace_bytes() > 0
    op.close()


@pytest.mark.parametrize("L", [65536, 131072])
def test_sort_of_long_segments(L):
    """Segments of 64 and 128 sort tiles (L above the bench's 65,536 too):
    buckets against the oracle's hash, the permutation equal to the oracle's
    stable sort."""
    w = W("c4k", batch=1, heads=1, seq_len=L, n_buckets=256, n_rounds=1, causal=False)
    _say(f"[long sort] {w}")
    inp = workloads.make_inputs(w)
    qk, v, rot = to_device(inp)
    op = make_op(w)
    try:
        _, ex = op(qk, v, rot, return_buckets=True, return_perm=True)
        torch.cuda.synchronize()
        gb = ex["buckets"].cpu().numpy()
        gp = ex["perm"].cpu().numpy()
    finally:
        op.close()
    check_buckets(w, inp, gb)
    check_perm(w, gb, gp)


@pytest.mark.parametrize("L,nb", [(16384, 1024), (16320, 1000), (4096, 2), (1024, 1026)])
def test_sort_segment_form(L, nb):
    """Segments short enough for the one-launch sort (L <= 16384 with at most
    1024 buckets: its longest segment and most buckets, a ragged last wave,
    two buckets), and just past its bucket limit (the tiled form): the
    permutation equal to the oracle's stable sort of the GPU's buckets."""
    w = W("c4k", batch=1, heads=2, seq_len=L, n_buckets=nb, n_rounds=2, causal=False)
    _say(f"[segment sort] {w}")
    inp = workloads.make_inputs(w)
    qk, v, rot = to_device(inp)
    op = make_op(w)
    try:
        _, ex = op(qk, v, rot, return_buckets=True, return_perm=True)
        torch.cuda.synchronize()
        gb = ex["buckets"].cpu().numpy()
        gp = ex["perm"].cpu().numpy()
    finally:
        op.close()
    check_buckets(w, inp, gb)
    check_perm(w, gb, gp)


LARGE = [
    # d = 128: |q| ~ 1,450, Cauchy-Schwarz shift ~185 > 60: the true-max softmax
    (W("text64k", batch=1, heads=2, seq_len=2048, n_buckets=64, n_rounds=2, causal=True), 7, 0),
    (W("text64k", batch=1, heads=1, seq_len=1024, n_buckets=16, n_rounds=3, causal=False), 7, 0),
    # d = 64, qk and v both scaled
    (W("c4k", batch=1, heads=2, seq_len=2048, n_buckets=32, n_rounds=3, causal=True), 7, 7),
    (W("image12k", batch=2, heads=1, seq_len=768, n_buckets=12, n_rounds=4, causal=False), 7, 0),
    # fp32 inputs (plain kernels)
    (W("tiny", n_rounds=2, causal=True), 7, 0),
]


@pytest.mark.parametrize("w,qk_exp,v_exp", LARGE,
                         ids=[f"{w.name}-{w.dtype}-L{w.seq_len}d{w.head_dim}R{w.n_rounds}"
                              f"{'c' if w.causal else 'n'}-qk2^{a}-v2^{b}" for w, a, b in LARGE])
def test_large_magnitudes(w, qk_exp, v_exp):
    """qk (and v) multiplied by a power of two, exact in the storage type: the
    hash certificate and the re-scoring at large norms (buckets equal to the
    oracle's and to those of the unscaled rows, since the definition is
    invariant to positive scaling), and the softmax branch that takes the true
    row maximum when the Cauchy-Schwarz shift is too large for exp2."""
    inp = workloads.make_inputs(w)
    big = scaled_inputs(inp, qk_exp, v_exp)
    _say(f"[large] {w} qk x 2^{qk_exp} v x 2^{v_exp}")
    gpu = run_gpu(w, big)
    r = check_forward(w, big, gpu, v_scale=2.0 ** v_exp, scaled_qk=qk_exp > 0)
    assert gpu["stats"]["n_round_rows_at_fp16_limit"] == 0
    base = run_gpu(w, inp)
    np.testing.assert_array_equal(gpu["buckets"], base["buckets"])
    _say(f"  buckets {r['buckets']} ties {r['ties']} out err {r['out_err']:.3g} "
         f"lse err {r['lse_err']:.3g}")


def test_round_rows_at_the_fp16_limit():
    """Per-round rows are fp16 by default: v x 2^13 (|v| < 65504) stays exact
    to the tolerance and reaches no limit; v x 2^16 takes some rows past
    +-65504, which the library counts, and with fp32 per-round rows the same
    inputs match the oracle again."""
    w = W("c4k", batch=1, heads=2, seq_len=1024, n_buckets=16, n_rounds=2, causal=True)
    inp = workloads.make_inputs(w)
    _say(f"[fp16 limit] {w}")
    mid = scaled_inputs(inp, 0, 13)
    assert np.abs(mid.v).max() < 65504
    g = run_gpu(w, mid)
    assert g["stats"]["n_round_rows_at_fp16_limit"] == 0
    check_forward(w, mid, g, v_scale=2.0 ** 13)
    big = scaled_inputs(inp, 0, 16)
    g = run_gpu(w, big)
    hits = g["stats"]["n_round_rows_at_fp16_limit"]
    _say(f"  v x 2^16: {hits} pieces at the fp16 limit")
    assert hits > 0
    g = run_gpu(w, big, fp32_round_outputs=True)
    assert g["stats"]["n_round_rows_at_fp16_limit"] == 0
    r = check_forward(w, big, g, v_scale=2.0 ** 16)
    _say(f"  fp32 round rows: out err {r['out_err']:.3g}")
