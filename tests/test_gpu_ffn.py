"""The chunked feed-forward (lsh_ffn_forward) against the fp64 oracle, element
by element, on seeded inputs; chunking on the GPU changes no bit; the
residual may be updated in place. Each case prints what it is first.

Tolerance, per output element (u = 2^-8 for bf16's 8-bit significand, 2^-24
for fp32; g = 2^-24, the fp32 unit roundoff of the accumulations): with h the
oracle's hidden row and K1 = d_model, K2 = d_ff,
  dh_j  = u |h_j| + (1 + u)(K1 + 1) g (sum_k |y1_k w1_jk| + |b1_j|)
          (the first layer's fp32 sum, ReLU being 1-Lipschitz, then the
          rounding of the hidden row to the layer dtype),
  bound = 2 (u |y2| + sum_j |w2_ej| dh_j
             + (K2 + 2) g (sum_j (|h_j| + dh_j) |w2_ej| + |b2_e| + |x2_e|))
          (the propagated hidden error, the second sum, the output rounding;
          a 2x margin).
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
import lsh_attention_hash_amd as lat

pytestmark = pytest.mark.gpu

G = 2.0 ** -24


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lat.load_library()


def _tensors(fi):
    if fi.dtype == "bf16":
        return {k: torch.from_numpy(b.view(np.int16)).cuda().view(torch.bfloat16)
                for k, b in fi.bits.items()}
    return {k: torch.from_numpy(getattr(fi, k)).cuda() for k in fi.bits}


def _gpu(fi, chunk, residual=True, t=None, out=None):
    dt = torch.bfloat16 if fi.dtype == "bf16" else torch.float32
    t = t or _tensors(fi)
    op = lat.ChunkedFeedForward(fi.rows, fi.d_model, fi.d_ff, chunk, dtype=dt)
    try:
        y2 = op(t["y1"], t["w1"], t["b1"], t["w2"], t["b2"],
                x2=t["x2"] if residual else None, out=out)
        torch.cuda.synchronize()
        return y2.float().cpu().numpy().astype(np.float64)
    finally:
        op.close()


def _check(fi, got, residual=True, rows=None):
    """rows: sample of rows (all when None)."""
    sel = slice(None) if rows is None else rows
    y1, x2 = fi.y1[sel], fi.x2[sel]
    ref, h = oracle.ffn(y1, fi.w1, fi.b1, fi.w2, fi.b2, x2=x2 if residual else None,
                        return_hidden=True)
    u = 2.0 ** -8 if fi.dtype == "bf16" else 2.0 ** -24
    a1 = np.abs(y1.astype(np.float64)) @ np.abs(fi.w1.astype(np.float64)).T \
        + np.abs(fi.b1.astype(np.float64))
    dh = u * h + (1 + u) * (fi.d_model + 1) * G * a1
    aw2 = np.abs(fi.w2.astype(np.float64)).T
    a2 = (h + dh) @ aw2 + np.abs(fi.b2.astype(np.float64))
    if residual:
        a2 = a2 + np.abs(x2.astype(np.float64))
    bound = 2.0 * (u * np.abs(ref) + dh @ aw2 + (fi.d_ff + 2) * G * a2)
    got = got if rows is None else got[rows]
    err = np.abs(got - ref)
    worst = float((err / bound).max()) if err.size else 0.0
    _say(f"  max err {err.max() if err.size else 0:.3g}, worst err/bound {worst:.3g}")
    assert (err <= bound).all(), "outside the feed-forward bound"


CASES = [
    # rows, d_model, d_ff, chunk, dtype, residual
    (300, 128, 512, 128, "bf16", True),     # chunks 128, 128, 44: ragged tail
    (256, 256, 1024, 0, "bf16", True),      # one chunk
    (77, 128, 256, 100, "bf16", False),     # fewer rows than a tile, no residual
    (1000, 384, 1536, 333, "bf16", True),   # several tiles per chunk, odd chunk size
    (200, 96, 200, 64, "bf16", True),       # off the matrix-core path (plain kernel)
    (150, 64, 256, 50, "fp32", True),       # fp32 (plain kernel)
    (1, 256, 512, 0, "bf16", True),         # a single row
    (257, 256, 768, 0, "bf16", True),       # one row past a 256-row tile
]


@pytest.mark.parametrize("rows,d_model,d_ff,chunk,dtype,residual", CASES,
                         ids=[f"r{r}-dm{a}-ff{b}-c{c}-{d}{'-res' if e else ''}"
                              for r, a, b, c, d, e in CASES])
def test_ffn_parity(rows, d_model, d_ff, chunk, dtype, residual):
    _say(f"[ffn] rows={rows} d_model={d_model} d_ff={d_ff} chunk={chunk} {dtype} "
         f"residual={residual}")
    fi = workloads.make_ffn_inputs(rows, d_model, d_ff, dtype, seed=rows)
    _check(fi, _gpu(fi, chunk, residual), residual)


def test_ffn_chunking_changes_no_bit():
    """Chunks of one row up to all rows (one-row chunks: a tile with a single
    live row; 7: every tile ragged) give the same bits."""
    fi = workloads.make_ffn_inputs(1000, 256, 1024, "bf16", seed=11)
    _say("[ffn chunks] rows=1000 d_model=256 d_ff=1024, chunks 0, 1, 7, 128, 200, 999")
    t = _tensors(fi)
    base = _gpu(fi, 0, t=t)
    for chunk in (1, 7, 128, 200, 999):
        np.testing.assert_array_equal(_gpu(fi, chunk, t=t), base)


def test_ffn_residual_in_place():
    """y2 written over x2 equals y2 written elsewhere."""
    fi = workloads.make_ffn_inputs(300, 128, 512, "bf16", seed=12)
    _say("[ffn in place] rows=300 d_model=128 d_ff=512 chunk=128")
    t = _tensors(fi)
    want = _gpu(fi, 128, t=t)
    t["x2"] = t["x2"].clone()
    got = _gpu(fi, 128, t=t, out=t["x2"])
    np.testing.assert_array_equal(got, want)


def test_ffn_full_size_sampled_rows():
    """65,536 rows, d_model 1024, d_ff 4096 in chunks of 16,384 rows (the
    benchmark's configuration): 96 sampled rows (first, last and chunk edges
    among them) against the oracle."""
    rows, dm, dff, chunk = 65536, 1024, 4096, 16384
    _say(f"[ffn full size] rows={rows} d_model={dm} d_ff={dff} chunk={chunk}")
    fi = workloads.make_ffn_inputs(rows, dm, dff, "bf16")
    got = _gpu(fi, chunk)
    rng = np.random.default_rng(13)
    sample = np.unique(np.concatenate([rng.choice(rows, size=88, replace=False),
                                       [0, chunk - 1, chunk, 2 * chunk, 3 * chunk - 1,
                                        3 * chunk, rows - 2, rows - 1]]))
    _check(fi, got, rows=sample)


def test_ffn_rejects_bad_calls():
    op = lat.ChunkedFeedForward(64, 128, 256, 0)
    try:
        z = torch.zeros(1 << 16, dtype=torch.bfloat16, device="cuda")
        p = z.data_ptr()
        f = op.lib.lsh_ffn_forward
        assert f(op.handle, 65, p, p, p, p, p, None, p, None) == 1     # rows > max_rows
        assert f(op.handle, -1, p, p, p, p, p, None, p, None) == 1
        assert f(op.handle, 8, p + 2, p, p, p, p, None, p, None) == 1  # misaligned y1
        assert f(op.handle, 8, p, p, None, p, p, None, p, None) == 1   # no b1
        assert f(op.handle, 0, p, p, p, p, p, None, p, None) == 0      # nothing to do
        assert op.workspace_bytes() == 64 * 256 * 2
    finally:
        op.close()
