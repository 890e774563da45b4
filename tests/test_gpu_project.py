"""The forward from a layer input (lsh_attn_forward_x): the shared-QK and value
projections against the fp64 oracle's, element by element, then the whole
forward on the GPU's qk and v as in the default parity, and the fused hash
preparation checked by the forward's bitwise agreement with lsh_attn_forward
on the same qk and v. Each case prints what it is first.

Projection tolerance: qk and v come back in the input dtype from fp32 sums
over model_dim products. For each element the bound is the output rounding
(the unit roundoff: 2^-8 relative for bf16's 8-bit significand, 2^-24 for
fp32) plus the worst-case fp32 summation error of its dot product,
K 2^-24 sum_k |x_k w_k| (K = model_dim), both with a 2x margin.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
import lsh_attention_hash_amd as lat
from parity import OUT_TOL, _cmp_lse, check_buckets

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


def _dev(a, bits, dtype):
    if dtype == "bf16":
        return torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def _run(w, li):
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    x = _dev(li.x, li.x_bits, w.dtype)
    wq = _dev(li.w_qk, li.w_qk_bits, w.dtype)
    wv = _dev(li.w_v, li.w_v_bits, w.dtype)
    rot = None if li.rotations is None else torch.from_numpy(li.rotations).cuda()
    op = lat.LSHAttention(w.batch, w.heads, w.seq_len, w.head_dim, w.n_buckets, w.n_rounds,
                          w.chunk_len, w.causal, dtype=dt)
    try:
        out, qk, v, ex = op.forward_x(x, wq, wv, rot, return_lse=True, return_buckets=True,
                                      return_perm=True)
        # the same forward from the qk and v it produced
        out2 = op(qk, v, rot)
        torch.cuda.synchronize()
        res = {"out": out.float().cpu().numpy().astype(np.float64),
               "out_direct": out2.float().cpu().numpy().astype(np.float64),
               "qk": qk.float().cpu().numpy().astype(np.float64),
               "v": v.float().cpu().numpy().astype(np.float64),
               "lse": ex["lse"].cpu().numpy(), "buckets": ex["buckets"].cpu().numpy(),
               "perm": ex["perm"].cpu().numpy()}
    finally:
        op.close()
    return res


def _check_projection(w, li, got_qk, got_v, rows=None):
    """rows: sample of (b, i) rows of x (all when None)."""
    xs = li.x if rows is None else li.x.reshape(-1, li.model_dim)[rows][None]
    c = oracle.config(w, batch=1 if rows is not None else w.batch,
                      seq_len=xs.shape[1])
    rq, rv = oracle.project(c, xs, li.w_qk, li.w_v)
    K = li.model_dim
    rel = 2.0 ** -8 if w.dtype == "bf16" else 2.0 ** -24
    for name, got, ref, wt in (("qk", got_qk, rq, li.w_qk), ("v", got_v, rv, li.w_v)):
        if rows is not None:  # [B, H, L, d] -> the sampled rows, as [1, H, n, d]
            B, H, L, d = got.shape
            got = got.transpose(1, 0, 2, 3).reshape(H, B * L, d)[:, rows][None]
        absdot = np.abs(xs.astype(np.float64)) @ np.abs(wt.astype(np.float64)).T  # [.., L, H*d]
        absdot = absdot.reshape(absdot.shape[0], absdot.shape[1], w.heads, w.head_dim)
        absdot = absdot.transpose(0, 2, 1, 3)
        bound = 2.0 * (rel * np.abs(ref) + K * 2.0 ** -24 * absdot)
        err = np.abs(got - ref)
        worst = float((err / np.maximum(bound, 1e-300)).max())
        _say(f"  {name}: max err {err.max():.3g}, worst err/bound {worst:.3g}")
        assert (err <= bound).all(), f"{name} outside the projection bound"


CASES = [
    (W("c4k", batch=1, heads=2, seq_len=256, n_buckets=8, n_rounds=2), 128),
    (W("text64k", batch=1, heads=2, seq_len=512, n_buckets=16, n_rounds=4), 256),
    (W("c4k", batch=1, heads=3, seq_len=320, n_buckets=8, n_rounds=1, causal=False), 192),  # ragged
    (W("c4k", batch=2, heads=2, seq_len=192, n_buckets=8, n_rounds=2), 64),
    (W("c4k", batch=1, heads=2, seq_len=256, n_buckets=8, n_rounds=2), 80),   # plain kernel
    (W("tiny", n_rounds=2), 96),                                            # fp32
    (W("c4k", batch=1, heads=2, seq_len=256, n_buckets=8, n_rounds=2), 96),   # 3 K slabs of 32
    # d = 128: two-head tiles (even H, model_dim of 64s), ragged rows
    (W("text64k", batch=1, heads=2, seq_len=320, n_buckets=16, n_rounds=2), 128),
    # d = 128: one-head tiles (odd H); two-head tiles over 3 K slabs
    (W("text64k", batch=1, heads=3, seq_len=320, n_buckets=16, n_rounds=2), 192),
    (W("text64k", batch=2, heads=2, seq_len=256, n_buckets=16, n_rounds=2), 96),
]


@pytest.mark.parametrize("w,model_dim", CASES,
                         ids=[f"{w.name}-{w.dtype}-B{w.batch}H{w.heads}L{w.seq_len}d{w.head_dim}"
                              f"-k{k}" for w, k in CASES])
def test_forward_from_layer_input(w, model_dim):
    _say(f"[forward_x] {w} model_dim={model_dim}")
    li = workloads.make_layer_inputs(w, model_dim)
    gpu = _run(w, li)
    _check_projection(w, li, gpu["qk"], gpu["v"])
    # the forward on the GPU's own qk and v
    inp = workloads.Inputs(w, gpu["qk"].astype(np.float32), gpu["v"].astype(np.float32),
                           li.rotations)
    check_buckets(w, inp, gpu["buckets"])
    c = oracle.config(w)
    ref = oracle.forward(c, gpu["qk"], gpu["v"], li.rotations, buckets_override=gpu["buckets"])
    np.testing.assert_array_equal(ref["perm"], gpu["perm"])
    err = np.abs(gpu["out"] - ref["out"])
    _say(f"  out max err {err.max():.3g}")
    assert err.max() <= OUT_TOL[w.dtype]
    _cmp_lse(w, gpu["lse"], ref["lse"])
    # the projection's hash preparation equals the hash's own
    np.testing.assert_array_equal(gpu["out"], gpu["out_direct"])


def test_forward_from_layer_input_full_size():
    """Text-64K (model_dim = H d = 1024) in the bench's configuration: sampled
    rows of qk and v against the oracle's projection, and the forward equal
    to lsh_attn_forward on the same qk and v."""
    w = workloads.get("text64k")
    model_dim = w.heads * w.head_dim
    _say(f"[forward_x full size] {w} model_dim={model_dim}")
    li = workloads.make_layer_inputs(w, model_dim)
    gpu = _run(w, li)
    rows = np.unique(np.random.default_rng(3).choice(w.batch * w.seq_len, size=256,
                                                     replace=False))
    _check_projection(w, li, gpu["qk"], gpu["v"], rows=rows)
    inp = workloads.Inputs(w, gpu["qk"].astype(np.float32), gpu["v"].astype(np.float32),
                           li.rotations)
    check_buckets(w, inp, gpu["buckets"])
    np.testing.assert_array_equal(gpu["out"], gpu["out_direct"])


def test_forward_x_rejects_bad_arguments():
    import ctypes
    op = lat.LSHAttention(1, 1, 256, 64, 4, 1, 64, True)
    try:
        z = torch.zeros(64, device="cuda")
        p = ctypes.c_void_p(z.data_ptr())
        f = op.lib.lsh_attn_forward_x
        assert f(op.handle, p, ctypes.c_int32(0), p, p, p, p, p, p, None, None, None, None) == 1
        assert f(op.handle, None, ctypes.c_int32(64), p, p, p, p, p, p, None, None, None,
                 None) == 1
    finally:
        op.close()
