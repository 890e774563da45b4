"""Pins of the oracle's backward (gradients at fixed buckets), CPU only.

The backward is the chain rule through the forward's steps; these tests check
it against things that do not share its formulas:
  * central finite differences of the oracle's own forward (buckets held
    fixed through buckets_override), element by element, on small inputs that
    span several chunks, several rounds, the causal and the plain mask, and
    queries that see only themselves;
  * for one bucket and one chunk covering the sequence, PyTorch fp64 autograd
    of dense shared-QK attention with unit keys and the self-mask, a separate
    formulation (the forward of that case is pinned to SDPA).
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _cfg(B, H, L, d, nb, R, m, causal):
    return oracle.config(batch=B, heads=H, seq_len=L, head_dim=d, n_buckets=nb, n_rounds=R,
                         chunk_len=m, causal=int(causal))


def _loss(c, qk, v, bk, dout):
    return float(np.sum(oracle.forward(c, qk, v, None, buckets_override=bk)["out"] * dout))


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_finite_differences(oracle_lib, causal):
    rng = np.random.default_rng(7 + int(causal))
    B, H, L, d, nb, R, m = 1, 2, 16, 4, 4, 2, 4
    c = _cfg(B, H, L, d, nb, R, m, causal)
    qk = rng.standard_normal((B, H, L, d))
    v = rng.standard_normal((B, H, L, d))
    rot = rng.standard_normal((R, d, nb // 2))
    bk, _ = oracle.hash(c, qk, rot)
    pm, _ = oracle.sort(c, bk)
    dout = rng.standard_normal((B, H, L, d))
    lse = oracle.forward(c, qk, v, None, buckets_override=bk)["lse"]
    if causal:
        assert (lse == oracle.SELF_LOGIT).any(), "case should hold self-only queries"
    dqk, dv = oracle.backward(c, qk, v, pm, dout)
    h = 1e-6
    for x, g in ((qk, dqk), (v, dv)):
        fd = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + h
            up = _loss(c, qk, v, bk, dout)
            x[idx] = keep - h
            dn = _loss(c, qk, v, bk, dout)
            x[idx] = keep
            fd[idx] = (up - dn) / (2 * h)
        np.testing.assert_allclose(g, fd, rtol=0, atol=2e-7)


def _dense_grads(qk, v, dout, causal):
    """Dense shared-QK attention, unit keys, self-mask (self only when nothing
    else is allowed), differentiated by torch autograd in float64."""
    L, d = qk.shape
    q = torch.tensor(qk, requires_grad=True)
    vv = torch.tensor(v, requires_grad=True)
    k = q / q.norm(dim=-1, keepdim=True)
    allowed = ~torch.eye(L, dtype=torch.bool)
    if causal:
        allowed &= torch.ones(L, L, dtype=torch.bool).tril()
    empty = ~allowed.any(dim=1)
    logits = (q @ k.T) / math.sqrt(d)
    p = torch.softmax(logits.masked_fill(~allowed, -math.inf).masked_fill(empty[:, None], 0.0),
                      dim=1)
    out = torch.where(empty[:, None], vv, p @ vv)
    (out * torch.tensor(dout)).sum().backward()
    return q.grad.numpy(), vv.grad.numpy()


@pytest.mark.parametrize("R,causal", [(1, False), (1, True), (3, False), (3, True)])
def test_backward_single_chunk_equals_dense_autograd(oracle_lib, R, causal):
    rng = np.random.default_rng(30 + R + int(causal))
    B, H, L, d = 1, 2, 24, 8
    c = _cfg(B, H, L, d, 1, R, L, causal)
    qk = rng.standard_normal((B, H, L, d))
    v = rng.standard_normal((B, H, L, d))
    dout = rng.standard_normal((B, H, L, d))
    pm = oracle.forward(c, qk, v, None)["perm"]
    dqk, dv = oracle.backward(c, qk, v, pm, dout)
    for b in range(B):
        for h in range(H):
            gq, gv = _dense_grads(qk[b, h], v[b, h], dout[b, h], causal)
            np.testing.assert_allclose(dqk[b, h], gq, rtol=0, atol=1e-12)
            np.testing.assert_allclose(dv[b, h], gv, rtol=0, atol=1e-12)


def test_backward_zero_key_stays_finite(oracle_lib):
    rng = np.random.default_rng(5)
    B, H, L, d, nb, R, m = 1, 1, 16, 4, 4, 2, 4
    c = _cfg(B, H, L, d, nb, R, m, False)
    qk = rng.standard_normal((B, H, L, d))
    qk[0, 0, 3] = 0.0
    v = rng.standard_normal((B, H, L, d))
    bk, _ = oracle.hash(c, qk, rng.standard_normal((R, d, nb // 2)))
    pm, _ = oracle.sort(c, bk)
    dqk, dv = oracle.backward(c, qk, v, pm, rng.standard_normal((B, H, L, d)))
    assert np.isfinite(dqk).all() and np.isfinite(dv).all()
