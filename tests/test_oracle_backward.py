"""Pins of the oracle's backward (gradients at fixed buckets), CPU only.

The backward is the chain rule through the forward's steps; these tests check
it against things that do not share its formulas:
  * central finite differences of the oracle's own forward (buckets held
    fixed through buckets_override), element by element, on small inputs that
    span several chunks, several rounds, the causal and the plain mask, and
    queries that see only themselves;
  * for one bucket and one chunk covering the sequence, PyTorch fp64 autograd
    of dense shared-QK attention with unit keys and the self-mask, a separate
    formulation (the forward of that case is pinned to SDPA); with unit
    queries too for NORM_QUERIES.
The variant readings (look-ahead, same-bucket, unit queries, de-duplication
and their combinations) are pinned the same way, by finite differences of the
forward of that reading (DEDUP's forward takes the union of the rounds' key
sets directly), and DEDUP also by identical rounds reducing to one round.
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


def _mag_case(seed, causal, R=3, m=4, L=24, d=6, nb=6):
    rng = np.random.default_rng(seed)
    c = _cfg(1, 2, L, d, nb, R, m, causal)
    qk = rng.standard_normal((1, 2, L, d))
    v = rng.standard_normal((1, 2, L, d))
    rot = rng.standard_normal((R, d, nb // 2))
    bk, _ = oracle.hash(c, qk, rot)
    pm, _ = oracle.sort(c, bk)
    dout = rng.standard_normal((1, 2, L, d))
    return c, qk, v, pm, dout


@pytest.mark.parametrize("causal", [False, True])
def test_backward_magnitudes_bound_the_gradients(oracle_lib, causal):
    """Each magnitude is a sum of upper bounds of the absolute values of the
    gradient's terms, so it bounds the gradient elementwise; for dv, whose
    terms are w P dout, it equals |dv| exactly when dout and v are
    non-negative (every term then has the same sign)."""
    c, qk, v, pm, dout = _mag_case(3 + int(causal), causal)
    dqk, dv = oracle.backward(c, qk, v, pm, dout)
    mq, mv = oracle.backward_magnitudes(c, qk, v, pm, dout)
    assert np.all(np.abs(dqk) <= mq * (1 + 1e-12) + 1e-300)
    assert np.all(np.abs(dv) <= mv * (1 + 1e-12) + 1e-300)
    # strictly larger somewhere: the bound is not the gradient itself
    assert np.any(mq > np.abs(dqk) * 1.5)
    _, dvp = oracle.backward(c, qk, np.abs(v), pm, np.abs(dout))
    _, mvp = oracle.backward_magnitudes(c, qk, np.abs(v), pm, np.abs(dout))
    np.testing.assert_allclose(mvp, dvp, rtol=1e-12, atol=0)


def test_backward_magnitudes_scale_with_dout(oracle_lib):
    """Positive homogeneity in dout: every term is linear in dout."""
    c, qk, v, pm, dout = _mag_case(11, True)
    mq, mv = oracle.backward_magnitudes(c, qk, v, pm, dout)
    mq2, mv2 = oracle.backward_magnitudes(c, qk, v, pm, -4.0 * dout)
    np.testing.assert_allclose(mq2, 4.0 * mq, rtol=1e-12, atol=0)
    np.testing.assert_allclose(mv2, 4.0 * mv, rtol=1e-12, atol=0)


def test_backward_magnitudes_of_one_key_window(oracle_lib):
    """A hand case: L = 2, one chunk of 2, causal. Position 0 sees only itself
    (dv_0 gets w dout_0 = dout_0: one round), position 1 attends only to key 0
    with P = 1, so dS = dout_1.v_0 - dout_1.out_1 = 0 (out_1 = v_0) and the
    magnitude of that term is |dout_1.v_0| + |dout_1.v_0| + 2 |dout_1.v_0|."""
    c = _cfg(1, 1, 2, 2, 1, 1, 2, True)
    qk = np.array([[[[3.0, 4.0], [1.0, 0.0]]]])
    v = np.array([[[[1.0, -2.0], [5.0, 7.0]]]])
    dout = np.array([[[[0.5, -1.0], [2.0, 3.0]]]])
    pm = np.array([[[[0, 1]]]], dtype=np.int32)
    mq, mv = oracle.backward_magnitudes(c, qk, v, pm, dout)
    dv1 = abs(2.0 * 1.0 + 3.0 * -2.0)        # |dout_1 . v_0| = 4
    A = 4.0 * dv1                             # 16
    khat0 = np.array([0.6, 0.8])
    # dv: key 0 gets |dout_1| (P = 1, w = 1) plus its own self-only |dout_0|
    np.testing.assert_allclose(mv[0, 0, 0], np.abs(dout[0, 0, 1]) + np.abs(dout[0, 0, 0]))
    np.testing.assert_allclose(mv[0, 0, 1], [0.0, 0.0])
    # dq of query 1: A |khat_0| / sqrt(2)
    np.testing.assert_allclose(mq[0, 0, 1], A * khat0 / math.sqrt(2), rtol=1e-14)
    # dkhat of key 0: A |q_1| / sqrt(2), then the Jacobian in absolute value
    mk = A * np.array([1.0, 0.0]) / math.sqrt(2)
    np.testing.assert_allclose(mq[0, 0, 0], (mk + khat0 * (khat0 @ mk)) / 5.0, rtol=1e-14)


# ---------------------------------------------------------------------------
# Variant readings: the same pins (finite differences of the oracle's own
# forward of that reading, which for DEDUP takes the union of the rounds' key
# sets directly, a separate formulation from the backward's per-round terms)

LA, SB, NQ, DD = oracle.LOOK_AHEAD, oracle.SAME_BUCKET, oracle.NORM_QUERIES, oracle.DEDUP
VARIANTS = [LA, SB, NQ, DD, LA | DD, SB | DD, LA | SB | NQ | DD]


def _vcfg(L, d, nb, R, m, causal, variant, H=2):
    return oracle.config(batch=1, heads=H, seq_len=L, head_dim=d, n_buckets=nb, n_rounds=R,
                         chunk_len=m, causal=int(causal), variant=variant)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("causal", [False, True])
def test_variant_backward_matches_finite_differences(oracle_lib, variant, causal):
    rng = np.random.default_rng(100 + variant + 17 * int(causal))
    L, d, nb, R, m = 16, 4, 4, 2, 4
    c = _vcfg(L, d, nb, R, m, causal, variant)
    qk = rng.standard_normal((1, 2, L, d))
    v = rng.standard_normal((1, 2, L, d))
    bk, _ = oracle.hash(c, qk, rng.standard_normal((R, d, nb // 2)))
    pm, _ = oracle.sort(c, bk)
    dout = rng.standard_normal((1, 2, L, d))
    dqk, dv = oracle.backward(c, qk, v, pm, dout, buckets=bk)
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


def _dense_grads_unit_queries(qk, v, dout, causal):
    """Dense shared-QK attention with unit queries and unit keys and the
    self-mask, differentiated by torch autograd in float64."""
    L, d = qk.shape
    q = torch.tensor(qk, requires_grad=True)
    vv = torch.tensor(v, requires_grad=True)
    k = q / q.norm(dim=-1, keepdim=True)
    allowed = ~torch.eye(L, dtype=torch.bool)
    if causal:
        allowed &= torch.ones(L, L, dtype=torch.bool).tril()
    empty = ~allowed.any(dim=1)
    logits = (k @ k.T) / math.sqrt(d)
    p = torch.softmax(logits.masked_fill(~allowed, -math.inf).masked_fill(empty[:, None], 0.0),
                      dim=1)
    out = torch.where(empty[:, None], vv, p @ vv)
    (out * torch.tensor(dout)).sum().backward()
    return q.grad.numpy(), vv.grad.numpy()


@pytest.mark.parametrize("causal", [False, True])
def test_unit_query_backward_single_chunk_equals_dense_autograd(oracle_lib, causal):
    rng = np.random.default_rng(40 + int(causal))
    L, d = 20, 6
    c = _vcfg(L, d, 1, 2, L, causal, NQ)
    qk = rng.standard_normal((1, 2, L, d))
    v = rng.standard_normal((1, 2, L, d))
    dout = rng.standard_normal((1, 2, L, d))
    pm = oracle.forward(c, qk, v, None)["perm"]
    dqk, dv = oracle.backward(c, qk, v, pm, dout)
    for h in range(2):
        gq, gv = _dense_grads_unit_queries(qk[0, h], v[0, h], dout[0, h], causal)
        np.testing.assert_allclose(dqk[0, h], gq, rtol=0, atol=1e-12)
        np.testing.assert_allclose(dv[0, h], gv, rtol=0, atol=1e-12)


def test_dedup_backward_of_identical_rounds_equals_one_round(oracle_lib):
    """With R rounds of the same buckets every pair is shared by all R rounds,
    so DEDUP's union is one round's key set and its gradients equal those of
    a single round of the default reading."""
    rng = np.random.default_rng(8)
    L, d, nb, m = 24, 5, 6, 4
    c1 = _vcfg(L, d, nb, 1, m, True, 0)
    c3 = _vcfg(L, d, nb, 3, m, True, DD)
    qk = rng.standard_normal((1, 2, L, d))
    v = rng.standard_normal((1, 2, L, d))
    dout = rng.standard_normal((1, 2, L, d))
    bk1, _ = oracle.hash(c1, qk, rng.standard_normal((1, d, nb // 2)))
    bk3 = np.repeat(bk1, 3, axis=2)
    pm1, _ = oracle.sort(c1, bk1)
    pm3, _ = oracle.sort(c3, bk3)
    g1 = oracle.backward(c1, qk, v, pm1, dout)
    g3 = oracle.backward(c3, qk, v, pm3, dout, buckets=bk3)
    for a, b in zip(g1, g3):
        np.testing.assert_allclose(b, a, rtol=0, atol=1e-12)


@pytest.mark.parametrize("variant", VARIANTS)
def test_variant_backward_magnitudes_bound_the_gradients(oracle_lib, variant):
    rng = np.random.default_rng(60 + variant)
    L, d, nb, R, m = 24, 6, 6, 3, 4
    c = _vcfg(L, d, nb, R, m, True, variant)
    qk = rng.standard_normal((1, 2, L, d))
    v = rng.standard_normal((1, 2, L, d))
    bk, _ = oracle.hash(c, qk, rng.standard_normal((R, d, nb // 2)))
    pm, _ = oracle.sort(c, bk)
    dout = rng.standard_normal((1, 2, L, d))
    dqk, dv = oracle.backward(c, qk, v, pm, dout, buckets=bk)
    mq, mv = oracle.backward_magnitudes(c, qk, v, pm, dout, buckets=bk)
    assert np.all(np.abs(dqk) <= mq * (1 + 1e-12) + 1e-300)
    assert np.all(np.abs(dv) <= mv * (1 + 1e-12) + 1e-300)
    _, dvp = oracle.backward(c, qk, np.abs(v), pm, np.abs(dout), buckets=bk)
    _, mvp = oracle.backward_magnitudes(c, qk, np.abs(v), pm, np.abs(dout), buckets=bk)
    np.testing.assert_allclose(mvp, dvp, rtol=1e-12, atol=0)


def test_same_bucket_backward_needs_buckets(oracle_lib):
    c = _vcfg(8, 2, 2, 1, 4, False, SB, H=1)
    z = np.zeros((1, 1, 8, 2))
    pm = np.tile(np.arange(8, dtype=np.int32), (1, 1, 1, 1))
    with pytest.raises(ValueError):
        oracle.backward(c, z, z, pm, z)
