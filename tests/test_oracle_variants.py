"""Pins of the oracle's variant readings (CPU only).

The variants are readings the pages also allow: the window reaching the next
chunk as well, a same-bucket mask inside the window, unit-normalised queries,
and a key counted once when several rounds give it to a query. Each is checked
against a dense L x L formulation written here from its definition (per round
a mask from chunk membership, the self and causal masks and bucket equality;
logits from unit keys and, with the variant, unit queries; the rounds combined
by their logsumexps, or, de-duplicated, one softmax over the union of the
rounds' masks), and against special cases with a known answer.
"""
import math

import numpy as np
import pytest

import oracle
import test_oracle_pins as pins

LA, SB, NQ, DD = oracle.LOOK_AHEAD, oracle.SAME_BUCKET, oracle.NORM_QUERIES, oracle.DEDUP


def _cfg(B, H, L, d, nb, R, m, causal, variant):
    return oracle.config(batch=B, heads=H, seq_len=L, head_dim=d, n_buckets=nb, n_rounds=R,
                         chunk_len=m, causal=int(causal), variant=variant)


def _mask(perm_r, bk_r, m, causal, variant):
    """Attendable (query, key) pairs of one round, from chunk membership."""
    L = perm_r.size
    slot = np.empty(L, np.int64)
    slot[perm_r] = np.arange(L)
    ch = slot // m
    diff = ch[None, :] - ch[:, None]  # key's chunk minus query's chunk
    allowed = (diff == 0) | (diff == -1)
    if variant & LA:
        allowed |= diff == 1
    np.fill_diagonal(allowed, False)
    if causal:
        allowed &= np.tri(L, dtype=bool)
    if variant & SB:
        allowed &= bk_r[None, :] == bk_r[:, None]
    return allowed


def _logits(qk, variant):
    d = qk.shape[1]
    k = qk / np.linalg.norm(qk, axis=1, keepdims=True)
    q = k if variant & NQ else qk
    return q @ k.T / math.sqrt(d)


def _softmax_rows(lg, allowed, v):
    L, d = v.shape
    o = np.empty((L, d))
    lse = np.empty(L)
    for i in range(L):
        if not allowed[i].any():
            o[i] = v[i]
            lse[i] = oracle.SELF_LOGIT
            continue
        mx = lg[i][allowed[i]].max()
        e = np.where(allowed[i], np.exp(lg[i] - mx), 0.0)
        lse[i] = mx + math.log(e.sum())
        o[i] = (e / e.sum()) @ v
    return o, lse


def _dense(qk, v, perm, bk, m, causal, variant):
    """out [L, d] of one (b, h) and, without de-duplication, per-round lse [R, L]."""
    R = perm.shape[0]
    lg = _logits(qk, variant)
    masks = [_mask(perm[r], bk[r], m, causal, variant) for r in range(R)]
    if variant & DD:
        out, _ = _softmax_rows(lg, np.logical_or.reduce(masks), v)
        return out, None
    os_, ls = zip(*[_softmax_rows(lg, al, v) for al in masks])
    ls = np.stack(ls)                              # [R, L]
    w = np.exp(ls - ls.max(axis=0))
    w /= w.sum(axis=0)
    out = np.einsum("rl,rld->ld", w, np.stack(os_))
    return out, ls


VARIANTS = [LA, SB, NQ, DD, LA | DD, SB | DD, LA | SB | NQ | DD]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("variant", VARIANTS)
def test_variant_equals_dense_definition(oracle_lib, variant, causal):
    rng = np.random.default_rng(300 + variant + 16 * int(causal))
    B, H, L, d, nb, R, m = 1, 2, 64, 8, 8, 3, 8
    c = _cfg(B, H, L, d, nb, R, m, causal, variant)
    qk = rng.standard_normal((B, H, L, d))
    v = rng.standard_normal((B, H, L, d))
    res = oracle.forward(c, qk, v, rng.standard_normal((R, d, nb // 2)))
    o, lse = oracle.attend(c, qk, v, res["perm"], res["buckets"])
    for h in range(H):
        want, want_lse = _dense(qk[0, h], v[0, h], res["perm"][0, h], res["buckets"][0, h], m,
                                causal, variant)
        np.testing.assert_allclose(res["out"][0, h], want, rtol=0, atol=1e-12)
        if want_lse is not None:
            np.testing.assert_allclose(lse[0, h], want_lse, rtol=0, atol=1e-12)
    if variant & DD:
        # the rounds with each logit lowered by log N_ij, combined as usual,
        # give the union's attention (the form the GPU computes)
        np.testing.assert_allclose(oracle.combine(c, o, lse), res["out"], rtol=0, atol=1e-12)


def test_look_ahead_over_two_chunks_is_full_attention(oracle_lib):
    """With two chunks, looking both ways every query sees the whole sequence."""
    rng = np.random.default_rng(41)
    B, H, L, d, nb, R = 1, 2, 48, 16, 8, 3
    for causal in (False, True):
        c = _cfg(B, H, L, d, nb, R, L // 2, causal, LA)
        qk = rng.standard_normal((B, H, L, d))
        v = rng.standard_normal((B, H, L, d))
        res = oracle.forward(c, qk, v, rng.standard_normal((R, d, nb // 2)))
        for h in range(H):
            want, want_lse, _ = pins._full_attention_sdpa(qk[0, h], v[0, h], causal)
            np.testing.assert_allclose(res["out"][0, h], want, rtol=0, atol=1e-12)
            for r in range(R):
                np.testing.assert_allclose(res["lse"][0, h, r], want_lse, rtol=0, atol=1e-12)


def test_same_bucket_with_one_bucket_is_the_default(oracle_lib):
    rng = np.random.default_rng(42)
    B, H, L, d, R, m = 1, 2, 64, 8, 2, 8
    qk = rng.standard_normal((B, H, L, d))
    v = rng.standard_normal((B, H, L, d))
    a = oracle.forward(_cfg(B, H, L, d, 1, R, m, True, 0), qk, v, None)
    b = oracle.forward(_cfg(B, H, L, d, 1, R, m, True, SB), qk, v, None)
    np.testing.assert_array_equal(a["out"], b["out"])
    np.testing.assert_array_equal(a["lse"], b["lse"])


def test_normalised_queries_ignore_query_scale(oracle_lib):
    """Scaling a row by c > 0 leaves every output unchanged when queries are
    normalised too (keys are normalised anyway; buckets held fixed), but not
    in the default reading."""
    rng = np.random.default_rng(43)
    B, H, L, d, nb, R, m = 1, 1, 64, 8, 8, 2, 8
    qk = rng.standard_normal((B, H, L, d))
    v = rng.standard_normal((B, H, L, d))
    rot = rng.standard_normal((R, d, nb // 2))
    bk, _ = oracle.hash(_cfg(B, H, L, d, nb, R, m, False, 0), qk, rot)
    scaled = qk.copy()
    scaled[0, 0, ::3] *= 4.0
    for variant, same in ((NQ, True), (0, False)):
        c = _cfg(B, H, L, d, nb, R, m, False, variant)
        a = oracle.forward(c, qk, v, None, buckets_override=bk)["out"]
        b = oracle.forward(c, scaled, v, None, buckets_override=bk)["out"]
        assert np.allclose(a, b, rtol=0, atol=1e-12) == same


def test_dedup_with_identical_rounds_is_one_round(oracle_lib):
    """R copies of one rotation: every pair is shared by all R rounds, so the
    union is one round's window set."""
    rng = np.random.default_rng(44)
    B, H, L, d, nb, m = 1, 2, 128, 8, 8, 8
    qk = rng.standard_normal((B, H, L, d))
    v = rng.standard_normal((B, H, L, d))
    rot1 = rng.standard_normal((1, d, nb // 2))
    for causal in (False, True):
        one = oracle.forward(_cfg(B, H, L, d, nb, 1, m, causal, 0), qk, v, rot1)
        many = oracle.forward(_cfg(B, H, L, d, nb, 4, m, causal, DD), qk, v,
                              np.repeat(rot1, 4, axis=0))
        np.testing.assert_allclose(many["out"], one["out"], rtol=0, atol=1e-14)
        # each per-round logsumexp is lowered by log 4
        for r in range(4):
            sel = one["lse"][:, :, 0] != oracle.SELF_LOGIT
            np.testing.assert_allclose(many["lse"][:, :, r][sel],
                                       one["lse"][:, :, 0][sel] - math.log(4.0), rtol=0,
                                       atol=1e-12)


def test_variant_rows_match_full_forward(oracle_lib):
    rng = np.random.default_rng(45)
    B, H, L, d, nb, R, m = 1, 2, 64, 8, 8, 3, 8
    variant = LA | SB | NQ | DD
    c = _cfg(B, H, L, d, nb, R, m, True, variant)
    qk = rng.standard_normal((B, H, L, d))
    v = rng.standard_normal((B, H, L, d))
    res = oracle.forward(c, qk, v, rng.standard_normal((R, d, nb // 2)))
    rows = np.array([0, 5, 63, 64, 100, 127])
    out, lse = oracle.attend_rows(c, qk, v, res["perm"], rows, res["buckets"])
    np.testing.assert_allclose(out, res["out"].reshape(-1, d)[rows], rtol=0, atol=1e-14)
    bh, i = rows // L, rows % L
    np.testing.assert_allclose(lse, res["lse"].reshape(B * H, R, L)[bh, :, i], rtol=0,
                               atol=1e-14)


def test_same_bucket_backward_rejects_missing_buckets(oracle_lib):
    """The variant backward is pinned in test_oracle_backward.py; here only
    that the same-bucket reading refuses to run without the bucket ids."""
    c = _cfg(1, 1, 16, 4, 4, 1, 4, False, SB)
    z = np.zeros((1, 1, 16, 4))
    pm = np.tile(np.arange(16, dtype=np.int32), (1, 1, 1, 1))
    with pytest.raises(ValueError):
        oracle.backward(c, z, z, pm, z)
