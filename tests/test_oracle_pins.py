"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these tests re-types the oracle's own formulas: each compares it with
a hand-worked fixture, a library routine that the method reduces to in a
special case, a closed form, or an invariant. A plausible slip in the oracle
(a dropped term, a wrong sign or index, a transposed operand, a wrong
look-back, wrong round weights) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cfg(B, H, L, d, nb, R, m, causal):
    return oracle.config(batch=B, heads=H, seq_len=L, head_dim=d, n_buckets=nb, n_rounds=R,
                         chunk_len=m, causal=int(causal))


# ---------------------------------------------------------------------------
# Hash: hand-worked examples (section on LSH of the p2.ttnews.xyz summary)
# ---------------------------------------------------------------------------
def test_hash_hand_worked_examples(oracle_lib):
    with open(os.path.join(GOLDEN, "hash_examples.json")) as f:
        fx = json.load(f)
    for case in fx["cases"]:
        x = np.array(case["x"], np.float64)
        Rm = np.array(case["R"], np.float64)
        d = x.size
        assert Rm.shape == (d, case["n_buckets"] // 2)
        c = _cfg(1, 1, 1, d, case["n_buckets"], 1, 1, False)
        bk, mg = oracle.hash(c, x.reshape(1, 1, 1, d), Rm.reshape(1, *Rm.shape))
        assert int(bk.ravel()[0]) == case["bucket"], case["work"]
        assert mg.ravel()[0] == pytest.approx(case["margin"], abs=1e-15), case["work"]


def test_hash_signed_permutation_closed_form(oracle_lib):
    """R[t][k] = s_k if t == pi(k) else 0 gives xR = (s_k x_pi(k)); the bucket is
    the k with the largest |x_pi(k)|, shifted by b/2 when s_k x_pi(k) < 0.
    d != b/2 so a transposed R or swapped strides gives other answers."""
    rng = np.random.default_rng(7)
    d, half = 11, 5
    L = 200
    pi = rng.permutation(d)[:half]
    s = rng.choice([-1.0, 1.0], size=half)
    Rm = np.zeros((d, half))
    Rm[pi, np.arange(half)] = s
    x = rng.standard_normal((L, d))
    c = _cfg(1, 1, L, d, 2 * half, 1, 1, False)
    bk, mg = oracle.hash(c, x.reshape(1, 1, L, d), Rm.reshape(1, d, half))
    vals = s[None, :] * x[:, pi]                      # (L, half)
    kstar = np.abs(vals).argmax(axis=1)
    want = np.where(vals[np.arange(L), kstar] > 0, kstar, kstar + half)
    np.testing.assert_array_equal(bk.ravel(), want)
    srt = np.sort(np.abs(vals), axis=1)
    np.testing.assert_allclose(mg.ravel(), srt[:, -1] - srt[:, -2], rtol=0, atol=1e-15)


def test_hash_rescale_invariance(oracle_lib):
    """h(c x) = h(x) for c > 0: bit-exact for c = 2^k (scaling is exact in fp64),
    and for general c wherever the decision is not a near-tie."""
    rng = np.random.default_rng(11)
    B, H, L, d, nb, R = 2, 3, 64, 16, 32, 3
    x = rng.standard_normal((B, H, L, d))
    rot = rng.standard_normal((R, d, nb // 2))
    c = _cfg(B, H, L, d, nb, R, 64, False)
    b0, m0 = oracle.hash(c, x, rot)
    for k in (-6, -1, 1, 5):
        bk, mg = oracle.hash(c, x * 2.0 ** k, rot)
        np.testing.assert_array_equal(bk, b0)
        np.testing.assert_array_equal(mg, m0 * 2.0 ** k)
    for cc in (0.37, 3.9, 1234.5):
        bk, _ = oracle.hash(c, x * cc, rot)
        ok = m0 > 1e-9
        np.testing.assert_array_equal(bk[ok], b0[ok])


def test_hash_antipodal(oracle_lib):
    """[(-x)R; -(-x)R] is [xR; -xR] with its halves swapped, so h(-x) = h(x) +- b/2."""
    rng = np.random.default_rng(12)
    B, H, L, d, nb, R = 1, 2, 100, 8, 12, 2
    x = rng.standard_normal((B, H, L, d))
    rot = rng.standard_normal((R, d, nb // 2))
    c = _cfg(B, H, L, d, nb, R, 4, False)
    b0, m0 = oracle.hash(c, x, rot)
    b1, m1 = oracle.hash(c, -x, rot)
    np.testing.assert_array_equal(b1, (b0 + nb // 2) % nb)
    np.testing.assert_array_equal(m1, m0)


def _pair_rates(theta, nb, n_draws, d=8, seed=0):
    """Fraction of independent rotations under which two unit vectors at angle
    theta share a bucket. Rounds are the independent draws."""
    rng = np.random.default_rng(seed)
    u = np.zeros(d); u[0] = 1.0
    w = np.zeros(d); w[0] = math.cos(theta); w[1] = math.sin(theta)
    x = np.stack([u, w]).reshape(1, 1, 2, d)
    rot = rng.standard_normal((n_draws, d, max(nb // 2, 1)))
    c = _cfg(1, 1, 2, d, nb, n_draws, 1, False)
    bk, _ = oracle.hash(c, x, rot)
    bk = bk.reshape(n_draws, 2)
    return float(np.mean(bk[:, 0] == bk[:, 1]))


def test_hash_collision_law_two_buckets(oracle_lib):
    """With b = 2 the hash is one sign bit sign(x.r); two vectors at angle theta
    agree with probability 1 - theta/pi (the random-hyperplane law the 2kiu.com
    page states for its sign-bit hash, section 2.2)."""
    n = 40000
    for theta in (math.pi / 6, math.pi / 3, math.pi / 2, 2 * math.pi / 3, 5 * math.pi / 6):
        p = 1.0 - theta / math.pi
        rate = _pair_rates(theta, 2, n, seed=int(theta * 1000))
        sigma = math.sqrt(p * (1 - p) / n)
        assert abs(rate - p) < 4.5 * sigma, (theta, rate, p)


def test_hash_collisions_fall_with_angle(oracle_lib):
    """Nearby vectors share a bucket more often than distant ones (LSH section of
    the p2.ttnews.xyz summary). theta = 0 always collides, theta = pi never does,
    and the rate does not rise along a 13-point angle grid."""
    n = 6000
    nb = 16
    thetas = np.linspace(0.0, math.pi, 13)
    rates = [_pair_rates(t, nb, n, seed=100 + k) for k, t in enumerate(thetas)]
    assert rates[0] == 1.0
    assert rates[-1] == 0.0
    for a, b in zip(rates, rates[1:]):
        tol = 4.5 * math.sqrt(max(a * (1 - a), 1.0 / n) / n)
        assert b <= a + tol, rates
    assert rates[3] < rates[1] < 1.0


# ---------------------------------------------------------------------------
# Sort: stable permutation (LSH attention section: bucket, then position)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("nb,skew", [(4, False), (64, False), (64, True), (1, False)])
def test_sort_is_the_stable_bucket_order(oracle_lib, nb, skew):
    rng = np.random.default_rng(nb + int(skew))
    B, H, R, L = 2, 2, 3, 512
    if skew:
        p = rng.dirichlet(np.full(nb, 0.05))
        bk = rng.choice(nb, size=(B, H, R, L), p=p).astype(np.int32)
    else:
        bk = rng.integers(0, nb, size=(B, H, R, L)).astype(np.int32)
    c = _cfg(B, H, L, 4, nb, R, 8, False)
    perm, inv = oracle.sort(c, bk)
    flat_b = bk.reshape(-1, L)
    flat_p = perm.reshape(-1, L)
    flat_i = inv.reshape(-1, L)
    for s in range(flat_b.shape[0]):
        pm = flat_p[s]
        np.testing.assert_array_equal(np.sort(pm), np.arange(L))          # bijection
        np.testing.assert_array_equal(flat_i[s][pm], np.arange(L))          # inv o perm = id
        bs = flat_b[s][pm]
        assert np.all(np.diff(bs) >= 0)                                     # buckets ascend
        same = np.diff(bs) == 0
        assert np.all(np.diff(pm)[same] > 0)                                # positions ascend
        np.testing.assert_array_equal(pm, np.argsort(flat_b[s], kind="stable"))  # library sort


# ---------------------------------------------------------------------------
# Windows and masks: hand-enumerated example (L = 8, m = 2, two rounds)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_windows_hand_enumerated(oracle_lib, causal):
    with open(os.path.join(GOLDEN, "windows_L8_m2.json")) as f:
        fx = json.load(f)
    L, m, nb = fx["seq_len"], fx["chunk_len"], fx["n_buckets"]
    rounds = fx["rounds"]
    R = len(rounds)
    d = L
    # zero queries/keys make every logit 0, so each round's output is the mean of
    # the attendable values; one-hot values reveal exactly which keys were used.
    qk = np.zeros((1, 1, L, d))
    v = np.eye(L).reshape(1, 1, L, d)
    bk = np.array([r["buckets"] for r in rounds], np.int32).reshape(1, 1, R, L)
    c = _cfg(1, 1, L, d, nb, R, m, causal)
    perm, _ = oracle.sort(c, bk)
    np.testing.assert_array_equal(perm.reshape(R, L), np.array([r["perm"] for r in rounds]))
    o, lse = oracle.attend(c, qk, v, perm)
    res = oracle.forward(c, qk, v, None, buckets_override=bk)
    key = "others_causal" if causal else "others_noncausal"
    for r, rd in enumerate(rounds):
        for i in range(L):
            others = rd[key][str(i)]
            want = np.zeros(d)
            if others:
                want[others] = 1.0 / len(others)
                assert lse[0, 0, r, i] == pytest.approx(math.log(len(others)), abs=1e-14)
            else:
                want[i] = 1.0
                assert lse[0, 0, r, i] == oracle.SELF_LOGIT
            np.testing.assert_allclose(o[0, 0, r, i], want, rtol=0, atol=1e-15)
    # combined: one softmax over the multiset union of the rounds' attendable keys
    for i in range(L):
        counts = np.zeros(d)
        for rd in rounds:
            for j in rd[key][str(i)]:
                counts[j] += 1
        want = counts / counts.sum() if counts.sum() > 0 else np.eye(L)[i]
        np.testing.assert_allclose(res["out"][0, 0, i], want, rtol=0, atol=1e-15)


# ---------------------------------------------------------------------------
# Whole path: one chunk covering the sequence reduces to full attention
# ---------------------------------------------------------------------------
def _full_attention_sdpa(qk, v, causal):
    """Shared-QK full softmax attention with unit keys and the self-mask, via
    torch's scaled_dot_product_attention in float64 (a library routine)."""
    L, d = qk.shape
    q = torch.from_numpy(qk)
    k = q / q.norm(dim=-1, keepdim=True)
    allowed = ~torch.eye(L, dtype=torch.bool)
    if causal:
        allowed &= torch.ones(L, L, dtype=torch.bool).tril()
    empty = ~allowed.any(dim=1)
    allowed_sdpa = allowed | (empty[:, None] & torch.eye(L, dtype=torch.bool))
    out = F.scaled_dot_product_attention(q[None, None], k[None, None],
                                         torch.from_numpy(v)[None, None],
                                         attn_mask=allowed_sdpa[None, None],
                                         scale=1.0 / math.sqrt(d))[0, 0]
    logits = (q @ k.T) / math.sqrt(d)
    lse = torch.logsumexp(logits.masked_fill(~allowed, -math.inf), dim=1)
    lse[empty] = oracle.SELF_LOGIT
    return out.numpy(), lse.numpy(), empty.numpy()


@pytest.mark.parametrize("nb,R,causal", [(1, 1, False), (1, 1, True), (8, 3, False),
                                         (8, 3, True), (2, 2, True), (32, 1, False)])
def test_single_chunk_equals_full_attention(oracle_lib, nb, R, causal):
    rng = np.random.default_rng(100 + nb + R + int(causal))
    B, H, L, d = 2, 2, 48, 16
    qk = rng.standard_normal((B, H, L, d))
    v = rng.standard_normal((B, H, L, d))
    rot = rng.standard_normal((R, d, nb // 2)) if nb > 1 else None
    c = _cfg(B, H, L, d, nb, R, L, causal)
    res = oracle.forward(c, qk, v, rot)
    for b in range(B):
        for h in range(H):
            want, want_lse, empty = _full_attention_sdpa(qk[b, h], v[b, h], causal)
            np.testing.assert_allclose(res["out"][b, h], want, rtol=0, atol=1e-12)
            for r in range(R):
                np.testing.assert_allclose(res["lse"][b, h, r], want_lse, rtol=0, atol=1e-12)
            if causal:
                assert empty[0] and not empty[1:].any()
                # every round is self-only at position 0: weights 1/R each
                np.testing.assert_allclose(res["out"][b, h, 0], v[b, h, 0], rtol=1e-15,
                                           atol=1e-15)


# ---------------------------------------------------------------------------
# Windows on random data: dense masked softmax, and the multiset-union identity
# ---------------------------------------------------------------------------
def _dense_round(qk, v, perm, m, causal):
    """One round written as a dense L x L mask built from chunk membership."""
    L, d = qk.shape
    slot = np.empty(L, np.int64)
    slot[perm] = np.arange(L)
    ch = slot // m
    allowed = (ch[None, :] == ch[:, None]) | (ch[None, :] == ch[:, None] - 1)
    np.fill_diagonal(allowed, False)
    if causal:
        allowed &= np.tri(L, dtype=bool)
    k = qk / np.linalg.norm(qk, axis=1, keepdims=True)
    logits = np.where(allowed, qk @ k.T / math.sqrt(d), -np.inf)
    o = np.empty((L, d))
    lse = np.empty(L)
    for i in range(L):
        if not allowed[i].any():
            o[i] = v[i]
            lse[i] = oracle.SELF_LOGIT
            continue
        mx = logits[i].max()
        e = np.exp(logits[i] - mx)
        lse[i] = mx + math.log(e.sum())
        o[i] = (e / e.sum()) @ v
    return o, lse, allowed, logits


@pytest.mark.parametrize("causal", [False, True])
def test_dense_mask_and_multiset_union(oracle_lib, causal):
    rng = np.random.default_rng(5 + int(causal))
    B, H, L, d, nb, R, m = 1, 2, 64, 8, 8, 3, 8
    qk = rng.standard_normal((B, H, L, d))
    v = rng.standard_normal((B, H, L, d))
    rot = rng.standard_normal((R, d, nb // 2))
    c = _cfg(B, H, L, d, nb, R, m, causal)
    res = oracle.forward(c, qk, v, rot)
    o, lse = oracle.attend(c, qk, v, res["perm"])
    for h in range(H):
        union_logits = []
        union_allowed = []
        for r in range(R):
            od, ld, al, lg = _dense_round(qk[0, h], v[0, h], res["perm"][0, h, r], m, causal)
            np.testing.assert_allclose(o[0, h, r], od, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[0, h, r], ld, rtol=0, atol=1e-12)
            union_logits.append(lg)
            union_allowed.append(al)
        # one softmax over the multiset union of the rounds' windows
        lg = np.concatenate(union_logits, axis=1)            # (L, R*L)
        al = np.concatenate(union_allowed, axis=1)
        vv = np.concatenate([v[0, h]] * R, axis=0)           # (R*L, d)
        for i in range(L):
            if not al[i].any():
                np.testing.assert_allclose(res["out"][0, h, i], v[0, h, i], rtol=0, atol=1e-14)
                continue
            mx = lg[i][al[i]].max()
            e = np.where(al[i], np.exp(lg[i] - mx), 0.0)
            want = (e / e.sum()) @ vv
            np.testing.assert_allclose(res["out"][0, h, i], want, rtol=0, atol=1e-12)


def test_identical_rounds_collapse(oracle_lib):
    """R copies of one rotation give R identical rounds: every lse_r agrees and
    the combined output equals the single-round output."""
    rng = np.random.default_rng(21)
    B, H, L, d, nb, m = 1, 2, 256, 16, 16, 16
    qk = rng.standard_normal((B, H, L, d))
    v = rng.standard_normal((B, H, L, d))
    rot1 = rng.standard_normal((1, d, nb // 2))
    for causal in (False, True):
        one = oracle.forward(_cfg(B, H, L, d, nb, 1, m, causal), qk, v, rot1)
        many = oracle.forward(_cfg(B, H, L, d, nb, 4, m, causal), qk, v,
                              np.repeat(rot1, 4, axis=0))
        for r in range(4):
            np.testing.assert_array_equal(many["lse"][:, :, r], one["lse"][:, :, 0])
            np.testing.assert_array_equal(many["perm"][:, :, r], one["perm"][:, :, 0])
        np.testing.assert_allclose(many["out"], one["out"], rtol=0, atol=1e-14)


def test_self_only_rows_return_their_value(oracle_lib):
    """Causal position 0 has nothing but itself in every round: out = v_0 and
    every round's lse is the self-logit constant."""
    rng = np.random.default_rng(3)
    B, H, L, d, nb, R, m = 2, 2, 128, 8, 8, 1, 8
    qk = rng.standard_normal((B, H, L, d))
    v = rng.standard_normal((B, H, L, d))
    rot = rng.standard_normal((R, d, nb // 2))
    res = oracle.forward(_cfg(B, H, L, d, nb, R, m, True), qk, v, rot)
    np.testing.assert_array_equal(res["out"][:, :, 0], v[:, :, 0])
    assert np.all(res["lse"][:, :, :, 0] == oracle.SELF_LOGIT)


def test_attend_rows_matches_full_forward(oracle_lib):
    """The sampled-rows entry point is the same definition restricted to a few
    positions (used for parity at sizes where the full oracle is too slow)."""
    w = workloads.get("c4k").with_(batch=1, heads=2, seq_len=512)
    inp = workloads.make_inputs(w)
    c = oracle.config(w)
    res = oracle.forward(c, inp.qk, inp.v, inp.rotations)
    rng = np.random.default_rng(0)
    rows = rng.choice(w.batch * w.heads * w.seq_len, size=50, replace=False)
    out_rows, lse_rows = oracle.attend_rows(c, inp.qk, inp.v, res["perm"], rows)
    flat_out = res["out"].reshape(-1, w.head_dim)
    np.testing.assert_array_equal(out_rows, flat_out[rows])
    bh, i = rows // w.seq_len, rows % w.seq_len
    lse = res["lse"].reshape(w.batch * w.heads, w.n_rounds, w.seq_len)
    np.testing.assert_array_equal(lse_rows, lse[bh, :, i])


def test_bad_configs_are_rejected(oracle_lib):
    for kw in (dict(seq_len=100, chunk_len=64), dict(n_buckets=3), dict(n_rounds=0),
               dict(causal=2), dict(head_dim=0)):
        base = dict(batch=1, heads=1, seq_len=128, head_dim=8, n_buckets=4, n_rounds=1,
                    chunk_len=64, causal=0)
        base.update(kw)
        with pytest.raises(ValueError):
            oracle.hash(oracle.config(**base), np.zeros((1, 1, base["seq_len"], 8)),
                        np.zeros((1, 8, 2)))


# ---------------------------------------------------------------------------
# Projections (shared-QK section of the p2.ttnews.xyz summary): one linear map
# for queries/keys, one for values
# ---------------------------------------------------------------------------
def test_projection_equals_library_matmul(oracle_lib):
    rng = np.random.default_rng(51)
    B, H, L, d, dm = 2, 3, 16, 8, 40
    c = _cfg(B, H, L, d, 4, 1, 4, False)
    x = rng.standard_normal((B, L, dm))
    wq = rng.standard_normal((H * d, dm))
    wv = rng.standard_normal((H * d, dm))
    qk, v = oracle.project(c, x, wq, wv)
    # numpy's matmul, then split the features into heads
    want_q = (x @ wq.T).reshape(B, L, H, d).transpose(0, 2, 1, 3)
    want_v = (x @ wv.T).reshape(B, L, H, d).transpose(0, 2, 1, 3)
    np.testing.assert_allclose(qk, want_q, rtol=0, atol=1e-12)
    np.testing.assert_allclose(v, want_v, rtol=0, atol=1e-12)


def test_projection_with_selection_weights_copies_the_input(oracle_lib):
    """Weights that pick input feature h*d + e for output (h, e) give x itself,
    split into heads, exactly; swapping the two weights swaps the outputs."""
    rng = np.random.default_rng(52)
    B, H, L, d = 1, 2, 8, 4
    dm = H * d
    c = _cfg(B, H, L, d, 4, 1, 4, False)
    x = rng.standard_normal((B, L, dm))
    eye = np.eye(dm)
    qk, v = oracle.project(c, x, eye, 2.0 * eye)
    want = x.reshape(B, L, H, d).transpose(0, 2, 1, 3)
    np.testing.assert_array_equal(qk, want)
    np.testing.assert_array_equal(v, 2.0 * want)
