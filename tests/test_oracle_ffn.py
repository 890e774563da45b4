"""Pins of the oracle's chunked feed-forward (CPU only).

The layer is the second half of the reversible block, y2 = x2 + FF(y1), with
FF the two-layer feed-forward (biases, ReLU between the layers) applied to
chunks of rows whose outputs are concatenated. Each pin below has an answer
fixed without the formula: weight matrices built so that the result is known
exactly (the input itself through relu(a) - relu(-a) = a, its positive part,
a bias picked out by a selection matrix), the positive homogeneity of ReLU,
and the independence of every row from the chunk it falls in.
"""
import numpy as np
import pytest

import oracle


def _perm_matrix(rng, n):
    p = np.zeros((n, n))
    p[np.arange(n), rng.permutation(n)] = 1.0
    return p


def _split_identity(rng, d):
    """W1 = [S P; -S P] and W2 = [P^T S^-1, -P^T S^-1] with P a permutation and
    S a diagonal of powers of two: FF(y) = relu(S P y) - relu(-S P y) mapped
    back, which is y exactly."""
    P = _perm_matrix(rng, d)
    S = np.diag(2.0 ** rng.integers(-3, 4, d))
    w1 = np.vstack([S @ P, -(S @ P)])                   # [2d, d]
    w2 = np.hstack([P.T @ np.linalg.inv(S), -(P.T @ np.linalg.inv(S))])  # [d, 2d]
    return w1, w2


def test_ffn_split_identity_returns_the_input(oracle_lib):
    rng = np.random.default_rng(61)
    rows, d = 37, 12
    y = rng.standard_normal((rows, d))
    w1, w2 = _split_identity(rng, d)
    y2, hid = oracle.ffn(y, w1, np.zeros(2 * d), w2, np.zeros(d), chunk_rows=8,
                         return_hidden=True)
    np.testing.assert_array_equal(y2, y)
    # the hidden layer holds the positive and negative parts of S P y
    sp = y @ w1[:d].T
    np.testing.assert_array_equal(hid, np.hstack([np.maximum(sp, 0), np.maximum(-sp, 0)]))


def test_ffn_half_of_the_split_is_the_positive_part(oracle_lib):
    rng = np.random.default_rng(62)
    rows, d = 21, 8
    y = rng.standard_normal((rows, d))
    w1, w2 = _split_identity(rng, d)
    w2[:, d:] = 0.0
    y2 = oracle.ffn(y, w1, np.zeros(2 * d), w2, np.zeros(d))
    np.testing.assert_array_equal(y2, np.maximum(y, 0.0))


def test_ffn_biases_through_selection_weights(oracle_lib):
    """W1 = 0: the hidden layer is relu(b1) for every row; W2 picks hidden unit
    sel[e] for output e, so y2[i, e] = relu(b1[sel[e]]) + b2[e] (+ x2)."""
    rng = np.random.default_rng(63)
    rows, d, dff = 9, 6, 24
    b1 = rng.integers(-4, 5, dff).astype(np.float64)
    b2 = rng.integers(-4, 5, d).astype(np.float64)
    sel = rng.choice(dff, size=d, replace=False)
    w2 = np.zeros((d, dff))
    w2[np.arange(d), sel] = 1.0
    y = rng.standard_normal((rows, d))
    want = np.broadcast_to(np.maximum(b1[sel], 0.0) + b2, (rows, d))
    np.testing.assert_array_equal(oracle.ffn(y, np.zeros((dff, d)), b1, w2, b2), want)
    x2 = rng.integers(-8, 9, (rows, d)).astype(np.float64)
    np.testing.assert_array_equal(oracle.ffn(y, np.zeros((dff, d)), b1, w2, b2, x2=x2),
                                  want + x2)


def test_ffn_residual_is_added(oracle_lib):
    """With the split identity and integer inputs every sum is exact: y2 = y1 + x2."""
    rng = np.random.default_rng(64)
    rows, d = 17, 10
    y = rng.integers(-50, 51, (rows, d)).astype(np.float64)
    x2 = rng.integers(-50, 51, (rows, d)).astype(np.float64)
    w1, w2 = _split_identity(rng, d)
    np.testing.assert_array_equal(
        oracle.ffn(y, w1, np.zeros(2 * d), w2, np.zeros(d), x2=x2, chunk_rows=4), y + x2)


def test_ffn_positive_homogeneity(oracle_lib):
    """Without biases, FF(2 y) = 2 FF(y) exactly (ReLU commutes with positive
    scaling, and scaling by 2 is exact)."""
    rng = np.random.default_rng(65)
    rows, d, dff = 13, 8, 32
    y = rng.standard_normal((rows, d))
    w1 = rng.standard_normal((dff, d))
    w2 = rng.standard_normal((d, dff))
    z1, z2 = np.zeros(dff), np.zeros(d)
    np.testing.assert_array_equal(oracle.ffn(2.0 * y, w1, z1, w2, z2),
                                  2.0 * oracle.ffn(y, w1, z1, w2, z2))


@pytest.mark.parametrize("chunk", [1, 3, 7, 16, 37, 64])
def test_ffn_chunking_changes_nothing(oracle_lib, chunk):
    """Every row is computed the same way whatever chunk it falls in: the
    concatenated chunk outputs equal the unchunked layer bit for bit (37 rows:
    the last chunk is ragged for most sizes)."""
    rng = np.random.default_rng(66)
    rows, d, dff = 37, 8, 32
    args = (rng.standard_normal((rows, d)), rng.standard_normal((dff, d)),
            rng.standard_normal(dff), rng.standard_normal((d, dff)), rng.standard_normal(d))
    x2 = rng.standard_normal((rows, d))
    whole, hid = oracle.ffn(*args, x2=x2, return_hidden=True)
    got, ghid = oracle.ffn(*args, x2=x2, chunk_rows=chunk, return_hidden=True)
    np.testing.assert_array_equal(got, whole)
    np.testing.assert_array_equal(ghid, hid)


def test_ffn_equals_library_matmul(oracle_lib):
    rng = np.random.default_rng(67)
    rows, d, dff = 29, 16, 64
    y, x2 = rng.standard_normal((rows, d)), rng.standard_normal((rows, d))
    w1, b1 = rng.standard_normal((dff, d)), rng.standard_normal(dff)
    w2, b2 = rng.standard_normal((d, dff)), rng.standard_normal(d)
    want = np.maximum(y @ w1.T + b1, 0.0) @ w2.T + b2 + x2
    np.testing.assert_allclose(oracle.ffn(y, w1, b1, w2, b2, x2=x2, chunk_rows=5), want,
                               rtol=0, atol=1e-12)


def test_ffn_empty_and_bad_shapes(oracle_lib):
    d, dff = 4, 8
    w1, b1, w2, b2 = np.zeros((dff, d)), np.zeros(dff), np.zeros((d, dff)), np.zeros(d)
    assert oracle.ffn(np.zeros((0, d)), w1, b1, w2, b2).shape == (0, d)
    with pytest.raises(ValueError):
        oracle.ffn(np.zeros((3, d)), w1, b1, w2.T, b2)
    with pytest.raises(ValueError):
        oracle.ffn(np.zeros((3, d)), w1, b1, w2, b2, x2=np.zeros((2, d)))
