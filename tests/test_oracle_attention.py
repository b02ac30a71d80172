"""Pins of the attention oracle against results fixed by the mathematics,
independent of the oracle's own arithmetic: closed forms, special cases,
symmetries, and scipy's softmax/logsumexp. Every plausible slip in the
oracle (a dropped scale, a sign, the max left unsubtracted, the wrong
normalisation axis, a transposed product, a wrong grouped-query head map, a
causal mask off by one, an lse without its max) fails at least one of them."""
import math

import numpy as np
import pytest
from scipy import special

import gemm_inputs as gi
from oracle.attention import (attention_bf16, attention_f64, attention_flops,
                              attention_pairs)
from oracle.formats import decode_bf16


def _rand(seed, *shape, std=1.0):
    n = int(np.prod(shape[:-1]))
    return gi.normal(seed, n, shape[-1], std).reshape(shape)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_scores_average_values(causal):
    # Q = 0: every visible key weighs the same, so O is a plain mean of V
    # (a running mean under the causal mask) and lse = log(#visible keys)
    B, H, N, D = 2, 3, 7, 8
    Q = np.zeros((B, H, N, D))
    K = _rand(1, B, H, N, D)
    V = _rand(2, B, H, N, D)
    O, lse = attention_f64(Q, K, V, causal=causal)
    if causal:
        counts = np.arange(1, N + 1)
        want = np.cumsum(V, axis=2) / counts[:, None]
        want_lse = np.broadcast_to(np.log(counts), (B, H, N))
    else:
        want = np.broadcast_to(V.mean(axis=2, keepdims=True), V.shape)
        want_lse = np.full((B, H, N), math.log(N))
    np.testing.assert_allclose(O, want, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, want_lse, rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_constant_value_rows_pass_through(causal):
    B, H, N, D = 1, 2, 9, 16
    Q = _rand(3, B, H, N, D, std=2.0)
    K = _rand(4, B, H, N, D)
    c = _rand(5, 1, D)[0]
    V = np.broadcast_to(c, (B, H, N, D)).copy()
    O, _ = attention_f64(Q, K, V, causal=causal)
    np.testing.assert_allclose(O, np.broadcast_to(c, O.shape), rtol=1e-14, atol=1e-14)


def test_single_key():
    # one key: weight 1, O = V[0], lse = the single scaled score
    D = 8
    Q = _rand(6, 1, 2, 5, D)
    K = _rand(7, 1, 1, 1, D)
    V = _rand(8, 1, 1, 1, D)
    scale = 0.37
    O, lse = attention_f64(Q, K, V, scale=scale)
    for h in range(2):
        for i in range(5):
            s = scale * math.fsum(Q[0, h, i, d] * K[0, 0, 0, d] for d in range(D))
            assert lse[0, h, i] == pytest.approx(s, abs=1e-14)
            np.testing.assert_allclose(O[0, h, i], V[0, 0, 0], rtol=0, atol=1e-15)


def test_two_keys_logistic():
    # two keys: w0 = sigmoid(s0 - s1), O = w0 v0 + (1 - w0) v1,
    # lse = logaddexp(s0, s1)
    D = 16
    Q = _rand(9, 1, 1, 6, D)
    K = _rand(10, 1, 1, 2, D)
    V = _rand(11, 1, 1, 2, D)
    scale = 0.8
    O, lse = attention_f64(Q, K, V, scale=scale)
    for i in range(6):
        s0 = scale * math.fsum(Q[0, 0, i] * K[0, 0, 0])
        s1 = scale * math.fsum(Q[0, 0, i] * K[0, 0, 1])
        w0 = special.expit(s0 - s1)
        np.testing.assert_allclose(O[0, 0, i], w0 * V[0, 0, 0] + (1 - w0) * V[0, 0, 1],
                                   rtol=1e-13, atol=1e-14)
        assert lse[0, 0, i] == pytest.approx(np.logaddexp(s0, s1), abs=1e-13)


def test_dominant_key_without_overflow():
    # one key's score exceeds the others by ~1000: its weight is 1 to double
    # precision; scores that large overflow exp() unless the max is removed
    D, N = 8, 12
    q = np.zeros(D)
    q[0] = 40.0
    Q = np.broadcast_to(q, (1, 1, 3, D)).copy()
    K = _rand(12, 1, 1, N, D, std=0.01)
    K[0, 0, 5, 0] = 200.0
    V = _rand(13, 1, 1, N, D)
    O, lse = attention_f64(Q, K, V, scale=1.0)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(lse))
    np.testing.assert_allclose(O[0, 0], np.broadcast_to(V[0, 0, 5], (3, D)), rtol=0, atol=1e-12)
    s_top = float(Q[0, 0, 0] @ K[0, 0, 5])
    assert lse[0, 0, 0] == pytest.approx(s_top, abs=1e-9)


def test_permutations():
    # permuting keys and values together leaves non-causal O unchanged;
    # permuting queries permutes the rows of O and lse
    B, H, Nq, Nk, D = 1, 2, 10, 13, 8
    Q = _rand(14, B, H, Nq, D)
    K = _rand(15, B, H, Nk, D)
    V = _rand(16, B, H, Nk, D)
    O, lse = attention_f64(Q, K, V)
    pk = gi.permutation(17, Nk)
    O2, lse2 = attention_f64(Q, K[:, :, pk], V[:, :, pk])
    np.testing.assert_allclose(O2, O, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse2, lse, rtol=1e-13, atol=1e-14)
    pq = gi.permutation(18, Nq)
    O3, lse3 = attention_f64(Q[:, :, pq], K, V)
    np.testing.assert_allclose(O3, O[:, :, pq], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse3, lse[:, :, pq], rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_grouped_query_equals_repeated_heads(causal):
    # query head h reads key/value head h // (Hq / Hkv): the same as giving
    # every query head its own copy of that key/value head
    B, Hq, Hkv, N, D = 2, 6, 2, 9, 8
    Q = _rand(19, B, Hq, N, D)
    K = _rand(20, B, Hkv, N, D)
    V = _rand(21, B, Hkv, N, D)
    O, lse = attention_f64(Q, K, V, causal=causal)
    Kr = np.repeat(K, Hq // Hkv, axis=1)
    Vr = np.repeat(V, Hq // Hkv, axis=1)
    O2, lse2 = attention_f64(Q, Kr, Vr, causal=causal)
    np.testing.assert_array_equal(O, O2)
    np.testing.assert_array_equal(lse, lse2)
    # and differs from the other plausible map, h % Hkv
    Kw = np.tile(K, (1, Hq // Hkv, 1, 1))
    Vw = np.tile(V, (1, Hq // Hkv, 1, 1))
    O3, _ = attention_f64(Q, Kw, Vw, causal=causal)
    assert np.max(np.abs(O3 - O)) > 1e-3


@pytest.mark.parametrize("causal", [False, True])
def test_rows_against_scipy(causal):
    # each row: scipy's softmax of the scaled scores times V, and scipy's
    # logsumexp; the scores come from per-element fsum dot products
    B, H, N, D = 1, 2, 11, 16
    qb, kb, vb = gi.attention_operands(22, B, H, H, N, N, D, std_q=2.0)
    Q, K, V = decode_bf16(qb), decode_bf16(kb), decode_bf16(vb)
    scale = 1.0 / math.sqrt(D)
    O, lse = attention_bf16(qb, kb, vb, causal=causal)
    for h in range(H):
        for i in range(N):
            n = i + 1 if causal else N
            s = np.array([scale * math.fsum(Q[0, h, i] * K[0, h, j]) for j in range(n)])
            p = special.softmax(s)
            want = np.array([math.fsum(p * V[0, h, :n, d]) for d in range(D)])
            np.testing.assert_allclose(O[0, h, i], want, rtol=1e-12, atol=1e-13)
            assert lse[0, h, i] == pytest.approx(special.logsumexp(s), abs=1e-12)


def test_causal_first_and_last_rows():
    B, H, N, D = 1, 2, 8, 8
    Q = _rand(23, B, H, N, D)
    K = _rand(24, B, H, N, D)
    V = _rand(25, B, H, N, D)
    Oc, lc = attention_f64(Q, K, V, causal=True)
    On, ln = attention_f64(Q, K, V, causal=False)
    np.testing.assert_allclose(Oc[:, :, 0], V[:, :, 0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(Oc[:, :, -1], On[:, :, -1], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(lc[:, :, -1], ln[:, :, -1], rtol=1e-14, atol=1e-15)
    # row 1 sees exactly keys 0 and 1
    s = Q[0, 0, 1] @ K[0, 0, :2].T / math.sqrt(D)
    w0 = special.expit(s[0] - s[1])
    np.testing.assert_allclose(Oc[0, 0, 1], w0 * V[0, 0, 0] + (1 - w0) * V[0, 0, 1],
                               rtol=1e-13, atol=1e-14)


def test_scale_folds_into_queries():
    # scores depend on scale * Q only: doubling Q and halving scale is exact
    Q = _rand(26, 1, 1, 6, 8)
    K = _rand(27, 1, 1, 7, 8)
    V = _rand(28, 1, 1, 7, 8)
    O, lse = attention_f64(Q, K, V, scale=0.3)
    O2, lse2 = attention_f64(2 * Q, K, V, scale=0.15)
    np.testing.assert_allclose(O2, O, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(lse2, lse, rtol=1e-14, atol=1e-15)
    # the default scale is 1/sqrt(D)
    O3, _ = attention_f64(Q, K, V)
    O4, _ = attention_f64(Q, K, V, scale=1 / math.sqrt(8))
    np.testing.assert_array_equal(O3, O4)


def test_brute_force_tiny():
    # pure-Python loops with math.exp on a 1 x 2 x 3 x 4 case
    B, H, N, D = 1, 2, 3, 4
    Q = _rand(29, B, H, N, D)
    K = _rand(30, B, H, N, D)
    V = _rand(31, B, H, N, D)
    for causal in (False, True):
        O, lse = attention_f64(Q, K, V, scale=0.5, causal=causal)
        for h in range(H):
            for i in range(N):
                js = range(i + 1) if causal else range(N)
                s = {j: 0.5 * sum(Q[0, h, i, d] * K[0, h, j, d] for d in range(D)) for j in js}
                top = max(s.values())
                e = {j: math.exp(s[j] - top) for j in js}
                z = sum(e.values())
                for d in range(D):
                    assert O[0, h, i, d] == pytest.approx(
                        sum(e[j] * V[0, h, j, d] for j in js) / z, abs=1e-14)
                assert lse[0, h, i] == pytest.approx(top + math.log(z), abs=1e-14)


def test_shapes_rejected_and_empty():
    Q = np.zeros((1, 2, 3, 8))
    K = np.zeros((1, 1, 4, 8))
    with pytest.raises(ValueError):
        attention_f64(Q, K, K, causal=True)          # Nq != Nk
    with pytest.raises(ValueError):
        attention_f64(np.zeros((1, 3, 3, 8)), np.zeros((1, 2, 3, 8)),
                      np.zeros((1, 2, 3, 8)))        # 3 % 2
    with pytest.raises(ValueError):
        attention_f64(Q, np.zeros((1, 1, 0, 8)), np.zeros((1, 1, 0, 8)))
    O, lse = attention_f64(np.zeros((0, 2, 3, 8)), np.zeros((0, 1, 3, 8)),
                           np.zeros((0, 1, 3, 8)))
    assert O.shape == (0, 2, 3, 8) and lse.shape == (0, 2, 3)
    O, lse = attention_f64(np.zeros((1, 2, 0, 8)), K, K)
    assert O.shape == (1, 2, 0, 8)


def test_flop_count():
    for n in (1, 5, 64):
        mask = np.tril(np.ones((n, n), dtype=bool))
        assert attention_pairs(n, n, True) == int(mask.sum())
    assert attention_pairs(3, 7, False) == 21
    assert attention_flops(2, 3, 4, 4, 64, False) == 4 * 64 * 2 * 3 * 16
