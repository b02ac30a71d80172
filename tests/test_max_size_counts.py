"""The closed forms behind the largest-size GPU cases (test_gpu_max_sizes):
for A[i, k] = 1 where k = i (mod 5) and B[j, k] = 1 where k = j (mod 7),
the product's counts, rounded to bf16, against the product itself computed
directly at small K (including K below, at and just past one period of
35); and the attention pattern's softmax against the attention oracle at
small Nk."""
import numpy as np
import pytest

from oracle.formats import round_to_bf16
from tests import test_gpu_max_sizes as mx


@pytest.mark.parametrize("K", [1, 4, 34, 35, 36, 71, 700, 4097])
def test_counts_match_direct_product(K):
    A = (np.arange(K)[None, :] % mx.P_A == np.arange(mx.M)[:, None] % mx.P_A).astype(float)
    B = (np.arange(K)[None, :] % mx.P_B == np.arange(mx.N)[:, None] % mx.P_B).astype(float)
    assert np.array_equal(mx._expected(K), round_to_bf16(A @ B.T))


def test_counts_stay_exact_in_fp32():
    # the largest count, at the 4-bit product's K, is below 2^24
    for K in (mx.K_BF16, mx.K_FP8, mx.K_FP4, *mx.K_MX.values()):
        assert mx._expected(K).max() < 2 ** 24


@pytest.mark.parametrize("Nk", [1, 2, 9, 10, 11, 37, 100])
@pytest.mark.parametrize("D", [64, 128])
def test_attention_closed_form_matches_oracle(Nk, D):
    from oracle.attention import attention_f64
    Nq = 3
    Q = np.zeros((1, 1, Nq, D))
    Q[..., 0] = 1.0
    K = np.zeros((1, 1, Nk, D))
    K[0, 0, 0::2, 0] = 1.0
    K[0, 0, 1::2, 0] = -1.0
    j, d = np.arange(Nk)[:, None], np.arange(D)[None, :]
    V = ((j + d) % 5 - 2).astype(np.float64)[None, None]
    R, Rlse = attention_f64(Q, K, V, scale=1.0, causal=False)
    A, _ = attention_f64(Q, K, np.abs(V), scale=1.0, causal=False)
    O, Ac, lse = mx.attention_closed_form(Nq, Nk, D)
    assert np.allclose(R[0, 0], O, rtol=1e-12, atol=1e-12)
    assert np.allclose(A[0, 0], Ac, rtol=1e-12, atol=1e-12)
    assert np.allclose(Rlse[0, 0], lse, rtol=1e-12, atol=0)


@pytest.mark.parametrize("D", [64, 128])
def test_uniform_rows_closed_form_matches_oracle(D):
    from oracle.attention import attention_f64
    Nq, Nk, scale = 7, mx.NK_WIDE, 1.0 / np.sqrt(D)
    Q = np.zeros((1, 1, Nq, D))
    Q[0, 0, :, 0] = (np.arange(Nq) % 3) - 1
    K = np.zeros((1, 1, Nk, D))
    K[..., 0] = 1.0
    j, d = np.arange(Nk)[:, None], np.arange(D)[None, :]
    V = ((j + d) % 5 - 2).astype(np.float64)[None, None]
    R, Rlse = attention_f64(Q, K, V, scale=scale, causal=False)
    O, lse = mx.uniform_rows_closed_form(Nk, D, scale, np.arange(Nq))
    assert np.allclose(R[0, 0], O[None, :], rtol=1e-12, atol=1e-12)
    assert np.allclose(Rlse[0, 0], lse, rtol=1e-12, atol=1e-12)
