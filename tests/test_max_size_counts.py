"""The closed form behind the largest-K GPU cases (test_gpu_max_sizes):
for A[i, k] = 1 where k = i (mod 5) and B[j, k] = 1 where k = j (mod 7),
the product's counts, rounded to bf16, against the product itself computed
directly at small K (including K below, at and just past one period of
35)."""
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
