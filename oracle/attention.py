"""CPU oracle for softmax attention forward -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call this module; it shares no code with the GPU
library.

What it computes is the plain definition, on the exact values of the bf16
inputs, in IEEE fp64:

    S[i, j] = scale * sum_d Q[i, d] * K[j, d]
    P[i, j] = exp(S[i, j] - max_j' S[i, j']) / sum_j'' exp(S[i, j''] - max ...)
    O[i, d] = sum_j P[i, j] * V[j, d]
    lse[i]  = log sum_j exp(S[i, j])      (natural log)

for every batch b and query head h, over the keys j the query may see.

* The operation and its steps (Q K^T, the row max subtracted before the
  exponential, normalisation by the row sum, then times V): page
  "ThunderKittens: Simple, Fast, and Adorable AI Kernels", section 3,
  "PyTorch-Like Operations on Tiles" (mma_ABt, sub_row, exp, div_row,
  mma_AB) and "The LCSF Template", "The Four Functions" (the finish step
  divides by the normalisation constant). The online form with running max and rescaling
  (mul_row) is a way to evaluate the same function block by block; the
  oracle evaluates the definition directly.
* Variants: causal and non-causal, grouped-query attention, head dimension
  64 or 128: same page, section 5, "Attention: Matching FA3 on Forward,
  Outperforming on Backward" (Figure 8), and "Global Layout Descriptors"
  (4D tensors); page 3 ("ThunderKittens DSL for GPU kernels", aixai.ru),
  the attention prefill example (non-causal prefill).
Readings where the pages are silent:
* scale defaults to 1/sqrt(D) (the usual scaled dot product); any finite
  value is accepted.
* Causal: query i sees keys j <= i, with Nq == Nk.
* Grouped-query: Hq query heads share Hkv key/value heads, Hq % Hkv == 0;
  query head h reads key/value head h // (Hq // Hkv).
* Layouts [B, H, N, D], rows contiguous in D.
* A row with no visible key (Nk == 0) has no softmax; the library rejects
  Nq > 0 with Nk == 0, so the oracle does too.

Pins (tests/test_oracle_attention.py): uniform weights (zero scores) give
running means of V, constant V rows pass through, a single key, the
two-key logistic closed form, dominance of one key, invariance under a
joint permutation of keys and values and equivariance under permuting
queries, the grouped-query head map against explicitly repeated heads,
scipy's softmax/logsumexp on random rows, and the causal first/last rows.
"""
from __future__ import annotations

import math

import numpy as np

from .formats import decode_bf16

__all__ = ["attention_f64", "attention_bf16", "attention_flops",
           "attention_pairs"]


def _check(Q, K, V, causal):
    if Q.ndim != 4 or K.ndim != 4 or V.ndim != 4:
        raise ValueError("Q, K, V must be [B, H, N, D]")
    B, Hq, Nq, D = Q.shape
    Bk, Hkv, Nk, Dk = K.shape
    if V.shape != K.shape or Bk != B or Dk != D:
        raise ValueError("shape mismatch: Q %s K %s V %s" % (Q.shape, K.shape, V.shape))
    if Hq and (Hkv == 0 or Hq % Hkv):
        raise ValueError("Hq=%d must be a multiple of Hkv=%d" % (Hq, Hkv))
    if causal and Nq != Nk:
        raise ValueError("causal attention needs Nq == Nk")
    if Nk == 0 and Nq > 0 and B * Hq > 0:
        raise ValueError("no keys: the softmax of an empty row is undefined")
    return B, Hq, Hkv, Nq, Nk, D


def attention_f64(Q, K, V, scale=None, causal=False):
    """O [B, Hq, Nq, D] and lse [B, Hq, Nq] (float64) of softmax attention
    on float64 arrays Q [B, Hq, Nq, D], K and V [B, Hkv, Nk, D]."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B, Hq, Hkv, Nq, Nk, D = _check(Q, K, V, causal)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    O = np.zeros((B, Hq, Nq, D))
    lse = np.zeros((B, Hq, Nq))
    if B * Hq * Nq == 0:
        return O, lse
    group = Hq // Hkv
    visible = None
    if causal:
        visible = np.tril(np.ones((Nq, Nk), dtype=bool))
    for b in range(B):
        for h in range(Hq):
            kv = h // group
            S = (Q[b, h] @ K[b, kv].T) * float(scale)
            if visible is not None:
                S = np.where(visible, S, -np.inf)
            m = S.max(axis=1)
            E = np.exp(S - m[:, None])
            l = E.sum(axis=1)
            O[b, h] = (E @ V[b, kv]) / l[:, None]
            lse[b, h] = m + np.log(l)
    return O, lse


def attention_bf16(Qb, Kb, Vb, scale=None, causal=False):
    """The same on bf16 bit patterns (uint16 arrays), decoded exactly."""
    return attention_f64(decode_bf16(Qb), decode_bf16(Kb), decode_bf16(Vb),
                         scale=scale, causal=causal)


def attention_pairs(Nq, Nk, causal):
    """Number of (query, key) pairs a head computes."""
    if causal:
        return Nq * (Nq + 1) // 2
    return Nq * Nk


def attention_flops(B, Hq, Nq, Nk, D, causal):
    """Algorithmic flops: two products (Q K^T and P V) of 2*D flops per
    visible (query, key) pair."""
    return 4 * D * B * Hq * attention_pairs(Nq, Nk, causal)
