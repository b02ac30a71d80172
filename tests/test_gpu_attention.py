"""GPU parity of tkg_attention_fwd against the CPU oracle
(oracle.attention: the fp64 definition on the exact bf16 input values).

Tolerance, from the kernel's arithmetic: scores are fp32 sums of exact
bf16 products; each probability is rounded to bf16 before the P V product
and the row sum adds the same rounded weights, so every weight is off by at
most 2^-9 relative and numerator and denominator agree; accumulation is
fp32 and O takes one bf16 rounding. Then

    |O - O_ref| <= 2^-9 (sum_j p_j |v_j| + 2 |O_ref|)  (+ fp32 terms)

and the test allows 2^-8 (sum_j p_j |v_j| + |O_ref|) + 1e-6, where
sum_j p_j |v_j| is the oracle applied to |V|. The log-sum-exp is off by at
most 2^-9 (the row sum's relative error): allowed 2^-8 + 1e-6 |lse|.
"""
import math

import numpy as np
import pytest
import torch

import gemm_inputs as gi
import gemm_inputs.device  # noqa: F401  (gi.device)
import tiled_dense_gemm_amd as tkg
from oracle.attention import attention_f64
from oracle.formats import decode_bf16
from tests.parity import to_numpy_u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU parity tests need the HIP device"
    return torch.device("cuda:0")


def _up(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev).view(torch.bfloat16)


def _run(q, k, v, dev, causal, scale=None):
    Q, K, V = _up(q, dev), _up(k, dev), _up(v, dev)
    O, lse = tkg.tkg_attention_fwd(Q, K, V, causal=causal, scale=scale, lse=True)
    torch.cuda.synchronize()
    return decode_bf16(to_numpy_u16(O)), lse.cpu().numpy().astype(np.float64)


def _check(G, Glse, Qf, Kf, Vf, causal, scale=None, what=""):
    R, Rlse = attention_f64(Qf, Kf, Vf, scale=scale, causal=causal)
    A, _ = attention_f64(Qf, Kf, np.abs(Vf), scale=scale, causal=causal)
    bound = 2.0 ** -8 * (A + np.abs(R)) + 1e-6
    err = np.abs(G - R)
    assert np.all(np.isfinite(G)), what
    assert np.all(err <= bound), (what, float(np.max(err - bound)),
                                  np.unravel_index(np.argmax(err - bound), err.shape))
    lerr = np.abs(Glse - Rlse)
    assert np.all(lerr <= 2.0 ** -8 + 1e-6 * np.abs(Rlse)), (what, float(lerr.max()))


CASES = [
    # B, Hq, Hkv, Nq, Nk, D, causal
    (1, 2, 2, 256, 256, 128, False),
    (1, 2, 2, 256, 256, 64, False),
    (2, 4, 2, 300, 300, 128, True),     # grouped-query, ragged, causal
    (1, 8, 1, 513, 513, 64, True),      # group of 8, three query blocks
    (1, 2, 2, 100, 700, 128, False),    # more keys than queries, key tail
    (1, 2, 1, 17, 1000, 64, False),
    (1, 3, 3, 1, 1, 64, False),         # one query, one key
    (1, 1, 1, 1, 1, 128, True),
    (2, 2, 2, 640, 640, 128, True),     # heaviest-first block order
    (1, 2, 2, 64, 64, 64, True),        # one key block
    (1, 2, 2, 65, 65, 128, True),       # one key past a block
    (3, 1, 1, 200, 129, 128, False),
]


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,D,causal", CASES)
def test_attention_matches_oracle(dev, B, Hq, Hkv, Nq, Nk, D, causal):
    print("attention", B, Hq, Hkv, Nq, Nk, D, causal, flush=True)
    q, k, v = gi.attention_operands(101 + Nq + D, B, Hq, Hkv, Nq, Nk, D)
    G, Gl = _run(q, k, v, dev, causal)
    _check(G, Gl, decode_bf16(q), decode_bf16(k), decode_bf16(v), causal,
           what=(B, Hq, Hkv, Nq, Nk, D, causal))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_peaked_scores(dev, D, causal):
    # std 4 queries: scores of tens, near one-hot rows, the max moves a lot
    q, k, v = gi.attention_operands(7 + D, 1, 2, 2, 384, 384, D, std_q=4.0)
    G, Gl = _run(q, k, v, dev, causal)
    _check(G, Gl, decode_bf16(q), decode_bf16(k), decode_bf16(v), causal, what="peaked")


@pytest.mark.parametrize("rising", [True, False])
def test_row_max_moving_every_block(dev, rising):
    # scores rising (falling) by 0.25 per key with scale 1: the row max
    # jumps by 0.25 * 32 * log2(e) = 11.5 (log2 units) every 32-key block,
    # past the kernel's rescale slack of 8 (or never moves after the first
    # block)
    D, N = 64, 512
    q = np.zeros((1, 1, 32, D))
    q[..., 0] = 1.0
    k = np.zeros((1, 1, N, D))
    k[0, 0, :, 0] = 0.25 * (np.arange(N) if rising else np.arange(N)[::-1])
    k[0, 0, :, 1:] = gi.normal(3, N, D - 1, 0.1)
    qb, kb = gi.bf16_bits(q), gi.bf16_bits(k)
    vb = gi.bf16_bits(gi.normal(4, N, D).reshape(1, 1, N, D))
    G, Gl = _run(qb, kb, vb, dev, False, scale=1.0)
    _check(G, Gl, decode_bf16(qb), decode_bf16(kb), decode_bf16(vb), False, scale=1.0,
           what="rising" if rising else "falling")


def test_uniform_rows_give_value_means(dev):
    # Q = 0: every weight is 1/Nk (exactly representable when Nk is a power
    # of two), O is the mean of V
    D, N = 128, 1024
    qb = np.zeros((1, 2, 64, D), np.uint16)
    _, kb, vb = gi.attention_operands(11, 1, 2, 2, 64, N, D)
    G, Gl = _run(qb, kb, vb, dev, False)
    R = decode_bf16(vb).mean(axis=2, keepdims=True)
    bound = 2.0 ** -8 * np.abs(R) + 2.0 ** -16
    assert np.all(np.abs(G - R) <= bound)
    np.testing.assert_allclose(Gl, math.log(N), rtol=0, atol=1e-5)


def test_scale_argument(dev):
    q, k, v = gi.attention_operands(12, 1, 2, 2, 128, 128, 64)
    for scale in (0.02, 0.5):
        G, Gl = _run(q, k, v, dev, False, scale=scale)
        _check(G, Gl, decode_bf16(q), decode_bf16(k), decode_bf16(v), False, scale=scale,
               what=scale)


def test_lse_optional_and_deterministic(dev):
    q, k, v = gi.attention_operands(13, 1, 4, 2, 300, 300, 128)
    Q, K, V = _up(q, dev), _up(k, dev), _up(v, dev)
    O1 = tkg.tkg_attention_fwd(Q, K, V, causal=True)
    O2, _ = tkg.tkg_attention_fwd(Q, K, V, causal=True, lse=True)
    torch.cuda.synchronize()
    assert torch.equal(O1.view(torch.int16), O2.view(torch.int16))


def test_empty_and_rejected(dev):
    Q = torch.zeros((1, 2, 0, 64), dtype=torch.bfloat16, device=dev)
    K = torch.zeros((1, 2, 5, 64), dtype=torch.bfloat16, device=dev)
    assert tkg.tkg_attention_fwd(Q, K, K).shape == (1, 2, 0, 64)
    Q = torch.zeros((1, 2, 3, 64), dtype=torch.bfloat16, device=dev)
    K0 = torch.zeros((1, 2, 0, 64), dtype=torch.bfloat16, device=dev)
    with pytest.raises(tkg.TkgError):
        tkg.tkg_attention_fwd(Q, K0, K0)
    with pytest.raises(tkg.TkgError):
        tkg.tkg_attention_fwd(Q, K, K, causal=True)


# ------------------------------------------------ full-size, sampled rows

FULL = [
    # the measured workloads (B, Hq, Hkv, N, D, causal) and the long end of
    # the pages' sequence range at D = 64
    (16, 16, 16, 4096, 128, False),
    (16, 16, 16, 4096, 128, True),
    (4, 32, 32, 4096, 64, False),
    (1, 16, 2, 16384, 128, True),
    (1, 32, 4, 16384, 64, True),
]


@pytest.mark.parametrize("B,Hq,Hkv,N,D,causal", FULL)
def test_full_size_sampled_rows(dev, B, Hq, Hkv, N, D, causal):
    print("attention full", B, Hq, Hkv, N, D, causal, flush=True)
    Q = gi.device.bf16_operand(201, B * Hq * N, D, device=dev).view(B, Hq, N, D)
    K = gi.device.bf16_operand(202, B * Hkv * N, D, device=dev).view(B, Hkv, N, D)
    V = gi.device.bf16_operand(203, B * Hkv * N, D, device=dev).view(B, Hkv, N, D)
    O, lse = tkg.tkg_attention_fwd(Q, K, V, causal=causal, lse=True)
    torch.cuda.synchronize()
    g = np.random.Generator(np.random.Philox(key=N + D))
    heads = [(0, 0), (B - 1, Hq - 1), (B // 2, Hq // 2 + 1)]
    for b, h in heads:
        kv = h // (Hq // Hkv)
        rows = np.unique(np.concatenate([[0, 1, 255, 256, N - 1],
                                         g.integers(0, N, 11)]))
        Kf = decode_bf16(to_numpy_u16(K[b, kv]))[None, None]
        Vf = decode_bf16(to_numpy_u16(V[b, kv]))[None, None]
        Qf = decode_bf16(to_numpy_u16(Q[b, h]))
        Gf = decode_bf16(to_numpy_u16(O[b, h]))
        Gl = lse[b, h].cpu().numpy().astype(np.float64)
        for i in rows:
            n = i + 1 if causal else N
            _check(Gf[i][None, None, None], Gl[i][None, None, None],
                   Qf[i][None, None, None], Kf[:, :, :n], Vf[:, :, :n], False,
                   what=(b, h, int(i)))


def test_full_size_more_keys_than_queries(dev):
    # 512 queries against 16384 keys (a prefill chunk against its context)
    B, Hq, Hkv, Nq, Nk, D = 2, 8, 2, 512, 16384, 128
    Q = gi.device.bf16_operand(211, B * Hq * Nq, D, device=dev).view(B, Hq, Nq, D)
    K = gi.device.bf16_operand(212, B * Hkv * Nk, D, device=dev).view(B, Hkv, Nk, D)
    V = gi.device.bf16_operand(213, B * Hkv * Nk, D, device=dev).view(B, Hkv, Nk, D)
    O, lse = tkg.tkg_attention_fwd(Q, K, V, lse=True)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (1, 7)):
        kv = h // (Hq // Hkv)
        Kf = decode_bf16(to_numpy_u16(K[b, kv]))[None, None]
        Vf = decode_bf16(to_numpy_u16(V[b, kv]))[None, None]
        rows = [0, 1, 127, 128, 511]
        Qf = decode_bf16(to_numpy_u16(Q[b, h, rows]))[None, None]
        _check(decode_bf16(to_numpy_u16(O[b, h, rows]))[None, None],
               lse[b, h, rows].cpu().numpy().astype(np.float64)[None, None],
               Qf, Kf, Vf, False, what=(b, h))


@pytest.mark.parametrize("B,Hq,Hkv,N,D", [
    (16, 16, 16, 4096, 128),   # 256 heads: longest-first windows of 4 heads per XCD
    (16, 32, 32, 1024, 64),    # 512 heads, 8 query blocks each: windows of 32
    (1, 16, 2, 16384, 128),    # grouped-query, 16 heads
    (3, 5, 5, 1000, 64),       # head count not a multiple of the 8 XCDs
])
def test_causal_grid_writes_every_row(dev, B, Hq, Hkv, N, D):
    # the causal work-item order is a permutation of (head, query block):
    # with O and lse pre-filled with NaN, every element must be written
    print("attention every row", B, Hq, Hkv, N, D, flush=True)
    Q = gi.device.bf16_operand(221, B * Hq * N, D, device=dev).view(B, Hq, N, D)
    K = gi.device.bf16_operand(222, B * Hkv * N, D, device=dev).view(B, Hkv, N, D)
    V = gi.device.bf16_operand(223, B * Hkv * N, D, device=dev).view(B, Hkv, N, D)
    O = torch.full((B, Hq, N, D), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((B, Hq, N), float("nan"), dtype=torch.float32, device=dev)
    tkg.tkg_attention_fwd(Q, K, V, causal=True, out=O, lse=lse)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(O).all()) and bool(torch.isfinite(lse).all())
    # row 0 of every head attends to key 0 alone: O = V[0], lse = score
    kv = torch.arange(Hq, device=dev) // (Hq // Hkv)
    assert torch.equal(O[:, :, 0].view(torch.int16), V[:, kv, 0].view(torch.int16))
