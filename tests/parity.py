"""Comparison helpers for the GPU parity tests (tolerances are stated in
the tests that use them)."""
import numpy as np

import oracle


def to_numpy_u16(t):
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_numpy_u8(t):
    import torch
    return t.contiguous().view(torch.uint8).cpu().numpy()


def relfro(G, R):
    n = np.linalg.norm(R)
    return float(np.linalg.norm(G - R) / (n if n > 0 else 1.0))


def sample_tiles(M, N, seed, tile=64, n_random=8):
    """Origins of 64x64 output tiles: the four corners, tiles that straddle
    the 128- and 256-row/column workgroup-tile boundaries, and random ones."""
    rng = np.random.default_rng(seed)
    tm, tn = min(tile, M), min(tile, N)
    out = {(0, 0), (M - tm, 0), (0, N - tn), (M - tm, N - tn)}
    if M > 160 and N > 160:
        out.add((96, 96))          # straddles the 128-row/column tiles
    if M > 288 and N > 288:
        out.add((224, 224))
        out.add((M // 2 // 256 * 256 - 32, N // 2 // 256 * 256 - 32))
    for _ in range(n_random):
        out.add((int(rng.integers(0, M - tm + 1)), int(rng.integers(0, N - tn + 1))))
    return sorted(out)
