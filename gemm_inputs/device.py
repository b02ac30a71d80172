"""Seeded synthetic operands generated on the GPU with torch, for shapes the
host cannot draw quickly (e.g. 16384^2 and 65536^2). Same recipes as the
host generators in ``gemm_inputs`` (normal draws, per-tensor fp8 scaling,
the block-scaled 4-bit recipe), drawn from torch's device generator, so the
values differ from the host ones for the same seed. Rows are generated in
chunks from per-chunk seeds, so a matrix never needs more than one chunk of
fp32 scratch."""
from __future__ import annotations

import math

import torch

E4M3_MAX = 448.0
E2M1_MAX = 6.0
CHUNK_ROWS = 4096
_E2M1_MIDS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def _chunks(rows):
    for r0 in range(0, rows, CHUNK_ROWS):
        yield r0, min(rows, r0 + CHUNK_ROWS)


def _normal_chunk(seed, ci, r, cols, std, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000003 + ci)
    x = torch.randn((r, cols), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x


def _amax(seed, rows, cols, std, device):
    m = 0.0
    for ci, (r0, r1) in enumerate(_chunks(rows)):
        m = max(m, float(_normal_chunk(seed, ci, r1 - r0, cols, std, device).abs().max()))
    return m


def bf16_operand(seed, rows, cols, std=1.0, device="cuda"):
    out = torch.empty((rows, cols), dtype=torch.bfloat16, device=device)
    for ci, (r0, r1) in enumerate(_chunks(rows)):
        out[r0:r1] = _normal_chunk(seed, ci, r1 - r0, cols, std, device)
    return out


def _e4m3_bytes(y):
    return y.clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn).view(torch.uint8)


def fp8_operand(seed, rows, cols, std=1.0, device="cuda"):
    """(uint8 e4m3 codes, fp32 scale amax/448)."""
    amax = _amax(seed, rows, cols, std, device)
    s = float(torch.tensor(amax / E4M3_MAX, dtype=torch.float32)) if amax > 0 else 1.0
    out = torch.empty((rows, cols), dtype=torch.uint8, device=device)
    for ci, (r0, r1) in enumerate(_chunks(rows)):
        x = _normal_chunk(seed, ci, r1 - r0, cols, std, device)
        out[r0:r1] = _e4m3_bytes(x.to(torch.float64) / s)
    return out, s


def _e2m1_codes(y):
    a = y.abs().clamp(max=E2M1_MAX)
    mids = torch.tensor(_E2M1_MIDS, dtype=a.dtype, device=a.device)
    code = torch.bucketize(a, mids)              # mids strictly below a
    tie = (code < 7) & (a == mids[code.clamp(max=6)])
    code = code + (tie & (code % 2 == 1)).to(code.dtype)   # ties to even
    return (code | ((y < 0).to(code.dtype) << 3)).to(torch.uint8)


def fp4_operand(seed, rows, cols, std=1.0, device="cuda", block=16):
    """(packed e2m1 uint8 rows x cols/2, e4m3 block scales uint8
    rows x cols/block, fp32 tensor scale t); recipe as gemm_inputs."""
    amax = _amax(seed, rows, cols, std, device)
    t = float(torch.tensor(amax / (E2M1_MAX * E4M3_MAX), dtype=torch.float32)) if amax > 0 else 1.0
    packed = torch.empty((rows, cols // 2), dtype=torch.uint8, device=device)
    scales = torch.empty((rows, cols // block), dtype=torch.uint8, device=device)
    for ci, (r0, r1) in enumerate(_chunks(rows)):
        x = _normal_chunk(seed, ci, r1 - r0, cols, std, device).to(torch.float64)
        xb = x.view(r1 - r0, cols // block, block)
        sc = _e4m3_bytes(xb.abs().amax(dim=2) / (E2M1_MAX * t))
        sval = sc.view(torch.float8_e4m3fn).to(torch.float64) * t
        y = torch.where(sval[..., None] > 0, xb / sval[..., None].clamp(min=1e-300),
                        torch.zeros_like(xb))
        codes = _e2m1_codes(y.view(r1 - r0, cols))
        packed[r0:r1] = codes[:, 0::2] | (codes[:, 1::2] << 4)
        scales[r0:r1] = sc
    return packed, scales, t


def mx_operand(seed, rows, cols, elem, std=1.0, device="cuda"):
    """(values, E8M0 scales rows x cols/32) in the recipe of
    gemm_inputs.mx_quantize: values are packed e2m1 (rows x cols/2) or e4m3
    (rows x cols) codes."""
    from . import MX_BLOCK, MX_EMAX
    fp4 = elem == "e2m1"
    vals = torch.empty((rows, cols // 2 if fp4 else cols), dtype=torch.uint8, device=device)
    scales = torch.empty((rows, cols // MX_BLOCK), dtype=torch.uint8, device=device)
    for ci, (r0, r1) in enumerate(_chunks(rows)):
        x = _normal_chunk(seed, ci, r1 - r0, cols, std, device).to(torch.float64)
        xb = x.view(r1 - r0, cols // MX_BLOCK, MX_BLOCK)
        amax = xb.abs().amax(dim=2)
        e = torch.where(amax > 0, torch.floor(torch.log2(amax.clamp(min=1e-300))) - MX_EMAX[elem],
                        torch.full_like(amax, -127.0)).clamp(-127, 127)
        y = (xb / torch.exp2(e)[..., None]).view(r1 - r0, cols)
        if fp4:
            codes = _e2m1_codes(y)
            vals[r0:r1] = codes[:, 0::2] | (codes[:, 1::2] << 4)
        else:
            vals[r0:r1] = _e4m3_bytes(y)
        scales[r0:r1] = (e + 127).to(torch.uint8)
    return vals, scales
