"""The seeded operand generators: encoders round-trip every code, round to
nearest even, saturate, and the quantization recipes keep their stated
properties. Decoding uses the oracle's independent format tables."""
import numpy as np

import gemm_inputs as gi
from oracle.formats import (E2M1_TABLE, E4M3_TABLE, decode_bf16,
                            decode_e4m3, round_to_bf16)
import oracle


def test_seeded_and_reproducible():
    a = gi.normal(3, 4, 5)
    assert np.array_equal(a, gi.normal(3, 4, 5))
    assert not np.array_equal(a, gi.normal(4, 4, 5))


def test_bf16_encoder_rounds_to_nearest():
    x = gi.normal(0, 200, 200)
    v = decode_bf16(gi.bf16_bits(x))
    # one rounding from fp32: within half a bf16 ulp of the fp32 value
    assert np.array_equal(v, round_to_bf16(x.astype(np.float32).astype(np.float64)))


def test_e4m3_encoder_roundtrip_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    vals = E4M3_TABLE[codes]
    ok = ~np.isnan(vals)
    back = gi.e4m3_codes(vals[ok])
    assert np.array_equal(back, codes[ok])


def test_e4m3_encoder_ties_to_even_and_saturates():
    one, nxt = E4M3_TABLE[0x38], E4M3_TABLE[0x39]
    assert gi.e4m3_codes(np.array([(one + nxt) / 2]))[0] == 0x38      # even
    a, b = E4M3_TABLE[0x39], E4M3_TABLE[0x3A]
    assert gi.e4m3_codes(np.array([(a + b) / 2]))[0] == 0x3A
    assert gi.e4m3_codes(np.array([1e6, -1e6, 460.0]))[0] == 0x7E
    assert gi.e4m3_codes(np.array([-1e6]))[0] == 0xFE
    sub = gi.e4m3_codes(np.array([2.0 ** -10, 3 * 2.0 ** -10]))
    assert list(sub) == [0x00, 0x02]            # ties in the subnormal range


def test_e4m3_encoder_is_nearest():
    y = gi.normal(1, 100, 100) * 50
    v = decode_e4m3(gi.e4m3_codes(y))
    finite = np.sort(np.unique(np.abs(E4M3_TABLE[~np.isnan(E4M3_TABLE)])))
    a = np.minimum(np.abs(y), 448.0).ravel()
    idx = np.clip(np.searchsorted(finite, a), 1, len(finite) - 1)
    best = np.minimum(np.abs(finite[idx] - a), np.abs(finite[idx - 1] - a))
    assert np.all(np.abs(np.abs(v).ravel() - a) <= best)


def test_e2m1_encoder_roundtrip_and_ties():
    assert np.array_equal(gi.e2m1_codes(E2M1_TABLE), np.arange(16))
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 100.0])
    want = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0]
    assert list(E2M1_TABLE[gi.e2m1_codes(ties)]) == want


def test_fp8_recipe_maps_amax_to_448():
    x = gi.normal(2, 64, 128)
    q, s = gi.fp8_quantize(x)
    assert s == float(np.float32(np.max(np.abs(x)) / 448.0))
    assert np.max(np.abs(decode_e4m3(q))) == 448.0
    err = np.linalg.norm(decode_e4m3(q) * s - x) / np.linalg.norm(x)
    assert err < 0.05


def test_fp4_recipe_properties():
    x = gi.normal(3, 32, 256)
    packed, sc, t = gi.fp4_quantize(x)
    assert packed.shape == (32, 128) and sc.shape == (32, 16)
    v = oracle.dequant_fp4_blockscaled(packed, sc)
    assert np.max(np.abs(v)) <= 6.0 * 448.0
    rel = np.linalg.norm(v * t - x) / np.linalg.norm(x)
    assert rel < 0.15
    # a zero block gets scale 0 and zero values
    x[0, :16] = 0.0
    packed, sc, t = gi.fp4_quantize(x)
    assert sc[0, 0] == 0 and not oracle.dequant_fp4_blockscaled(packed, sc)[0, :16].any()
