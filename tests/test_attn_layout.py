"""Host-side checks of the attention kernel's LDS addressing (no GPU): the
ring copies place every (key, d) element of a key block exactly once, and
the K fragment reads and transposing V reads then hand each lane the MFMA
operand values the kernel's accumulator layout needs.

The transposing read's lane rule (ds_read_b64_tr_b16 on gfx950) was
measured on the GPU with an in-bounds probe that filled LDS with each
element's own index: lane 16g + 4a + b receives, in element j, the b-th
16-bit value of the 8 bytes addressed by lane 16g + a + 4j."""
import numpy as np
import pytest

import tiled_dense_gemm_amd as tkg

BK = 32  # keys per ring slot


def tr_read(image_u16, addrs):
    """Simulate one transposing 8-byte read of 64 lanes on a uint16 LDS image."""
    out = np.zeros((64, 4), dtype=np.int64)
    for lane in range(64):
        g, i = divmod(lane, 16)
        a, b = divmod(i, 4)
        for j in range(4):
            src = addrs[16 * g + a + 4 * j]
            assert src % 8 == 0
            out[lane, j] = image_u16[src // 2 + b]
    return out


def tile_image(d, kind):
    """LDS image (uint16 element ids key * d + dim) of one K (kind 2) or V
    (kind 3) tile as the ring copies fill it."""
    img = np.full(BK * d, -1, dtype=np.int64)
    for piece in range(BK * 2 * d // 1024):
        src = tkg.attn_lds_offsets(d, kind, piece)
        for lane in range(64):
            key, byte = divmod(src[lane], 2 * d)
            assert byte % 16 == 0 and key < BK
            dst = (1024 * piece + 16 * lane) // 2
            img[dst:dst + 8] = key * d + byte // 2 + np.arange(8)
    return img


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("kind", [2, 3])
def test_ring_copies_place_every_element_once(d, kind):
    img = tile_image(d, kind)
    assert sorted(img.tolist()) == list(range(BK * d))


@pytest.mark.parametrize("d", [64, 128])
def test_k_fragment_reads(d):
    # MFMA A operand of k-step ks: lane l holds key l % 32, dims
    # 16 ks + 8 (l / 32) .. +7
    img = tile_image(d, 2)
    for kb in range(BK // 32):
        for ks in range(d // 16):
            offs = tkg.attn_lds_offsets(d, 0, kb, ks)
            for lane in range(64):
                got = img[offs[lane] // 2: offs[lane] // 2 + 8]
                key = 32 * kb + lane % 32
                want = key * d + 16 * ks + 8 * (lane // 32) + np.arange(8)
                np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("d", [64, 128])
def test_v_transposing_reads(d):
    # MFMA A operand of V^T for k-step s of 32-key block kb, output rows
    # 32 db .. +31: lane l holds dim 32 db + l % 32 and, in k-slot
    # j = 4 t + jj, key 32 kb + 16 s + 8 t + 4 (l / 32) + jj -- the order of
    # the score accumulator's elements 8 s .. 8 s + 7 (rows 8 (e / 4) +
    # 4 (l / 32) + e % 4 of the 32x32 block)
    img = tile_image(d, 3)
    for kb in range(BK // 32):
        for s in range(2):
            for db in range(d // 32):
                for t in range(2):
                    got = tr_read(img, tkg.attn_lds_offsets(d, 1, kb, s, t, db))
                    for lane in range(64):
                        for jj in range(4):
                            key = 32 * kb + 16 * s + 8 * t + 4 * (lane // 32) + jj
                            assert got[lane, jj] == key * d + 32 * db + lane % 32
                # the accumulator row of element e = 8 s + j is this key
                for lane in range(64):
                    for j in range(8):
                        e = 8 * s + j
                        acc_key = 8 * (e // 4) + 4 * (lane // 32) + e % 4
                        slot_key = 16 * s + 8 * (j // 4) + 4 * (lane // 32) + j % 4
                        assert acc_key == slot_key


def test_argument_errors():
    with pytest.raises(tkg.TkgError):
        tkg.attn_lds_offsets(96, 0, 0, 0)
    with pytest.raises(tkg.TkgError):
        tkg.attn_lds_offsets(64, 0, 1, 0)
    with pytest.raises(tkg.TkgError):
        tkg.attn_lds_offsets(128, 1, 0, 0, 0, 4)
    with pytest.raises(tkg.TkgError):
        tkg.attn_lds_offsets(64, 2, 4)


@pytest.mark.parametrize("d", [64, 128])
def test_kernel_address_decomposition(d):
    # the kernel forms every read address from one per-lane base with a
    # compile-time XOR and a compile-time add
    k0 = tkg.attn_lds_offsets(d, 0, 0, 0)
    for kb in range(BK // 32):
        for ks in range(d // 16):
            want = [(k0[l] ^ (32 * ks)) + 32 * kb * 2 * d for l in range(64)]
            assert tkg.attn_lds_offsets(d, 0, kb, ks) == want
    v0 = tkg.attn_lds_offsets(d, 1, 0, 0, 0, 0)
    for kb in range(BK // 32):
        for s in range(2):
            for t in range(2):
                for db in range(d // 32):
                    want = [(v0[l] ^ (64 * db)) + (32 * kb + 16 * s + 8 * t) * 2 * d
                            for l in range(64)]
                    assert tkg.attn_lds_offsets(d, 1, kb, s, t, db) == want
