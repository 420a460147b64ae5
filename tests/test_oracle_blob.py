"""Pins of the oracle's blob reader: hand-placed bytes and round trips."""
import numpy as np
import pytest

from oracle import blob_ref


def test_sizes_closed_form():
    # 3*I*H/2 nibble bytes + 3 matrices * (I*H/G) groups * (s, b) * 2 bytes
    assert blob_ref.blob_bytes(2048, 512, 64) == 1_769_472 == 432 * 4096
    assert blob_ref.blob_bytes(256, 64, 32) == 30_720
    off = blob_ref.section_offsets(2048, 512, 64)
    assert off == dict(gu_q=0, d_q=1_048_576, gu_s=1_572_864, d_s=1_703_936, end=1_769_472)
    for v in off.values():
        assert v % 256 == 0


@pytest.mark.parametrize("bad", [(100, 64, 32), (256, 96, 32), (256, 64, 48), (256, 64, 128)])
def test_bad_shapes(bad):
    with pytest.raises(ValueError):
        blob_ref.section_offsets(*bad)


def _empty(h, i, g):
    z = lambda r, c: np.zeros((r, c), np.uint8)  # noqa: E731
    zs = lambda r, c: np.zeros((r, c // g), np.uint16)  # noqa: E731
    return dict(gate=(z(i, h), zs(i, h), zs(i, h)), up=(z(i, h), zs(i, h), zs(i, h)),
                down=(z(h, i), zs(h, i), zs(h, i)))


def test_hand_placed_nibbles():
    h, i, g = 128, 64, 32
    buf = np.zeros(blob_ref.blob_bytes(h, i, g), np.uint8)
    # gate q[17, 75] = 9: pair-tile p = 1, row n = 1, chunk c = 1 (cols 64..127),
    # column 75 = 64 + 0*32 + 1*8 + 3 -> ks = 0, kb = 1, j = 3 -> nibble 1 + 4 = 5.
    # lane l = 16*kb + n = 17; word 0 (tile A, ks 0).  Block (p*2 + c) = 3.
    # byte = 3*1024 + 17*16 + 0*4 + 5//2 = 3072 + 272 + 2 = 3346, high nibble.
    buf[3346] = 9 << 4
    # up q[2, 40] = 6: p = 0, n = 2, c = 0, 40 = 32 + 8*1 + 0 -> ks 1, kb 1, j 0 -> nibble 0;
    # lane 18, word 3 (tile B, ks 1) -> byte 0*1024 + 18*16 + 12 = 300, low nibble.
    buf[300] = 6
    # down q[47, 10] = 15: pair-tile p = 1 (rows 32..63), tile B (rows 48..63)? no:
    # row 47 = 32*1 + 15 -> tile A, n = 15.  Column 10 = 0*32 + 8*1 + 2 -> c 0, ks 0, kb 1,
    # j 2 -> nibble 1.  D_Q starts at I*H = 8192; pair-tile 1 chunk 0 -> block 1.
    # lane 31, word 0 -> byte 8192 + 1024 + 31*16 + 0 = 9712, high nibble of byte 0.
    buf[9712] = 15 << 4
    # down q[63, 63] = 1: row 63 = 32 + 16 + 15 -> tile B, n 15; col 63 = 32 + 24 + 7 ->
    # ks 1, kb 3, j 7 -> nibble 3 + 4 = 7 (high nibble of byte 3); lane 63, word 3.
    # byte = 8192 + 1024 + 63*16 + 12 + 3 = 10239.
    buf[10239] = 1 << 4
    p = blob_ref.parse_blob(buf, h, i, g)
    gate_q, up_q, down_q = p["gate"][0], p["up"][0], p["down"][0]
    assert gate_q[17, 75] == 9 and np.count_nonzero(gate_q) == 1
    assert up_q[2, 40] == 6 and np.count_nonzero(up_q) == 1
    assert down_q[47, 10] == 15 and down_q[63, 63] == 1 and np.count_nonzero(down_q) == 2


def test_hand_placed_scales():
    h, i, g = 128, 64, 32
    off = blob_ref.section_offsets(h, i, g)
    buf = np.zeros(off["end"], np.uint8)
    u16 = buf.view(np.uint16)
    # up bias of row 21, group 3: pair-tile 1, n 5, (H/G) = 4 groups -> entry
    # ((1*4 + 3)*16 + 5) = 117, fp16 slot 3 (b_B) -> byte gu_s + 117*8 + 6.
    u16[(off["gu_s"] + 117 * 8 + 6) // 2] = 0x1234
    # down scale of row 50, group 1: pair-tile 1, tile B (50 = 32+16+2), n 2,
    # (I/G) = 2 groups -> entry ((1*2 + 1)*16 + 2) = 50, slot 2 (s_B).
    u16[(off["d_s"] + 50 * 8 + 4) // 2] = 0x2345
    p = blob_ref.parse_blob(buf, h, i, g)
    assert p["up"][2][21, 3] == 0x1234 and np.count_nonzero(p["up"][2]) == 1
    assert p["down"][1][50, 1] == 0x2345 and np.count_nonzero(p["down"][1]) == 1
    assert np.count_nonzero(p["gate"][1]) == 0 and np.count_nonzero(p["down"][2]) == 0


@pytest.mark.parametrize("shape", [(256, 64, 32), (128, 128, 64), (256, 128, 128), (2048, 512, 64)])
def test_round_trip(shape):
    h, i, g = shape
    rng = np.random.default_rng(h + i + g)
    m = {}
    for name, rows, cols in (("gate", i, h), ("up", i, h), ("down", h, i)):
        m[name] = (rng.integers(0, 16, (rows, cols)).astype(np.uint8),
                   rng.integers(0, 65536, (rows, cols // g)).astype(np.uint16),
                   rng.integers(0, 65536, (rows, cols // g)).astype(np.uint16))
    buf = blob_ref.pack_blob(m["gate"], m["up"], m["down"], h, i, g)
    assert buf.size == blob_ref.blob_bytes(h, i, g)
    p = blob_ref.parse_blob(buf, h, i, g)
    for name in m:
        for a, b in zip(m[name], p[name]):
            assert np.array_equal(a, b)
    # and bytes -> values -> bytes
    assert np.array_equal(blob_ref.pack_blob(p["gate"], p["up"], p["down"], h, i, g), buf)


def test_value_order_in_word():
    # value j sits in nibble (j >> 1) + 4*(j & 1): j = 0..7 -> 0,4,1,5,2,6,3,7
    assert blob_ref.NIBBLE_OF_VALUE.tolist() == [0, 4, 1, 5, 2, 6, 3, 7]
    words = np.array([0x76543210], np.uint32)
    assert blob_ref._words_to_values(words)[0].tolist() == [0, 4, 1, 5, 2, 6, 3, 7]


# ---- int8 experts: value sections twice as wide, bytes in natural order ----

def test_int8_sizes_closed_form():
    # 3*I*H value bytes + the same scale sections as int4
    assert blob_ref.blob_bytes(2048, 512, 64, bits=8) == 3 * 512 * 2048 + 12 * 512 * 2048 // 64 == 3_342_336
    off = blob_ref.section_offsets(2048, 512, 64, bits=8)
    assert off == dict(gu_q=0, d_q=2_097_152, gu_s=3_145_728, d_s=3_276_800, end=3_342_336)
    with pytest.raises(ValueError):
        blob_ref.section_offsets(256, 64, 32, bits=6)


def test_int8_hand_placed_bytes():
    h, i, g = 128, 64, 32
    buf = np.zeros(blob_ref.blob_bytes(h, i, g, bits=8), np.uint8)
    # byte of (tile, lane l, ks, j) in a 2048-byte chunk block: 1024*tile + 16*l + 8*ks + j
    # gate q[5, 115] = 0xAB: pair-tile p = 0, tile A, row n = 5, chunk c = 1 (cols 64..127),
    # 115 = 64 + 32 + 8*2 + 3 -> ks = 1, kb = 2, j = 3; lane l = 16*2 + 5 = 37.
    # Block p*2 + c = 1 -> byte 1*2048 + 0 + 37*16 + 8 + 3 = 2651.
    buf[2651] = 0xAB
    # up q[20, 7] = 0x5C: p = 1, tile B, n = 4, c = 0, 7 = 0 + 8*0 + 7 -> ks 0, kb 0, j 7;
    # lane 4; block 1*2 + 0 = 2 -> byte 2*2048 + 1024 + 4*16 + 0 + 7 = 5191.
    buf[5191] = 0x5C
    # down q[40, 33] = 0xFF: pair-tile p = 1 (rows 32..63), tile A = rows 32..47 -> n = 8;
    # in_dim = 64: c = 0, 33 = 32 + 0*8 + 1 -> ks 1, kb 0, j 1; lane 8.
    # D_Q starts at 2*I*H = 16384; block p*1 + c = 1 -> 16384 + 2048 + 0 + 8*16 + 8 + 1 = 18569.
    buf[18569] = 0xFF
    r = blob_ref.parse_blob(buf, h, i, g, bits=8)
    gate, up, down = r["gate"][0], r["up"][0], r["down"][0]
    assert gate[5, 115] == 0xAB and int(gate.sum()) == 0xAB
    assert up[20, 7] == 0x5C and int(up.sum()) == 0x5C
    assert down[40, 33] == 0xFF and int(down.sum()) == 0xFF


@pytest.mark.parametrize("shape", [(128, 64, 32), (256, 128, 64), (320, 192, 64), (256, 128, 128)])
def test_int8_round_trip(shape):
    h, i, g = shape
    rng = np.random.default_rng(h + i + g)
    q = lambda r, c: rng.integers(0, 256, (r, c)).astype(np.uint8)  # noqa: E731
    sb = lambda r, c: rng.integers(0, 65536, (r, c // g)).astype(np.uint16)  # noqa: E731
    raw = dict(gate=(q(i, h), sb(i, h), sb(i, h)), up=(q(i, h), sb(i, h), sb(i, h)), down=(q(h, i), sb(h, i), sb(h, i)))
    buf = blob_ref.pack_blob(raw["gate"], raw["up"], raw["down"], h, i, g, bits=8)
    assert buf.size == blob_ref.blob_bytes(h, i, g, bits=8)
    back = blob_ref.parse_blob(buf, h, i, g, bits=8)
    for k in raw:
        for a, b in zip(raw[k], back[k]):
            assert np.array_equal(a, b)
