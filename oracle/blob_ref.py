"""Independent reader/writer of the fixed-stride expert blob (TEST INFRASTRUCTURE ONLY).

The pages store every routed expert as one fixed-stride blob so that fetching
an expert is a single read (Show HN page, how-it-works list; creativeainews
explainer, "How Expert Streaming Works").  They do not give the bytes inside a
blob; the layout below is this project's own, documented in the public C
header, and this module reads it from that written description alone.
Parity status: pinned by hand-placed bytes and round trips in
tests/test_oracle_blob.py.

Layout of one expert with hidden size H, intermediate size I, group size G
(H % 64 == 0, I % 64 == 0, G in {32, 64, 128} dividing H and I):

  section  offset            size        contents
  GU_Q     0                 I*H         gate/up nibbles, pair-tiles p < I/16
  D_Q      I*H               H*I/2       down nibbles, pair-tiles p < H/32
  GU_S     3*I*H/2           8*I*H/G     gate/up fp16 scale/bias
  D_S      3*I*H/2+8*I*H/G   4*H*I/G     down fp16 scale/bias

A pair-tile joins two 16-row tiles of one matrix product: for GU_Q tile A is
gate rows 16p..16p+15 and tile B is up rows 16p..16p+15; for D_Q tile A is
down rows 32p..32p+15 and tile B is down rows 32p+16..32p+31.  Each pair-tile
covers the input dimension in chunks of 64 columns; chunk c of pair-tile p is
a 1024-byte block at ((p * n_chunks) + c) * 1024.  Byte 16*l of that block
starts lane l's four little-endian 32-bit words (n = l % 16, kb = l // 16):

  word 0: tile A row n, columns 64c +      8kb + j   (j = 0..7)
  word 1: tile A row n, columns 64c + 32 + 8kb + j
  word 2: tile B row n, columns 64c +      8kb + j
  word 3: tile B row n, columns 64c + 32 + 8kb + j

and value j of a word sits in bits [4p, 4p+4) with p = (j >> 1) + 4*(j & 1).

int8 experts (bits = 8) double the value sections: GU_Q is 2*I*H bytes and
D_Q is I*H; the scale sections follow at 3*I*H and 3*I*H + 8*I*H/G.  A chunk
is then a 2048-byte block of two 1024-byte planes, tile A first.  In plane
`tile`, lane l owns the 16 bytes at 16*l: the 8 values of half ks = 0, then
the 8 of half ks = 1 (columns 64c + 32ks + 8kb + j as above), value j as byte
j of its 8 in natural order.  So byte 1024*tile + 16*l + 8*ks + j of the block.

The scale/bias sections hold, for pair-tile p, group g (G columns of the
input dimension) and n < 16, eight bytes at ((p * n_groups + g) * 16 + n) * 8:
four fp16 values [s_A, b_A, s_B, b_B] for row n of tiles A and B.
"""
from __future__ import annotations

import numpy as np

# nibble position of the j-th value of a 32-bit word
NIBBLE_OF_VALUE = np.array([(j >> 1) + 4 * (j & 1) for j in range(8)], dtype=np.int64)


def check_shape(hidden: int, inter: int, group: int) -> None:
    if hidden <= 0 or inter <= 0 or hidden % 64 or inter % 64:
        raise ValueError("hidden and inter must be positive multiples of 64")
    if group not in (32, 64, 128) or hidden % group or inter % group:
        raise ValueError("group must be 32, 64 or 128 and divide hidden and inter")


def section_offsets(hidden: int, inter: int, group: int, bits: int = 4):
    check_shape(hidden, inter, group)
    if bits not in (4, 8):
        raise ValueError("bits must be 4 or 8")
    gu_q = 0
    d_q = inter * hidden * bits // 4
    gu_s = d_q + hidden * inter * bits // 8
    d_s = gu_s + 8 * inter * hidden // group
    end = d_s + 4 * hidden * inter // group
    return dict(gu_q=gu_q, d_q=d_q, gu_s=gu_s, d_s=d_s, end=end)


def blob_bytes(hidden: int, inter: int, group: int, bits: int = 4) -> int:
    return section_offsets(hidden, inter, group, bits)["end"]


def _words_to_values(words: np.ndarray) -> np.ndarray:
    """uint32 words [...] -> values [..., 8] in value order j."""
    shifts = (4 * NIBBLE_OF_VALUE).astype(np.uint32)
    return ((words[..., None] >> shifts) & np.uint32(0xF)).astype(np.uint8)


def _values_to_words(vals: np.ndarray) -> np.ndarray:
    """values [..., 8] (0..15) -> uint32 words, inverse of _words_to_values."""
    shifts = (4 * NIBBLE_OF_VALUE).astype(np.uint32)
    return np.bitwise_or.reduce(vals.astype(np.uint32) << shifts, axis=-1).astype(np.uint32)


def _parse_pair_tiles(raw: np.ndarray, n_pairs: int, in_dim: int, bits: int = 4):
    """Value section -> (tile-A values, tile-B values), each [n_pairs*16, in_dim]."""
    n_chunks = in_dim // 64
    if bits == 8:
        vals = raw.reshape(n_pairs, n_chunks, 2, 4, 16, 2, 8)         # p, c, tile, kb, n, ks, j
        vals = vals.transpose(0, 1, 3, 4, 2, 5, 6)                    # p, c, kb, n, tile, ks, j
    else:
        words = raw.view("<u4").reshape(n_pairs, n_chunks, 4, 16, 4)  # p, c, kb, n, word
        vals = _words_to_values(words)                                # p, c, kb, n, word, j
        vals = vals.reshape(n_pairs, n_chunks, 4, 16, 2, 2, 8)       # p, c, kb, n, tile, ks, j
    # row = (p, tile, n); column = 64c + 32ks + 8kb + j
    arr = vals.transpose(0, 4, 3, 1, 5, 2, 6)                        # p, tile, n, c, ks, kb, j
    return arr.reshape(n_pairs, 2, 16, in_dim)


def _pack_pair_tiles(tile_a: np.ndarray, tile_b: np.ndarray, n_pairs: int, in_dim: int, bits: int = 4) -> np.ndarray:
    n_chunks = in_dim // 64
    both = np.stack([tile_a.reshape(n_pairs, 16, in_dim), tile_b.reshape(n_pairs, 16, in_dim)], axis=1)
    arr = both.reshape(n_pairs, 2, 16, n_chunks, 2, 4, 8)            # p, tile, n, c, ks, kb, j
    if bits == 8:
        planes = arr.transpose(0, 3, 1, 5, 2, 4, 6)                  # p, c, tile, kb, n, ks, j
        return np.ascontiguousarray(planes).astype(np.uint8).reshape(-1)
    vals = arr.transpose(0, 3, 5, 2, 1, 4, 6)                        # p, c, kb, n, tile, ks, j
    words = _values_to_words(vals.reshape(n_pairs, n_chunks, 4, 16, 4, 8))
    return words.astype("<u4").view(np.uint8).reshape(-1)


def _parse_scales(raw: np.ndarray, n_pairs: int, n_groups: int):
    """Scale section -> (s, b) each [n_pairs, 2 (tile), 16, n_groups] fp16 bits."""
    arr = raw.view("<u2").reshape(n_pairs, n_groups, 16, 2, 2)       # p, g, n, tile, (s|b)
    arr = arr.transpose(0, 3, 2, 1, 4)                               # p, tile, n, g, (s|b)
    return arr[..., 0], arr[..., 1]


def _pack_scales(s: np.ndarray, b: np.ndarray, n_pairs: int, n_groups: int) -> np.ndarray:
    arr = np.stack([s, b], axis=-1).reshape(n_pairs, 2, 16, n_groups, 2)
    arr = arr.transpose(0, 3, 2, 1, 4).astype("<u2")                 # p, g, n, tile, (s|b)
    return arr.view(np.uint8).reshape(-1)


def parse_blob(buf, hidden: int, inter: int, group: int, bits: int = 4):
    """Blob bytes -> dict(gate=(q,s,b), up=(q,s,b), down=(q,s,b)).

    gate/up q: [I, H] uint8, s/b: [I, H/G] fp16 bits; down q: [H, I], s/b: [H, I/G].
    """
    off = section_offsets(hidden, inter, group, bits)
    raw = np.frombuffer(bytes(buf) if not isinstance(buf, np.ndarray) else buf.tobytes(), dtype=np.uint8)
    if raw.size < off["end"]:
        raise ValueError("blob too short")
    gu = _parse_pair_tiles(raw[off["gu_q"]:off["d_q"]].copy(), inter // 16, hidden, bits)
    dn = _parse_pair_tiles(raw[off["d_q"]:off["gu_s"]].copy(), hidden // 32, inter, bits)
    gs, gb = _parse_scales(raw[off["gu_s"]:off["d_s"]].copy(), inter // 16, hidden // group)
    ds, db = _parse_scales(raw[off["d_s"]:off["end"]].copy(), hidden // 32, inter // group)
    gate = (gu[:, 0].reshape(inter, hidden), gs[:, 0].reshape(inter, -1), gb[:, 0].reshape(inter, -1))
    up = (gu[:, 1].reshape(inter, hidden), gs[:, 1].reshape(inter, -1), gb[:, 1].reshape(inter, -1))
    down = (dn.reshape(hidden, inter), ds.reshape(hidden, -1), db.reshape(hidden, -1))
    return dict(gate=gate, up=up, down=down)


def pack_blob(gate, up, down, hidden: int, inter: int, group: int, bits: int = 4) -> np.ndarray:
    """Inverse of parse_blob (used to pin the reader by round trips)."""
    off = section_offsets(hidden, inter, group, bits)
    out = np.zeros(off["end"], dtype=np.uint8)
    out[off["gu_q"]:off["d_q"]] = _pack_pair_tiles(np.asarray(gate[0]), np.asarray(up[0]), inter // 16, hidden, bits)
    dq = np.asarray(down[0]).reshape(hidden // 32, 2, 16, inter)
    out[off["d_q"]:off["gu_s"]] = _pack_pair_tiles(dq[:, 0], dq[:, 1], hidden // 32, inter, bits)
    ng = hidden // group
    s_gu = np.stack([np.asarray(gate[1]).reshape(inter // 16, 16, ng), np.asarray(up[1]).reshape(inter // 16, 16, ng)], 1)
    b_gu = np.stack([np.asarray(gate[2]).reshape(inter // 16, 16, ng), np.asarray(up[2]).reshape(inter // 16, 16, ng)], 1)
    out[off["gu_s"]:off["d_s"]] = _pack_scales(s_gu, b_gu, inter // 16, ng)
    ngd = inter // group
    s_d = np.asarray(down[1]).reshape(hidden // 32, 2, 16, ngd)
    b_d = np.asarray(down[2]).reshape(hidden // 32, 2, 16, ngd)
    out[off["d_s"]:off["end"]] = _pack_scales(s_d, b_d, hidden // 32, ngd)
    return out
