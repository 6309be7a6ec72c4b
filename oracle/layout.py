"""Packed expert blob (oracle's own packer, written from the layout specification).

The pages say only that routed experts are packed once into the form the kernel
consumes and that a cache miss moves "packed weights and scales" (ExactMoE abstract;
Fig. 1 caption). The form used here is this project's gfx950 tile layout:

Blob = [int4 tiles: n_tiles * 1024 B][bf16 scales: n_tiles * 32 B],
n_tiles = 2*(I/16)*(H/128) + (H/16)*(I/128), size = 3HI/2 + 3HI/64 bytes.

Tile order: first gate/up -- for row block b in 0..I/16-1, for matrix in (gate, up), for
input group g in 0..H/128-1 -- then down -- for row block b in 0..H/16-1, for group g in
0..I/128-1. A tile covers output rows 16b..16b+15 and inputs 128g..128g+127 of its matrix.

Inside a tile, byte 16*l + 4*s (lane l in 0..63, word s in 0..3) starts a little-endian
32-bit word holding row 16b + (l % 16), inputs 128g + 32s + 8*(l // 16) + j, j = 0..7,
as nibbles u = q + 8: input j sits at bits 4*(j//2) (j even) or 16 + 4*(j//2) (j odd).

Scales of tile t: 16 little-endian bf16 values (rows 0..15 of the tile) at byte
1024*n_tiles + 32*t + 2*r.
"""
from __future__ import annotations

import numpy as np

TILE_ROWS = 16
GROUP = 128
TILE_BYTES = 1024
SCALE_BYTES = 32


def n_tiles(H: int, I: int) -> int:
    return 2 * (I // TILE_ROWS) * (H // GROUP) + (H // TILE_ROWS) * (I // GROUP)


def packed_expert_bytes(H: int, I: int) -> int:
    return n_tiles(H, I) * (TILE_BYTES + SCALE_BYTES)


def _tile_list(H: int, I: int):
    """[(matrix, row_block, group)] in blob order; matrix 0 gate, 1 up, 2 down."""
    tiles = []
    for b in range(I // TILE_ROWS):
        for mat in (0, 1):
            for g in range(H // GROUP):
                tiles.append((mat, b, g))
    for b in range(H // TILE_ROWS):
        for g in range(I // GROUP):
            tiles.append((2, b, g))
    return tiles


def _nibble_shift(j: int) -> int:
    return 4 * (j // 2) if j % 2 == 0 else 16 + 4 * (j // 2)


def _tile_words(q_tile: np.ndarray) -> np.ndarray:
    """q_tile int8 [16, 128] -> uint32 [64 lanes, 4 words]."""
    u = (q_tile.astype(np.int32) + 8).astype(np.uint32)
    words = np.zeros((64, 4), dtype=np.uint32)
    for l in range(64):
        r = l % 16
        for s in range(4):
            w = 0
            for j in range(8):
                w |= int(u[r, 32 * s + 8 * (l // 16) + j]) << _nibble_shift(j)
            words[l, s] = w
    return words


def _tile_words_fast(q_blocks: np.ndarray) -> np.ndarray:
    """Vectorized form of _tile_words over a stack: int8 [n, 16, 128] -> uint32 [n, 64, 4].
    Tests check it equals the per-element loop above on random tiles."""
    n = q_blocks.shape[0]
    u = (q_blocks.astype(np.int32) + 8).astype(np.uint32)
    # index K = 32 s + 8 (l // 16) + j  ->  u[:, r, s, l//16, j]
    u5 = u.reshape(n, 16, 4, 4, 8)          # [n, r, s, lg, j]
    words = np.zeros((n, 4, 16, 4), dtype=np.uint32)   # [n, lg, r, s]  (lane = 16*lg + r)
    for j in range(8):
        words |= np.transpose(u5[:, :, :, :, j], (0, 3, 1, 2)) << np.uint32(_nibble_shift(j))
    return words.reshape(n, 64, 4)


def pack_expert(qg, sg, qu, su, qd, sd, H: int, I: int, fast: bool = True) -> bytes:
    """Quantized expert -> blob bytes.

    qg, qu int8 [I, H] with scales sg, su bf16 bits [I, H/128]; qd int8 [H, I] with
    sd [H, I/128].
    """
    assert H % GROUP == 0 and I % GROUP == 0
    mats_q = (qg, qu, qd)
    mats_s = (sg, su, sd)
    tiles = _tile_list(H, I)
    nt = len(tiles)
    qt = np.empty((nt, TILE_ROWS, GROUP), dtype=np.int8)
    st = np.empty((nt, TILE_ROWS), dtype=np.uint16)
    for t, (mat, b, g) in enumerate(tiles):
        qt[t] = mats_q[mat][TILE_ROWS * b:TILE_ROWS * (b + 1), GROUP * g:GROUP * (g + 1)]
        st[t] = mats_s[mat][TILE_ROWS * b:TILE_ROWS * (b + 1), g]
    if fast:
        words = _tile_words_fast(qt)
    else:
        words = np.stack([_tile_words(qt[t]) for t in range(nt)])
    return words.astype("<u4").tobytes() + st.astype("<u2").tobytes()


def unpack_expert(blob: bytes, H: int, I: int):
    """Blob -> (qg, sg, qu, su, qd, sd), the inverse of pack_expert."""
    nt = n_tiles(H, I)
    assert len(blob) == packed_expert_bytes(H, I)
    words = np.frombuffer(blob, dtype="<u4", count=nt * 256).reshape(nt, 4, 16, 4)  # [t, lg, r, s]
    st = np.frombuffer(blob, dtype="<u2", offset=nt * TILE_BYTES).reshape(nt, TILE_ROWS)
    u = np.zeros((nt, 16, 4, 4, 8), dtype=np.int32)   # [t, r, s, lg, j]
    for j in range(8):
        nib = (words >> np.uint32(_nibble_shift(j))) & np.uint32(0xF)
        u[:, :, :, :, j] = np.transpose(nib, (0, 2, 3, 1))
    qt = (u - 8).reshape(nt, 16, 128).astype(np.int8)
    qg = np.empty((I, H), np.int8); qu = np.empty((I, H), np.int8); qd = np.empty((H, I), np.int8)
    sg = np.empty((I, H // GROUP), np.uint16); su = np.empty_like(sg); sd = np.empty((H, I // GROUP), np.uint16)
    mats_q = (qg, qu, qd)
    mats_s = (sg, su, sd)
    for t, (mat, b, g) in enumerate(_tile_list(H, I)):
        mats_q[mat][TILE_ROWS * b:TILE_ROWS * (b + 1), GROUP * g:GROUP * (g + 1)] = qt[t]
        mats_s[mat][TILE_ROWS * b:TILE_ROWS * (b + 1), g] = st[t]
    return qg, sg, qu, su, qd, sd


# ---------------------------------------------------------------------------- dense bf16 blob
# The comparator layer runs the same experts with bf16 weights (abstract; Tab. 1 and Tab. 4,
# the BF16 rows). Its blob (this project's layout) holds 1 KiB tiles of 16 rows x 32 inputs
# and no scales: first, for row block b in 0..I/16-1, the gate tiles c in 0..H/32-1 and then
# the up tiles; then, for row block b in 0..H/16-1, the down tiles c in 0..I/32-1. Bytes
# 16*l .. 16*l+15 of a tile hold row 16b + l % 16, inputs 32c + 8*(l // 16) + j (j = 0..7)
# as little-endian bf16.
def bf16_expert_bytes(H: int, I: int) -> int:
    return 6 * H * I


def pack_expert_bf16(g_bits: np.ndarray, u_bits: np.ndarray, d_bits: np.ndarray) -> bytes:
    """bf16 bits gate [I,H], up [I,H], down [H,I] -> blob bytes, one tile at a time."""
    I, H = g_bits.shape
    out = np.empty(bf16_expert_bytes(H, I) // 2, dtype=np.uint16)
    pos = 0

    def tile(W, b, c):
        nonlocal pos
        blk = W[16 * b:16 * b + 16, 32 * c:32 * c + 32]          # [16 rows, 32 inputs]
        for l in range(64):
            out[pos + 8 * l: pos + 8 * l + 8] = blk[l % 16, 8 * (l // 16): 8 * (l // 16) + 8]
        pos += 512

    for b in range(I // 16):
        for W in (g_bits, u_bits):
            for c in range(H // 32):
                tile(W, b, c)
    for b in range(H // 16):
        for c in range(I // 32):
            tile(d_bits, b, c)
    assert pos == out.size
    return out.astype("<u2").tobytes()

