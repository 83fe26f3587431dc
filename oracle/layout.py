"""int3 packed weight layout, version 1 (oracle implementation of the spec).

[talk] MiLo Kernel, "Bit Packing": 32 three-bit values are stored in three
32-bit words with no bit wasted.  This layout keeps that density (a *triplet*
of 3 words holds 32 codes of one row) but uses its own bit assignment, chosen
for 16-byte coalesced loads and the 16x16x32 f16 matrix-core operand order on
gfx950.  The spec (the GPU packer is written separately from the same text):

Matrix of R rows (output features) and K columns (input features),
R % 64 == 0, K % 128 == 0.

Tiles.  Tile (rt, kb) covers rows [64 rt, 64 rt + 64) and k in
[128 kb, 128 kb + 128).  Tile index t = rt * (K / 128) + kb; its 768 words
sit at words [768 t, 768 t + 768).

Within a tile, word index 256 p + 4 L + i for plane p in 0..2, lane L in 0..63,
row-group i in 0..3.  The three words (p = 0, 1, 2) with the same (L, i) form a
triplet:
    row  r = 64 rt + 16 i + (L mod 16)
    code c in 0..31 of the triplet has
         k = 128 kb + 32 (c div 8) + 8 (L div 16) + (c mod 8).

Bits of a triplet.  Code c belongs to pair pi = c div 2 and half h = c mod 2.
    pi < 15: plane p = pi div 5, slot o = pi mod 5; the code occupies bits
             [16 h + 1 + 3 o, 16 h + 4 + 3 o) of word p (least significant bit
             first).
    pi = 15: (codes 30 and 31) bit b (b = 0, 1, 2) of code 30 + h is bit 16 h of
             word p = b.
All 96 bits are used exactly once.

Scale/zero tiling.  For row r and group gg = k div 64, one 32-bit word holds
the float16 bits of the scale (low half) and the zero point (high half), at
word index 128 t + 8 (r mod 16) + 2 ((r mod 64) div 16) + (gg mod 2), with
t = (r div 64) * (K / 128) + gg div 2.
"""
import numpy as np

LAYOUT_VERSION = 1


def packed_words(R: int, K: int) -> int:
    return 3 * R * K // 32


def _check(R, K):
    if R % 64 or K % 128:
        raise ValueError("layout v1 needs rows % 64 == 0 and K % 128 == 0")


def _gather_index(R, K):
    """row/col index arrays of shape [RT, KB, 64 (L), 4 (i), 32 (c)]."""
    RT, KB = R // 64, K // 128
    rt = np.arange(RT)[:, None, None, None, None]
    kb = np.arange(KB)[None, :, None, None, None]
    L = np.arange(64)[None, None, :, None, None]
    i = np.arange(4)[None, None, None, :, None]
    c = np.arange(32)[None, None, None, None, :]
    row = 64 * rt + 16 * i + (L % 16)
    col = 128 * kb + 32 * (c // 8) + 8 * (L // 16) + (c % 8)
    row, col = np.broadcast_arrays(row, col)
    return row, col


def pack_v1(codes) -> np.ndarray:
    """codes uint8 [R][K] (values 0..7) -> uint32 words [3 R K / 32]."""
    codes = np.asarray(codes)
    R, K = codes.shape
    _check(R, K)
    if codes.max(initial=0) > 7:
        raise ValueError("codes must be in 0..7")
    RT, KB = R // 64, K // 128
    row, col = _gather_index(R, K)
    q = codes[row, col].astype(np.uint32)          # [RT, KB, 64, 4, 32]
    planes = np.zeros((RT, KB, 3, 64, 4), dtype=np.uint32)
    for c in range(32):
        pi, h = c // 2, c % 2
        qc = q[..., c]                              # [RT, KB, 64, 4]
        if pi < 15:
            p, o = pi // 5, pi % 5
            planes[:, :, p] |= qc << np.uint32(16 * h + 1 + 3 * o)
        else:
            for b in range(3):
                planes[:, :, b] |= ((qc >> np.uint32(b)) & np.uint32(1)) << np.uint32(16 * h)
    # word index within tile = 256 p + 4 L + i  ->  planes[rt, kb, p, L, i] is
    # already in that order.
    return planes.reshape(-1)


def unpack_v1(words, R: int, K: int) -> np.ndarray:
    """Inverse of pack_v1."""
    _check(R, K)
    RT, KB = R // 64, K // 128
    words = np.asarray(words, dtype=np.uint32)
    if words.size != packed_words(R, K):
        raise ValueError("wrong number of packed words")
    planes = words.reshape(RT, KB, 3, 64, 4)
    q = np.zeros((RT, KB, 64, 4, 32), dtype=np.uint32)
    for c in range(32):
        pi, h = c // 2, c % 2
        if pi < 15:
            p, o = pi // 5, pi % 5
            q[..., c] = (planes[:, :, p] >> np.uint32(16 * h + 1 + 3 * o)) & np.uint32(7)
        else:
            v = np.zeros((RT, KB, 64, 4), dtype=np.uint32)
            for b in range(3):
                v |= ((planes[:, :, b] >> np.uint32(16 * h)) & np.uint32(1)) << np.uint32(b)
            q[..., c] = v
    row, col = _gather_index(R, K)
    out = np.zeros((R, K), dtype=np.uint8)
    out[row, col] = q.astype(np.uint8)
    return out


def _locate(r: int, k: int, K: int):
    """Spec read backwards: where does code (r, k) live?  Returns (tile, L, i, c)."""
    rt, rr = divmod(r, 64)
    i, r16 = divmod(rr, 16)
    kb, kk = divmod(k, 128)
    step, rem = divmod(kk, 32)
    kq, t8 = divmod(rem, 8)
    L = 16 * kq + r16
    c = 8 * step + t8
    tile = rt * (K // 128) + kb
    return tile, L, i, c


def pack_v1_scalar(codes) -> list:
    """Pure-Python, one code at a time (for tiny shapes): walks (r, k), finds
    the code's triplet and bit positions from the spec, sets the bits."""
    R = len(codes)
    K = len(codes[0])
    _check(R, K)
    words = [0] * packed_words(R, K)
    for r in range(R):
        for k in range(K):
            v = int(codes[r][k])
            tile, L, i, c = _locate(r, k, K)
            pi, h = divmod(c, 2)
            base = 768 * tile + 4 * L + i
            if pi < 15:
                p, o = divmod(pi, 5)
                words[base + 256 * p] |= v << (16 * h + 1 + 3 * o)
            else:
                for b in range(3):
                    words[base + 256 * b] |= ((v >> b) & 1) << (16 * h)
    return words


def unpack_v1_scalar(words, R: int, K: int) -> list:
    _check(R, K)
    out = [[0] * K for _ in range(R)]
    for r in range(R):
        for k in range(K):
            tile, L, i, c = _locate(r, k, K)
            pi, h = divmod(c, 2)
            base = 768 * tile + 4 * L + i
            if pi < 15:
                p, o = divmod(pi, 5)
                out[r][k] = (int(words[base + 256 * p]) >> (16 * h + 1 + 3 * o)) & 7
            else:
                v = 0
                for b in range(3):
                    v |= ((int(words[base + 256 * b]) >> (16 * h)) & 1) << b
                out[r][k] = v
    return out


def pack_sz_v1(scale, zero) -> np.ndarray:
    """scale, zero fp16 [R][K/64] -> uint32 [R K / 64] tiled per the spec."""
    s = np.asarray(scale, dtype=np.float16).view(np.uint16).astype(np.uint32)
    z = np.asarray(zero, dtype=np.float16).view(np.uint16).astype(np.uint32)
    R, G = s.shape
    K = 64 * G
    _check(R, K)
    out = np.zeros(R * G, dtype=np.uint32)
    r = np.arange(R)[:, None]
    gg = np.arange(G)[None, :]
    t = (r // 64) * (K // 128) + gg // 2
    idx = 128 * t + 8 * (r % 16) + 2 * ((r % 64) // 16) + (gg % 2)
    out[idx] = s | (z << np.uint32(16))
    return out


def unpack_sz_v1(words, R: int, K: int):
    _check(R, K)
    G = K // 64
    words = np.asarray(words, dtype=np.uint32)
    r = np.arange(R)[:, None]
    gg = np.arange(G)[None, :]
    t = (r // 64) * (K // 128) + gg // 2
    idx = 128 * t + 8 * (r % 16) + 2 * ((r % 64) // 16) + (gg % 2)
    w = words[idx]
    s = (w & np.uint32(0xFFFF)).astype(np.uint16).view(np.float16)
    z = (w >> np.uint32(16)).astype(np.uint16).view(np.float16)
    return s, z
