"""int3 compensators (oracle side): quantization of the low-rank factors and
their two packed layouts.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

[talk] MiLo Algorithm, last step, and Experimental Setup & Results,
"Compensator Quantization": after compensation the factors U and V are
themselves quantized to int3 with simple asymmetric linear quantization, at
almost no cost in accuracy.  The pages fix neither the grouping nor the
rounding; the reading used here is the weights' own RTN rule (oracle.quant:
float16 scale and zero point, round half to even), with groups along the
dimension each factor is summed over in x . W^T = x . deq(Wq)^T + (x V^T) U^T:

    V = A^T, R x K (contracted with the activations over K):
        groups of 64 consecutive k in each rank row j;
    U = B^T, N x R (contracted with t = x V^T over the ranks):
        one group per output row n holding that expert's r ranks (r <= 64).

Layouts (one expert; the spec the GPU packer is written from separately).
Both keep the weights' triplet: 32 codes in three 32-bit words with the bit
assignment of layout v1 (oracle/layout.py): code c = 2 pi + h, pair pi < 15 at
bits [16 h + 1 + 3 (pi mod 5), +3) of word pi div 5; pair 15: bit b of code
30 + h is bit 16 h of word b.

V layout.  max_rank rows (rank rows j; rows j >= rank are padding), each
the K / 32 triplets of that row in order tau = 4 kb + kq (kb = 0..K/128-1,
kq = 0..3).  Triplet tau of row j is at words [3 (j K/32 + tau), +3) (word p
of the triplet at offset p); its code c sits at k = 128 kb + 32 (c div 8) +
8 kq + (c mod 8).  Scale/zero of row j, group gg = k div 64: word
j (K / 64) + gg, scale bits low, zero bits high.  Rows j >= rank hold code 0
and the word 0x00003C00 (scale 1, zero 0).

U layout.  Ranks padded to R32 = max_rank rounded up to 32.  Tile (nt, jt)
covers rows n in [64 nt, 64 nt + 64) and ranks [32 jt, 32 jt + 32), tile index
t = nt (R32 / 32) + jt, 192 words.  Word 64 p + L is word p of the triplet
whose code c is U[n][j] with n = 64 nt + 16 (c div 8) + (L mod 16),
j = 32 jt + 8 (L div 16) + (c mod 8).  Ranks j >= rank hold code 0.  Scale/zero
(one group per row): word 64 (n div 64) + 4 (n mod 16) + (n mod 64) div 16.
"""
import numpy as np

from .quant import dequant_int3, quantize_rtn_int3

PAD_SZ_WORD = 0x00003C00   # float16 scale 1.0, zero 0.0


# ----------------------------------------------------------------------------
# quantization

def quantize_compensator(A, B):
    """A [K][r] and B [r][N] (the compensator as X A B, V = A^T, U = B^T).
    Returns a dict with
        v_codes uint8 [r][K], v_scale, v_zero fp16 [r][K/64]   (groups of 64 along K)
        u_codes uint8 [N][r], u_scale, u_zero fp16 [N][1]      (one group of r per row)
    For r = 0 every array is empty."""
    A = np.asarray(A)
    B = np.asarray(B)
    K, r = A.shape
    N = B.shape[1]
    if B.shape[0] != r:
        raise ValueError("A is K x r and B is r x N")
    if r == 0:
        return {"v_codes": np.zeros((0, K), np.uint8), "v_scale": np.zeros((0, K // 64), np.float16),
                "v_zero": np.zeros((0, K // 64), np.float16), "u_codes": np.zeros((N, 0), np.uint8),
                "u_scale": np.zeros((N, 1), np.float16), "u_zero": np.zeros((N, 1), np.float16)}
    if r > 64:
        raise ValueError("rank above 64")
    vq, vs, vz = quantize_rtn_int3(A.T.astype(np.float64), group=64)
    uq, us, uz = quantize_rtn_int3(B.T.astype(np.float64), group=r)
    return {"v_codes": vq, "v_scale": vs, "v_zero": vz, "u_codes": uq, "u_scale": us, "u_zero": uz}


def dequant_compensator(q):
    """Inverse of quantize_compensator up to the rounding: returns
    (A_deq [K][r], B_deq [r][N]) in float64."""
    vq, uq = q["v_codes"], q["u_codes"]
    r = vq.shape[0]
    K, N = vq.shape[1], uq.shape[0]
    if r == 0:
        return np.zeros((K, 0)), np.zeros((0, N))
    Vd = dequant_int3(vq, q["v_scale"], q["v_zero"], 64)
    Ud = dequant_int3(uq, q["u_scale"], q["u_zero"], r)
    return Vd.T, Ud.T


# ----------------------------------------------------------------------------
# triplet bits (the layout v1 rule), vectorised over leading axes

def _encode(q):
    """q uint [..., 32] codes -> uint32 [..., 3] words."""
    q = q.astype(np.uint32)
    w = np.zeros(q.shape[:-1] + (3,), dtype=np.uint32)
    for c in range(32):
        pi, h = divmod(c, 2)
        if pi < 15:
            p, o = divmod(pi, 5)
            w[..., p] |= q[..., c] << np.uint32(16 * h + 1 + 3 * o)
        else:
            for b in range(3):
                w[..., b] |= ((q[..., c] >> np.uint32(b)) & np.uint32(1)) << np.uint32(16 * h)
    return w


def _decode(w):
    """uint32 [..., 3] words -> uint8 [..., 32] codes."""
    w = w.astype(np.uint32)
    q = np.zeros(w.shape[:-1] + (32,), dtype=np.uint32)
    for c in range(32):
        pi, h = divmod(c, 2)
        if pi < 15:
            p, o = divmod(pi, 5)
            q[..., c] = (w[..., p] >> np.uint32(16 * h + 1 + 3 * o)) & np.uint32(7)
        else:
            for b in range(3):
                q[..., c] |= ((w[..., b] >> np.uint32(16 * h)) & np.uint32(1)) << np.uint32(b)
    return q.astype(np.uint8)


def _sz_word(scale, zero):
    s = np.asarray(scale, dtype=np.float16).view(np.uint16).astype(np.uint32)
    z = np.asarray(zero, dtype=np.float16).view(np.uint16).astype(np.uint32)
    return s | (z << np.uint32(16))


def _round_up(v, a):
    return (v + a - 1) // a * a


# ----------------------------------------------------------------------------
# V layout

def lr_v_words(max_rank: int, K: int) -> int:
    return 3 * max_rank * K // 32


def lr_v_sz_words(max_rank: int, K: int) -> int:
    return max_rank * K // 64


def _v_index(R, K):
    """(row, col) of code c of triplet (j, tau): arrays [R, K/32, 32]."""
    j = np.arange(R)[:, None, None]
    tau = np.arange(K // 32)[None, :, None]
    c = np.arange(32)[None, None, :]
    kb, kq = tau // 4, tau % 4
    col = 128 * kb + 32 * (c // 8) + 8 * kq + (c % 8)
    return np.broadcast_arrays(j, col)


def pack_lr_v(codes, scale, zero, max_rank):
    """codes uint8 [rank][K], scale/zero fp16 [rank][K/64] -> (words, sz) of
    the V layout for max_rank rows."""
    codes = np.asarray(codes)
    rank, K = codes.shape
    if K % 128 or rank > max_rank or rank % 8 or max_rank % 8:
        raise ValueError("V layout needs K % 128 == 0 and rank <= max_rank, both multiples of 8")
    full = np.zeros((max_rank, K), np.uint8)
    full[:rank] = codes
    row, col = _v_index(max_rank, K)
    words = _encode(full[row, col]).reshape(-1)     # [R, K/32, 3] in that order
    sz = np.full((max_rank, K // 64), PAD_SZ_WORD, dtype=np.uint32)
    if rank:
        sz[:rank] = _sz_word(scale, zero)
    return words, sz.reshape(-1)


def unpack_lr_v(words, sz, max_rank, K):
    """Inverse of pack_lr_v over all max_rank rows: (codes [R][K], scale,
    zero fp16 [R][K/64])."""
    w = np.asarray(words, np.uint32).reshape(max_rank, K // 32, 3)
    out = np.zeros((max_rank, K), np.uint8)
    row, col = _v_index(max_rank, K)
    out[row, col] = _decode(w)
    szw = np.asarray(sz, np.uint32).reshape(max_rank, K // 64)
    s = (szw & np.uint32(0xFFFF)).astype(np.uint16).view(np.float16)
    z = (szw >> np.uint32(16)).astype(np.uint16).view(np.float16)
    return out, s, z


# ----------------------------------------------------------------------------
# U layout

def lr_u_words(N: int, max_rank: int) -> int:
    return 3 * N * _round_up(max_rank, 32) // 32


def lr_u_sz_words(N: int) -> int:
    return N


def _u_index(N, R32):
    """(row n, rank j) of code c of lane L in tile (nt, jt): [NT, JT, 64, 32]."""
    NT, JT = N // 64, R32 // 32
    nt = np.arange(NT)[:, None, None, None]
    jt = np.arange(JT)[None, :, None, None]
    L = np.arange(64)[None, None, :, None]
    c = np.arange(32)[None, None, None, :]
    n = 64 * nt + 16 * (c // 8) + (L % 16)
    j = 32 * jt + 8 * (L // 16) + (c % 8)
    return np.broadcast_arrays(n, j)


def _u_sz_index(N):
    n = np.arange(N)
    return 64 * (n // 64) + 4 * (n % 16) + (n % 64) // 16


def pack_lr_u(codes, scale, zero, max_rank):
    """codes uint8 [N][rank], scale/zero fp16 [N] (or [N][1]) -> (words, sz)
    of the U layout for ranks padded to max_rank rounded up to 32."""
    codes = np.asarray(codes)
    N, rank = codes.shape
    if N % 64 or rank > max_rank or rank % 8 or max_rank % 8:
        raise ValueError("U layout needs N % 64 == 0 and rank <= max_rank, both multiples of 8")
    R32 = _round_up(max_rank, 32)
    full = np.zeros((N, R32), np.uint8)
    full[:, :rank] = codes
    if R32 == 0:
        return np.zeros(0, np.uint32), np.zeros(N, np.uint32)
    n, j = _u_index(N, R32)
    w = _encode(full[n, j])                         # [NT, JT, 64, 3]
    words = np.ascontiguousarray(np.moveaxis(w, 3, 2)).reshape(-1)
    sz = np.zeros(N, np.uint32)
    if rank:
        sz[_u_sz_index(N)] = _sz_word(np.asarray(scale).reshape(N), np.asarray(zero).reshape(N))
    else:
        sz[:] = PAD_SZ_WORD
    return words, sz


def unpack_lr_u(words, sz, N, max_rank):
    """Inverse of pack_lr_u: (codes [N][R32], scale, zero fp16 [N])."""
    R32 = _round_up(max_rank, 32)
    NT, JT = N // 64, R32 // 32
    w = np.moveaxis(np.asarray(words, np.uint32).reshape(NT, JT, 3, 64), 2, 3)
    out = np.zeros((N, R32), np.uint8)
    n, j = _u_index(N, R32)
    out[n, j] = _decode(w)
    szw = np.asarray(sz, np.uint32)[_u_sz_index(N)]
    s = (szw & np.uint32(0xFFFF)).astype(np.uint16).view(np.float16)
    z = (szw >> np.uint32(16)).astype(np.uint16).view(np.float16)
    return out, s, z


# ----------------------------------------------------------------------------
# one code at a time, from the spec read backwards (tiny shapes only)

def _put(words, base, c, v, plane_stride):
    pi, h = divmod(c, 2)
    if pi < 15:
        p, o = divmod(pi, 5)
        words[base + plane_stride * p] |= v << (16 * h + 1 + 3 * o)
    else:
        for b in range(3):
            words[base + plane_stride * b] |= ((v >> b) & 1) << (16 * h)


def pack_lr_v_scalar(codes, max_rank):
    """Codes only: walks every (j, k), finds its triplet and code slot."""
    rank = len(codes)
    K = len(codes[0]) if rank else 0
    words = [0] * lr_v_words(max_rank, K)
    for j in range(rank):
        for k in range(K):
            kb, kk = divmod(k, 128)
            step, rem = divmod(kk, 32)
            kq, t8 = divmod(rem, 8)
            tau = 4 * kb + kq
            c = 8 * step + t8
            _put(words, 3 * (j * (K // 32) + tau), c, int(codes[j][k]), 1)
    return words


def pack_lr_u_scalar(codes, max_rank):
    N = len(codes)
    rank = len(codes[0]) if N else 0
    R32 = _round_up(max_rank, 32)
    words = [0] * lr_u_words(N, max_rank)
    for n in range(N):
        for j in range(rank):
            nt, n64 = divmod(n, 64)
            i, n16 = divmod(n64, 16)
            jt, j32 = divmod(j, 32)
            kq, t8 = divmod(j32, 8)
            L = 16 * kq + n16
            c = 8 * i + t8
            tile = nt * (R32 // 32) + jt
            _put(words, 192 * tile + L, c, int(codes[n][j]), 64)
    return words
