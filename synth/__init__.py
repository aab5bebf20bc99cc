"""Seeded synthetic inputs shared by the tests, the bench and the oracle's callers.

This module only draws random numbers and lays them out as the stored bytes of each
weight format; it holds none of the product's arithmetic (no unpacking, no scale
decoding, no dot products).  Both the HIP path and the CPU oracle consume what it
returns, so neither side can tilt the comparison.

Stored formats (byte offsets inside one 256-weight superblock, little-endian):

* Q4_K, 144 B: fp16 d @0, fp16 dmin @2, 12 packed 6-bit scale/min bytes @4,
  128 quant bytes @16 (two 4-bit quants per byte).
* Q5_K, 176 B: as Q4_K, with 32 high-bit bytes @16 and the 128 quant bytes @48.
* Q6_K, 210 B: 128 low-nibble bytes @0, 64 high-2-bit bytes @128, 16 int8
  scales @192, fp16 d @208.
* NVFP4: codes [M][K/2] (two e2m1 codes per byte), scales [M][K/16] e4m3.
* FP8 (block-scaled e4m3): codes [M][K] (one OCP E4M3FN code per byte), scales
  [ceil(M/128)][K/128] bf16, one per 128-row x 128-column block.

Value distributions follow the workload description of the decode-GEMV pages'
Qwen3-4B Q4_K_M setting: fp16 d and dmin uniform in [1e-3, 2e-2]; the packed 6-bit
scale/min bytes uniform (every 6-bit field is then uniform in 0..63, because each
field is built from disjoint bits of independent uniform bytes); quant bytes
uniform; Q6_K int8 scales uniform in 0..63; NVFP4 codes uniform over all 16 codes
with e4m3 scales = round-to-nearest-even(uniform real in [0.01, 1]); x is
fp16(N(0, 1)).  The FP8 format has no workload distribution in the pages; its
codes are uniform over the 254 non-NaN e4m3 codes and its block scales are
bf16(uniform real in [1e-3, 1e-2]).
"""
from __future__ import annotations

import numpy as np

Q4_K, Q5_K, Q6_K, NVFP4, FP8 = 12, 13, 14, 1001, 1002
TYPE_NAMES = {Q4_K: "q4_k", Q5_K: "q5_k", Q6_K: "q6_k", NVFP4: "nvfp4", FP8: "fp8_b128"}
BLOCK_BYTES = {Q4_K: 144, Q5_K: 176, Q6_K: 210}
QK = 256          # weights per K-quant superblock
NVFP4_GROUP = 16  # weights per NVFP4 scale
FP8_BLOCK = 128   # rows and columns per FP8 scale block


def row_bytes(wtype: int, k: int) -> int:
    """Bytes of one stored weight row (codes only for NVFP4)."""
    if wtype == NVFP4:
        return k // 2
    if wtype == FP8:
        return k
    return (k // QK) * BLOCK_BYTES[wtype]


def rng_for(seed, *path) -> np.random.Generator:
    """PCG64 stream for `seed`, optionally refined by a path of integers."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), *map(int, path)])))


def _fp16_bits(vals: np.ndarray) -> np.ndarray:
    return vals.astype(np.float16).view(np.uint16)


def _put_u16(blocks: np.ndarray, off: int, bits: np.ndarray) -> None:
    blocks[..., off] = (bits & 0xFF).astype(np.uint8)
    blocks[..., off + 1] = (bits >> 8).astype(np.uint8)


def kquant_weights(wtype: int, m: int, k: int, rng: np.random.Generator,
                   d_range=(1e-3, 2e-2), q6_scale_range=(0, 64)) -> np.ndarray:
    """Random K-quant weight matrix as raw bytes, shape [m, row_bytes].

    q6_scale_range is the half-open integer range of the Q6_K int8 scales
    ((-128, 128) covers every code).
    """
    if k % QK:
        raise ValueError("k must be a multiple of 256")
    nb = k // QK
    bb = BLOCK_BYTES[wtype]
    blocks = rng.integers(0, 256, size=(m, nb, bb), dtype=np.uint8)
    lo, hi = d_range
    if wtype in (Q4_K, Q5_K):
        _put_u16(blocks, 0, _fp16_bits(rng.uniform(lo, hi, size=(m, nb))))
        _put_u16(blocks, 2, _fp16_bits(rng.uniform(lo, hi, size=(m, nb))))
    elif wtype == Q6_K:
        lo, hi = q6_scale_range
        blocks[..., 192:208] = rng.integers(lo, hi, size=(m, nb, 16)).astype(np.int8).view(np.uint8)
        lo, hi = d_range
        _put_u16(blocks, 208, _fp16_bits(rng.uniform(lo, hi, size=(m, nb))))
    else:
        raise ValueError(f"not a K-quant type: {wtype}")
    return blocks.reshape(m, nb * bb)


def e4m3_bits(vals: np.ndarray) -> np.ndarray:
    """Round reals to OCP E4M3FN (nearest-even) and return the code bytes."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(vals, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def nvfp4_weights(m: int, k: int, rng: np.random.Generator, scale_range=(0.01, 1.0)):
    """Random NVFP4 weight matrix: (codes [m, k/2] u8, scales [m, k/16] e4m3 bytes)."""
    if k % NVFP4_GROUP:
        raise ValueError("k must be a multiple of 16")
    codes = rng.integers(0, 256, size=(m, k // 2), dtype=np.uint8)
    scales = e4m3_bits(rng.uniform(*scale_range, size=(m, k // NVFP4_GROUP)))
    return codes, scales


def bf16_bits(vals: np.ndarray) -> np.ndarray:
    """Round reals to bfloat16 (nearest-even) and return the 16-bit patterns."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(vals, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def fp8_weights(m: int, k: int, rng: np.random.Generator, scale_range=(1e-3, 1e-2)):
    """Random block-scaled FP8 weight matrix: (codes [m, k] u8 e4m3, scales
    [ceil(m/128), k/128] as little-endian bf16 bytes, shape [ceil(m/128), k/64] u8)."""
    if k % FP8_BLOCK:
        raise ValueError("k must be a multiple of 128")
    ok = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)   # no NaN codes
    codes = ok[rng.integers(0, ok.size, size=(m, k))]
    rb = (m + FP8_BLOCK - 1) // FP8_BLOCK
    sb = bf16_bits(rng.uniform(*scale_range, size=(rb, k // FP8_BLOCK)))
    return codes, np.ascontiguousarray(sb).view(np.uint8).reshape(rb, 2 * (k // FP8_BLOCK))


def activations(n: int, k: int, rng: np.random.Generator) -> np.ndarray:
    """x as fp16 N(0, 1), shape [n, k]."""
    return rng.standard_normal(size=(n, k)).astype(np.float16)


def weights(wtype: int, m: int, k: int, rng: np.random.Generator, **kw):
    """(data, scales-or-None) for any supported type."""
    if wtype == NVFP4:
        return nvfp4_weights(m, k, rng, **kw)
    if wtype == FP8:
        return fp8_weights(m, k, rng, **kw)
    return kquant_weights(wtype, m, k, rng, **kw), None


def duplicate_rows(x: np.ndarray) -> np.ndarray:
    """Copy some rows onto others so that a multi-row call holds repeated inputs.

    Row 0 goes to rows n//2 and n-1, row 1 goes to row n//3, whenever those
    targets are distinct and above 1.
    """
    x = x.copy()
    n = x.shape[0]
    for src, dst in ((0, n // 2), (0, n - 1), (1, n // 3)):
        if dst > 1 and dst < n and src < n and dst != src:
            x[dst] = x[src]
    return x


# The decode-layer projections of a Qwen3-4B-shaped model (hidden 2560, FFN 9728,
# 32 query heads and 8 KV heads of width 128): (name, type, M, K).
QWEN3_4B_LAYER = (
    ("wq", Q4_K, 4096, 2560),
    ("wk", Q4_K, 1024, 2560),
    ("wv", Q6_K, 1024, 2560),
    ("wo", Q4_K, 2560, 4096),
    ("gate", Q4_K, 9728, 2560),
    ("up", Q4_K, 9728, 2560),
    ("down", Q6_K, 2560, 9728),
)


# ---------------------------------------------------------------------------
# Adversarial K-quant rows: weights d*sc*q - dmin*m whose two terms cancel.
#
# These are built from integer relations between the stored fields (no weight is
# decoded here).  With d = D * 2^e and dmin = Dm * 2^(e + j) (D, Dm the 11-bit fp16
# significands), a sub-block whose 32 quants all equal q has every weight equal to
# 2^e * (D*sc*q - Dm*m*2^j).
#   * "exact": D*sc*q == Dm*m*2^j, every weight exactly 0 (sum|w||x| = 0);
#   * "near":  D*sc*q - Dm*m*2^j = +-1 with D*sc*q >= 10^6, so 0 < |w| <= 1e-6 * d*sc*q;
#   * "mixed": per superblock, sub-blocks of both kinds beside ordinary small ones
#     (sc = 1, m = 0, random quants), so sum|w||x| is small next to the cancelling terms.


def _pack_scale_min(sc, mn):
    """The 12 packed bytes of eight 6-bit (scale, min) pairs, GGML K-quant packing:
    pairs 0..3 in the low 6 bits of bytes j (scale) and j+4 (min); pairs 4..7 with
    their low 4 bits in byte j+4 (scale low nibble, min high nibble) and their top 2
    bits in bits 6..7 of bytes j-4 (scale) and j (min)."""
    sc = np.asarray(sc, dtype=np.int64)
    mn = np.asarray(mn, dtype=np.int64)
    out = np.zeros(sc.shape[:-1] + (12,), dtype=np.int64)
    for j in range(4):
        out[..., j] = sc[..., j] | ((sc[..., j + 4] >> 4) << 6)
        out[..., j + 4] = mn[..., j] | ((mn[..., j + 4] >> 4) << 6)
        out[..., j + 8] = (sc[..., j + 4] & 15) | ((mn[..., j + 4] & 15) << 4)
    return out.astype(np.uint8)


def _fp16_from_parts(sig, e):
    """fp16 bits of sig * 2^e for an 11-bit significand sig in [1024, 2047] (normal)."""
    sig = np.asarray(sig, dtype=np.int64)
    e = np.asarray(e, dtype=np.int64)
    field = e + 10 + 15
    assert np.all((sig >= 1024) & (sig < 2048)) and np.all((field >= 1) & (field <= 30))
    return ((field << 10) | (sig - 1024)).astype(np.uint16)


def _exact_triples(R, qmax):
    """(sc, q, m) with sc*q == R*m, 1 <= sc, m <= 63, 1 <= q <= qmax."""
    out = []
    for sc in range(1, 64):
        for q in range(1, qmax + 1):
            if (sc * q) % R == 0 and 1 <= (sc * q) // R <= 63:
                out.append((sc, q, (sc * q) // R))
    return out


_NEAR_POOLS = {}


def _near_pool(qmax):
    """Every (D, Dm, j) -> [(sc, q, m)] with D*sc*q - Dm*m*2^j = +-1 and D*sc*q >= 10^6
    (D odd in [1025, 2047], Dm in [1024, 2047], j in 3..5, sc, m in 1..63, q in 1..qmax),
    found once by exhaustive search."""
    if qmax in _NEAR_POOLS:
        return _NEAR_POOLS[qmax]
    sc = np.arange(1, 64, 2)[:, None, None]          # D*sc*q must be odd
    q = np.arange(1, qmax + 1, 2)[None, :, None]
    mm = np.arange(1, 64)[None, None, :]
    pool = {}
    for j in (3, 4, 5):
        for D in range(1025, 2048, 2):
            P = D * sc * q
            for delta in (-1, 1):
                num = P - delta
                den = mm * (1 << j)
                Dm = num // den
                ok = (num % den == 0) & (Dm >= 1024) & (Dm < 2048) & (P >= 10 ** 6)
                for a, b, c in zip(*np.nonzero(ok)):
                    key = (D, int(Dm[a, b, c]), j)
                    pool.setdefault(key, []).append((int(sc[a, 0, 0]), int(q[0, b, 0]), int(mm[0, 0, c])))
    keys = sorted(pool)
    _NEAR_POOLS[qmax] = (keys, pool)
    return _NEAR_POOLS[qmax]


def kquant_cancelling(wtype: int, m: int, k: int, rng: np.random.Generator, mode: str = "exact"):
    """Q4_K / Q5_K rows of cancelling superblocks (see above), as raw bytes [m, row_bytes],
    plus the fields they were built from: a dict of arrays d, dmin (fp16 bits, [m, nb]),
    sc, mn, q ([m, nb, 8]: every quant of sub-block j is q[..., j])."""
    if wtype not in (Q4_K, Q5_K):
        raise ValueError("cancellation needs the Q4_K / Q5_K affine")
    if mode not in ("exact", "near", "mixed"):
        raise ValueError(mode)
    qmax = 15 if wtype == Q4_K else 31
    nb = k // QK
    d_bits = np.zeros((m, nb), np.uint16)
    dm_bits = np.zeros((m, nb), np.uint16)
    sc = np.zeros((m, nb, 8), np.int64)
    mn = np.zeros((m, nb, 8), np.int64)
    qv = np.zeros((m, nb, 8), np.int64)
    exact_pool = {R: _exact_triples(R, qmax) for R in range(1, 64)}
    for r in range(m):
        for b in range(nb):
            kind = mode if mode != "mixed" else ("exact", "near")[int(rng.integers(0, 2))]
            if kind == "exact":
                if rng.integers(0, 2):   # d a power of two, dmin = R * d (R <= 63 fits 11 bits)
                    e = int(rng.integers(-10, -6))
                    R = int(rng.integers(2, 64))
                    while not exact_pool[R]:
                        R = int(rng.integers(2, 64))
                    D, De, Dm, Dme = 1024, e - 10, R, e   # d = 2^e = 1024 * 2^(e-10), dmin = R * 2^e
                    while Dm < 1024:
                        Dm, Dme = Dm * 2, Dme - 1
                    trip = exact_pool[R]
                else:                    # any d, dmin = 2^r * d
                    D, De = int(rng.integers(1024, 2048)), int(rng.integers(-20, -16))
                    r_ = int(rng.integers(0, 4))
                    Dm, Dme = D, De + r_
                    trip = exact_pool[1 << r_]
            else:
                keys, pool = _near_pool(qmax)
                D, Dm, j = keys[int(rng.integers(0, len(keys)))]
                trip = pool[(D, Dm, j)]
                De = int(rng.integers(-20, -18))
                Dme = De + j
            d_bits[r, b] = _fp16_from_parts(D, De)
            dm_bits[r, b] = _fp16_from_parts(Dm, Dme)
            picks = rng.integers(0, len(trip), size=8)
            for s in range(8):
                sc[r, b, s], qv[r, b, s], mn[r, b, s] = trip[picks[s]]
            if mode == "mixed":          # ordinary small sub-blocks beside the cancelling ones
                for s in np.nonzero(rng.integers(0, 3, size=8) == 0)[0]:
                    sc[r, b, s], mn[r, b, s], qv[r, b, s] = 1, 0, -1   # -1: random quants
    bb = BLOCK_BYTES[wtype]
    blocks = np.zeros((m, nb, bb), np.uint8)
    _put_u16(blocks, 0, d_bits)
    _put_u16(blocks, 2, dm_bits)
    blocks[..., 4:16] = _pack_scale_min(sc, mn)
    qoff = 16 if wtype == Q4_K else 48
    rnd = rng.integers(0, qmax + 1, size=(m, nb, 8, 32))
    quants = np.where(qv[..., None] >= 0, qv[..., None], rnd)         # [m, nb, 8 sub-blocks, 32]
    for c in range(4):   # chunk c: sub-block 2c in the low nibbles, 2c+1 in the high ones
        lo, hi = quants[:, :, 2 * c] & 15, quants[:, :, 2 * c + 1] & 15
        blocks[..., qoff + 32 * c:qoff + 32 * c + 32] = (lo | (hi << 4)).astype(np.uint8)
    if wtype == Q5_K:    # fifth bit of position l of sub-block j: bit j of qh[l]
        qh = np.zeros((m, nb, 32), np.int64)
        for s in range(8):
            qh |= ((quants[:, :, s] >> 4) & 1) << s
        blocks[..., 16:48] = qh.astype(np.uint8)
    fields = {"d": d_bits, "dmin": dm_bits, "sc": sc, "mn": mn, "q": quants}
    return blocks.reshape(m, nb * bb), fields
