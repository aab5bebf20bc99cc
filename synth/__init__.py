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
