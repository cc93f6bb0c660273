"""Oracle of the 8-bit KV cache (numpy; slow and plain).

TEST INFRASTRUCTURE ONLY: part of the CPU oracle package.  Only the tests, the smoke check
and the CPU-baseline leg of the benchmark may use it; the library never does.

What the pages fix: an 8-bit KV cache keeps one scale for every 32 values, so it takes
34/64 = 53.1% of a 16-bit cache (sotaaz.com, KV-cache measurements, planning notes of the
full-attention section: Qwen3-8B at 32K goes from 4,608 to 2,448 MiB; the same ratio holds
for the other models measured there).  34 bytes per 32 values means 32 one-byte codes and
one two-byte scale.

Readings where the pages are silent (each listed in the design notes):
  * the code of value x in a group with scale s is round-half-to-even(x / s), clamped to
    [-127, 127]; a value is decoded as s * code (symmetric, no offset);
  * s is the group's largest |x| divided by 127 in fp32 (IEEE division, round to nearest
    even), then rounded to fp16; a scale that would overflow fp16 is held at 65504 and the
    codes saturate; an all-zero group has scale 0 and codes 0;
  * x / s is an fp32 division of the value (fp16 / bf16 widened exactly) by the fp16 scale
    widened to fp32;
  * a group is 32 consecutive elements of one token's row for one KV head
    (head_dim / 32 groups per row);
  * cache tile layout: each (block, KV head) tile is 17 rows of head_dim bytes: rows 0-15
    hold the codes of the block's 16 tokens, row 16 holds their scales, token-major
    ([16][head_dim / 32] fp16, little-endian), so a tile is one contiguous run of
    17 * head_dim bytes.
"""
from __future__ import annotations

import numpy as np

GROUP = 32
QMAX = 127
SCALE_MAX = np.float16(65504.0)


def quantize(x: np.ndarray):
    """x: float32 [..., d] (d a multiple of 32) -> (codes int8 [..., d], scales fp16 [..., d/32])."""
    x = np.asarray(x, np.float32)
    g = x.reshape(*x.shape[:-1], x.shape[-1] // GROUP, GROUP)
    amax = np.abs(g).max(axis=-1)
    d = amax / np.float32(QMAX)                       # fp32 division, round to nearest even
    with np.errstate(over="ignore"):
        s = d.astype(np.float16)                       # fp16, round to nearest even
    s = np.where(np.isinf(s), SCALE_MAX, s).astype(np.float16)
    sf = s.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(sf > 0, g / np.where(sf > 0, sf, np.float32(1)), np.float32(0))
    c = np.clip(np.rint(r.astype(np.float32)), -QMAX, QMAX).astype(np.int8)
    return c.reshape(x.shape), s


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """codes int8 [..., d], scales fp16 [..., d/32] -> float64 [..., d] (exact)."""
    c = np.asarray(codes, np.int8).astype(np.float64)
    s = np.asarray(scales, np.float16).astype(np.float64)
    d = c.shape[-1]
    return (c.reshape(*c.shape[:-1], d // GROUP, GROUP) * s[..., None]).reshape(c.shape)


def empty_cache(num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int = 16,
                fill: int = 0xFF) -> np.ndarray:
    """A pool of tiles, every byte set to `fill` (0xFF: codes -1, scales fp16 NaN)."""
    assert block_size == 16 and head_dim % GROUP == 0
    return np.full((num_blocks, num_kv_heads, block_size + 1, head_dim), fill, np.uint8)


def _tile_scales(cache: np.ndarray) -> np.ndarray:
    """View of the scale rows: fp16 [NB][Hkv][16][d/32]."""
    nb, hkv, rows, d = cache.shape
    return cache[:, :, rows - 1, :].copy().view(np.float16).reshape(nb, hkv, rows - 1, d // GROUP)


def write_kv(k_f32: np.ndarray, v_f32: np.ndarray, slots, k_cache: np.ndarray,
             v_cache: np.ndarray) -> None:
    """Quantize k/v rows [T][Hkv][d] (float32 values) into the slots of the tile pools."""
    slots = np.asarray(slots, np.int64)
    nb, hkv, rows, d = k_cache.shape
    bs = rows - 1
    for src, cache in ((k_f32, k_cache), (v_f32, v_cache)):
        codes, scales = quantize(src)
        for t, s in enumerate(slots):
            if s < 0 or s >= nb * bs:
                continue
            blk, off = divmod(int(s), bs)
            cache[blk, :, off, :] = codes[t].view(np.uint8)
            sb = scales[t].view(np.uint8).reshape(hkv, -1)          # [Hkv][2 * d / 32]
            w = sb.shape[1]
            cache[blk, :, bs, off * w:(off + 1) * w] = sb


def copy_block(k_cache: np.ndarray, v_cache: np.ndarray, src: int, dst: int, n: int) -> None:
    """Copy-on-write of the first n tokens of block src to block dst: their codes and their
    scales, for every KV head, K and V."""
    bs, d = k_cache.shape[2] - 1, k_cache.shape[3]
    w = 2 * (d // GROUP)
    for cache in (k_cache, v_cache):
        cache[dst, :, :n] = cache[src, :, :n]
        cache[dst, :, bs, :n * w] = cache[src, :, bs, :n * w]


def dequantize_cache(cache: np.ndarray) -> np.ndarray:
    """Tile pool -> float32 [NB][Hkv][16][d] of decoded values (exact in float32)."""
    nb, hkv, rows, d = cache.shape
    codes = cache[:, :, :rows - 1, :].view(np.int8)
    return dequantize(codes, _tile_scales(cache)).astype(np.float32)
