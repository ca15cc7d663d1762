"""Seeded synthetic inputs for the heterogeneous KV decode path.

This module is shared by the CPU oracle and by the GPU harness. It holds none
of the method's arithmetic: it only turns (seed, stream, key, index) counters
into numbers, so either side can regenerate any token's K/V/indexer key on its
own, at random access, without storing the batch.

Generator (counter based, no state):
    ctr = stream << 56 | key << 32 | (i >> 1)
    h   = mix64(seed + (ctr + 1) * 0x9E3779B97F4A7C15)          (mod 2**64)
    w   = low 32 bits of h if i is even, else high 32 bits
    S   = byte0(w) + byte1(w) + byte2(w)                         (0 .. 765)
    z   = (2*S - 765) / 256

mix64 is the output function of SplitMix64 (Steele, Lea and Flood,
"Fast splittable pseudorandom number generators", OOPSLA 2014). z is the sum of
three independent uniform bytes, centred and scaled: an Irwin-Hall(3) stand-in
for N(0, 1) with mean 0, variance 65535/65536 and range +-2.99. Every z is an
odd multiple of 2**-8, exact in float32. bf16 inputs take z rounded to nearest
even in bf16 (standard float32 -> bf16 bit rounding).

Index layout per token position p (h = head, d = dim):
    K, V, Q   : i = p*2048 + h*128 + d    (16 heads x 128)
    idxK, qI  : i = p*256  + h*64  + d    (4 indexer heads x 64)

The same generator is written in HIP in synth/synth_gen.hip; a GPU test checks
the two bit for bit.
"""

from __future__ import annotations

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

# stream ids
STREAM_K = 1
STREAM_V = 2
STREAM_IDXK = 3
STREAM_Q = 4
STREAM_QI = 5

N_HEADS = 16
HEAD_DIM = 128
IDX_HEADS = 4
IDX_DIM = 64
KV_ROW = N_HEADS * HEAD_DIM      # 2048 values per token
IDX_ROW = IDX_HEADS * IDX_DIM    # 256 values per token


def mix64(x: np.ndarray) -> np.ndarray:
    """SplitMix64 output function on a uint64 array (wrapping arithmetic)."""
    x = np.asarray(x, dtype=np.uint64)
    with np.errstate(over="ignore"):
        x = (x ^ (x >> np.uint64(30))) * _M1
        x = (x ^ (x >> np.uint64(27))) * _M2
    return x ^ (x >> np.uint64(31))


def raw_words(seed: int, stream: int, key, idx) -> np.ndarray:
    """32-bit generator words for counters (stream, key, idx). key/idx broadcast."""
    key = np.asarray(key, dtype=np.uint64)
    idx = np.asarray(idx, dtype=np.uint64)
    ctr = (np.uint64(stream) << np.uint64(56)) | (key << np.uint64(32)) | (idx >> np.uint64(1))
    with np.errstate(over="ignore"):
        h = mix64(np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + (ctr + np.uint64(1)) * GOLDEN)
    hi = (idx & np.uint64(1)).astype(bool)
    w = np.where(hi, h >> np.uint64(32), h & np.uint64(0xFFFFFFFF))
    return w.astype(np.uint32)


def z_ints(seed: int, stream: int, key, idx) -> np.ndarray:
    """Odd integers 2*S - 765 in [-765, 765]; z = z_ints / 256."""
    w = raw_words(seed, stream, key, idx).astype(np.int32)
    s = (w & 0xFF) + ((w >> 8) & 0xFF) + ((w >> 16) & 0xFF)
    return 2 * s - 765


def z_f32(seed: int, stream: int, key, idx) -> np.ndarray:
    """Exact float32 values z = (2S - 765) / 256."""
    return (z_ints(seed, stream, key, idx).astype(np.float32) / np.float32(256.0)).astype(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return (u >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit pattern -> float32 value (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _token_index(pos, row: int) -> np.ndarray:
    pos = np.asarray(pos, dtype=np.int64).reshape(-1, 1)
    return (pos * row + np.arange(row, dtype=np.int64)[None, :]).astype(np.uint64)


def tokens_bf16(seed: int, stream: int, key, pos) -> np.ndarray:
    """bf16 bits [n][16][128] of K, V or Q rows at token positions `pos` under `key`.

    `key` is a scalar or one key per position.
    """
    pos = np.asarray(pos, dtype=np.int64).reshape(-1)
    key = np.broadcast_to(np.asarray(key, dtype=np.uint64).reshape(-1, 1), (pos.size, 1))
    z = z_f32(seed, stream, key, _token_index(pos, KV_ROW))
    return f32_to_bf16_bits(z).reshape(pos.size, N_HEADS, HEAD_DIM)


def tokens_f32(seed: int, stream: int, key, pos) -> np.ndarray:
    """float32 [n][4][64] of indexer keys or indexer queries at positions `pos`."""
    pos = np.asarray(pos, dtype=np.int64).reshape(-1)
    key = np.broadcast_to(np.asarray(key, dtype=np.uint64).reshape(-1, 1), (pos.size, 1))
    z = z_f32(seed, stream, key, _token_index(pos, IDX_ROW))
    return z.reshape(pos.size, IDX_HEADS, IDX_DIM)


def gate_weights(seed: int) -> tuple[np.ndarray, np.ndarray]:
    """Compressor gate weights (W_csa, W_hca), float32 [16][128] each, ~ N(0, 0.02^2)."""
    g = np.random.default_rng(seed + 1).standard_normal((2, N_HEADS, HEAD_DIM)) * 0.02
    g = g.astype(np.float32)
    return np.ascontiguousarray(g[0]), np.ascontiguousarray(g[1])
