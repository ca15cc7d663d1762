"""The five synthetic workloads (shapes, lengths, keys, seeds).

Every workload is one layer, 16 heads x 128 bf16 K/V/Q, indexer 4 x 64 fp32,
m = 4 (CSA), m' = 128 (HCA), blocks of lcm(4, 128) = 128 tokens. Values come
from the counter generator in `synth`; lengths from numpy's default_rng.
Nothing here computes any part of the method.

  1  "l130"     1 request, prefill L = 130 (the pages' worked example: one
                sealed block plus a 2-token tail), then 126 decode steps to
                L = 256; n_win 128, top-k 16.
  2  "b32"      32 requests, L0 ~ U{1..8192}, 64 decode steps, n_win 128,
                top-k 512.  (the headline decode workload)
  3  "prefix"   64 requests, L0 ~ U{16384..65536}, n_win 4096, top-k 1024,
                32 decode steps. Request b belongs to prefix group b mod 8;
                positions below 32768 carry the group's prefix stream, so the
                first floor(min(L0, 32768)/128) blocks are shared by fork.
  4  "bulk"     8 requests x 131072 tokens appended in one call (no decode);
                n_win 4096.
  5  "long"     4 requests, L0 = 2**20 - 8, 16 decode steps (step 8 seals
                block 8192), n_win 128, top-k 2048.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

PREFIX_KEY_BASE = 0x800000


@dataclass
class Workload:
    index: int
    name: str
    batch: int
    n_win: int
    topk: int
    decode_steps: int
    prefill: np.ndarray            # L0 per request (int64)
    prefix_len: int = 0            # shared-prefix length in tokens (0 = none)
    n_groups: int = 0              # number of prefix groups
    seed: int = 0
    notes: str = ""
    extra: dict = field(default_factory=dict)

    def group(self, b: int) -> int:
        return b % self.n_groups if self.n_groups else -1

    def key(self, b: int, p) -> np.ndarray:
        """Generator key of request b at token position(s) p."""
        p = np.asarray(p, dtype=np.int64)
        if self.prefix_len:
            pk = PREFIX_KEY_BASE | self.group(b)
            return np.where(p < self.prefix_len, pk, b).astype(np.uint64)
        return np.full(p.shape, b, dtype=np.uint64)

    def fork_len(self, b: int) -> int:
        """Length at which request b forks off its group's parent (multiple of 128)."""
        if not self.prefix_len:
            return 0
        return 128 * (min(int(self.prefill[b]), self.prefix_len) // 128)

    @property
    def final_len(self) -> np.ndarray:
        return self.prefill + self.decode_steps

    def max_blocks_total(self, extra_steps: int = 0) -> int:
        """Upper bound on physical blocks needed (no sharing assumed)."""
        L = self.prefill + self.decode_steps + extra_steps
        nb = int((L // 128).sum())
        if self.prefix_len:
            nb += self.n_groups * (self.prefix_len // 128)
        return nb

    def max_len(self, extra_steps: int = 0) -> int:
        return int((self.prefill + self.decode_steps + extra_steps).max())


class RequestTokens:
    """Token source of request b of a workload: (K, V, kI) at any positions, as
    float32 values (K and V are bf16 values), each keyed as the workload keys it.
    Picklable, so that worker processes can regenerate tokens themselves."""

    def __init__(self, index: int, b: int):
        self.index, self.b = int(index), int(b)
        self._wl = None

    def __getstate__(self):
        return {"index": self.index, "b": self.b}

    def __setstate__(self, st):
        self.index, self.b, self._wl = st["index"], st["b"], None

    def __call__(self, pos):
        from . import (STREAM_IDXK, STREAM_K, STREAM_V, bf16_bits_to_f32, tokens_bf16,
                       tokens_f32)
        if self._wl is None:
            self._wl = make(self.index)
        wl = self._wl
        pos = np.asarray(pos, dtype=np.int64).reshape(-1)
        key = wl.key(self.b, pos)
        K = bf16_bits_to_f32(tokens_bf16(wl.seed, STREAM_K, key, pos))
        V = bf16_bits_to_f32(tokens_bf16(wl.seed, STREAM_V, key, pos))
        KI = tokens_f32(wl.seed, STREAM_IDXK, key, pos)
        return K, V, KI

    def query(self, p: int):
        """(q [16][128] bf16 values as float32, q_idx [4][64]) of the decode token at p."""
        from . import STREAM_Q, STREAM_QI, bf16_bits_to_f32, tokens_bf16, tokens_f32
        if self._wl is None:
            self._wl = make(self.index)
        wl = self._wl
        pos = np.array([p], np.int64)
        key = wl.key(self.b, pos)
        return (bf16_bits_to_f32(tokens_bf16(wl.seed, STREAM_Q, key, pos))[0],
                tokens_f32(wl.seed, STREAM_QI, key, pos)[0])


def seed_of(index: int) -> int:
    return 0x48534100 + index


def make(index: int) -> Workload:
    s = seed_of(index)
    if index == 1:
        return Workload(1, "l130", 1, 128, 16, 126, np.array([130], np.int64), seed=s,
                        notes="prefill 130 -> decode to 256")
    if index == 2:
        L0 = np.random.default_rng(s).integers(1, 8193, size=32).astype(np.int64)
        return Workload(2, "b32", 32, 128, 512, 64, L0, seed=s)
    if index == 3:
        L0 = np.random.default_rng(s).integers(16384, 65537, size=64).astype(np.int64)
        return Workload(3, "prefix", 64, 4096, 1024, 32, L0, prefix_len=32768, n_groups=8, seed=s)
    if index == 4:
        return Workload(4, "bulk", 8, 4096, 0, 0, np.full(8, 131072, np.int64), seed=s)
    if index == 5:
        return Workload(5, "long", 4, 128, 2048, 16, np.full(4, (1 << 20) - 8, np.int64), seed=s)
    raise ValueError(f"no workload {index}")


ALL = (1, 2, 3, 4, 5)
