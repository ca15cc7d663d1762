"""Plain, slow fp64 oracle of the Block Cache + State Cache decode path.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the GPU path.

Page keys used in the citations below:
  [Q&A]    "V4 为何要分池？块对齐与尾缓冲怎么配合？" (deepseek-tech-notes Q&A on the
           two pools, block alignment and the tail buffer)
  [Layout] "V4 KV Layout：Classical + State 双池" (deepseek-tech-notes)
  [Ch12]   "Ch 12 · 推理框架 — KV 的异构调度" (DeepSeek-V4-book)
  [Disk]   "V4 磁盘 Prefix Cache" (deepseek-tech-notes)

Arithmetic is float64. Values that the layout stores as bf16 (compressed CSA and
HCA entries) are rounded to bf16, nearest-even, when stored, and kept in
float32 arrays that hold those bf16 values exactly; raw K/V/Q arrive as bf16
values and indexer keys/queries as float32 values, both exact in float64.

Readings taken where the pages leave a step open (each also in the design notes):
  R1  compressor: per head h, gate logits g_t = <W[h], K_t[h]>, alpha =
      softmax over the m tokens, entry = sum_t alpha_t (K_t, V_t); separate W
      for CSA (m = 4) and HCA (m' = 128). The pages never define it.
  R2  C4 and HCA entries are written together when a 128-token block fills
      ([Q&A] §2.2, §2.3; [Ch12] Demo); csa_tail = L mod 4, hca_tail = L mod 128
      count tokens of the one raw tail.
  R3  indexer keys: 128 per block, one per token, 4 heads x 64 ([Ch12] §2.2).
  R4  indexer score of token t: sum over heads and dims of qI * kI_t; score of
      C4 entry j of a block = mean of its 4 tokens' scores. No ReLU, no head
      weights (not on the pages).
  R5  no de-duplication: one softmax over SWA + HCA + selected C4 even where a
      token is also inside a sealed block ([Q&A] §2.3 leaves it to the kernel).
  R6  the tail is read through the SWA (tail is a subset of SWA since
      n_win >= 128 > L mod 128).
  R8  top-k candidates are the sealed C4 entries only; kk = min(k, N_c); the
      rest of the row is padded with -1.
  R9  top-k selection: the kk entries that come first under (score descending,
      ordinal ascending), i.e. ties go to the lowest C4 ordinal. The pages fix no
      output order; the entries are returned in ascending ordinal order, or in
      selection order (score descending, ordinal ascending) when sorted=True.
  R10 block ids: lowest free id first, requests in call order, blocks in token
      order; state slots: lowest free first.
  R11 share(src, dst): dst (fresh) references every sealed block of src
      (refcount + 1 each) and gets a copy of src's State (SWA, tail, L).
  R12 softmax scale 1/sqrt(128); no positional encoding, no mask.
  R15 FP8 entries (optional format): the pages account compressed entries in FP8
      ([Ch12] §2.2) without a scale scheme. Reading: each C4 entry's K and V are
      stored per head as 128 OCP FP8 E4M3 codes and one float32 scale
      s = max_d |x_d| / 448, so that the largest magnitude maps onto E4M3's largest
      finite value; the stored value of x_d is code_d * s. Since the stored value
      multiplies by s, the quantiser divides by the same s: code_d is the E4M3 of
      x_d / s, nearest, ties to the even code. x, s and the quotient are float32
      values, each division correctly rounded (the precision the kernel computes
      in). A head whose s would not be a normal float32 (all zero, or max |x| below
      448 * 2**-126) keeps s = 1; its codes, by the same rule, are then all 0.
      HCA entries stay bf16.
  R20 FP8 SWA ring and HCA entries (optional format, kv_format="fp8"): the pages
      account every KV kind in FP8, the SWA's raw tokens and the HCA entries too
      ([Ch12] §1 worked figures: SWA 2048 B, HCA 16 B per token), without a scale
      scheme. Reading: the R15 per-head quantiser applied to each token's K and V as
      it enters the State (the ring slot holds its codes and scales; the stored
      value is code * s) and to each HCA entry as it is sealed (from the float64
      pooled entry, in place of the bf16 rounding). The State keeps no other copy
      of a token, so a block's compressor pools the stored (dequantized) K/V of its
      128 tokens, and attention reads the stored values. Indexer keys are not
      affected.
  R16 low-bit indexer keys (optional format): the pages store the indexer keys
      of the Block Cache as FP4 ([Ch12] §1 worked figures, §2.2) without a scale
      scheme. Reading: OCP MXFP4 (Microscaling Formats v1.0): each sealed key's
      256 values split into 8 blocks of 32 (head h, half j = block 2h + j); a
      block has one E8M0 scale 2**E, E = floor(log2 max|x|) - 2 (2 is E2M1's
      largest exponent), at least -127 (-127 for an all-zero block), and each
      value is the E2M1 code of x / 2**E: nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6,
      ties to the even code, saturating at 6, sign bit set for x < 0. The key
      reads as code value * 2**E. The open block's keys (the State's indexer
      tail) stay float32 until the block seals; the query stays float32.
  R17 prefix hits under the three SWA policies ([Ch12] §3.1; [Disk] SWA three
      policies): a prefix entry holds the prefix's sealed blocks (a block
      reference with no State). Zero: a new request takes the blocks and length
      len and rebuilds its window from the prefix's raw tokens [len - n_win, len)
      (in a model they come from a partial prefill; here the caller passes them),
      never sealing the shared blocks again. Periodic: a checkpoint of the State
      (SWA window, indexer tail, length) is kept every p tokens; a hit restores the
      latest checkpoint c <= len and replays [c, len). Full: the checkpoint at len
      itself. Each yields the State a fork of a live prefix request would have.
  R18 layer types ([Ch12] Figure 12-1: one State quota per request over all
      layers, per block every layer's compressed KV). Every layer keeps an SWA
      window; "csa" layers keep 32 C4 entries + 128 indexer keys per block and
      attend SWA + top-k C4; "hca" layers keep 1 HCA entry per block and attend SWA
      + every HCA entry; "swa" layers keep nothing in the Block Cache; "mixed"
      (the single-layer path) keeps both and attends all three. Layers share the
      State lengths and the block ids; a multi-layer cache is one oracle per
      layer, driven by the same calls.
  R19 eager C4 (optional mode; the other reading of [Q&A] §3.1, where the CSA tail
      is full at L mod 4 = 0): the C4 entry of each complete group of 4 tokens of
      the open block exists as soon as the group is, pooled exactly as the seal
      pools it, and is a top-k candidate and an attention key like a sealed one.
      The open block's g = (L mod 128) // 4 entries (32 with a deferred full tail)
      take ordinals 32 nb .. 32 nb + g - 1 after the sealed entries; their scores
      use the tail's indexer keys. When the block seals, the entries move into it
      unchanged. Supported with bf16 entries and float32 indexer keys.
"""

from __future__ import annotations

import heapq
import math
from collections import deque

import numpy as np

BLOCK = 128          # lcm(m, m') tokens per block ([Q&A] §2.2; [Ch12] 公式白话翻译)
M_CSA = 4            # CSA: 4 tokens -> 1 entry ([Q&A] §1.2)
M_HCA = 128          # HCA: 128 tokens -> 1 entry ([Q&A] §1.2)
C4_PER_BLOCK = BLOCK // M_CSA   # 32 ([Ch12] §2.2)
N_HEADS = 16
HEAD_DIM = 128
IDX_HEADS = 4
IDX_DIM = 64


class OracleError(Exception):
    """kind in {'invalid', 'oom_blocks', 'oom_states', 'state'}; raised before any change."""

    def __init__(self, kind: str, msg: str = ""):
        super().__init__(f"{kind}: {msg}")
        self.kind = kind


# ---------------------------------------------------------------- arithmetic

def bf16_round(x) -> np.ndarray:
    """Nearest bf16 value of float64 x, ties to even (8 significant bits).

    Written from the definition: x = m * 2**e with 0.5 <= |m| < 1, keep 8
    significant bits of m with round-half-to-even. Finite normal range only.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


# OCP FP8 E4M3 (E4M3FN): 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; no
# infinities; exponent 15 with mantissa 7 is NaN; largest finite value 448.
E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 code (float64; NaN for 0x7f and 0xff), from the format:
    exponent field 0 is subnormal, 2**-6 * m / 8; otherwise 2**(e - 7) * (1 + m / 8)."""
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & ((c & 7) == 7), np.nan, mag)
    return sign * mag


def e4m3_encode(x) -> np.ndarray:
    """E4M3 code of each value (round to nearest, ties to the even code). Written
    from the format: the representable magnitudes are enumerated and x goes to the
    nearest; on a tie, to the one whose code is even. |x| above the largest finite
    value rounds to it when below the midpoint toward the next binade (464) and is
    NaN beyond; NaN stays NaN; -0 keeps its sign."""
    x = np.asarray(x, dtype=np.float64)
    finite_codes = np.arange(0, 0x7F)                         # 0 .. 126: 0 .. 448
    vals = e4m3_decode(finite_codes)
    a = np.abs(x)
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, len(vals) - 1)
    lo = np.clip(hi - 1, 0, len(vals) - 1)
    d_lo = a - vals[lo]
    d_hi = vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (finite_codes[hi] % 2 == 0))
    code = np.where(pick_hi, finite_codes[hi], finite_codes[lo])
    code = np.where(a >= 464.0, 0x7F, code)
    code = np.where(np.isnan(x), 0x7F, code)
    code = code | np.where(np.signbit(x), 0x80, 0)
    return code.astype(np.uint8)


def quantize_e4m3_rows(x) -> tuple:
    """Per-row FP8 storage of [..., 128] rows (reading R15): returns (codes uint8,
    scales float32 [...], values float64 = code value * scale). The row is taken as
    float32; with amax = max |x|, s = float32(amax / 448), or 1 where that is not a
    normal float32; each code is the E4M3 of float32(x / s)."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    amax = np.abs(x32).max(axis=-1)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    s = np.where(s >= np.float32(np.finfo(np.float32).tiny), s, np.float32(1.0)).astype(np.float32)
    y = (x32 / s[..., None]).astype(np.float32)
    codes = e4m3_encode(y)
    vals = e4m3_decode(codes) * s[..., None].astype(np.float64)
    return codes, s, vals


# ---------------------------------------------------------------- MXFP4 (reading R16)
# OCP Microscaling: E2M1 elements (sign, 2 exponent bits with bias 1, 1 mantissa
# bit; exponent field 0 is subnormal) under an E8M0 scale (a byte b = 2**(b - 127)).

MX_BLOCK = 32


def e2m1_decode(codes) -> np.ndarray:
    """Value of each 4-bit E2M1 code (float64): exponent field 0 gives m / 2,
    otherwise 2**(e - 1) * (1 + m / 2)."""
    c = np.asarray(codes, dtype=np.int64) & 0xF
    sign = np.where(c & 8, -1.0, 1.0)
    e = (c >> 1) & 3
    m = (c & 1).astype(np.float64)
    mag = np.where(e == 0, m / 2.0, np.ldexp(1.0 + m / 2.0, e - 1))
    return sign * mag


def e2m1_encode(y) -> np.ndarray:
    """E2M1 code of each value: the nearest representable magnitude, ties to the
    even code, magnitudes beyond the largest (6) saturating to it; the sign bit is
    set for y < 0 (also when the magnitude rounds to 0)."""
    y = np.asarray(y, dtype=np.float64)
    codes = np.arange(8)
    vals = e2m1_decode(codes)
    a = np.abs(y)
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, 7)
    lo = np.clip(hi - 1, 0, 7)
    d_lo, d_hi = a - vals[lo], vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (codes[hi] % 2 == 0))
    c = np.where(pick_hi, codes[hi], codes[lo])
    c = np.where(a >= vals[-1], 7, c)
    return (c | np.where(y < 0, 8, 0)).astype(np.uint8)


def quantize_mxfp4_rows(x) -> tuple:
    """MXFP4 storage of indexer keys [..., 256] (reading R16): returns (codes uint8
    [..., 128] with value 2i in the low nibble of byte i and value 2i + 1 in the
    high nibble, scales uint8 [..., 8] E8M0 bytes E + 127, values float64 [..., 256]
    = code value * 2**E). Keys are taken as float32."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    shp = x32.shape
    blocks = x32.reshape(*shp[:-1], shp[-1] // MX_BLOCK, MX_BLOCK)
    amax = np.abs(blocks).max(axis=-1)
    _, ex = np.frexp(amax)                    # amax = f * 2**ex, f in [0.5, 1)
    E = np.where(amax > 0, np.maximum(ex - 1 - 2, -127), -127).astype(np.int64)
    y = blocks / np.ldexp(1.0, E)[..., None]   # exact: a power-of-two scale
    c = e2m1_encode(y)
    vals = (e2m1_decode(c) * np.ldexp(1.0, E)[..., None]).reshape(shp)
    c = c.reshape(shp).astype(np.uint8)
    codes = (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)
    return codes, (E + 127).astype(np.uint8), vals


def length_split(L: int) -> dict:
    """L = 128 q + r: q sealed blocks hold 32q C4 + q HCA entries, r tokens stay
    in the tail ([Q&A] §2.2, §3.1; [Ch12] Demo)."""
    q, r = divmod(int(L), BLOCK)
    return {"blocks": q, "c4": C4_PER_BLOCK * q, "hca": q, "tail": r,
            "csa_tail": int(L) % M_CSA, "hca_tail": int(L) % M_HCA}


def gated_pool(Kg: np.ndarray, Vg: np.ndarray, W: np.ndarray, rounded: bool = True):
    """Compress m consecutive tokens into one entry (reading R1).

    Kg, Vg: [m][H][D] token K/V; W: [H][D] gate weights. Per head h:
    g_t = <W[h], K_t[h]>, alpha = softmax_t(g), entry = sum_t alpha_t K_t[h]
    (and the same alpha for V). Returns bf16-rounded (K, V) [H][D] as float32, or
    the float64 values when not `rounded`.
    The m -> 1 compression and its alignment to the block: [Q&A] §2.1.
    """
    Kg = np.asarray(Kg, dtype=np.float64)
    Vg = np.asarray(Vg, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    g = np.einsum("thd,hd->th", Kg, W)                  # [m][H]
    g = g - g.max(axis=0, keepdims=True)
    a = np.exp(g)
    a = a / a.sum(axis=0, keepdims=True)                # softmax over the m tokens
    Kh = np.einsum("th,thd->hd", a, Kg)
    Vh = np.einsum("th,thd->hd", a, Vg)
    if not rounded:
        return Kh, Vh
    return bf16_round(Kh).astype(np.float32), bf16_round(Vh).astype(np.float32)


def token_scores(idx_keys: np.ndarray, q_idx: np.ndarray) -> np.ndarray:
    """Indexer score per token (reading R4): sum over 4 heads x 64 dims of qI * kI_t.
    idx_keys: [n][4][64]; q_idx: [4][64] -> [n] float64."""
    k = np.asarray(idx_keys, dtype=np.float64).reshape(len(idx_keys), -1)
    return k @ np.asarray(q_idx, dtype=np.float64).reshape(-1)


def c4_scores(idx_keys: np.ndarray, q_idx: np.ndarray) -> np.ndarray:
    """C4 entry scores of one block: entry j covers tokens 4j..4j+3; score = mean
    of their token scores (reading R4). idx_keys: [128][4][64] -> [32]."""
    s = token_scores(idx_keys, q_idx)
    return s.reshape(C4_PER_BLOCK, M_CSA).sum(axis=1) / 4.0


def select_topk(scores: np.ndarray, k: int, sorted: bool = False):
    """The kk = min(k, N) entries first under (score desc, ordinal asc), padded to k
    with -1 (readings R8, R9): in ascending ordinal order, or in that selection
    order when sorted. Returns (idx int32 [k], score float64 [k], -inf padded)."""
    scores = np.asarray(scores, dtype=np.float64)
    n = scores.size
    kk = min(int(k), n)
    order = np.lexsort((np.arange(n), -scores))[:kk]    # primary: -score, then ordinal
    if not sorted:
        order = np.sort(order)
    idx = np.full(k, -1, np.int32)
    val = np.full(k, -np.inf, np.float64)
    idx[:kk] = order
    val[:kk] = scores[order]
    return idx, val


def attention(q: np.ndarray, Kc: np.ndarray, Vc: np.ndarray) -> np.ndarray:
    """One softmax over all N cached keys, per head (reading R12).
    q: [H][D]; Kc, Vc: [N][H][D] -> out [H][D] float64."""
    q = np.asarray(q, dtype=np.float64)
    Kc = np.asarray(Kc, dtype=np.float64)
    Vc = np.asarray(Vc, dtype=np.float64)
    s = np.einsum("nhd,hd->hn", Kc, q) / math.sqrt(q.shape[-1])
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=1, keepdims=True)
    return np.einsum("hn,nhd->hd", p, Vc)


# ---------------------------------------------------------------- one request, streamed

def block_range_summary(args):
    """HCA entries and C4 scores of the sealed blocks b0 .. b1-1 of one request.

    args = (seq, gate_hca, q_idx_list, b0, b1[, kv_format]); seq(pos) returns the
    request's (K [n][H][D], V [n][H][D], kI [n][4][64]) at token positions pos, as
    the State stores them. Block b holds tokens 128b .. 128b+127 ([Q&A] §2.2): its
    HCA entry pools all 128 (reading R1), stored as bf16 or (kv_format "fp8",
    reading R20) as per-head E4M3, and its 32 C4 scores follow reading R4, once per
    indexer query.
    Returns (hca_k [n][H][D], hca_v, scores [len(q_idx_list)][32 n]).
    """
    seq, gate_hca, qis, b0, b1 = args[:5]
    kv_format = args[5] if len(args) > 5 else "bf16"
    n = b1 - b0
    K, V, KI = seq(np.arange(BLOCK * b0, BLOCK * b1, dtype=np.int64))
    hk = np.empty((n, N_HEADS, HEAD_DIM), np.float64)
    hv = np.empty_like(hk)
    sc = np.empty((len(qis), C4_PER_BLOCK * n), np.float64)
    for i in range(n):
        g = slice(BLOCK * i, BLOCK * (i + 1))
        if kv_format == "fp8":                        # reading R20: the pooled entry's storage
            Kh, Vh = gated_pool(K[g], V[g], gate_hca, rounded=False)
            hk[i], hv[i] = quantize_e4m3_rows(Kh)[2], quantize_e4m3_rows(Vh)[2]
        else:
            hk[i], hv[i] = gated_pool(K[g], V[g], gate_hca)
        for c, qi in enumerate(qis):
            sc[c, C4_PER_BLOCK * i:C4_PER_BLOCK * (i + 1)] = c4_scores(KI[g], qi)
    return hk, hv, sc


class StoredTokens:
    """A token source whose K and V are what FP8 KV storage holds (reading R20): each
    token's per-head E4M3 codes times their scale, as float64. Picklable."""

    def __init__(self, seq):
        self.seq = seq

    def __call__(self, pos):
        K, V, KI = self.seq(pos)
        return quantize_e4m3_rows(K)[2], quantize_e4m3_rows(V)[2], KI


def decode_reference(seq, n_win: int, gate_csa, gate_hca, cases, pmap=map, chunk: int = 32,
                     kv_format: str = "bf16"):
    """Decode outputs of one request at several lengths, without holding its cache.

    The same arithmetic as driving Oracle token by token, streamed block by block
    so that a request of 2**20 tokens fits in memory: for each case (L, q, q_idx,
    k), with L the length after the step's append, the request has L // 128 sealed
    blocks (reading R2); every sealed C4 entry is scored (R4), the top-k is
    selected (R8, R9), and one softmax runs over the SWA (the last min(L, n_win)
    tokens, oldest first), the HCA entries of the sealed blocks in order, and the
    selected C4 entries in ascending ordinal order ([Q&A] §4; R5, R6, R12).
    seq(pos) gives the request's tokens (see block_range_summary); pmap maps
    block_range_summary over block ranges (a process pool's map works).
    With kv_format "fp8" (reading R20) every token is taken as the State stores it
    (StoredTokens): the SWA, the tokens the C4 entries pool and the HCA entries.
    Returns [(idx int32 [k], scores float64 [k], out float64 [H][D])] per case.
    """
    if kv_format not in ("bf16", "fp8"):
        raise OracleError("invalid", f"kv_format {kv_format!r}")
    if kv_format == "fp8":
        seq = StoredTokens(seq)
    W_csa = np.asarray(gate_csa, dtype=np.float64).reshape(N_HEADS, HEAD_DIM)
    W_hca = np.asarray(gate_hca, dtype=np.float64).reshape(N_HEADS, HEAD_DIM)
    qis = [np.asarray(c[2], dtype=np.float64) for c in cases]
    nb_max = max(int(c[0]) // BLOCK for c in cases)
    ranges = [(seq, W_hca, qis, b, min(b + chunk, nb_max), kv_format) for b in range(0, nb_max, chunk)]
    hk = np.empty((nb_max, N_HEADS, HEAD_DIM), np.float64)
    hv = np.empty_like(hk)
    sc = np.empty((len(cases), C4_PER_BLOCK * nb_max), np.float64)
    for (_, _, _, b0, b1, _), (k_, v_, s_) in zip(ranges, pmap(block_range_summary, ranges)):
        hk[b0:b1], hv[b0:b1], sc[:, C4_PER_BLOCK * b0:C4_PER_BLOCK * b1] = k_, v_, s_
    res = []
    for c, (L, q, _, k) in enumerate(cases):
        L = int(L)
        nb = L // BLOCK
        idx, val = select_topk(sc[c, :C4_PER_BLOCK * nb], int(k))
        sel = idx[idx >= 0].astype(np.int64)
        Ks, Vs, _ = seq(np.arange(L - min(L, n_win), L, dtype=np.int64))
        parts_k, parts_v = [np.asarray(Ks, np.float64), hk[:nb].astype(np.float64)], \
                           [np.asarray(Vs, np.float64), hv[:nb].astype(np.float64)]
        if sel.size:
            pos = (M_CSA * sel[:, None] + np.arange(M_CSA)).reshape(-1)
            Kc, Vc, _ = seq(pos)
            Kc = np.asarray(Kc, np.float64).reshape(sel.size, M_CSA, N_HEADS, HEAD_DIM)
            Vc = np.asarray(Vc, np.float64).reshape(sel.size, M_CSA, N_HEADS, HEAD_DIM)
            ek = np.empty((sel.size, N_HEADS, HEAD_DIM))
            ev = np.empty_like(ek)
            for i in range(sel.size):                 # C4 entry j: tokens 4j .. 4j+3
                ek[i], ev[i] = gated_pool(Kc[i], Vc[i], W_csa)
            parts_k.append(ek)
            parts_v.append(ev)
        out = attention(q, np.concatenate(parts_k), np.concatenate(parts_v))
        res.append((idx, val, out))
    return res


# ---------------------------------------------------------------- cache state

class _Block:
    """One sealed, immutable Block Cache block: 32 C4 + 1 HCA + 128 indexer keys
    ([Ch12] §2.2; [Q&A] §2.2). With FP8 entries (R15) csa_k / csa_v hold the stored
    values (code value * scale) and the codes and scales are kept beside them; with
    MXFP4 indexer keys (R16) idx holds the stored values and idx_codes / idx_scales
    the codes and E8M0 scales; with FP8 KV (R20) hca_k / hca_v hold the stored HCA
    values and hca_*_codes / hca_*_scale their codes and scales."""
    __slots__ = ("csa_k", "csa_v", "hca_k", "hca_v", "idx", "csa_k_codes", "csa_v_codes",
                 "csa_k_scale", "csa_v_scale", "idx_codes", "idx_scales", "hca_k_codes", "hca_v_codes",
                 "hca_k_scale", "hca_v_scale")


class _State:
    """Per-request State block: SWA window of exact K/V (oldest first) and the
    in-flight tail of fewer than 128 tokens ([Q&A] §1.1, §3.3; [Ch12] §2.1).
    After a prefix attach (R17) the window and tail hold None until replayed."""

    def __init__(self, n_win: int):
        self.L = 0
        self.swa = deque(maxlen=n_win)     # (K, V) per token; drops the oldest ([Q&A] §4)
        self.swa_q = deque(maxlen=n_win)   # FP8 KV (R20): (K codes, K scales, V codes,
                                           # V scales) of each window token, else None
        self.tail = []                     # (K, V, kI) per token of the open block
        self.blocks = []                   # physical block ids, logical order


class Oracle:
    """The cache, driven call by call like the C ABI."""

    def __init__(self, n_win: int, gate_csa, gate_hca, max_states: int, max_blocks: int,
                 entry_format: str = "bf16", index_format: str = "f32", layer_type: str = "mixed",
                 c4_mode: str = "sealed", kv_format: str = "bf16"):
        if n_win < BLOCK or n_win % BLOCK:
            raise OracleError("invalid", "n_win must be a positive multiple of 128")
        if entry_format not in ("bf16", "fp8"):
            raise OracleError("invalid", "entry format is bf16 or fp8")
        if index_format not in ("f32", "mxfp4"):
            raise OracleError("invalid", "index format is f32 or mxfp4")
        if layer_type not in ("mixed", "swa", "csa", "hca"):
            raise OracleError("invalid", "layer type is mixed, swa, csa or hca")
        if c4_mode not in ("sealed", "eager"):
            raise OracleError("invalid", "c4 mode is sealed or eager")
        if kv_format not in ("bf16", "fp8"):
            raise OracleError("invalid", "kv format is bf16 or fp8")
        if c4_mode == "eager" and (entry_format != "bf16" or index_format != "f32" or kv_format != "bf16"):
            raise OracleError("invalid", "eager C4 takes bf16 entries, bf16 KV and f32 indexer keys")
        self.kv_format = kv_format
        self.eager = c4_mode == "eager"                       # reading R19
        self.layer_type = layer_type
        self.has_c4 = layer_type in ("mixed", "csa")          # reading R18
        self.has_hca = layer_type in ("mixed", "hca")
        self.entry_format = entry_format
        self.index_format = index_format
        self.n_win = int(n_win)
        self.W_csa = np.asarray(gate_csa, dtype=np.float64).reshape(N_HEADS, HEAD_DIM)
        self.W_hca = np.asarray(gate_hca, dtype=np.float64).reshape(N_HEADS, HEAD_DIM)
        self.max_states = int(max_states)
        self.max_blocks = int(max_blocks)
        self.free_states = list(range(self.max_states))
        self.free_blocks = list(range(self.max_blocks))
        heapq.heapify(self.free_states)
        heapq.heapify(self.free_blocks)
        self.refcount = np.zeros(self.max_blocks, np.int64)
        self.store: dict[int, _Block] = {}
        self.states: dict[int, _State] = {}

    def _stored(self, K, V):
        """A token's K and V as the State stores them: bf16 values as they come, or
        (R20) the per-head FP8 storage: returns (k, v, q), q = (K codes, K scales,
        V codes, V scales) with FP8 KV, else None."""
        if self.kv_format != "fp8":
            return np.asarray(K, dtype=np.float32), np.asarray(V, dtype=np.float32), None
        kc, ks, kv_ = quantize_e4m3_rows(np.asarray(K, dtype=np.float64))
        vc, vs, vv = quantize_e4m3_rows(np.asarray(V, dtype=np.float64))
        return kv_, vv, (kc, ks, vc, vs)

    # -- State pool --------------------------------------------------------
    def state_alloc(self) -> int:
        """Lowest free State slot, L = 0 ([Ch12] §2.1: one State block per request)."""
        if not self.free_states:
            raise OracleError("oom_states")
        s = heapq.heappop(self.free_states)
        self.states[s] = _State(self.n_win)
        return s

    def _get(self, s) -> _State:
        st = self.states.get(int(s))
        if st is None:
            raise OracleError("invalid", f"state {s} not allocated")
        return st

    def state_free(self, s: int):
        """Release the whole State block; drop one reference of each block
        ([Ch12] §2.1 release on request end; §2.2 refcount)."""
        st = self._get(s)
        for b in st.blocks:
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                del self.store[b]
                heapq.heappush(self.free_blocks, b)
        del self.states[int(s)]
        heapq.heappush(self.free_states, int(s))

    # -- append / seal ---------------------------------------------------------
    def append(self, states, tokens, defer_seal: bool = False):
        """Append tokens to each listed state, in list order.

        tokens[i] = (K [n][H][D], V [n][H][D], kI [n][4][64]). Per token
        ([Q&A] §4): K/V into the tail and SWA (SWA drops its oldest token),
        L += 1; when the tail holds 128 tokens the block is sealed ([Q&A] §3.1).
        With defer_seal the full tail waits for compress_flush; appending to a
        state whose tail is full is an error.
        """
        states = [int(s) for s in states]
        if len(set(states)) != len(states) or len(tokens) != len(states):
            raise OracleError("invalid", "duplicate or mismatched states")
        need = 0
        for s, (K, V, KI) in zip(states, tokens):
            st = self._get(s)
            n = len(K)
            if len(V) != n or len(KI) != n:
                raise OracleError("invalid", "ragged K/V/kI")
            if n == 0:
                continue
            if len(st.tail) == BLOCK:
                raise OracleError("state", "tail full: flush before appending")
            self._filled(st)
            if defer_seal:
                if len(st.tail) + n > BLOCK:
                    raise OracleError("state", "deferred append past one block")
            else:
                need += (len(st.tail) + n) // BLOCK
        if need > len(self.free_blocks):
            raise OracleError("oom_blocks")
        for s, (K, V, KI) in zip(states, tokens):
            st = self.states[s]
            for t in range(len(K)):
                k, v, q = self._stored(K[t], V[t])
                ki = np.asarray(KI[t], dtype=np.float32)
                st.swa.append((k, v))
                st.swa_q.append(q)
                st.tail.append((k, v, ki))
                st.L += 1
                if len(st.tail) == BLOCK and not defer_seal:
                    self._seal(st)

    def compress_flush(self, states):
        """Seal every listed state whose tail holds a full block (deferred seals)."""
        states = [int(s) for s in states]
        if len(set(states)) != len(states):
            raise OracleError("invalid", "duplicate states")
        need = sum(1 for s in states if len(self._get(s).tail) == BLOCK)
        if need > len(self.free_blocks):
            raise OracleError("oom_blocks")
        for s in states:
            st = self.states[s]
            if len(st.tail) == BLOCK:
                self._seal(st)

    def _seal(self, st: _State):
        """Compress the 128-token tail into 32 C4 + 1 HCA entries and keep its 128
        indexer keys, in a new immutable block ([Q&A] §2.2, §3.1; [Ch12] §2.2)."""
        b = heapq.heappop(self.free_blocks)
        Kt = np.stack([t[0] for t in st.tail]).astype(np.float64)   # [128][H][D]
        Vt = np.stack([t[1] for t in st.tail]).astype(np.float64)
        blk = _Block()
        for name in _Block.__slots__:
            setattr(blk, name, None)
        self.store[b] = blk
        self.refcount[b] = 1
        st.blocks.append(b)
        if self.has_c4:
            self._seal_c4(blk, st, Kt, Vt)
        if self.has_hca:                              # all 128 tokens
            if self.kv_format == "fp8":               # reading R20
                Kh, Vh = gated_pool(Kt, Vt, self.W_hca, rounded=False)
                blk.hca_k_codes, blk.hca_k_scale, blk.hca_k = quantize_e4m3_rows(Kh)
                blk.hca_v_codes, blk.hca_v_scale, blk.hca_v = quantize_e4m3_rows(Vh)
            else:
                blk.hca_k, blk.hca_v = gated_pool(Kt, Vt, self.W_hca)
        st.tail = []                                  # tail cleared ([Q&A] §3.1)

    def _seal_c4(self, blk: _Block, st: _State, Kt, Vt):
        """The 32 C4 entries and 128 indexer keys of the block being sealed."""
        fp8 = self.entry_format == "fp8"
        blk.csa_k = np.empty((C4_PER_BLOCK, N_HEADS, HEAD_DIM), np.float64 if fp8 else np.float32)
        blk.csa_v = np.empty_like(blk.csa_k)
        if fp8:
            blk.csa_k_codes = np.empty((C4_PER_BLOCK, N_HEADS, HEAD_DIM), np.uint8)
            blk.csa_v_codes = np.empty_like(blk.csa_k_codes)
            blk.csa_k_scale = np.empty((C4_PER_BLOCK, N_HEADS), np.float32)
            blk.csa_v_scale = np.empty_like(blk.csa_k_scale)
        for j in range(C4_PER_BLOCK):                 # C4 entry j: tokens 4j .. 4j+3
            g = slice(M_CSA * j, M_CSA * (j + 1))
            if fp8:                                   # reading R15
                Kj, Vj = gated_pool(Kt[g], Vt[g], self.W_csa, rounded=False)
                blk.csa_k_codes[j], blk.csa_k_scale[j], blk.csa_k[j] = quantize_e4m3_rows(Kj)
                blk.csa_v_codes[j], blk.csa_v_scale[j], blk.csa_v[j] = quantize_e4m3_rows(Vj)
            else:
                blk.csa_k[j], blk.csa_v[j] = gated_pool(Kt[g], Vt[g], self.W_csa)
        keys = np.stack([t[2] for t in st.tail]).astype(np.float32)       # [128][4][64]
        if self.index_format == "mxfp4":              # reading R16
            codes, scales, vals = quantize_mxfp4_rows(keys.reshape(BLOCK, -1))
            blk.idx = vals.reshape(keys.shape)
            blk.idx_codes, blk.idx_scales = codes, scales
        else:
            blk.idx = keys

    # -- prefix sharing --------------------------------------------------------
    def share(self, src: int, dst: int):
        """dst becomes a fork of src (reading R11; [Ch12] §2.2 refcount sharing)."""
        a, d = self._get(src), self._get(dst)
        if int(src) == int(dst):
            raise OracleError("invalid", "src == dst")
        if d.L != 0 or d.blocks:
            raise OracleError("state", "dst not fresh")
        if len(a.tail) == BLOCK:
            raise OracleError("state", "src has a pending seal")
        self._filled(a)
        for b in a.blocks:
            self.refcount[b] += 1
        d.blocks = list(a.blocks)
        d.L = a.L
        d.swa = deque(a.swa, maxlen=self.n_win)
        d.swa_q = deque(a.swa_q, maxlen=self.n_win)
        d.tail = list(a.tail)

    # -- prefix hits (reading R17) -------------------------------------------------
    def block_ref(self, blocks, delta: int):
        """Add delta (+1 or -1) to each listed block's refcount: a prefix entry
        holding blocks without a State ([Ch12] §2.2 refcount; [Disk]). A block whose
        count reaches 0 is freed. All-or-nothing."""
        blocks = [int(b) for b in blocks]
        if delta not in (1, -1):
            raise OracleError("invalid", "delta must be +1 or -1")
        for b in set(blocks):
            if not (0 <= b < self.max_blocks) or self.refcount[b] <= 0:
                raise OracleError("invalid", f"block {b} not in use")
            if delta < 0 and blocks.count(b) > self.refcount[b]:
                raise OracleError("invalid", f"block {b} released more than held")
        for b in blocks:
            self.refcount[b] += delta
            if self.refcount[b] == 0:
                del self.store[b]
                heapq.heappush(self.free_blocks, b)

    def prefix_attach(self, dst: int, blocks, length: int):
        """dst (fresh) takes the prefix's first length // 128 blocks (refcount + 1)
        and length; its window and tail are unfilled until replayed or restored."""
        d = self._get(dst)
        length = int(length)
        if d.L != 0 or d.blocks:
            raise OracleError("state", "dst not fresh")
        nb = length // BLOCK if length >= 0 else -1
        blocks = [int(b) for b in blocks][:max(nb, 0)]
        if length < 0 or len(blocks) < nb:
            raise OracleError("invalid", "length needs length // 128 blocks")
        for b in blocks:
            if not (0 <= b < self.max_blocks) or self.refcount[b] <= 0:
                raise OracleError("invalid", f"block {b} not in use")
        for b in blocks:
            self.refcount[b] += 1
        d.blocks = blocks
        d.L = length
        d.swa = deque([None] * min(length, self.n_win), maxlen=self.n_win)
        d.swa_q = deque([None] * min(length, self.n_win), maxlen=self.n_win)
        d.tail = [None] * (length - BLOCK * nb)

    def state_write(self, states, tokens, pos0):
        """Replay raw tokens into States without sealing: tokens[i] = (K, V, kI) of
        positions pos0[i] .. pos0[i] + n - 1, all below the state's L. Positions in
        the window [L - n_win, L) fill their SWA slot, those of the open block also
        their tail slot; older ones are dropped. L and blocks are unchanged."""
        states = [int(x) for x in states]
        if len(set(states)) != len(states) or len(tokens) != len(states) or len(pos0) != len(states):
            raise OracleError("invalid", "duplicate or mismatched states")
        for s_, (K, V, KI), p0 in zip(states, tokens, pos0):
            st = self._get(s_)
            n = len(K)
            if len(V) != n or len(KI) != n:
                raise OracleError("invalid", "ragged K/V/kI")
            if n and (int(p0) < 0 or int(p0) + n > st.L):
                raise OracleError("invalid", "positions outside [0, L)")
        for s_, (K, V, KI), p0 in zip(states, tokens, pos0):
            st = self.states[s_]
            w0 = st.L - len(st.swa)                    # first position in the window
            t0 = st.L - len(st.tail)                   # first position of the tail
            for t in range(len(K)):
                p = int(p0) + t
                k, v, q = self._stored(K[t], V[t])
                if p >= w0:
                    st.swa[p - w0] = (k, v)
                    st.swa_q[p - w0] = q
                if p >= t0:
                    st.tail[p - t0] = (k, v, np.asarray(KI[t], dtype=np.float32))

    def checkpoint(self, s: int) -> dict:
        """The State's SWA window, tail and length (a Periodic / Full checkpoint)."""
        st = self._get(s)
        if any(x is None for x in st.swa) or any(x is None for x in st.tail):
            raise OracleError("state", "state not filled")
        return {"len": st.L, "swa": list(st.swa), "swa_q": list(st.swa_q), "tail": list(st.tail)}

    def restore(self, s: int, ck: dict):
        """Fill a state attached at L >= c from the checkpoint taken at c: window
        positions [max(c - n_win, L - n_win), c) and the tail positions below c that
        belong to the state's open block. Positions [c, L) stay for replay."""
        st = self._get(s)
        c = int(ck["len"])
        if c > st.L or c < 0:
            raise OracleError("invalid", "checkpoint is past the state's length")
        w0, t0 = st.L - len(st.swa), st.L - len(st.tail)
        for i, (item, q) in enumerate(zip(ck["swa"], ck["swa_q"])):
            p = c - len(ck["swa"]) + i
            if p >= w0:
                st.swa[p - w0] = item
                st.swa_q[p - w0] = q
        for i, item in enumerate(ck["tail"]):
            p = c - len(ck["tail"]) + i
            if p >= t0:
                st.tail[p - t0] = item

    def _open_groups(self, st: _State) -> int:
        """Complete groups of 4 tokens in the open block that have eager entries."""
        return len(st.tail) // M_CSA if (self.eager and self.has_c4) else 0

    def _open_entry(self, st: _State, i: int):
        """C4 entry of group i of the open block, pooled as the seal pools it."""
        g = st.tail[M_CSA * i:M_CSA * (i + 1)]
        Kg = np.stack([t[0] for t in g]).astype(np.float64)
        Vg = np.stack([t[1] for t in g]).astype(np.float64)
        return gated_pool(Kg, Vg, self.W_csa)

    def _filled(self, st: _State):
        if any(x is None for x in st.swa) or any(x is None for x in st.tail):
            raise OracleError("state", "state not filled: replay or restore first")

    # -- indexer top-k -----------------------------------------------------------
    def scores(self, s: int, q_idx) -> np.ndarray:
        """Scores of the request's sealed C4 entries, ordinal j = 32 * block + slot."""
        st = self._get(s)
        if not self.has_c4:
            return np.zeros(0)
        out = [c4_scores(self.store[b].idx, q_idx) for b in st.blocks]
        g = self._open_groups(st)
        if g:                                          # the open block's entries (R19)
            keys = np.stack([t[2] for t in st.tail[:M_CSA * g]])
            out.append(c4_scores(np.concatenate([keys, np.zeros((BLOCK - len(keys),) + keys.shape[1:])]),
                                 q_idx)[:g])
        return np.concatenate(out) if out else np.zeros(0)

    def topk(self, s: int, q_idx, k: int, sorted: bool = False):
        if k < 1:
            raise OracleError("invalid", "k must be >= 1")
        return select_topk(self.scores(s, q_idx), k, sorted)

    # -- heterogeneous attention -------------------------------------------------
    def keys(self, s: int, sel, k: int | None = None):
        """Materialise the key/value list: SWA (oldest -> newest), HCA of every
        sealed block, then C4 entries named by `sel` ([Q&A] §4; [Layout]
        Classical KV cache read modes). Only the first min(k, N_c) entries of sel
        are read; -1 and out-of-range ordinals are skipped."""
        st = self._get(s)
        self._filled(st)
        K = [t[0] for t in st.swa]
        V = [t[1] for t in st.swa]
        for b in st.blocks if self.has_hca else []:
            K.append(self.store[b].hca_k)
            V.append(self.store[b].hca_v)
        ns = C4_PER_BLOCK * len(st.blocks) if self.has_c4 else 0
        nc = ns + self._open_groups(st)
        sel = np.asarray(sel if sel is not None else [], dtype=np.int64).reshape(-1)
        kk = min(len(sel) if k is None else int(k), nc)
        for j in sel[:kk]:
            if 0 <= j < ns:
                blk = self.store[st.blocks[j // C4_PER_BLOCK]]
                K.append(blk.csa_k[j % C4_PER_BLOCK])
                V.append(blk.csa_v[j % C4_PER_BLOCK])
            elif ns <= j < nc:                         # an open-block entry (R19)
                ke, ve = self._open_entry(st, int(j - ns))
                K.append(ke)
                V.append(ve)
        return np.stack(K), np.stack(V)

    def attend(self, s: int, q, sel, k: int | None = None) -> np.ndarray:
        st = self._get(s)
        if st.L == 0:
            raise OracleError("invalid", "empty state")
        K, V = self.keys(s, sel, k)
        return attention(q, K, V)

    # -- introspection -------------------------------------------------------------
    def info(self, s: int) -> dict:
        st = self._get(s)
        d = length_split(st.L)
        return {"len": st.L, "n_blocks": len(st.blocks), "csa_tail": st.L % M_CSA,
                "hca_tail": len(st.tail), "swa_len": len(st.swa), "split": d}

    def table(self, s: int) -> list:
        return list(self._get(s).blocks)

    def block(self, b: int) -> _Block:
        return self.store[int(b)]
