"""Helpers of the GPU parity tests: seeded inputs for both sides and comparisons.

The oracle receives values generated on the host by `synth`; the GPU receives the
same values generated on the device by synth/synth_gen.hip (checked equal bit
for bit by test_gpu_synth) or uploaded from the host arrays.
"""

from __future__ import annotations

import numpy as np

import synth

H, D, HI, DI = 16, 128, 4, 64


def host_tokens(seed, keys, pos):
    """float64 K, V [n][16][128] (bf16 values) and kI [n][4][64] for (key, position) rows."""
    keys = np.broadcast_to(np.asarray(keys, np.uint64), np.shape(pos))
    K = synth.bf16_bits_to_f32(synth.tokens_bf16(seed, synth.STREAM_K, keys, pos)).astype(np.float64)
    V = synth.bf16_bits_to_f32(synth.tokens_bf16(seed, synth.STREAM_V, keys, pos)).astype(np.float64)
    KI = synth.tokens_f32(seed, synth.STREAM_IDXK, keys, pos).astype(np.float64)
    return K, V, KI


def host_queries(seed, keys, pos):
    keys = np.broadcast_to(np.asarray(keys, np.uint64), np.shape(pos))
    Q = synth.bf16_bits_to_f32(synth.tokens_bf16(seed, synth.STREAM_Q, keys, pos)).astype(np.float64)
    QI = synth.tokens_f32(seed, synth.STREAM_QI, keys, pos).astype(np.float64)
    return Q, QI


def dev_rows(seed, stream_id, keys, pos, bf16: bool):
    """Device tensor of generator rows for per-row keys and positions."""
    import torch
    from synth.device import fill_rows
    keys = np.asarray(keys, np.int64).reshape(-1)
    pos = np.asarray(pos, np.int64).reshape(-1)
    n = pos.size
    if bf16:
        out = torch.empty((n, H, D), dtype=torch.bfloat16, device="cuda")
    else:
        out = torch.empty((n, HI, DI), dtype=torch.float32, device="cuda")
    if n == 0:
        return out
    kt = torch.from_numpy(keys.astype(np.uint32).view(np.int32)).cuda()
    pt = torch.from_numpy(pos).cuda()
    fill_rows(out, seed, stream_id, keys=kt, pos=pt)
    return out


def dev_tokens(seed, keys, pos):
    keys = np.broadcast_to(np.asarray(keys, np.int64), np.shape(pos))
    return (dev_rows(seed, synth.STREAM_K, keys, pos, True),
            dev_rows(seed, synth.STREAM_V, keys, pos, True),
            dev_rows(seed, synth.STREAM_IDXK, keys, pos, False))


def dev_queries(seed, keys, pos):
    keys = np.broadcast_to(np.asarray(keys, np.int64), np.shape(pos))
    return (dev_rows(seed, synth.STREAM_Q, keys, pos, True),
            dev_rows(seed, synth.STREAM_QI, keys, pos, False))


def bf16_to_f64(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def topk_accept(gpu_idx, gpu_val, ref_scores, k, eps_rel=1e-4, sorted=False):
    """True if the GPU's top-k row is an acceptable answer for the oracle scores:
    kk = min(k, N) distinct valid entries, -1 after, and every index outside the
    oracle's set (or missing from it) has an oracle score within eps of the
    oracle's kk-th score tau; ascending ordinals, or scores non-increasing (within
    eps) when sorted."""
    from oracle import select_topk
    N = len(ref_scores)
    kk = min(k, N)
    ref_idx, ref_val = select_topk(ref_scores, k, sorted=True)
    g = np.asarray(gpu_idx)
    if np.any(g[kk:] != -1) or np.any(g[:kk] < 0) or np.any(g[:kk] >= N):
        return False
    if len(set(g[:kk].tolist())) != kk:
        return False
    if kk == 0:
        return True
    tau = ref_val[kk - 1]
    eps = eps_rel * max(1.0, abs(tau))
    diff = set(g[:kk].tolist()) ^ set(ref_idx[:kk].tolist())
    if any(abs(ref_scores[j] - tau) > eps for j in diff):
        return False
    if not sorted:
        return bool(np.all(np.diff(g[:kk]) > 0))
    s = ref_scores[g[:kk]]
    return bool(np.all(np.diff(s) <= eps))
