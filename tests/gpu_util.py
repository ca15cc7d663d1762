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


# ---- FP8 storage of pooled entries: the GPU pools in float32, the oracle in float64

EPS_POOL = 5e-5   # bound on the float32 pooling error, relative to sum_t alpha_t |x_t|


def pool_magnitude(Kg, Vg, W):
    """Per head and dim, sum_t alpha_t |K_t| and sum_t alpha_t |V_t| for the gated
    pooling of the tokens Kg, Vg [m][H][D] with gate weights W [H][D] (reading R1).

    This is the scale of the float32 rounding error of a pooled value: its weighted
    sum of m <= 128 products is off by at most about 128 * 2**-24 (7.6e-6) times
    this, and its weights alpha_t = softmax(<W, K_t>) by at most about
    128 * 2**-24 * sum_d |W_d K_td| in relative terms, which for gates of scale 0.02
    and tokens below 3 in magnitude is at most about 2.5 times that again. The sum,
    2.7e-5 times this, is the bound EPS_POOL = 5e-5 holds with a margin of about 2."""
    Kg = np.asarray(Kg, np.float64)
    Vg = np.asarray(Vg, np.float64)
    g = np.einsum("thd,hd->th", Kg, np.asarray(W, np.float64))
    a = np.exp(g - g.max(axis=0, keepdims=True))
    a /= a.sum(axis=0, keepdims=True)
    return np.einsum("th,thd->hd", a, np.abs(Kg)), np.einsum("th,thd->hd", a, np.abs(Vg))


def check_fp8(codes, scale, ref_codes, ref_scale, x, what, mag=None):
    """FP8 storage of an entry pooled on the GPU in float32 and by the oracle in
    float64 (x: the oracle's unquantised entry [..][128]). The scales agree to 1e-6.
    A code is an integer decided from the pooled value, and the two poolings differ
    in their last bits, so a code may differ from the oracle's only where either
    rounding is correct: the two codes' values are neighbours on the signed E4M3
    grid (+0 and -0 are the same value there), and the oracle's scaled value
    y = x / s lies within the pooling error of the midpoint between them. The error
    is EPS_POOL * max(|y|, mag / s), with mag the pool_magnitude of the element
    (without mag, EPS_POOL * max(|y|, 2**-9))."""
    from oracle import e4m3_decode
    pos = e4m3_decode(np.arange(0x7F))                      # 0 .. 448
    grid = np.concatenate([-pos[:0:-1], pos])               # the signed grid, 0 once
    assert np.allclose(scale, ref_scale, rtol=1e-6, atol=0), what
    diff = codes != ref_codes
    assert np.mean(diff) < 0.005, (what, np.mean(diff))
    if not diff.any():
        return
    s = np.broadcast_to(ref_scale[..., None].astype(np.float64), x.shape)
    y = (x / s)[diff]
    a, b = e4m3_decode(codes[diff]), e4m3_decode(ref_codes[diff])
    same = a == b                                           # +0 against -0
    steps = np.abs(np.searchsorted(grid, a) - np.searchsorted(grid, b))
    assert np.all(same | (steps == 1)), (what, "codes are not neighbours", a[~same & (steps != 1)],
                                         b[~same & (steps != 1)])
    mid = (a + b) / 2
    if mag is None:
        tol = EPS_POOL * np.maximum(np.abs(y), 2.0 ** -9)
    else:
        tol = EPS_POOL * np.maximum(np.abs(y), (np.asarray(mag, np.float64) / s)[diff])
    # a sign of zero differs only where y itself is within the error of 0
    assert np.all(np.abs(y - mid) <= tol), (what, y, a, b, tol)
