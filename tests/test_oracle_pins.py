"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test ties one oracle function to something other than itself: the pages'
worked example (tests/golden/l130_example.json), closed forms, invariants,
exact integer arithmetic, library routines (torch bf16 conversion, torch SDPA,
Python's sort) or brute force on small inputs.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import synth
from oracle import (BLOCK, C4_PER_BLOCK, HEAD_DIM, N_HEADS, Oracle, OracleError,
                    attention, bf16_round, c4_scores, gated_pool, length_split,
                    select_topk, token_scores)

SEED = 0x1234


def toks(key, p0, n, seed=SEED):
    """Raw inputs of n tokens at positions p0.. as float64 (exact bf16 / fp32 values)."""
    pos = np.arange(p0, p0 + n)
    K = synth.bf16_bits_to_f32(synth.tokens_bf16(seed, synth.STREAM_K, key, pos)).astype(np.float64)
    V = synth.bf16_bits_to_f32(synth.tokens_bf16(seed, synth.STREAM_V, key, pos)).astype(np.float64)
    KI = synth.tokens_f32(seed, synth.STREAM_IDXK, key, pos).astype(np.float64)
    return K, V, KI


def make_oracle(n_win=128, max_states=8, max_blocks=64, gates=None):
    Wc, Wh = gates if gates is not None else synth.gate_weights(SEED)
    return Oracle(n_win, Wc, Wh, max_states, max_blocks)


# ------------------------------------------------------------------ the pages' example

def test_l130_worked_example(root):
    g = json.load(open(os.path.join(root, "tests", "golden", "l130_example.json")))
    o = make_oracle()
    s = o.state_alloc()
    K, V, KI = toks(0, 0, g["L"])
    o.append([s], [(K, V, KI)])
    info = o.info(s)
    assert info["len"] == g["L"]
    assert info["n_blocks"] == g["blocks"]
    assert info["split"]["c4"] == g["c4_entries"] and info["split"]["hca"] == g["hca_entries"]
    assert info["hca_tail"] == g["tail_tokens"] and info["csa_tail"] == g["csa_tail"]
    # Classical holds exactly tokens [0, 128): rebuild the block from them
    a, b = g["classical_positions"]
    blk = o.block(o.table(s)[0])
    for j in range(C4_PER_BLOCK):
        ck, cv = gated_pool(K[a + 4 * j:a + 4 * j + 4], V[a + 4 * j:a + 4 * j + 4], o.W_csa)
        assert np.array_equal(ck, blk.csa_k[j]) and np.array_equal(cv, blk.csa_v[j])
    hk, hv = gated_pool(K[a:b], V[a:b], o.W_hca)
    assert np.array_equal(hk, blk.hca_k) and np.array_equal(hv, blk.hca_v)
    assert np.array_equal(blk.idx, KI[a:b].astype(np.float32))
    # tokens 128, 129 stay in the tail (State pool), not in Classical
    t0, t1 = g["tail_positions"]
    st = o.states[s]
    assert len(st.tail) == t1 - t0
    for i, p in enumerate(range(t0, t1)):
        assert np.array_equal(st.tail[i][0], K[p].astype(np.float32))


@pytest.mark.parametrize("L", [0, 1, 3, 4, 127, 128, 129, 130, 255, 256, 257, 383, 640, 1000])
def test_length_decomposition(L):
    """L = 128 q + r -> 32q C4 + q HCA, tail r; CSA tail <= 3, HCA tail <= 127."""
    o = make_oracle(max_blocks=16)
    s = o.state_alloc()
    K, V, KI = toks(1, 0, L)
    o.append([s], [(K, V, KI)])
    info = o.info(s)
    q, r = L // 128, L % 128
    assert info["n_blocks"] == q and len(o.table(s)) == q
    assert info["split"] == length_split(L)
    assert info["split"]["c4"] == 32 * q and info["hca_tail"] == r
    assert 0 <= info["csa_tail"] <= 3 and 0 <= info["hca_tail"] <= 127
    assert info["csa_tail"] == L % 4


def test_length_split_closed_form():
    for L in range(0, 5000, 7):
        d = length_split(L)
        assert 128 * d["blocks"] + d["tail"] == L and 0 <= d["tail"] < 128
        assert d["c4"] == 32 * d["blocks"] and d["hca"] == d["blocks"]


@pytest.mark.parametrize("n_win,L", [(128, 5), (128, 128), (128, 300), (256, 255), (256, 700)])
def test_swa_is_last_window(n_win, L):
    """The SWA holds exactly the last min(L, n_win) tokens, oldest first."""
    o = make_oracle(n_win=n_win, max_blocks=16)
    s = o.state_alloc()
    K, V, KI = toks(2, 0, L)
    # append in uneven pieces
    cuts = [0, 1, 7, 100, 129, L]
    cuts = sorted(set(min(c, L) for c in cuts))
    for a, b in zip(cuts[:-1], cuts[1:]):
        o.append([s], [(K[a:b], V[a:b], KI[a:b])])
    w = min(L, n_win)
    swa = o.states[s].swa
    assert len(swa) == w
    for i, (k, v) in enumerate(swa):
        assert np.array_equal(k, K[L - w + i].astype(np.float32))
        assert np.array_equal(v, V[L - w + i].astype(np.float32))


def test_sealed_blocks_immutable():
    o = make_oracle(max_blocks=16)
    s = o.state_alloc()
    K, V, KI = toks(3, 0, 700)
    o.append([s], [(K[:300], V[:300], KI[:300])])
    b0 = o.table(s)[0]
    snap = {a: getattr(o.block(b0), a).copy() for a in ("csa_k", "csa_v", "hca_k", "hca_v", "idx")}
    o.append([s], [(K[300:], V[300:], KI[300:])])
    for a, v in snap.items():
        assert np.array_equal(getattr(o.block(b0), a), v)


# ------------------------------------------------------------------ bf16 rounding

def test_bf16_round_matches_torch_on_float32():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(200000) * 10.0 ** rng.integers(-6, 6, 200000),
                        synth.bf16_bits_to_f32(np.arange(0x0080, 0x7F00, 7, dtype=np.uint16))
                        * (1 + 2.0 ** -8)]).astype(np.float32)   # exact ties
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(bf16_round(x.astype(np.float64)), ref)


def test_bf16_round_exact_nearest_float64():
    """Brute force with exact rationals: the nearest of the two bf16 neighbours."""
    rng = np.random.default_rng(6)
    xs = rng.standard_normal(3000) * 3.0
    for x in xs:
        y = float(bf16_round(x))
        e = math.frexp(x)[1]
        ulp = Fraction(2) ** (e - 8)
        lo = Fraction(math.floor(Fraction(x) / ulp)) * ulp
        hi = lo + ulp
        dx = Fraction(x)
        if dx - lo < hi - dx:
            exp = lo
        elif dx - lo > hi - dx:
            exp = hi
        else:
            exp = lo if (lo / ulp) % 2 == 0 else hi
        assert Fraction(y) == exp


# ------------------------------------------------------------------ compressor (reading R1)

def test_pool_zero_gates_is_mean():
    K, V, _ = toks(4, 0, 128)
    Z = np.zeros((N_HEADS, HEAD_DIM))
    for m in (4, 128):
        ck, cv = gated_pool(K[:m], V[:m], Z)
        assert np.array_equal(ck, bf16_round(np.mean(K[:m], axis=0)).astype(np.float32))
        assert np.array_equal(cv, bf16_round(np.mean(V[:m], axis=0)).astype(np.float32))


def test_pool_two_tokens_logistic():
    """m = 2: alpha_0 = 1 / (1 + exp(g1 - g0)), alpha_1 = 1 - alpha_0."""
    K, V, _ = toks(5, 0, 2)
    W = synth.gate_weights(99)[0].astype(np.float64) * 10
    ck, cv = gated_pool(K, V, W)
    for h in range(N_HEADS):
        g0 = float(np.dot(W[h], K[0, h]))
        g1 = float(np.dot(W[h], K[1, h]))
        a0 = 1.0 / (1.0 + math.exp(g1 - g0))
        exp_k = bf16_round(a0 * K[0, h] + (1 - a0) * K[1, h])
        exp_v = bf16_round(a0 * V[0, h] + (1 - a0) * V[1, h])
        # one bf16 ulp of slack for fp64 rounding order at exact ties
        assert np.allclose(ck[h], exp_k, rtol=2 ** -7, atol=0)
        assert np.allclose(cv[h], exp_v, rtol=2 ** -7, atol=0)
        assert np.mean(ck[h] == exp_k) > 0.98


def test_pool_permutation_invariant_and_convex():
    K, V, _ = toks(6, 0, 128)
    W = synth.gate_weights(7)[1]
    rng = np.random.default_rng(0)
    for m in (4, 128):
        perm = rng.permutation(m)
        a = gated_pool(K[:m], V[:m], W)
        b = gated_pool(K[:m][perm], V[:m][perm], W)
        assert np.allclose(a[0], b[0], rtol=2 ** -7, atol=0) and np.allclose(a[1], b[1], rtol=2 ** -7, atol=0)
        for ent, src in ((a[0], K[:m]), (a[1], V[:m])):
            assert np.all(ent >= src.min(axis=0)) and np.all(ent <= src.max(axis=0))


def test_pool_dominant_gate_selects_token():
    K, V, _ = toks(8, 0, 4)
    W = 1000.0 * K[2]          # gate of token 2 dominates in every head
    ck, cv = gated_pool(K, V, W)
    assert np.array_equal(ck, K[2].astype(np.float32)) and np.array_equal(cv, V[2].astype(np.float32))


def test_seal_uses_csa_gates_for_c4_and_hca_gates_for_hca():
    K, V, KI = toks(9, 0, 128)
    Wr = synth.gate_weights(11)[0] * 50
    Z = np.zeros((N_HEADS, HEAD_DIM), np.float32)
    for Wc, Wh in ((Z, Wr), (Wr, Z)):
        o = make_oracle(gates=(Wc, Wh))
        s = o.state_alloc()
        o.append([s], [(K, V, KI)])
        blk = o.block(o.table(s)[0])
        mean_c = np.array([bf16_round(K[4 * j:4 * j + 4].mean(axis=0)) for j in range(32)])
        mean_h = bf16_round(K.mean(axis=0))
        if Wc is Z:
            assert np.array_equal(blk.csa_k, mean_c.astype(np.float32))
            assert not np.array_equal(blk.hca_k, mean_h.astype(np.float32))
        else:
            assert np.array_equal(blk.hca_k, mean_h.astype(np.float32))
            assert not np.array_equal(blk.csa_k, mean_c.astype(np.float32))


# ------------------------------------------------------------------ indexer (reading R4)

def test_indexer_scores_exact_integer():
    """Inputs are odd multiples of 2**-8: scores * 2**18 are exact integers; compare
    with integer arithmetic on the generator's integers."""
    pos = np.arange(0, 128)
    zi = synth.z_ints(SEED, synth.STREAM_IDXK, 3, (pos[:, None] * 256 + np.arange(256)).astype(np.uint64))
    qi = synth.z_ints(SEED, synth.STREAM_QI, 3, np.arange(256, dtype=np.uint64))
    KI = zi.reshape(128, 4, 64) / 256.0
    q = qi.reshape(4, 64) / 256.0
    S = c4_scores(KI, q)
    for j in range(32):
        exact = sum(int(qi[e]) * int(zi[4 * j + u, e]) for u in range(4) for e in range(256))
        assert Fraction(float(S[j])) == Fraction(exact, 4 * 65536)


def test_indexer_one_hot_query_picks_coordinate():
    _, _, KI = toks(10, 0, 128)
    for h, d in ((0, 0), (3, 63), (1, 17)):
        q = np.zeros((4, 64))
        q[h, d] = 1.0
        S = c4_scores(KI, q)
        for j in range(32):
            assert S[j] == np.mean([KI[4 * j + u, h, d] for u in range(4)])
        assert np.array_equal(token_scores(KI, q), KI[:, h, d])


# ------------------------------------------------------------------ top-k (readings R8, R9)

def test_topk_full_sort_when_k_covers_all():
    rng = np.random.default_rng(1)
    s = np.round(rng.standard_normal(100) * 4) / 4      # many ties
    idx, val = select_topk(s, 128, sorted=True)
    ref = sorted(range(100), key=lambda j: (-s[j], j))
    assert list(idx[:100]) == ref and np.all(idx[100:] == -1)
    idx, val = select_topk(s, 128)
    assert list(idx[:100]) == list(range(100)) and np.array_equal(val[:100], s)
    assert np.all(np.isneginf(val[100:]))


def test_topk_brute_force_small():
    rng = np.random.default_rng(2)
    for trial in range(200):
        n = int(rng.integers(1, 40))
        k = int(rng.integers(1, 50))
        s = rng.integers(-3, 4, n).astype(np.float64)
        kk = min(k, n)
        # brute force: j is chosen iff fewer than kk entries beat it under (score desc, ordinal asc)
        beats = lambda a, b: s[a] > s[b] or (s[a] == s[b] and a < b)
        exp = [j for j in range(n) if sum(beats(i, j) for i in range(n)) < kk]
        idx, val = select_topk(s, k)
        assert idx[:kk].tolist() == exp and np.all(idx[kk:] == -1)
        assert np.array_equal(val[:kk], s[exp])
        idx, _ = select_topk(s, k, sorted=True)
        chosen = idx[:kk]
        assert sorted(chosen.tolist()) == exp
        for a, b in zip(chosen[:-1], chosen[1:]):
            assert beats(a, b)
        assert np.all(idx[kk:] == -1)


def test_topk_ties_lowest_index_and_negzero():
    s = np.array([1.0, 0.0, -0.0, 1.0, 0.0, 2.0])
    idx, _ = select_topk(s, 4, sorted=True)
    assert list(idx) == [5, 0, 3, 1]
    idx, _ = select_topk(s, 4)
    assert list(idx) == [0, 1, 3, 5]


# ------------------------------------------------------------------ attention

def sdpa64(q, Kc, Vc):
    qt = torch.from_numpy(np.asarray(q, np.float64))[:, None, :]            # [H][1][D]
    kt = torch.from_numpy(np.asarray(Kc, np.float64)).permute(1, 0, 2).contiguous()
    vt = torch.from_numpy(np.asarray(Vc, np.float64)).permute(1, 0, 2).contiguous()
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[:, 0, :].numpy()


def test_attention_matches_sdpa():
    K, V, _ = toks(11, 0, 50)
    q = toks(12, 0, 1)[0][0]
    assert np.allclose(attention(q, K, V), sdpa64(q, K, V), rtol=1e-12, atol=1e-12)


def test_attention_uniform_keys_is_mean_of_values():
    K, V, _ = toks(13, 0, 9)
    q = toks(14, 0, 1)[0][0]
    Ku = np.repeat(K[:1], 9, axis=0)
    assert np.allclose(attention(q, Ku, V), V.mean(axis=0), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("L", [1, 37, 127])
def test_decode_without_blocks_is_plain_mha(L):
    """L < 128: no blocks, the SWA holds every token: plain MHA decode."""
    o = make_oracle()
    s = o.state_alloc()
    K, V, KI = toks(15, 0, L)
    o.append([s], [(K, V, KI)])
    q = toks(16, 0, 1)[0][0]
    out = o.attend(s, q, [], k=16)
    assert np.allclose(out, sdpa64(q, K, V), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("n_win,L,k", [(128, 130, 16), (128, 256, 64), (256, 777, 40), (128, 1000, 1000)])
def test_attention_brute_force_concatenated_cache(n_win, L, k):
    """Brute force from the raw tokens: SWA = last min(L, n_win) tokens, HCA = pool of
    each 128-token group, C4 = pool of each selected 4-token group; one softmax."""
    o = make_oracle(n_win=n_win, max_blocks=16)
    s = o.state_alloc()
    K, V, KI = toks(17, 0, L)
    o.append([s], [(K, V, KI)])
    qi = synth.tokens_f32(SEED, synth.STREAM_QI, 17, [L - 1])[0]
    q = toks(18, 0, 1)[0][0]
    sel, _ = o.topk(s, qi, k)
    w = min(L, n_win)
    nb = L // 128
    Kc = [K[L - w:]]
    Vc = [V[L - w:]]
    for b in range(nb):
        hk, hv = gated_pool(K[128 * b:128 * b + 128], V[128 * b:128 * b + 128], o.W_hca)
        Kc.append(hk[None]); Vc.append(hv[None])
    # the selection, checked by brute force on the raw indexer keys
    allS = np.concatenate([c4_scores(KI[128 * b:128 * b + 128], qi) for b in range(nb)])
    assert list(sel[:min(k, 32 * nb)]) == sorted(sorted(range(32 * nb), key=lambda j: (-allS[j], j))[:min(k, 32 * nb)])
    for j in sel:
        if j >= 0:
            ck, cv = gated_pool(K[4 * j:4 * j + 4], V[4 * j:4 * j + 4], o.W_csa)
            Kc.append(ck[None]); Vc.append(cv[None])
    Kc = np.concatenate(Kc)
    Vc = np.concatenate(Vc)
    assert len(Kc) == w + nb + min(k, 32 * nb)
    ref = sdpa64(q, Kc, Vc)
    assert np.allclose(o.attend(s, q, sel, k), ref, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ sharing, refcounts, ids

def test_share_bit_identical_to_independent_rebuild():
    o = make_oracle(n_win=256, max_states=8, max_blocks=32)
    K, V, KI = toks(19, 0, 900)
    p = o.state_alloc()
    o.append([p], [(K[:384], V[:384], KI[:384])])
    c1, c2 = o.state_alloc(), o.state_alloc()
    o.share(p, c1)
    o.share(p, c2)
    for b in o.table(p):
        assert o.refcount[b] == 3
    o.append([c1, c2], [(K[384:900], V[384:900], KI[384:900]), (K[384:500], V[384:500], KI[384:500])])
    o.state_free(p)
    for b in o.table(c1)[:3]:
        assert o.refcount[b] == 2
    r = o.state_alloc()
    o.append([r], [(K, V, KI)])
    assert o.table(c1)[:3] == o.table(c2)[:3]
    for a, b in zip(o.table(c1), o.table(r)):
        A, B = o.block(a), o.block(b)
        for f in ("csa_k", "csa_v", "hca_k", "hca_v", "idx"):
            assert np.array_equal(getattr(A, f), getattr(B, f))
    for (k1, v1), (k2, v2) in zip(o.states[c1].swa, o.states[r].swa):
        assert np.array_equal(k1, k2) and np.array_equal(v1, v2)


def test_free_returns_blocks_only_at_zero_refcount_and_lowest_id_first():
    o = make_oracle(max_states=4, max_blocks=8)
    K, V, KI = toks(20, 0, 512)
    a = o.state_alloc()
    o.append([a], [(K[:256], V[:256], KI[:256])])          # blocks 0, 1
    b = o.state_alloc()
    o.share(a, b)
    o.append([b], [(K[256:512], V[256:512], KI[256:512])])  # blocks 2, 3
    assert o.table(a) == [0, 1] and o.table(b) == [0, 1, 2, 3]
    o.state_free(a)
    assert sorted(o.free_blocks) == [4, 5, 6, 7]
    o.state_free(b)
    assert sorted(o.free_blocks) == list(range(8))
    c = o.state_alloc()
    assert c == 0
    o.append([c], [(K[:128], V[:128], KI[:128])])
    assert o.table(c) == [0]


def test_deferred_seal_equals_default():
    K, V, KI = toks(21, 0, 256)
    o1, o2 = make_oracle(), make_oracle()
    s1, s2 = o1.state_alloc(), o2.state_alloc()
    o1.append([s1], [(K, V, KI)])
    o2.append([s2], [(K[:128], V[:128], KI[:128])], defer_seal=True)
    assert o2.info(s2)["n_blocks"] == 0 and o2.info(s2)["hca_tail"] == 128
    with pytest.raises(OracleError) as e:
        o2.append([s2], [(K[128:129], V[128:129], KI[128:129])])
    assert e.value.kind == "state"
    o2.compress_flush([s2])
    o2.append([s2], [(K[128:], V[128:], KI[128:])])
    for a, b in zip(o1.table(s1), o2.table(s2)):
        for f in ("csa_k", "csa_v", "hca_k", "hca_v", "idx"):
            assert np.array_equal(getattr(o1.block(a), f), getattr(o2.block(b), f))


def test_errors_leave_state_unchanged():
    o = make_oracle(max_states=2, max_blocks=2)
    K, V, KI = toks(22, 0, 400)
    a, b = o.state_alloc(), o.state_alloc()
    with pytest.raises(OracleError) as e:
        o.state_alloc()
    assert e.value.kind == "oom_states"
    o.append([a], [(K[:200], V[:200], KI[:200])])
    with pytest.raises(OracleError) as e:       # needs 2 more blocks, 1 free
        o.append([a, b], [(K[200:300], V[200:300], KI[200:300]), (K[:128], V[:128], KI[:128])])
    assert e.value.kind == "oom_blocks"
    assert o.info(a)["len"] == 200 and o.info(b)["len"] == 0
    o.append([b], [(K[:5], V[:5], KI[:5])])
    with pytest.raises(OracleError) as e:
        o.share(a, b)
    assert e.value.kind == "state"
    with pytest.raises(OracleError):
        o.append([a, a], [(K[:1], V[:1], KI[:1])] * 2)


# ------------------------------------------------------------------ streamed reference

@pytest.mark.parametrize("n_win,k,kv", [(128, 20, "bf16"), (256, 4096, "bf16"), (128, 20, "fp8"),
                                        (256, 4096, "fp8")])
def test_streamed_reference_matches_token_by_token(n_win, k, kv):
    """decode_reference (one request streamed block by block, used for the large
    workloads) computes what the cache driven token by token computes: same top-k
    rows, same selected scores, and the same attention output up to summation order.
    Also with FP8 KV storage (reading R20), where the window, the pooled tokens and
    the HCA entries are the stored values."""
    from oracle import decode_reference
    from synth.workloads import RequestTokens, make

    src = RequestTokens(2, 5)
    wl = make(2)
    Wc, Wh = synth.gate_weights(wl.seed)
    o = Oracle(n_win, Wc, Wh, 2, 64, kv_format=kv)
    s = o.state_alloc()
    L_cases = [5, 127, 128, 300, 640, 777]
    cases, expect = [], []
    L = 0
    for Lc in L_cases:
        K, V, KI = src(np.arange(L, Lc))
        o.append([s], [(K, V, KI)])
        L = Lc
        q, qi = src.query(Lc - 1)
        idx, val = o.topk(s, qi, k)
        expect.append((idx, val, o.attend(s, q, idx, k)))
        cases.append((Lc, q, qi, k))
    got = decode_reference(src, n_win, Wc, Wh, cases, chunk=2, kv_format=kv)
    if kv == "fp8":   # the storage changes the output: the two formats must differ
        ref = decode_reference(src, n_win, Wc, Wh, cases[-1:], chunk=2)
        assert not np.allclose(ref[0][2], got[-1][2], rtol=1e-6, atol=0)
    for (i0, v0, o0), (i1, v1, o1) in zip(expect, got):
        np.testing.assert_array_equal(i0, i1)
        np.testing.assert_array_equal(v0, v1)
        np.testing.assert_allclose(o0, o1, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ FP8 E4M3 entries (reading R15)

def test_e4m3_decode_follows_the_format():
    """Values fixed by the E4M3 definition (bias 7, 3 mantissa bits, subnormals,
    no infinities, 0x7f / 0xff NaN), computed here with exact fractions."""
    from oracle import e4m3_decode
    c = np.arange(256)
    v = e4m3_decode(c)
    for code in range(256):
        s, e, m = code >> 7, (code >> 3) & 15, code & 7
        if e == 15 and m == 7:
            assert math.isnan(v[code])
            continue
        mag = Fraction(m, 8) * Fraction(1, 2 ** 6) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
        assert v[code] == float(-mag if s else mag), code
    assert v[0x38] == 1.0 and v[0x7E] == 448.0 and v[0x01] == 2.0 ** -9 and v[0x08] == 2.0 ** -6
    assert np.isnan(v).sum() == 2
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)                      # codes 0..126 ascend


def test_e4m3_encode_is_nearest_ties_to_even():
    """Brute force against every finite value: the code's value is the nearest, and
    exact midpoints go to the even code; decode(encode(v)) == v for every finite v."""
    from oracle import e4m3_decode, e4m3_encode
    vals = e4m3_decode(np.arange(0x7F))
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.uniform(0, 448, 4000), rng.uniform(0, 2 ** -5, 2000),
                        (vals[1:] + vals[:-1]) / 2])      # every midpoint
    codes = e4m3_encode(x)
    for xi, c in zip(x, codes):
        d = np.abs(vals - xi)
        best = np.flatnonzero(d == d.min())
        assert c in best
        if len(best) == 2:
            assert c % 2 == 0
    fin = np.arange(256)[~np.isnan(e4m3_decode(np.arange(256)))]
    assert np.array_equal(e4m3_encode(e4m3_decode(fin)), fin.astype(np.uint8))
    assert np.array_equal(e4m3_encode(-x), codes | 0x80)
    assert e4m3_encode([460.0])[0] == 0x7E and e4m3_encode([464.0])[0] == 0x7F


def test_quantize_rows_bounds_and_special_cases():
    """Per-row FP8 storage: the largest magnitude stores as +-448 (code 0x7e); every
    code is within half a code spacing of x / s, s the stored scale, up to the
    float32 rounding of the quotient (at most 2**-24 |x / s|, which is at most
    2**-20 of half a spacing anywhere on the E4M3 grid, hence the 1e-6 margin); an
    all-zero row, or one whose s would not be a normal float32, stays zero with
    scale 1; a row and its negation store with mirrored codes."""
    from oracle import e4m3_decode, quantize_e4m3_rows
    rng = np.random.default_rng(9)
    x = rng.standard_normal((64, 128)) * np.exp(rng.uniform(-8, 8, (64, 1)))
    codes, s, vals = quantize_e4m3_rows(x)
    x32 = x.astype(np.float32).astype(np.float64)
    amax_i = np.abs(x32).argmax(axis=1)
    assert np.all((codes[np.arange(64), amax_i] & 0x7F) == 0x7E)
    np.testing.assert_allclose(s, np.abs(x32).max(axis=1) / 448.0, rtol=2.0 ** -24)
    y = x32 / s[:, None].astype(np.float64)
    grid = e4m3_decode(np.arange(0x7F))
    idx = np.clip(np.searchsorted(grid, np.abs(y)), 1, len(grid) - 1)
    spacing = grid[idx] - grid[idx - 1]
    assert np.all(np.abs(np.abs(e4m3_decode(codes)) - np.abs(y)) <= spacing / 2 * (1 + 1e-6) + 1e-12)
    assert np.allclose(vals, e4m3_decode(codes) * s[:, None])
    zc, zs, zv = quantize_e4m3_rows(np.zeros((2, 128)))
    assert np.all(zc == 0) and np.all(zs == 1.0) and np.all(zv == 0)
    # s = amax / 448 is a normal float32 from amax = 448 * 2**-126 (about 5.27e-36) up;
    # below, the row keeps s = 1 and its codes (x / 1 < 2**-10) are 0
    edge = 448.0 * 2.0 ** -126
    tiny = np.array([np.full(128, 1e-38), np.full(128, edge * 0.99), np.full(128, edge),
                     np.full(128, 2.0e-35)])
    tc, ts, tv = quantize_e4m3_rows(tiny)
    assert np.all(tc[:2] == 0) and np.all(ts[:2] == 1.0) and np.all(tv[:2] == 0)
    assert ts[2] == np.float32(2.0 ** -126) and np.all(tc[2] == 0x7E) and np.all(tv[2] == edge)
    assert np.all(tc[3] == 0x7E) and np.isclose(tv[3], 2.0e-35, rtol=1e-6).all()
    nc, ns, _ = quantize_e4m3_rows(-x)
    assert np.array_equal(ns, s) and np.array_equal(nc, codes ^ 0x80)


def _f32_exact(v: Fraction) -> Fraction:
    """v rounded to the nearest float32 (ties to even; normal and subnormal range),
    in exact rational arithmetic."""
    if v == 0:
        return Fraction(0)
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    ulp = Fraction(2) ** (max(e, -126) - 23)
    q = a / ulp
    n = q.numerator // q.denominator
    r = q - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return (n * ulp) if v > 0 else -(n * ulp)


def _e4m3_exact(y: Fraction) -> int:
    """E4M3 code of y: nearest finite value, ties to the even code, by enumeration."""
    best = None
    for c in range(0x7F):
        e, m = c >> 3, c & 7
        val = Fraction(m, 8 * 2 ** 6) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
        d = abs(abs(y) - val)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1] | (0x80 if y < 0 else 0)


def test_quantize_rows_exact_fractions():
    """The quantiser rule computed in exact rational arithmetic, in its own order of
    operations: s = float32(amax / 448) (1 if not a normal float32), y =
    float32(x / s), code = nearest E4M3 value of y with ties to the even code. Rows:
    random magnitudes; rows with amax = 448 * 2**k (s exact) holding every E4M3
    midpoint, so that the ties are decided by the even-code rule; and rows with an
    inexact s."""
    from oracle import quantize_e4m3_rows
    rng = np.random.default_rng(41)
    grid = np.array([float(Fraction(m, 8 * 2 ** 6) if (c >> 3) == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** ((c >> 3) - 7))
                     for c in range(0x7F) for m in [c & 7]])
    mids = (grid[1:] + grid[:-1]) / 2
    rows = [rng.standard_normal(128) * np.exp(rng.uniform(-6, 6)) for _ in range(10)]
    for k in (0, -3, 5):
        r = np.resize(np.concatenate([mids, -mids]), 128) * 2.0 ** k
        r[0] = 448.0 * 2.0 ** k
        rows.append(r)
    for amax in (1.0, 3.0, 0.1):
        r = rng.uniform(-amax, amax, 128)
        r[7] = -amax
        rows.append(r)
    x = np.array(rows).astype(np.float32)
    codes, s, _ = quantize_e4m3_rows(x)
    for i, row in enumerate(x):
        xf = [Fraction(float(v)) for v in row]
        amax = max(abs(v) for v in xf)
        se = _f32_exact(amax / 448)
        if se < Fraction(2) ** -126:
            se = Fraction(1)
        assert Fraction(float(s[i])) == se, i
        for d in range(128):
            assert codes[i, d] == _e4m3_exact(_f32_exact(xf[d] / se)), (i, d)
    # the midpoint rows hit ties: the even code wins there
    assert np.all(codes[10:13, 1:126] % 2 == 0)


# ------------------------------------------------------------------ FP8 SWA ring and HCA entries (R20)

def fp8_grid_tokens(rng, n):
    """Tokens every head of which already sits on its own E4M3 grid: values are E4M3
    values times 2**e (one e per token, head and K/V) and each head holds +-448 * 2**e,
    so the per-head quantiser stores them exactly (s = 2**e, x / s = a code value).
    E4M3 values have at most 4 significant bits, so the tokens are bf16 values too."""
    from oracle import e4m3_decode
    codes = rng.integers(0, 0x7F, (2, n, N_HEADS, HEAD_DIM))
    vals = e4m3_decode(codes) * np.where(rng.random(codes.shape) < 0.5, -1.0, 1.0)
    vals[..., 0] = 448.0 * np.where(rng.random(vals.shape[:-1]) < 0.5, -1.0, 1.0)
    e = rng.integers(-12, -6, (2, n, N_HEADS, 1)).astype(np.float64)
    vals = vals * np.exp2(e)
    assert np.array_equal(bf16_round(vals), vals)
    return vals[0], vals[1]


def test_fp8_kv_is_exact_on_fp8_grid_tokens():
    """On tokens that the FP8 storage holds exactly, the FP8-KV oracle's window, C4
    entries, top-k rows and attention equal the bf16 oracle's; its HCA entries are
    the per-head E4M3 storage of the unrounded pooled entry of those tokens."""
    from oracle import quantize_e4m3_rows
    rng = np.random.default_rng(20)
    Wc, Wh = synth.gate_weights(SEED)
    K, V = fp8_grid_tokens(rng, 300)
    KI = rng.standard_normal((300, 4, 64))
    a = Oracle(128, Wc, Wh, 1, 4)
    b = Oracle(128, Wc, Wh, 1, 4, kv_format="fp8")
    for o in (a, b):
        assert o.state_alloc() == 0
        o.append([0], [(K[:257], V[:257], KI[:257])])
    for (ka, va), (kb, vb) in zip(a.states[0].swa, b.states[0].swa):
        assert np.array_equal(ka, kb) and np.array_equal(va, vb)
    for lb in range(2):
        ba, bb = a.block(a.table(0)[lb]), b.block(b.table(0)[lb])
        assert np.array_equal(ba.csa_k, bb.csa_k) and np.array_equal(ba.csa_v, bb.csa_v)
        Kh, Vh = gated_pool(K[128 * lb:128 * (lb + 1)], V[128 * lb:128 * (lb + 1)], Wh, rounded=False)
        codes, sc, vals = quantize_e4m3_rows(Kh)
        assert np.array_equal(bb.hca_k_codes, codes) and np.array_equal(bb.hca_k_scale, sc)
        assert np.array_equal(bb.hca_k, vals)
        assert np.array_equal(bb.hca_v, quantize_e4m3_rows(Vh)[2])
    q = rng.standard_normal((N_HEADS, HEAD_DIM))
    qi = rng.standard_normal((4, 64))
    ia, _ = a.topk(0, qi, 20)
    ib, _ = b.topk(0, qi, 20)
    assert np.array_equal(ia, ib)
    Ka, Va = a.keys(0, ia, 20)
    Kb, Vb = b.keys(0, ib, 20)
    n_hca = 2
    keep = np.r_[0:128, 128 + n_hca:len(Ka)]           # every key but the HCA entries
    assert np.array_equal(Ka[keep], Kb[keep]) and np.array_equal(Va[keep], Vb[keep])


def test_fp8_kv_stores_each_token_through_the_quantiser():
    """With FP8 KV every path that writes the window stores a token's per-head E4M3
    codes and scales: append, replay (state_write), fork (share) and restore. The
    stored values stay within half a code spacing (times s) of the raw ones, and a
    block pools the stored values of its 128 tokens."""
    from oracle import e4m3_decode, quantize_e4m3_rows
    Wc, Wh = synth.gate_weights(SEED)
    o = Oracle(128, Wc, Wh, 4, 8, kv_format="fp8")
    grid = e4m3_decode(np.arange(0x7F))
    K, V, KI = toks(3, 0, 260)
    s0 = o.state_alloc()
    o.append([s0], [(K, V, KI)])

    def check_window(s):
        st = o.states[s]
        L = st.L
        for i, ((k, v), q) in enumerate(zip(st.swa, st.swa_q)):
            p = L - len(st.swa) + i
            for raw, got, (codes, sc) in ((K[p], k, q[0:2]), (V[p], v, q[2:4])):
                rc, rs, rv = quantize_e4m3_rows(raw)
                assert np.array_equal(codes, rc) and np.array_equal(sc, rs) and np.array_equal(got, rv)
                assert np.array_equal(got, e4m3_decode(codes) * sc[:, None].astype(np.float64))
                y = np.abs(raw) / sc[:, None].astype(np.float64)
                idx = np.clip(np.searchsorted(grid, y), 1, len(grid) - 1)
                half = (grid[idx] - grid[idx - 1]) / 2 * sc[:, None].astype(np.float64)
                assert np.all(np.abs(got - raw) <= half * (1 + 1e-6))
    check_window(s0)
    # the seal pooled the stored tokens
    blk = o.block(o.table(s0)[1])
    Kq = quantize_e4m3_rows(K[128:256])[2]
    Vq = quantize_e4m3_rows(V[128:256])[2]
    for j in (0, 17, 31):
        ek, ev = gated_pool(Kq[4 * j:4 * j + 4], Vq[4 * j:4 * j + 4], Wc)
        assert np.array_equal(blk.csa_k[j], ek) and np.array_equal(blk.csa_v[j], ev)
    # fork, attach + replay, and restore store the same codes
    s1 = o.state_alloc()
    o.share(s0, s1)
    check_window(s1)
    s2 = o.state_alloc()
    o.prefix_attach(s2, o.table(s0), 260)
    o.state_write([s2], [(K[132:260], V[132:260], KI[132:260])], [132])
    check_window(s2)
    ck = o.checkpoint(s0)
    s3 = o.state_alloc()
    o.prefix_attach(s3, o.table(s0), 260)
    o.restore(s3, ck)
    check_window(s3)


def test_fp8_kv_attention_without_blocks_is_sdpa_over_the_stored_window():
    """Below one block there are no entries: attention is plain softmax attention over
    the window's stored (dequantized) K/V, checked against the library routine."""
    Wc, Wh = synth.gate_weights(SEED)
    o = Oracle(128, Wc, Wh, 1, 2, kv_format="fp8")
    K, V, KI = toks(5, 0, 100)
    o.append([o.state_alloc()], [(K, V, KI)])
    st = o.states[0]
    Ks = torch.tensor(np.stack([t[0] for t in st.swa]), dtype=torch.float64)   # [n][H][D]
    Vs = torch.tensor(np.stack([t[1] for t in st.swa]), dtype=torch.float64)
    q = synth.bf16_bits_to_f32(synth.tokens_bf16(SEED, synth.STREAM_Q, 5, np.array([99])))[0].astype(np.float64)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q)[:, None, :], Ks.permute(1, 0, 2), Vs.permute(1, 0, 2))[:, 0, :].numpy()
    np.testing.assert_allclose(o.attend(0, q, [], 0), ref, rtol=1e-12, atol=1e-12)
    # and it stays close to the bf16 oracle's (FP8 storage error only)
    b = Oracle(128, Wc, Wh, 1, 2)
    b.append([b.state_alloc()], [(K, V, KI)])
    r = b.attend(0, q, [], 0)
    assert np.linalg.norm(o.attend(0, q, [], 0) - r) / np.linalg.norm(r) < 0.05


def test_fp8_kv_refuses_eager_c4():
    Wc, Wh = synth.gate_weights(SEED)
    with pytest.raises(OracleError):
        Oracle(128, Wc, Wh, 1, 1, c4_mode="eager", kv_format="fp8")
    with pytest.raises(OracleError):
        Oracle(128, Wc, Wh, 1, 1, kv_format="fp4")


def test_fp8_oracle_entries_quantize_the_pooled_entry():
    """With FP8 entries the oracle's C4 entries are the per-head E4M3 storage of the
    unrounded pooled entry (the bf16 oracle's entries come from the same pooling),
    HCA entries and indexer keys are unchanged, and attention reads the stored
    values."""
    from oracle import quantize_e4m3_rows
    Wc, Wh = synth.gate_weights(SEED)
    a = Oracle(128, Wc, Wh, 2, 4)
    b = Oracle(128, Wc, Wh, 2, 4, entry_format="fp8")
    K, V, KI = toks(0, 0, 200)
    for o in (a, b):
        assert o.state_alloc() == 0
        o.append([0], [(K, V, KI)])
    ba, bb = a.block(0), b.block(0)
    assert np.array_equal(ba.hca_k, bb.hca_k) and np.array_equal(ba.idx, bb.idx)
    for j in (0, 13, 31):
        kj, vj = gated_pool(K[4 * j:4 * j + 4], V[4 * j:4 * j + 4], Wc, rounded=False)
        assert np.allclose(bf16_round(kj), ba.csa_k[j])
        codes, sc, vals = quantize_e4m3_rows(kj)
        assert np.array_equal(codes, bb.csa_k_codes[j]) and np.array_equal(sc, bb.csa_k_scale[j])
        assert np.array_equal(vals, bb.csa_k[j])
        rel = np.linalg.norm(bb.csa_v[j] - vj) / np.linalg.norm(vj)
        assert rel < 0.05
    q = synth.bf16_bits_to_f32(synth.tokens_bf16(SEED, synth.STREAM_Q, 0, np.array([199])))[0]
    sel = np.array([3, 9, 30])
    Kc = np.concatenate([np.stack([t[0] for t in b.states[0].swa]), bb.hca_k[None], bb.csa_k[sel]])
    Vc = np.concatenate([np.stack([t[1] for t in b.states[0].swa]), bb.hca_v[None], bb.csa_v[sel]])
    assert np.allclose(b.attend(0, q, sel, 3), attention(q, Kc, Vc), atol=1e-12)


# ---------------------------------------------------------------- MXFP4 indexer keys (R16)

def test_e2m1_decode_is_the_format_table():
    """The 16 E2M1 codes against the element table of the OCP Microscaling spec:
    magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 for codes 0..7, the same negated for 8..15."""
    from oracle import e2m1_decode
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert np.array_equal(e2m1_decode(np.arange(8)), table)
    assert np.array_equal(e2m1_decode(np.arange(8, 16)), [-t for t in table])


def test_e2m1_encode_is_nearest_ties_to_even_saturating():
    """Brute force over the 8 magnitudes for random values and every midpoint: the
    code is a nearest one, the even one on a tie; beyond 6 it saturates; the sign
    bit follows y < 0."""
    from oracle import e2m1_decode, e2m1_encode
    vals = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    rng = np.random.default_rng(3)
    y = np.concatenate([rng.uniform(0, 7, 3000), (vals[1:] + vals[:-1]) / 2, vals])
    c = e2m1_encode(y)
    for yi, ci in zip(y, c):
        d = np.abs(vals - min(yi, 6.0))
        best = np.flatnonzero(d == d.min())
        assert ci in best
        if len(best) == 2:
            assert ci % 2 == 0
    assert list(e2m1_encode([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])) == [0, 2, 2, 4, 4, 6, 6]
    assert list(e2m1_encode([6.0, 7.9, 100.0])) == [7, 7, 7]
    nz = y > 0
    assert np.array_equal(e2m1_encode(-y[nz]), c[nz] | 8) and e2m1_encode([-0.0])[0] == 0
    assert e2m1_encode([-0.1])[0] == 8 and e2m1_decode([8])[0] == 0.0


def test_mxfp4_hand_worked_row():
    """A row worked by hand. Block 0 = [1, 2, -0.3, 0...]: max 2, E = 1 - 2 = -1, so
    x / 2**E = [2, 4, -0.6]: codes 4 (2.0), 6 (4.0), 9 (-0.5); bytes 0x64, 0x09.
    Block 1 all zero: E = -127 (byte 0), codes 0. Block 2 = [6 * 2**-5, 5 * 2**-5]:
    max 0.1875 = 1.5 * 2**-3, E = -5: 6 -> code 7, 5 is the 4/6 midpoint -> code 6
    (4.0, even); byte 0x67, value 4 * 2**-5 = 0.125."""
    from oracle import quantize_mxfp4_rows
    x = np.zeros(256, np.float32)
    x[0:3] = [1.0, 2.0, -0.3]
    x[64:66] = [6 * 2.0 ** -5, 5 * 2.0 ** -5]
    codes, scales, vals = quantize_mxfp4_rows(x)
    assert codes[0] == 0x64 and codes[1] == 0x09 and np.all(codes[2:16] == 0)
    assert codes[32] == 0x67
    assert scales[0] == 127 - 1 and scales[1] == 0 and scales[2] == 127 - 5
    assert list(vals[:3]) == [1.0, 2.0, -0.25] and vals[64] == 0.1875 and vals[65] == 0.125


def test_mxfp4_bounds_round_trip_and_scale():
    """Each value within half an E2M1 spacing (times 2**E) of the key, block maxima
    landing on code 6 or 7 (x / 2**E in [4, 8)), exact round trip of values already
    on the grid, mirrored codes under negation, and 2**E as the E8M0 byte."""
    from oracle import e2m1_decode, quantize_mxfp4_rows
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((40, 256)) * np.exp(rng.uniform(-10, 10, (40, 8))).repeat(32, axis=1)).astype(np.float32)
    codes, scales, vals = quantize_mxfp4_rows(x)
    E = scales.astype(np.int64) - 127
    step = np.ldexp(1.0, E).repeat(32, axis=1)               # 2**E per value
    c = np.stack([codes & 15, codes >> 4], axis=-1).reshape(40, 256)
    assert np.array_equal(vals, e2m1_decode(c) * step)
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    y = np.abs(x.astype(np.float64)) / step
    idx = np.clip(np.searchsorted(grid, np.minimum(y, 6.0)), 1, 7)
    half = (grid[idx] - grid[idx - 1]) / 2
    assert np.all(np.abs(np.abs(vals) / step - np.minimum(y, 6.0)) <= half + 1e-12)
    blk = np.abs(x.astype(np.float64)).reshape(40, 8, 32)
    amax = blk.max(axis=-1)
    assert np.all((amax / np.ldexp(1.0, E) >= 4) & (amax / np.ldexp(1.0, E) < 8))
    cm = (c.reshape(40, 8, 32)[np.arange(40)[:, None], np.arange(8)[None], blk.argmax(-1)]) & 7
    assert np.all((cm == 6) | (cm == 7))
    c2, s2, v2 = quantize_mxfp4_rows(vals)
    assert np.array_equal(v2, vals)
    cn, sn, _ = quantize_mxfp4_rows(-x)
    assert np.array_equal(sn, scales)
    nz = (np.stack([codes & 15, codes >> 4], -1).reshape(40, 256) != 0) | (x != 0)
    assert np.all(((np.stack([cn & 15, cn >> 4], -1).reshape(40, 256) ^ c) == 8)[nz])


def test_mxfp4_scores_are_exact_in_float32():
    """The property the bit-exact top-k parity rests on: with the dyadic synthetic
    keys and queries (odd multiples of 2**-8 below 3), every partial sum of a C4
    score over MXFP4 keys is a multiple of 2**(E_min - 9) far below 2**24 such
    units, so float32 sums in any order equal the float64 score. Checked by summing
    in float32 in two orders against c4_scores in float64."""
    from oracle import quantize_mxfp4_rows
    KI = synth.tokens_f32(SEED, synth.STREAM_IDXK, 7, np.arange(1024)).reshape(1024, -1).astype(np.float64)
    qi = synth.tokens_f32(SEED, synth.STREAM_QI, 7, np.array([1024])).reshape(-1).astype(np.float64)
    codes, scales, vals = quantize_mxfp4_rows(KI)
    ref = c4_scores(vals.reshape(1024, 4, 64)[:128], qi.reshape(4, 64))
    prod = (vals[:128] * qi[None, :]).reshape(32, 4 * 256)
    E_min = int(scales.min()) - 127
    assert np.abs(prod).sum(axis=1).max() < 2.0 ** (24 + E_min - 9)
    fwd = np.zeros(32, np.float32)
    for i in range(prod.shape[1]):
        fwd = (fwd + prod[:, i].astype(np.float32)).astype(np.float32)
    rev = np.zeros(32, np.float32)
    for i in reversed(range(prod.shape[1])):
        rev = (rev + prod[:, i].astype(np.float32)).astype(np.float32)
    assert np.array_equal(fwd.astype(np.float64) / 4, ref) and np.array_equal(rev, fwd)


def test_mxfp4_oracle_blocks_store_quantized_keys():
    """With MXFP4 indexer keys the sealed block holds the MXFP4 storage of the raw
    keys, C4/HCA entries are unchanged, and the scores read the stored values."""
    from oracle import quantize_mxfp4_rows
    Wc, Wh = synth.gate_weights(SEED)
    a = Oracle(128, Wc, Wh, 2, 4)
    b = Oracle(128, Wc, Wh, 2, 4, index_format="mxfp4")
    K, V, KI = toks(0, 0, 300)
    for o in (a, b):
        assert o.state_alloc() == 0
        o.append([0], [(K, V, KI)])
    for blk in range(2):
        ba, bb = a.block(blk), b.block(blk)
        assert np.array_equal(ba.csa_k, bb.csa_k) and np.array_equal(ba.hca_v, bb.hca_v)
        codes, scales, vals = quantize_mxfp4_rows(KI[128 * blk:128 * blk + 128].reshape(128, -1))
        assert np.array_equal(bb.idx_codes, codes) and np.array_equal(bb.idx_scales, scales)
        assert np.array_equal(bb.idx.reshape(128, -1), vals)
    qi = synth.tokens_f32(SEED, synth.STREAM_QI, 0, np.array([299]))[0].astype(np.float64)
    want = np.concatenate([c4_scores(b.block(i).idx, qi) for i in range(2)])
    assert np.array_equal(b.scores(0, qi), want)
    assert not np.array_equal(a.scores(0, qi), want)


# ---------------------------------------------------------------- prefix hits (R17)

def _same_state(o, a, b):
    sa, sb = o.states[a], o.states[b]
    assert sa.L == sb.L and sa.blocks == sb.blocks
    assert len(sa.swa) == len(sb.swa) and len(sa.tail) == len(sb.tail)
    for x, y in zip(sa.swa, sb.swa):
        assert np.array_equal(x[0], y[0]) and np.array_equal(x[1], y[1])
    for x, y in zip(sa.tail, sb.tail):
        assert all(np.array_equal(u, w) for u, w in zip(x, y))


@pytest.mark.parametrize("n_win,P,c", [(128, 1000, 512), (128, 1000, 900), (256, 640, 0), (256, 200, 128),
                                       (128, 384, 256), (512, 1500, 1024)])
def test_prefix_policies_equal_the_fork(n_win, P, c):
    """Zero (attach + replay of the window), Periodic (attach + checkpoint at c +
    replay of [c, P)) and Full (attach + checkpoint at P) each give the State that
    forking the live prefix request gives, with the blocks shared, not sealed again;
    the next decode step's top-k and attention agree exactly."""
    o = make_oracle(n_win=n_win, max_states=8, max_blocks=64)
    K, V, KI = toks(3, 0, P + 1)
    src = o.state_alloc()
    o.append([src], [(K[:c], V[:c], KI[:c])])
    ck_c = o.checkpoint(src)
    o.append([src], [(K[c:P], V[c:P], KI[c:P])])
    ck_p = o.checkpoint(src)
    fork = o.state_alloc()
    o.share(src, fork)
    blocks = o.table(src)
    o.block_ref(blocks, +1)                      # the prefix entry holds the blocks
    o.state_free(src)
    free_before = len(o.free_blocks)
    zero, per, full = o.state_alloc(), o.state_alloc(), o.state_alloc()
    for d in (zero, per, full):
        o.prefix_attach(d, blocks, P)
    w0 = max(0, P - n_win)
    o.state_write([zero], [(K[w0:P], V[w0:P], KI[w0:P])], [w0])
    o.restore(per, ck_c)
    o.state_write([per], [(K[c:P], V[c:P], KI[c:P])], [c])
    o.restore(full, ck_p)
    assert len(o.free_blocks) == free_before     # nothing sealed again
    for d in (zero, per, full):
        _same_state(o, fork, d)
        assert all(o.refcount[b] == 5 for b in blocks)   # fork, entry and three hits
    qi = synth.tokens_f32(SEED, synth.STREAM_QI, 3, np.array([P]))[0].astype(np.float64)
    q = synth.bf16_bits_to_f32(synth.tokens_bf16(SEED, synth.STREAM_Q, 3, np.array([P])))[0]
    for d in (zero, per, full):
        o.append([d], [(K[P:P + 1], V[P:P + 1], KI[P:P + 1])])
    o.append([fork], [(K[P:P + 1], V[P:P + 1], KI[P:P + 1])])
    kk = 64
    ref_idx, ref_val = o.topk(fork, qi, kk)
    ref_out = o.attend(fork, q, ref_idx, kk)
    for d in (zero, per, full):
        idx, val = o.topk(d, qi, kk)
        assert np.array_equal(idx, ref_idx) and np.array_equal(val, ref_val)
        assert np.array_equal(o.attend(d, q, idx, kk), ref_out)


def test_prefix_attach_errors_and_unfilled_state():
    """An attached state cannot be read, appended to or forked before its window is
    filled; a partial replay leaves it unfilled; bad arguments change nothing; a
    released prefix entry frees its blocks at refcount 0."""
    o = make_oracle(n_win=128, max_states=4, max_blocks=16)
    K, V, KI = toks(4, 0, 300)
    src = o.state_alloc()
    o.append([src], [(K, V, KI)])
    blocks = o.table(src)
    d = o.state_alloc()
    with pytest.raises(OracleError):
        o.prefix_attach(d, blocks[:1], 300)      # needs 2 blocks
    with pytest.raises(OracleError):
        o.prefix_attach(src, blocks, 300)        # not fresh
    assert o.states[d].L == 0 and all(o.refcount[b] == 1 for b in blocks)
    o.prefix_attach(d, blocks, 300)
    q = np.zeros((N_HEADS, HEAD_DIM))
    with pytest.raises(OracleError):
        o.attend(d, q, [], 1)
    o.state_write([d], [(K[200:300], V[200:300], KI[200:300])], [200])   # window is [172, 300)
    with pytest.raises(OracleError):
        o.append([d], [(K[:1], V[:1], KI[:1])])
    with pytest.raises(OracleError):
        o.state_write([d], [(K[250:300], V[250:300], KI[250:300])], [251])   # past L
    o.state_write([d], [(K[100:200], V[100:200], KI[100:200])], [100])     # 100..171 dropped
    assert all(x is not None for x in o.states[d].swa)
    e = o.state_alloc()
    o.share(src, e)
    _same_state(o, e, d)
    with pytest.raises(OracleError):
        o.block_ref(blocks + blocks + blocks + blocks, -1)   # more than held (3 each)
    o.block_ref(blocks, +1)
    for s_ in (src, d, e):
        o.state_free(s_)
    assert all(o.refcount[b] == 1 for b in blocks) and len(o.free_blocks) == 14
    o.block_ref(blocks, -1)
    assert len(o.free_blocks) == 16 and all(b not in o.store for b in blocks)


# ---------------------------------------------------------------- layer types (R18)

def test_layer_types_attend_their_parts_of_the_block():
    """One call sequence into a mixed, an SWA, a CSA and an HCA layer (same gates,
    same tokens): block ids match across types; the CSA layer's C4 entries and keys
    and the HCA layer's HCA entries equal the mixed layer's; the SWA layer's output
    is plain attention over the window; the CSA and HCA outputs equal brute force
    over SWA + the selected C4 / SWA + every HCA; layers without C4 select nothing."""
    Wc, Wh = synth.gate_weights(SEED)
    orc = {t: Oracle(128, Wc, Wh, 4, 16, layer_type=t) for t in ("mixed", "swa", "csa", "hca")}
    K, V, KI = toks(6, 0, 700)
    for o in orc.values():
        assert o.state_alloc() == 0
        o.append([0], [(K[:650], V[:650], KI[:650])])
        o.append([0], [(K[650:], V[650:], KI[650:])])
    tables = {t: o.table(0) for t, o in orc.items()}
    assert all(tb == tables["mixed"] for tb in tables.values()) and len(tables["mixed"]) == 5
    m, c, h = orc["mixed"], orc["csa"], orc["hca"]
    for b in tables["mixed"]:
        assert np.array_equal(m.block(b).csa_k, c.block(b).csa_k) and np.array_equal(m.block(b).idx, c.block(b).idx)
        assert np.array_equal(m.block(b).hca_v, h.block(b).hca_v)
        assert c.block(b).hca_k is None and h.block(b).csa_k is None and orc["swa"].block(b).csa_k is None
    q = synth.bf16_bits_to_f32(synth.tokens_bf16(SEED, synth.STREAM_Q, 6, np.array([699])))[0].astype(np.float64)
    qi = synth.tokens_f32(SEED, synth.STREAM_QI, 6, np.array([699]))[0].astype(np.float64)
    kk = 40
    sel, _ = m.topk(0, qi, kk)
    assert np.array_equal(c.topk(0, qi, kk)[0], sel)
    for t in ("swa", "hca"):
        assert np.all(orc[t].topk(0, qi, kk)[0] == -1)
    Kw, Vw = K[700 - 128:], V[700 - 128:]
    assert np.allclose(orc["swa"].attend(0, q, [], kk), attention(q, Kw, Vw), atol=1e-13)
    blocks = [m.block(b) for b in tables["mixed"]]
    Kc = np.stack([blocks[j // 32].csa_k[j % 32] for j in sel])
    Vc = np.stack([blocks[j // 32].csa_v[j % 32] for j in sel])
    assert np.allclose(c.attend(0, q, sel, kk), attention(q, np.concatenate([Kw, Kc]), np.concatenate([Vw, Vc])),
                       atol=1e-13)
    Kh = np.stack([x.hca_k for x in blocks])
    Vh = np.stack([x.hca_v for x in blocks])
    assert np.allclose(h.attend(0, q, sel, kk), attention(q, np.concatenate([Kw, Kh]), np.concatenate([Vw, Vh])),
                       atol=1e-13)
    assert np.allclose(m.attend(0, q, sel, kk),
                       attention(q, np.concatenate([Kw, Kh, Kc]), np.concatenate([Vw, Vh, Vc])), atol=1e-13)


# ---------------------------------------------------------------- eager C4 (R19)

def test_eager_c4_entries_match_the_sealed_ones():
    """Eager mode: the open block's candidates are its complete groups (g = (L mod
    128) // 4) after the sealed ones; each open entry and its score equal the entry
    and score the same group has once its block seals; blocks are the sealed mode's;
    with k covering every candidate, attention is brute force over SWA + HCA + all
    sealed C4 + the open entries."""
    Wc, Wh = synth.gate_weights(SEED)
    e = Oracle(128, Wc, Wh, 2, 8, c4_mode="eager")
    d = Oracle(128, Wc, Wh, 2, 8)
    K, V, KI = toks(9, 0, 400)
    qi = synth.tokens_f32(SEED, synth.STREAM_QI, 9, np.array([0]))[0].astype(np.float64)
    q = synth.bf16_bits_to_f32(synth.tokens_bf16(SEED, synth.STREAM_Q, 9, np.array([0])))[0].astype(np.float64)
    for o in (e, d):
        assert o.state_alloc() == 0
        o.append([0], [(K[:290], V[:290], KI[:290])])     # 2 blocks + 34 tail tokens
    se, sd = e.scores(0, qi), d.scores(0, qi)
    assert len(sd) == 64 and len(se) == 64 + 8 and np.array_equal(se[:64], sd)
    st = e.states[0]
    open_entries = [e._open_entry(st, i) for i in range(8)]
    for o in (e, d):
        o.append([0], [(K[290:384], V[290:384], KI[290:384])])   # the block seals at 384
    assert len(e.scores(0, qi)) == 96 and len(e.states[0].tail) == 0
    blk = e.block(e.table(0)[2])
    for i, (ke, ve) in enumerate(open_entries):
        assert np.array_equal(ke, blk.csa_k[i]) and np.array_equal(ve, blk.csa_v[i])
    assert np.array_equal(e.scores(0, qi)[64:72], se[64:72])
    assert np.array_equal(e.scores(0, qi), d.scores(0, qi))
    e.append([0], [(K[384:391], V[384:391], KI[384:391])])      # 7 tokens: one open group
    sel, _ = e.topk(0, qi, 200)
    assert (sel >= 0).sum() == 97 and sel[96] == 96
    st = e.states[0]
    Kc = [e.block(b).csa_k[j] for b in e.table(0) for j in range(32)] + [e._open_entry(st, 0)[0]]
    Vc = [e.block(b).csa_v[j] for b in e.table(0) for j in range(32)] + [e._open_entry(st, 0)[1]]
    Kh = [e.block(b).hca_k for b in e.table(0)]
    Vh = [e.block(b).hca_v for b in e.table(0)]
    Kw, Vw = K[391 - 128:391], V[391 - 128:391]
    ref = attention(q, np.concatenate([Kw, np.stack(Kh), np.stack(Kc)]),
                    np.concatenate([Vw, np.stack(Vh), np.stack(Vc)]))
    assert np.allclose(e.attend(0, q, sel, 200), ref, atol=1e-13)
    with pytest.raises(OracleError):
        Oracle(128, Wc, Wh, 1, 1, c4_mode="eager", entry_format="fp8")
