"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, element by
element, at sizes the oracle finishes in seconds that still span several blocks,
several attention chunks and a ragged tail.

Bars: integer state (lengths, block tables, refcounts, top-k ordinals) bit exact;
the indexer scores are bit exact too, because every input is an odd multiple of
2**-8 and every partial sum is an exact float32 (the top-k acceptance band is
checked as well); bf16 entries and fp32 attention outputs within relative L2
1e-3 of the fp64 oracle.
"""

import numpy as np
import pytest

import synth
from oracle import Oracle
from synth import workloads
from tests.gpu_util import (bf16_to_f64, dev_queries, dev_tokens, host_queries, host_tokens,
                            rel_l2, topk_accept)

pytestmark = pytest.mark.gpu

TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import heterogeneous_sparse_attention_amd as hsa
    hsa.load()          # raises if the library is missing: no fallback


def new_pair(n_win, max_states, max_blocks, seed, **kw):
    from heterogeneous_sparse_attention_amd import Cache
    Wc, Wh = synth.gate_weights(seed)
    return (Cache(n_win, max_states, max_blocks, Wc, Wh, **kw),
            Oracle(n_win, Wc, Wh, max_states, max_blocks))


def check_block(cache, o, b_gpu, b_orc, exact_idx=True):
    g = cache.export_block(b_gpu)
    r = o.block(b_orc)
    for name, ref in (("csa_k", r.csa_k), ("csa_v", r.csa_v), ("hca_k", r.hca_k), ("hca_v", r.hca_v)):
        val = bf16_to_f64(g[name])
        assert rel_l2(val, ref) <= TOL, (name, rel_l2(val, ref))
        assert np.mean(val == ref) > 0.97, name    # bf16 rounding of fp32 vs fp64 rarely differs
    if exact_idx:
        assert np.array_equal(g["idx"], r.idx)


def check_state(cache, o, s_gpu, s_orc):
    info = cache.state_query(s_gpu)
    oi = o.info(s_orc)
    assert info["len"] == oi["len"] and info["n_blocks"] == oi["n_blocks"]
    assert info["hca_tail"] == oi["hca_tail"] and info["csa_tail"] == oi["csa_tail"]
    assert info["swa_len"] == oi["swa_len"]
    ex = cache.export_state(s_gpu)
    L, W = oi["len"], cache.n_win
    for i, (k, v) in enumerate(o.states[s_orc].swa):
        p = L - len(o.states[s_orc].swa) + i
        assert np.array_equal(bf16_to_f64(ex["swa_k"][p % W]), k)
        assert np.array_equal(bf16_to_f64(ex["swa_v"][p % W]), v)
    for i, (_, _, ki) in enumerate(o.states[s_orc].tail):
        p = L - len(o.states[s_orc].tail) + i
        assert np.array_equal(ex["idx_tail"][p % 128], ki)


def test_synth_device_matches_host():
    import torch
    from tests.gpu_util import dev_rows
    keys = np.array([0, 3, 0x800005, 7, 31], np.int64)
    pos = np.array([0, 1, 12345, (1 << 20) + 7, 65535], np.int64)
    for stream in (1, 2, 4):
        d = dev_rows(77, stream, keys, pos, True).view(torch.int16).cpu().numpy().view(np.uint16)
        h = synth.tokens_bf16(77, stream, keys.astype(np.uint64), pos)
        assert np.array_equal(d, h)
    for stream in (3, 5):
        d = dev_rows(77, stream, keys, pos, False).cpu().numpy()
        h = synth.tokens_f32(77, stream, keys.astype(np.uint64), pos)
        assert np.array_equal(d, h)


def test_l130_example_then_decode_to_256():
    """The pages' L = 130 example (one sealed block of 32 C4 + 1 HCA, a 2-token tail),
    then 126 decode steps to L = 256, checked after every step."""
    import torch
    wl = workloads.make(1)
    seed = wl.seed
    cache, o = new_pair(wl.n_win, 2, 4, seed)
    s = cache.state_alloc()
    assert s == o.state_alloc() == 0
    pos = np.arange(130)
    K, V, KI = dev_tokens(seed, 0, pos)
    cache.append_kv([s], [0, 130], K, V, KI)
    o.append([s], [host_tokens(seed, 0, pos)])
    info = cache.state_query(s)
    assert (info["len"], info["n_blocks"], info["hca_tail"], info["csa_tail"]) == (130, 1, 2, 2)
    assert cache.block_table(s) == o.table(s) == [0]
    check_block(cache, o, 0, 0)
    check_state(cache, o, s, s)
    k = wl.topk
    for p in range(130, 256):
        Kn, Vn, KIn = dev_tokens(seed, 0, [p])
        Q, QI = dev_queries(seed, 0, [p])
        sc = torch.empty((1, k), dtype=torch.float32, device="cuda")
        srt = p % 2 == 1          # odd steps ask for score-ordered rows
        idx, _, out = cache.decode_step([s], Kn, Vn, KIn, Q, QI, k, score_out=sc, sorted=srt)
        o.append([s], [host_tokens(seed, 0, [p])])
        q, qi = host_queries(seed, 0, [p])
        ridx, rval = o.topk(s, qi[0], k, sorted=srt)
        gidx = idx.cpu().numpy()[0]
        assert np.array_equal(gidx, ridx), p
        g = sc.cpu().numpy()[0]
        assert np.array_equal(g[ridx >= 0], rval[ridx >= 0])
        ref = o.attend(s, q[0], ridx, k)
        assert rel_l2(out.cpu().numpy()[0], ref) <= TOL, p
    assert cache.state_query(s)["n_blocks"] == 2 and cache.block_table(s) == [0, 1]
    check_block(cache, o, 1, 1)
    check_state(cache, o, s, s)


def test_bulk_equals_token_by_token_bit_exact():
    """Appending in one call, in ragged pieces, or one token per call gives
    bit-identical blocks and State (the seal has one arithmetic)."""
    import heterogeneous_sparse_attention_amd as hsa
    Wc, Wh = synth.gate_weights(5)
    caches = [hsa.Cache(128, 1, 4, Wc, Wh) for _ in range(3)]
    L = 300
    K, V, KI = dev_tokens(5, 9, np.arange(L))
    s = [c.state_alloc() for c in caches]
    caches[0].append_kv([s[0]], [0, L], K, V, KI)
    a = 0
    for n in (1, 7, 100, 120, 72):
        caches[1].append_kv([s[1]], [0, n], K[a:a + n], V[a:a + n], KI[a:a + n])
        a += n
    for p in range(L):
        caches[2].append_kv([s[2]], [0, 1], K[p:p + 1], V[p:p + 1], KI[p:p + 1])
    ref_b = [caches[0].export_block(b) for b in caches[0].block_table(s[0])]
    ref_s = caches[0].export_state(s[0])
    for c, st in zip(caches[1:], s[1:]):
        assert c.block_table(st) == caches[0].block_table(s[0])
        for b, rb in zip(c.block_table(st), ref_b):
            eb = c.export_block(b)
            for f in rb:
                assert np.array_equal(eb[f], rb[f]), f
        es = c.export_state(st)
        for f in ("swa_k", "swa_v"):          # L > n_win: every ring slot holds a token
            assert np.array_equal(es[f], ref_s[f])
        assert np.array_equal(es["idx_tail"][:L % 128], ref_s["idx_tail"][:L % 128])


def test_deferred_seal_flush_equals_default():
    import heterogeneous_sparse_attention_amd as hsa
    Wc, Wh = synth.gate_weights(6)
    a, b = hsa.Cache(128, 1, 4, Wc, Wh), hsa.Cache(128, 1, 4, Wc, Wh)
    K, V, KI = dev_tokens(6, 1, np.arange(256))
    sa, sb = a.state_alloc(), b.state_alloc()
    a.append_kv([sa], [0, 256], K, V, KI)
    b.append_kv([sb], [0, 128], K[:128], V[:128], KI[:128], defer=True)
    assert b.state_query(sb)["pending_seal"] == 1 and b.state_query(sb)["n_blocks"] == 0
    with pytest.raises(hsa.HsaError) as e:
        b.append_kv([sb], [0, 1], K[128:129], V[128:129], KI[128:129])
    assert e.value.code == -4
    b.compress_flush([sb])
    b.append_kv([sb], [0, 128], K[128:], V[128:], KI[128:])
    for x, y in zip(a.block_table(sa), b.block_table(sb)):
        ea, eb = a.export_block(x), b.export_block(y)
        for f in ea:
            assert np.array_equal(ea[f], eb[f])


def _decode_batch(cache, o, states, keys, seed, k, check_scores=True, sorted=False):
    """One decode step for `states` (token position = current length), GPU vs oracle."""
    import torch
    pos = np.array([o.info(s)["len"] for s in states])
    Kn, Vn, KIn = dev_tokens(seed, keys, pos)
    Q, QI = dev_queries(seed, keys, pos)
    sc = torch.empty((len(states), k), dtype=torch.float32, device="cuda")
    idx, _, out = cache.decode_step(states, Kn, Vn, KIn, Q, QI, k, score_out=sc, sorted=sorted)
    Kh, Vh, KIh = host_tokens(seed, keys, pos)
    o.append(states, [(Kh[i:i + 1], Vh[i:i + 1], KIh[i:i + 1]) for i in range(len(states))])
    q, qi = host_queries(seed, keys, pos)
    gidx = idx.cpu().numpy()
    gsc = sc.cpu().numpy()
    gout = out.cpu().numpy()
    for i, s in enumerate(states):
        ref_scores = o.scores(s, qi[i])
        ridx, rval = o.topk(s, qi[i], k, sorted=sorted)
        assert topk_accept(gidx[i], gsc[i], ref_scores, k, sorted=sorted)
        if check_scores:
            assert np.array_equal(gidx[i], ridx)
            m = ridx >= 0
            assert np.array_equal(gsc[i][m], rval[m])
        ref = o.attend(s, q[i], gidx[i], k)
        assert rel_l2(gout[i], ref) <= TOL, (s, rel_l2(gout[i], ref))
    return gidx


@pytest.mark.parametrize("fused", ["0", "1"])
def test_ragged_batch_over_64_requests(monkeypatch, fused):
    """70 requests (two launch batches), lengths 1..1500, 4 decode steps, with the
    decode step in four launches and in three."""
    monkeypatch.setenv("HSA_STEP_FUSED", fused)
    seed = 0x5150
    rng = np.random.default_rng(seed)
    B = 70
    L0 = rng.integers(1, 1501, B)
    cache, o = new_pair(128, B, int((L0 + 8).sum() // 128 + B), seed)
    states = [cache.state_alloc() for _ in range(B)]
    assert states == [o.state_alloc() for _ in range(B)]
    keys = np.arange(B)
    cu = np.concatenate([[0], np.cumsum(L0)])
    pos = np.concatenate([np.arange(n) for n in L0])
    kk = np.repeat(keys, L0)
    K, V, KI = dev_tokens(seed, kk, pos)
    cache.append_kv(states, cu, K, V, KI)
    Kh, Vh, KIh = host_tokens(seed, kk, pos)
    o.append(states, [(Kh[a:b], Vh[a:b], KIh[a:b]) for a, b in zip(cu[:-1], cu[1:])])
    for s in states:
        assert cache.block_table(s) == o.table(s)
    for s in states[::9]:
        check_state(cache, o, s, s)
        for b in o.table(s)[:2]:
            check_block(cache, o, b, b)
    for step in range(4):
        _decode_batch(cache, o, states, keys, seed, 96, sorted=step == 3)


def test_prefix_share_fork_and_free():
    """Parents prefilled per group; children fork at block boundaries and below; the
    shared blocks are one physical copy, refcounted, bit identical to an
    independent rebuild; freeing parents keeps the children's blocks alive."""
    seed = 0x7070
    n_win = 256
    cache, o = new_pair(n_win, 12, 64, seed)
    groups = 2
    parents = [cache.state_alloc() for _ in range(groups)]
    assert parents == [o.state_alloc() for _ in range(groups)]
    pk = [0x800000 | g for g in range(groups)]
    children, ckeys = [], []
    for g in range(groups):
        forks = [256, 384, 200]            # 200: fork mid-block (the open block is in State)
        done = 0
        for f in sorted(forks):
            pos = np.arange(done, f)
            K, V, KI = dev_tokens(seed, pk[g], pos)
            cache.append_kv([parents[g]], [0, len(pos)], K, V, KI)
            o.append([parents[g]], [host_tokens(seed, pk[g], pos)])
            done = f
            c = cache.state_alloc()
            assert c == o.state_alloc()
            cache.block_table_share(parents[g], c)
            o.share(parents[g], c)
            children.append(c)
            ckeys.append(100 + c)
    for b in range(64):
        if o.refcount[b]:
            assert cache.refcount(b) == o.refcount[b]
    # children continue with their own tokens
    for c, key in zip(children, ckeys):
        L = o.info(c)["len"]
        pos = np.arange(L, L + 300)
        K, V, KI = dev_tokens(seed, key, pos)
        cache.append_kv([c], [0, 300], K, V, KI)
        o.append([c], [host_tokens(seed, key, pos)])
        assert cache.block_table(c) == o.table(c)
        check_state(cache, o, c, c)
    for g in range(groups):
        cache.state_free(parents[g])
        o.state_free(parents[g])
    for b in range(64):
        assert cache.refcount(b) == o.refcount[b]
    # independent rebuild of group 0's 384-token prefix: bit-identical shared blocks
    r = cache.state_alloc()
    o.state_alloc()
    pos = np.arange(384)
    K, V, KI = dev_tokens(seed, pk[0], pos)
    cache.append_kv([r], [0, 384], K, V, KI)
    shared = cache.block_table(children[2])[:3]      # group 0's fork at 384
    assert shared == o.table(children[2])[:3]
    for x, y in zip(shared, cache.block_table(r)):
        ex, ey = cache.export_block(x), cache.export_block(y)
        for f in ex:
            assert np.array_equal(ex[f], ey[f])
    for step in range(3):
        _decode_batch(cache, o, children, np.array(ckeys), seed, 40)


def test_edge_cases_short_states_and_k_bounds():
    import torch
    seed = 0x2222
    cache, o = new_pair(128, 6, 16, seed)
    st = [cache.state_alloc() for _ in range(5)]
    [o.state_alloc() for _ in range(5)]
    L0 = [1, 5, 127, 128, 129]          # no block, no block, no block, exactly one, one + 1
    cu = np.concatenate([[0], np.cumsum(L0)])
    pos = np.concatenate([np.arange(n) for n in L0])
    keys = np.repeat(np.arange(5), L0)
    K, V, KI = dev_tokens(seed, keys, pos)
    cache.append_kv(st, cu, K, V, KI)
    Kh, Vh, KIh = host_tokens(seed, keys, pos)
    o.append(st, [(Kh[a:b], Vh[a:b], KIh[a:b]) for a, b in zip(cu[:-1], cu[1:])])
    for k in (1, 31, 32, 33, 4096):
        _decode_batch(cache, o, st, np.arange(5), seed, k)
    _decode_batch(cache, o, st, np.arange(5), seed, 4096, sorted=True)
    # attention without CSA (k = 0) and with user top-k rows holding -1 / out of range
    pos = np.array([o.info(s)["len"] for s in st]) - 1
    Q, _ = dev_queries(seed, np.arange(5), pos)
    q, _ = host_queries(seed, np.arange(5), pos)
    out = cache.decode_attend(st, Q, None, 0).cpu().numpy()
    for i, s in enumerate(st):
        assert rel_l2(out[i], o.attend(s, q[i], [], 0)) <= TOL
    sel = np.array([[-1, 0, 31, 32, 5000, -7, 1, 1]] * 5, np.int32)
    out = cache.decode_attend(st, Q, torch.from_numpy(sel).cuda(), 8).cpu().numpy()
    for i, s in enumerate(st):
        assert rel_l2(out[i], o.attend(s, q[i], sel[i], 8)) <= TOL
    # an append where some requests bring no tokens (bulk path), then decode
    cu = np.array([0, 0, 3, 3, 130, 130])
    pos = np.concatenate([np.arange(o.info(s)["len"], o.info(s)["len"] + n)
                          for s, n in zip(st, np.diff(cu))])
    keys = np.repeat(np.arange(5), np.diff(cu))
    K, V, KI = dev_tokens(seed, keys, pos)
    cache.append_kv(st, cu, K, V, KI)
    Kh, Vh, KIh = host_tokens(seed, keys, pos)
    o.append(st, [(Kh[a:b], Vh[a:b], KIh[a:b]) for a, b in zip(cu[:-1], cu[1:])])
    for s in st:
        assert cache.block_table(s) == o.table(s)
        check_state(cache, o, s, s)
    _decode_batch(cache, o, st, np.arange(5), seed, 64)


def test_topk_large_rows_with_ties():
    """Rows longer than the selection's LDS cache (N = 9600 > 4096 entries) stream
    their scores from L2; request 1 has zero indexer keys in its first 150 blocks,
    so 4800 entries score exactly 0 and the cut falls inside that tie. Both
    selection kernels (hsa_indexer_topk and the decode step), sorted and unsorted,
    against the oracle bit for bit; request 2 stays on the cached path."""
    _topk_rows_with_ties()


@pytest.mark.parametrize("slice_n", [32, 1024])
def test_topk_sliced_rows_with_ties(monkeypatch, slice_n):
    """The same rows selected in two rounds (per-slice candidates, then a select
    over them), with slices far shorter than the default so that 9600-entry rows
    are cut into 10 or 300 slices: the tie of 4800 zero scores spans several slices,
    short last slices pad their candidates, and request 2 (1280 entries) is sliced
    for small k and whole for k = 4096."""
    monkeypatch.setenv("HSA_SELECT_SLICE", str(slice_n))
    _topk_rows_with_ties()


def _topk_rows_with_ties():
    import torch
    seed = 0x7070
    L0 = [128 * 300 + 5, 128 * 300 + 5, 128 * 40 + 3]
    cache, o = new_pair(128, 4, sum(L0) // 128 + 8, seed)
    st = [cache.state_alloc() for _ in L0]
    assert st == [o.state_alloc() for _ in L0]
    cu = np.concatenate([[0], np.cumsum(L0)])
    pos = np.concatenate([np.arange(n) for n in L0])
    keys = np.repeat(np.arange(3), L0)
    K, V, KI = dev_tokens(seed, keys, pos)
    Kh, Vh, KIh = host_tokens(seed, keys, pos)
    zero = np.nonzero((keys == 1) & (pos < 150 * 128))[0]
    KI[torch.from_numpy(zero).cuda()] = 0.0
    KIh[zero] = 0.0
    cache.append_kv(st, cu, K, V, KI)
    o.append(st, [(Kh[a:b], Vh[a:b], KIh[a:b]) for a, b in zip(cu[:-1], cu[1:])])
    qpos = np.array(L0) - 1
    _, QI = dev_queries(seed, np.arange(3), qpos)
    _, qi = host_queries(seed, np.arange(3), qpos)
    for k in (1, 777, 4096):
        for srt in (False, True):
            sc = torch.empty((3, k), dtype=torch.float32, device="cuda")
            idx, _ = cache.indexer_topk(st, QI, k, score_out=sc, sorted=srt)
            idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
            for i, s in enumerate(st):
                ridx, rval = o.topk(s, qi[i], k, sorted=srt)
                assert np.array_equal(idx[i], ridx), (k, srt, i)
                m = ridx >= 0
                assert np.array_equal(sc[i][m], rval[m]), (k, srt, i)
    for k, srt in ((4096, False), (777, True), (1, False)):
        _decode_batch(cache, o, st, np.arange(3), seed, k, sorted=srt)


def test_errors_change_nothing_on_device():
    import heterogeneous_sparse_attention_amd as hsa
    seed = 3
    cache, o = new_pair(128, 2, 2, seed)
    a, b = cache.state_alloc(), cache.state_alloc()
    with pytest.raises(hsa.HsaError) as e:
        cache.state_alloc()
    assert e.value.code == -3
    K, V, KI = dev_tokens(seed, 0, np.arange(400))
    cache.append_kv([a], [0, 200], K[:200], V[:200], KI[:200])
    before = cache.export_state(a)
    with pytest.raises(hsa.HsaError) as e:
        cache.append_kv([a, b], [0, 100, 356], K[:356], V[:356], KI[:356])
    assert e.value.code == -2
    assert cache.state_query(a)["len"] == 200 and cache.state_query(b)["len"] == 0
    after = cache.export_state(a)
    for f in before:   # bit for bit: slots past the valid tokens hold whatever was there
        assert np.array_equal(before[f].view(np.uint8), after[f].view(np.uint8)), f
    with pytest.raises(hsa.HsaError):
        cache.decode_attend([b], *dev_queries(seed, 0, [0])[:1], None, 0)   # empty state
    with pytest.raises(hsa.HsaError):
        cache.indexer_topk([a], dev_queries(seed, 0, [0])[1], 0)            # k < 1
    _, qi = dev_queries(seed, 0, [0])
    idx, _ = cache.indexer_topk([a], qi, 40)                                   # standalone call
    _, hqi = host_queries(seed, 0, [0])
    o.state_alloc()
    o.append([0], [host_tokens(seed, 0, np.arange(200))])
    assert np.array_equal(idx.cpu().numpy()[0], o.topk(0, hqi[0], 40)[0])


@pytest.mark.parametrize("fused", ["0", "1"])
def test_decode_step_matches_separate_calls(monkeypatch, fused):
    """The decode step, in four launches or in three (part-B workgroups selecting
    for themselves, several per request so each writes a share of the top-k row),
    equals append_kv + indexer_topk + decode_attend: same block tables and State,
    bit-identical blocks, top-k ordinals and scores (sorted and unsorted), attention
    equal to fp32 rounding (only the order of the softmax sum differs)."""
    import torch
    import heterogeneous_sparse_attention_amd as hsa
    monkeypatch.setenv("HSA_STEP_FUSED", fused)
    seed = 0x4455
    Wc, Wh = synth.gate_weights(seed)
    rng = np.random.default_rng(seed)
    B, k = 9, 40
    L0 = np.array([1, 126, 127, 128, 255, 300, 511, 700, 1023])    # several seal on step 1 or 2
    a = hsa.Cache(128, B, 64, Wc, Wh)
    b = hsa.Cache(128, B, 64, Wc, Wh)
    sa = [a.state_alloc() for _ in range(B)]
    sb = [b.state_alloc() for _ in range(B)]
    cu = np.concatenate([[0], np.cumsum(L0)])
    pos = np.concatenate([np.arange(n) for n in L0])
    keys = np.repeat(np.arange(B), L0)
    K, V, KI = dev_tokens(seed, keys, pos)
    a.append_kv(sa, cu, K, V, KI)
    b.append_kv(sb, cu, K, V, KI)
    for step in range(3):
        p = L0 + step
        srt = step == 1
        Kn, Vn, KIn = dev_tokens(seed, np.arange(B), p)
        Q, QI = dev_queries(seed, np.arange(B), p)
        sa_sc = torch.full((B, k), 7.0, dtype=torch.float32, device="cuda")
        sb_sc = torch.full((B, k), 7.0, dtype=torch.float32, device="cuda")
        ta, _, oa = a.decode_step(sa, Kn, Vn, KIn, Q, QI, k, score_out=sa_sc, sorted=srt)
        b.append_kv(sb, np.arange(B + 1), Kn, Vn, KIn)
        tb, _ = b.indexer_topk(sb, QI, k, score_out=sb_sc, sorted=srt)
        ob = b.decode_attend(sb, Q, tb, k)
        assert torch.equal(ta, tb), step
        assert torch.equal(sa_sc, sb_sc), step
        assert rel_l2(oa.cpu().numpy(), ob.cpu().numpy()) <= 1e-5
    for x, y in zip(sa, sb):
        assert a.block_table(x) == b.block_table(y)
        for i, j in zip(a.block_table(x), b.block_table(y)):
            ea, eb = a.export_block(i), b.export_block(j)
            for f in ea:
                assert np.array_equal(ea[f], eb[f]), f
        ea, eb = a.export_state(x), b.export_state(y)
        info = a.state_query(x)
        L, nb = info["len"], info["n_blocks"]
        live_swa = [p % 128 for p in range(max(0, L - 128), L)]
        live_tail = [p % 128 for p in range(128 * nb, L)]
        for f in ("swa_k", "swa_v"):
            assert np.array_equal(ea[f][live_swa], eb[f][live_swa]), f
        assert np.array_equal(ea["idx_tail"][live_tail], eb["idx_tail"][live_tail])
