"""GPU parity of eager C4 (reading R19): the open block's complete groups of 4 tokens
have their C4 entries at once, are top-k candidates (ordinals after the sealed
entries, scored from the indexer tail) and attention keys; the seal later stores
the same entries. Against the eager oracle: bulk appends that leave open groups,
decode steps that complete groups and seal blocks, both forms of the step, k up to
every candidate, a deferred full tail, standalone top-k and attention, a fork and a
Zero-policy prefix hit of a state with open groups.
"""

import numpy as np
import pytest

import synth
from oracle import Oracle
from tests.gpu_util import dev_queries, dev_tokens, host_queries, host_tokens, rel_l2

pytestmark = pytest.mark.gpu

TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import heterogeneous_sparse_attention_amd as hsa
    hsa.load()          # raises if the library is missing: no fallback


def _pair(seed, n_win, max_states, max_blocks):
    import heterogeneous_sparse_attention_amd as hsa
    Wc, Wh = synth.gate_weights(seed)
    return (hsa.Cache(n_win, max_states, max_blocks, Wc, Wh, c4_mode="eager"),
            Oracle(n_win, Wc, Wh, max_states, max_blocks, c4_mode="eager"))


def _step(cache, o, st, keys, p, seed, k):
    import torch
    B = len(st)
    Kn, Vn, KIn = dev_tokens(seed, keys, p)
    Q, QI = dev_queries(seed, keys, p)
    sc = torch.empty((B, k), dtype=torch.float32, device="cuda")
    idx, _, out = cache.decode_step(st, Kn, Vn, KIn, Q, QI, k, score_out=sc)
    Kh, Vh, KIh = host_tokens(seed, keys, p)
    o.append(st, [(Kh[i:i + 1], Vh[i:i + 1], KIh[i:i + 1]) for i in range(B)])
    q, qi = host_queries(seed, keys, p)
    gidx, gout, gsc = idx.cpu().numpy(), out.cpu().numpy(), sc.cpu().numpy()
    for i, s in enumerate(st):
        ridx, rval = o.topk(s, qi[i], k)
        assert np.array_equal(gidx[i], ridx), (k, i, int(p[i]))
        m = ridx >= 0
        assert np.array_equal(gsc[i][m].astype(np.float64), rval[m]), (k, i)
        ref = o.attend(s, q[i], ridx, k)
        assert rel_l2(gout[i], ref) <= TOL, (k, i, rel_l2(gout[i], ref))
    return Q, QI, idx, q, qi


@pytest.mark.parametrize("fused", ["1", "0"])
def test_eager_matches_oracle(monkeypatch, fused):
    monkeypatch.setenv("HSA_STEP_FUSED", fused)
    seed = 0xEA6
    L0 = np.array([1, 3, 4, 126, 127, 131, 260, 700, 1021])
    B = len(L0)
    cache, o = _pair(seed, 128, B + 2, int((L0 + 10).sum() // 128 + B + 4))
    st = [cache.state_alloc() for _ in range(B)]
    assert st == [o.state_alloc() for _ in range(B)]
    cu = np.concatenate([[0], np.cumsum(L0)])
    pos = np.concatenate([np.arange(n) for n in L0])
    keys = np.repeat(np.arange(B), L0)
    cache.append_kv(st, cu, *dev_tokens(seed, keys, pos))
    Kh, Vh, KIh = host_tokens(seed, keys, pos)
    o.append(st, [(Kh[a:b], Vh[a:b], KIh[a:b]) for a, b in zip(cu[:-1], cu[1:])])
    L = L0.copy()
    for step, k in enumerate((40, 4096, 7, 40, 512, 40)):
        Q, QI, idx, q, qi = _step(cache, o, st, np.arange(B), L, seed, k)
        L = L + 1
        if step in (1, 4):
            tidx, _ = cache.indexer_topk(st, QI, k)
            assert np.array_equal(tidx.cpu().numpy(), idx.cpu().numpy())
            att = cache.decode_attend(st, Q, idx, k)
            for i, s in enumerate(st):
                assert rel_l2(att[i].cpu().numpy(), o.attend(s, q[i], idx[i].cpu().numpy(), k)) <= TOL
    # a fork and a Zero-policy hit of the state with open groups (L mod 128 = 3 now)
    src = st[7]
    assert (o.info(src)["len"] % 128) // 4 >= 1
    f = cache.state_alloc()
    assert f == o.state_alloc()
    cache.block_table_share(src, f)
    o.share(src, f)
    z = cache.state_alloc()
    assert z == o.state_alloc()
    Ls = o.info(src)["len"]
    blocks = cache.block_table(src)
    cache.prefix_attach(z, blocks, Ls)
    o.prefix_attach(z, blocks, Ls)
    w = np.arange(Ls - 128, Ls)
    cache.state_write([z], [0, 128], [Ls - 128], *dev_tokens(seed, 7, w))
    o.state_write([z], [host_tokens(seed, 7, w)], [Ls - 128])
    _step(cache, o, [src, f, z], np.array([7, 7, 7]), np.full(3, Ls), seed, 600)


def test_eager_deferred_full_tail():
    """A deferred full tail: its 32 groups are all open candidates until the flush
    seals them into a block with the same entries."""
    seed = 0xEA7
    cache, o = _pair(seed, 128, 2, 8)
    a = cache.state_alloc()
    assert a == o.state_alloc()
    pos = np.arange(256)
    cache.append_kv([a], [0, 128], *dev_tokens(seed, 0, pos[:128]))
    o.append([a], [host_tokens(seed, 0, pos[:128])])
    cache.append_kv([a], [0, 128], *dev_tokens(seed, 0, pos[128:])
                    , defer=True)
    o.append([a], [host_tokens(seed, 0, pos[128:])], defer_seal=True)
    import torch
    _, QI = dev_queries(seed, np.array([0]), np.array([256]))
    _, qi = host_queries(seed, np.array([0]), np.array([256]))
    sc = torch.empty((1, 80), dtype=torch.float32, device="cuda")
    idx, _ = cache.indexer_topk([a], QI, 80, score_out=sc)
    ridx, rval = o.topk(a, qi[0], 80)
    assert (ridx >= 0).sum() == 64 and np.array_equal(idx[0].cpu().numpy(), ridx)
    assert np.array_equal(sc[0].cpu().numpy()[:64].astype(np.float64), rval[:64])
    cache.compress_flush([a])
    o.compress_flush([a])
    idx2, _ = cache.indexer_topk([a], QI, 80, score_out=sc)
    assert np.array_equal(idx2[0].cpu().numpy(), ridx)      # the same 64 entries, now sealed
    assert np.array_equal(sc[0].cpu().numpy()[:64].astype(np.float64), rval[:64])
