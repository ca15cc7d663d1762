"""GPU parity of prefix hits under the three SWA policies (reading R17): Zero
(hsa_prefix_attach + hsa_state_write of the window), Periodic (attach +
hsa_state_restore of an earlier checkpoint + replay of the gap) and Full (attach +
restore of the checkpoint at the prefix end), against a fork of the live prefix
request and against the oracle.

Each policy's state must equal the fork's slot for slot (ring, indexer tail,
length, table), bit for bit, with the prefix's blocks shared and never sealed again
(the prefix entry holds them by hsa_block_ref after the source request is freed).
The next decode step must then give the fork's top-k and output bit for bit, and the
oracle's within the usual tolerance.
"""

import numpy as np
import pytest

from tests.gpu_util import dev_queries, dev_tokens, host_queries, host_tokens, rel_l2
from tests.test_gpu_parity import check_state, new_pair

pytestmark = pytest.mark.gpu

TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import heterogeneous_sparse_attention_amd as hsa
    hsa.load()          # raises if the library is missing: no fallback


@pytest.mark.parametrize("n_win,P,c", [(128, 1000, 512), (128, 1000, 900), (256, 640, 0),
                                       (512, 1500, 1024), (128, 384, 256), (256, 100, 64)])
def test_prefix_policies_match_the_fork(n_win, P, c):
    import torch
    seed = 0x5A5
    key = 3
    cache, o = new_pair(n_win, 8, 64, seed)
    src = cache.state_alloc()
    assert src == o.state_alloc()
    for a, b in ((0, c), (c, P)):
        if b > a:
            pos = np.arange(a, b)
            cache.append_kv([src], [0, b - a], *dev_tokens(seed, key, pos))
            o.append([src], [host_tokens(seed, key, pos)])
        if b == c:
            buf_c, len_c = cache.state_checkpoint(src)
            ck_c = o.checkpoint(src)
            assert len_c == c
    buf_p, len_p = cache.state_checkpoint(src)
    ck_p = o.checkpoint(src)
    assert len_p == P
    fork = cache.state_alloc()
    assert fork == o.state_alloc()
    cache.block_table_share(src, fork)
    o.share(src, fork)
    blocks = cache.block_table(src)
    assert blocks == o.table(src)
    cache.block_ref(blocks, +1)
    o.block_ref(blocks, +1)
    cache.state_free(src)
    o.state_free(src)
    hits = [cache.state_alloc() for _ in range(3)]
    assert hits == [o.state_alloc() for _ in range(3)]
    zero, per, full = hits
    cache.prefix_attach(hits, blocks, [P] * 3)            # one batched call, one shared list
    for d in hits:
        o.prefix_attach(d, blocks, P)
    m = min(P, n_win)
    pos = np.arange(P - m, P)
    cache.state_write([zero], [0, m], [P - m], *dev_tokens(seed, key, pos))
    o.state_write([zero], [host_tokens(seed, key, pos)], [P - m])
    cache.state_restore(per, buf_c, c)
    o.restore(per, ck_c)
    pos = np.arange(c, P)
    if P > c:
        cache.state_write([per], [0, P - c], [c], *dev_tokens(seed, key, pos))
        o.state_write([per], [host_tokens(seed, key, pos)], [c])
    cache.state_restore(full, buf_p, P)
    o.restore(full, ck_p)
    ef = cache.export_state(fork)
    for d in hits:
        assert cache.state_query(d) == cache.state_query(fork)
        assert cache.block_table(d) == blocks
        check_state(cache, o, d, d)
        ed = cache.export_state(d)
        for p in range(P - m, P):
            assert np.array_equal(ed["swa_k"][p % n_win], ef["swa_k"][p % n_win]), (d, p)
            assert np.array_equal(ed["swa_v"][p % n_win], ef["swa_v"][p % n_win]), (d, p)
        t = P % 128
        assert np.array_equal(ed["idx_tail"][:t], ef["idx_tail"][:t])
    for b in blocks:
        assert cache.refcount(b) == o.refcount[b] == 5
    # the next decode step: all four states see the same token and query
    states = [fork] + hits
    k = 24
    Kn, Vn, KIn = dev_tokens(seed, np.full(4, key), np.full(4, P))
    Q, QI = dev_queries(seed, np.full(4, key), np.full(4, P))
    sc = torch.empty((4, k), dtype=torch.float32, device="cuda")
    idx, _, out = cache.decode_step(states, Kn, Vn, KIn, Q, QI, k, score_out=sc)
    Kh, Vh, KIh = host_tokens(seed, np.full(4, key), np.full(4, P))
    o.append(states, [(Kh[i:i + 1], Vh[i:i + 1], KIh[i:i + 1]) for i in range(4)])
    q, qi = host_queries(seed, np.full(4, key), np.full(4, P))
    gidx, gout, gsc = idx.cpu().numpy(), out.cpu().numpy(), sc.cpu().numpy()
    for i in range(1, 4):
        assert np.array_equal(gidx[i], gidx[0]) and np.array_equal(gsc[i], gsc[0])
        assert np.array_equal(gout[i], gout[0])
    ridx, _ = o.topk(fork, qi[0], k)
    assert np.array_equal(gidx[0], ridx)
    assert rel_l2(gout[0], o.attend(fork, q[0], ridx, k)) <= TOL
    # releasing everything frees the prefix's blocks
    for s in states:
        cache.state_free(s)
        o.state_free(s)
    cache.block_ref(blocks, -1)
    o.block_ref(blocks, -1)
    for b in blocks:
        assert cache.refcount(b) == o.refcount[b] == 0


def test_prefix_errors_change_nothing():
    import heterogeneous_sparse_attention_amd as hsa
    seed = 0x5A6
    cache, o = new_pair(128, 4, 16, seed)
    a = cache.state_alloc()
    cache.append_kv([a], [0, 300], *dev_tokens(seed, 1, np.arange(300)))
    blocks = cache.block_table(a)
    d = cache.state_alloc()
    with pytest.raises(ValueError):
        cache.prefix_attach(d, blocks[:1], 300)          # needs 2 blocks (binding check)
    with pytest.raises(hsa.HsaError):
        cache.prefix_attach(d, [blocks[0], 15], 300)     # block 15 not in use
    with pytest.raises(hsa.HsaError):
        cache.prefix_attach(a, blocks, 300)              # not empty
    assert cache.state_query(d)["len"] == 0 and all(cache.refcount(b) == 1 for b in blocks)
    with pytest.raises(hsa.HsaError):
        cache.block_ref(blocks + [15], +1)
    with pytest.raises(hsa.HsaError):
        cache.block_ref(blocks + blocks, -1)             # more than held
    assert all(cache.refcount(b) == 1 for b in blocks)
    e = cache.state_alloc()
    with pytest.raises(hsa.HsaError):                    # batch with one bad entry: nothing attached
        cache.prefix_attach([e, d], [15] + blocks, [300, 300], offsets=[1, 0])
    assert cache.state_query(e)["len"] == 0 and all(cache.refcount(b) == 1 for b in blocks)
    cache.prefix_attach([e, d], [15] + blocks, [300, 129], offsets=[1, 1])   # offsets into one list
    assert cache.block_table(e) == blocks and cache.block_table(d) == blocks[:1]
    assert cache.refcount(blocks[0]) == 3 and cache.refcount(blocks[1]) == 2
    cache.state_free(d)
    d = cache.state_alloc()
    cache.prefix_attach(d, blocks, 300)
    with pytest.raises(hsa.HsaError):                    # positions past L
        cache.state_write([d], [0, 10], [295], *dev_tokens(seed, 1, np.arange(295, 305)))
    buf, n = cache.state_checkpoint(a)
    with pytest.raises(hsa.HsaError):
        cache.state_restore(d, buf, 301)                 # checkpoint past L
    cache.close()


@pytest.mark.parametrize("c4_mode", ["sealed", "eager"])
def test_restore_batch_matches_single_restores(c4_mode):
    """hsa_state_restore_batch: one launch for many states, each with its own
    checkpoint (lengths inside and past the first window, with and without a tail),
    equals one hsa_state_restore per state bit for bit, and the oracle's restore;
    the next decode step agrees too (eager C4: the open blocks' entries recomputed)."""
    import ctypes
    import torch
    import heterogeneous_sparse_attention_amd as hsa
    seed = 0x5A7
    W = 256
    lens = [100, 256, 300, 700, 1000]
    n = len(lens)
    cache, o = new_pair(W, 3 * n + 2, 64, seed, c4_mode=c4_mode)
    srcs, bufs, cks, blocks = [], [], [], []
    for i, L in enumerate(lens):
        s = cache.state_alloc()
        assert s == o.state_alloc()
        pos = np.arange(L)
        cache.append_kv([s], [0, L], *dev_tokens(seed, i, pos))
        o.append([s], [host_tokens(seed, i, pos)])
        b, ln = cache.state_checkpoint(s)
        assert ln == L
        srcs.append(s), bufs.append(b), cks.append(o.checkpoint(s)), blocks.append(cache.block_table(s))
    one = [cache.state_alloc() for _ in range(n)]
    many = [cache.state_alloc() for _ in range(n)]
    assert one + many == [o.state_alloc() for _ in range(2 * n)]
    for group in (one, many):
        for i, d in enumerate(group):
            cache.prefix_attach(d, blocks[i], lens[i])
            o.prefix_attach(d, blocks[i], lens[i])
    for i, d in enumerate(one):
        cache.state_restore(d, bufs[i], lens[i])
    cache.state_restore_batch(many[::-1], bufs[::-1], lens[::-1])     # any order
    for i in range(n):
        o.restore(one[i], cks[i])
        o.restore(many[i], cks[i])
    for i in range(n):
        ea, eb = cache.export_state(one[i]), cache.export_state(many[i])
        L = lens[i]
        for p in range(max(0, L - W), L):
            assert np.array_equal(ea["swa_k"][p % W], eb["swa_k"][p % W]), (i, p)
            assert np.array_equal(ea["swa_v"][p % W], eb["swa_v"][p % W]), (i, p)
        assert np.array_equal(ea["idx_tail"][:L % 128], eb["idx_tail"][:L % 128]), i
        if c4_mode == "sealed":
            check_state(cache, o, many[i], many[i])
    # pinned host memory: the kernel reads it through its device address
    pinned = bufs[2].cpu().pin_memory()
    st = np.array([many[2]], np.int32)
    ln = np.array([lens[2]], np.int64)
    ptr = (ctypes.c_void_p * 1)(pinned.data_ptr())
    hsa._check(hsa._lib.hsa_state_restore_batch(cache._ctx, 1, st.ctypes.data_as(ctypes.c_void_p),
                                                ctypes.cast(ptr, ctypes.c_void_p),
                                                ln.ctypes.data_as(ctypes.c_void_p), None),
               "hsa_state_restore_batch")
    torch.cuda.synchronize()
    ea, eb = cache.export_state(one[2]), cache.export_state(many[2])
    for p in range(lens[2] - W, lens[2]):
        assert np.array_equal(ea["swa_k"][p % W], eb["swa_k"][p % W]), p
        assert np.array_equal(ea["swa_v"][p % W], eb["swa_v"][p % W]), p
    assert np.array_equal(ea["idx_tail"][:lens[2] % 128], eb["idx_tail"][:lens[2] % 128])
    # the next decode step of every pair agrees bit for bit
    states = one + many
    k = 24
    keys = np.tile(np.arange(n), 2)
    P = np.tile(np.array(lens), 2)
    Kn, Vn, KIn = dev_tokens(seed, keys, P)
    Q, QI = dev_queries(seed, keys, P)
    sc = torch.empty((2 * n, k), dtype=torch.float32, device="cuda")
    idx, _, out = cache.decode_step(states, Kn, Vn, KIn, Q, QI, k, score_out=sc)
    gidx, gout, gsc = idx.cpu().numpy(), out.cpu().numpy(), sc.cpu().numpy()
    for i in range(n):
        assert np.array_equal(gidx[i], gidx[n + i]) and np.array_equal(gsc[i], gsc[n + i]), i
        assert np.array_equal(gout[i], gout[n + i]), i
    cache.close()


def test_restore_batch_errors_change_nothing():
    import ctypes
    import heterogeneous_sparse_attention_amd as hsa
    seed = 0x5A8
    cache, _ = new_pair(128, 6, 16, seed)
    a = cache.state_alloc()
    cache.append_kv([a], [0, 300], *dev_tokens(seed, 1, np.arange(300)))
    buf, n = cache.state_checkpoint(a)
    blocks = cache.block_table(a)
    d, e = cache.state_alloc(), cache.state_alloc()
    cache.prefix_attach([d, e], blocks + blocks, [300, 300], offsets=[0, 0])
    cache.state_restore(d, buf, 300)
    before = cache.export_state(d)
    with pytest.raises(hsa.HsaError):                    # a state twice
        cache.state_restore_batch([e, e], [buf, buf], [300, 300])
    with pytest.raises(hsa.HsaError):                    # past the state's length
        cache.state_restore_batch([d, e], [buf, buf], [300, 301])
    with pytest.raises(hsa.HsaError):                    # not an allocated state
        cache.state_restore_batch([d, 5], [buf, buf], [300, 0])
    host = np.zeros(cache.checkpoint_bytes(), np.uint8)  # pageable host memory
    st = np.array([d], np.int32)
    ln = np.array([300], np.int64)
    ptr = (ctypes.c_void_p * 1)(host.ctypes.data)
    assert hsa._lib.hsa_state_restore_batch(cache._ctx, 1, st.ctypes.data_as(ctypes.c_void_p),
                                            ctypes.cast(ptr, ctypes.c_void_p),
                                            ln.ctypes.data_as(ctypes.c_void_p), None) != 0
    ptr = (ctypes.c_void_p * 1)(buf.data_ptr() + 8)      # misaligned
    assert hsa._lib.hsa_state_restore_batch(cache._ctx, 1, st.ctypes.data_as(ctypes.c_void_p),
                                            ctypes.cast(ptr, ctypes.c_void_p),
                                            ln.ctypes.data_as(ctypes.c_void_p), None) != 0
    after = cache.export_state(d)
    for name in before:
        assert np.array_equal(before[name].view(np.uint8), after[name].view(np.uint8)), name
    cache.state_restore_batch([], [], [])                # nothing to do
    cache.close()
