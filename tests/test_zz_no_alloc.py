"""hsa_decode_step_noalloc against hsa_decode_step, through the C ABI.

Two contexts hold the same requests, built by the same calls. One runs each decode
step through hsa_decode_step, with scratch from the context's own buffers. The other
runs the allocation-free entry point, with scratch from the library's fixed device
buffer. The kernels and launch plans are the same, so top-k rows, scores, outputs
and every pool must agree bit for bit. This is checked on two calls in a row, the
second with a smaller batch, in both step forms, and with long rows that take the
two-round top-k. A step that needs more scratch than the fixed buffer holds is
refused, and nothing changes.
"""

import numpy as np
import pytest

import synth
from tests.gpu_util import dev_queries, dev_tokens

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import heterogeneous_sparse_attention_amd as hsa
    hsa.load()          # raises if the library is missing: no fallback


SEED = 0x4E4F41


def _pair(n_win, max_states, max_blocks, **fmt):
    from heterogeneous_sparse_attention_amd import Cache
    Wc, Wh = synth.gate_weights(SEED)
    return (Cache(n_win, max_states, max_blocks, Wc, Wh, **fmt),
            Cache(n_win, max_states, max_blocks, Wc, Wh, **fmt))


def _prefill(caches, L0):
    st = None
    for c in caches:
        s = [c.state_alloc() for _ in L0]
        assert st is None or s == st
        st = s
    cu = np.concatenate([[0], np.cumsum(L0)])
    pos = np.concatenate([np.arange(n) for n in L0])
    keys = np.repeat(np.arange(len(L0)), L0)
    toks = dev_tokens(SEED, keys, pos)
    for c in caches:
        c.append_kv(st, cu, *toks)
    return st


def _step(caches, st, keys, pos, k, sorted=False, noalloc=(False, True)):
    """One decode step of the listed states in both contexts: by default the first
    through hsa_decode_step, the second through hsa_decode_step_noalloc."""
    import torch
    toks = dev_tokens(SEED, keys, pos)
    qs = dev_queries(SEED, keys, pos)
    n = len(st)
    res = []
    for i, c in enumerate(caches):
        topk = torch.full((n, k), -7, dtype=torch.int32, device="cuda")
        score = torch.full((n, k), 7.0, dtype=torch.float32, device="cuda")
        out = torch.full((n, 16, 128), 7.0, dtype=torch.float32, device="cuda")
        c.decode_step(st, *toks, *qs, k, topk_out=topk, score_out=score, out=out, sorted=sorted,
                      noalloc=noalloc[i])
        res.append((topk, score, out))
    torch.cuda.synchronize()
    return res


def _same_results(res):
    import torch
    (t0, s0, o0), (t1, s1, o1) = res
    assert torch.equal(t0, t1)
    assert torch.equal(s0, s1)
    assert torch.equal(o0, o1)
    assert not torch.isnan(o1).any()


def _same_pools(caches, st):
    a, b = caches
    for s in st:
        info = a.state_query(s)
        assert info == b.state_query(s)
        assert a.block_table(s) == b.block_table(s)
        ea, eb = a.export_state(s), b.export_state(s)
        L, W = info["len"], a.n_win
        ring = np.arange(L - info["swa_len"], L) % W        # slots holding the window
        tail = np.arange(L - info["hca_tail"], L) % 128     # slots holding the open block
        for name in ea:   # ring rows (bf16, or FP8 codes and scales) and the indexer tail
            slots = tail if name == "idx_tail" else ring
            assert np.array_equal(ea[name][slots], eb[name][slots]), (s, name)
    for blk in sorted({x for s in st for x in a.block_table(s)}):
        ea, eb = a.export_block(blk), b.export_block(blk)
        for name in ea:
            assert np.array_equal(ea[name], eb[name]), (blk, name)


FORMATS = [{}, {"entry_format": "fp8", "index_format": "mxfp4", "kv_format": "fp8"}]


@pytest.mark.parametrize("fmt", FORMATS, ids=["bf16", "fp8_mxfp4_fp8kv"])
def test_noalloc_step_equals_decode_step_two_calls(fmt):
    """Call 1: 12 requests (seals, a request with no block, rows long enough for the
    four-launch form); call 2: 5 of them with a smaller k. Both step forms; the
    measured storage and the low-bit one (FP8 entries and KV, MXFP4 keys)."""
    caches = _pair(128, 16, 600, **fmt)
    try:
        L0 = np.array([127, 1, 255, 130, 17000, 383, 4096, 5, 128, 900, 2047, 3000])
        st = _prefill(caches, L0)
        L = L0.copy()
        for sorted_ in (False, True):
            res = _step(caches, st, np.arange(len(st)), L, 512, sorted=sorted_)
            _same_results(res)
            L += 1
            sub = [0, 2, 4, 8, 11]
            res = _step(caches, [st[i] for i in sub], np.array(sub), L[sub], 40, sorted=sorted_)
            _same_results(res)
            L[sub] += 1
        _same_pools(caches, st)
        # hsa_decode_step is unchanged after no-alloc calls on the same context
        res = _step(caches, st[:3], np.arange(3), L[:3], 16, noalloc=(False, False))
        _same_results(res)
    finally:
        for c in caches:
            c.close()


def test_noalloc_step_sliced_rows(monkeypatch):
    """Rows cut into slices (two-round top-k, scratch for the slices' candidates)."""
    monkeypatch.setenv("HSA_SELECT_SLICE", "1024")
    caches = _pair(128, 8, 300)
    try:
        L0 = np.array([9000, 20000, 130, 6000])
        st = _prefill(caches, L0)
        res = _step(caches, st, np.arange(4), L0, 600)
        _same_results(res)
        res = _step(caches, st[:2], np.arange(2), L0[:2] + 1, 64)
        _same_results(res)
        _same_pools(caches, st)
    finally:
        for c in caches:
            c.close()


def test_noalloc_step_refuses_oversized_batch():
    """64 requests, one of them 524,800 tokens long: its 131,200-score row, kept once
    per request of the batch (33.6 MB), needs more scratch than the fixed buffer
    holds. The call is refused and changes nothing; the same step of that request
    alone fits."""
    import torch
    import heterogeneous_sparse_attention_amd as hsa
    nbytes = ctypes_bytes()
    assert nbytes == 32 << 20
    from heterogeneous_sparse_attention_amd import Cache
    Wc, Wh = synth.gate_weights(SEED)
    c = Cache(128, 64, 4200, Wc, Wh)
    try:
        L0 = np.array([4100 * 128] + [1] * 63)
        st = _prefill([c], L0)
        k_new, v_new, i_new = dev_tokens(SEED, np.arange(64), L0)
        q, qi = dev_queries(SEED, np.arange(64), L0)
        topk = torch.empty((64, 16), dtype=torch.int32, device="cuda")
        out = torch.empty((64, 16, 128), dtype=torch.float32, device="cuda")
        with pytest.raises(hsa.HsaError) as e:
            c.decode_step(st, k_new, v_new, i_new, q, qi, 16, topk_out=topk, out=out, noalloc=True)
        assert e.value.code == -1 and "scratch" in str(e.value)
        assert [c.state_query(s)["len"] for s in st] == L0.tolist()
        c.decode_step(st[:1], k_new[:1], v_new[:1], i_new[:1], q[:1], qi[:1], 16, noalloc=True)
        torch.cuda.synchronize()
        assert c.state_query(st[0])["len"] == L0[0] + 1
    finally:
        c.close()


def ctypes_bytes():
    import ctypes

    import heterogeneous_sparse_attention_amd as hsa
    n = ctypes.c_int64()
    assert hsa.load().hsa_noalloc_scratch_bytes(ctypes.byref(n)) == 0
    return n.value
