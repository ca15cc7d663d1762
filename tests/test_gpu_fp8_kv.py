"""GPU parity of FP8 KV storage (reading R20): the SWA ring's tokens and the HCA
entries as per-head E4M3 codes and float32 scales (the R15 quantiser), against the
CPU oracle with kv_format="fp8".

- Ring slots: codes and scales bit for bit. The ring quantises a bf16 input token,
  so both sides see the same float32 values.
- HCA entries (pooled in float32 on the GPU, in float64 by the oracle) and C4
  entries (pooled from the stored tokens). Codes agree except where the two
  poolings straddle a rounding boundary; scales within 1e-6; values within rel L2
  1e-3. Indexer keys are exact.
- Decode steps in both launch forms, with bf16 and with FP8 C4 entries: top-k
  exact, attention within rel L2 1e-3. The same for hsa_indexer_topk and
  hsa_decode_attend.
- The paths that fill a State: fork, checkpoint and restore (single and batched),
  and replay. Each gives the oracle's ring and the same next step.
"""

import numpy as np
import pytest

import synth
from oracle import Oracle
from tests.gpu_util import (bf16_to_f64, check_fp8, dev_queries, dev_tokens, host_queries, host_tokens,
                            pool_magnitude, rel_l2)

pytestmark = pytest.mark.gpu

TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import heterogeneous_sparse_attention_amd as hsa
    hsa.load()          # raises if the library is missing: no fallback


def _pair(seed, n_win, max_states, max_blocks, entries="bf16"):
    import heterogeneous_sparse_attention_amd as hsa
    Wc, Wh = synth.gate_weights(seed)
    return (hsa.Cache(n_win, max_states, max_blocks, Wc, Wh, entry_format=entries, kv_format="fp8"),
            Oracle(n_win, Wc, Wh, max_states, max_blocks, entry_format=entries, kv_format="fp8"))


def check_ring(cache, o, sg, so):
    """Every window slot of the state: codes and scales exactly the oracle's."""
    ex = cache.export_state(sg)
    st = o.states[so]
    L, W = st.L, cache.n_win
    for i, q in enumerate(st.swa_q):
        p = L - len(st.swa_q) + i
        kc, ks, vc, vs = q
        assert np.array_equal(ex["swa_k_codes"][p % W], kc), (so, p)
        assert np.array_equal(ex["swa_v_codes"][p % W], vc), (so, p)
        assert np.array_equal(ex["swa_k_scale"][p % W], ks), (so, p)
        assert np.array_equal(ex["swa_v_scale"][p % W], vs), (so, p)
    for i, (_, _, ki) in enumerate(st.tail):
        p = L - len(st.tail) + i
        assert np.array_equal(ex["idx_tail"][p % 128], ki)


def check_block(cache, o, bg, bo, entries, toks):
    """A sealed block against the oracle; toks: its 128 raw tokens (K, V), from
    which the oracle's unquantised entries are recomputed for the code check."""
    from oracle import gated_pool, quantize_e4m3_rows
    g = cache.export_block(bg)
    r = o.block(bo)
    assert np.array_equal(g["idx"], r.idx)
    Kq = quantize_e4m3_rows(toks[0])[2]
    Vq = quantize_e4m3_rows(toks[1])[2]
    hk, hv = gated_pool(Kq, Vq, o.W_hca, rounded=False)
    mags = pool_magnitude(Kq, Vq, o.W_hca)
    for i, (n, x) in enumerate((("k", hk), ("v", hv))):
        check_fp8(g[f"hca_{n}_codes"], g[f"hca_{n}_scale"], getattr(r, f"hca_{n}_codes"),
                  getattr(r, f"hca_{n}_scale"), x, ("hca", n, bo), mags[i])
    if entries == "fp8":
        c4 = [gated_pool(Kq[4 * j:4 * j + 4], Vq[4 * j:4 * j + 4], o.W_csa, rounded=False) for j in range(32)]
        c4m = [pool_magnitude(Kq[4 * j:4 * j + 4], Vq[4 * j:4 * j + 4], o.W_csa) for j in range(32)]
        for i, n in enumerate(("k", "v")):
            check_fp8(g[f"csa_{n}_codes"], g[f"csa_{n}_scale"], getattr(r, f"csa_{n}_codes"),
                      getattr(r, f"csa_{n}_scale"), np.stack([e[i] for e in c4]), ("c4", n, bo),
                      np.stack([m[i] for m in c4m]))
    else:
        for n in ("k", "v"):
            val = bf16_to_f64(g[f"csa_{n}"])
            ref = getattr(r, f"csa_{n}")
            assert rel_l2(val, ref) <= TOL and np.mean(val == ref) > 0.97, ("c4", n, bo)


def prefill(cache, o, seed, L0):
    B = len(L0)
    st = [cache.state_alloc() for _ in range(B)]
    assert st == [o.state_alloc() for _ in range(B)]
    cu = np.concatenate([[0], np.cumsum(L0)])
    pos = np.concatenate([np.arange(n) for n in L0])
    keys = np.repeat(np.arange(B), L0)
    cache.append_kv(st, cu, *dev_tokens(seed, keys, pos))
    Kh, Vh, KIh = host_tokens(seed, keys, pos)
    o.append(st, [(Kh[a:b], Vh[a:b], KIh[a:b]) for a, b in zip(cu[:-1], cu[1:])])
    return st


def step_and_check(cache, o, seed, st, keys, p, k, sorted=False):
    import torch
    B = len(st)
    Kn, Vn, KIn = dev_tokens(seed, keys, p)
    Q, QI = dev_queries(seed, keys, p)
    sc = torch.empty((B, k), dtype=torch.float32, device="cuda")
    idx, _, out = cache.decode_step(st, Kn, Vn, KIn, Q, QI, k, score_out=sc, sorted=sorted)
    Kh, Vh, KIh = host_tokens(seed, keys, p)
    o.append(st, [(Kh[i:i + 1], Vh[i:i + 1], KIh[i:i + 1]) for i in range(B)])
    q, qi = host_queries(seed, keys, p)
    gidx, gout = idx.cpu().numpy(), out.cpu().numpy()
    for i, s in enumerate(st):
        ridx, _ = o.topk(s, qi[i], k, sorted=sorted)
        assert np.array_equal(gidx[i], ridx), (i, s)
        r = rel_l2(gout[i], o.attend(s, q[i], ridx, k))
        assert r <= TOL, (i, s, r)
    return idx, Q, q


@pytest.mark.parametrize("entries", ["bf16", "fp8"])
@pytest.mark.parametrize("fused", ["1", "0"])
def test_fp8_kv_cache_matches_oracle(monkeypatch, fused, entries):
    monkeypatch.setenv("HSA_STEP_FUSED", fused)
    seed = 0x8F9
    rng = np.random.default_rng(seed)
    B = 9
    L0 = np.concatenate([[1, 127, 128, 255], rng.integers(300, 2500, B - 4)])
    cache, o = _pair(seed, 128, B, int((L0 + 8).sum() // 128 + B), entries)
    try:
        st = prefill(cache, o, seed, L0)

        def blocks_ok():
            for i, s in enumerate(st):
                check_ring(cache, o, s, s)
                for lb, (bg, bo) in enumerate(zip(cache.block_table(s), o.table(s))):
                    K, V, _ = host_tokens(seed, np.full(128, i), np.arange(128 * lb, 128 * lb + 128))
                    check_block(cache, o, bg, bo, entries, (K, V))
        blocks_ok()
        for step, k in enumerate((40, 512, 40)):
            idx, Q, q = step_and_check(cache, o, seed, st, np.arange(B), L0 + step, k, sorted=step == 2)
            att = cache.decode_attend(st, Q, idx, k)   # the standalone call, same selection
            for i, s in enumerate(st):
                assert rel_l2(att[i].cpu().numpy(), o.attend(s, q[i], idx.cpu().numpy()[i], k)) <= TOL
        blocks_ok()
    finally:
        cache.close()


def test_fp8_kv_fill_paths():
    """Fork, checkpoint / restore (single and batched), attach + replay: each state's
    ring equals the oracle's slot for slot, and the next decode step matches."""
    seed = 0x8FA
    L0 = np.array([300, 700])
    cache, o = _pair(seed, 256, 8, 40)
    try:
        st = prefill(cache, o, seed, L0)
        # fork
        f = cache.state_alloc()
        assert f == o.state_alloc()
        cache.block_table_share(st[1], f)
        o.share(st[1], f)
        check_ring(cache, o, f, f)
        # checkpoint of st[1], restored into a state attached to its blocks
        nbytes = cache.checkpoint_bytes()
        assert nbytes == 256 * (4096 + 128) + 128 * 1024
        buf, L = cache.state_checkpoint(st[1])
        ck = o.checkpoint(st[1])
        r1 = cache.state_alloc()
        assert r1 == o.state_alloc()
        blocks = cache.block_table(st[1])
        cache.prefix_attach([r1], blocks, [L])
        o.prefix_attach(r1, o.table(st[1]), L)
        cache.state_restore(r1, buf, L)
        o.restore(r1, ck)
        check_ring(cache, o, r1, r1)
        # the batched restore (one copy launch)
        r2 = cache.state_alloc()
        assert r2 == o.state_alloc()
        cache.prefix_attach([r2], blocks, [L])
        o.prefix_attach(r2, o.table(st[1]), L)
        cache.state_restore_batch([r2], [buf.clone()], [L])
        o.restore(r2, ck)
        check_ring(cache, o, r2, r2)
        # attach + replay of the window's raw tokens (Zero policy)
        z = cache.state_alloc()
        assert z == o.state_alloc()
        cache.prefix_attach([z], blocks, [L])
        o.prefix_attach(z, o.table(st[1]), L)
        p0 = L - 256
        pos = np.arange(p0, L)
        cache.state_write([z], [0, len(pos)], [p0], *dev_tokens(seed, np.full(len(pos), 1), pos))
        Kh, Vh, KIh = host_tokens(seed, np.full(len(pos), 1), pos)
        o.state_write([z], [(Kh, Vh, KIh)], [p0])
        check_ring(cache, o, z, z)
        # one decode step of every state: the copies continue as the original
        sts = [st[1], f, r1, r2, z]
        step_and_check(cache, o, seed, sts, np.full(5, 1), np.full(5, L), 64)
        for s in sts:
            check_ring(cache, o, s, s)
    finally:
        cache.close()


def test_fp8_kv_errors():
    import heterogeneous_sparse_attention_amd as hsa
    Wc, Wh = synth.gate_weights(1)
    with pytest.raises(ValueError):
        hsa.Cache(128, 1, 1, Wc, Wh, kv_format="fp4")
    with pytest.raises(hsa.HsaError):      # eager C4 takes bf16 KV
        hsa.Cache(128, 1, 1, Wc, Wh, kv_format="fp8", c4_mode="eager")
    c = hsa.Cache(128, 1, 2, Wc, Wh, kv_format="fp8")
    try:
        s = c.state_alloc()
        c.append_kv([s], [0, 128], *dev_tokens(1, 0, np.arange(128)))
        import ctypes
        k = np.zeros((128, 16, 128), np.uint16)
        with pytest.raises(hsa.HsaError):  # the ring is FP8: no bf16 export
            hsa._check(hsa._lib.hsa_export_state(c._ctx, s, k.ctypes.data_as(ctypes.c_void_p), None, None, None),
                       "hsa_export_state")
    finally:
        c.close()
    bf = hsa.Cache(128, 1, 2, Wc, Wh)
    try:
        with pytest.raises(hsa.HsaError):  # bf16 KV: no FP8 ring export
            hsa._check(hsa._lib.hsa_export_state_fp8(bf._ctx, 0, None, None, None), "hsa_export_state_fp8")
    finally:
        bf.close()
