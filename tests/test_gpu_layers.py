"""GPU parity of a multi-layer cache (reading R18): one State quota and one Block
Cache over layers of the four types (SWA, CSA, HCA, mixed), each layer with its own
gates and its own tokens, against one oracle per layer driven by the same calls.

Checked per layer: block tables (shared), sealed blocks (C4 entries and indexer keys
of C4 layers, HCA entries of HCA layers), SWA rings and indexer tails, decode steps
in both forms (top-k rows bit exact, all padding without C4 entries; attention
within relative L2 1e-3), hsa_indexer_topk and hsa_decode_attend; and the layer
protocol: an append goes layer 0, 1, ..., n-1 with the same call, and state
changes wait until it has.
"""

import numpy as np
import pytest

import synth
from oracle import Oracle, e4m3_decode
from tests.gpu_util import bf16_to_f64, dev_queries, dev_tokens, host_queries, host_tokens, rel_l2

pytestmark = pytest.mark.gpu

TOL = 1e-3
TYPES = ["swa", "csa", "hca", "mixed"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import heterogeneous_sparse_attention_amd as hsa
    hsa.load()          # raises if the library is missing: no fallback


def _stack(seed):
    import heterogeneous_sparse_attention_amd as hsa
    gates = [synth.gate_weights(seed + 7 * l) for l in range(len(TYPES))]
    Wc = np.stack([g[0] for g in gates])
    Wh = np.stack([g[1] for g in gates])
    return gates, Wc, Wh


def _check_layer(cache, o, states, t):
    fp8, mx4 = cache.entry_format == "fp8", cache.index_format == "mxfp4"
    for s in states:
        assert cache.block_table(s) == o.table(s)
        for b in cache.block_table(s):
            g = cache.export_block(b)
            r = o.block(b)
            c4 = t in ("csa", "mixed")
            kv8 = cache.kv_format == "fp8"
            assert (("csa_k" in g) or ("csa_k_codes" in g)) == c4
            assert (("hca_k" in g) or ("hca_k_codes" in g)) == (t in ("hca", "mixed"))
            if c4 and fp8:
                for n in ("k", "v"):
                    val = e4m3_decode(g[f"csa_{n}_codes"]) * g[f"csa_{n}_scale"][..., None].astype(np.float64)
                    assert rel_l2(val, getattr(r, f"csa_{n}")) <= TOL, (t, n)
            elif c4:
                for n in ("csa_k", "csa_v"):
                    assert rel_l2(bf16_to_f64(g[n]), getattr(r, n)) <= TOL, (t, n)
            if c4 and mx4:
                assert np.array_equal(g["idx_codes"], r.idx_codes) and np.array_equal(g["idx_scales"], r.idx_scales)
            elif c4:
                assert np.array_equal(g["idx"], r.idx)
            if t in ("hca", "mixed") and kv8:   # codes decided from float32 vs float64 pools
                for n in ("k", "v"):
                    assert np.mean(g[f"hca_{n}_codes"] == getattr(r, f"hca_{n}_codes")) > 0.99, (t, n)
                    assert np.allclose(g[f"hca_{n}_scale"], getattr(r, f"hca_{n}_scale"), rtol=1e-6, atol=0)
            elif t in ("hca", "mixed"):
                for n in ("hca_k", "hca_v"):
                    assert rel_l2(bf16_to_f64(g[n]), getattr(r, n)) <= TOL, (t, n)
        ex = cache.export_state(s)
        assert ("idx_tail" in ex) == (t in ("csa", "mixed"))
        st = o.states[s]
        L, W = st.L, cache.n_win
        for i, (k, v) in enumerate(st.swa):
            p = L - len(st.swa) + i
            if cache.kv_format == "fp8":   # ring slots: the oracle's codes and scales exactly
                kc, ks, vc, vs = st.swa_q[i]
                assert np.array_equal(ex["swa_k_codes"][p % W], kc) and np.array_equal(ex["swa_v_codes"][p % W], vc)
                assert np.array_equal(ex["swa_k_scale"][p % W], ks) and np.array_equal(ex["swa_v_scale"][p % W], vs)
                continue
            assert np.array_equal(bf16_to_f64(ex["swa_k"][p % W]), k) and np.array_equal(bf16_to_f64(ex["swa_v"][p % W]), v)
        if t in ("csa", "mixed"):
            for i, (_, _, ki) in enumerate(st.tail):
                assert np.array_equal(ex["idx_tail"][(L - len(st.tail) + i) % 128], ki)


MODES = [("1", "bf16", "f32", "sealed", "bf16"), ("0", "bf16", "f32", "sealed", "bf16"),
         ("1", "fp8", "f32", "sealed", "bf16"), ("0", "bf16", "mxfp4", "sealed", "bf16"),
         ("1", "bf16", "f32", "eager", "bf16"), ("0", "bf16", "f32", "eager", "bf16"),
         ("1", "bf16", "f32", "sealed", "fp8"), ("0", "fp8", "mxfp4", "sealed", "fp8")]


@pytest.mark.parametrize("fused,entries,index,c4_mode,kv", MODES)
def test_layers_match_per_layer_oracles(monkeypatch, fused, entries, index, c4_mode, kv):
    import torch
    import heterogeneous_sparse_attention_amd as hsa
    monkeypatch.setenv("HSA_STEP_FUSED", fused)
    seed = 0x1A7
    gates, Wc, Wh = _stack(seed)
    B = 6
    # decode steps: request 0 inside its first window, the others past it (ring
    # wrap); requests 3 and 4 seal a block at the second step (lengths 256, 768), so
    # an HCA layer's step then runs its seal launch and the others skip it
    L0 = np.array([1, 127, 128, 254, 766, 1100])
    nbk = int((L0 + 140).sum() // 128 + B)
    kw = dict(entry_format=entries, index_format=index, c4_mode=c4_mode, kv_format=kv)
    cache = hsa.Cache(128, B, nbk, Wc, Wh, layer_types=TYPES, **kw)
    orc = [Oracle(128, g[0], g[1], B, nbk, layer_type=t, **kw) for g, t in zip(gates, TYPES)]
    st = [cache.state_alloc() for _ in range(B)]
    for o in orc:
        assert [o.state_alloc() for _ in range(B)] == st
    lseed = [seed + 101 * l for l in range(len(TYPES))]   # each layer has its own tokens
    cu = np.concatenate([[0], np.cumsum(L0)])
    pos = np.concatenate([np.arange(n) for n in L0])
    keys = np.repeat(np.arange(B), L0)
    for l, o in enumerate(orc):
        cache.set_layer(l)
        cache.append_kv(st, cu, *dev_tokens(lseed[l], keys, pos))
        Kh, Vh, KIh = host_tokens(lseed[l], keys, pos)
        o.append(st, [(Kh[a:b], Vh[a:b], KIh[a:b]) for a, b in zip(cu[:-1], cu[1:])])
    # a deferred append that fills request 1's block exactly, then the flush, per layer
    for l, o in enumerate(orc):
        cache.set_layer(l)
        cache.append_kv([st[1]], [0, 1], *dev_tokens(lseed[l], 1, np.array([127])), defer=True)
        o.append([st[1]], [host_tokens(lseed[l], 1, np.array([127]))], defer_seal=True)
    for l, o in enumerate(orc):
        cache.set_layer(l)
        cache.compress_flush([st[1]])
        o.compress_flush([st[1]])
    L = L0.copy()
    L[1] += 1
    for l, (o, t) in enumerate(zip(orc, TYPES)):
        cache.set_layer(l)
        _check_layer(cache, o, st, t)
    for step, k in enumerate((24, 300, 24)):
        p = L + step
        for l, (o, t) in enumerate(zip(orc, TYPES)):
            cache.set_layer(l)
            Kn, Vn, KIn = dev_tokens(lseed[l], np.arange(B), p)
            Q, QI = dev_queries(lseed[l], np.arange(B), p)
            sc = torch.empty((B, k), dtype=torch.float32, device="cuda")
            idx, _, out = cache.decode_step(st, Kn, Vn, KIn, Q, QI, k, score_out=sc)
            Kh, Vh, KIh = host_tokens(lseed[l], np.arange(B), p)
            o.append(st, [(Kh[i:i + 1], Vh[i:i + 1], KIh[i:i + 1]) for i in range(B)])
            q, qi = host_queries(lseed[l], np.arange(B), p)
            gidx, gout = idx.cpu().numpy(), out.cpu().numpy()
            for i, s in enumerate(st):
                ridx, _ = o.topk(s, qi[i], k)
                assert np.array_equal(gidx[i], ridx), (t, step, i)
                ref = o.attend(s, q[i], ridx, k)
                assert rel_l2(gout[i], ref) <= TOL, (t, step, i, rel_l2(gout[i], ref))
            tidx, _ = cache.indexer_topk(st, QI, k)
            assert np.array_equal(tidx.cpu().numpy(), gidx), t
            att = cache.decode_attend(st, Q, idx, k)
            for i, s in enumerate(st):
                assert rel_l2(att[i].cpu().numpy(), o.attend(s, q[i], gidx[i], k)) <= TOL, t
    for l, (o, t) in enumerate(zip(orc, TYPES)):
        cache.set_layer(l)
        _check_layer(cache, o, st, t)
    cache.close()


def test_layer_protocol_errors():
    import heterogeneous_sparse_attention_amd as hsa
    seed = 0x1A8
    gates, Wc, Wh = _stack(seed)
    cache = hsa.Cache(128, 3, 8, Wc, Wh, layer_types=TYPES)
    a, b = cache.state_alloc(), cache.state_alloc()
    cache.append_kv([a], [0, 200], *dev_tokens(seed, 0, np.arange(200)))      # layer 0
    assert cache.state_query(a)["len"] == 200
    cache.set_layer(2)
    with pytest.raises(hsa.HsaError):      # layer 1 comes first
        cache.append_kv([a], [0, 200], *dev_tokens(seed, 0, np.arange(200)))
    cache.set_layer(1)
    with pytest.raises(hsa.HsaError):      # not the call made at layer 0
        cache.append_kv([a], [0, 199], *dev_tokens(seed, 0, np.arange(199)))
    with pytest.raises(hsa.HsaError):      # state changes wait for every layer
        cache.state_free(b)
    with pytest.raises(hsa.HsaError):
        cache.block_table_share(a, b)
    cache.set_layer(0)
    with pytest.raises(hsa.HsaError):      # the previous append is still pending
        cache.append_kv([b], [0, 5], *dev_tokens(seed, 1, np.arange(5)))
    for l in (1, 2, 3):
        cache.set_layer(l)
        cache.append_kv([a], [0, 200], *dev_tokens(seed + l, 0, np.arange(200)))
    cache.block_table_share(a, b)          # now allowed: a fork copies every layer's State
    assert cache.state_query(b)["len"] == 200
    with pytest.raises(hsa.HsaError):
        cache.set_layer(4)
    cache.set_layer(0)                     # an SWA layer exports no C4 entries or HCA
    import ctypes
    buf = np.zeros((16, 128), np.uint16)
    with pytest.raises(hsa.HsaError):
        hsa._check(hsa._lib.hsa_export_block(cache._ctx, cache.block_table(a)[0], None, None,
                                             buf.ctypes.data_as(ctypes.c_void_p), None, None, None),
                   "hsa_export_block")
    assert cache.export_block(cache.block_table(a)[0]) == {}
    cache.state_free(a)
    cache.state_free(b)
    cache.close()
