"""Run-twice determinism, and no reads of memory that was never written.

Two contexts are created with HSA_CREATE_POISON. Every pool and scratch buffer
then starts as 0xFF bytes, which is NaN in bf16, fp32 and E4M3. Each context gets
the same b32 prefill (32 requests, L0 ~ U{1..8192}) and the same decode steps:
six in the three-launch form, then two with sorted rows (four-launch form). Then
each runs one hsa_indexer_topk and one hsa_decode_attend.

Checks, between the two contexts:
- every top-k row, score and attention output is free of NaN and identical,
  byte for byte;
- so is every written pool slot: the ring and indexer-tail slots of each state,
  and every sealed block's entries and indexer keys.
A kernel that read a slot never written would put NaN into its results. One whose
result depended on timing (a race between workgroups) would differ between the
two runs. The measured storage is covered, and so are the low-bit formats (FP8
ring, HCA and C4 entries with MXFP4 indexer keys) and eager C4.
"""

import numpy as np
import pytest

import synth
from synth import workloads
from tests.gpu_util import dev_queries, dev_tokens

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import heterogeneous_sparse_attention_amd as hsa
    hsa.load()          # raises if the library is missing: no fallback


def say(msg):
    print(msg, flush=True)


def bf16_nan(bits):
    return (np.asarray(bits).view(np.uint16) & 0x7FFF) > 0x7F80


def run_once(entries, index, c4_mode, kv="bf16", steps=8):
    """One poisoned context through the b32 prefill and `steps` decode steps;
    returns the per-step results and every written pool slot, as host arrays."""
    import torch
    from heterogeneous_sparse_attention_amd import Cache
    wl = workloads.make(2)
    B, k = wl.batch, wl.topk
    L0 = wl.prefill.astype(np.int64)
    Wc, Wh = synth.gate_weights(wl.seed)
    nb = int(((L0 + steps) // 128).sum()) + B
    cache = Cache(wl.n_win, B, nb, Wc, Wh, entry_format=entries, index_format=index, c4_mode=c4_mode,
                  poison=True, kv_format=kv)
    try:
        st = [cache.state_alloc() for _ in range(B)]
        cu = np.concatenate([[0], np.cumsum(L0)])
        pos = np.concatenate([np.arange(n) for n in L0])
        keys = np.repeat(np.arange(B), L0)
        cache.append_kv(st, cu, *dev_tokens(wl.seed, keys, pos))
        res = []
        for t in range(steps):
            p = L0 + t
            topk = torch.empty((B, k), dtype=torch.int32, device="cuda")
            sc = torch.empty((B, k), dtype=torch.float32, device="cuda")
            out = torch.empty((B, 16, 128), dtype=torch.float32, device="cuda")
            cache.decode_step(st, *dev_tokens(wl.seed, np.arange(B), p), *dev_queries(wl.seed, np.arange(B), p),
                              k, topk_out=topk, score_out=sc, out=out, sorted=t >= steps - 2)
            res.append((topk.cpu().numpy(), sc.cpu().numpy(), out.cpu().numpy()))
        q, qi = dev_queries(wl.seed + 1, np.arange(B), L0)
        sc = torch.empty((B, 2048), dtype=torch.float32, device="cuda")
        idx, _ = cache.indexer_topk(st, qi, 2048, score_out=sc)
        out = cache.decode_attend(st, q, idx, 2048)
        res.append((idx.cpu().numpy(), sc.cpu().numpy(), out.cpu().numpy()))
        pools = {}
        for s in st:
            info = cache.state_query(s)
            L = info["len"]
            ex = cache.export_state(s)
            ring = np.arange(L - info["swa_len"], L) % wl.n_win
            if kv == "fp8":
                pools[("ring_k", s)] = ex["swa_k_codes"][ring]
                pools[("ring_v", s)] = ex["swa_v_codes"][ring]
                pools[("ring_ks", s)] = ex["swa_k_scale"][ring]
                pools[("ring_vs", s)] = ex["swa_v_scale"][ring]
            else:
                pools[("ring_k", s)] = ex["swa_k"][ring]
                pools[("ring_v", s)] = ex["swa_v"][ring]
            pools[("tail", s)] = ex["idx_tail"][np.arange(L - info["hca_tail"], L) % 128]
            pools[("table", s)] = np.array(cache.block_table(s))
            for lb, b in enumerate(cache.block_table(s)):
                for name, a in cache.export_block(b).items():
                    pools[(name, s, lb)] = a
        return res, pools
    finally:
        cache.close()


@pytest.mark.parametrize("entries,index,c4_mode,kv", [("bf16", "f32", "sealed", "bf16"),
                                                      ("fp8", "mxfp4", "sealed", "fp8"),
                                                      ("bf16", "f32", "eager", "bf16")])
def test_two_poisoned_runs_agree_byte_for_byte(entries, index, c4_mode, kv):
    r1, p1 = run_once(entries, index, c4_mode, kv)
    r2, p2 = run_once(entries, index, c4_mode, kv)
    for t, ((i1, s1, o1), (i2, s2, o2)) in enumerate(zip(r1, r2)):
        assert not np.isnan(o1).any() and not np.isnan(s1).any(), t
        assert np.array_equal(i1, i2), t
        assert s1.tobytes() == s2.tobytes(), t
        assert o1.tobytes() == o2.tobytes(), t
    assert p1.keys() == p2.keys()
    for key, a in p1.items():
        b = p2[key]
        assert a.tobytes() == b.tobytes(), key
        name = key[0]
        if a.dtype == np.uint16:                      # bf16 rows and entries
            assert not bf16_nan(a).any(), key
        elif a.dtype == np.float32:                   # indexer keys, FP8 scales
            assert not np.isnan(a).any(), key
        elif name in ("csa_k_codes", "csa_v_codes", "hca_k_codes", "hca_v_codes",
                      "ring_k", "ring_v") and a.dtype == np.uint8:   # E4M3 NaN codes
            assert not ((a & 0x7F) == 0x7F).any(), key
        elif name == "idx_scales":                    # E8M0 NaN
            assert not (a == 0xFF).any(), key
    say(f"{entries}/{index}/{c4_mode}: {len(r1)} results and {len(p1)} pool arrays identical, no NaN")
