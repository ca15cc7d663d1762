"""GPU parity with narrow launches: 16 attention workgroups per step launch and per
hsa_decode_attend call, so that each wave of a workgroup streams well over 64 keys.
That runs the attention's later 64-key address groups, long key rings and, with
mixed storage (FP8 KV with bf16 entries, or the reverse), waves whose key list
changes format inside a group. Both step forms and every pair of KV and entry
formats: top-k exact, attention within rel L2 1e-3 of the oracle, and the
standalone call on the same selection.
"""

import numpy as np
import pytest

import synth
from oracle import Oracle
from tests.test_gpu_fp8_kv import prefill
from tests.gpu_util import rel_l2

pytestmark = pytest.mark.gpu

TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import heterogeneous_sparse_attention_amd as hsa
    hsa.load()          # raises if the library is missing: no fallback


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("entries", ["bf16", "fp8"])
def test_narrow_launches_match_oracle(monkeypatch, entries, kv):
    """One oracle, two caches: the three-launch and the four-launch step form (the
    form is fixed when a context is created)."""
    import heterogeneous_sparse_attention_amd as hsa
    monkeypatch.setenv("HSA_STEP_SLOTS", "16")
    monkeypatch.setenv("HSA_ATTEND_WGS", "16")
    seed = 0x4A7
    rng = np.random.default_rng(seed)
    B = 8
    # rows of 1050-1300 C4 entries: k = 1024 still fits the three-launch form's LDS
    # cache. 16 slots over 8 requests leave about two workgroups per request, so a
    # mixed workgroup holds its request's 1024 part-B keys (128 per wave), a k_step3
    # workgroup about 512 (4 waves) and a standalone attention workgroup about 600
    L0 = rng.integers(4200, 5200, B)
    Wc, Wh = synth.gate_weights(seed)
    nblk = int((L0 + 8).sum() // 128 + B)
    caches = []
    try:
        for fused in ("1", "0"):
            monkeypatch.setenv("HSA_STEP_FUSED", fused)
            caches.append(hsa.Cache(128, B, nblk, Wc, Wh, entry_format=entries, kv_format=kv))
        o = Oracle(128, Wc, Wh, B, nblk, entry_format=entries, kv_format=kv)
        st = prefill(caches[0], o, seed, L0)
        assert prefill_ids(caches[1], seed, L0) == st
        for step, k in enumerate((1024, 700)):
            p = L0 + step
            gpu = [step_gpu(c, seed, st, np.arange(B), p, k) for c in caches]
            ref_idx, ref_out, q = step_oracle(o, seed, st, np.arange(B), p, k)
            for form, (idx, out, att) in zip(("three-launch", "four-launch"), gpu):
                for i in range(B):
                    assert np.array_equal(idx[i], ref_idx[i]), (form, step, i)
                    r = rel_l2(out[i], ref_out[i])
                    assert r <= TOL, (form, step, i, r)
                    r = rel_l2(att[i], ref_out[i])
                    assert r <= TOL, (form, "attend", step, i, r)
    finally:
        for c in caches:
            c.close()


def prefill_ids(cache, seed, L0):
    """The GPU side of prefill() for a second cache (its states get the same ids)."""
    from tests.gpu_util import dev_tokens
    B = len(L0)
    st = [cache.state_alloc() for _ in range(B)]
    cu = np.concatenate([[0], np.cumsum(L0)])
    pos = np.concatenate([np.arange(n) for n in L0])
    cache.append_kv(st, cu, *dev_tokens(seed, np.repeat(np.arange(B), L0), pos))
    return st


def step_gpu(cache, seed, st, keys, p, k):
    """One decode step and the standalone attention on its selection."""
    from tests.gpu_util import dev_queries, dev_tokens
    Kn, Vn, KIn = dev_tokens(seed, keys, p)
    Q, QI = dev_queries(seed, keys, p)
    idx, _, out = cache.decode_step(st, Kn, Vn, KIn, Q, QI, k)
    att = cache.decode_attend(st, Q, idx, k)
    return idx.cpu().numpy(), out.cpu().numpy(), att.cpu().numpy()


def step_oracle(o, seed, st, keys, p, k):
    from tests.gpu_util import host_queries, host_tokens
    Kh, Vh, KIh = host_tokens(seed, keys, p)
    o.append(st, [(Kh[i:i + 1], Vh[i:i + 1], KIh[i:i + 1]) for i in range(len(st))])
    q, qi = host_queries(seed, keys, p)
    ref_idx, ref_out = [], []
    for i, s in enumerate(st):
        ridx, _ = o.topk(s, qi[i], k)
        ref_idx.append(ridx)
        ref_out.append(o.attend(s, q[i], ridx, k))
    return ref_idx, ref_out, q
