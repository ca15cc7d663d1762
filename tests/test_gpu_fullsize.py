"""GPU parity at the workloads' full sizes, in the launch configuration the bench
times (one hsa_decode_step per step over the whole batch, default launch shapes).

- b32 (32 requests, L0 up to 8192, 64 steps): every step of every request against
  the oracle driven token by token.
- long (4 requests of 2**20 tokens, k 2048, 16 steps across a block boundary) and
  prefix (64 requests of 16K-64K tokens sharing 8 prefixes by fork, n_win 4096,
  k 1024, 32 steps): every request's full top-k row and attention output against
  tests/golden/*_decode.npz (every step of the long workload; steps 0, 10, 21 and
  31 of the prefix workload), which tests/golden/make_fullsize.py writes with the
  oracle alone. Also: integer state and refcounts exactly, the selected scores
  exactly against the oracle's scores of those entries, the selection against the
  oracle's scores of sampled blocks, the rings and tails, and at least 64 sealed
  blocks per request against the oracle's compressor. The sampled blocks always
  include the first and the last, the block sealed during the decode steps, and
  the first and last shared-prefix blocks.
- prefix again with FP8 KV storage (reading R20: every ring token and HCA entry
  as per-head E4M3 codes and scales; the SWA alone is 2 GiB of codes per step):
  every request's top-k row and output at steps 0 and 31 against
  tests/golden/prefix_decode_fp8kv.npz, ring codes and scales bit for bit, and the
  sampled blocks' HCA codes by the FP8 rule of tests/gpu_util.py (check_fp8).
- bulk (8 x 131072 tokens in one append): state, tables, sampled blocks, rings.
"""

import os

import numpy as np
import pytest

import synth
from oracle import BLOCK, C4_PER_BLOCK, M_CSA, Oracle, gated_pool, token_scores
from synth.workloads import RequestTokens, make
from tests.gpu_util import bf16_to_f64, check_fp8, dev_rows, pool_magnitude, rel_l2

pytestmark = pytest.mark.gpu

TOL = 1e-3
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import heterogeneous_sparse_attention_amd as hsa
    hsa.load()          # raises if the library is missing: no fallback


def say(msg):
    print(msg, flush=True)


# ------------------------------------------------------------------ oracle-side helpers

def entry_scores(src, ordinals, q_idx):
    """Oracle scores of the C4 entries `ordinals` of one request (reading R4)."""
    ordinals = np.asarray(ordinals, np.int64)
    pos = (M_CSA * ordinals[:, None] + np.arange(M_CSA)).reshape(-1)
    _, _, KI = src(pos)
    return token_scores(KI, q_idx).reshape(-1, M_CSA).sum(axis=1) / 4.0


def check_selection(src, idx, val, nb, k, q_idx, sample_blocks):
    """One request's top-k row against the oracle: kk valid ascending ordinals, -1
    after; the returned scores equal the oracle's scores of those entries; and on
    the sampled blocks no unselected entry beats the cut (ties go to the lowest
    ordinal)."""
    nc = C4_PER_BLOCK * nb
    kk = min(k, nc)
    assert np.all(idx[kk:] == -1) and np.all(np.isneginf(val[kk:]))
    sel = idx[:kk].astype(np.int64)
    assert np.all(sel >= 0) and np.all(sel < nc) and np.all(np.diff(sel) > 0)
    ref = entry_scores(src, sel, q_idx)
    assert np.array_equal(val[:kk].astype(np.float64), ref)
    if kk == nc:
        return
    tau = ref.min()
    tie_max = sel[ref == tau].max()
    chosen = set(sel.tolist())
    for lb in sample_blocks:
        if lb >= nb:
            continue
        js = np.arange(C4_PER_BLOCK * lb, C4_PER_BLOCK * (lb + 1))
        s = entry_scores(src, js, q_idx)
        for j, sj in zip(js.tolist(), s.tolist()):
            if j in chosen:
                continue
            assert sj <= tau, (j, sj, tau)
            if sj == tau:
                assert j > tie_max, (j, tie_max)


def expected_block(index, b, lb, gates, kv="bf16"):
    """The oracle's entries of sealed block lb of request b of a workload: bf16-rounded
    C4 and HCA entries (float32) and the block's indexer keys. With FP8 KV (reading
    R20) the tokens are their stored values, and the HCA entry is given as the
    unquantised pooled value (hca_k_x, hca_v_x) with its E4M3 codes and scales."""
    from oracle import quantize_e4m3_rows
    Wc, Wh = gates
    K, V, KI = RequestTokens(index, b)(np.arange(BLOCK * lb, BLOCK * (lb + 1)))
    if kv == "fp8":
        K, V = quantize_e4m3_rows(K)[2], quantize_e4m3_rows(V)[2]
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    ck = np.empty((C4_PER_BLOCK, 16, 128), np.float32)
    cv = np.empty_like(ck)
    for j in range(C4_PER_BLOCK):
        ck[j], cv[j] = gated_pool(K[M_CSA * j:M_CSA * (j + 1)], V[M_CSA * j:M_CSA * (j + 1)], Wc)
    ref = {"csa_k": ck, "csa_v": cv, "idx": KI}
    if kv == "fp8":
        hk, hv = gated_pool(K, V, Wh, rounded=False)
        mags = pool_magnitude(K, V, Wh)
        for n, x, m in (("k", hk, mags[0]), ("v", hv, mags[1])):
            codes, scale, _ = quantize_e4m3_rows(x)
            ref[f"hca_{n}_x"], ref[f"hca_{n}_codes"], ref[f"hca_{n}_scale"] = x, codes, scale
            ref[f"hca_{n}_mag"] = m
        return ref
    hk, hv = gated_pool(K, V, Wh)
    ref["hca_k"], ref["hca_v"] = hk.astype(np.float32), hv.astype(np.float32)
    return ref


def _expected_block_job(job):
    return expected_block(*job)


def compare_block(g, ref, where):
    if "hca_k_x" in ref:   # FP8 KV: the HCA codes by the FP8 rule
        for n in ("k", "v"):
            check_fp8(g[f"hca_{n}_codes"], g[f"hca_{n}_scale"], ref[f"hca_{n}_codes"], ref[f"hca_{n}_scale"],
                      ref[f"hca_{n}_x"], ("hca", n, where), ref[f"hca_{n}_mag"])
    for name in ("csa_k", "csa_v") if "hca_k_x" in ref else ("csa_k", "csa_v", "hca_k", "hca_v"):
        val = bf16_to_f64(g[name])
        r = ref[name].astype(np.float64)
        assert rel_l2(val, r) <= TOL, (name, where, rel_l2(val, r))
        assert np.mean(val == r) > 0.97, (name, where)
    assert np.array_equal(g["idx"], ref["idx"]), where


def check_block(cache, block_id, src, lb, gates):
    """A sealed block's device entries against the oracle's compressor of its tokens."""
    compare_block(cache.export_block(block_id), expected_block(src.index, src.b, lb, gates), (src.b, lb))


def check_blocks(cache, items, index, gates, workers=None, kv="bf16"):
    """Check many sealed blocks: items = [(physical id, request, logical block)], each
    physical id once. The oracle's entries come from worker processes (spawned: they
    never touch the GPU), the device's from hsa_export_block."""
    import multiprocessing as mp
    workers = workers or max(1, min(16, len(os.sched_getaffinity(0))))
    jobs = [(index, b, lb, gates, kv) for _, b, lb in items]
    with mp.get_context("spawn").Pool(workers) as pool:
        for (bid, b, lb), ref in zip(items, pool.imap(_expected_block_job, jobs, chunksize=4)):
            compare_block(cache.export_block(bid), ref, (b, lb))
    return len(items)


def sample_blocks(rng, nb, must, n=64):
    """At least n distinct logical blocks of [0, nb) (all of them if fewer), always
    including `must`."""
    picks = {x for x in must if 0 <= x < nb}
    extra = rng.permutation(nb)
    i = 0
    while len(picks) < min(n, nb):
        picks.add(int(extra[i]))
        i += 1
    return sorted(picks)


def check_ring(cache, state, src, L, n_win, kv="bf16"):
    ex = cache.export_state(state)
    p = np.arange(max(0, L - n_win), L)
    K, V, KI = src(p)
    if kv == "fp8":   # reading R20: each token's per-head codes and scales, bit for bit
        from oracle import quantize_e4m3_rows
        for n, x in (("k", K), ("v", V)):
            codes, scale, _ = quantize_e4m3_rows(x)
            assert np.array_equal(ex[f"swa_{n}_codes"][p % n_win], codes)
            assert np.array_equal(ex[f"swa_{n}_scale"][p % n_win], scale)
    else:
        assert np.array_equal(bf16_to_f64(ex["swa_k"][p % n_win]), K)
        assert np.array_equal(bf16_to_f64(ex["swa_v"][p % n_win]), V)
    t = np.arange(L - L % BLOCK, L)
    assert np.array_equal(ex["idx_tail"][t % BLOCK], KI[len(p) - len(t):])


def check_info(cache, state, L):
    info = cache.state_query(state)
    assert info["len"] == L and info["n_blocks"] == L // BLOCK
    assert info["hca_tail"] == L % BLOCK and info["csa_tail"] == L % M_CSA


def load_golden(name):
    with np.load(os.path.join(GOLDEN, name), allow_pickle=False) as z:
        return {k: z[k] for k in z.files}


def step_inputs(wl, reqs, L0, t):
    """Device inputs of decode step t: the token at position L0[b] + t of each request,
    keyed as the workload keys it."""
    pos = np.array([int(L0[b]) + t for b in reqs], np.int64)
    keys = np.array([int(wl.key(b, p)) for b, p in zip(reqs, pos)], np.int64)
    return (dev_rows(wl.seed, synth.STREAM_K, keys, pos, True),
            dev_rows(wl.seed, synth.STREAM_V, keys, pos, True),
            dev_rows(wl.seed, synth.STREAM_IDXK, keys, pos, False),
            dev_rows(wl.seed, synth.STREAM_Q, keys, pos, True),
            dev_rows(wl.seed, synth.STREAM_QI, keys, pos, False))


def run_steps(cache, states, wl, L0, steps, on_step):
    import torch
    B, k = len(states), wl.topk
    topk = torch.empty((B, k), dtype=torch.int32, device="cuda")
    sc = torch.empty((B, k), dtype=torch.float32, device="cuda")
    out = torch.empty((B, 16, 128), dtype=torch.float32, device="cuda")
    for t in range(steps):
        kn, vn, ikn, q, qi = step_inputs(wl, list(range(B)), L0, t)
        cache.decode_step(states, kn, vn, ikn, q, qi, k, topk_out=topk, score_out=sc, out=out)
        torch.cuda.synchronize()
        on_step(t, topk.cpu().numpy(), sc.cpu().numpy(), out.cpu().numpy())


def check_golden_rows(gold, b, t, idx, out):
    hit = np.nonzero((gold["req"] == b) & (gold["step"] == t))[0]
    for i in hit:
        assert np.array_equal(idx, gold["idx"][i]), (b, t)
        assert rel_l2(out, gold["out"][i]) <= TOL, (b, t, rel_l2(out, gold["out"][i]))
    return len(hit)


# ------------------------------------------------------------------ b32

B32_MODES = [("bf16", "f32", "sealed", 64, "bf16"), ("fp8", "mxfp4", "sealed", 16, "fp8"),
             ("bf16", "f32", "eager", 16, "bf16")]


@pytest.mark.parametrize("entries,index,c4_mode,steps,kv", B32_MODES)
def test_b32_every_step_against_oracle(entries, index, c4_mode, steps, kv):
    """Every step of every request; besides the measured storage, the pages' own
    (FP8 SWA ring, HCA and C4 entries, MXFP4 indexer keys) and eager C4 for 16
    steps each."""
    import bench
    wl = make(2)
    B, k = wl.batch, wl.topk
    L0 = wl.prefill.astype(np.int64)
    cache, inst = bench.setup_decode(wl, steps, 1, entries, index, None, c4_mode, kv)
    states = inst[0]
    say(f"b32 ({entries}, {index}, {c4_mode}, kv {kv}): prefilled {int(L0.sum())} tokens on the GPU")
    Wc, Wh = synth.gate_weights(wl.seed)
    o = Oracle(wl.n_win, Wc, Wh, B, int(((L0 + steps) // BLOCK).sum()) + B, entry_format=entries,
               index_format=index, c4_mode=c4_mode, kv_format=kv)
    srcs = [RequestTokens(2, b) for b in range(B)]
    ost = []
    for b in range(B):
        s = o.state_alloc()
        o.append([s], [srcs[b](np.arange(L0[b]))])
        ost.append(s)
    say("b32: oracle prefilled")
    worst = [0.0]

    def on_step(t, topk, sc, out):
        for b in range(B):
            p = int(L0[b]) + t
            K, V, KI = srcs[b](np.array([p]))
            o.append([ost[b]], [(K, V, KI)])
            q, qi = srcs[b].query(p)
            idx, val = o.topk(ost[b], qi, k)
            assert np.array_equal(topk[b], idx), (t, b)
            assert np.array_equal(sc[b].astype(np.float64), val), (t, b)
            r = rel_l2(out[b], o.attend(ost[b], q, idx, k))
            assert r <= TOL, (t, b, r)
            worst[0] = max(worst[0], r)

    run_steps(cache, states, wl, L0, steps, on_step)
    for b in range(B):
        check_info(cache, states[b], int(L0[b]) + steps)
    say(f"b32: {steps} steps x {B} requests match; worst rel L2 {worst[0]:.2e}")
    cache.close()


# ------------------------------------------------------------------ long

def test_long_context_full_size():
    import bench
    wl = make(5)
    B, k, steps = wl.batch, wl.topk, wl.decode_steps
    L0 = wl.prefill.astype(np.int64)
    cache, inst = bench.setup_decode(wl, steps, 1)
    states = inst[0]
    say(f"long: prefilled {B} x {int(L0[0])} tokens on the GPU")
    gold = load_golden("long_decode.npz")
    srcs = [RequestTokens(5, b) for b in range(B)]
    rng = np.random.default_rng(wl.seed + 7)
    checked = [0]

    def on_step(t, topk, sc, out):
        for b in range(B):
            L = int(L0[b]) + t + 1
            nb = L // BLOCK
            check_info(cache, states[b], L)
            _, qi = srcs[b].query(L - 1)
            sample = sorted({0, nb // 2, nb - 2, nb - 1, *rng.integers(0, nb, 4).tolist()})
            check_selection(srcs[b], topk[b], sc[b], nb, k, qi, sample)
            checked[0] += check_golden_rows(gold, b, t, topk[b], out[b])
        say(f"long: step {t} ok")

    run_steps(cache, states, wl, L0, steps, on_step)
    assert checked[0] == len(gold["req"]) == B * steps
    gates = synth.gate_weights(wl.seed)
    items = []
    for b in range(B):
        table = cache.block_table(states[b])
        nb = len(table)
        # the first, second, middle and last blocks and the block sealed by step 8
        must = {0, 1, nb // 2, nb - 2, nb - 1, int(L0[b]) // BLOCK}
        items += [(table[lb], b, lb) for lb in sample_blocks(rng, nb, must)]
        check_ring(cache, states[b], srcs[b], int(L0[b]) + steps, wl.n_win)
    n = check_blocks(cache, items, 5, gates)
    say(f"long: {n} sampled blocks (at least 64 per request) and every ring ok")
    cache.close()


# ------------------------------------------------------------------ prefix

@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_prefix_sharing_full_size(kv):
    import torch

    from heterogeneous_sparse_attention_amd import Cache
    wl = make(3)
    B, k, steps = wl.batch, wl.topk, wl.decode_steps
    L0 = wl.prefill.astype(np.int64)
    Wc, Wh = synth.gate_weights(wl.seed)
    max_len = wl.max_len()
    cache = Cache(wl.n_win, B + wl.n_groups, wl.max_blocks_total() + 64, Wc, Wh,
                  max_blocks_per_state=max_len // BLOCK + 2, kv_format=kv)
    states = [None] * B
    fork = {b: wl.fork_len(b) for b in range(B)}

    def append(sts, reqs, p0s, p1s):
        """Append positions [p0, p1) of each request, in pieces of at most 64K tokens."""
        i = 0
        while i < len(reqs):
            grp, tot = [], 0
            while i < len(reqs) and (tot + p1s[i] - p0s[i] <= 65536 or not grp):
                grp.append(i)
                tot += p1s[i] - p0s[i]
                i += 1
            pos = np.concatenate([np.arange(p0s[j], p1s[j]) for j in grp]).astype(np.int64)
            keys = np.concatenate([wl.key(reqs[j], np.arange(p0s[j], p1s[j])) for j in grp])
            keys = keys.astype(np.int64)
            cu = np.concatenate([[0], np.cumsum([p1s[j] - p0s[j] for j in grp])]).astype(np.int64)
            K = dev_rows(wl.seed, synth.STREAM_K, keys, pos, True)
            V = dev_rows(wl.seed, synth.STREAM_V, keys, pos, True)
            KI = dev_rows(wl.seed, synth.STREAM_IDXK, keys, pos, False)
            cache.append_kv([sts[j] for j in grp], cu, K, V, KI)
            del K, V, KI

    # each group's parent grows through the shared prefix; children fork from it
    for g in range(wl.n_groups):
        kids = sorted((b for b in range(B) if wl.group(b) == g), key=lambda b: fork[b])
        parent = cache.state_alloc()
        cur = 0
        for b in kids:
            if fork[b] > cur:
                append([parent], [b], [cur], [fork[b]])
                cur = fork[b]
            states[b] = cache.state_alloc()
            cache.block_table_share(parent, states[b])
        cache.state_free(parent)
    append(states, list(range(B)), [fork[b] for b in range(B)], [int(L0[b]) for b in range(B)])
    torch.cuda.synchronize()
    say(f"prefix (kv {kv}): forks and prefills done")

    # shared blocks: one physical copy per group, refcount = number of sharers
    for g in range(wl.n_groups):
        kids = [b for b in range(B) if wl.group(b) == g]
        tabs = {b: cache.block_table(states[b]) for b in kids}
        for lb in range(wl.prefix_len // BLOCK):
            users = [b for b in kids if fork[b] > BLOCK * lb]
            if not users:
                continue
            ids = {tabs[b][lb] for b in users}
            assert len(ids) == 1, (g, lb, ids)
            assert cache.refcount(ids.pop()) == len(users)

    gold = load_golden("prefix_decode.npz" if kv == "bf16" else "prefix_decode_fp8kv.npz")
    gold_steps = set(gold["step"].tolist())
    srcs = {b: RequestTokens(3, b) for b in range(B)}
    rng = np.random.default_rng(wl.seed + 7)
    checked = [0]

    def on_step(t, topk, sc, out):
        for b in range(B):
            L = int(L0[b]) + t + 1
            check_info(cache, states[b], L)
            if t in gold_steps or t == steps - 1:
                nb = L // BLOCK
                _, qi = srcs[b].query(L - 1)
                sample = sorted({0, nb - 1, *rng.integers(0, nb, 3).tolist()})
                check_selection(srcs[b], topk[b], sc[b], nb, k, qi, sample)
            checked[0] += check_golden_rows(gold, b, t, topk[b], out[b])
        if t % 8 == 7:
            say(f"prefix (kv {kv}): step {t} ok")

    run_steps(cache, states, wl, L0, steps, on_step)
    assert checked[0] == len(gold["req"]) == B * len(gold_steps)
    gates = (Wc, Wh)
    items, seen = [], set()
    for b in range(B):
        table = cache.block_table(states[b])
        nb = len(table)
        shared = fork[b] // BLOCK            # blocks [0, shared) are the group's prefix
        # the first and last blocks, the first and last shared-prefix blocks, the
        # first block of its own, and the block sealed during the decode steps
        must = {0, nb - 1, shared - 1, shared, int(L0[b]) // BLOCK}
        for lb in sample_blocks(rng, nb, must):
            if table[lb] not in seen:        # a shared block is checked once
                seen.add(table[lb])
                items.append((table[lb], b, lb))
        if b < wl.n_groups:                  # one ring per group
            check_ring(cache, states[b], srcs[b], int(L0[b]) + steps, wl.n_win, kv)
    n = check_blocks(cache, items, 3, gates, kv=kv)
    say(f"prefix (kv {kv}): {n} distinct sampled blocks (at least 64 per request) and rings ok")
    cache.close()


# ------------------------------------------------------------------ bulk

def test_bulk_append_full_size():
    import torch

    from heterogeneous_sparse_attention_amd import Cache
    wl = make(4)
    B, n = wl.batch, int(wl.prefill[0])
    Wc, Wh = synth.gate_weights(wl.seed)
    nbq = n // BLOCK
    cache = Cache(wl.n_win, B, B * nbq, Wc, Wh, max_blocks_per_state=nbq)
    states = [cache.state_alloc() for _ in range(B)]
    pos = np.tile(np.arange(n, dtype=np.int64), B)
    keys = np.repeat(np.arange(B, dtype=np.int64), n)
    K = dev_rows(wl.seed, synth.STREAM_K, keys, pos, True)
    V = dev_rows(wl.seed, synth.STREAM_V, keys, pos, True)
    KI = dev_rows(wl.seed, synth.STREAM_IDXK, keys, pos, False)
    cache.append_kv(states, np.arange(B + 1, dtype=np.int64) * n, K, V, KI)   # one call
    torch.cuda.synchronize()
    del K, V, KI
    say(f"bulk: appended {B} x {n} tokens in one call")
    gates = (Wc, Wh)
    rng = np.random.default_rng(wl.seed + 7)
    for b in range(B):
        check_info(cache, states[b], n)
        table = cache.block_table(states[b])
        # lowest free ids, requests in call order, blocks in token order (reading R10)
        assert table == list(range(b * nbq, (b + 1) * nbq))
        assert all(cache.refcount(i) == 1 for i in (table[0], table[-1]))
        src = RequestTokens(4, b)
        for lb in sorted({0, nbq // 2, nbq - 1, *rng.integers(0, nbq, 2).tolist()}):
            check_block(cache, table[lb], src, lb, gates)
        if b in (0, B - 1):
            check_ring(cache, states[b], src, n, wl.n_win)
    say("bulk: state, tables, sampled blocks and rings ok")
    cache.close()
