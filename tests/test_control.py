"""Host control plane (C++, run on the CPU through libhsa_host.so) against the
oracle's integer state: State slots, block ids, tables, refcounts, lengths and
error codes must match bit for bit on random operation sequences."""

import os
import subprocess

import numpy as np
import pytest

from heterogeneous_sparse_attention_amd import build
from heterogeneous_sparse_attention_amd.host import HostControl
from oracle import Oracle, OracleError

CODE = {"invalid": -1, "oom_blocks": -2, "oom_states": -3, "state": -4}
Z = np.zeros((16, 128), np.float32)


def zeros(n):
    return (np.zeros((n, 16, 128)), np.zeros((n, 16, 128)), np.zeros((n, 4, 64)))


def run_oracle(fn):
    try:
        return 0, fn()
    except OracleError as e:
        return CODE[e.kind], None


def compare(o, h, live, max_blocks):
    for s in live:
        info = o.info(s)
        r, (L, nb, pend) = h.query(s)
        assert r == 0
        assert (L, nb) == (info["len"], info["n_blocks"])
        assert pend == int(info["hca_tail"] == 128)
        assert h.table(s) == o.table(s)
    for b in range(max_blocks):
        assert h.refcount(b) == o.refcount[b]
    assert h.free_blocks() == len(o.free_blocks)


@pytest.mark.parametrize("seed", range(6))
def test_control_matches_oracle(seed):
    rng = np.random.default_rng(seed)
    n_win, max_states, max_blocks = 256, 6, 24
    o = Oracle(n_win, Z, Z, max_states, max_blocks)
    h = HostControl(n_win, max_states, max_blocks)
    live, held = [], []
    for op in range(160):
        kind = int(rng.integers(8))
        if kind == 0:
            ro, so = run_oracle(o.state_alloc)
            rh, sh = h.state_alloc()
            assert ro == rh
            if ro == 0:
                assert so == sh
                live.append(so)
        elif kind == 1 and live:
            s = live.pop(int(rng.integers(len(live))))
            assert run_oracle(lambda: o.state_free(s))[0] == h.state_free(s) == 0
        elif kind in (2, 3) and live:
            sel = [s for s in live if rng.random() < 0.6]
            if rng.random() < 0.1 and sel:
                sel = sel + sel[:1]                      # duplicate -> invalid
            counts = [int(rng.integers(0, 300)) for _ in sel]
            defer = kind == 3
            if defer:
                counts = [int(rng.integers(0, 140)) for _ in sel]
            ro, _ = run_oracle(lambda: o.append(sel, [zeros(n) for n in counts], defer_seal=defer))
            rh, seals = h.append(sel, counts, defer)
            assert ro == rh, (ro, rh)
            if rh == 0:
                # seals: lowest free ids, requests in call order, blocks in token order
                for st, lb, sid in seals:
                    assert o.table(st)[lb] == sid
        elif kind == 4 and live:
            sel = [s for s in live if rng.random() < 0.7]
            assert run_oracle(lambda: o.compress_flush(sel))[0] == h.flush(sel)
        elif kind == 5 and len(live) >= 2:
            a, b = (int(x) for x in rng.choice(live, 2))
            assert run_oracle(lambda: o.share(a, b))[0] == h.share(a, b)
        elif kind == 6 and len(live) >= 2:
            # prefix hit: attach to a (prefix of a) live state's blocks, then fill the
            # window in the oracle (the host plane does not track filling)
            a, d = (int(x) for x in rng.choice(live, 2))
            blocks = o.table(a)
            n = int(rng.integers(0, len(blocks) + 1))
            length = 128 * n + int(rng.integers(0, 128)) if rng.random() < 0.9 else 128 * (n + 1)
            ro, _ = run_oracle(lambda: o.prefix_attach(d, blocks, length))
            assert ro == h.attach(d, blocks, length), (ro, length, n)
            if ro == 0:
                m = min(length, n_win)
                o.state_write([d], [zeros(m)], [length - m])
        elif kind == 7:
            if held and rng.random() < 0.5:
                blocks = held.pop(int(rng.integers(len(held))))
                delta = -1
            else:
                pool = [b for s in live for b in o.table(s)]
                blocks = [int(x) for x in rng.choice(pool, int(rng.integers(1, 4)))] if pool else [0]
                if rng.random() < 0.1:
                    blocks = blocks + [int(rng.integers(max_blocks))]   # maybe a free one -> invalid
                delta = 1
            ro, _ = run_oracle(lambda: o.block_ref(blocks, delta))
            assert ro == h.block_ref(blocks, delta)
            if ro == 0 and delta == 1:
                held.append(blocks)
            elif ro != 0 and delta == -1:
                held.append(blocks)
        compare(o, h, live, max_blocks)


def test_lowest_free_block_order():
    h = HostControl(128, 4, 8)
    _, a = h.state_alloc()
    _, b = h.state_alloc()
    assert h.append([a, b], [256, 128])[1] == [(a, 0, 0), (a, 1, 1), (b, 0, 2)]
    assert h.state_free(a) == 0
    assert h.append([b], [200])[1] == [(b, 1, 0)]          # lowest free id is 0 again
    assert h.table(b) == [2, 0]


def test_failed_calls_change_nothing():
    h = HostControl(128, 2, 3)
    _, a = h.state_alloc()
    _, b = h.state_alloc()
    assert h.state_alloc()[0] == -3
    assert h.append([a], [300])[0] == 0                     # 2 blocks
    assert h.append([a, b], [10, 256])[0] == -2             # needs 2, 1 free
    assert h.query(a)[1] == (300, 2, 0) and h.query(b)[1] == (0, 0, 0)
    assert h.append([b], [128], defer=True)[0] == 0
    assert h.query(b)[1] == (128, 0, 1)
    assert h.append([b], [1])[0] == -4                      # full deferred tail
    assert h.share(b, a) == -4                              # dst not empty
    assert h.flush([b]) == 0 and h.query(b)[1] == (128, 1, 0)
    assert h.state_free(7) == -1


def test_control_selftest_with_sanitizers(tmp_path):
    exe = build.build_selftest(str(tmp_path / "selftest"))
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "control selftest ok" in r.stdout


# ------------------------------------------------------------------ launch planning

def _brute_min_max(keys, lat, mins, slots, min_keys=16):
    """Smallest achievable largest estimate lat + keys / wgs over every assignment of
    at most `slots` workgroups (each item between its floor and its split cap)."""
    import itertools
    lo = [max(1 if k > 0 else 0, m) for k, m in zip(keys, mins)]
    hi = [max(l, k // min_keys) if k >= 2 * min_keys else l for k, l in zip(keys, lo)]
    best = None
    for w in itertools.product(*[range(a, b + 1) for a, b in zip(lo, hi)]):
        if sum(w) > max(slots, sum(lo)):
            continue
        t = max((la + k / x) if x else 0.0 for k, la, x in zip(keys, lat, w))
        best = t if best is None else min(best, t)
    return best


@pytest.mark.parametrize("seed", range(6))
def test_balance_wgs_is_optimal_on_small_cases(seed):
    """The planner's greedy hand-out reaches the smallest possible largest estimate
    (brute force over every assignment), never gives a workgroup fewer than 16 keys
    of a splittable item, and gives every request with keys a workgroup."""
    from heterogeneous_sparse_attention_amd.host import balance_wgs
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 4))
    ka = rng.integers(0, 120, n)
    kb = rng.integers(0, 120, n)
    slots = int(rng.integers(1, 12))
    lat_b = int(rng.integers(0, 20))
    used, wa, wb = balance_wgs(slots, ka, 0, 0, kb, lat_b, 1)
    assert used == wa.sum() + wb.sum()
    assert np.all(wb >= 1) and np.all((ka == 0) | (wa >= 1))
    floor = int(((ka > 0).sum()) + n)
    assert used <= max(slots, floor)
    for k, w in list(zip(ka, wa)) + list(zip(kb, wb)):
        assert w <= max(1, k // 16)
    est = max([k / w for k, w in zip(ka, wa) if w] + [lat_b + k / w for k, w in zip(kb, wb)])
    ref = _brute_min_max(list(ka) + list(kb), [0] * n + [lat_b] * n, [0] * n + [1] * n, slots)
    assert abs(est - ref) < 1e-9, (est, ref)


def _greedy(slots, parts):
    """One slot at a time to the (part, request) with the largest lat + keys / w that
    can still split (keys >= 16 (w + 1)); parts = [(keys, lat, min_wgs)]."""
    import heapq
    ws, heap, used = [], [], 0
    for p, (keys, lat, mn) in enumerate(parts):
        w = [max(1 if k > 0 else 0, mn) for k in keys]
        used += sum(w)
        ws.append(w)
        for i, k in enumerate(keys):
            if w[i] > 0 and k >= 16 * (w[i] + 1):
                heapq.heappush(heap, (-(lat + k / w[i]), p, i))
    while used < slots and heap:
        _, p, i = heapq.heappop(heap)
        keys, lat, _ = parts[p]
        ws[p][i] += 1
        used += 1
        if keys[i] >= 16 * (ws[p][i] + 1):
            heapq.heappush(heap, (-(lat + keys[i] / ws[p][i]), p, i))
    return used, ws


@pytest.mark.parametrize("seed", range(8))
def test_balance_wgs_matches_the_greedy_hand_out(seed):
    """The planner starts every item at a feasible share and hands out the rest one
    at a time; it must end where the one-at-a-time greedy ends: same workgroups used
    and the same largest estimate (b32-like and long-request sizes, two parts)."""
    from heterogeneous_sparse_attention_amd.host import balance_wgs
    rng = np.random.default_rng(100 + seed)
    for _ in range(40):
        n = int(rng.integers(1, 41))
        ka = rng.integers(0, 3000, n) * (rng.random(n) > 0.2)
        kb = rng.integers(0, 1500, n)
        slots = int(rng.integers(1, 600))
        lat_b = int(rng.integers(0, 50))
        used, wa, wb = balance_wgs(slots, ka, 0, 0, kb, lat_b, 1)
        g_used, (ga, gb) = _greedy(slots, [(ka, 0, 0), (kb, lat_b, 1)])
        assert used == g_used
        est = max([k / w for k, w in zip(ka, wa) if w] + [lat_b + k / w for k, w in zip(kb, wb)])
        g_est = max([k / w for k, w in zip(ka, ga) if w] + [lat_b + k / w for k, w in zip(kb, gb)])
        assert abs(est - g_est) <= 1e-9 * max(1.0, g_est)


def test_balance_wgs_fills_the_launch():
    """b32-like sizes: the planner hands out exactly the slots when work allows."""
    from heterogeneous_sparse_attention_amd.host import balance_wgs
    rng = np.random.default_rng(7)
    keys = rng.integers(130, 700, 32)
    used, w, _ = balance_wgs(256, keys, 0, 1)
    assert used == 256 and w.sum() == 256 and np.all(w >= 1)
    t = keys / w
    assert t.max() <= np.sort(t)[-2] * 1.5 + 1


def test_plan_slices():
    """Rows longer than the slice and than k1 are cut into ceil(n / slice) slices;
    the default slice is max(16384, 16 k1); first[] is the workgroup prefix."""
    from heterogeneous_sparse_attention_amd.host import plan_slices
    first, gmax, sl, k1 = plan_slices([262144, 100, 16384, 16385], 2048)
    assert (sl, k1) == (32768, 2048)
    assert list(first) == [0, 8, 9, 10, 11] and gmax == 8
    first, gmax, sl, k1 = plan_slices([9600, 1280, 1280], 777, slice_override=1024)
    assert (sl, k1) == (1024, 780)
    assert list(first) == [0, 10, 12, 14] and gmax == 10
    # a row no longer than k1 stays whole even when it is longer than the slice
    first, gmax, _, k1 = plan_slices([2048, 4096], 4096, slice_override=1024)
    assert k1 == 4096 and list(first) == [0, 1, 2] and gmax == 1
    first, gmax, sl, _ = plan_slices([16384, 16416], 512)
    assert sl == 16384 and list(first) == [0, 1, 3] and gmax == 2
