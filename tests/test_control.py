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
    live = []
    for op in range(120):
        kind = int(rng.integers(6))
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
