"""GPU parity of the FP8 C4 entry format (reading R15: per head, OCP E4M3 codes and
a float32 scale) against the CPU oracle.

- The quantisation alone (hsa_fp8_quantize_rows) on the same float32 rows as the
  oracle: codes and scales bit for bit, on rows built to hit exact ties of the
  E4M3 grid, the subnormal range, zero rows and a wide range of magnitudes.
- A ragged batch in an FP8 cache against the FP8 oracle: HCA entries and indexer
  keys as in bf16 mode; C4 codes and scales equal except where the float32 pooled
  value (GPU) and the rounded float64 one (oracle) fall on opposite sides of a
  rounding boundary; top-k bit exact; attention (both forms of the decode step
  and hsa_decode_attend) within relative L2 1e-3 of the oracle's FP8 attention.
"""

import numpy as np
import pytest

import synth
from oracle import Oracle, e4m3_decode, quantize_e4m3_rows
from tests.gpu_util import bf16_to_f64, dev_queries, dev_tokens, host_queries, host_tokens, rel_l2

pytestmark = pytest.mark.gpu

TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import heterogeneous_sparse_attention_amd as hsa
    hsa.load()          # raises if the library is missing: no fallback


def _tie_rows():
    """Rows whose largest magnitude is 448, so the multiplier is exactly 1 and the
    other values reach the encoder unchanged: every midpoint of the finite E4M3
    grid, values just off each midpoint, subnormal ties, both signs."""
    grid = e4m3_decode(np.arange(0x7F))
    mids = (grid[1:] + grid[:-1]) / 2
    vals = np.concatenate([mids, np.nextafter(mids.astype(np.float32), np.float32(np.inf)),
                           np.nextafter(mids.astype(np.float32), np.float32(0)), grid,
                           [2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -11, 2.0 ** -12, 1e-30]]).astype(np.float32)
    vals = np.concatenate([vals, -vals])
    n = -(-len(vals) // 127)
    rows = np.zeros((n, 128), np.float32)
    rows[:, 0] = 448.0
    flat = rows[:, 1:].reshape(-1)
    flat[:len(vals)] = vals
    rows[:, 1:] = flat.reshape(n, 127)
    return rows


def test_fp8_quantizer_matches_oracle_bit_exact():
    import torch
    import heterogeneous_sparse_attention_amd as hsa
    rng = np.random.default_rng(11)
    rand = (rng.standard_normal((512, 128)) * np.exp(rng.uniform(-20, 20, (512, 1)))).astype(np.float32)
    rows = np.concatenate([_tie_rows(), rand, np.zeros((3, 128), np.float32),
                           -np.abs(rand[:5]), np.full((2, 128), 1e-38, np.float32),
                           np.full((1, 128), 2e-36, np.float32)])
    for n in (len(rows), 1, 17):                      # ragged counts of 16-row workgroups
        x = torch.from_numpy(rows[:n].copy()).cuda()
        codes, scales = hsa.fp8_quantize_rows(x)
        rc, rs, _ = quantize_e4m3_rows(rows[:n])
        assert np.array_equal(scales.cpu().numpy(), rs), n
        got = codes.cpu().numpy()
        bad = np.argwhere(got != rc)
        assert bad.size == 0, (n, bad[:5], got[tuple(bad[0])], rc[tuple(bad[0])], rows[tuple(bad[0])])
    c0, s0 = hsa.fp8_quantize_rows(torch.zeros((0, 128), dtype=torch.float32, device="cuda"))
    assert c0.shape == (0, 128) and s0.shape == (0,)


def _pair(seed, n_win, max_states, max_blocks):
    import heterogeneous_sparse_attention_amd as hsa
    Wc, Wh = synth.gate_weights(seed)
    return (hsa.Cache(n_win, max_states, max_blocks, Wc, Wh, entry_format="fp8"),
            Oracle(n_win, Wc, Wh, max_states, max_blocks, entry_format="fp8"))


def _check_block(cache, o, bg, bo):
    g = cache.export_block(bg)
    r = o.block(bo)
    assert np.array_equal(bf16_to_f64(g["hca_k"]), r.hca_k) or rel_l2(bf16_to_f64(g["hca_k"]), r.hca_k) <= TOL
    assert np.array_equal(g["idx"], r.idx)
    for n in ("k", "v"):
        codes, scale = g[f"csa_{n}_codes"], g[f"csa_{n}_scale"]
        assert np.mean(codes == getattr(r, f"csa_{n}_codes")) > 0.995, n
        assert np.allclose(scale, getattr(r, f"csa_{n}_scale"), rtol=1e-6, atol=0), n
        val = e4m3_decode(codes) * scale[..., None].astype(np.float64)
        assert rel_l2(val, getattr(r, f"csa_{n}")) <= TOL, (n, rel_l2(val, getattr(r, f"csa_{n}")))


@pytest.mark.parametrize("fused", ["1", "0"])
def test_fp8_cache_matches_oracle(monkeypatch, fused):
    import torch
    monkeypatch.setenv("HSA_STEP_FUSED", fused)
    seed = 0x8F8
    rng = np.random.default_rng(seed)
    B = 9
    L0 = np.concatenate([[1, 127, 128, 255], rng.integers(300, 2500, B - 4)])
    cache, o = _pair(seed, 128, B, int((L0 + 8).sum() // 128 + B))
    st = [cache.state_alloc() for _ in range(B)]
    assert st == [o.state_alloc() for _ in range(B)]
    cu = np.concatenate([[0], np.cumsum(L0)])
    pos = np.concatenate([np.arange(n) for n in L0])
    keys = np.repeat(np.arange(B), L0)
    cache.append_kv(st, cu, *dev_tokens(seed, keys, pos))
    Kh, Vh, KIh = host_tokens(seed, keys, pos)
    o.append(st, [(Kh[a:b], Vh[a:b], KIh[a:b]) for a, b in zip(cu[:-1], cu[1:])])
    for s in st:
        for bg, bo in zip(cache.block_table(s), o.table(s)):
            _check_block(cache, o, bg, bo)
    for step, k in enumerate((40, 512, 40)):
        p = L0 + step
        Kn, Vn, KIn = dev_tokens(seed, np.arange(B), p)
        Q, QI = dev_queries(seed, np.arange(B), p)
        sc = torch.empty((B, k), dtype=torch.float32, device="cuda")
        idx, _, out = cache.decode_step(st, Kn, Vn, KIn, Q, QI, k, score_out=sc)
        Kh, Vh, KIh = host_tokens(seed, np.arange(B), p)
        o.append(st, [(Kh[i:i + 1], Vh[i:i + 1], KIh[i:i + 1]) for i in range(B)])
        q, qi = host_queries(seed, np.arange(B), p)
        gidx, gout = idx.cpu().numpy(), out.cpu().numpy()
        for i, s in enumerate(st):
            ridx, rval = o.topk(s, qi[i], k)
            assert np.array_equal(gidx[i], ridx), (step, i)
            ref = o.attend(s, q[i], ridx, k)
            assert rel_l2(gout[i], ref) <= TOL, (step, i, rel_l2(gout[i], ref))
        # the standalone attention call over the same selection
        att = cache.decode_attend(st, Q, idx, k)
        for i, s in enumerate(st):
            assert rel_l2(att[i].cpu().numpy(), o.attend(s, q[i], gidx[i], k)) <= TOL
    for s in st:
        for bg, bo in zip(cache.block_table(s), o.table(s)):
            _check_block(cache, o, bg, bo)


def test_fp8_errors():
    import heterogeneous_sparse_attention_amd as hsa
    Wc, Wh = synth.gate_weights(1)
    with pytest.raises(ValueError):
        hsa.Cache(128, 1, 1, Wc, Wh, entry_format="fp4")
    bf = hsa.Cache(128, 1, 2, Wc, Wh)
    s = bf.state_alloc()
    bf.append_kv([s], [0, 128], *dev_tokens(1, 0, np.arange(128)))
    with pytest.raises(hsa.HsaError):       # bf16 context: no FP8 export
        hsa._check(hsa._lib.hsa_export_c4_fp8(bf._ctx, 0, None, None, None, None, None), "hsa_export_c4_fp8")
    bf.close()
