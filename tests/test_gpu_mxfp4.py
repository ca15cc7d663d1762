"""GPU parity of the MXFP4 indexer key format (reading R16: OCP Microscaling, 32
values per E8M0 scale, E2M1 codes) against the CPU oracle.

- The quantisation alone (hsa_mxfp4_quantize_rows) on the same float32 keys as the
  oracle: codes and scale bytes bit for bit, on keys built to hit every tie of the
  E2M1 grid, saturation, zero and subnormal blocks, and a wide range of magnitudes.
- A ragged batch in an MXFP4 cache (alone and with FP8 entries) against the oracle
  in the same formats: every sealed block's codes and scales bit for bit (seal
  stores keys lane-cooperatively, the decode step scores the block it seals from
  the float32 tail, quantising per lane: both must agree with the oracle); top-k
  rows and their scores bit exact (the scores over MXFP4 keys are exact in float32
  for the dyadic synthetic inputs); attention of both forms of the decode step
  within relative L2 1e-3 of the oracle; the standalone hsa_indexer_topk.
"""

import numpy as np
import pytest

import synth
from oracle import Oracle, quantize_mxfp4_rows
from tests.gpu_util import dev_queries, dev_tokens, host_queries, host_tokens, rel_l2

pytestmark = pytest.mark.gpu

TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import heterogeneous_sparse_attention_amd as hsa
    hsa.load()          # raises if the library is missing: no fallback


def _tie_keys():
    """Keys whose blocks have max |x| in [4, 8), so E = 0 and x / 2^E = x: every
    E2M1 midpoint, values just off each, the grid itself, saturation (6 .. 8), both
    signs; plus zero, tiny and subnormal blocks."""
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    mids = (grid[1:] + grid[:-1]) / 2
    f32 = np.float32
    vals = np.concatenate([mids, np.nextafter(mids.astype(f32), f32(8)), np.nextafter(mids.astype(f32), f32(0)),
                           grid, [6.5, 7.0, 7.99, 5.0, 4.75]]).astype(np.float32)
    vals = np.concatenate([vals, -vals])
    per = 31                                   # value 0 of each block holds its max 7.5
    n_blk = -(-len(vals) // per)
    blocks = np.zeros((n_blk, 32), np.float32)
    blocks[:, 0] = 7.5
    flat = blocks[:, 1:].reshape(-1)
    flat[:len(vals)] = vals
    blocks[:, 1:] = flat.reshape(n_blk, per)
    extra = np.stack([np.zeros(32, np.float32), np.full(32, 1e-40, np.float32),
                      np.full(32, 3e-38, np.float32), np.linspace(-1e-30, 1e-30, 32).astype(np.float32)])
    blocks = np.concatenate([blocks, extra])
    pad = (-len(blocks)) % 8
    blocks = np.concatenate([blocks, np.zeros((pad, 32), np.float32)])
    return blocks.reshape(-1, 256)


def test_mxfp4_quantizer_matches_oracle_bit_exact():
    import torch
    import heterogeneous_sparse_attention_amd as hsa
    rng = np.random.default_rng(21)
    rand = (rng.standard_normal((300, 256)) *
            np.exp(rng.uniform(-30, 30, (300, 8))).repeat(32, axis=1)).astype(np.float32)
    hand = np.zeros((1, 256), np.float32)
    hand[0, 0:3] = [1.0, 2.0, -0.3]
    hand[0, 64:66] = [6 * 2.0 ** -5, 5 * 2.0 ** -5]
    rows = np.concatenate([_tie_keys(), rand, hand, -np.abs(rand[:7])])
    for n in (len(rows), 1, 6):                  # ragged counts of 4-row workgroups
        x = torch.from_numpy(rows[:n].copy()).cuda()
        codes, scales = hsa.mxfp4_quantize_rows(x)
        rc, rs, _ = quantize_mxfp4_rows(rows[:n])
        assert np.array_equal(scales.cpu().numpy(), rs), n
        got = codes.cpu().numpy()
        bad = np.argwhere(got != rc)
        assert bad.size == 0, (n, bad[:5], got[tuple(bad[0])], rc[tuple(bad[0])])
    c0, s0 = hsa.mxfp4_quantize_rows(torch.zeros((0, 256), dtype=torch.float32, device="cuda"))
    assert c0.shape == (0, 128) and s0.shape == (0, 8)


def _pair(seed, n_win, max_states, max_blocks, entry_format):
    import heterogeneous_sparse_attention_amd as hsa
    Wc, Wh = synth.gate_weights(seed)
    return (hsa.Cache(n_win, max_states, max_blocks, Wc, Wh, entry_format=entry_format, index_format="mxfp4"),
            Oracle(n_win, Wc, Wh, max_states, max_blocks, entry_format=entry_format, index_format="mxfp4"))


def _check_keys(cache, o, bg, bo):
    g = cache.export_block(bg)
    r = o.block(bo)
    assert "idx" not in g
    assert np.array_equal(g["idx_scales"], r.idx_scales), bo
    assert np.array_equal(g["idx_codes"], r.idx_codes), bo


# mx_unit: MXFP4 blocks per scoring workgroup ("" = the default, one 3-block pass);
# 1 pads every pass with two repeated reads, 8 runs passes of 3, 3 and 2 blocks
@pytest.mark.parametrize("fused,entries,mx_unit", [("1", "bf16", ""), ("0", "bf16", ""), ("1", "fp8", ""),
                                                   ("1", "bf16", "1"), ("0", "bf16", "8")])
def test_mxfp4_cache_matches_oracle(monkeypatch, fused, entries, mx_unit):
    import torch
    monkeypatch.setenv("HSA_STEP_FUSED", fused)
    if mx_unit:
        monkeypatch.setenv("HSA_MX_UNIT", mx_unit)
    seed = 0x4F4
    rng = np.random.default_rng(seed)
    B = 9
    L0 = np.concatenate([[1, 127, 128, 255], rng.integers(300, 2500, B - 4)])
    cache, o = _pair(seed, 128, B, int((L0 + 8).sum() // 128 + B), entries)
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
            _check_keys(cache, o, bg, bo)
    for step, k in enumerate((40, 512, 40)):
        p = L0 + step
        Kn, Vn, KIn = dev_tokens(seed, np.arange(B), p)
        Q, QI = dev_queries(seed, np.arange(B), p)
        sc = torch.empty((B, k), dtype=torch.float32, device="cuda")
        idx, _, out = cache.decode_step(st, Kn, Vn, KIn, Q, QI, k, score_out=sc)
        Kh, Vh, KIh = host_tokens(seed, np.arange(B), p)
        o.append(st, [(Kh[i:i + 1], Vh[i:i + 1], KIh[i:i + 1]) for i in range(B)])
        q, qi = host_queries(seed, np.arange(B), p)
        gidx, gout, gsc = idx.cpu().numpy(), out.cpu().numpy(), sc.cpu().numpy()
        for i, s in enumerate(st):
            ridx, rval = o.topk(s, qi[i], k)
            assert np.array_equal(gidx[i], ridx), (step, i)
            assert np.array_equal(gsc[i].astype(np.float64), rval), (step, i)
            ref = o.attend(s, q[i], ridx, k)
            assert rel_l2(gout[i], ref) <= TOL, (step, i, rel_l2(gout[i], ref))
        # the standalone selection over the same keys
        tsc = torch.empty((B, k), dtype=torch.float32, device="cuda")
        tidx, _ = cache.indexer_topk(st, QI, k, score_out=tsc)
        for i, s in enumerate(st):
            assert np.array_equal(tidx[i].cpu().numpy(), gidx[i]) and np.array_equal(tsc[i].cpu().numpy(), gsc[i])
    for s in st:
        for bg, bo in zip(cache.block_table(s), o.table(s)):
            _check_keys(cache, o, bg, bo)


def test_mxfp4_errors():
    import heterogeneous_sparse_attention_amd as hsa
    Wc, Wh = synth.gate_weights(1)
    with pytest.raises(ValueError):
        hsa.Cache(128, 1, 1, Wc, Wh, index_format="fp4")
    f32 = hsa.Cache(128, 1, 2, Wc, Wh)
    s = f32.state_alloc()
    f32.append_kv([s], [0, 128], *dev_tokens(1, 0, np.arange(128)))
    with pytest.raises(hsa.HsaError):       # fp32 keys: no MXFP4 export
        hsa._check(hsa._lib.hsa_export_idx_mxfp4(f32._ctx, 0, None, None, None), "hsa_export_idx_mxfp4")
    f32.close()
    mx = hsa.Cache(128, 1, 2, Wc, Wh, index_format="mxfp4")
    s = mx.state_alloc()
    mx.append_kv([s], [0, 128], *dev_tokens(1, 0, np.arange(128)))
    import ctypes
    buf = np.zeros((128, 4, 64), np.float32)
    with pytest.raises(hsa.HsaError):       # MXFP4 keys: no fp32 key export
        hsa._check(hsa._lib.hsa_export_block(mx._ctx, 0, None, None, None, None,
                                             buf.ctypes.data_as(ctypes.c_void_p), None), "hsa_export_block")
    mx.close()
