"""Decode-step benchmark of the heterogeneous KV cache on one MI355X.

A step is one pass of the whole hot path over the batch: append one token per
request into its State (sealing full blocks into the Block Cache), indexer
scores + top-k over every sealed C4 entry, and heterogeneous attention over
SWA + HCA + selected C4 entries (hsa_decode_step). Inputs are synthetic and
resident in HBM before timing starts.

  python bench.py [--steps K] [--warmup W] [--workload 2]
prints one JSON line. The default is the headline workload, b32 (2). The other
workloads time the same step at their own shapes (1 l130, 3 prefix, 5 long) or,
for 4 (bulk), whole append calls of 8 x 131072 tokens with fused seal.
Other modes (for the profiles):
  python bench.py --copy-calibration      a plain copy kernel of known size
  python bench.py --counters DIR          summarise rocprofv3 --pmc output
"""

from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402
from synth import workloads  # noqa: E402

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
METRIC = "decode tokens/s + achieved HBM GB/s (% of peak), append+attend, B=32 L<=8K"
LENGTHS = {"l130": "L0 = 130", "b32": "L0 ~ U{1..8192}",
           "prefix": "L0 ~ U{16384..65536}, 8 groups sharing a 32768-token prefix by fork",
           "bulk": "131072 tokens each", "long": "L0 = 2**20 - 8"}
ROW = 8192                     # K + V bytes of one token or entry (2 x 16 x 128 bf16)
C4_FP8 = 4224                  # K + V bytes of one FP8 C4 entry (2 x 16 x 128 E4M3 + 2 x 16 fp32 scales)
IDX_BLOCK = 131072             # indexer keys of one block (128 x 4 x 64 fp32)
IDX_BLOCK_MX = 17408           # MXFP4 indexer keys of one block (128 x (128 code + 8 scale bytes))
SEAL_BYTES = 1581056           # per seal: read 128 tokens K/V + 128 indexer keys, write 32 C4 + 1 HCA + 128 keys


def c4_bytes(entries: str) -> int:
    return C4_FP8 if entries == "fp8" else ROW


def idx_bytes(index: str) -> int:
    return IDX_BLOCK_MX if index == "mxfp4" else IDX_BLOCK


def kv_bytes(kv: str) -> int:
    """K + V bytes of one SWA ring token or HCA entry as stored (bf16, or FP8 codes and
    per-head scales)."""
    return C4_FP8 if kv == "fp8" else ROW


def seal_bytes(entries: str, index: str = "f32", kv: str = "bf16") -> int:
    """Bytes a seal moves: the block's 128 stored tokens and indexer keys read, 32 C4
    entries, 1 HCA entry and 128 indexer keys written."""
    return (SEAL_BYTES - 32 * (ROW - c4_bytes(entries)) - (IDX_BLOCK - idx_bytes(index))
            - 129 * (ROW - kv_bytes(kv)))
KERNEL_SYMBOL = {"append": "k_decode_append", "score": "k_score", "select": "k_select",
                 "attend": "k_attend", "merge": "k_merge", "seal": "k_seal_merge",
                 "write": "k_bulk_write", "step1": "k_step1", "step2": "k_step2",
                 "step2b": "k_step2b", "step3": "k_step3", "step4": "k_step4",
                 "bulk_seal": "k_bulk_seal"}
STEP_SOURCES = ["step.hip", "attn_dev.h", "score_dev.h", "seal_dev.h", "device.h"]
KERNEL_SOURCES = {"step1": STEP_SOURCES, "step2": STEP_SOURCES, "step2b": STEP_SOURCES,
                  "step3": STEP_SOURCES, "step4": STEP_SOURCES,
                  "bulk_seal": ["append_seal.hip", "seal_dev.h", "device.h"],
                  "write": ["append_seal.hip", "seal_dev.h", "device.h"]}
STEP_KERNELS = ("step1", "step2", "step2b", "step3", "step4")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


# ------------------------------------------------------------------ algorithmic bytes

CACHE_N = 4096                 # score rows up to this length are selected in LDS


def step_fused(nb: np.ndarray, open_g=None) -> bool:
    """Whether the library runs this step in three launches: every score row fits the
    selection's LDS cache (unless HSA_STEP_FUSED=0). open_g: eager C4 open groups."""
    rows = 32 * (nb + (open_g > 0 if open_g is not None else 0))
    return os.environ.get("HSA_STEP_FUSED", "1") != "0" and bool((rows <= CACHE_N).all())


def step_bytes(L_after: np.ndarray, nb: np.ndarray, n_win: int, k: int, sealed: np.ndarray,
               entries: str = "bf16", index: str = "f32", layer: str = "mixed", c4_mode: str = "sealed",
               kv: str = "bf16") -> dict:
    """Bytes the method must move in one decode step, per launch (scratch excluded).

    L_after: lengths after the append; nb: sealed blocks after it; sealed: 1 where
    the step sealed a block; entries, index: storage formats of the C4 entries and
    of the sealed indexer keys (the block sealed in the step is scored from the
    float32 tail)."""
    if layer != "mixed":
        return layer_step_bytes(L_after, nb, n_win, k, sealed, entries, index, layer, kv)
    C4 = c4_bytes(entries)
    KV = kv_bytes(kv)              # one ring token or HCA entry as stored
    SEAL = seal_bytes(entries, index, kv)
    # eager C4: the open block's g entries are candidates too; its 4g tokens' indexer
    # keys are scanned, and a step that completes a group reads 3 ring tokens and
    # writes the entry
    g = (L_after - 128 * nb) // 4 if c4_mode == "eager" else 0 * nb
    done = ((L_after % 4 == 0) & (L_after % 128 != 0)) if c4_mode == "eager" else 0 * nb
    scan = (nb - sealed) * idx_bytes(index) + sealed * IDX_BLOCK + 4 * g * 1024
    swa = np.minimum(L_after, n_win)
    kk = np.minimum(k, 32 * nb + g)
    B = len(L_after)
    eager_b = int((done * (3 * ROW + ROW)).sum())
    if step_fused(nb, g):
        out = {
            "step1": int(B * (ROW + 1024 + KV + 1024) + sealed.sum() * (SEAL - KV)
                         + scan.sum() + B * 1024) + eager_b,
            # S2 (three-launch form): top-k out; HCA entries of new blocks; K/V rows
            # of the SWA tokens, earlier HCA entries and selected C4 entries + the query
            "step2": int((kk * 8).sum() + sealed.sum() * KV
                         + ((swa + nb - sealed) * KV + kk * C4).sum() + B * 4096),
            "step2b": 0,
            "step3": 0,
            # S4: the new HCA entries (K/V rows) and the fp32 output
            "step4": int(sealed.sum() * KV + B * 8192),
        }
        out["step"] = sum(out.values())
        return out
    out = {
        # S1: token K, V, indexer key in + ring and tail slots out; seals (minus the
        # HCA entry written in S2); indexer keys of every sealed block + the
        # indexer query
        "step1": int(B * (ROW + 1024 + KV + 1024) + sealed.sum() * (SEAL - KV)
                     + scan.sum() + B * 1024) + eager_b,
        # S2: top-k ordinals (and scores) out; HCA entries of new blocks; K/V rows
        # of the SWA tokens and earlier HCA entries + the query
        "step2": int((kk * 8).sum() + sealed.sum() * KV
                     + ((swa + nb - sealed) * KV).sum() + B * 4096),
        # S2b (rows cut into slices): the second selection round reads scratch only
        "step2b": 0,
        # S3: K/V rows of the new HCA entries and selected C4 entries, their
        # ordinals, the query
        "step3": int((sealed * KV + kk * C4).sum() + (kk * 4).sum() + B * 4096),
        # S4: fp32 output
        "step4": int(B * 8192),
    }
    out["step"] = sum(out.values())
    return out


def layer_step_bytes(L_after, nb, n_win, k, sealed, entries, index, layer, kv="bf16") -> dict:
    """step_bytes of an SWA, CSA or HCA layer, always in three launches: what the
    layer keeps and attends (the SWA always; C4 entries, indexer keys and the tail
    for CSA; HCA entries for HCA)."""
    c4, hca = layer == "csa", layer == "hca"
    C4 = c4_bytes(entries)
    KV = kv_bytes(kv)
    swa = np.minimum(L_after, n_win)
    kk = np.minimum(k, 32 * nb) if c4 else 0 * nb
    B = len(L_after)
    tok_in, tok_st = ROW + (1024 if c4 else 0), KV + (1024 if c4 else 0)   # one token in, into the State
    seal = 128 * KV + (128 * 1024 + 32 * C4 + idx_bytes(index) if c4 else 0) + (KV if hca else 0)
    scan = ((nb - sealed) * idx_bytes(index) + sealed * IDX_BLOCK) if c4 else 0 * nb
    out = {
        "step1": int(B * (tok_in + tok_st) + sealed.sum() * (seal - (KV if hca else 0)) + (scan.sum() if c4 else 0)
                     + (B * 1024 if c4 else 0)),
        "step2": int((kk * 8).sum() + B * k * 4 * (0 if c4 else 1) + (sealed.sum() * KV if hca else 0)
                     + (swa * KV + (nb - sealed) * KV * hca + kk * C4).sum() + B * 4096),
        "step2b": 0,
        "step3": 0,
        "step4": int((sealed.sum() * KV if hca else 0) + B * 8192),
    }
    out["step"] = sum(out.values())
    return out


def storage_formats(args):
    """(C4 entry, indexer key, KV) storage formats of a run."""
    return (getattr(args, "entries", "bf16"), getattr(args, "index", "f32"), getattr(args, "kv", "bf16"))


def traffic_key(workload: str, args) -> str:
    """traffic.json key of a workload's counters: the workload name, with the storage
    formats appended when they are not the default ones (b32:fp8-mxfp4-fp8)."""
    fmt = storage_formats(args)
    return workload if fmt == ("bf16", "f32", "bf16") else workload + ":" + "-".join(fmt)


def counted_traffic(kernel: str, workload: str, args):
    """HBM bytes per launch of `kernel` on `workload` from profiles/traffic.json (scaled
    rocprofv3 FETCH_SIZE + WRITE_SIZE), or None when the counters were taken on other
    sources, formats or launch settings."""
    try:
        tr = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    ent = tr.get("kernels", {}).get(traffic_key(workload, args), {}).get(KERNEL_SYMBOL[kernel])
    if not ent or ent.get("src_sha") != src_hash(kernel):
        return None
    if (ent.get("entries", "bf16"), ent.get("index", "f32"), ent.get("kv", "bf16")) != storage_formats(args):
        return None
    if ent.get("env", "") != launch_env():
        return None
    return ent.get("traffic_bytes_per_launch")


# the library's launch-shape settings read from the environment (tuning hooks)
LAUNCH_KNOBS = ("HSA_ATTEND_WGS", "HSA_STEP_SLOTS", "HSA_STEP_FUSED", "HSA_MX_UNIT", "HSA_SELECT_SLICE",
                "HSA_MIXED_A", "HSA_SEL_LAT")


def launch_env() -> str:
    """The launch settings set in the environment, as one string."""
    return " ".join(f"{k}={os.environ[k]}" for k in LAUNCH_KNOBS if k in os.environ)


def src_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(kernel, []):
        with open(os.path.join(ROOT, "heterogeneous_sparse_attention_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------------ the b32 decode workload

def _append_device(cache, wl, states, reqs, p0s, p1s, chunk=65536, seeds=None):
    """Append positions [p0, p1) of workload requests `reqs` to `states`, in calls of
    at most `chunk` tokens, with inputs generated on the device (keys as the
    workload keys them: shared-prefix positions carry their group's stream)."""
    import torch
    from synth.device import fill_rows
    i = 0
    while i < len(reqs):
        grp, tot = [], 0
        while i < len(reqs) and (tot + p1s[i] - p0s[i] <= chunk or not grp):
            grp.append(i)
            tot += p1s[i] - p0s[i]
            i += 1
        grp = [j for j in grp if p1s[j] > p0s[j]]
        if not grp:
            continue
        pos = np.concatenate([np.arange(p0s[j], p1s[j]) for j in grp]).astype(np.int64)
        keys = np.concatenate([wl.key(reqs[j], np.arange(p0s[j], p1s[j])) for j in grp]).astype(np.int64)
        cu = np.concatenate([[0], np.cumsum([p1s[j] - p0s[j] for j in grp])]).astype(np.int64)
        T = int(cu[-1])
        kt = torch.from_numpy(keys.astype(np.int32)).cuda()
        pt = torch.from_numpy(pos).cuda()
        K = torch.empty((T, 16, 128), dtype=torch.bfloat16, device="cuda")
        V = torch.empty_like(K)
        KI = torch.empty((T, 4, 64), dtype=torch.float32, device="cuda")
        # a layer stack: the same append through every layer, each with its own tokens
        for l, sd in enumerate(seeds or [wl.seed]):
            if seeds:
                cache.set_layer(l)
            fill_rows(K, sd, synth.STREAM_K, keys=kt, pos=pt)
            fill_rows(V, sd, synth.STREAM_V, keys=kt, pos=pt)
            fill_rows(KI, sd, synth.STREAM_IDXK, keys=kt, pos=pt)
            cache.append_kv([states[j] for j in grp], cu, K, V, KI)
        del K, V, KI


def layer_seed(wl, layer: int) -> int:
    """Token seed of one layer of a layer stack (layer 0 keeps the workload's)."""
    return wl.seed + 101 * layer


def setup_decode(wl, extra_steps: int, copies: int = 1, entries: str = "bf16", index: str = "f32",
                 layers=None, c4_mode: str = "sealed", kv: str = "bf16"):
    """Cache holding `copies` identical instances of the batch, every request
    prefilled to L0 (bulk appends of device-generated tokens; in a prefix workload
    each request forks off its group's parent at its fork length, sharing those
    blocks, and appends the rest itself). Returns the cache and one list of state
    ids per instance."""
    import torch
    import heterogeneous_sparse_attention_amd as hsa

    types = layers or ["mixed"]
    if layers:
        gates = [synth.gate_weights(wl.seed + 7 * l) for l in range(len(types))]
        Wc, Wh = np.stack([g[0] for g in gates]), np.stack([g[1] for g in gates])
    else:
        Wc, Wh = synth.gate_weights(wl.seed)
    L0 = wl.prefill.astype(np.int64)
    B = wl.batch
    max_len = int(L0.max()) + extra_steps + 1
    max_blocks = copies * (int(((L0 + extra_steps) // 128).sum()) + B) + 8
    n_parents = wl.n_groups if wl.prefix_len else 0
    cache = hsa.Cache(wl.n_win, copies * (B + n_parents), max_blocks + copies * n_parents * (wl.prefix_len // 128),
                      Wc, Wh, max_blocks_per_state=max_len // 128 + 2, entry_format=entries,
                      index_format=index, layer_types=layers, c4_mode=c4_mode, kv_format=kv)
    if layers and wl.prefix_len:
        raise SystemExit("layer stacks are measured on workloads without shared prefixes")
    inst = []
    for _ in range(copies):
        states = [None] * B
        start = [0] * B
        if wl.prefix_len:
            fork = {b: wl.fork_len(b) for b in range(B)}
            for g in range(wl.n_groups):
                kids = sorted((b for b in range(B) if wl.group(b) == g), key=lambda b: fork[b])
                parent, cur = cache.state_alloc(), 0
                for b in kids:
                    if fork[b] > cur:
                        _append_device(cache, wl, [parent], [b], [cur], [fork[b]])
                        cur = fork[b]
                    states[b] = cache.state_alloc()
                    cache.block_table_share(parent, states[b])
                    start[b] = fork[b]
                cache.state_free(parent)
        else:
            states = [cache.state_alloc() for _ in range(B)]
        _append_device(cache, wl, states, list(range(B)), start, [int(x) for x in L0],
                       seeds=[layer_seed(wl, l) for l in range(len(types))] if layers else None)
        inst.append(states)
    torch.cuda.synchronize()
    return cache, inst


def decode_inputs(wl, L0: np.ndarray, n_steps: int, seed=None):
    """Per-step device inputs: the token at position L0 + t for each request."""
    import torch
    from synth.device import fill_rows
    B = wl.batch
    pos = (L0[None, :] + np.arange(n_steps)[:, None]).reshape(-1).astype(np.int64)
    req = np.tile(np.arange(B), n_steps)
    keys = np.array([int(wl.key(int(b), p)) for b, p in zip(req, pos)], np.int64).astype(np.int32)
    kt = torch.from_numpy(keys).cuda()
    pt = torch.from_numpy(pos).cuda()
    n = n_steps * B
    t = {
        "k": torch.empty((n, 16, 128), dtype=torch.bfloat16, device="cuda"),
        "v": torch.empty((n, 16, 128), dtype=torch.bfloat16, device="cuda"),
        "ki": torch.empty((n, 4, 64), dtype=torch.float32, device="cuda"),
        "q": torch.empty((n, 16, 128), dtype=torch.bfloat16, device="cuda"),
        "qi": torch.empty((n, 4, 64), dtype=torch.float32, device="cuda"),
    }
    for name, sid in (("k", synth.STREAM_K), ("v", synth.STREAM_V), ("ki", synth.STREAM_IDXK),
                      ("q", synth.STREAM_Q), ("qi", synth.STREAM_QI)):
        fill_rows(t[name], wl.seed if seed is None else seed, sid, keys=kt, pos=pt)
    return {n_: x.view(n_steps, B, *x.shape[1:]) for n_, x in t.items()}


def measured_roof(gib: int = 1, reps: int = 5) -> dict:
    """The HBM bandwidth plain kernels reach on this GPU, beside the vendor's 8 TB/s:
    the harness's streaming read of `gib` GiB (synth/libhsa_synth.so), the runtime's
    device copy of `gib` GiB (read + write counted) and torch's sum over `gib` GiB.
    Median of `reps` runs each, on buffers larger than the 256 MB last-level cache."""
    import torch
    from synth.device import roof_read
    n = (gib << 30) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def median_ms(fn):
        ts = []
        for _ in range(reps):
            torch.cuda.synchronize()
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))
    blocks = 2048
    fold = torch.empty(blocks, dtype=torch.int32, device="cuda")
    b.copy_(a)                                   # warm up the kernels
    a.sum()
    roof_read(a, fold, blocks)
    stream_ms = median_ms(lambda: (roof_read(a, fold, blocks), roof_read(b, fold, blocks)))
    copy_ms = median_ms(lambda: b.copy_(a))
    read_ms = median_ms(lambda: a.sum())
    nbytes = n * 4
    out = {"stream_read_gbps": 2 * nbytes / (stream_ms * 1e-3) / 1e9,
           "copy_gbps": 2 * nbytes / (copy_ms * 1e-3) / 1e9, "sum_gbps": nbytes / (read_ms * 1e-3) / 1e9,
           "what": f"streaming read (a contiguous chunk per workgroup, 16-byte non-temporal loads, 8 in "
                   f"flight per thread, {blocks} x 256 threads) of two {gib} GiB buffers in turn; torch copy_ of {gib} GiB (read + write); "
                   f"torch sum over {gib} GiB; median of {reps} each"}
    del a, b, fold
    torch.cuda.empty_cache()
    return out


def gpu_lead(cycles: int = 500_000):
    """Keep the GPU busy for about 0.2 ms (a spin kernel) so that the host queues the
    first timed steps before the start event fires: the timed region then holds the
    steps' GPU time back to back, without the host's latency to its first launch."""
    import torch
    try:
        torch.cuda._sleep(cycles)
    except (AttributeError, RuntimeError):
        pass


def run_decode(args) -> dict:
    import torch
    wl = workloads.make(args.workload)
    B, k = wl.batch, wl.topk
    W, K = args.warmup, args.steps
    reps = max(1, args.repeats)
    layers = args.layers.split(",") * args.layer_repeat if args.layers else None
    types = layers or ["mixed"]
    # a layer stack streams different data layer after layer by itself: one copy
    R = args.copies if args.copies is not None else (4 if wl.name == "b32" and not layers else 1)
    # Cache instances: set 0 (R copies) takes the warmup, the per-kernel timing steps
    # and the roofline pass; sets 1 .. reps (R copies each) each take one timed pass of
    # K steps from the prefill lengths, i.e. every timed pass runs the same workload,
    # as from a restored snapshot of the pools.
    n_kt = max(4, min(K, 16))                     # steps per kernel in the kernel timing
    set0 = W + len(STEP_KERNELS) * n_kt + K
    local_steps = (max(set0, K) + R - 1) // R
    cache, inst = setup_decode(wl, local_steps, R * (1 + reps), args.entries, args.index, layers,
                               args.c4_mode, args.kv)
    L0 = wl.prefill.astype(np.int64)
    inp = [decode_inputs(wl, L0, local_steps, seed=layer_seed(wl, l)) for l in range(len(types))]
    topk = torch.empty((B, k), dtype=torch.int32, device="cuda")
    out = torch.empty((B, 16, 128), dtype=torch.float32, device="cuda")

    # step t of set c advances instance c R + t % R by its step t // R: consecutive
    # steps read different copies of the cache, as consecutive layers of a model
    # would; a step of a layer stack is one decode step of every layer, in layer order
    def step(t, c=0):
        j = t // R
        for l, x in enumerate(inp):
            if layers:
                cache.set_layer(l)
            cache.decode_step(inst[c * R + t % R], x["k"][j], x["v"][j], x["ki"][j], x["q"][j],
                              x["qi"][j], k, topk_out=topk, out=out)

    for t in range(W):                            # warmup
        step(t)
    torch.cuda.synchronize()
    # per-kernel timing: n_kt steps per step kernel, one kernel timed at a time (an
    # event pair on every kernel of a step lets the first kernel's start event fire
    # while the host still writes its dispatch, which inflates it whenever the host
    # falls behind)
    t_next = W
    per_step, timed_at, launches = {}, {}, {}
    for n in STEP_KERNELS:
        cache.timing_enable([n])
        gpu_lead()
        timed_at[n] = list(range(t_next, t_next + n_kt))
        for t in timed_at[n]:
            step(t)
        t_next += n_kt
        torch.cuda.synchronize()
        ms_, cnt = cache.timing_read()[n]
        per_step[n] = ms_ / n_kt
        launches[n] = cnt
    cache.timing_enable([])
    dominant = args.kernel or max(STEP_KERNELS, key=lambda n: per_step[n])
    # the byte split assumes the library's choice of form; check it against the launches
    def open_g(L):
        return (L - 128 * (L // 128)) // 4 if args.c4_mode == "eager" else None
    def fused_at(t):
        return step_fused((L0 + t // R + 1) // 128, open_g(L0 + t // R + 1))
    has_c4 = any(ty in ("mixed", "csa") for ty in types)   # layers with a part B
    if (launches["step3"] > 0) != (has_c4 and not all(map(fused_at, timed_at["step3"]))):
        raise RuntimeError("decode-step form differs from the one the byte split assumes")

    # roofline pass: K steps of set 0, the library attaching a start/stop event pair
    # to each dispatch of the dominant kernel on the launch stream
    cache.timing_enable([dominant])
    roof_from = t_next
    gpu_lead()
    for t in range(roof_from, roof_from + K):
        step(t)
    torch.cuda.synchronize()
    kt = cache.timing_read()
    cache.timing_enable([])

    # timed passes (value): whole steps between two events, nothing inside; one pass
    # per set of fresh copies, the median reported
    times, walls = [], []
    for c in range(1, reps + 1):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        gpu_lead()
        ev0.record()
        for t in range(K):
            step(t, c)
        ev1.record()
        torch.cuda.synchronize()
        walls.append(time.perf_counter() - t0)
        times.append(ev0.elapsed_time(ev1))
    ms_total = float(np.median(times))
    wall = float(np.median(walls))

    def bytes_over(t_from, t_to):
        acc = {n: 0 for n in STEP_KERNELS + ("step",)}
        for t in range(t_from, t_to):
            L_after = L0 + t // R + 1
            nb = L_after // 128
            sealed = (L_after % 128 == 0).astype(np.int64)
            for typ in types:
                sb = step_bytes(L_after, nb, wl.n_win, k, sealed, args.entries, args.index, typ, args.c4_mode,
                                args.kv)
                for n in acc:
                    acc[n] += sb[n]
        return acc

    bytes_1 = bytes_over(0, K)                       # every timed pass
    bytes_2 = bytes_over(roof_from, roof_from + K)
    ms_per_step = ms_total / K
    dom_ms, dom_n = kt[dominant]
    achieved = (bytes_2[dominant] / dom_n) / (dom_ms / dom_n * 1e-3) / 1e9 if dom_n else None
    step_gbs = bytes_1["step"] / (ms_total * 1e-3) / 1e9

    traffic = counted_traffic(dominant, wl.name, args) if not layers else None

    fp8 = args.entries == "fp8"
    mx4 = args.index == "mxfp4"
    metric = METRIC if wl.name == "b32" else f"decode tokens/s + achieved HBM GB/s, append+attend, {wl.name}"
    stack = f", {len(types)}-layer stack ({args.layers} x {args.layer_repeat})" if layers else ""
    res = {
        "metric": metric + (", FP8 C4 entries" if fp8 else "") + (", FP8 SWA and HCA" if args.kv == "fp8" else "")
                  + (", MXFP4 indexer keys" if mx4 else "") + stack
                  + (", eager C4" if args.c4_mode == "eager" else ""),
        "value": B * K / (ms_total * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: {B} requests, {LENGTHS[wl.name]} (seed {wl.seed:#x}), "
                               f"decode steps, n_win {wl.n_win}, top-k {k}, 16x128 bf16 K/V/Q"
                               f"{' (SWA ring and HCA entries FP8 E4M3, fp32 scale per head)' if args.kv == 'fp8' else ''}"
                               f"{' (C4 entries FP8 E4M3, fp32 scale per head)' if fp8 else ''}, "
                               f"indexer 4x64 fp32{' (sealed keys MXFP4)' if mx4 else ''}, m=4, m'=128, "
                               f"{len(types)} layer{'s' if len(types) > 1 else ''}"
                               f"{' (' + ','.join(types) + ')' if layers else ''}; steps rotate over {R} "
                               f"copies of the cache",
                   "batch": B, "n_win": wl.n_win, "topk": k, "kv_dtype": "bf16",
                   "c4_entries": args.entries, "swa_hca": args.kv, "index_keys": args.index, "cache_copies": R,
                   "layers": types, "c4_mode": args.c4_mode,
                   "L0_mean": float(L0.mean()), "parallelism": "single GPU"},
        "hbm_gbps": step_gbs,
        "hbm_frac_of_peak": step_gbs / PEAK_HBM_GBS,
        "bytes_per_step": bytes_1["step"] / K,
        "wall_s": wall,
        "timed_passes_ms": times,
        "timing": f"median of {reps} passes of {K} steps, each on its own fresh copies of the "
                  f"prefilled cache; events around each pass",
        "roofline": {"bound": "hbm", "kernel": KERNEL_SYMBOL[dominant],
                     "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": (achieved / PEAK_HBM_GBS) if achieved else None,
                     "traffic": traffic,
                     "traffic_gbps": (traffic / (dom_ms / dom_n * 1e-3) / 1e9) if (traffic and dom_n) else None,
                     "avg_launch_us": (dom_ms / dom_n * 1e3) if dom_n else None,
                     "algorithmic_bytes_per_launch": (bytes_2[dominant] / dom_n) if dom_n else None,
                     "measured": f"HIP event pair attached to each {KERNEL_SYMBOL[dominant]} "
                                 f"dispatch (hipExtLaunchKernel) over {K} steps"},
        "kernels_us_per_step": {n: per_step[n] * 1e3 for n in STEP_KERNELS},
        "bytes_per_step_by_kernel": {n: bytes_1[n] / K for n in STEP_KERNELS},
    }
    cache.close()
    return res


def run_bulk(args) -> dict:
    """Bulk prefill packing: every request's whole prompt appended in one call (fused
    seal), into fresh states each time. Inputs are generated on the device first."""
    import torch
    import heterogeneous_sparse_attention_amd as hsa
    from synth.device import fill_rows
    wl = workloads.make(args.workload)
    B = wl.batch
    L0 = wl.prefill.astype(np.int64)
    T = int(L0.sum())
    Wc, Wh = synth.gate_weights(wl.seed)
    nb = L0 // 128
    cache = hsa.Cache(wl.n_win, B, int(nb.sum()) + B, Wc, Wh, max_blocks_per_state=int(L0.max()) // 128 + 2,
                      entry_format=args.entries, index_format=args.index)
    C4 = c4_bytes(args.entries)
    IDX = idx_bytes(args.index)
    cu = np.concatenate([[0], np.cumsum(L0)]).astype(np.int64)
    pos = torch.from_numpy(np.concatenate([np.arange(n) for n in L0]).astype(np.int64)).cuda()
    keys = torch.from_numpy(np.repeat(np.arange(B), L0).astype(np.int32)).cuda()
    K = torch.empty((T, 16, 128), dtype=torch.bfloat16, device="cuda")
    V = torch.empty_like(K)
    KI = torch.empty((T, 4, 64), dtype=torch.float32, device="cuda")
    fill_rows(K, wl.seed, synth.STREAM_K, keys=keys, pos=pos)
    fill_rows(V, wl.seed, synth.STREAM_V, keys=keys, pos=pos)
    fill_rows(KI, wl.seed, synth.STREAM_IDXK, keys=keys, pos=pos)
    torch.cuda.synchronize()
    # bytes the method must move: every token's K, V and indexer key read, every
    # block's 32 C4 + 1 HCA entries and 128 indexer keys written, the ring's last
    # n_win tokens and the indexer tail written
    seal_b = int(nb.sum()) * (128 * (ROW + 1024) + 32 * C4 + ROW + IDX)
    write_bytes = int((np.minimum(L0, wl.n_win) * 2 * ROW + (L0 % 128) * 2 * 1024).sum())
    alg = T * (ROW + 1024) + int(nb.sum()) * (32 * C4 + ROW + IDX) \
        + int((np.minimum(L0, wl.n_win) * ROW + (L0 % 128) * 1024).sum())
    reps = max(2, args.steps)
    times = []
    for rep in range(reps + 1):
        states = [cache.state_alloc() for _ in range(B)]
        torch.cuda.synchronize()
        if rep == reps:
            cache.timing_enable(["seal", "write"])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        cache.append_kv(states, cu, K, V, KI)
        e1.record()
        torch.cuda.synchronize()
        if rep > 0 and rep < reps:
            times.append(e0.elapsed_time(e1))
        for st in states:
            cache.state_free(st)
    kt = cache.timing_read()
    cache.timing_enable([])
    cache.close()
    ms = float(np.median(times))
    seal_ms = kt["seal"][0]
    gbs = alg / (ms * 1e-3) / 1e9
    return {
        "metric": f"bulk append tokens/s + achieved HBM GB/s, append+compress, {wl.name}"
                  + (", FP8 C4 entries" if args.entries == "fp8" else "")
                  + (", MXFP4 indexer keys" if args.index == "mxfp4" else ""),
        "value": T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": len(times), "warmup": 1,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{wl.name}: {B} requests x {LENGTHS[wl.name]} (seed {wl.seed:#x}) in one "
                               f"append call with fused seal, n_win {wl.n_win}; 16x128 bf16 K/V, indexer "
                               f"4x64 fp32, m=4, m'=128, 1 layer",
                   "batch": B, "tokens": T, "c4_entries": args.entries, "index_keys": args.index, "n_win": wl.n_win, "parallelism": "single GPU"},
        "hbm_gbps": gbs, "hbm_frac_of_peak": gbs / PEAK_HBM_GBS, "bytes_per_step": alg,
        "roofline": {"bound": "hbm", "kernel": "k_bulk_seal",
                     "achieved": seal_b / (seal_ms * 1e-3) / 1e9 if seal_ms else None,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": seal_b / (seal_ms * 1e-3) / 1e9 / PEAK_HBM_GBS if seal_ms else None,
                     "traffic": counted_traffic("bulk_seal", wl.name, args),
                     "avg_launch_us": seal_ms * 1e3 if seal_ms else None,
                     "algorithmic_bytes_per_launch": seal_b,
                     "measured": "HIP event pair attached to the k_bulk_seal dispatch of one call"},
        "kernels_us_per_call": {"seal": kt["seal"][0] * 1e3, "write": kt["write"][0] * 1e3},
        "bytes_per_call_by_kernel": {"seal": seal_b, "write": write_bytes},
    }


# ------------------------------------------------------------------ prefix hits (SWA policies)

PERIOD = 16384                 # Periodic policy: a State checkpoint every 16384 tokens


def run_hits(args) -> dict:
    """A batch of prefix hits on the prefix workload: each of its 64 requests starts
    fresh at its fork length (16K-32K tokens, a multiple of 128) of its group's shared
    prefix, which a prefix entry holds as blocks only (the source request is freed).
    zero: attach + replay of the last n_win prefix tokens; periodic: attach + restore
    of the checkpoint at 16384 floor(len / 16384) + replay of the gap; full: attach +
    restore of the checkpoint at len. The timed region is the whole batch, host calls
    included, with the replayed tokens already in HBM."""
    import torch
    import heterogeneous_sparse_attention_amd as hsa
    from synth.device import fill_rows
    wl = workloads.make(3)
    B, W, pol = wl.batch, wl.n_win, args.hit
    P = np.array([wl.fork_len(b) for b in range(B)], np.int64)
    grp = np.array([wl.group(b) for b in range(B)])
    Wc, Wh = synth.gate_weights(wl.seed)
    n_blk = wl.n_groups * (wl.prefix_len // 128) + 8
    cache = hsa.Cache(W, 2 * B + wl.n_groups, n_blk, Wc, Wh, max_blocks_per_state=wl.prefix_len // 128 + 2)
    lists, ck = [], {}
    for g in range(wl.n_groups):
        kids = np.flatnonzero(grp == g)
        stops = sorted(set(int(x) for x in P[kids]) | {PERIOD * (int(x) // PERIOD) for x in P[kids]})
        par = cache.state_alloc()
        done = 0
        for stop in stops:
            if stop > done:
                _append_device(cache, wl, [par], [int(kids[0])], [done], [stop])
                done = stop
            if stop > 0:
                ck[(g, stop)] = cache.state_checkpoint(par)[0]
        blocks = cache.block_table(par)
        cache.block_ref(blocks, +1)                      # the prefix entry
        cache.state_free(par)
        lists.append(blocks)
    off = np.concatenate([[0], np.cumsum([len(x) for x in lists])[:-1]]).astype(np.int64)
    flat = np.concatenate(lists).astype(np.int32)
    # replayed rows: zero [len - n_win, len); periodic [c, len); full none
    c = PERIOD * (P // PERIOD)
    lo = np.maximum(P - W, 0) if pol == "zero" else (c if pol == "periodic" else P)
    rows = P - lo
    T = int(rows.sum())
    cu = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
    if T:
        pos = np.concatenate([np.arange(a, b) for a, b in zip(lo, P)]).astype(np.int64)
        keys = np.concatenate([wl.key(b, np.arange(a, e)) for b, (a, e) in enumerate(zip(lo, P))]).astype(np.int64)
        kt, pt = torch.from_numpy(keys.astype(np.int32)).cuda(), torch.from_numpy(pos).cuda()
        K = torch.empty((T, 16, 128), dtype=torch.bfloat16, device="cuda")
        V = torch.empty_like(K)
        KI = torch.empty((T, 4, 64), dtype=torch.float32, device="cuda")
        for t, sid in ((K, synth.STREAM_K), (V, synth.STREAM_V), (KI, synth.STREAM_IDXK)):
            fill_rows(t, wl.seed, sid, keys=kt, pos=pt)
    torch.cuda.synchronize()

    def hit_batch():
        states = [cache.state_alloc() for _ in range(B)]
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        cache.prefix_attach(states, flat, P, offsets=off[grp])
        if pol in ("periodic", "full"):
            at = [int(c[b]) if pol == "periodic" else int(P[b]) for b in range(B)]
            rb = [b for b in range(B) if at[b] > 0]
            cache.state_restore_batch([states[b] for b in rb], [ck[(int(grp[b]), at[b])] for b in rb],
                                      [at[b] for b in rb])
        if T:
            cache.state_write(states, cu, lo, K, V, KI)
        e1.record()
        torch.cuda.synchronize()
        for s in states:
            cache.state_free(s)
        return e0.elapsed_time(e1)

    for _ in range(max(1, args.warmup)):
        hit_batch()
    times = [hit_batch() for _ in range(args.steps)]
    cache.timing_enable(["write"])
    hit_batch()
    kt_ = cache.timing_read()
    cache.timing_enable([])
    cache.close()
    ms = float(np.median(times))
    # algorithmic bytes: ring slots (and tail keys) read + written by restores and
    # replays, table rows written
    rest = np.minimum(c if pol == "periodic" else (P if pol == "full" else 0), W)
    repl = np.minimum(rows, W)
    write_b = int((repl * 2 * ROW).sum())
    alg = int((rest * 2 * ROW).sum()) + write_b + int((P // 128).sum()) * 8
    wr_ms = kt_["write"][0]
    return {
        "metric": f"prefix-hit setup, hits/s + achieved HBM GB/s, {pol} SWA policy",
        "value": B / (ms * 1e-3), "unit": "hits/s", "n_gpus": 1, "steps": len(times),
        "warmup": max(1, args.warmup), "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"prefix: {B} requests each starting at its fork length (16K-32K tokens) "
                               f"of one of {wl.n_groups} shared 32768-token prefixes held as blocks; "
                               f"n_win {W}; {pol} policy (checkpoint period {PERIOD})",
                   "batch": B, "n_win": W, "policy": pol, "replayed_tokens": T,
                   "parallelism": "single GPU"},
        "hbm_gbps": alg / (ms * 1e-3) / 1e9, "hbm_frac_of_peak": alg / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "bytes_per_step": alg,
        "roofline": {"bound": "hbm", "kernel": "k_bulk_write" if T else "k_copy_segs (restore)",
                     "achieved": (write_b / (wr_ms * 1e-3) / 1e9) if (T and wr_ms) else alg / (ms * 1e-3) / 1e9,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": ((write_b / (wr_ms * 1e-3) / 1e9) if (T and wr_ms) else alg / (ms * 1e-3) / 1e9)
                     / PEAK_HBM_GBS,
                     "traffic": None, "avg_launch_us": wr_ms * 1e3 if T else None,
                     "algorithmic_bytes_per_launch": write_b if T else alg,
                     "measured": "HIP event pair on the k_bulk_write dispatch of one batch" if T
                                 else "events around the whole batch"},
    }


# ------------------------------------------------------------------ CPU baseline (the oracle)

def _oracle_worker(job):
    """One host worker of the CPU baseline: build the oracle state of its requests
    (untimed), wait for the others, then run decode steps of its requests until the
    budget is spent. Returns (tokens, seconds)."""
    from threadpoolctl import threadpool_limits

    from oracle import Oracle

    index, reqs, budget_s, max_steps, barrier = job
    wl = workloads.make(index)
    Wc, Wh = synth.gate_weights(wl.seed)
    L0 = wl.prefill.astype(np.int64)
    with threadpool_limits(1):
        o = Oracle(wl.n_win, Wc, Wh, len(reqs), int((L0[reqs] // 128).sum()) + len(reqs) * (max_steps // 128 + 2))
        st = {}
        for b in reqs:
            st[b] = o.state_alloc()
            pos = np.arange(L0[b])
            key = np.full(pos.shape, b, np.uint64)
            K = synth.bf16_bits_to_f32(synth.tokens_bf16(wl.seed, synth.STREAM_K, key, pos))
            V = synth.bf16_bits_to_f32(synth.tokens_bf16(wl.seed, synth.STREAM_V, key, pos))
            KI = synth.tokens_f32(wl.seed, synth.STREAM_IDXK, key, pos)
            o.append([st[b]], [(K, V, KI)])
        steps_in = {}                                 # each request's decode inputs, by step
        for b in reqs:
            p = L0[b] + np.arange(max_steps)
            key = np.full(p.shape, b, np.uint64)
            steps_in[b] = (synth.bf16_bits_to_f32(synth.tokens_bf16(wl.seed, synth.STREAM_K, key, p)),
                           synth.bf16_bits_to_f32(synth.tokens_bf16(wl.seed, synth.STREAM_V, key, p)),
                           synth.tokens_f32(wl.seed, synth.STREAM_IDXK, key, p),
                           synth.bf16_bits_to_f32(synth.tokens_bf16(wl.seed, synth.STREAM_Q, key, p)),
                           synth.tokens_f32(wl.seed, synth.STREAM_QI, key, p))
        inputs = [[tuple(a[t:t + 1] for a in steps_in[b][:3]) + (steps_in[b][3][t], steps_in[b][4][t])
                   for b in reqs] for t in range(max_steps)]
        barrier.wait()
        t0 = time.perf_counter()
        tokens = 0
        for t in range(max_steps):
            for b, (K, V, KI, q, qi) in zip(reqs, inputs[t]):
                o.append([st[b]], [(K, V, KI)])
                idx, _ = o.topk(st[b], qi, wl.topk)
                o.attend(st[b], q, idx, wl.topk)
            tokens += len(reqs)
            if time.perf_counter() - t0 > budget_s:
                break
        return tokens, time.perf_counter() - t0


def cpu_baseline(args, budget_s: float = 10.0) -> dict:
    """The oracle, as it stands, on the host's cores: the batch's requests split over
    worker processes (one BLAS thread each), each running decode steps of its
    requests (append with seals, indexer top-k, attention) for about budget_s."""
    import multiprocessing as mp

    wl = workloads.make(args.workload)
    visible = len(os.sched_getaffinity(0))
    # the host's share of cores for this GPU: the affinity set, capped by the thread
    # count the environment grants (OMP_NUM_THREADS)
    share = int(os.environ.get("OMP_NUM_THREADS", visible) or visible)
    workers = max(1, min(visible, share, wl.batch))
    groups = [list(range(w, wl.batch, workers)) for w in range(workers)]
    ctx = mp.get_context("spawn")            # the workers never touch the GPU
    with ctx.Manager() as mgr:
        barrier = mgr.Barrier(workers)
        with ctx.Pool(workers) as pool:
            res = pool.map(_oracle_worker, [(args.workload, g, budget_s, 3072, barrier) for g in groups])
    tokens = sum(r[0] for r in res)
    secs = max(r[1] for r in res)
    steps = [r[0] // len(g) for r, g in zip(res, groups)]
    return {"value": tokens / secs, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "cpus_visible": visible, "blas_threads_per_worker": 1,
            "sample": f"all {wl.batch} requests over {workers} worker processes (one BLAS thread each); "
                      f"{min(steps)}-{max(steps)} decode steps per request (append with seals, indexer "
                      f"top-k, attention; fp64 NumPy) in {secs:.1f} s; prefill state built untimed"}


# ------------------------------------------------------------------ counters

def copy_calibration(args):
    """A plain copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = 256 << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "launches": 3}))


def summarize_counters(args):
    """Read rocprofv3 --pmc counter_collection CSVs (FETCH_SIZE, WRITE_SIZE, in KiB per
    dispatch) for the copy calibration and the bench, and write profiles/traffic.json."""
    import csv
    d = args.counters
    rows = []
    dirs = d.split(",")
    for p in [q for dd in dirs for q in glob.glob(os.path.join(dd, "**", "*counter_collection.csv"),
                                                  recursive=True)]:
        with open(p) as fh:
            for r in csv.DictReader(fh):
                r["_file"] = p
                rows.append(r)
    if not rows:
        raise SystemExit(f"no counter_collection.csv under {d}")

    def per_kernel(counter, match):
        vals = [float(r["Counter_Value"]) for r in rows
                if r.get("Counter_Name") == counter and match(r.get("Kernel_Name", ""))]
        return (sum(vals) / len(vals), len(vals)) if vals else (None, 0)

    copy_bytes = 256 << 20
    # the calibration copy (torch copy_ of 256 MiB on the device) runs as the runtime's
    # copyBuffer kernel; the bench's own setup copies are excluded by the file name
    is_copy = lambda n: "copyBuffer" in n
    def per_copy(counter):
        vals = [float(r["Counter_Value"]) for r in rows if r.get("Counter_Name") == counter
                and is_copy(r.get("Kernel_Name", "")) and "copy_counter" in os.path.basename(r["_file"])]
        return sum(vals) / len(vals) if vals else None
    cf, cw = per_copy("FETCH_SIZE"), per_copy("WRITE_SIZE")
    try:
        out = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        out = {}
    if "kernels" not in out:   # an older single-workload file
        out = {}
    cal = out.get("calibration", {})
    if cf and cw:   # this set of runs has its own calibration
        cal = {"copy_fetch_kib": cf, "copy_write_kib": cw, "copy_bytes": copy_bytes,
               "fetch_scale": copy_bytes / (cf * 1024), "write_scale": copy_bytes / (cw * 1024)}
    out["calibration"] = cal
    sf, sw = cal.get("fetch_scale"), cal.get("write_scale")
    wl_out = out.setdefault("kernels", {})
    key = traffic_key(args.counters_workload, args)   # the counter runs' formats: --entries/--index/--kv
    entries, index, kv = storage_formats(args)
    wl_out[key] = {}
    for name, sym in KERNEL_SYMBOL.items():
        # the symbol, possibly with template arguments (k_step1<false>(...))
        hit = lambda n, s=sym: (s + "(") in n or (s + "<") in n
        f, nf = per_kernel("FETCH_SIZE", hit)
        w, nw = per_kernel("WRITE_SIZE", hit)
        if not nf:
            continue
        ent = {"fetch_kib": f, "write_kib": w, "dispatches": nf, "src_sha": src_hash(name),
               "entries": entries, "index": index, "kv": kv, "env": launch_env()}
        if sf and sw and f is not None and w is not None:
            ent["traffic_bytes_per_launch"] = f * 1024 * sf + w * 1024 * sw
        wl_out[key][sym] = ent
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    json.dump(out, open(TRAFFIC_FILE, "w"), indent=1)
    print(json.dumps(out, indent=1))


# ------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--repeats", type=int, default=5,
                    help="timed passes of --steps steps, each on fresh copies; the median is reported")
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5],
                    help="1 l130, 2 b32 (the headline), 3 prefix, 4 bulk append, 5 long")
    ap.add_argument("--kernel", default=None, help="time this kernel in the timed region")
    ap.add_argument("--copies", type=int, default=None,
                    help="identical cache instances the steps rotate over (defeats the 256 MB "
                         "last-level cache between steps)")
    ap.add_argument("--entries", default="bf16", choices=["bf16", "fp8"],
                    help="storage format of the C4 entries (bf16, or FP8 E4M3 with a per-head scale)")
    ap.add_argument("--kv", default="bf16", choices=["bf16", "fp8"],
                    help="storage of SWA ring tokens and HCA entries (bf16, or FP8 E4M3 with a "
                         "per-head scale)")
    ap.add_argument("--index", default="f32", choices=["f32", "mxfp4"],
                    help="storage format of sealed indexer keys (fp32, or MXFP4 with E8M0 block scales)")
    ap.add_argument("--hit", default=None, choices=["zero", "periodic", "full"],
                    help="time a batch of prefix hits on the prefix workload under this SWA policy")
    ap.add_argument("--layers", default=None,
                    help="a layer stack: comma-separated types (mixed, swa, csa, hca), each step "
                         "runs every layer")
    ap.add_argument("--layer-repeat", type=int, default=1, help="repeat the --layers pattern")
    ap.add_argument("--c4-mode", default="sealed", choices=["sealed", "eager"],
                    help="when C4 entries exist: at block seal, or at every completed group of 4")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--counters", default=None, help="comma-separated rocprofv3 --pmc output dirs")
    ap.add_argument("--counters-workload", default="b32")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the library has no multi-GPU "
              "path: the cache shards by request, see the design notes.", file=sys.stderr)
        sys.exit(2)
    if args.counters:
        summarize_counters(args)
        return
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration(args)
        return
    args.warmup = max(args.warmup, 2)
    if args.hit:
        print(json.dumps(run_hits(args)), flush=True)
        return
    res = run_bulk(args) if args.workload == 4 else run_decode(args)
    if not args.no_cpu_baseline and args.workload == 2 and args.entries == "bf16" \
            and args.index == "f32" and not args.layers and args.c4_mode == "sealed" and args.kv == "bf16":
        res["cpu_baseline"] = cpu_baseline(args)
    res["measured_roof"] = measured_roof()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
