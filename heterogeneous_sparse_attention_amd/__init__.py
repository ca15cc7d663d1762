"""Heterogeneous sparse-attention KV cache for MI355X (gfx950).

Thin Python binding of the C ABI in include/hsa.h: it checks tensor dtypes and
shapes and passes device pointers and the current HIP stream; every step of the
decode path runs in the library's HIP kernels. There is no Python or CPU
fallback: without the built library every call raises.

PyTorch supplies device memory and streams only.
"""

from __future__ import annotations

import array
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhsa.so")

H, D, HI, DI = 16, 128, 4, 64
MAX_TOPK = 4096
APPEND_DEFER_SEAL = 1

KERNELS = ("append", "seal", "write", "score", "select", "attend", "merge",
           "step1", "step2", "step3", "step4", "step2b")
TOPK_SORTED = 1
CREATE_POISON = 1
KERNEL_ID = {n: i for i, n in enumerate(KERNELS)}

_STATUS = {0: "ok", -1: "invalid argument", -2: "Block Cache full", -3: "no free State slot",
           -4: "lifecycle error", -5: "HIP runtime error"}


class HsaError(RuntimeError):
    def __init__(self, code: int, where: str, detail: str):
        super().__init__(f"{where}: {_STATUS.get(code, code)} ({code}): {detail}")
        self.code = code


class _Config(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("m_csa", ctypes.c_int32), ("m_hca", ctypes.c_int32),
                ("n_win", ctypes.c_int32), ("idx_heads", ctypes.c_int32),
                ("idx_dim", ctypes.c_int32), ("max_states", ctypes.c_int32),
                ("max_blocks", ctypes.c_int64), ("max_blocks_per_state", ctypes.c_int64),
                ("gate_csa", ctypes.POINTER(ctypes.c_float)),
                ("gate_hca", ctypes.POINTER(ctypes.c_float)),
                ("entry_format", ctypes.c_int32), ("index_format", ctypes.c_int32),
                ("n_layers", ctypes.c_int32), ("layer_types", ctypes.c_void_p),
                ("c4_mode", ctypes.c_int32), ("create_flags", ctypes.c_uint32),
                ("kv_format", ctypes.c_int32), ("reserved", ctypes.c_int32)]

ENTRY_FORMATS = {"bf16": 0, "fp8": 1}     # HSA_ENTRY_BF16, HSA_ENTRY_FP8
INDEX_FORMATS = {"f32": 0, "mxfp4": 1}    # HSA_INDEX_F32, HSA_INDEX_MXFP4
LAYER_TYPES = {"mixed": 0, "swa": 1, "csa": 2, "hca": 3}   # HSA_LAYER_*
C4_MODES = {"sealed": 0, "eager": 1}                       # HSA_C4_SEALED, HSA_C4_EAGER
KV_FORMATS = {"bf16": 0, "fp8": 1}                         # HSA_KV_BF16, HSA_KV_FP8


class _StateInfo(ctypes.Structure):
    _fields_ = [("len", ctypes.c_int64), ("n_blocks", ctypes.c_int64),
                ("csa_tail", ctypes.c_int32), ("hca_tail", ctypes.c_int32),
                ("swa_len", ctypes.c_int32), ("pending_seal", ctypes.c_int32)]


_lib = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_U32 = ctypes.c_uint32

# name -> argument types (all return int32 status)
SIGNATURES = {
    "hsa_create": [ctypes.POINTER(_Config), ctypes.c_int, ctypes.POINTER(_P)],
    "hsa_destroy": [_P],
    "hsa_state_alloc": [_P, ctypes.POINTER(_I32)],
    "hsa_state_free": [_P, _I32],
    "hsa_append_kv": [_P, _I32, _P, _P, _P, _P, _P, _U32, _P],
    "hsa_compress_flush": [_P, _I32, _P, _P],
    "hsa_block_table_share": [_P, _I32, _I32, _P],
    "hsa_indexer_topk": [_P, _I32, _P, _P, _I32, _U32, _P, _P, _P],
    "hsa_decode_attend": [_P, _I32, _P, _P, _P, _I32, _P, _P],
    "hsa_decode_step": [_P, _I32, _P, _P, _P, _P, _P, _P, _I32, _U32, _P, _P, _P, _P],
    "hsa_decode_step_noalloc": [_P, _I32, _P, _P, _P, _P, _P, _P, _I32, _U32, _P, _P, _P, _P],
    "hsa_noalloc_scratch_bytes": [_P],
    "hsa_state_query": [_P, _I32, ctypes.POINTER(_StateInfo)],
    "hsa_block_table_get": [_P, _I32, _P, _I64, ctypes.POINTER(_I64)],
    "hsa_block_refcount": [_P, _I32, ctypes.POINTER(_I32)],
    "hsa_export_block": [_P, _I32, _P, _P, _P, _P, _P, _P],
    "hsa_export_state": [_P, _I32, _P, _P, _P, _P],
    "hsa_export_c4_fp8": [_P, _I32, _P, _P, _P, _P, _P],
    "hsa_export_state_fp8": [_P, _I32, _P, _P, _P],
    "hsa_export_hca_fp8": [_P, _I32, _P, _P, _P],
    "hsa_fp8_quantize_rows": [_P, _I64, _P, _P, _P],
    "hsa_export_idx_mxfp4": [_P, _I32, _P, _P, _P],
    "hsa_block_ref": [_P, _P, _I64, _I32],
    "hsa_set_layer": [_P, _I32],
    "hsa_prefix_attach": [_P, _I32, _P, _P, _P, _I64, _P, _P],
    "hsa_state_write": [_P, _I32, _P, _P, _P, _P, _P, _P, _P],
    "hsa_checkpoint_bytes": [_P, _P],
    "hsa_state_checkpoint": [_P, _I32, _P, _P, _P],
    "hsa_state_restore": [_P, _I32, _P, _I64, _P],
    "hsa_state_restore_batch": [_P, _I32, _P, _P, _P, _P],
    "hsa_mxfp4_quantize_rows": [_P, _I64, _P, _P, _P],
    "hsa_timing_enable": [_P, _U32],
    "hsa_timing_read": [_P, _P, _P],
}


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libhsa.so (raises if it has not been built).

    torch is imported first so that the library binds to the HIP runtime torch
    already loaded (one runtime per process: the library shares torch's device
    memory and streams)."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m heterogeneous_sparse_attention_amd.build` "
                           "(there is no fallback)")
    lib = ctypes.CDLL(path)
    for name, argt in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = argt
        fn.restype = _I32
    lib.hsa_status_str.restype = ctypes.c_char_p
    lib.hsa_status_str.argtypes = [_I32]
    lib.hsa_last_error.restype = ctypes.c_char_p
    lib.hsa_last_error.argtypes = []
    _lib = lib
    return lib


def _check(code: int, where: str):
    if code != 0:
        raise HsaError(code, where, _lib.hsa_last_error().decode(errors="replace"))


def _stream(stream):
    import torch
    if stream is None:   # the current stream's handle (no Stream object: ~3 us less per call)
        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        if raw is not None:
            return ctypes.c_void_p(raw(torch.cuda.current_device()))
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


_I32_MIN, _I32_MAX = -(1 << 31), (1 << 31) - 1


def _host_i32(a):
    """Host int32 copy of ids; values outside int32 raise OverflowError (a cast
    would wrap them onto other, valid ids)."""
    a = np.asarray(a)
    if a.size and a.dtype != np.int32:
        if a.dtype.kind not in "iu":
            a = a.astype(np.int64)
        if int(a.min()) < _I32_MIN or int(a.max()) > _I32_MAX:
            raise OverflowError("an id does not fit int32")
    a = np.ascontiguousarray(a.astype(np.int32, copy=False).reshape(-1))
    return a, a.ctypes.data_as(ctypes.c_void_p)


def _host_i32_fast(a):
    """(length, address, owner) of a host int32 copy of a list or array of ids: the
    per-step calls take this path (array.array: about 1 us for 32 ids, against
    about 4 us through numpy's ctypes view)."""
    if isinstance(a, np.ndarray):
        b, _ = _host_i32(a)
        return b.size, b.ctypes.data, b
    buf = array.array("i", a)
    return len(buf), buf.buffer_info()[0], buf


def _host_i64(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.int64).reshape(-1))
    return a, a.ctypes.data_as(ctypes.c_void_p)


def _dev(t, dtype, shape, name):
    """Device pointer of a contiguous CUDA tensor of the given dtype and shape."""
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr() if t.numel() else 0)


class Cache:
    """One Block Cache + State Cache on one GPU (an hsa_ctx)."""

    def __init__(self, n_win: int, max_states: int, max_blocks: int, gate_csa, gate_hca,
                 max_blocks_per_state: int = 0, device: int = 0, entry_format: str = "bf16",
                 index_format: str = "f32", layer_types=None, c4_mode: str = "sealed",
                 poison: bool = False, kv_format: str = "bf16"):
        """layer_types: None (one heterogeneous layer) or a list of "mixed", "swa",
        "csa", "hca"; then gate_csa / gate_hca hold one [16][128] set per layer.
        poison: fill every pool and scratch buffer with NaN bytes when allocated
        (HSA_CREATE_POISON), so that reads of never-written slots show."""
        lib = load()
        if entry_format not in ENTRY_FORMATS:
            raise ValueError(f"entry_format must be one of {sorted(ENTRY_FORMATS)}")
        if index_format not in INDEX_FORMATS:
            raise ValueError(f"index_format must be one of {sorted(INDEX_FORMATS)}")
        if c4_mode not in C4_MODES:
            raise ValueError(f"c4_mode must be one of {sorted(C4_MODES)}")
        if kv_format not in KV_FORMATS:
            raise ValueError(f"kv_format must be one of {sorted(KV_FORMATS)}")
        self.kv_format = kv_format
        self.c4_mode = c4_mode
        types = ["mixed"] if layer_types is None else list(layer_types)
        if not types or any(t not in LAYER_TYPES for t in types):
            raise ValueError(f"layer_types must be a non-empty list of {sorted(LAYER_TYPES)}")
        nl = len(types)
        self._gc = np.ascontiguousarray(np.asarray(gate_csa, np.float32).reshape(nl * H * D))
        self._gh = np.ascontiguousarray(np.asarray(gate_hca, np.float32).reshape(nl * H * D))
        self._lt = np.ascontiguousarray(np.array([LAYER_TYPES[t] for t in types], np.int32))
        self.layer_types = types
        self.layer = 0
        cfg = _Config(H, D, 4, 128, n_win, HI, DI, max_states, max_blocks, max_blocks_per_state,
                      self._gc.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
                      self._gh.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
                      ENTRY_FORMATS[entry_format], INDEX_FORMATS[index_format], nl,
                      self._lt.ctypes.data_as(ctypes.c_void_p), C4_MODES[c4_mode],
                      CREATE_POISON if poison else 0, KV_FORMATS[kv_format], 0)
        self.entry_format = entry_format
        self.index_format = index_format
        ctx = ctypes.c_void_p()
        _check(lib.hsa_create(ctypes.byref(cfg), device, ctypes.byref(ctx)), "hsa_create")
        self._ctx = ctx
        self.n_win = n_win
        self.max_states = max_states
        self.max_blocks = max_blocks
        self.device = device

    def close(self):
        if getattr(self, "_ctx", None):
            _lib.hsa_destroy(self._ctx)
            self._ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *a):
        self.close()

    # -- State pool -------------------------------------------------------------
    def state_alloc(self) -> int:
        s = _I32()
        _check(_lib.hsa_state_alloc(self._ctx, ctypes.byref(s)), "hsa_state_alloc")
        return s.value

    def state_free(self, s: int):
        _check(_lib.hsa_state_free(self._ctx, int(s)), "hsa_state_free")

    # -- append / seal ------------------------------------------------------------
    def append_kv(self, states, cu_tokens, k, v, idx_k, defer: bool = False, stream=None):
        import torch
        st, stp = _host_i32(states)
        cu, cup = _host_i64(cu_tokens)
        if cu.size != st.size + 1:
            raise ValueError("cu_tokens must have len(states) + 1 entries")
        T = int(cu[-1]) if cu.size else 0
        kp = _dev(k, torch.bfloat16, (T, H, D), "k")
        vp = _dev(v, torch.bfloat16, (T, H, D), "v")
        ip = _dev(idx_k, torch.float32, (T, HI, DI), "idx_k")
        _check(_lib.hsa_append_kv(self._ctx, st.size, stp, cup, kp, vp, ip,
                                  APPEND_DEFER_SEAL if defer else 0, _stream(stream)),
               "hsa_append_kv")

    def compress_flush(self, states, stream=None):
        st, stp = _host_i32(states)
        _check(_lib.hsa_compress_flush(self._ctx, st.size, stp, _stream(stream)), "hsa_compress_flush")

    def block_table_share(self, src: int, dst: int, stream=None):
        _check(_lib.hsa_block_table_share(self._ctx, int(src), int(dst), _stream(stream)),
               "hsa_block_table_share")

    # -- layers ------------------------------------------------------------------------
    def set_layer(self, layer: int):
        """Data calls act on this layer from now on (appends go 0, 1, ..., n-1)."""
        _check(_lib.hsa_set_layer(self._ctx, int(layer)), "hsa_set_layer")
        self.layer = int(layer)

    # -- prefix hits (Zero / Periodic / Full SWA policies) ----------------------------
    def block_ref(self, blocks, delta: int):
        """Hold (+1) or release (-1) one reference of each listed block."""
        b, bp = _host_i32(blocks)
        _check(_lib.hsa_block_ref(self._ctx, bp, b.size, int(delta)), "hsa_block_ref")

    def prefix_attach(self, states, blocks, lengths, offsets=None, stream=None):
        """states[i] (empty) takes blocks[offsets[i] : offsets[i] + lengths[i] // 128]
        (offsets default to 0: every state attaches to the same list) and length
        lengths[i]; fill its window next. A single state and length are accepted."""
        st, stp = _host_i32([states] if np.isscalar(states) else states)
        ln, lnp = _host_i64([lengths] if np.isscalar(lengths) else lengths)
        off, offp = _host_i64(np.zeros(st.size, np.int64) if offsets is None else offsets)
        b, bp = _host_i32(blocks)
        if ln.size != st.size or off.size != st.size:
            raise ValueError("lengths and offsets need one entry per state")
        if np.any(off + ln // 128 > b.size):
            raise ValueError("prefix_attach needs length // 128 blocks from each offset")
        _check(_lib.hsa_prefix_attach(self._ctx, st.size, stp, lnp, bp, b.size, offp, _stream(stream)),
               "hsa_prefix_attach")

    def state_write(self, states, cu_tokens, pos0, k, v, idx_k, stream=None):
        """Replay raw tokens (rows cu[i] .. cu[i+1]) as positions pos0[i] .. of states[i]."""
        import torch
        st, stp = _host_i32(states)
        cu, cup = _host_i64(cu_tokens)
        p0, p0p = _host_i64(pos0)
        if cu.size != st.size + 1 or p0.size != st.size:
            raise ValueError("cu_tokens needs len(states) + 1 entries and pos0 len(states)")
        T = int(cu[-1]) if cu.size else 0
        kp = _dev(k, torch.bfloat16, (T, H, D), "k")
        vp = _dev(v, torch.bfloat16, (T, H, D), "v")
        ip = _dev(idx_k, torch.float32, (T, HI, DI), "idx_k")
        _check(_lib.hsa_state_write(self._ctx, st.size, stp, cup, p0p, kp, vp, ip, _stream(stream)),
               "hsa_state_write")

    def checkpoint_bytes(self) -> int:
        n = ctypes.c_int64()
        _check(_lib.hsa_checkpoint_bytes(self._ctx, ctypes.byref(n)), "hsa_checkpoint_bytes")
        return n.value

    def state_checkpoint(self, s: int, buf=None, stream=None):
        """Checkpoint of a state's window and tail into a device uint8 tensor (new if
        buf is None); returns (buf, length)."""
        import torch
        nb = self.checkpoint_bytes()
        if buf is None:
            buf = torch.empty((nb,), dtype=torch.uint8, device=f"cuda:{self.device}")
        n = ctypes.c_int64()
        _check(_lib.hsa_state_checkpoint(self._ctx, int(s), _dev(buf, torch.uint8, (nb,), "buf"),
                                         ctypes.byref(n), _stream(stream)), "hsa_state_checkpoint")
        return buf, n.value

    def state_restore(self, s: int, buf, length: int, stream=None):
        import torch
        nb = self.checkpoint_bytes()
        _check(_lib.hsa_state_restore(self._ctx, int(s), _dev(buf, torch.uint8, (nb,), "buf"), int(length),
                                      _stream(stream)), "hsa_state_restore")

    def state_restore_batch(self, states, bufs, lengths, stream=None):
        """hsa_state_restore of several states in one launch: states[i] takes the
        checkpoint bufs[i] (a device uint8 tensor) taken at lengths[i]."""
        import torch
        nb = self.checkpoint_bytes()
        st, stp = _host_i32(states)
        ln, lnp = _host_i64(lengths)
        if len(bufs) != st.size or ln.size != st.size:
            raise ValueError("states, bufs and lengths must have the same length")
        ptrs = (ctypes.c_void_p * max(1, st.size))(*[_dev(b, torch.uint8, (nb,), "bufs[i]").value for b in bufs])
        _check(_lib.hsa_state_restore_batch(self._ctx, int(st.size), stp, ctypes.cast(ptrs, ctypes.c_void_p),
                                            lnp, _stream(stream)), "hsa_state_restore_batch")

    # -- indexer top-k --------------------------------------------------------------
    def indexer_topk(self, states, q_idx, k: int, idx_out=None, score_out=None, sorted=False,
                     stream=None):
        import torch
        st, stp = _host_i32(states)
        n = st.size
        qp = _dev(q_idx, torch.float32, (n, HI, DI), "q_idx")
        if idx_out is None:
            idx_out = torch.empty((n, k), dtype=torch.int32, device=q_idx.device)
        op = _dev(idx_out, torch.int32, (n, k), "idx_out")
        sp = ctypes.c_void_p(0)
        if score_out is not None:
            sp = _dev(score_out, torch.float32, (n, k), "score_out")
        _check(_lib.hsa_indexer_topk(self._ctx, n, stp, qp, int(k), TOPK_SORTED if sorted else 0,
                                     op, sp, _stream(stream)), "hsa_indexer_topk")
        return idx_out, score_out

    # -- attention -----------------------------------------------------------------
    def decode_attend(self, states, q, topk, k: int, out=None, stream=None):
        import torch
        st, stp = _host_i32(states)
        n = st.size
        qp = _dev(q, torch.bfloat16, (n, H, D), "q")
        tp = ctypes.c_void_p(0)
        if k > 0:
            tp = _dev(topk, torch.int32, (n, k), "topk")
        if out is None:
            out = torch.empty((n, H, D), dtype=torch.float32, device=q.device)
        op = _dev(out, torch.float32, (n, H, D), "out")
        _check(_lib.hsa_decode_attend(self._ctx, n, stp, qp, tp, int(k), op, _stream(stream)),
               "hsa_decode_attend")
        return out

    def decode_step(self, states, k_new, v_new, idx_new, q, q_idx, k: int,
                    topk_out=None, score_out=None, out=None, sorted=False, stream=None,
                    noalloc: bool = False):
        """hsa_decode_step, or with noalloc=True hsa_decode_step_noalloc (scratch from
        the library's fixed buffer; the caller passes every output)."""
        import torch
        n, stp, _keep = _host_i32_fast(states)
        dev = q.device
        if topk_out is None:
            topk_out = torch.empty((n, k), dtype=torch.int32, device=dev)
        if out is None:
            out = torch.empty((n, H, D), dtype=torch.float32, device=dev)
        sp = ctypes.c_void_p(0)
        if score_out is not None:
            sp = _dev(score_out, torch.float32, (n, k), "score_out")
        fn, name = ((_lib.hsa_decode_step_noalloc, "hsa_decode_step_noalloc") if noalloc
                    else (_lib.hsa_decode_step, "hsa_decode_step"))
        _check(fn(
            self._ctx, n, stp,
            _dev(k_new, torch.bfloat16, (n, H, D), "k_new"),
            _dev(v_new, torch.bfloat16, (n, H, D), "v_new"),
            _dev(idx_new, torch.float32, (n, HI, DI), "idx_new"),
            _dev(q, torch.bfloat16, (n, H, D), "q"),
            _dev(q_idx, torch.float32, (n, HI, DI), "q_idx"),
            int(k), TOPK_SORTED if sorted else 0, _dev(topk_out, torch.int32, (n, k), "topk_out"), sp,
            _dev(out, torch.float32, (n, H, D), "out"), _stream(stream)), name)
        return topk_out, score_out, out

    # -- introspection -----------------------------------------------------------------
    def state_query(self, s: int) -> dict:
        info = _StateInfo()
        _check(_lib.hsa_state_query(self._ctx, int(s), ctypes.byref(info)), "hsa_state_query")
        return {f: getattr(info, f) for f, _ in _StateInfo._fields_}

    def block_table(self, s: int) -> list:
        n = _I64()
        _check(_lib.hsa_block_table_get(self._ctx, int(s), None, 0, ctypes.byref(n)), "hsa_block_table_get")
        ids = np.zeros(max(n.value, 1), np.int32)
        _check(_lib.hsa_block_table_get(self._ctx, int(s), ids.ctypes.data_as(ctypes.c_void_p),
                                        ids.size, ctypes.byref(n)), "hsa_block_table_get")
        return ids[:n.value].tolist()

    def refcount(self, b: int) -> int:
        rc = _I32()
        _check(_lib.hsa_block_refcount(self._ctx, int(b), ctypes.byref(rc)), "hsa_block_refcount")
        return rc.value

    def export_block(self, b: int, stream=None) -> dict:
        """bf16 arrays as uint16 bits; indexer keys as float32. With FP8 entries the C4
        entries come as E4M3 codes (csa_k_codes, csa_v_codes uint8 [32][16][128]) and
        per-head scales (csa_k_scale, csa_v_scale float32 [32][16]). With MXFP4 indexer
        keys they come as idx_codes uint8 [128][128] and idx_scales uint8 [128][8]
        (E8M0 bytes) instead of idx."""
        t = self.layer_types[self.layer]        # what the current layer keeps
        c4, hca = t in ("mixed", "csa"), t in ("mixed", "hca")
        fp8 = self.entry_format == "fp8" and c4
        mx4 = self.index_format == "mxfp4" and c4
        out = {}
        if hca and self.kv_format != "fp8":
            out["hca_k"] = np.zeros((H, D), np.uint16)
            out["hca_v"] = np.zeros((H, D), np.uint16)
        if c4 and not mx4:
            out["idx"] = np.zeros((128, HI, DI), np.float32)
        if c4 and not fp8:
            out["csa_k"] = np.zeros((32, H, D), np.uint16)
            out["csa_v"] = np.zeros((32, H, D), np.uint16)
        p = {n: a.ctypes.data_as(ctypes.c_void_p) for n, a in out.items()}
        _check(_lib.hsa_export_block(self._ctx, int(b), p.get("csa_k"), p.get("csa_v"), p.get("hca_k"),
                                     p.get("hca_v"), p.get("idx"), _stream(stream)), "hsa_export_block")
        if fp8:
            q = {"csa_k_codes": np.zeros((32, H, D), np.uint8), "csa_v_codes": np.zeros((32, H, D), np.uint8),
                 "csa_k_scale": np.zeros((32, H), np.float32), "csa_v_scale": np.zeros((32, H), np.float32)}
            pq = {n: a.ctypes.data_as(ctypes.c_void_p) for n, a in q.items()}
            _check(_lib.hsa_export_c4_fp8(self._ctx, int(b), pq["csa_k_codes"], pq["csa_v_codes"],
                                          pq["csa_k_scale"], pq["csa_v_scale"], _stream(stream)),
                   "hsa_export_c4_fp8")
            out.update(q)
        if hca and self.kv_format == "fp8":
            codes = np.zeros((2, H, D), np.uint8)
            sc = np.zeros((2, H), np.float32)
            _check(_lib.hsa_export_hca_fp8(self._ctx, int(b), codes.ctypes.data_as(ctypes.c_void_p),
                                           sc.ctypes.data_as(ctypes.c_void_p), _stream(stream)),
                   "hsa_export_hca_fp8")
            out.update({"hca_k_codes": codes[0], "hca_v_codes": codes[1], "hca_k_scale": sc[0],
                        "hca_v_scale": sc[1]})
        if mx4:
            q = {"idx_codes": np.zeros((128, HI * DI // 2), np.uint8),
                 "idx_scales": np.zeros((128, HI * DI // 32), np.uint8)}
            _check(_lib.hsa_export_idx_mxfp4(self._ctx, int(b), q["idx_codes"].ctypes.data_as(ctypes.c_void_p),
                                             q["idx_scales"].ctypes.data_as(ctypes.c_void_p), _stream(stream)),
                   "hsa_export_idx_mxfp4")
            out.update(q)
        return out

    def export_state(self, s: int, stream=None) -> dict:
        """The current layer's SWA ring and (layers with C4 entries) indexer tail. bf16
        KV: swa_k, swa_v uint16 bits [n_win][16][128]. FP8 KV: swa_k_codes, swa_v_codes
        uint8 [n_win][16][128] and swa_k_scale, swa_v_scale float32 [n_win][16]."""
        fp8 = self.kv_format == "fp8"
        out = {} if fp8 else {"swa_k": np.zeros((self.n_win, H, D), np.uint16),
                              "swa_v": np.zeros((self.n_win, H, D), np.uint16)}
        if self.layer_types[self.layer] in ("mixed", "csa"):
            out["idx_tail"] = np.zeros((128, HI, DI), np.float32)
        p = {n: a.ctypes.data_as(ctypes.c_void_p) for n, a in out.items()}
        _check(_lib.hsa_export_state(self._ctx, int(s), p.get("swa_k"), p.get("swa_v"), p.get("idx_tail"),
                                     _stream(stream)), "hsa_export_state")
        if fp8:
            codes = np.zeros((self.n_win, 2, H, D), np.uint8)
            sc = np.zeros((self.n_win, 2, H), np.float32)
            _check(_lib.hsa_export_state_fp8(self._ctx, int(s), codes.ctypes.data_as(ctypes.c_void_p),
                                             sc.ctypes.data_as(ctypes.c_void_p), _stream(stream)),
                   "hsa_export_state_fp8")
            out.update({"swa_k_codes": codes[:, 0], "swa_v_codes": codes[:, 1], "swa_k_scale": sc[:, 0],
                        "swa_v_scale": sc[:, 1]})
        return out

    # -- timing -----------------------------------------------------------------------
    def timing_enable(self, kernels=()):
        mask = 0
        for k in kernels:
            mask |= 1 << KERNEL_ID[k]
        _check(_lib.hsa_timing_enable(self._ctx, mask), "hsa_timing_enable")

    def timing_read(self) -> dict:
        ms = np.zeros(len(KERNELS), np.float64)
        n = np.zeros(len(KERNELS), np.int64)
        _check(_lib.hsa_timing_read(self._ctx, ms.ctypes.data_as(ctypes.c_void_p),
                                    n.ctypes.data_as(ctypes.c_void_p)), "hsa_timing_read")
        return {k: (float(ms[i]), int(n[i])) for i, k in enumerate(KERNELS)}


def fp8_quantize_rows(x, stream=None):
    """The FP8 entry quantisation alone (hsa_fp8_quantize_rows): device float32
    [n][128] -> (codes uint8 [n][128], scales float32 [n]) as device tensors."""
    import torch
    load()
    n = x.shape[0]
    codes = torch.empty((n, D), dtype=torch.uint8, device=x.device)
    scales = torch.empty((n,), dtype=torch.float32, device=x.device)
    _check(_lib.hsa_fp8_quantize_rows(_dev(x, torch.float32, (n, D), "x"), n,
                                      _dev(codes, torch.uint8, (n, D), "codes"),
                                      _dev(scales, torch.float32, (n,), "scales"), _stream(stream)),
           "hsa_fp8_quantize_rows")
    return codes, scales


def mxfp4_quantize_rows(x, stream=None):
    """The MXFP4 indexer key quantisation alone (hsa_mxfp4_quantize_rows): device
    float32 [n][256] -> (codes uint8 [n][128], E8M0 scale bytes uint8 [n][8]) as
    device tensors."""
    import torch
    load()
    n = x.shape[0]
    R = HI * DI
    codes = torch.empty((n, R // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((n, R // 32), dtype=torch.uint8, device=x.device)
    _check(_lib.hsa_mxfp4_quantize_rows(_dev(x, torch.float32, (n, R), "x"), n,
                                        _dev(codes, torch.uint8, (n, R // 2), "codes"),
                                        _dev(scales, torch.uint8, (n, R // 32), "scales"), _stream(stream)),
           "hsa_mxfp4_quantize_rows")
    return codes, scales
