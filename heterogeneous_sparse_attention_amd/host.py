"""Binding of libhsa_host.so: the host control plane alone (State slots, block ids,
tables, refcounts, seal planning), runnable without a GPU. The GPU library links
the same control.cpp."""

from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB_PATH = os.path.join(HERE, "libhsa_host.so")

_P, _I32, _I64, _U32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32
_lib = None


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(HOST_LIB_PATH):
            raise RuntimeError(f"{HOST_LIB_PATH} missing: run the build")
        lib = ctypes.CDLL(HOST_LIB_PATH)
        sig = {
            "hsah_create": (_P, [_I32, _I32, _I64, _I64]),
            "hsah_destroy": (None, [_P]),
            "hsah_state_alloc": (_I32, [_P, ctypes.POINTER(_I32)]),
            "hsah_state_free": (_I32, [_P, _I32]),
            "hsah_append": (_I32, [_P, _I32, _P, _P, _U32, _P, _I64, ctypes.POINTER(_I64)]),
            "hsah_flush": (_I32, [_P, _I32, _P, ctypes.POINTER(_I64)]),
            "hsah_share": (_I32, [_P, _I32, _I32]),
            "hsah_block_ref": (_I32, [_P, _P, _I64, _I32]),
            "hsah_attach": (_I32, [_P, _I32, _P, _I64]),
            "hsah_query": (_I32, [_P, _I32, ctypes.POINTER(_I64), ctypes.POINTER(_I64), ctypes.POINTER(_I32)]),
            "hsah_table": (_I32, [_P, _I32, _P, _I64, ctypes.POINTER(_I64)]),
            "hsah_refcount": (_I32, [_P, _I64]),
            "hsah_free_blocks": (_I64, [_P]),
            "hsah_balance": (_I64, [_I32, _P, _I64, _I32, _P, _I64, _I32, _I64, _P, _P]),
            "hsah_slices": (None, [_I32, _P, _I32, _I32, _I32, _P, _P]),
        }
        for n, (res, args) in sig.items():
            f = getattr(lib, n)
            f.restype = res
            f.argtypes = args
        _lib = lib
    return _lib


class HostControl:
    """Returns status codes instead of raising, so tests can compare error kinds."""

    def __init__(self, n_win, max_states, max_blocks, max_bps=0):
        self._lib = load()
        self._c = self._lib.hsah_create(n_win, max_states, max_blocks, max_bps)

    def __del__(self):
        if getattr(self, "_c", None):
            self._lib.hsah_destroy(self._c)
            self._c = None

    def state_alloc(self):
        s = _I32()
        st = self._lib.hsah_state_alloc(self._c, ctypes.byref(s))
        return st, s.value

    def state_free(self, s):
        return self._lib.hsah_state_free(self._c, int(s))

    def append(self, states, counts, defer=False):
        st = np.ascontiguousarray(np.asarray(states, np.int32).reshape(-1))
        cu = np.concatenate([[0], np.cumsum(np.asarray(counts, np.int64))]).astype(np.int64)
        cap = int(cu[-1] // 128 + 2 * len(st) + 4)
        seals = np.zeros(3 * cap, np.int64)
        n = _I64()
        r = self._lib.hsah_append(self._c, st.size, st.ctypes.data_as(_P), cu.ctypes.data_as(_P),
                                  1 if defer else 0, seals.ctypes.data_as(_P), cap, ctypes.byref(n))
        return r, [tuple(seals[3 * i:3 * i + 3]) for i in range(min(n.value, cap))] if r == 0 else []

    def flush(self, states):
        st = np.ascontiguousarray(np.asarray(states, np.int32).reshape(-1))
        n = _I64()
        return self._lib.hsah_flush(self._c, st.size, st.ctypes.data_as(_P), ctypes.byref(n))

    def share(self, src, dst):
        return self._lib.hsah_share(self._c, int(src), int(dst))

    def block_ref(self, blocks, delta):
        b = np.ascontiguousarray(np.asarray(blocks, dtype=np.int32).reshape(-1))
        return self._lib.hsah_block_ref(self._c, b.ctypes.data_as(_P), b.size, int(delta))

    def attach(self, dst, blocks, length):
        b = np.ascontiguousarray(np.asarray(blocks, dtype=np.int32).reshape(-1))
        return self._lib.hsah_attach(self._c, int(dst), b.ctypes.data_as(_P) if b.size else None, int(length))

    def query(self, s):
        L, nb, pend = _I64(), _I64(), _I32()
        r = self._lib.hsah_query(self._c, int(s), ctypes.byref(L), ctypes.byref(nb), ctypes.byref(pend))
        return r, (L.value, nb.value, pend.value)

    def table(self, s):
        n = _I64()
        self._lib.hsah_table(self._c, int(s), None, 0, ctypes.byref(n))
        ids = np.zeros(max(n.value, 1), np.int32)
        self._lib.hsah_table(self._c, int(s), ids.ctypes.data_as(_P), ids.size, ctypes.byref(n))
        return ids[:n.value].tolist()

    def refcount(self, b):
        return self._lib.hsah_refcount(self._c, int(b))

    def free_blocks(self):
        return self._lib.hsah_free_blocks(self._c)


def balance_wgs(slots, keys_a, lat_a=0, min_a=0, keys_b=None, lat_b=0, min_b=0):
    """Attention workgroups per request for one or two launch parts (launch_plan.h).
    Returns (handed out, wgs_a, wgs_b or None)."""
    lib = load()
    ka = np.ascontiguousarray(np.asarray(keys_a, np.int64))
    n = ka.size
    wa = np.zeros(n, np.int64)
    kb = wb = None
    if keys_b is not None:
        kb = np.ascontiguousarray(np.asarray(keys_b, np.int64))
        wb = np.zeros(n, np.int64)
    used = lib.hsah_balance(n, ka.ctypes.data_as(_P), lat_a, min_a, kb.ctypes.data_as(_P) if kb is not None else None,
                            lat_b, min_b, slots, wa.ctypes.data_as(_P), wb.ctypes.data_as(_P) if wb is not None else None)
    return used, wa, wb


def plan_slices(n_scores, k, slice_override=0, default_slice=16384):
    """Top-k slices of score rows (launch_plan.h): (first [n + 1], gmax, slice, k1)."""
    lib = load()
    ns = np.ascontiguousarray(np.asarray(n_scores, np.int64))
    first = np.zeros(ns.size + 1, np.int32)
    out = np.zeros(3, np.int32)
    lib.hsah_slices(ns.size, ns.ctypes.data_as(_P), k, slice_override, default_slice, first.ctypes.data_as(_P),
                    out.ctypes.data_as(_P))
    return first, int(out[0]), int(out[1]), int(out[2])
