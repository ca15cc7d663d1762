"""The C-ABI libraries load and export every symbol include/*.h declares (no GPU
needed: nothing here launches work)."""

import ctypes
import glob
import os
import re

import pytest

from heterogeneous_sparse_attention_amd import LIB_PATH, SIGNATURES
from heterogeneous_sparse_attention_amd.host import HOST_LIB_PATH
from synth.device import SYNTH_LIB_PATH


def declared(root, header):
    txt = open(os.path.join(root, "include", header)).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(hsa_\w+)\s*\(", txt)))


def test_headers_declare_the_boundary(root):
    names = declared(root, "hsa.h")
    for n in ("hsa_create", "hsa_destroy", "hsa_state_alloc", "hsa_state_free", "hsa_append_kv",
              "hsa_compress_flush", "hsa_block_table_share", "hsa_indexer_topk",
              "hsa_decode_attend", "hsa_decode_step"):
        assert n in names
    assert declared(root, "hsa_synth.h") == ["hsa_roof_read", "hsa_synth_rows"]


def test_libhsa_exports_every_declared_symbol(root):
    assert os.path.exists(LIB_PATH), "run the build first"
    lib = ctypes.CDLL(LIB_PATH)
    for n in declared(root, "hsa.h"):
        assert hasattr(lib, n), n
    # the Python binding covers every declared entry point
    for n in declared(root, "hsa.h"):
        assert n in SIGNATURES or n in ("hsa_status_str", "hsa_last_error"), n


def test_synth_lib_exports(root):
    lib = ctypes.CDLL(SYNTH_LIB_PATH)
    for n in declared(root, "hsa_synth.h"):
        assert hasattr(lib, n)


def test_status_strings():
    lib = ctypes.CDLL(LIB_PATH)
    lib.hsa_status_str.restype = ctypes.c_char_p
    assert lib.hsa_status_str(0) == b"ok"
    assert lib.hsa_status_str(-2) == b"Block Cache full"


def test_every_header_is_checked(root):
    assert sorted(os.path.basename(p) for p in glob.glob(os.path.join(root, "include", "*.h"))) == \
        ["hsa.h", "hsa_synth.h"]


def test_product_path_does_not_import_oracle(root):
    pkg = os.path.join(root, "heterogeneous_sparse_attention_amd")
    for p in glob.glob(os.path.join(pkg, "**", "*.*"), recursive=True):
        if p.endswith((".py", ".cpp", ".hip", ".h")):
            txt = open(p, errors="replace").read()
            assert "import oracle" not in txt and "from oracle" not in txt, p


def test_state_list_marshalling():
    """The per-step state list reaches the C ABI as host int32 values, whether it is
    a list or an array; values outside int32 are refused, not wrapped."""
    import numpy as np
    from heterogeneous_sparse_attention_amd import _host_i32_fast
    for ids in ([3, 0, 7, 2 ** 31 - 1], np.array([3, 0, 7, 2 ** 31 - 1], np.int64), (5,)):
        n, addr, keep = _host_i32_fast(ids)
        got = np.ctypeslib.as_array((ctypes.c_int32 * n).from_address(addr))
        assert n == len(ids) and np.array_equal(got, np.asarray(ids, np.int64))
    with pytest.raises(OverflowError):
        _host_i32_fast([2 ** 31])
    # arrays too: an int64 id past int32 must not wrap onto a valid id
    for bad in (np.array([2 ** 32 + 3], np.int64), np.array([1, -(2 ** 31) - 1], np.int64),
                np.array([2 ** 31], np.uint64)):
        with pytest.raises(OverflowError):
            _host_i32_fast(bad)
    from heterogeneous_sparse_attention_amd import _host_i32
    with pytest.raises(OverflowError):
        _host_i32(np.array([2 ** 31, 2 ** 32 + 3], np.int64))
    a, _ = _host_i32(np.array([-(2 ** 31), 2 ** 31 - 1], np.int64))
    assert a.dtype == np.int32 and a.tolist() == [-(2 ** 31), 2 ** 31 - 1]
