"""GPU side of the synthetic-input generator (binding of synth/libhsa_synth.so), and
the benchmark's streaming-read roof.

Produces on the device exactly what `synth.tokens_bf16` / `synth.tokens_f32`
produce on the host."""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
SYNTH_LIB_PATH = os.path.join(HERE, "libhsa_synth.so")
_lib = None


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(SYNTH_LIB_PATH):
            raise RuntimeError(f"{SYNTH_LIB_PATH} missing: run the build")
        lib = ctypes.CDLL(SYNTH_LIB_PATH)
        P = ctypes.c_void_p
        lib.hsa_synth_rows.restype = ctypes.c_int32
        lib.hsa_synth_rows.argtypes = [ctypes.c_uint64, ctypes.c_uint32, P, ctypes.c_uint32, P,
                                       ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                       P, P]
        lib.hsa_roof_read.restype = ctypes.c_int32
        lib.hsa_roof_read.argtypes = [P, ctypes.c_int64, P, ctypes.c_int32, P]
        _lib = lib
    return _lib


def roof_read(buf, out, blocks: int):
    """Enqueue the streaming read of the whole contiguous device tensor buf on the
    current stream; out: a device tensor of at least `blocks` int32 (the folds)."""
    import torch
    lib = load()
    assert buf.is_cuda and buf.is_contiguous() and out.is_cuda and out.numel() >= blocks
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    r = lib.hsa_roof_read(ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(),
                          ctypes.c_void_p(out.data_ptr()), blocks, st)
    if r != 0:
        raise RuntimeError(f"hsa_roof_read failed ({r})")


def fill_rows(out, seed: int, stream_id: int, *, key: int = 0, keys=None, pos0: int = 0, pos=None):
    """Fill a contiguous device tensor out[n][...]: bf16 (16x128 rows) or float32 (4x64 rows).

    keys / pos: optional device tensors (uint32 as int32, int64) with one entry per row.
    """
    import torch
    lib = load()
    assert out.is_cuda and out.is_contiguous()
    n = out.shape[0]
    row = out[0].numel() if n else (out.numel())
    as_bf16 = 1 if out.dtype == torch.bfloat16 else 0
    if not as_bf16:
        assert out.dtype == torch.float32
    kp = ctypes.c_void_p(keys.data_ptr()) if keys is not None else ctypes.c_void_p(0)
    pp = ctypes.c_void_p(pos.data_ptr()) if pos is not None else ctypes.c_void_p(0)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    r = lib.hsa_synth_rows(seed & 0xFFFFFFFFFFFFFFFF, stream_id, kp, key & 0xFFFFFFFF, pp, pos0, n, row,
                           as_bf16, ctypes.c_void_p(out.data_ptr()), st)
    if r != 0:
        raise RuntimeError(f"hsa_synth_rows failed ({r})")
    return out
