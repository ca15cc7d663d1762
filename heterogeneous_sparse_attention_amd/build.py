"""Build the native libraries in-tree.

  heterogeneous_sparse_attention_amd/libhsa.so       the cache (HIP, gfx950) + C ABI
  heterogeneous_sparse_attention_amd/libhsa_host.so  the host control plane alone (g++, CPU)
  synth/libhsa_synth.so                              GPU synthetic-input generator (harness)

`python -m heterogeneous_sparse_attention_amd.build` or build_all().
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# packed fp32 instructions are switched off in device code (-packed-fp32-ops)
HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

HIP_SOURCES = ["append_seal.hip", "indexer_topk.hip", "attend.hip", "step.hip", "noalloc.hip",
               "hsa.cpp", "control.cpp", "launch_plan.cpp"]

LIB = os.path.join(HERE, "libhsa.so")
HOST_LIB = os.path.join(HERE, "libhsa_host.so")
SYNTH_LIB = os.path.join(ROOT, "synth", "libhsa_synth.so")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    _run([HIPCC, *HIP_FLAGS, "-c", src, "-o", obj], verbose)
    return obj


def build_hip(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = [os.path.join(CSRC, s) for s in HIP_SOURCES]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


def build_synth(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    tmp = SYNTH_LIB + ".tmp"
    _run([HIPCC, *HIP_FLAGS, "-shared", os.path.join(ROOT, "synth", "synth_gen.hip"), "-o", tmp], verbose)
    os.replace(tmp, SYNTH_LIB)
    return SYNTH_LIB


def build_host(verbose: bool = False) -> str:
    tmp = HOST_LIB + ".tmp"
    _run(["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-Wall",
          os.path.join(CSRC, "control.cpp"), os.path.join(CSRC, "launch_plan.cpp"),
          os.path.join(CSRC, "host_api.cpp"), "-o", tmp], verbose)
    os.replace(tmp, HOST_LIB)
    return HOST_LIB


def build_selftest(out: str, verbose: bool = False) -> str:
    """Sanitizer build (host code only) of the control-plane self-test."""
    _run(["g++", "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
          os.path.join(CSRC, "control.cpp"), os.path.join(CSRC, "control_selftest.cpp"), "-o", out],
         verbose)
    return out


def build_all(verbose: bool = False) -> None:
    with cf.ThreadPoolExecutor(max_workers=3) as ex:
        futs = [ex.submit(build_hip, verbose), ex.submit(build_synth, verbose),
                ex.submit(build_host, verbose)]
        for f in futs:
            f.result()


def clean() -> None:
    shutil.rmtree(BUILD, ignore_errors=True)


if __name__ == "__main__":
    build_all(verbose="-v" in sys.argv)
    print("built", LIB, HOST_LIB, SYNTH_LIB)
