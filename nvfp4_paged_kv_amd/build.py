"""Build the gfx950 HIP library (libnvfp4kv.so) in-tree with hipcc.

Every source is compiled for gfx950 only.  Packed-fp32 VALU forms are
disabled for all device code; the append translation unit additionally
disables fused multiply-add contraction, since its fp32 operation order is
part of the format's bit-exact contract.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libnvfp4kv.so")

ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", os.path.join(ROOT, "include"),
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument"]
# (source, object, extra flags): the prefill source is compiled as three
# shards (each instantiates a third of the kernels; compiled in parallel)
SOURCES = [
    ("append.hip", "append", ["-ffp-contract=off"]),
    ("prefill.hip", "prefill_0", ["-DNVFP4KV_PREFILL_SHARD=0"]),
    ("prefill.hip", "prefill_1", ["-DNVFP4KV_PREFILL_SHARD=1"]),
    ("prefill.hip", "prefill_2", ["-DNVFP4KV_PREFILL_SHARD=2"]),
    ("decode.hip", "decode", []),
    ("host.cpp", "host", ["-x", "hip"]),
]


def _hipcc():
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _compile(src, name, extra, defines):
    obj = os.path.join(BUILD, name + ".o")
    cmd = [_hipcc(), *COMMON, *extra, *defines, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stderr}")
    return obj


def build(out: str = LIB, defines=()) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(lambda e: _compile(e[0], e[1], e[2], list(defines)), SOURCES))
    tmp = out + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    return out


PEAK_LIB = os.path.join(PKG, "libnvfp4kv_peak.so")


def build_bench_helpers() -> str:
    """The achievable-peak probe (an MFMA-only loop) that bench.py loads."""
    cmd = [_hipcc(), *COMMON, "-shared", os.path.join(CSRC, "peak.hip"), "-o", PEAK_LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build failed:\n{' '.join(cmd)}\n{r.stderr}")
    return PEAK_LIB


def build_test_helpers() -> None:
    """The GPU probe library and the host build of the codec used by tests/."""
    tests = os.path.join(ROOT, "tests")
    cmds = [
        [_hipcc(), *COMMON, "-shared", os.path.join(tests, "gpu_probes.hip"), "-o",
         os.path.join(tests, "libnvfp4kv_probes.so")],
        ["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fPIC", "-shared",
         os.path.join(tests, "codec_host.cpp"), "-o", os.path.join(tests, "libcodec_host.so")],
    ]
    for cmd in cmds:
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"build failed:\n{' '.join(cmd)}\n{r.stderr}")


if __name__ == "__main__":
    print(build(defines=sys.argv[1:]))
    build_test_helpers()
    build_bench_helpers()
