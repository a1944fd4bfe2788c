"""Builds libexattn.so (HIP, gfx950) in-tree with hipcc, and the separate unit-rate
probe library libexattn_probes.so (see unit_probes.py; libexattn.so never loads it).

    python -m exact_attention_81_amd.build

Every HIP source is compiled with packed-fp32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); the host-only API file
is compiled with the same driver. The library lands next to this file, where
the binding looks for it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libexattn.so"
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

HIP_SOURCES = ["attn_fwd.hip", "attn_fwd_fp8.hip", "attn_fp8.hip", "attn_decode.hip", "attn_bwd.hip"]
HOST_SOURCES = ["exattn_api.cpp"]
PROBE_SOURCES = ["unit_probes.hip"]
PROBE_LIB_NAME = "libexattn_probes.so"

COMMON = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall", "-Wno-unused-function",
          "-Wno-inline-asm"]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-mfma-vgpr-form"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP toolchain is required to build libexattn.so")
    return path


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd)}")
    return r


def _link(cc, objs, tmp, name):
    out = os.path.join(PKG, name)
    tmp_out = os.path.join(tmp, name)
    _run([cc, "-shared", f"--offload-arch={ARCH}", "-Wl,--no-undefined", *objs, "-o", tmp_out])
    shutil.copyfile(tmp_out, out + ".tmp")
    os.replace(out + ".tmp", out)
    return out


def build_probes(verbose: bool = False) -> str:
    """Compile the unit-rate probes into libexattn_probes.so; returns its path."""
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="exattn_probes_") as tmp:
        objs = []
        for src in PROBE_SOURCES:
            obj = os.path.join(tmp, src + ".o")
            _run([cc, *COMMON, *DEVICE, "-c", os.path.join(CSRC, src), "-o", obj])
            objs.append(obj)
        out = _link(cc, objs, tmp, PROBE_LIB_NAME)
    if verbose:
        print(f"built {out}")
    return out


def build(verbose: bool = False) -> str:
    """Compile every source and link libexattn.so; returns its path."""
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="exattn_build_") as tmp:
        objs = []
        for src in HIP_SOURCES:
            obj = os.path.join(tmp, src + ".o")
            _run([cc, *COMMON, *DEVICE, "-c", os.path.join(CSRC, src), "-o", obj])
            objs.append(obj)
        for src in HOST_SOURCES:
            obj = os.path.join(tmp, src + ".o")
            _run([cc, *COMMON, "-x", "c++", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", "-c",
                  os.path.join(CSRC, src), "-o", obj])
            objs.append(obj)
        out = _link(cc, objs, tmp, LIB_NAME)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True)
    build_probes(verbose=True)
