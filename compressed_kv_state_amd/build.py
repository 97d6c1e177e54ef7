"""Build the gfx950 C-ABI library libkvm.so in-tree with hipcc.

    python -m compressed_kv_state_amd.build

Compiles csrc/kvm_kernels.hip (device code) and csrc/kvm_api.cpp (host ABI)
for gfx950 only and links them into compressed_kv_state_amd/libkvm.so.

Packed FP32 (v_pk_fma_f32, v_pk_mul_f32, v_pk_add_f32) is kept out of the
device code: the target feature is switched off with
`-Xclang -target-feature -Xclang -packed-fp32-ops`.  The device compile honours
it; the host compile does not know the feature and says so in a warning, which
is left in the log.  As a check that does not depend on the flag, the device
assembly of the kernels is generated beside the object and the build fails if
any packed FP32 instruction appears in it.
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkvm.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wno-unused-command-line-argument",
]
SOURCES = ["kvm_kernels.hip", "kvm_backward.hip", "kvm_proj.hip", "kvm_api.cpp"]


PACKED_FP32 = re.compile(r"\bv_pk_(fma|mul|add)_f32\b")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}")
    return r.stdout


def _check_no_packed_fp32(asm_path: str):
    with open(asm_path) as f:
        hits = [l.strip() for l in f if PACKED_FP32.search(l)]
    if hits:
        raise RuntimeError(f"packed FP32 instructions in {asm_path}: {hits[:5]} ({len(hits)} in all)")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    asms = []
    for src in SOURCES:
        base = src.rsplit(".", 1)[0]
        obj = os.path.join(BUILD, base + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmds.append([HIPCC, *COMMON, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
        if src.endswith(".hip"):
            asm = os.path.join(BUILD, base + ".gfx950.s")
            cmds.append([HIPCC, *COMMON, *lang, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", asm])
            asms.append(asm)
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        outs = list(ex.map(_run, cmds))
    for asm in asms:
        _check_no_packed_fp32(asm)
    tmp = LIB + ".tmp"
    outs.append(_run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]))
    os.replace(tmp, LIB)
    log = "\n".join(o.strip() for o in outs if o.strip())
    if log:
        print(log, file=sys.stderr if not verbose else sys.stdout)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
