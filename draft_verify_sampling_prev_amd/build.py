"""Build libdspark.so (gfx950) in-tree with hipcc.

Every translation unit is compiled to an object in parallel, then linked into
``draft_verify_sampling_prev_amd/libdspark.so``; the load-only measurement
kernel (``csrc/dspark_probe.hip``) goes into its own
``libdspark_probe.so``, outside the library's ABI.  Flags:
  --offload-arch=gfx950                 MI355X only
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                        no packed fp32 VALU instructions
  -fhip-fp32-correctly-rounded-divide-sqrt
                                        IEEE fp32 division in the survival
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdspark.so")
PROBE_LIB = os.path.join(PKG, "libdspark_probe.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["dspark_api.hip", "dspark_draft.hip", "dspark_schedule.hip", "dspark_verify.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    probe_tmp = PROBE_LIB + ".tmp"
    cmds.append([HIPCC, *FLAGS, "-shared", os.path.join(CSRC, "dspark_probe.hip"), "-o", probe_tmp])
    with cf.ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 4)) as ex:
        outs = list(ex.map(_run, cmds))
    os.replace(probe_tmp, PROBE_LIB)
    tmp = LIB + ".tmp"
    outs.append(_run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]))
    os.replace(tmp, LIB)
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
