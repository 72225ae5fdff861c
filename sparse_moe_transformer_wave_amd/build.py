"""Compiles the in-tree native libraries for gfx950.

  libflint_moe.so          the C-ABI MoE library (csrc/*.hip)            hipcc
  datagen/libflint_gen_device.so   device-side pool generator            hipcc
  datagen/libflint_gen_host.so     host-side seeded generator            gcc
Every HIP source is built with packed-fp32 instruction selection switched off.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libflint_moe.so")
GEN_DEV = os.path.join(HERE, "datagen", "libflint_gen_device.so")
BUILD_DIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument"]
SOURCES = ["api.hip", "route.hip", "permute.hip", "gemv.hip", "gemm.hip", "decode1.hip", "decode_few.hip"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed: %s\n%s" % (" ".join(cmd), r.stdout))
    return r.stdout


def _hip_objects(sources, src_dir, tag):
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs, cmds = [], []
    for s in sources:
        o = os.path.join(BUILD_DIR, "%s_%s.o" % (tag, os.path.splitext(s)[0]))
        objs.append(o)
        cmds.append([HIPCC] + HIP_FLAGS + ["-c", os.path.join(src_dir, s), "-o", o])
    with cf.ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
        list(ex.map(_run, cmds))
    return objs


def _link(objs, out):
    tmp = out + ".tmp%d" % os.getpid()
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, out)


def build_moe():
    _link(_hip_objects(SOURCES, CSRC, "moe"), LIB)
    return LIB


def build_gen_device():
    _link(_hip_objects(["gen_device.hip"], os.path.join(HERE, "datagen"), "gen"), GEN_DEV)
    return GEN_DEV


def build_all():
    from . import datagen
    with cf.ThreadPoolExecutor(max_workers=2) as ex:
        f1 = ex.submit(build_moe)
        f2 = ex.submit(build_gen_device)
        f1.result()
        f2.result()
    datagen.build(force=True)
    return [LIB, GEN_DEV]


if __name__ == "__main__":
    print(build_all())
