"""Builds libdvm.so (host encoder/fuser/C ABI + gfx950 VM kernels) in-tree."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdvm.so")

SOURCES = ["dvm_host.cpp", "verify.cpp", "vm_vector.hip", "vm_vector_wide.hip", "vm_mix.hip", "scratch_static.hip"]
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         # no packed-fp32 VALU forms in device code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]
# Device sources: the interpreter loop branches only on wave-uniform values
# (opcode, operand kinds, tile geometry), so its regions need no conversion
# to exec-masked form; skipping that keeps the tile registers in place across
# the opcode dispatch instead of copying them at every join.
DEVICE_FLAGS = ["-mllvm", "-structurizecfg-skip-uniform-regions=true"]


def build(verbose=False):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cmds, objs = [], []
    for src in SOURCES:
        obj = os.path.join(CSRC, os.path.splitext(src)[0] + ".o")
        extra = DEVICE_FLAGS if src.endswith(".hip") else []
        cmds.append([hipcc] + [f for f in FLAGS if f != "-shared"] + extra + ["-c", os.path.join(CSRC, src),
                                                                       "-I", os.path.join(ROOT, "include"),
                                                                       "-I", CSRC, "-o", obj])
        objs.append(obj)
    # the translation units compile independently: run them side by side
    procs = []
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    failed = []
    for src, pr in zip(SOURCES, procs):
        out, err = pr.communicate()
        if pr.returncode != 0:
            sys.stderr.write(out + err)
            failed.append(src)
    if failed:
        raise RuntimeError(f"compiling {', '.join(failed)} failed")
    tmp = LIB + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("linking libdvm.so failed")
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
