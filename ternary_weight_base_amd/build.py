"""Build libtq.so in-tree: host packer (g++, OpenMP) + HIP kernels (hipcc, gfx950)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INC = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libtq.so")
ARCH = os.environ.get("TQ_OFFLOAD_ARCH", "gfx950")

# Packed-fp32 VALU ops are kept out of every device compile.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


NOISE = "is not a recognized feature for this target"


def _report(cmd, rc, out):
    if rc != 0:
        sys.stderr.write(out)
        raise RuntimeError("build step failed: " + " ".join(cmd))
    # keep real diagnostics, drop hipcc's host-pass notice about the device-only feature
    for line in out.splitlines():
        if NOISE not in line and line.strip():
            sys.stderr.write(line + "\n")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    _report(cmd, r.returncode, r.stdout + r.stderr)


def _run_parallel(cmds, jobs=None):
    """Run the compile commands, at most `jobs` at once (default: the CPUs this
    process may use, capped at 16)."""
    jobs = jobs or max(1, min(16, len(os.sched_getaffinity(0))))
    pending, running = list(cmds), []
    while pending or running:
        while pending and len(running) < jobs:
            c = pending.pop(0)
            running.append((c, subprocess.Popen(c, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                                text=True)))
        c, p = running.pop(0)
        out, _ = p.communicate()
        _report(c, p.returncode, out)


def build() -> str:
    bdir = os.path.join(HERE, "_build")
    os.makedirs(bdir, exist_ok=True)
    host_objs = []
    for src in ("tq_host.cpp", "tq_ternarize.cpp"):
        o = os.path.join(bdir, src.replace(".cpp", ".o"))
        _run(["g++", "-O2", "-std=c++17", "-fPIC", "-fopenmp", "-Wall", "-Wextra", "-I", INC,
              "-c", os.path.join(CSRC, src), "-o", o])
        host_objs.append(o)
    objs, cmds = [], []
    # kernel-argument preloading (-mllvm -amdgpu-kernarg-preload-count=16):
    # the leading scalar arguments of the launch-latency-bound kernels (the
    # quantisers, the GEMVs) arrive in SGPRs with the wave
    preload = ["-mllvm", "-amdgpu-kernarg-preload-count=16"]
    units = [(src, src.replace(".hip", ".o"), preload if src in ("tq_kernels.hip", "tq_gemv_mfma.hip",
                                                                   "tq_hadamard.hip") else [])
             for src in ("tq_kernels.hip", "tq_proj.hip", "tq_gemv_mfma.hip", "tq_hadamard.hip",
                         "tq_gemm.hip", "tq_stream.hip", "tq_noalloc.hip", "tq_workspace.hip")]
    # the projection kernel: one object per (packed format, activation form, output kind)
    for fmt, fname in ((0, "b3"), (1, "2b"), (2, "bp"), (3, "b3r")):
        for lx in (1, 0):
            for sums in (0, 1):
                obj = f"tq_proj_{fname}{'' if lx else '_sg'}{'_sums' if sums else ''}.o"
                # with kernel-argument preloading (tq_proj_kernel.h)
                units.append(("tq_proj_inst.hip", obj,
                              [f"-DTQ_INST_FMT={fmt}", f"-DTQ_INST_LX={lx}", f"-DTQ_INST_SUMS={sums}",
                               *preload]))
    # the projection kernel over 2..4 token rows (the batch decode stack and
    # its group-sum hook): one object per (multi-token format, activation
    # form, rows, output kind)
    for fmt, fname in ((0, "b3"), (1, "2b")):
        for lx in (1, 0):
            for mt in (2, 3, 4):
                for sums in (0, 1):
                    obj = f"tq_proj_{fname}{'' if lx else '_sg'}_r{mt}{'_sums' if sums else ''}.o"
                    units.append(("tq_proj_inst.hip", obj,
                                  [f"-DTQ_INST_FMT={fmt}", f"-DTQ_INST_LX={lx}", f"-DTQ_INST_MT={mt}",
                                   f"-DTQ_INST_SUMS={sums}", *preload]))
    # the persistent decode-token kernel: one object per packed format
    for fmt, fname in ((0, "b3"), (1, "2b"), (2, "bp")):
        units.append(("tq_stack.hip", f"tq_stack_{fname}.o", [f"-DTQ_STACK_FMT={fmt}"]))
    for src, obj, defs in units:
        o = os.path.join(bdir, obj)
        cmds.append(["hipcc", *HIP_FLAGS, *defs, "-I", INC, "-I", CSRC, "-c", os.path.join(CSRC, src),
                     "-o", o])
        objs.append(o)
    _run_parallel(cmds)
    tmp = LIB + ".tmp"
    _run(["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs, *host_objs,
          "-fopenmp=libgomp", "-lgomp"])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
