"""Build libreplayssm.so (HIP for gfx950) in-tree, and the benchmark's bandwidth probes
(libreplayssm_probes.so, not part of the library's C ABI).

    python -m hybrid_model_ssm_amd.build            # build the library
    python -m hybrid_model_ssm_amd.build --verbose  # show the hipcc commands

Each source is compiled to an object in parallel, then linked with hipcc.  Packed
FP32 instructions are switched off for device code (``-packed-fp32-ops``); hipcc's
host pass warns that it does not know the feature, which is harmless.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libreplayssm.so")
PROBE_LIB = os.path.join(PKG, "libreplayssm_probes.so")
PROBE_SOURCES = [("probes.hip", "probes", [])]

# (source, object name, extra defines); the Mamba2 kernel templates are instantiated in
# slices (io dtype x replay mode x read copy, and the conventional kernels) that compile
# in parallel.
SOURCES = [("api.cpp", "api", []), ("mamba2_launch.hip", "mamba2_launch", []),
           # the GDN fold's matrix instructions accumulate in ordinary VGPRs, which keeps the
           # kernel at its occupancy (accumulation registers would count on top)
           ("gdn_kernels.hip", "gdn_kernels", ["-mllvm", "-amdgpu-mfma-vgpr-form"]),
           ("cursor_kernels.hip", "cursor_kernels", []), ("emulate_kernels.hip", "emulate_kernels", [])]
SOURCES += [("mamba2_inst.hip", f"mamba2_inst_io{io}_part{part}_lp{lp}",
             [f"-DRSSM_IO={io}", f"-DRSSM_PART={part}", f"-DRSSM_LP={lp}"])
            for io in (0, 1) for part in (0, 1, 2, 3) for lp in (0, 1, 2, 3)]
SOURCES += [("mamba2_inst.hip", f"mamba2_inst_io{io}_conv", [f"-DRSSM_IO={io}", "-DRSSM_PART=4"]) for io in (0, 1)]
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (expected /opt/rocm/bin/hipcc)")


def common_flags():
    return ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            "-Wno-unused-command-line-argument"]


def _compile(item, verbose):
    src, name, defines = item
    obj = os.path.join(BUILD, name + ".o")
    cmd = [hipcc(), *common_flags(), *defines, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib, verbose):
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking {os.path.basename(lib)} failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose=False, jobs=None):
    """Compile every source and link the library and the probe library; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    items = SOURCES + PROBE_SOURCES
    jobs = jobs or min(len(items), int(os.environ.get("MAX_JOBS", 0)) or os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), items))
    _link(objs[:len(SOURCES)], LIB, verbose)
    _link(objs[len(SOURCES):], PROBE_LIB, verbose)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    args = ap.parse_args(argv)
    print(build(verbose=args.verbose))


if __name__ == "__main__":
    sys.exit(main())
