"""Builds libiqlher.so (the HIP kernels and the C ABI) for gfx950, in-tree,
and libiqlh_probes.so (measurement probes run by bench.py --probe, not part
of the step).

Usage: python offline_rl_step_amd/build.py   (runs without importing the package,
which would load the library being rebuilt)
"""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libiqlher.so")
PROBE_LIB = os.path.join(HERE, "libiqlh_probes.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


# Per-file flags, each measured: the reduction / SAXPY and Adam launches
# (step.hip) and the PER passes (per.hip) are chains of dependent loads, and
# the ILP-first scheduler is faster for them (slower for the forward/backward
# kernel).  These files raise a wave's priority while it issues its
# vector-memory loads (s_setprio), so that its loads go out ahead of the
# other waves' arithmetic.
FILE_FLAGS = {
    "step.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp", "-mllvm", "-amdgpu-set-wave-priority"],
    "per.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp", "-mllvm", "-amdgpu-set-wave-priority"],
    "iql.hip": ["-mllvm", "-amdgpu-set-wave-priority"],
}


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def build(verbose=False, jobs=8):
    """Compile every .hip source to an object, then link the shared library."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs = []
    objs = []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-I", os.path.join(ROOT, "include"), "-c",
               src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            _wait(procs)
            procs = []
    _wait(procs)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout)
    os.replace(tmp, LIB)
    build_probes(verbose)
    return LIB


def build_probes(verbose=False):
    """The probe library: one source, compiled and linked in one step."""
    src = os.path.join(HERE, "probes", "probes.hip")
    tmp = PROBE_LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-shared", src, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("probe library build failed:\n" + r.stdout)
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def _wait(procs):
    errors = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        if p.returncode != 0:
            errors.append(f"{os.path.basename(src)}:\n{text}")
        elif text.strip():
            sys.stderr.write(text)
    if errors:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errors))


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
