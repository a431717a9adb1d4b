"""Builds librpa.so (the HIP kernels and the C ABI) and librpa_probes.so (the
measurement probes) in-tree with hipcc for gfx950; on request (--timeline)
also the measurement build librpa_timeline.so.

Run as ``python -m ragged_paged_kv_scatter_amd.build``, or call :func:`build`.
Every call recompiles."""
import os
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "librpa.so")
SOURCES = ["rpa_api.cpp", "scatter.hip", "plan.hip", "decode.hip", "prefill.hip", "slots.hip",
           "validate.hip"]
# measurement probes (include/rpa_probes.h), a library of their own
PROBES_LIB = os.path.join(HERE, "librpa_probes.so")
PROBES_SOURCES = ["probes.hip", "probes_vacc.hip"]
# per-source extra flags: the VGPR-accumulator copy of the MFMA-beside-VALU probe
EXTRA_FLAGS = {"probes_vacc.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"]}
# measurement build of librpa.so with the row kernels' per-wave clock stamps
# (RPA_WAVE_TIMELINE; read by bench.py --op timeline), built on request only
TIMELINE_LIB = os.path.join(HERE, "librpa_timeline.so")
ARCH = os.environ.get("RPA_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++20", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


def _compile(sources, obj_dir, jobs, verbose, defines=()):
    procs, objs = [], []
    for src in sources:
        obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmd = [hipcc(), *FLAGS, *EXTRA_FLAGS.get(src, []), *[f"-D{d}" for d in defines], "-c",
               os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        procs.append((src, cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                 stderr=subprocess.STDOUT, text=True)))
        while len([p for p in procs if p[2].poll() is None]) >= jobs:
            time.sleep(0.05)
    failed = []
    for src, cmd, p in procs:
        out, _ = p.communicate()
        if p.returncode != 0:
            failed.append((src, out))
        elif verbose and out.strip():
            print(f"[{src}]\n{out}")
    if failed:
        msg = "\n".join(f"--- {s} ---\n{o}" for s, o in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    return objs


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}")
    os.replace(tmp, lib)


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile and link librpa.so and librpa_probes.so; returns librpa.so's path."""
    obj_dir = os.path.join(HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    t0 = time.time()
    objs = _compile(SOURCES + PROBES_SOURCES, obj_dir, jobs, verbose)
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBES_LIB)
    if verbose:
        print(f"built {LIB} and {PROBES_LIB} in {time.time() - t0:.1f}s")
    return LIB


def build_timeline(verbose: bool = False, jobs: int = 8) -> str:
    """Compile and link librpa_timeline.so: librpa.so with the row kernels'
    per-wave clock stamps (a measurement build; the product is librpa.so)."""
    obj_dir = os.path.join(HERE, "_build", "timeline")
    os.makedirs(obj_dir, exist_ok=True)
    t0 = time.time()
    _link(_compile(SOURCES, obj_dir, jobs, verbose, defines=("RPA_WAVE_TIMELINE",)), TIMELINE_LIB)
    if verbose:
        print(f"built {TIMELINE_LIB} in {time.time() - t0:.1f}s")
    return TIMELINE_LIB


if __name__ == "__main__":
    if "--timeline" in sys.argv[1:]:
        build_timeline(verbose=True)
    else:
        build(verbose=True)
    sys.exit(0)
