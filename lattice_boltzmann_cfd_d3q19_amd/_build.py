"""Build liblbm.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

    python lattice_boltzmann_cfd_d3q19_amd/_build.py [-v]

Each translation unit is compiled to an object in parallel, then linked into
lattice_boltzmann_cfd_d3q19_amd/liblbm.so (in-tree, next to the binding).
The bandwidth probes the benchmark compares against (csrc/probes.hip) go
into a library of their own, libprobes.so, which the lattice never loads.
Floating-point contraction is off so the collision arithmetic is fixed by the
source (every layout and scheme then agrees bit for bit); packed fp32
instructions are disabled.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "liblbm.so")
PROBES_LIB = os.path.join(HERE, "libprobes.so")
SOURCES = ["launch_f32.hip", "launch_f64.hip", "compact_build.hip", "capi.cpp"]
PROBE_SOURCES = ["probes.hip"]
ARCH = os.environ.get("LBM_OFFLOAD_ARCH", "gfx950")


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Wno-unused-parameter",
          "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I" + os.path.join(ROOT, "include")]


def _compile(src, verbose, defines=()):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc(), "--offload-arch=" + ARCH, *COMMON, *["-D" + d for d in defines], "-x", "hip", "-c",
           os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if verbose and warn:
        print(warn)
    return obj


def _link(objs, out, verbose):
    cmd = [_hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", out + ".tmp", *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)


def build(verbose: bool = False, out: str = LIB, defines=(), probes: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + (PROBE_SOURCES if probes else [])
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 1)) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, verbose, defines), srcs)))
    _link([objs[s] for s in SOURCES], out, verbose)
    if probes:
        _link([objs[s] for s in PROBE_SOURCES], PROBES_LIB, verbose)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
