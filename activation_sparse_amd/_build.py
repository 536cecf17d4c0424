"""Build commands for every native part of the repository.

libpi.so (the HIP library, gfx950), libpi_host.so (the CPU side of the hybrid
layer), libsynth.so / libsynth_gpu.so (the
synthetic-input generator, host and device) and liboracle.so (the CPU
oracle, test infrastructure only).  Everything is built in-tree so the
shared objects travel with the source tree.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBPI = os.path.join(PKG, "libpi.so")

HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             # packed fp32 instructions stay off (the compiler would otherwise form them)
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

PI_SOURCES = ["pi_generic.hip", "pi_fast.hip", "pi_fc2.hip", "pi_mfma.hip", "pi_attn.hip", "pi_abi.hip"]
LIBHOST = os.path.join(PKG, "libpi_host.so")
# the host (CPU) operator: no target-wide vector flags (its AVX2 path is chosen at run time),
# no contraction of separate multiplies and adds (its sums have one fixed rounding order)
HOST_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-fopenmp", "-ffp-contract=off"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    return out


def build_libpi(jobs: int = 8) -> str:
    with tempfile.TemporaryDirectory() as tmp:
        objs = [os.path.join(tmp, s.replace(".hip", ".o")) for s in PI_SOURCES]
        cmds = [["hipcc", *HIP_FLAGS, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(PI_SOURCES, objs)]
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            list(ex.map(_run, cmds))
        tmp_so = LIBPI + ".tmp"
        _run(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp_so, *objs])
        os.replace(tmp_so, LIBPI)
    return LIBPI


ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_libpi_host() -> str:
    """libpi_host.so: the host operator and the hybrid executor, which drives libpi and the HIP
    runtime (so libpi.so must be built first; found next to it at run time)."""
    tmp_so = LIBHOST + ".tmp"
    _run(["g++", *HOST_FLAGS, "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", "-shared",
          os.path.join(CSRC, "pi_host.cpp"), os.path.join(CSRC, "pi_hybrid.cpp"), "-o", tmp_so,
          f"-L{PKG}", "-lpi", f"-L{ROCM}/lib", "-lamdhip64", "-Wl,-rpath,$ORIGIN", f"-Wl,-rpath,{ROCM}/lib"])
    os.replace(tmp_so, LIBHOST)
    return LIBHOST


def build_all() -> None:
    sys.path.insert(0, ROOT)
    import synth
    import oracle
    with ThreadPoolExecutor(max_workers=4) as ex:
        futs = [ex.submit(lambda: (build_libpi(), build_libpi_host())), ex.submit(synth.build_host),
                ex.submit(oracle.build), ex.submit(_run, synth.build_gpu_cmd())]
        for f in futs:
            f.result()


if __name__ == "__main__":
    build_all()
