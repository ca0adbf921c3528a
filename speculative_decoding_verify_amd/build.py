"""Build the HIP library libldv.so (and the measurement probe libldv_peaks.so
and the test helpers libldv_checks.so) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libldv.so")
SOURCES = ["verify.hip", "commit.hip", "gather.hip", "read.hip", "select.hip", "ldv_api.hip"]
# the MFMA-rate probe of the measurement harness: a library of its own, so
# that libldv.so exports exactly the calls include/ldv.h declares
PEAKS_LIB = os.path.join(HERE, "libldv_peaks.so")
PEAKS_SOURCES = ["peaks.hip"]
# device helpers of the library run on caller data, for the tests only
CHECKS_LIB = os.path.join(HERE, "libldv_checks.so")
CHECKS_SOURCES = ["checks.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    # no packed fp32 arithmetic (v_pk_*_f32) on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False, jobs: int = 4) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [HIPCC] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        # hipcc's host pass does not know the packed-fp32 feature; drop that note
        err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed on %s:\n%s" % (src, err))
        if err.strip() and verbose:
            print(err, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES + PEAKS_SOURCES + CHECKS_SOURCES))
    nmain, npeaks = len(SOURCES), len(PEAKS_SOURCES)
    for lib, lobjs in ((LIB, objs[:nmain]), (PEAKS_LIB, objs[nmain:nmain + npeaks]),
                       (CHECKS_LIB, objs[nmain + npeaks:])):
        tmp = lib + ".tmp%d" % os.getpid()
        cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC"] + lobjs + ["-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
