"""Debug builds under AddressSanitizer and UndefinedBehaviorSanitizer (CPU
only): the fp64 oracle with every pin and edge case run against it, and the
host side of the C ABI (argument checks) with the ABI tests run against it.
Each runs in a child process with the sanitizer runtime preloaded, and any
report fails the test (halt on the first error)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def runtime(name):
    p = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


ASAN = runtime("libasan.so")
pytestmark = pytest.mark.skipif(ASAN is None or shutil.which("gcc") is None, reason="gcc sanitizer runtime missing")

ENV = {
    "LD_PRELOAD": ASAN or "",
    "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
    "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
}


def clang_runtime():
    """The ASan runtime of the clang that hipcc drives (the host pass of a
    .hip file is clang's, which gcc's runtime does not serve)."""
    import glob
    root = os.path.dirname(os.path.dirname(os.path.realpath(HIPCC)))
    hits = sorted(glob.glob(os.path.join(root, "lib", "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    return hits[-1] if hits else None


def child(code, timeout=900, preload=None):
    env = dict(os.environ)
    env.update(ENV)
    if preload:
        env["LD_PRELOAD"] = preload
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=timeout)
    assert r.returncode == 0, (r.stdout[-3000:] + r.stderr[-6000:])
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-6000:]
    return r.stdout


def test_oracle_pins_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared", "-pthread",
                    "-fno-fast-math", "-ffp-contract=off", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    os.path.join(ROOT, "oracle", "oracle.c"), "-o", lib, "-lm"], check=True)
    out = child("""
import sys, inspect
sys.path.insert(0, 'tests')
import pins, test_oracle_pins as t
from oracle import Oracle
orc = Oracle(%r)
for pin in pins.ALL_PINS:
    pin(orc)
n = 0
for name, fn in sorted(vars(t).items()):
    if name.startswith('test_') and 'orc' in inspect.signature(fn).parameters:
        params = inspect.signature(fn).parameters
        if len(params) == 1:
            fn(orc); n += 1
import numpy as np
# empty and degenerate sizes
assert orc.verify(np.zeros((0, 3, 1, 4), np.float32), np.zeros((0, 3, 1, 4), np.float32),
                  np.zeros((0, 3, 1, 4), np.float32), np.zeros((0, 3, 1), np.float32),
                  np.zeros((0, 3, 1), np.float32), np.zeros((0, 1, 4, 4), np.float32))[2] == 0
t0 = orc.select(np.zeros((2, 1, 5), np.float32), np.zeros((2, 0), np.int32))
assert list(t0[1]) == [-1, -1] and list(t0[2]) == [0, 0]
print('pins', len(pins.ALL_PINS), 'edge tests', n)
""" % lib)
    words = out.split()
    assert int(words[words.index("pins") + 1]) >= 18 and int(words[words.index("tests") + 1]) >= 8, out


@pytest.mark.skipif(not os.path.exists(HIPCC) or clang_runtime() is None, reason="hipcc or its ASan runtime missing")
def test_abi_checks_under_asan_ubsan(tmp_path):
    """The C ABI's host code (argument checks, workspace sizes) built with
    the sanitizers on the host pass only; the ABI tests, which never reach a
    kernel launch, run against it."""
    csrc = os.path.join(ROOT, "speculative_decoding_verify_amd", "csrc")
    objs = []
    for src in ("verify.hip", "commit.hip", "gather.hip", "read.hip", "select.hip", "ldv_api.hip"):
        obj = str(tmp_path / src.replace(".hip", ".o"))
        subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-fvisibility=hidden",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                        "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                        "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
                        "-I", os.path.join(ROOT, "include"), "-c", os.path.join(csrc, src), "-o", obj],
                       check=True, capture_output=True)
        objs.append(obj)
    lib = str(tmp_path / "libldv_san.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                    "-Xarch_host", "-fsanitize=undefined", "-shared-libsan"] + objs + ["-o", lib],
                   check=True, capture_output=True)
    out = child("""
import sys, inspect
sys.path.insert(0, 'tests')
import test_abi as t
from speculative_decoding_verify_amd import ldv
lib = ldv.load(%r)
n = 0
for name, fn in sorted(vars(t).items()):
    if name.startswith('test_') and list(inspect.signature(fn).parameters) == ['lib']:
        fn(lib); n += 1
print('abi tests', n)
""" % lib, preload=clang_runtime())
    n = int(out.split("abi tests")[1].split()[0])
    assert n >= 8, out
