"""The kernels' MFMA results reach memory only after enough wait states.

An MFMA writes its result registers some cycles after it issues; an
instruction that reads them earlier needs wait states in between, which the
compiler inserts.  On a path that enters a block through a taken branch the
compiler has been seen to emit too few (a store then wrote stale upper
registers), so the kernels are shaped to keep such stores and LDS writes in
straight-line code.  This test compiles each kernel source with the library's
flags to gfx950 assembly and, for every store and LDS write whose data an
MFMA produced, follows every path back to that MFMA (the preceding line, and
every branch that targets a label in between) and counts the wait states on
the shortest one.  Every such path must keep at least as many as the
straight-line code the compiler emits (8).  Verify and the in-block read store
MFMA registers directly (the check must find such stores there); gather moves
its results through other registers first, so for it the check only guards
against a change that would make it store them directly on a short path.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "speculative_decoding_verify_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
MIN_WAIT_STATES = 8
HORIZON = 40  # wait states beyond which no MFMA result is still in flight


def regs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def wait_states(line):
    t = line.strip()
    if not t or t.startswith(";") or t.startswith(".") or t.endswith(":"):
        return 0
    if t.startswith("s_nop"):
        return int(t.split()[1]) + 1
    return 1


def branches_to(body):
    """label -> indices of the branch instructions that target it."""
    out = {}
    for j, line in enumerate(body):
        m = re.match(r"s_(?:c)?branch\w*\s+(\.LBB\w+)$", line.strip())
        if m:
            out.setdefault(m.group(1), []).append(j)
    return out


def min_wait(body, targets, n, want, seen, depth=0):
    """Fewest wait states between an MFMA writing any register in `want` and
    line n, over every path back from n (within HORIZON)."""
    best = 10 ** 6
    acc = 0
    k = n - 1
    while k >= 0:
        t = body[k].strip()
        if t.startswith("v_mfma"):
            if regs(t.split()[1].rstrip(",")) & want:
                return min(best, acc)
        if t.endswith(":") and t.startswith(".LBB") and depth < 8:
            for j in targets.get(t[:-1], []):
                if (j, t) not in seen:
                    seen.add((j, t))
                    best = min(best, acc + min_wait(body, targets, j + 1, want, seen, depth + 1))
        if t.startswith("s_branch") and k < n - 1:
            return best  # the line before falls through only if it is not an unconditional branch
        acc += wait_states(body[k])
        if acc > HORIZON:
            return best
        k -= 1
    return best


def kernel_bodies(asm):
    for name in re.findall(r"^(_ZN3ldv\w+):", asm, re.M):
        i = asm.index(name + ":")
        yield name, asm[i:asm.index(".Lfunc_end", i)].splitlines()


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("src", ["verify.hip", "read.hip", "gather.hip"])
def test_mfma_results_reach_memory_after_wait_states(tmp_path, src):
    out = tmp_path / (src + ".s")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
                    "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "--cuda-device-only", "-S",
                    os.path.join(CSRC, src), "-o", str(out)], check=True, capture_output=True)
    asm = out.read_text()
    checked, short = 0, []
    for name, body in kernel_bodies(asm):
        targets = branches_to(body)
        for n, line in enumerate(body):
            t = line.strip()
            op = t.split()[0] if t else ""
            if not (op.startswith("buffer_store") or op.startswith("global_store") or op.startswith("ds_write")):
                continue
            toks = t.replace(",", " ").split()
            # buffer stores name the data first; global stores and LDS writes
            # name the address first
            data = regs(toks[1] if op.startswith("buffer_store") else toks[2])
            w = min_wait(body, targets, n, data, set())
            if w < 10 ** 6:
                checked += 1
                if w < MIN_WAIT_STATES:
                    short.append((name, n, t, w))
    if src != "gather.hip":  # gather copies its MFMA results before it writes them to LDS
        assert checked > 0, "no MFMA-fed store found: the check is not looking at the kernels"
    assert not short, short[:5]
