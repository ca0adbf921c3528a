"""Throughput of the verify -> commit -> gather path on one MI355X.

One step = ldv_verify_chain / ldv_verify_tree over every draft node of the
batch (ldv_verify_chain_long for chains longer than 64 nodes),
ldv_commit_state of the accepted node (in place), and, for workloads with
drafter reads, ldv_gather_states (o = S q for every query): one pass of the
whole path over one batch of seeded synthetic inputs already resident in
HBM.  Buffer sets are rotated (at least 4, at least 1 GB in all) so that the
256 MB Infinity Cache cannot hold a step's working set.

By default the five workloads run in one process, in order: tiny-chain,
gdn1.3b-chain, tree64, hybrid27b-chain-gather, batch256-tree-commit.  The
JSON line's headline (value, ms_per_step, kernels, roofline, cpu_baseline)
is the 27B-hybrid-shaped workload; `workloads` holds the same fields for
each of the five.  --workload NAME runs one workload (the long chains
included) and makes it the headline.

Timing: K steps captured in one HIP graph.  After the W warm-up steps, the
graph is replayed untimed until at least 30 ms of GPU work has run (the GPU
lowers its clock while the host captures; the first replay after a capture
measured 8% slower per step at K = 20), then `repeats` replays of exactly K
steps are each timed with HIP events (created without the system-scope
fence, recorded on the stream the library launches on) and synchronised;
ms_per_step is the median replay / K.  Per-kernel durations come the same
way from K back-to-back launches of that kernel alone.  Each kernel's
algorithmic bytes over its duration are graded against 8 TB/s and against
the measured stream probe nearest its read/write mix.

Parity in the same run: the CPU leg (the fp64 oracle on the host cores, the
reported CPU baseline) also computes the first sequences' verify o, log P,
committed states and gather o, and `max_rel_err` compares them with the GPU
outputs of one untimed step on fresh buffers in the timed launch
configuration.

    python bench.py [--steps K] [--warmup W] [--workload NAME|all] [--no-cpu]

Prints one JSON line.  --gpus N with N > 1 is refused: this path runs on one
GPU (every (sequence, head) is independent, so batch or head sharding needs
no exchange inside the path).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from workloads import (LONG_WORKLOADS, WORKLOADS, make_block_read_inputs, make_inputs, make_select_inputs,  # noqa: E402
                       tree_depths)

METRIC = "verified draft nodes/sec (B*H*N) on MFMA; commit+gather HBM GB/s vs peak"
HEADLINE = "hybrid27b-chain-gather"
FIVE = ["tiny-chain", "gdn1.3b-chain", "tree64", "hybrid27b-chain-gather", "batch256-tree-commit"]
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, AMD published
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, AMD published
WARM_S = 0.03              # untimed GPU work after each capture
CPU_THREADS_MAX = 16       # the host-core share of one GPU


def algorithmic(wl, x, P2=0, Qn2=0):
    """Algorithmic bytes read and written per launch of each kernel, from the
    shapes alone (every input read once, every output written once), and the
    verify flops (ancestor pairs only)."""
    B, H, D, T = wl.B, wl.H, wl.D, wl.T
    esz = 2 if wl.qkv == "bf16" else 4
    tree = B * T * 4 if wl.topology == "tree" else 0
    depth = np.stack([tree_depths(r) for r in x["parent"]])         # [B, T]
    A = depth.sum(axis=1)                                           # sum of depths per sequence
    # a chain longer than 64 nodes is verified in 64-node chunks: each reads
    # its base state, and all but the last write the next one; the ancestor
    # pairs the closed form evaluates are those inside a chunk, and each
    # chunk end state costs 2 * 64 * d^2 flops
    nch = -(-T // 64)
    out = {}
    out["verify"] = (B * H * (nch * D * D * 4 + T * (3 * D * esz + 8)) + tree,
                     B * H * ((nch - 1) * D * D * 4 + T * (2 * D * 4 + 4)))
    if nch > 1:
        lens = [min(64, T - 64 * c) for c in range(nch)]
        A = np.full(B, sum(n * (n + 1) // 2 for n in lens))
    flops = float(np.sum(H * (4 * T * D * D + 2 * D * (4 * A - 2 * T)))) + B * H * (nch - 1) * 2 * 64 * D * D
    acc = x["accepted"]
    L = np.where(acc >= 0, depth[np.arange(B), np.maximum(acc, 0)], 0)
    com = int(np.sum(acc >= 0))
    out["commit"] = (H * (com * D * D * 4 + int(np.sum(L)) * (D * 4 + D * esz + 4)) + B * 4
                     + (com * T * 4 if wl.topology == "tree" else 0), H * com * D * D * 4)
    if wl.P > 0:
        units = B * wl.P * H
        out["gather"] = (units * (D * D * 4 + wl.Qn * D * esz) + B * wl.P * 4, units * wl.Qn * D * 4)
        out["gather_packed_bf16"] = (out["gather"][0], units * wl.Qn * D * 2)
    if P2:
        out["read_block"] = (B * H * (D * D * 4 + T * (D * esz + D * 4 + 4) + P2 * Qn2 * D * esz) + B * P2 * 4 + tree,
                             B * H * P2 * Qn2 * D * 4)
    if wl.V > 0 and P2:
        out["select"] = (B * (T + 1) * wl.V * esz + B * T * 4 + tree, B * (T + 1) * 4 + 3 * B * 4)
    return out, flops


def set_bytes(wl):
    """Bytes of one rotated verify/commit buffer set (inputs and outputs)."""
    esz = 2 if wl.qkv == "bf16" else 4
    return wl.B * wl.H * wl.D * wl.D * 4 + wl.B * wl.T * wl.H * (3 * wl.D * esz + 2 * wl.D * 4 + 12)


class HipEvents:
    """HIP events recorded on a given stream, created without the system-scope
    fence that a default event record adds (the fence flushes caches and
    stretches the gaps between the kernels being timed)."""

    DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.lib = ctypes.CDLL("libamdhip64.so")
        vp = ctypes.c_void_p
        self.lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
        self.lib.hipEventRecord.argtypes = [vp, vp]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
        self.lib.hipEventDestroy.argtypes = [vp]

    def create(self):
        e = self.ct.c_void_p()
        rc = self.lib.hipEventCreateWithFlags(self.ct.byref(e), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError("hipEventCreateWithFlags failed: %d" % rc)
        return e

    def record(self, e, stream_handle):
        rc = self.lib.hipEventRecord(e, self.ct.c_void_p(stream_handle))
        if rc != 0:
            raise RuntimeError("hipEventRecord failed: %d" % rc)

    def elapsed_s(self, a, b):
        f = self.ct.c_float()
        rc = self.lib.hipEventElapsedTime(self.ct.byref(f), a, b)
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed: %d" % rc)
        return f.value * 1e-3

    def destroy(self, e):
        self.lib.hipEventDestroy(e)


def traffic_from_profiles(kernel_name, src_files, workload):
    """HBM bytes per launch measured by rocprofv3 counters, if they were taken
    on this workload and on the kernel sources as they are now (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    h = hashlib.sha256()
    for s in src_files:
        with open(os.path.join(ROOT, s), "rb") as f:
            h.update(f.read())
    ent = rec.get(workload, {}).get(kernel_name)
    if not ent or ent.get("source_sha256") != h.hexdigest():
        return None
    return ent.get("bytes_per_launch")


KERNEL_SOURCES = {
    "verify": "speculative_decoding_verify_amd/csrc/verify.hip",
    "commit": "speculative_decoding_verify_amd/csrc/commit.hip",
    "gather": "speculative_decoding_verify_amd/csrc/gather.hip",
    "gather_packed_bf16": "speculative_decoding_verify_amd/csrc/gather.hip",
    "read_block": "speculative_decoding_verify_amd/csrc/read.hip",
    "select": "speculative_decoding_verify_amd/csrc/select.hip",
}


def kernel_sources(name):
    return [KERNEL_SOURCES[name], "speculative_decoding_verify_amd/csrc/ldv_device.hpp"]


class Runner:
    """Buffers and launch functions of the path on one workload; launch i
    uses buffer set i mod nsets."""

    def __init__(self, ldv, torch, wl, x, nsets, next_rows):
        self.ldv, self.torch, self.wl = ldv, torch, wl
        self.chain = wl.topology == "chain"
        self.dt = dt = torch.bfloat16 if wl.qkv == "bf16" else torch.float32
        base = dict(q=self.cuda(x["q"], dt), k=self.cuda(x["k"], dt), v=self.cuda(x["v"], dt), a=self.cuda(x["a"]),
                    beta=self.cuda(x["beta"]), S0=self.cuda(x["S0"]), parent=self.cuda(x["parent"]),
                    acc=self.cuda(x["accepted"]))
        self.sets = []
        for i in range(nsets):
            st = {n: t.clone() for n, t in base.items()}
            self.outputs(st)
            self.sets.append(st)
        del base
        self.status = torch.zeros(1, dtype=torch.int32, device="cuda")
        if wl.P > 0:
            self.pool = self.cuda(x["pool"])
            self.slot = self.cuda(x["slot"])
            self.queries = self.cuda(x["queries"], dt)
            self.go = torch.empty((wl.B, wl.P, wl.H, wl.Qn, wl.D), device="cuda")
            if next_rows:  # drafter features: one bf16 row of H * Qn * D reads per (sequence, position)
                self.gfeat = torch.empty((wl.B, wl.P, wl.H * wl.Qn * wl.D), device="cuda", dtype=torch.bfloat16)
        self.P2 = self.Qn2 = 0
        if next_rows:
            r = make_block_read_inputs(wl)
            self.P2, self.Qn2 = r["pos"].shape[1], r["queries"].shape[3]
            self.pos, self.rq = self.cuda(r["pos"]), self.cuda(r["queries"], dt)
            self.ro = torch.empty((wl.B, self.P2, wl.H, self.Qn2, wl.D), device="cuda")
            self.logits = []
            if wl.V > 0:
                sel = make_select_inputs(wl, x["parent"], x["accepted"])
                lb = sel["logits"].size * (2 if wl.qkv == "bf16" else 4)
                nlog = int(min(nsets, max(4, -(-1_000_000_000 // lb))))
                self.logits = [self.cuda(sel["logits"], dt) for _ in range(nlog)]
                self.tokens = self.cuda(sel["tokens"])
                del sel
                self.sel_out = [torch.empty((wl.B, wl.T + 1), dtype=torch.int32, device="cuda")] + \
                               [torch.empty((wl.B,), dtype=torch.int32, device="cuda") for _ in range(3)]
                # the selection's workspace (rows split over workgroups when they are few)
                nws = self.ldv.select_workspace_bytes(wl.B, wl.T, wl.V)
                self.sel_ws = torch.empty(nws, dtype=torch.uint8, device="cuda") if nws > 0 else None

    def cuda(self, a, t=None):
        g = self.torch.from_numpy(np.ascontiguousarray(a)).cuda()
        return g if t is None else g.to(t)

    def outputs(self, st):
        wl, torch = self.wl, self.torch
        st["o"] = torch.empty((wl.B, wl.T, wl.H, wl.D), device="cuda")
        st["u"] = torch.empty((wl.B, wl.T, wl.H, wl.D), device="cuda")
        st["logp"] = torch.empty((wl.B, wl.T, wl.H), device="cuda")
        if wl.T > 64:  # the work state of a long chain
            st["S_work"] = torch.empty_like(st["S0"])

    def verify_set(self, s):
        if self.chain and self.wl.T > 64:
            self.ldv.verify_chain_long(s["q"], s["k"], s["v"], s["a"], s["beta"], s["S0"], o=s["o"], u=s["u"],
                                       logp=s["logp"], S_work=s["S_work"], status=self.status)
        elif self.chain:
            self.ldv.verify_chain(s["q"], s["k"], s["v"], s["a"], s["beta"], s["S0"], o=s["o"], u=s["u"],
                                  logp=s["logp"], status=self.status)
        else:
            self.ldv.verify_tree(s["q"], s["k"], s["v"], s["a"], s["beta"], s["S0"], s["parent"], o=s["o"],
                                 u=s["u"], logp=s["logp"], status=self.status)

    def commit_set(self, s):
        self.ldv.commit_state(s["k"], s["u"], s["logp"], s["acc"], s["S0"], S_out=s["S0"],
                              parent=None if self.chain else s["parent"], status=self.status)

    def verify(self, i):
        self.verify_set(self.sets[i % len(self.sets)])

    def commit(self, i):
        self.commit_set(self.sets[i % len(self.sets)])

    def gather(self, i):
        self.ldv.gather_states(self.pool, self.slot, self.queries, o=self.go, status=self.status)

    def gather_packed(self, i):
        self.ldv.gather_states_packed(self.pool, self.slot, self.queries, self.gfeat, col=0, status=self.status)

    def read(self, i):
        s = self.sets[i % len(self.sets)]
        self.ldv.read_block_states(s["k"], s["u"], s["logp"], s["S0"], self.pos, self.rq,
                                   parent=None if self.chain else s["parent"], o=self.ro, status=self.status)

    def select(self, i):
        s = self.sets[i % len(self.sets)]
        t, a, l, b = self.sel_out
        self.ldv.select_accepted(self.logits[i % len(self.logits)], self.tokens,
                                 None if self.chain else s["parent"], target=t, accepted=a, accepted_len=l,
                                 bonus=b, status=self.status, workspace=self.sel_ws)

    def step_fns(self):
        return [self.verify, self.commit] + ([self.gather] if self.wl.P > 0 else [])

    def parity_step(self, x, ns):
        """One untimed step on fresh buffers (the inputs as generated, in the
        launch configuration of the timed steps): verify, commit in place,
        gather.  Returns the first ns sequences' outputs as host arrays."""
        torch = self.torch
        s = dict(q=self.cuda(x["q"], self.dt), k=self.cuda(x["k"], self.dt), v=self.cuda(x["v"], self.dt),
                 a=self.cuda(x["a"]), beta=self.cuda(x["beta"]), S0=self.cuda(x["S0"]),
                 parent=self.cuda(x["parent"]), acc=self.cuda(x["accepted"]))
        self.outputs(s)
        self.verify_set(s)
        self.commit_set(s)
        out = {}
        if self.wl.P > 0:
            go = torch.empty_like(self.go)
            self.ldv.gather_states(self.pool, self.slot, self.queries, o=go, status=self.status)
            out["gather_o"] = go[:ns].double().cpu().numpy()
        torch.cuda.synchronize()
        out.update(verify_o=s["o"][:ns].double().cpu().numpy(), logp=s["logp"][:ns].double().cpu().numpy(),
                   commit_S=s["S0"][:ns].double().cpu().numpy())
        del s
        return out


class Timer:
    def __init__(self, torch, hev, stream_handle):
        self.torch, self.hev, self.sh = torch, hev, stream_handle

    def once(self, fn):
        e0, e1 = self.hev.create(), self.hev.create()
        self.hev.record(e0, self.sh)
        fn()
        self.hev.record(e1, self.sh)
        self.torch.cuda.synchronize()
        t = self.hev.elapsed_s(e0, e1)
        self.hev.destroy(e0)
        self.hev.destroy(e1)
        return t

    warm_s = WARM_S

    def warm(self, fn):
        """Untimed runs of fn until warm_s of GPU time has passed (at least one)."""
        t, n = 0.0, 0
        while t < self.warm_s or n < 1:
            t += self.once(fn)
            n += 1
        return n

    def repeated(self, fn, repeats):
        self.warm(fn)
        return [self.once(fn) for _ in range(repeats)]


def capture(torch, fns, K):
    """One HIP graph holding K launches of each function in fns, in order."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(K):
            for fn in fns:
                fn(i)
    return g


def measure_peaks(torch):
    """Achievable rates on this GPU, each the best of 3 timed runs of 8
    back-to-back launches after a warm-up: stream probes over 1 GiB (libldv_peaks.so; non-temporal loads
    and stores) reading only, copying, rewriting in place, and writing one
    float4 per 2, 4 or 8 read, each the best of 2, 4 or 8 loads in flight per
    thread on grid-stride grids of 256 to 16384 blocks and on a grid of one
    block per step of the stream (steps in order, or 128 KiB units spread
    over the XCDs as the library's per-head kernels spread heads); a loop of
    independent v_mfma_f32_16x16x32_bf16 chains on every SIMD; an 8192^3 bf16
    GEMM (hipBLASLt through torch.matmul)."""
    import ctypes
    plib = ctypes.CDLL(os.path.join(ROOT, "speculative_decoding_verify_amd", "libldv_peaks.so"))
    vp = ctypes.c_void_p
    plib.ldv_peak_mfma.argtypes = [ctypes.c_int, vp, vp]
    plib.ldv_peak_mfma_flops.argtypes = [ctypes.c_int]
    plib.ldv_peak_mfma_flops.restype = ctypes.c_double
    plib.ldv_peak_stream.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, ctypes.c_longlong, ctypes.c_int, ctypes.c_int,
                                     vp]
    plib.ldv_peak_stream_granule.restype = ctypes.c_longlong
    g = plib.ldv_peak_stream_granule()
    n4 = (1 << 30) // 16 // g * g
    src = torch.ones(n4 * 4, device="cuda")
    dst = torch.empty(n4 * 4, device="cuda")
    a = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    nblk = 4 * torch.cuda.get_device_properties(0).multi_processor_count
    pout = torch.empty(nblk * 256, device="cuda")

    def stream_call(ratio, loads, blocks, in_place=False, spread=0):
        def f():
            rc = plib.ldv_peak_stream(ratio, loads, vp(src.data_ptr()), vp((src if in_place else dst).data_ptr()),
                                      n4, blocks, spread, vp(torch.cuda.current_stream().cuda_stream))
            assert rc == 0, "stream probe launch failed (%d)" % rc
        return f

    def mfma_loop():
        rc = plib.ldv_peak_mfma(nblk, vp(pout.data_ptr()), vp(torch.cuda.current_stream().cuda_stream))
        assert rc == 0, "MFMA probe launch failed (%d)" % rc

    def best_rate(fn, work, launches=8, repeats=3):
        """work per second of `launches` back-to-back launches (as the
        library's kernels are timed), the best of `repeats`."""
        fn()
        torch.cuda.synchronize()
        best = None
        for _ in range(repeats):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(launches):
                fn()
            e1.record()
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) * 1e-3 / launches
            best = t if best is None else min(best, t)
        return work / best

    out = {}
    nbytes = n4 * 16
    for name, ratio, in_place in (("read_GB_s", 0, False), ("copy_GB_s", 1, False), ("rmw_GB_s", 1, True),
                                  ("read2write1_GB_s", 2, False), ("read4write1_GB_s", 4, False),
                                  ("read8write1_GB_s", 8, False)):
        wr = nbytes // ratio if ratio else 0
        rates = []
        for loads in (2, 4, 8):
            if loads < ratio:
                continue
            one_shot = n4 // (loads * 256)  # one block per step of the stream: no grid-stride loop
            rates += [best_rate(stream_call(ratio, loads, blk, in_place), (nbytes + wr) / 1e9)
                      for blk in (256, 512, 1024, 2048, 4096, 16384, one_shot)]
            rates.append(best_rate(stream_call(ratio, loads, one_shot, in_place, 1), (nbytes + wr) / 1e9))
        out[name] = max(rates)
    out["bf16_mfma_loop_TFLOP_s"] = best_rate(mfma_loop, plib.ldv_peak_mfma_flops(nblk) / 1e12)
    out["bf16_gemm_TFLOP_s"] = best_rate(lambda: torch.matmul(a, b), 2 * 8192 ** 3 / 1e12)
    del src, dst, a, b, pout
    torch.cuda.empty_cache()
    return out


def ceiling_for(rd, wr, in_place, peaks):
    """The achievable streaming rate for a kernel's read/write mix: the best
    stream probe whose read:write ratio is at most the kernel's (a kernel
    that reads more per byte written can stream at least as fast), the
    reads-only probe counting as a 32:1 mix (kernels that write less than
    that are graded as reading only).  The in-place probe counts as a 1:1
    mix; an in-place commit is graded against it alone."""
    if not peaks:
        return None, None
    if in_place:
        return "rmw_GB_s", peaks["rmw_GB_s"]
    r = rd / wr if wr > 0 else float("inf")
    cands = [(1, "copy_GB_s"), (1, "rmw_GB_s"), (2, "read2write1_GB_s"), (4, "read4write1_GB_s"),
             (8, "read8write1_GB_s"), (32, "read_GB_s")]
    ok = [(peaks[n], n) for ratio, n in cands if ratio <= r * (1 + 1e-9)]
    if not ok:
        return "copy_GB_s", peaks["copy_GB_s"]
    v, n = max(ok)
    return n, v


def host_threads():
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:
        aff = os.cpu_count() or 1
    return min(CPU_THREADS_MAX, aff), os.cpu_count() or 1, aff


def cpu_baseline(wl, x, seconds_min, gpu_out, ns):
    """The fp64 oracle (every path walked token by token) on the host cores,
    over the same workload: sequences in order, in chunks of max(1, B / 16),
    until at least seconds_min has passed; the rate is scaled to nodes/s.
    The first chunk's outputs (its first ns sequences) are compared with the
    GPU outputs of the same sequences (gpu_out): the relative error
    max |gpu - oracle| / max |oracle| of each output tensor."""
    import oracle
    threads, ncpu, aff = host_threads()
    chain = wl.topology == "chain"
    long_chain = chain and wl.T > 64  # sequential decode: walking every path would be O(T^2) per head
    par = None if chain else x["parent"]
    done, t_total, used = 0, 0.0, 1
    step = max(1, wl.B // 16)
    errs = None
    while t_total < seconds_min:
        b0 = done % wl.B
        sl = slice(b0, min(wl.B, b0 + step))
        used = max(used, min(threads, (sl.stop - sl.start) * wl.H))
        psl = None if chain else par[sl]
        t0 = time.perf_counter()
        if long_chain:
            ro = oracle.chain_decode(x["q"][sl], x["k"][sl], x["v"][sl], x["a"][sl], x["beta"][sl], x["S0"][sl],
                                     nthreads=threads)
        else:
            ro, _, _ = oracle.verify(x["q"][sl], x["k"][sl], x["v"][sl], x["a"][sl], x["beta"][sl], x["S0"][sl],
                                     psl, nthreads=threads)
        rS, _ = oracle.commit(x["k"][sl], x["v"][sl], x["a"][sl], x["beta"][sl], x["S0"][sl], x["accepted"][sl],
                              psl, nthreads=threads)
        rg = None
        if wl.P > 0:
            rg, _, _ = oracle.gather(x["pool"], x["slot"][sl], x["queries"][sl], want_states=False, nthreads=threads)
        t_total += time.perf_counter() - t0
        if errs is None and gpu_out is not None:
            rel = lambda g, r: float(np.max(np.abs(g - r)) / max(np.max(np.abs(r)), 1e-300))
            n = min(ns, sl.stop - sl.start)
            rlp, _ = oracle.log_decay(x["a"][sl][:n], None if chain else psl[:n])
            errs = {"verify_o": rel(gpu_out["verify_o"][:n], ro[:n]), "logp": rel(gpu_out["logp"][:n], rlp),
                    "commit_S": rel(gpu_out["commit_S"][:n], rS[:n])}
            if rg is not None:
                errs["gather_o"] = rel(gpu_out["gather_o"][:n], rg[:n])
            errs["sequences"] = n
        done += sl.stop - sl.start
    nodes = done * wl.H * wl.T
    cpu = {"value": nodes / t_total, "unit": "nodes/s", "cores": used, "kind": "oracle",
           "host_cpus": ncpu, "affinity_cpus": aff,
           "sample": "%d sequences in chunks of %d from sequence 0, wrapping (all %d heads; every node verified by "
                     "%s, the accepted node committed%s), %.1f s" % (
                         done, step, wl.H, "sequential decode" if long_chain else "its path walk",
                         ", 4 positions x 16 queries read per sequence" if wl.P else "", t_total)}
    return cpu, errs


def run_workload(torch, ldv, timer, wl, args, peaks, cpu_seconds):
    """Everything measured on one workload: the step, each kernel, the
    parity of one step and the CPU baseline.  Returns its JSON object."""
    no_next = args.no_next or wl.T > 64  # the in-block reads and the selection take drafts of at most 64 nodes
    K = args.steps
    nsets = int(min(64, max(4, -(-1_000_000_000 // set_bytes(wl)))))
    print("[bench] %s: generating inputs (%d rotated buffer sets)" % (wl.key, nsets), file=sys.stderr, flush=True)
    x = make_inputs(wl)
    run = Runner(ldv, torch, wl, x, nsets, not no_next)
    fns = run.step_fns()
    for i in range(args.warmup):
        for fn in fns:
            fn(i)
    torch.cuda.synchronize()
    assert int(run.status.item()) == 0, "device status %d" % int(run.status.item())

    # the timed region: K steps in one HIP graph (or K eager steps)
    if args.eager:
        replay = lambda: [fn(i) for i in range(K) for fn in fns]
    else:
        g_step = capture(torch, fns, K)
        replay = g_step.replay
    t0 = time.perf_counter()
    ts = timer.repeated(replay, args.repeats)
    wall = time.perf_counter() - t0
    t_step = float(np.median(ts)) / K
    nodes = wl.B * wl.H * wl.T

    # per-kernel durations: K back-to-back launches of one kernel in one graph
    def per_kernel(fn):
        if args.eager:
            rep = lambda: [fn(i) for i in range(K)]
        else:
            g = capture(torch, [fn], K)
            rep = g.replay
        t = [v / K for v in timer.repeated(rep, args.repeats)]
        return float(np.median(t)), float(np.min(t)), float(np.max(t))

    alg, vflops = algorithmic(wl, x, run.P2, run.Qn2)
    names = [("verify", run.verify), ("commit", run.commit)]
    if wl.P > 0:
        names.append(("gather", run.gather))
        if not no_next:
            names.append(("gather_packed_bf16", run.gather_packed))
    if not no_next:
        names.append(("read_block", run.read))
        if wl.V > 0:
            names.append(("select", run.select))
    kern = {}
    for name, fn in names:
        med, lo, hi = per_kernel(fn)
        rd, wr = alg[name]
        by = rd + wr
        k = {"us": med * 1e6, "us_min": lo * 1e6, "us_max": hi * 1e6, "launches": K, "alg_bytes": int(by),
             "alg_read_bytes": int(rd), "alg_write_bytes": int(wr), "GB_s": by / med / 1e9,
             "hbm_frac": by / med / 1e9 / HBM_PEAK_GBS}
        cname, cval = ceiling_for(rd, wr, name == "commit", peaks)
        if cval:
            k.update({"ceiling": cname, "ceiling_GB_s": cval, "frac_of_ceiling": k["GB_s"] / cval})
        kern[name] = k
    assert int(run.status.item()) == 0, "device status %d" % int(run.status.item())
    kv = kern["verify"]
    kv["nodes_per_s"] = nodes / kv["us"] * 1e6
    kv["alg_flops"] = vflops
    kv["mfma_frac"] = vflops / (kv["us"] * 1e-6) / (BF16_PEAK_TFLOPS * 1e12)
    # o = S q products of the state reads (2 d^2 flops per query)
    for name, nq in (("gather", wl.B * wl.P * wl.H * wl.Qn), ("gather_packed_bf16", wl.B * wl.P * wl.H * wl.Qn),
                     ("read_block", wl.B * run.P2 * wl.H * run.Qn2)):
        if name in kern and nq:
            fl = 2.0 * wl.D * wl.D * nq
            kern[name]["alg_flops"] = fl
            kern[name]["mfma_frac"] = fl / (kern[name]["us"] * 1e-6) / (BF16_PEAK_TFLOPS * 1e12)
    if peaks:
        for v in kern.values():
            if "mfma_frac" in v:
                v["mfma_frac_of_measured_loop"] = v["mfma_frac"] * BF16_PEAK_TFLOPS / peaks["bf16_mfma_loop_TFLOP_s"]
    if "read_block" in kern:
        kern["read_block"].update({"P": run.P2, "Qn": run.Qn2})
    if "select" in kern:
        kern["select"].update({"V": wl.V, "logits": wl.qkv})
    step_names = [n for n in ("verify", "commit", "gather") if n in kern]
    dom = max(step_names, key=lambda n: kern[n]["us"])
    roof = {"kernel": dom, "bound": "hbm", "achieved": kern[dom]["GB_s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": kern[dom]["hbm_frac"], "traffic": traffic_from_profiles(dom, kernel_sources(dom), wl.key)}
    if "ceiling" in kern[dom]:
        roof.update({"ceiling": kern[dom]["ceiling"], "ceiling_GB_s": kern[dom]["ceiling_GB_s"],
                     "frac_of_ceiling": kern[dom]["frac_of_ceiling"]})

    cpu, errs = None, None
    if not args.no_cpu:
        ns = max(1, min(wl.B, wl.B // 16))
        gpu_out = run.parity_step(x, ns)
        print("[bench] %s: CPU oracle (%.0f s)" % (wl.key, cpu_seconds), file=sys.stderr, flush=True)
        cpu, errs = cpu_baseline(wl, x, cpu_seconds, gpu_out, ns)
    del run
    torch.cuda.empty_cache()
    return {
        "value": nodes / t_step, "unit": "nodes/s", "ms_per_step": t_step * 1e3,
        "ms_per_step_replays": [t / K * 1e3 for t in ts],
        "config": {"workload": wl.key, "B": wl.B, "H": wl.H, "d_k": wl.D, "d_v": wl.D, "T": wl.T,
                   "topology": wl.topology, "qkv": wl.qkv, "state": "f32",
                   "gather": ({"P": wl.P, "Qn": wl.Qn, "pool_slots": wl.B * wl.R} if wl.P else None),
                   "step": "+".join(step_names), "rotated_sets": nsets,
                   "timing": "eager launches" if args.eager else "HIP graph replay"},
        "kernels": kern, "roofline": roof, "cpu_baseline": cpu, "max_rel_err": errs, "wall_s": wall,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="all", choices=["all"] + sorted({**WORKLOADS, **LONG_WORKLOADS}))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline and the parity check")
    ap.add_argument("--no-next", action="store_true", help="skip timing the in-block read and the selection")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU-oracle time on the headline workload")
    ap.add_argument("--cpu-seconds-other", type=float, default=3.0, help="CPU-oracle time on each other workload")
    ap.add_argument("--repeats", type=int, default=5, help="timed replays of each graph")
    ap.add_argument("--warm-ms", type=float, default=WARM_S * 1e3,
                    help="untimed GPU work before each timed graph (at least one replay; 0 for counter runs)")
    ap.add_argument("--no-peaks", action="store_true", help="skip measuring the stream, MFMA and GEMM rates")
    ap.add_argument("--eager", action="store_true",
                    help="launch from Python each step instead of replaying HIP graphs (for profilers)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes (5 times), to scale "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE counters, and print its bandwidth")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(each (sequence, head) is independent, so the batch or the heads shard with no exchange).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        n = args.copy_calibration // 4
        src = torch.ones(n, device="cuda")
        dst = torch.empty(n, device="cuda")
        dst.copy_(src)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / 5
        print(json.dumps({"copy_bytes": n * 4, "copy_us": t * 1e6, "copy_GB_s_read_plus_write": 2 * n * 4 / t / 1e9}))
        return
    import speculative_decoding_verify_amd as ldv

    keys = FIVE if args.workload == "all" else [args.workload]
    head = HEADLINE if args.workload == "all" else args.workload
    allw = {**WORKLOADS, **LONG_WORKLOADS}
    hev = HipEvents()
    timer = Timer(torch, hev, torch.cuda.current_stream().cuda_stream)  # the stream the library launches on
    timer.warm_s = args.warm_ms * 1e-3
    peaks = None if args.no_peaks else measure_peaks(torch)
    res = {}
    for key in keys:
        res[key] = run_workload(torch, ldv, timer, allw[key], args, peaks,
                                args.cpu_seconds if key == head else args.cpu_seconds_other)
    h = res[head]
    if peaks:
        h["roofline"]["measured_peaks"] = peaks
    out = {
        "metric": METRIC, "value": h["value"], "unit": "nodes/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": h["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": h["config"], "kernels": h["kernels"], "roofline": h["roofline"], "cpu_baseline": h["cpu_baseline"],
        "max_rel_err": h["max_rel_err"], "ms_per_step_replays": h["ms_per_step_replays"],
        "workloads": {k: {kk: vv for kk, vv in v.items()} for k, v in res.items()},
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
