"""Throughput of the verify -> commit -> gather path on one MI355X.

One step = ldv_verify_chain / ldv_verify_tree over every draft node of the
batch (ldv_verify_chain_long for the chains longer than 64 nodes),
ldv_commit_state of the accepted node (in place), and, for workloads with
drafter reads, ldv_gather_states (o = S q for every query) - one pass of the
whole path over one batch of seeded synthetic inputs already resident in
HBM.  Buffer sets are rotated (at least 4, at least 1 GB in all) so that the
256 MB Infinity Cache cannot hold a step's working set.

Timing uses HIP events created without the system-scope fence, recorded on
the stream the library launches on.  The timed region is K steps captured in
one HIP graph and replayed once (--eager: launched from Python instead; the
Python launch cost then dominates the small workloads).  Per-kernel
durations come from K back-to-back launches of that kernel alone in one
graph, the median of 5 replays; they include the two steps around verify
(ldv_read_block_states at 4 in-block positions x 16 queries per sequence,
and ldv_select_accepted on target logits [B, T+1, V]; --no-next skips them).

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

Prints one JSON line.  --gpus N with N > 1 is refused: this path runs on one
GPU (every (sequence, head) is independent, so batch or head sharding needs
no exchange inside the path).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from workloads import (LONG_WORKLOADS, WORKLOADS, make_block_read_inputs, make_inputs, make_select_inputs,  # noqa: E402
                       tree_depths)

METRIC = "verified draft nodes/sec (B*H*N) on MFMA; commit+gather HBM GB/s vs peak"
DEFAULT_WORKLOAD = "hybrid27b-chain-gather"
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, AMD published
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, AMD published


def algorithmic(wl, x):
    """Algorithmic bytes (and flops) per launch of each kernel, from the
    shapes alone: every input read once, every output written once."""
    B, H, D, T = wl.B, wl.H, wl.D, wl.T
    esz = 2 if wl.qkv == "bf16" else 4
    depth = np.stack([tree_depths(r) for r in x["parent"]])         # [B, T]
    A = depth.sum(axis=1)                                           # sum of depths per sequence
    # a chain longer than 64 nodes is verified in 64-node chunks: each reads
    # its base state, and all but the last write the next one; the ancestor
    # pairs the closed form evaluates are those inside a chunk, and each
    # chunk end state costs 2 * 64 * d^2 flops
    nch = -(-T // 64)
    per_head = (2 * nch - 1) * D * D * 4 + T * (3 * D * esz + 8 + 2 * D * 4 + 4)  # states, q k v, a beta, o u, logp
    verify_bytes = B * H * per_head + (B * T * 4 if wl.topology == "tree" else 0)
    if nch > 1:
        lens = [min(64, T - 64 * c) for c in range(nch)]
        A = np.full(B, sum(n * (n + 1) // 2 for n in lens))
    verify_flops = float(np.sum(H * (4 * T * D * D + 2 * D * (4 * A - 2 * T)))) + B * H * (nch - 1) * 2 * 64 * D * D
    acc = x["accepted"]
    L = np.where(acc >= 0, depth[np.arange(B), np.maximum(acc, 0)], 0)
    committing = int(np.sum(acc >= 0))
    commit_bytes = H * (committing * 2 * D * D * 4 + int(np.sum(L)) * (D * 4 + D * esz + 4)) + B * 4
    gather_bytes = 0
    if wl.P > 0:
        gather_bytes = B * wl.P * H * (D * D * 4 + wl.Qn * D * esz + wl.Qn * D * 4) + B * wl.P * 4
    return dict(verify=verify_bytes, verify_flops=verify_flops, commit=commit_bytes, gather=gather_bytes)


def algorithmic_next(wl, P, Qn):
    """Algorithmic bytes per launch of the in-block read and the selection."""
    B, H, D, T = wl.B, wl.H, wl.D, wl.T
    esz = 2 if wl.qkv == "bf16" else 4
    tree = B * T * 4 if wl.topology == "tree" else 0
    read = B * H * (D * D * 4 + T * (D * esz + D * 4 + 4) + P * Qn * (D * esz + D * 4)) + B * P * 4 + tree
    sel = B * (T + 1) * wl.V * esz + B * T * 4 + tree + B * (T + 1) * 4 + 3 * B * 4
    return read, sel


def cpu_baseline(wl, x, seconds_min=10.0, seconds_cap=30.0):
    """The fp64 oracle (the path walked token by token) on the host cores,
    over the same workload: sequences in order, in chunks, repeating whole
    passes until at least seconds_min has elapsed (stopping early at
    seconds_cap); the rate is scaled to nodes/s."""
    import oracle
    threads = min(16, os.cpu_count() or 1)
    chain = wl.topology == "chain"
    long_chain = chain and wl.T > 64  # sequential decode: walking every path would be O(T^2) per head
    done, t_total = 0, 0.0
    step = max(1, wl.B // 16)
    while (t_total < seconds_min or done % wl.B) and t_total < seconds_cap:
        b0 = done % wl.B
        sl = slice(b0, min(wl.B, b0 + step))
        t0 = time.perf_counter()
        if long_chain:
            oracle.chain_decode(x["q"][sl], x["k"][sl], x["v"][sl], x["a"][sl], x["beta"][sl], x["S0"][sl],
                                nthreads=threads)
        else:
            oracle.verify(x["q"][sl], x["k"][sl], x["v"][sl], x["a"][sl], x["beta"][sl], x["S0"][sl],
                          None if chain else x["parent"][sl], nthreads=threads)
        oracle.commit(x["k"][sl], x["v"][sl], x["a"][sl], x["beta"][sl], x["S0"][sl], x["accepted"][sl],
                      None if chain else x["parent"][sl], nthreads=threads)
        if wl.P > 0:
            oracle.gather(x["pool"], x["slot"][sl], x["queries"][sl], want_states=False, nthreads=threads)
        t_total += time.perf_counter() - t0
        done += sl.stop - sl.start
    nodes = done * wl.H * wl.T
    return {"value": nodes / t_total, "unit": "nodes/s", "cores": threads, "kind": "oracle",
            "sample": "%d sequence passes over the %d sequences (all %d heads; every node verified by %s, "
                      "the accepted node committed%s), %.1f s" % (
                          done, wl.B, wl.H, "sequential decode" if long_chain else "its path walk",
                          ", 4 positions x 16 queries read per sequence" if wl.P else "", t_total)}


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
    on this workload and on the kernel source as it is now (else None)."""
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
    ent = rec.get(kernel_name)
    if not ent or ent.get("source_sha256") != h.hexdigest() or ent.get("workload") != workload:
        return None
    return ent.get("bytes_per_launch")


def set_bytes(wl):
    """Bytes of one rotated verify/commit buffer set (inputs and outputs)."""
    esz = 2 if wl.qkv == "bf16" else 4
    return wl.B * wl.H * wl.D * wl.D * 4 + wl.B * wl.T * wl.H * (3 * wl.D * esz + 2 * wl.D * 4 + 12)


class Runner:
    """Buffers and launch functions of the path on one workload; launch i
    uses buffer set i mod nsets."""

    def __init__(self, ldv, torch, wl, x, nsets, next_rows):
        self.ldv, self.torch, self.wl = ldv, torch, wl
        self.chain = wl.topology == "chain"
        dt = torch.bfloat16 if wl.qkv == "bf16" else torch.float32
        cuda = lambda a, t=None: (torch.from_numpy(np.ascontiguousarray(a)).cuda() if t is None
                                  else torch.from_numpy(np.ascontiguousarray(a)).cuda().to(t))
        base = dict(q=cuda(x["q"], dt), k=cuda(x["k"], dt), v=cuda(x["v"], dt), a=cuda(x["a"]),
                    beta=cuda(x["beta"]), S0=cuda(x["S0"]), parent=cuda(x["parent"]), acc=cuda(x["accepted"]))
        self.sets = []
        for i in range(nsets):
            st = {n: t.clone() for n, t in base.items()}
            st["o"] = torch.empty((wl.B, wl.T, wl.H, wl.D), device="cuda")
            st["u"] = torch.empty((wl.B, wl.T, wl.H, wl.D), device="cuda")
            st["logp"] = torch.empty((wl.B, wl.T, wl.H), device="cuda")
            if wl.T > 64:  # the work state of a long chain
                st["S_work"] = torch.empty_like(st["S0"])
            self.sets.append(st)
        del base
        self.status = torch.zeros(1, dtype=torch.int32, device="cuda")
        if wl.P > 0:
            self.pool = cuda(x["pool"])
            self.slot = cuda(x["slot"])
            self.queries = cuda(x["queries"], dt)
            self.go = torch.empty((wl.B, wl.P, wl.H, wl.Qn, wl.D), device="cuda")
            if next_rows:  # drafter features: one bf16 row of H * Qn * D reads per (sequence, position)
                self.gfeat = torch.empty((wl.B, wl.P, wl.H * wl.Qn * wl.D), device="cuda", dtype=torch.bfloat16)
        self.next = None
        if next_rows:
            r = make_block_read_inputs(wl)
            self.P2, self.Qn2 = r["pos"].shape[1], r["queries"].shape[3]
            self.pos, self.rq = cuda(r["pos"]), cuda(r["queries"], dt)
            self.ro = torch.empty((wl.B, self.P2, wl.H, self.Qn2, wl.D), device="cuda")
            self.logits = []
            if wl.V > 0:
                sel = make_select_inputs(wl, x["parent"], x["accepted"])
                lb = sel["logits"].size * (2 if wl.qkv == "bf16" else 4)
                nlog = int(min(nsets, max(4, -(-1_000_000_000 // lb))))
                self.logits = [cuda(sel["logits"], dt) for _ in range(nlog)]
                self.tokens = cuda(sel["tokens"])
                del sel
                self.sel_out = [torch.empty((wl.B, wl.T + 1), dtype=torch.int32, device="cuda")] + \
                               [torch.empty((wl.B,), dtype=torch.int32, device="cuda") for _ in range(3)]
                # the selection's workspace (rows split over workgroups when they are few)
                nws = self.ldv.select_workspace_bytes(wl.B, wl.T, wl.V)
                self.sel_ws = torch.empty(nws, dtype=torch.uint8, device="cuda") if nws > 0 else None

    def verify(self, i):
        s = self.sets[i % len(self.sets)]
        if self.chain and self.wl.T > 64:
            self.ldv.verify_chain_long(s["q"], s["k"], s["v"], s["a"], s["beta"], s["S0"], o=s["o"], u=s["u"],
                                       logp=s["logp"], S_work=s["S_work"], status=self.status)
        elif self.chain:
            self.ldv.verify_chain(s["q"], s["k"], s["v"], s["a"], s["beta"], s["S0"], o=s["o"], u=s["u"],
                                  logp=s["logp"], status=self.status)
        else:
            self.ldv.verify_tree(s["q"], s["k"], s["v"], s["a"], s["beta"], s["S0"], s["parent"], o=s["o"],
                                 u=s["u"], logp=s["logp"], status=self.status)

    def commit(self, i):
        s = self.sets[i % len(self.sets)]
        self.ldv.commit_state(s["k"], s["u"], s["logp"], s["acc"], s["S0"], S_out=s["S0"],
                              parent=None if self.chain else s["parent"], status=self.status)

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


def measure_peaks(torch):
    """Achievable peaks on this GPU, each the best of 5 timed runs after a
    warm-up: a 2 GiB device-to-device copy (HBM read plus write); a loop of
    independent v_mfma_f32_16x16x32_bf16 chains on every SIMD
    (libldv_peaks.so, four waves per SIMD); and an 8192^3 bf16 GEMM
    (hipBLASLt through torch.matmul)."""
    import ctypes
    n = (2 << 30) // 4
    src = torch.ones(n, device="cuda")
    dst = torch.empty(n, device="cuda")
    a = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    plib = ctypes.CDLL(os.path.join(ROOT, "speculative_decoding_verify_amd", "libldv_peaks.so"))
    plib.ldv_peak_mfma.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    plib.ldv_peak_mfma_flops.argtypes = [ctypes.c_int]
    plib.ldv_peak_mfma_flops.restype = ctypes.c_double
    nblk = 4 * torch.cuda.get_device_properties(0).multi_processor_count
    pout = torch.empty(nblk * 256, device="cuda")

    def mfma_loop():
        rc = plib.ldv_peak_mfma(nblk, ctypes.c_void_p(pout.data_ptr()),
                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert rc == 0, "MFMA probe launch failed (%d)" % rc

    out = {}
    for name, fn, work in (("copy_GB_s", lambda: dst.copy_(src), 2 * n * 4 / 1e9),
                           ("bf16_mfma_loop_TFLOP_s", mfma_loop, plib.ldv_peak_mfma_flops(nblk) / 1e12),
                           ("bf16_gemm_TFLOP_s", lambda: torch.matmul(a, b), 2 * 8192 ** 3 / 1e12)):
        fn()
        torch.cuda.synchronize()
        best = None
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) * 1e-3
            best = t if best is None else min(best, t)
        out[name] = work / best
    del src, dst, a, b, pout
    torch.cuda.empty_cache()
    return out


def capture(torch, fns, K):
    """One HIP graph holding K launches of each function in fns, in order."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(K):
            for fn in fns:
                fn(i)
    return g


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted({**WORKLOADS, **LONG_WORKLOADS}))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-next", action="store_true", help="skip timing the in-block read and the selection")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="minimum CPU-oracle time")
    ap.add_argument("--repeats", type=int, default=5, help="timed replays of each per-kernel graph")
    ap.add_argument("--no-peaks", action="store_true", help="skip measuring the copy and GEMM peaks")
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

    wl = {**WORKLOADS, **LONG_WORKLOADS}[args.workload]
    if wl.T > 64:  # the in-block reads and the selection take drafts of at most 64 nodes
        args.no_next = True
    K = args.steps
    nsets = int(min(64, max(4, -(-1_000_000_000 // set_bytes(wl)))))
    print("[bench] generating %s inputs (%d rotated buffer sets)" % (wl.key, nsets), file=sys.stderr, flush=True)
    x = make_inputs(wl)
    run = Runner(ldv, torch, wl, x, nsets, not args.no_next)
    hev = HipEvents()
    sh = torch.cuda.current_stream().cuda_stream  # the stream the library launches on (outside capture)

    def timed(fn_replay):
        e0, e1 = hev.create(), hev.create()
        hev.record(e0, sh)
        fn_replay()
        hev.record(e1, sh)
        torch.cuda.synchronize()
        t = hev.elapsed_s(e0, e1)
        hev.destroy(e0)
        hev.destroy(e1)
        return t

    fns = run.step_fns()
    for i in range(args.warmup):
        for fn in fns:
            fn(i)
    torch.cuda.synchronize()
    assert int(run.status.item()) == 0, "device status %d" % int(run.status.item())

    # the timed region: K steps (one HIP graph, or K eager steps)
    if args.eager:
        replay = lambda: [fn(i) for i in range(K) for fn in fns]
    else:
        g_step = capture(torch, fns, K)
        g_step.replay()  # untimed: first replay uploads the graph
        replay = g_step.replay
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_total = timed(replay)
    wall = time.perf_counter() - t0
    ms_per_step = t_total / K * 1e3
    nodes = wl.B * wl.H * wl.T
    value = nodes * K / t_total

    # per-kernel durations: K back-to-back launches of one kernel in one
    # graph (rotating buffer sets), median of `repeats` timed replays
    def per_kernel(fn):
        if args.eager:
            rep = lambda: [fn(i) for i in range(K)]
        else:
            g = capture(torch, [fn], K)
            g.replay()
            rep = g.replay
        torch.cuda.synchronize()
        ts = [timed(rep) / K for _ in range(args.repeats)]
        return float(np.median(ts)), float(np.min(ts)), float(np.max(ts))

    alg = algorithmic(wl, x)
    peaks = None if args.no_peaks else measure_peaks(torch)
    kern = {}
    names = [("verify", run.verify, alg["verify"]), ("commit", run.commit, alg["commit"])]
    if wl.P > 0:
        names.append(("gather", run.gather, alg["gather"]))
    if not args.no_next:
        read_bytes, sel_bytes = algorithmic_next(wl, run.P2, run.Qn2)
        if wl.P > 0:  # the gather's reads written into packed bf16 drafter features
            esz = 2 if wl.qkv == "bf16" else 4
            pk = wl.B * wl.P * wl.H * (wl.D * wl.D * 4 + wl.Qn * wl.D * esz + wl.Qn * wl.D * 2) + wl.B * wl.P * 4
            names.append(("gather_packed_bf16", run.gather_packed, pk))
        names.append(("read_block", run.read, read_bytes))
        if wl.V > 0:
            names.append(("select", run.select, sel_bytes))
    for name, fn, by in names:
        med, lo, hi = per_kernel(fn)
        kern[name] = {"us": med * 1e6, "us_min": lo * 1e6, "us_max": hi * 1e6, "launches": K,
                      "alg_bytes": int(by), "GB_s": by / med / 1e9, "hbm_frac": by / med / 1e9 / HBM_PEAK_GBS}
    assert int(run.status.item()) == 0, "device status %d" % int(run.status.item())
    kern["verify"]["nodes_per_s"] = nodes / kern["verify"]["us"] * 1e6
    kern["verify"]["alg_flops"] = alg["verify_flops"]
    kern["verify"]["mfma_frac"] = alg["verify_flops"] / (kern["verify"]["us"] * 1e-6) / (BF16_PEAK_TFLOPS * 1e12)
    # o = S q products of the state reads (2 d^2 flops per query)
    for name, nq in (("gather", wl.B * wl.P * wl.H * wl.Qn), ("gather_packed_bf16", wl.B * wl.P * wl.H * wl.Qn),
                     ("read_block", wl.B * (run.P2 if not args.no_next else 0) * wl.H * (run.Qn2 if not args.no_next else 0))):
        if name in kern and nq:
            fl = 2.0 * wl.D * wl.D * nq
            kern[name]["alg_flops"] = fl
            kern[name]["mfma_frac"] = fl / (kern[name]["us"] * 1e-6) / (BF16_PEAK_TFLOPS * 1e12)
    if peaks:
        for v in kern.values():
            v["hbm_frac_of_measured_copy"] = v["GB_s"] / peaks["copy_GB_s"]
            if "mfma_frac" in v:
                v["mfma_frac_of_measured_loop"] = v["mfma_frac"] * BF16_PEAK_TFLOPS / peaks["bf16_mfma_loop_TFLOP_s"]
    if "read_block" in kern:
        kern["read_block"].update({"P": run.P2, "Qn": run.Qn2})
    if "select" in kern:
        kern["select"].update({"V": wl.V, "logits": wl.qkv})
    step_names = [n for n in ("verify", "commit", "gather") if n in kern]
    dom = max(step_names, key=lambda n: kern[n]["us"])
    srcs = {"verify": "speculative_decoding_verify_amd/csrc/verify.hip",
            "commit": "speculative_decoding_verify_amd/csrc/commit.hip",
            "gather": "speculative_decoding_verify_amd/csrc/gather.hip"}
    roof = {"kernel": dom, "bound": "hbm", "achieved": kern[dom]["GB_s"], "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": kern[dom]["hbm_frac"],
            "traffic": traffic_from_profiles(dom, [srcs[dom], "speculative_decoding_verify_amd/csrc/ldv_device.hpp"],
                                             wl.key)}
    if peaks:
        roof["measured_peaks"] = peaks
        roof["frac_of_measured_copy"] = kern[dom]["GB_s"] / peaks["copy_GB_s"]

    cpu = None
    if not args.no_cpu:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, x, args.cpu_seconds, max(30.0, args.cpu_seconds))

    out = {
        "metric": METRIC, "value": value, "unit": "nodes/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.key, "B": wl.B, "H": wl.H, "d_k": wl.D, "d_v": wl.D, "T": wl.T,
                   "topology": wl.topology, "qkv": wl.qkv, "state": "f32",
                   "gather": ({"P": wl.P, "Qn": wl.Qn, "pool_slots": wl.B * wl.R} if wl.P else None),
                   "step": "+".join(step_names), "rotated_sets": nsets,
                   "timing": "eager launches" if args.eager else "HIP graph replay"},
        "kernels": kern,
        "roofline": roof,
        "cpu_baseline": cpu,
        "wall_s": wall,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
