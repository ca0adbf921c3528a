"""Throughput of the verify -> commit -> gather path on one MI355X.

One step = ldv_verify_chain / ldv_verify_tree over every draft node of the
batch, ldv_commit_state of the accepted node (in place), and, for workloads
with drafter reads, ldv_gather_states (o = S q for every query) - one pass of
the whole path over one batch of seeded synthetic inputs already resident in
HBM.  Each kernel is bracketed by HIP events (created without the
system-scope fence) on the stream it runs on, inside the timed region, so
the per-kernel durations come from the same run.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

Prints one JSON line.  --gpus N with N > 1 is refused: this path runs on one
GPU (every (sequence, head) is independent; see the design doc for how it shards).
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

from workloads import WORKLOADS, make_inputs, tree_depths  # noqa: E402

METRIC = "verified draft nodes/sec (B*H*N) on MFMA; commit+gather HBM GB/s vs peak"
DEFAULT_WORKLOAD = "hybrid27b-chain-gather"
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, AMD published
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, AMD published
NSETS = 3                  # rotated verify/commit buffer sets (defeats the 256 MB MALL)


def algorithmic(wl, x):
    """Algorithmic bytes (and flops) per launch of each kernel, from the
    shapes alone: every input read once, every output written once."""
    B, H, D, T = wl.B, wl.H, wl.D, wl.T
    esz = 2 if wl.qkv == "bf16" else 4
    depth = np.stack([tree_depths(r) for r in x["parent"]])         # [B, T]
    A = depth.sum(axis=1)                                           # sum of depths per sequence
    per_head = D * D * 4 + T * (3 * D * esz + 8 + 2 * D * 4 + 4)    # S0, q k v, a beta, o u, logp
    verify_bytes = B * H * per_head + (B * T * 4 if wl.topology == "tree" else 0)
    verify_flops = float(np.sum(H * (4 * T * D * D + 2 * D * (4 * A - 2 * T))))
    acc = x["accepted"]
    L = np.where(acc >= 0, depth[np.arange(B), np.maximum(acc, 0)], 0)
    committing = int(np.sum(acc >= 0))
    commit_bytes = H * (committing * 2 * D * D * 4 + int(np.sum(L)) * (D * 4 + D * esz + 4)) + B * 4
    gather_bytes = 0
    if wl.P > 0:
        gather_bytes = B * wl.P * H * (D * D * 4 + wl.Qn * D * esz + wl.Qn * D * 4) + B * wl.P * 4
    return dict(verify=verify_bytes, verify_flops=verify_flops, commit=commit_bytes, gather=gather_bytes)


def cpu_baseline(wl, x, seconds_min=10.0, seconds_cap=30.0):
    """The fp64 oracle (the path walked token by token) on the host cores,
    over the same workload: sequences in order, in chunks, repeating whole
    passes until at least seconds_min has elapsed (stopping early at
    seconds_cap); the rate is scaled to nodes/s."""
    import oracle
    threads = min(16, os.cpu_count() or 1)
    chain = wl.topology == "chain"
    done, t_total = 0, 0.0
    step = max(1, wl.B // 16)
    while (t_total < seconds_min or done % wl.B) and t_total < seconds_cap:
        b0 = done % wl.B
        sl = slice(b0, min(wl.B, b0 + step))
        t0 = time.perf_counter()
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
            "sample": "%d sequence passes over the %d sequences (all %d heads; every node verified by its "
                      "path walk, the accepted node committed%s), %.1f s" % (
                          done, wl.B, wl.H, ", 4 positions x 16 queries read per sequence" if wl.P else "",
                          t_total)}


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


def traffic_from_profiles(kernel_name, src_files):
    """HBM bytes per launch measured by rocprofv3 counters, if they were taken
    on the kernel source as it is now (else None)."""
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
    if not ent or ent.get("source_sha256") != h.hexdigest():
        return None
    return ent.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="minimum CPU-oracle time")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes (5 times), to scale "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE counters, and print its bandwidth")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(each (sequence, head) is independent; sharding is described in DESIGN.md).",
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

    wl = WORKLOADS[args.workload]
    chain = wl.topology == "chain"
    print("[bench] generating %s inputs" % wl.key, file=sys.stderr, flush=True)
    x = make_inputs(wl)
    dt = torch.bfloat16 if wl.qkv == "bf16" else torch.float32
    cuda = lambda a, t=None: (torch.from_numpy(np.ascontiguousarray(a)).cuda() if t is None
                              else torch.from_numpy(np.ascontiguousarray(a)).cuda().to(t))
    base = dict(q=cuda(x["q"], dt), k=cuda(x["k"], dt), v=cuda(x["v"], dt), a=cuda(x["a"]),
                beta=cuda(x["beta"]), S0=cuda(x["S0"]), parent=cuda(x["parent"]), acc=cuda(x["accepted"]))
    sets = []
    for i in range(NSETS):
        s = {n: t.clone() for n, t in base.items()}
        s["o"] = torch.empty((wl.B, wl.T, wl.H, wl.D), device="cuda")
        s["u"] = torch.empty((wl.B, wl.T, wl.H, wl.D), device="cuda")
        s["logp"] = torch.empty((wl.B, wl.T, wl.H), device="cuda")
        sets.append(s)
    del base
    if wl.P > 0:
        pool = cuda(x["pool"])
        slot = cuda(x["slot"])
        queries = cuda(x["queries"], dt)
        go = torch.empty((wl.B, wl.P, wl.H, wl.Qn, wl.D), device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream  # the stream the library launches on
    hev = HipEvents()

    def step(i, ev=None):
        s = sets[i % NSETS]
        if ev is not None:
            hev.record(ev[0], sh)
        if chain:
            ldv.verify_chain(s["q"], s["k"], s["v"], s["a"], s["beta"], s["S0"], o=s["o"], u=s["u"],
                             logp=s["logp"], status=status)
        else:
            ldv.verify_tree(s["q"], s["k"], s["v"], s["a"], s["beta"], s["S0"], s["parent"], o=s["o"],
                            u=s["u"], logp=s["logp"], status=status)
        if ev is not None:
            hev.record(ev[1], sh)
        ldv.commit_state(s["k"], s["u"], s["logp"], s["acc"], s["S0"], S_out=s["S0"],
                         parent=None if chain else s["parent"], status=status)
        if ev is not None:
            hev.record(ev[2], sh)
        if wl.P > 0:
            ldv.gather_states(pool, slot, queries, o=go, status=status)
        if ev is not None:
            hev.record(ev[3], sh)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "device status %d" % int(status.item())

    K = args.steps
    evs = [[hev.create() for _ in range(4)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_ver = np.array([hev.elapsed_s(evs[i][0], evs[i][1]) for i in range(K)])
    t_com = np.array([hev.elapsed_s(evs[i][1], evs[i][2]) for i in range(K)])
    t_gat = np.array([hev.elapsed_s(evs[i][2], evs[i][3]) for i in range(K)])
    t_total = hev.elapsed_s(evs[0][0], evs[K - 1][3])
    for e in (e for row in evs for e in row):
        hev.destroy(e)
    ms_per_step = t_total / K * 1e3
    nodes = wl.B * wl.H * wl.T
    value = nodes * K / t_total

    alg = algorithmic(wl, x)
    kern = {}
    for name, t, by in (("verify", t_ver, alg["verify"]), ("commit", t_com, alg["commit"]),
                        ("gather", t_gat, alg["gather"])):
        if name == "gather" and wl.P == 0:
            continue
        m = float(np.mean(t))
        kern[name] = {"us_mean": m * 1e6, "us_median": float(np.median(t)) * 1e6,
                      "alg_bytes": int(by), "GB_s": by / m / 1e9, "hbm_frac": by / m / 1e9 / HBM_PEAK_GBS}
    kern["verify"]["nodes_per_s"] = nodes / kern["verify"]["us_mean"] * 1e6
    kern["verify"]["alg_flops"] = alg["verify_flops"]
    kern["verify"]["mfma_frac"] = alg["verify_flops"] / (kern["verify"]["us_mean"] * 1e-6) / (BF16_PEAK_TFLOPS * 1e12)
    dom = max(kern, key=lambda n: kern[n]["us_mean"])
    srcs = {"verify": "speculative_decoding_verify_amd/csrc/verify.hip",
            "commit": "speculative_decoding_verify_amd/csrc/commit.hip",
            "gather": "speculative_decoding_verify_amd/csrc/gather.hip"}
    roof = {"kernel": dom, "bound": "hbm", "achieved": kern[dom]["GB_s"], "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": kern[dom]["hbm_frac"],
            "traffic": traffic_from_profiles(dom, [srcs[dom], "speculative_decoding_verify_amd/csrc/ldv_device.hpp"])}

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
                   "step": "verify+commit" + ("+gather" if wl.P else ""), "rotated_sets": NSETS},
        "kernels": kern,
        "roofline": roof,
        "cpu_baseline": cpu,
        "wall_s": wall,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
