"""Seeded synthetic inputs for gated-delta-rule draft verification.

This module is the ONLY code shared by the fp64 oracle (``oracle/``) and the
HIP path (``speculative_decoding_verify_amd/``).  It draws random numbers and
shapes them into inputs; it holds none of the method's arithmetic (no state
update, no closed form, no decay products).

Workload shapes follow the linear-attention layers that the pages speculate
through: a GDN-1.3B-shaped layer (SpecLA, "Stuff That Spins" page, key stats:
GDN-1.3B on H100) and a hybrid-27B-shaped layer with drafter state reads
(ReaDy, arXiv 2610.20503, Fig. 2a-4).  Trees follow the Bole page (arXiv
2608.01651, section IV): a parent-index array in topological order.

Distributions (the second argument of N(mu, s) is the standard deviation):
  q, k    N(0, 1), L2-normalised per (sequence, node, head) in fp32, then cast
          to the input dtype (bf16 by round-to-nearest-even, or kept fp32)
  v       N(0, 1), cast the same way
  beta    sigmoid(N(0, 1))                 fp32, [B, T, H]
  a       exp(-softplus(N(0, 1)))          fp32, [B, T, H], in (0, 1)
  S0      N(0, s0_std)                     fp32, [B, H, dv, dk]
The draw order per workload is fixed: S0, q, k, v, a, beta, parent,
acceptance, then (gather only) pool, slots, queries.

Two further input sets come from generators of their own, seeded from the
workload seed and a fixed stream tag, so they leave the draws above alone:
  block reads    positions [B, P]: P distinct nodes of the block per sequence
                 (uniform without replacement); queries [B, P, H, Qn, d] as
                 for the gather
  selection      draft tokens [B, T] uniform over a vocabulary of V; target
                 logits [B, T+1, V] N(0, 1), cast like q/k/v, with the token of
                 every node on the root path of the drawn accepted node set to
                 8 in the row that predicts it (so the target agrees with the
                 draft along that path; which node is accepted is still decided
                 by the selection itself)
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = ["Workload", "WORKLOADS", "make_inputs", "bf16_round",
           "make_tree", "make_chain", "draw_acceptance", "tree_depths",
           "l2_normalise_f32", "make_block_read_inputs", "make_select_inputs"]

# stream tags of the generators that do not share the main draw sequence
_READ_STREAM = 101
_SELECT_STREAM = 102


@dataclasses.dataclass(frozen=True)
class Workload:
    key: str
    desc: str
    B: int
    H: int
    D: int            # d_k = d_v
    T: int            # draft nodes per sequence
    topology: str     # "chain" | "tree"
    qkv: str          # "bf16" | "f32"
    s0_std: float
    accept: str       # "uniform-len" | "geometric" | "root-path" | "uniform-node"
    seed: int
    # gather (drafter state reads); P == 0 means no gather in this workload
    P: int = 0        # positions read per sequence
    R: int = 0        # pool slots owned by each sequence
    Qn: int = 0       # query vectors per (sequence, position, head)
    max_depth: int = 8
    max_fanout: int = 4
    # vocabulary of the target logits for accepted-node selection (0 = none)
    V: int = 0

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny-chain": Workload(
        "tiny-chain", "tiny chain: B1 H2 d16, chain of 4, fp32 q/k/v",
        B=1, H=2, D=16, T=4, topology="chain", qkv="f32", s0_std=0.1,
        accept="uniform-len", seed=1),
    "gdn1.3b-chain": Workload(
        "gdn1.3b-chain", "GDN-1.3B-shaped layer, chain verify: B16 H16 d128, chain of 8",
        B=16, H=16, D=128, T=8, topology="chain", qkv="bf16", s0_std=0.05,
        accept="geometric", seed=2, V=32000),
    "tree64": Workload(
        "tree64", "tree verify: B32 H16 d128, 64-node tree (depth<=8, fan-out<=4)",
        B=32, H=16, D=128, T=64, topology="tree", qkv="bf16", s0_std=0.05,
        accept="root-path", seed=3, V=32000),
    "hybrid27b-chain-gather": Workload(
        "hybrid27b-chain-gather",
        "27B-hybrid-shaped layer: B64 H32 d128, chain of 16 + state reads at 4 positions x 16 queries",
        B=64, H=32, D=128, T=16, topology="chain", qkv="bf16", s0_std=0.05,
        accept="geometric", seed=4, P=4, R=16, Qn=16, V=151936),
    "batch256-tree-commit": Workload(
        "batch256-tree-commit", "large-batch commit: B256 H32 d128, 32-node tree, accepted uniform over nodes",
        B=256, H=32, D=128, T=32, topology="tree", qkv="bf16", s0_std=0.05,
        accept="uniform-node", seed=5, V=151936),
}


# Chains longer than one 64-node chunk (ldv_verify_chain_long): the
# 27B-hybrid- and GDN-1.3B-shaped layers with long draft blocks.  Kept apart
# from WORKLOADS, every entry of which the per-call tests run at full size.
LONG_WORKLOADS = {
    "hybrid27b-chain256": Workload(
        "hybrid27b-chain256", "27B-hybrid-shaped layer, long chain: B64 H32 d128, chain of 256 (4 chunks)",
        B=64, H=32, D=128, T=256, topology="chain", qkv="bf16", s0_std=0.05,
        accept="geometric", seed=6),
    "gdn1.3b-chain1024": Workload(
        "gdn1.3b-chain1024", "GDN-1.3B-shaped layer, long chain: B16 H16 d128, chain of 1024 (16 chunks)",
        B=16, H=16, D=128, T=1024, topology="chain", qkv="bf16", s0_std=0.05,
        accept="geometric", seed=7),
}


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); return fp32.

    Done bitwise so that it needs no torch: add the rounding bias
    0x7FFF + lsb to the fp32 bit pattern and clear the low 16 bits.  Inputs are
    finite (drawn from normals), so no NaN handling is needed.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    return r.view(np.float32)


def l2_normalise_f32(x: np.ndarray) -> np.ndarray:
    """Unit-normalise along the last axis in fp32."""
    x = x.astype(np.float32, copy=False)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    return (x / n).astype(np.float32)


def make_chain(B: int, T: int) -> np.ndarray:
    par = np.tile(np.arange(-1, T - 1, dtype=np.int32), (B, 1))
    return par.reshape(B, T)


def make_tree(rng: np.random.Generator, B: int, T: int,
              max_depth: int = 8, max_fanout: int = 4) -> np.ndarray:
    """Seeded random attach trees in topological order.

    Node 0 is the root (parent -1).  Node n >= 1 attaches to a uniformly chosen
    earlier node whose depth is below ``max_depth`` (root depth = 1) and that
    has fewer than ``max_fanout`` children.
    """
    par = np.empty((B, T), dtype=np.int32)
    for b in range(B):
        depth = np.zeros(T, dtype=np.int64)
        nchild = np.zeros(T, dtype=np.int64)
        par[b, 0] = -1
        depth[0] = 1
        for n in range(1, T):
            cand = np.nonzero((depth[:n] < max_depth) & (nchild[:n] < max_fanout))[0]
            if cand.size == 0:
                raise ValueError("tree cannot grow under the depth/fan-out limits")
            p = int(cand[rng.integers(cand.size)])
            par[b, n] = p
            depth[n] = depth[p] + 1
            nchild[p] += 1
    return par


def tree_depths(parent_row: np.ndarray) -> np.ndarray:
    """Depth of every node (root = 1) of one topologically ordered parent row."""
    T = parent_row.shape[0]
    d = np.zeros(T, dtype=np.int64)
    for n in range(T):
        p = int(parent_row[n])
        d[n] = 1 if p < 0 else d[p] + 1
    return d


def _geom0(rng: np.random.Generator, p_stop: float) -> int:
    # successes before the first failure, each draft kept with prob 1 - p_stop
    return int(rng.geometric(p_stop)) - 1


def draw_acceptance(rng: np.random.Generator, wl: Workload,
                    parent: np.ndarray) -> np.ndarray:
    """Accepted node per sequence (-1 = nothing accepted)."""
    B, T = parent.shape
    acc = np.empty(B, dtype=np.int32)
    for b in range(B):
        if wl.accept == "uniform-len":
            A = int(rng.integers(0, T + 1))
            acc[b] = A - 1
        elif wl.accept == "geometric":
            A = min(_geom0(rng, 0.3), T)
            acc[b] = A - 1
        elif wl.accept == "root-path":
            children = [[] for _ in range(T)]
            for n in range(T):
                if parent[b, n] >= 0:
                    children[int(parent[b, n])].append(n)
            path = [0]
            while children[path[-1]]:
                ch = children[path[-1]]
                path.append(ch[int(rng.integers(len(ch)))])
            A = min(_geom0(rng, 0.3), len(path))
            acc[b] = path[A - 1] if A > 0 else -1
        elif wl.accept == "uniform-node":
            acc[b] = int(rng.integers(0, T))
        else:
            raise ValueError(wl.accept)
    return acc


def _cast(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_round(x) if dtype == "bf16" else x.astype(np.float32)


def make_inputs(wl: Workload, seed: Optional[int] = None,
                with_gather: Optional[bool] = None) -> dict:
    """Draw every input of a workload.  Returns fp32/int32 numpy arrays.

    Arrays holding bf16 inputs contain bf16-exact fp32 values; the GPU side
    casts them to bf16 without loss, the oracle upcasts them to fp64 without
    loss, so both see identical numbers.
    """
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    B, H, D, T = wl.B, wl.H, wl.D, wl.T
    out = {}
    out["S0"] = (rng.standard_normal((B, H, D, D), dtype=np.float32)
                 * np.float32(wl.s0_std)).astype(np.float32)
    q = l2_normalise_f32(rng.standard_normal((B, T, H, D), dtype=np.float32))
    k = l2_normalise_f32(rng.standard_normal((B, T, H, D), dtype=np.float32))
    v = rng.standard_normal((B, T, H, D), dtype=np.float32)
    out["q"] = _cast(q, wl.qkv)
    out["k"] = _cast(k, wl.qkv)
    out["v"] = _cast(v, wl.qkv)
    a_raw = rng.standard_normal((B, T, H), dtype=np.float32)
    b_raw = rng.standard_normal((B, T, H), dtype=np.float32)
    # a = exp(-softplus(x)) = 1 / (1 + e^x); beta = sigmoid(x)
    out["a"] = (1.0 / (1.0 + np.exp(a_raw.astype(np.float64)))).astype(np.float32)
    out["beta"] = (1.0 / (1.0 + np.exp(-b_raw.astype(np.float64)))).astype(np.float32)
    if wl.topology == "chain":
        out["parent"] = make_chain(B, T)
    else:
        out["parent"] = make_tree(rng, B, T, wl.max_depth, wl.max_fanout)
    out["accepted"] = draw_acceptance(rng, wl, out["parent"])
    g = wl.P > 0 if with_gather is None else with_gather
    if g:
        out.update(make_gather_inputs(rng, wl))
    return out


def make_gather_inputs(rng: np.random.Generator, wl: Workload) -> dict:
    B, H, D, P, R, Qn = wl.B, wl.H, wl.D, wl.P, wl.R, wl.Qn
    pool = (rng.standard_normal((B * R, H, D, D), dtype=np.float32)
            * np.float32(wl.s0_std)).astype(np.float32)
    slot = np.empty((B, P), dtype=np.int32)
    for b in range(B):
        slot[b] = b * R + rng.choice(R, size=P, replace=False)
    queries = l2_normalise_f32(rng.standard_normal((B, P, H, Qn, D), dtype=np.float32))
    return {"pool": pool, "slot": slot, "queries": _cast(queries, wl.qkv)}


def make_block_read_inputs(wl: Workload, P: Optional[int] = None, Qn: Optional[int] = None,
                           seed: Optional[int] = None) -> dict:
    """Positions and queries for reads of states inside the verified block.

    P distinct node positions per sequence (default: the workload's gather P,
    at most T) and Qn queries per (sequence, position, head), unit-normalised
    and cast like q.
    """
    rng = np.random.default_rng([wl.seed if seed is None else seed, _READ_STREAM])
    B, H, D, T = wl.B, wl.H, wl.D, wl.T
    P = min(wl.P or 4, T) if P is None else P
    Qn = (wl.Qn or 16) if Qn is None else Qn
    pos = np.empty((B, P), dtype=np.int32)
    for b in range(B):
        pos[b] = rng.choice(T, size=P, replace=P > T)
    queries = l2_normalise_f32(rng.standard_normal((B, P, H, Qn, D), dtype=np.float32))
    return {"pos": pos, "queries": _cast(queries, wl.qkv)}


def make_select_inputs(wl: Workload, parent: np.ndarray, accepted: np.ndarray,
                       V: Optional[int] = None, logits_dtype: Optional[str] = None,
                       seed: Optional[int] = None) -> dict:
    """Draft tokens and target logits for greedy accepted-node selection.

    ``accepted`` (the workload's drawn acceptance) only shapes the logits: the
    row that predicts each node on its root path gets the value 8 at that
    node's token.  Returns tokens [B, T] int32 and logits [B, T+1, V] fp32
    (bf16-exact when the dtype is bf16).
    """
    rng = np.random.default_rng([wl.seed if seed is None else seed, _SELECT_STREAM])
    B, T = parent.shape
    V = wl.V if V is None else V
    if V <= 0:
        raise ValueError("workload has no vocabulary")
    tokens = rng.integers(0, V, size=(B, T), dtype=np.int32)
    logits = rng.standard_normal((B, T + 1, V), dtype=np.float32)
    for b in range(B):
        n = int(accepted[b])
        while n >= 0:
            p = int(parent[b, n])
            logits[b, p + 1, tokens[b, n]] = 8.0
            n = p
    return {"tokens": tokens, "logits": _cast(logits, logits_dtype or wl.qkv)}
