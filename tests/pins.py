"""Independent checks that pin the fp64 oracle to something other than itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when the oracle disagrees with:
  * a hand-worked example (tests/golden/tree4_d2_handworked.json),
  * the closed form of the Bole page (arXiv 2608.01651, section IV, Eq. (2)),
    evaluated here in numpy with a library linear solve,
  * the commit-from-factors identity that the same section's "Lemma 1" and
    Eq. (9) rest on (only P, K, U and the committed state are kept),
  * brute-force matrix products of the recurrence on tiny sizes,
  * special cases with closed forms (b = 0: pure decay; a = 1, b = 0: pure
    read; b = 1 with a unit key: the delta rule overwrites the value at that
    key).
For the reads of in-block states and the accepted-node selection:
  * the hand-worked tree above and a hand-worked selection example
    (tests/golden/select_forest6_handworked.json),
  * the factorised state P_j S0 + sum (P_j/P_m) u_m k_m^T with U from the
    library solve, and brute-force matrices,
  * a set-based restatement of the greedy walk (a node is accepted iff every
    node on its path is the first child whose token the target predicts) with
    an argmax written as a minimum over sort keys, and numpy's argmax on
    chains.
The same functions run against oracle builds with planted mistakes
(test_oracle_mutants.py) to show that each plausible mistake fails one.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np

from workloads import l2_normalise_f32, make_chain, make_tree

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ------------------------------------------------------------------ helpers

def rel_err(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(x - ref)) / (den if den > 0 else 1.0))


def random_case(seed, B, T, H, dk, dv, topology="tree", s0_std=0.1, max_depth=8, max_fanout=4,
                a=None, beta=None, unit_k=True):
    rng = np.random.default_rng(seed)
    S0 = (rng.standard_normal((B, H, dv, dk)) * s0_std).astype(np.float32)
    q = l2_normalise_f32(rng.standard_normal((B, T, H, dk)).astype(np.float32))
    k = rng.standard_normal((B, T, H, dk)).astype(np.float32)
    if unit_k:
        k = l2_normalise_f32(k)
    v = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    aa = (1.0 / (1.0 + np.exp(rng.standard_normal((B, T, H))))).astype(np.float32)
    bb = (1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))).astype(np.float32)
    if a is not None:
        aa = np.full((B, T, H), a, dtype=np.float32)
    if beta is not None:
        bb = np.full((B, T, H), beta, dtype=np.float32)
    if topology == "chain":
        par = make_chain(B, T)
    else:
        par = make_tree(rng, B, T, max_depth, max_fanout)
    return dict(q=q, k=k, v=v, a=aa, beta=bb, S0=S0, parent=par)


def path_of(par_row, n):
    p = []
    m = n
    while m >= 0:
        p.append(m)
        m = int(par_row[m])
    return p[::-1]


def closed_form_head(q, k, v, a, beta, S0, par_row):
    """Eq. (2) of the Bole page for one (sequence, head), fp64.

    O = D_P Q S_pre + C (I + G)^{-1} D_beta (V - D_P K S_pre), with S_pre = S0^T
    (Eq. (2) writes O = Q S_pre with S_pre of shape d_k x d_v; the recurrence
    reads o = S q with S of shape d_v x d_k).  G and C are not printed on the
    page; unrolling the recurrence gives, for m on the path of n,
      C[n, m] = (P_n / P_m) q_n . k_m              (m = n included)
      G[n, m] = beta_n (P_n / P_m) k_n . k_m       (m a strict ancestor)
    Returns (O [T, dv], U [T, dv], P [T], G [T, T]).
    """
    T = q.shape[0]
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    a = np.asarray(a, np.float64)
    beta = np.asarray(beta, np.float64)
    Spre = np.asarray(S0, np.float64).T
    P = np.empty(T)
    for n in range(T):
        P[n] = np.prod([a[m] for m in path_of(par_row, n)])
    C = np.zeros((T, T))
    G = np.zeros((T, T))
    for n in range(T):
        for m in path_of(par_row, n):
            C[n, m] = P[n] / P[m] * (q[n] @ k[m])
            if m != n:
                G[n, m] = beta[n] * P[n] / P[m] * (k[n] @ k[m])
    DP = np.diag(P)
    Db = np.diag(beta)
    R = Db @ (v - DP @ k @ Spre)
    U = np.linalg.solve(np.eye(T) + G, R)
    O = DP @ q @ Spre + C @ U
    return O, U, P, G


def brute_force_states(k, v, a, beta, S0, par_row):
    """S_n for every node by explicit matrices: S = a S_p (I - b k k^T) + b v k^T."""
    T, dk = k.shape
    k, v = np.asarray(k, np.float64), np.asarray(v, np.float64)
    out = []
    for n in range(T):
        S = np.asarray(S0, np.float64).copy()
        for m in path_of(par_row, n):
            km = k[m][:, None]
            S = a[m] * S @ (np.eye(dk) - beta[m] * km @ km.T) + beta[m] * v[m][:, None] @ km.T
        out.append(S)
    return np.stack(out)


# --------------------------------------------------------------------- pins

def load_golden():
    with open(os.path.join(GOLDEN, "tree4_d2_handworked.json")) as f:
        g = json.load(f)
    fr = lambda x: np.vectorize(lambda s: float(Fraction(s)))(np.array(x, dtype=object)).astype(np.float64)
    return g, fr


def pin_golden(orc):
    """Hand-worked 4-node tree at d = 2: every value exact (dyadic)."""
    g, fr = load_golden()
    T = len(g["parent"])
    q = fr(g["q"]).reshape(1, T, 1, 2).astype(np.float32)
    k = fr(g["k"]).reshape(1, T, 1, 2).astype(np.float32)
    v = fr(g["v"]).reshape(1, T, 1, 2).astype(np.float32)
    a = fr(g["a"]).reshape(1, T, 1).astype(np.float32)
    beta = fr(g["beta"]).reshape(1, T, 1).astype(np.float32)
    S0 = fr(g["S0"]).reshape(1, 1, 2, 2).astype(np.float32)
    par = np.array(g["parent"], dtype=np.int32).reshape(1, T)
    o, st, status = orc.verify(q, k, v, a, beta, S0, par, want_states=True)
    assert status == 0
    assert np.array_equal(o[0, :, 0, :], fr(g["o"])), (o[0, :, 0, :], fr(g["o"]))
    assert np.array_equal(st[0, :, 0], fr(g["states"]))
    # log P_n: the log of the hand-worked gate products
    lp, status = orc.log_decay(a, par)
    assert status == 0
    assert np.max(np.abs(lp[0, :, 0] - np.log(fr(g["P"])))) <= 1e-15, (lp[0, :, 0], fr(g["P"]))
    for n in range(-1, T):
        S, status = orc.commit(k, v, a, beta, S0, np.array([n], np.int32), par)
        assert status == 0
        want = fr(g["S0"]) if n < 0 else fr(g["states"])[n]
        assert np.array_equal(S[0, 0], want), (n, S[0, 0], want)


def pin_closed_form(orc, seed=11, B=2, T=20, H=2, dk=16, dv=12, topology="tree", tol=1e-10):
    """Oracle outputs equal Eq. (2) evaluated with a library solve."""
    c = random_case(seed, B, T, H, dk, dv, topology, max_depth=6)
    o, u, _, status = orc.verify(**c, want_u=True)
    assert status == 0
    for b in range(B):
        for h in range(H):
            O, U, P, G = closed_form_head(c["q"][b, :, h], c["k"][b, :, h], c["v"][b, :, h],
                                          c["a"][b, :, h], c["beta"][b, :, h], c["S0"][b, h].astype(np.float64),
                                          c["parent"][b])
            e = rel_err(o[b, :, h], O)
            assert e <= tol, ("closed form", b, h, e)
            e = rel_err(u[b, :, h], U)
            assert e <= tol, ("closed form U", b, h, e)


def pin_commit_from_factors(orc, seed=12, B=2, T=16, H=2, d=8, tol=1e-10):
    """Committed state equals P_n* S0 + sum_{m on path} (P_n*/P_m) u_m k_m^T
    with U from Eq. (2)'s solve (the factorised speculative states)."""
    c = random_case(seed, B, T, H, d, d, "tree", max_depth=5)
    rng = np.random.default_rng(seed + 1)
    acc = rng.integers(0, T, size=B).astype(np.int32)
    S, status = orc.commit(c["k"], c["v"], c["a"], c["beta"], c["S0"], acc, c["parent"])
    assert status == 0
    for b in range(B):
        for h in range(H):
            _, U, P, _ = closed_form_head(c["q"][b, :, h], c["k"][b, :, h], c["v"][b, :, h],
                                          c["a"][b, :, h], c["beta"][b, :, h], c["S0"][b, h].astype(np.float64),
                                          c["parent"][b])
            n = int(acc[b])
            want = P[n] * c["S0"][b, h].astype(np.float64)
            for m in path_of(c["parent"][b], n):
                want = want + (P[n] / P[m]) * np.outer(U[m], c["k"][b, m, h].astype(np.float64))
            e = rel_err(S[b, h], want)
            assert e <= tol, ("factors", b, h, e)


def pin_brute_force(orc, seed=13, B=2, T=10, H=2, dk=6, dv=5, tol=1e-12):
    """Every node state and output equals explicit matrix products on tiny sizes."""
    c = random_case(seed, B, T, H, dk, dv, "tree", max_depth=5, unit_k=False)
    o, st, status = orc.verify(**c, want_states=True)
    assert status == 0
    for b in range(B):
        for h in range(H):
            S = brute_force_states(c["k"][b, :, h], c["v"][b, :, h], c["a"][b, :, h].astype(np.float64),
                                   c["beta"][b, :, h].astype(np.float64), c["S0"][b, h], c["parent"][b])
            assert rel_err(st[b, :, h], S) <= tol
            want_o = np.einsum("nij,nj->ni", S, c["q"][b, :, h].astype(np.float64))
            assert rel_err(o[b, :, h], want_o) <= tol


def pin_pure_decay(orc, seed=14, B=2, T=24, H=3, d=8, tol=1e-14):
    """beta = 0: S_n = P_n S0 and o_n = P_n S0 q_n, P_n the gate product on the path."""
    c = random_case(seed, B, T, H, d, d, "tree", beta=0.0)
    o, st, status = orc.verify(**c, want_states=True)
    assert status == 0
    for b in range(B):
        for h in range(H):
            S0 = c["S0"][b, h].astype(np.float64)
            for n in range(T):
                P = 1.0
                for m in path_of(c["parent"][b], n):
                    P *= float(c["a"][b, m, h])
                assert rel_err(st[b, n, h], P * S0) <= tol
                assert rel_err(o[b, n, h], P * (S0 @ c["q"][b, n, h].astype(np.float64))) <= tol


def pin_log_decay(orc, seed=26, B=3, T=20, H=4, d=4):
    """log P_n against closed forms: a chain with one gate value per head has
    log P_n = (n + 1) log a; on a tree, b = 0 makes every node state the
    decayed committed state, S_n = P_n S0, so exp(log P_n) S0 must equal the
    walk's state; and each node's value minus its parent's is log a_n."""
    c = random_case(seed, B, T, H, d, d, "chain")
    gate = np.array([0.5, 0.9, 0.25, 0.999], np.float32)[:H]
    c["a"] = np.broadcast_to(gate, (B, T, H)).copy()
    lp, status = orc.log_decay(c["a"], None)
    assert status == 0
    want = (np.arange(1, T + 1)[:, None] * np.log(gate.astype(np.float64))[None, :])[None]
    assert np.max(np.abs(lp - want)) <= 1e-13 * np.max(np.abs(want))
    t = random_case(seed + 1, B, T, H, d, d, "tree", beta=0.0)
    lp, status = orc.log_decay(t["a"], t["parent"])
    assert status == 0
    _, st, status = orc.verify(**t, want_states=True)
    assert status == 0
    S0 = t["S0"].astype(np.float64)
    assert rel_err(st, np.exp(lp)[..., None, None] * S0[:, None]) <= 1e-14
    # a chain far past the fp64 range of the plain product (|log P| ~ 1e4)
    long = (np.full((1, 20000, 1), 0.5, np.float32), 20000 * np.log(0.5))
    lpl, status = orc.log_decay(long[0], None)
    assert status == 0 and abs(lpl[0, -1, 0] - long[1]) <= 1e-12 * abs(long[1])
    la = np.log(t["a"].astype(np.float64))
    for b in range(B):
        for n in range(T):
            p = int(t["parent"][b, n])
            base = lp[b, p] if p >= 0 else 0.0
            assert np.max(np.abs(lp[b, n] - base - la[b, n])) <= 1e-12


def pin_pure_read(orc, seed=15, B=2, T=12, H=2, d=16):
    """a = 1, beta = 0: every node reads the committed state, o_n = S0 q_n."""
    c = random_case(seed, B, T, H, d, d, "tree", a=1.0, beta=0.0)
    o, _, status = orc.verify(**c)
    assert status == 0
    want = np.einsum("bhij,bnhj->bnhi", c["S0"].astype(np.float64), c["q"].astype(np.float64))
    assert rel_err(o, want) <= 1e-15


def pin_overwrite(orc, seed=16, B=2, T=12, H=2, d=16):
    """beta_n = 1 with a unit key: S_n k_n = v_n for any a_n and parent state
    (the delta rule replaces the value stored at key k_n).  With q_n = k_n the
    node output is v_n.  Keys are unit in fp32, so |k|^2 = 1 within ~1e-7."""
    c = random_case(seed, B, T, H, d, d, "tree", beta=1.0)
    c["q"] = c["k"].copy()
    o, st, status = orc.verify(**c, want_states=True)
    assert status == 0
    Sk = np.einsum("bnhij,bnhj->bnhi", st, c["k"].astype(np.float64))
    assert rel_err(Sk, c["v"]) <= 1e-6
    assert rel_err(o, c["v"]) <= 1e-6


def pin_chain_equals_decode(orc, seed=17, B=2, T=9, H=3, d=8):
    """A chain (explicit parent n-1, or no parent array) equals sequential
    decode with one running state, bit for bit (same operation order)."""
    c = random_case(seed, B, T, H, d, d, "chain")
    o_dec = orc.chain_decode(c["q"], c["k"], c["v"], c["a"], c["beta"], c["S0"])
    o_tree, _, s1 = orc.verify(**c)
    c2 = dict(c)
    c2["parent"] = None
    o_chain, _, s2 = orc.verify(**c2)
    assert s1 == 0 and s2 == 0
    assert np.array_equal(o_tree, o_dec)
    assert np.array_equal(o_chain, o_dec)


def pin_chunk_form(orc, seed=25, B=2, T=23, H=2, dk=6, dv=5, L=8, tol=1e-10):
    """The chunk form of long chains: verifying a chain chunk by chunk with
    Eq. (2) (numpy, library solve), each chunk from the state that Eq. (9)
    forms at the previous chunk's last node, gives the outputs of sequential
    decode, and the state after the last chunk is the oracle's commit of the
    chain's last node."""
    c = random_case(seed, B, T, H, dk, dv, "chain")
    o_dec = orc.chain_decode(c["q"], c["k"], c["v"], c["a"], c["beta"], c["S0"])
    S_last, status = orc.commit(c["k"], c["v"], c["a"], c["beta"], c["S0"], np.full(B, T - 1, np.int32))
    assert status == 0
    for b in range(B):
        for h in range(H):
            S = c["S0"][b, h].astype(np.float64)
            for t0 in range(0, T, L):
                n = min(L, T - t0)
                sl = slice(t0, t0 + n)
                kc = c["k"][b, sl, h].astype(np.float64)
                O, U, P, _ = closed_form_head(c["q"][b, sl, h], kc, c["v"][b, sl, h], c["a"][b, sl, h],
                                              c["beta"][b, sl, h], S, np.arange(-1, n - 1))
                assert rel_err(O, o_dec[b, sl, h]) <= tol, ("chunk o", b, h, t0)
                S = P[n - 1] * S + sum((P[n - 1] / P[m]) * np.outer(U[m], kc[m]) for m in range(n))
            assert rel_err(S, S_last[b, h]) <= tol, ("chunk end state", b, h)


def pin_tree_equals_dfs(orc, seed=18, B=3, T=40, H=2, d=8):
    """Path walk per node equals branch-by-branch DFS traversal, bit for bit."""
    c = random_case(seed, B, T, H, d, d, "tree")
    o, _, s1 = orc.verify(**c)
    o_dfs, s2 = orc.verify_dfs(**c)
    assert s1 == 0 and s2 == 0
    assert np.array_equal(o, o_dfs)


def pin_gather(orc, seed=19):
    """Gathered states are bit copies of pool[slot]; o = S q per query."""
    rng = np.random.default_rng(seed)
    pool = rng.standard_normal((7, 3, 16, 16)).astype(np.float32)
    slot = np.array([[6, 0, 2], [2, 2, 5]], dtype=np.int32)
    qs = rng.standard_normal((2, 3, 3, 5, 16)).astype(np.float32)
    o, st, status = orc.gather(pool, slot, qs)
    assert status == 0
    for b in range(2):
        for p in range(3):
            assert np.array_equal(st[b, p], pool[slot[b, p]])
            want = np.einsum("hij,hqj->hqi", pool[slot[b, p]].astype(np.float64), qs[b, p].astype(np.float64))
            assert rel_err(o[b, p], want) <= 1e-15


def pin_read_golden(orc):
    """Reads of the hand-worked tree's states: o = S_j q, exact (dyadic)."""
    g, fr = load_golden()
    T = len(g["parent"])
    k = fr(g["k"]).reshape(1, T, 1, 2).astype(np.float32)
    v = fr(g["v"]).reshape(1, T, 1, 2).astype(np.float32)
    a = fr(g["a"]).reshape(1, T, 1).astype(np.float32)
    beta = fr(g["beta"]).reshape(1, T, 1).astype(np.float32)
    S0 = fr(g["S0"]).reshape(1, 1, 2, 2).astype(np.float32)
    par = np.array(g["parent"], dtype=np.int32).reshape(1, T)
    pos = np.array([[-1, 1, 3, 2, 0]], dtype=np.int32)
    qs = np.array([[1, 0], [0, 1], [1, -2]], dtype=np.float32)
    queries = np.broadcast_to(qs, (1, pos.shape[1], 1, 3, 2)).copy()
    o, status = orc.read_states(k, v, a, beta, S0, pos, queries, par)
    assert status == 0
    states = fr(g["states"])
    for p, n in enumerate(pos[0]):
        S = fr(g["S0"]) if n < 0 else states[n]
        want = S @ qs.T.astype(np.float64)
        assert np.array_equal(o[0, p, 0], want.T), (n, o[0, p, 0], want.T)


def pin_read_from_factors(orc, seed=21, B=2, T=16, H=2, d=8, P=6, Qn=3, tol=1e-10):
    """In-block reads equal P_j S0 q + sum_{m on path(j)} (P_j/P_m)(k_m . q) u_m,
    U from Eq. (2)'s library solve; position -1 reads S0 itself."""
    c = random_case(seed, B, T, H, d, d, "tree", max_depth=5)
    rng = np.random.default_rng(seed + 1)
    pos = rng.integers(-1, T, size=(B, P)).astype(np.int32)
    pos[0, 0] = -1
    queries = rng.standard_normal((B, P, H, Qn, d)).astype(np.float32)
    o, status = orc.read_states(c["k"], c["v"], c["a"], c["beta"], c["S0"], pos, queries, c["parent"])
    assert status == 0
    for b in range(B):
        for h in range(H):
            _, U, Pn, _ = closed_form_head(c["q"][b, :, h], c["k"][b, :, h], c["v"][b, :, h],
                                           c["a"][b, :, h], c["beta"][b, :, h],
                                           c["S0"][b, h].astype(np.float64), c["parent"][b])
            S0 = c["S0"][b, h].astype(np.float64)
            for p in range(P):
                j = int(pos[b, p])
                q = queries[b, p, h].astype(np.float64)  # [Qn, d]
                if j < 0:
                    want = q @ S0.T
                else:
                    want = Pn[j] * (q @ S0.T)
                    for m in path_of(c["parent"][b], j):
                        km = c["k"][b, m, h].astype(np.float64)
                        want = want + (Pn[j] / Pn[m]) * np.outer(q @ km, U[m])
                e = rel_err(o[b, p, h], want)
                assert e <= tol, ("read factors", b, h, p, e)


def pin_read_brute_force(orc, seed=22, B=2, T=9, H=2, dk=6, dv=5, P=5, Qn=2, tol=1e-12):
    """In-block reads equal explicit matrix products on tiny sizes."""
    c = random_case(seed, B, T, H, dk, dv, "tree", max_depth=4, unit_k=False)
    rng = np.random.default_rng(seed + 1)
    pos = rng.integers(-1, T, size=(B, P)).astype(np.int32)
    queries = rng.standard_normal((B, P, H, Qn, dk)).astype(np.float32)
    o, status = orc.read_states(c["k"], c["v"], c["a"], c["beta"], c["S0"], pos, queries, c["parent"])
    assert status == 0
    for b in range(B):
        for h in range(H):
            S = brute_force_states(c["k"][b, :, h], c["v"][b, :, h], c["a"][b, :, h].astype(np.float64),
                                   c["beta"][b, :, h].astype(np.float64), c["S0"][b, h], c["parent"][b])
            for p in range(P):
                j = int(pos[b, p])
                Sj = c["S0"][b, h].astype(np.float64) if j < 0 else S[j]
                want = queries[b, p, h].astype(np.float64) @ Sj.T
                assert rel_err(o[b, p, h], want) <= tol


def _argmax_by_keys(row):
    """Index of the winner: the minimum of (is NaN, -value, index)."""
    keys = [(bool(np.isnan(x)), 0.0 if np.isnan(x) else -float(x), i) for i, x in enumerate(row)]
    return min(keys)[2]


def _select_by_sets(target, tokens, par_row):
    """Accepted node as the deepest node whose whole path is 'taken': node m is
    taken iff tokens[m] == target[parent(m) + 1] and no lower-index sibling has
    the same token.  The taken-path nodes form one chain."""
    T = len(tokens)
    taken = []
    for m in range(T):
        p = int(par_row[m])
        first = all(not (int(par_row[s]) == p and tokens[s] == tokens[m]) for s in range(m))
        taken.append(tokens[m] == target[p + 1] and first)
    ok = [all(taken[x] for x in path_of(par_row, n)) for n in range(T)]
    deepest, depth = -1, 0
    for n in range(T):
        d = len(path_of(par_row, n))
        if ok[n]:
            assert d != depth or n == deepest, "two accepted paths"
            if d > depth:
                deepest, depth = n, d
    return deepest, depth


def pin_select_golden(orc):
    """Hand-worked selection with equal maxima, NaN, -inf and signed zeros."""
    with open(os.path.join(GOLDEN, "select_forest6_handworked.json")) as f:
        g = json.load(f)
    logits = np.array([[float(x) for x in row] for row in g["logits"]], dtype=np.float32)[None]
    tokens = np.array([g["tokens"]], dtype=np.int32)
    par = np.array([g["parent"]], dtype=np.int32)
    target, acc, alen, bonus, status = orc.select(logits, tokens, par)
    assert status == 0
    assert target[0].tolist() == g["target"], target
    assert (int(acc[0]), int(alen[0]), int(bonus[0])) == (g["accepted"], g["accepted_len"], g["bonus"])


def pin_select_sets(orc, seed=23, B=24, T=12, V=4):
    """Greedy walk equals the set-based restatement, on small vocabularies with
    many equal logits, NaN and matching siblings."""
    rng = np.random.default_rng(seed)
    par = make_tree(rng, B, T, 5, 3)
    tokens = rng.integers(0, V, size=(B, T)).astype(np.int32)
    logits = rng.integers(-2, 3, size=(B, T + 1, V)).astype(np.float32)
    logits[rng.random(logits.shape) < 0.1] = np.nan
    target, acc, alen, bonus, status = orc.select(logits, tokens, par)
    assert status == 0
    for b in range(B):
        want_t = [_argmax_by_keys(logits[b, r]) for r in range(T + 1)]
        assert target[b].tolist() == want_t
        n, d = _select_by_sets(want_t, tokens[b].tolist(), par[b])
        assert (int(acc[b]), int(alen[b]), int(bonus[b])) == (n, d, want_t[n + 1]), (b, acc[b], n)


def pin_select_chain(orc, seed=24, B=16, T=10, V=50):
    """On a chain the accepted length is the leading run of nodes whose token
    is numpy's argmax of the row before them."""
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((B, T + 1, V)).astype(np.float32)
    tokens = rng.integers(0, V, size=(B, T)).astype(np.int32)
    for b in range(B):  # plant agreement on a random prefix
        for n in range(int(rng.integers(0, T + 1))):
            tokens[b, n] = int(np.argmax(logits[b, n]))
    for par in (None, make_chain(B, T)):
        target, acc, alen, bonus, status = orc.select(logits, tokens, par)
        assert status == 0
        am = np.argmax(logits, axis=-1)
        assert np.array_equal(target, am)
        run = np.cumprod(tokens == am[:, :T], axis=1).sum(axis=1)
        assert np.array_equal(alen, run)
        assert np.array_equal(acc, run - 1)
        assert np.array_equal(bonus, am[np.arange(B), run])


ALL_PINS = [pin_golden, pin_closed_form, pin_commit_from_factors, pin_brute_force, pin_pure_decay, pin_log_decay,
            pin_pure_read, pin_overwrite, pin_chain_equals_decode, pin_chunk_form, pin_tree_equals_dfs, pin_gather,
            pin_read_golden, pin_read_from_factors, pin_read_brute_force, pin_select_golden,
            pin_select_sets, pin_select_chain]
