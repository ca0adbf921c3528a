"""A batch of drafts of different lengths, padded to one node count.

The calls take one node count T for the whole batch.  A sequence whose draft
is shorter is padded with extra nodes placed after its real ones (each under
any earlier node, or a root) and given the draft token -1.  A node's outputs
depend only on its own path (Bole page, section IV, Eq. (2)), so padding
changes no real node; token -1 never equals a target argmax, so the greedy
selection never accepts a padding node and commit forms a real node's state.
Each sequence is checked against the oracle run on that sequence alone, at
its own length.
"""
import numpy as np
import pytest

from gpu_util import check, dev, host, to_device
from workloads import WORKLOADS, make_inputs, make_tree

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ldv():
    import speculative_decoding_verify_amd as m
    return m


CASES = [  # topology, padded node count, real draft lengths
    ("chain", 16, [1, 7, 16, 3, 12]),
    ("tree", 40, [20, 5, 37, 1, 33]),
    ("tree", 64, [64, 2, 17, 40]),
    ("tree", 12, [12, 1, 9]),
]


def ragged_parents(rng, topology, T, lens):
    par = np.empty((len(lens), T), dtype=np.int32)
    for b, n in enumerate(lens):
        if topology == "chain":
            par[b] = np.arange(-1, T - 1, dtype=np.int32)
        else:
            par[b, :n] = make_tree(rng, 1, n)[0]
            par[b, n:] = [rng.integers(-1, m) for m in range(n, T)]
    return par


def draft_tokens(rng, logits, par, lens, p_match=0.75):
    """Real nodes take their parent row's argmax with probability p_match
    (else a random token); padding nodes take -1."""
    B, T = par.shape
    V = logits.shape[2]
    best = logits.argmax(axis=2)
    tok = np.full((B, T), -1, dtype=np.int32)
    for b, n in enumerate(lens):
        for m in range(n):
            tok[b, m] = best[b, par[b, m] + 1] if rng.random() < p_match else rng.integers(0, V)
    return tok


@pytest.mark.parametrize("topology,T,lens", CASES, ids=lambda v: str(v))
def test_ragged_batch(ldv, orc, topology, T, lens):
    B, H, D, V = len(lens), 3, 128, 1000
    seed = 9100 + T + len(lens)
    wl = WORKLOADS["tree64"].replace(B=B, H=H, D=D, T=T, topology="tree", qkv="bf16",
                                     accept="uniform-node", seed=seed)
    x = make_inputs(wl, with_gather=False)
    rng = np.random.default_rng(seed)
    chain = topology == "chain"
    par = ragged_parents(rng, topology, T, lens)
    x["parent"] = par
    logits = rng.standard_normal((B, T + 1, V)).astype(np.float32)
    tokens = draft_tokens(rng, logits, par, lens)
    print("ragged %s T=%d lens=%s" % (topology, T, lens), flush=True)

    d = to_device(x, "bf16")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    if chain:
        o, u, lp = ldv.verify_chain(d["q"], d["k"], d["v"], d["a"], d["beta"], d["S0"], status=st)
    else:
        o, u, lp = ldv.verify_tree(d["q"], d["k"], d["v"], d["a"], d["beta"], d["S0"], d["parent"],
                                   status=st)
    dpar = None if chain else d["parent"]
    _, acc, alen, bonus = ldv.select_accepted(dev(logits), dev(tokens), dpar, status=st)
    S = ldv.commit_state(d["k"], u, lp, acc, d["S0"], parent=dpar, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    go, gu = host(o), host(u)
    gacc, galen, gbonus = acc.cpu().numpy(), alen.cpu().numpy(), bonus.cpu().numpy()
    gS = host(S)

    for b, n in enumerate(lens):
        cut = lambda a: np.ascontiguousarray(a[b:b + 1, :n])
        spar = None if chain else cut(par)
        ro, ru, _, s = orc.verify(cut(x["q"]), cut(x["k"]), cut(x["v"]), cut(x["a"]), cut(x["beta"]),
                                  x["S0"][b:b + 1], spar, want_u=True)
        assert s == 0
        check("seq %d (%d of %d nodes) o" % (b, n, T), go[b:b + 1, :n], ro)
        check("seq %d (%d of %d nodes) u" % (b, n, T), gu[b:b + 1, :n], ru)
        _, racc, ralen, rbonus, s = orc.select(np.ascontiguousarray(logits[b:b + 1, :n + 1]),
                                               cut(tokens), spar)
        assert s == 0
        assert (int(gacc[b]), int(galen[b]), int(gbonus[b])) == (int(racc[0]), int(ralen[0]), int(rbonus[0])), b
        assert -1 <= gacc[b] < n  # never a padding node
        rS, s = orc.commit(cut(x["k"]), cut(x["v"]), cut(x["a"]), cut(x["beta"]), x["S0"][b:b + 1],
                           racc, spar)
        assert s == 0
        check("seq %d committed state" % b, gS[b:b + 1], rS)
    print("accepted", gacc.tolist(), flush=True)
