"""HIP commit (the accepted node's state only) against the fp64 oracle."""
import numpy as np
import pytest

import pins
from gpu_util import check, dev, host, to_device
from workloads import WORKLOADS, make_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ldv():
    import speculative_decoding_verify_amd as m
    return m


def verify_then_commit(ldv, x, qkv, chain, accepted, in_place):
    d = to_device(x, qkv)
    par = None if chain else d["parent"]
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    if chain:
        o, u, lp = ldv.verify_chain(d["q"], d["k"], d["v"], d["a"], d["beta"], d["S0"], status=st)
    else:
        o, u, lp = ldv.verify_tree(d["q"], d["k"], d["v"], d["a"], d["beta"], d["S0"], d["parent"], status=st)
    S0 = d["S0"]
    out = S0 if in_place else torch.full_like(S0, 3.0)
    S = ldv.commit_state(d["k"], u, lp, dev(accepted), S0, S_out=out, parent=par, status=st)
    torch.cuda.synchronize()
    return S, int(st.item())


CASES = [
    # D, T, topology, qkv, in_place
    (128, 8, "chain", "bf16", True), (128, 16, "chain", "bf16", False), (128, 37, "tree", "bf16", True),
    (128, 64, "tree", "bf16", False), (128, 64, "chain", "bf16", True), (64, 20, "tree", "bf16", False),
    (32, 9, "chain", "f32", False), (16, 4, "chain", "f32", True), (16, 50, "tree", "bf16", False),
    (128, 64, "tree", "f32", True), (128, 30, "chain", "f32", False),
]


@pytest.mark.parametrize("D,T,topology,qkv,in_place", CASES, ids=lambda v: str(v))
def test_commit_grid(ldv, orc, D, T, topology, qkv, in_place):
    wl = WORKLOADS["tree64"].replace(B=6, H=3, D=D, T=T, topology=topology, qkv=qkv,
                                     accept="uniform-node", seed=2000 + D + T)
    x = make_inputs(wl)
    acc = np.array([T - 1, -1, 0, T // 2, -1, T - 1], dtype=np.int32)
    chain = topology == "chain"
    S, st = verify_then_commit(ldv, x, qkv, chain, acc, in_place)
    assert st == 0
    ref, s = orc.commit(x["k"], x["v"], x["a"], x["beta"], x["S0"], acc, None if chain else x["parent"])
    assert s == 0
    check("commit D%d T%d %s" % (D, T, topology), S, ref, slices=(0, 1))
    # accepted = -1: the committed state, bit for bit
    g = S.cpu().numpy()
    for b in np.nonzero(acc < 0)[0]:
        assert np.array_equal(g[b], x["S0"][b])


@pytest.mark.parametrize("key", list(WORKLOADS))
def test_commit_workload_full_size(ldv, orc, key):
    wl = WORKLOADS[key]
    x = make_inputs(wl, with_gather=False)
    chain = wl.topology == "chain"
    S, st = verify_then_commit(ldv, x, wl.qkv, chain, x["accepted"], in_place=True)
    assert st == 0
    ref, s = orc.commit(x["k"], x["v"], x["a"], x["beta"], x["S0"], x["accepted"], None if chain else x["parent"])
    assert s == 0
    check(key + " commit", S, ref, slices=(0, 1))
    g = S.cpu().numpy()
    for b in np.nonzero(x["accepted"] < 0)[0]:
        assert np.array_equal(g[b], x["S0"][b])


def test_commit_selects_the_accepted_node(ldv, orc):
    """Committing node j gives, among all node states of the walk, the one
    closest to the oracle's S_j (the selection is right, not just close)."""
    wl = WORKLOADS["tree64"].replace(B=1, H=2, T=12, D=16, seed=94)
    x = make_inputs(wl)
    _, _, states, _ = orc.verify(x["q"], x["k"], x["v"], x["a"], x["beta"], x["S0"], x["parent"],
                                 want_states=True, want_u=True)
    for j in range(12):
        S, st = verify_then_commit(ldv, x, "bf16", False, np.array([j], np.int32), in_place=False)
        assert st == 0
        g = host(S)[0]
        dist = [np.max(np.abs(g - states[0, i])) for i in range(12)]
        assert int(np.argmin(dist)) == j


def test_bad_accepted(ldv):
    wl = WORKLOADS["tree64"].replace(B=3, H=2, T=10, seed=95)
    x = make_inputs(wl)
    acc = np.array([3, 10, -2], np.int32)
    S, st = verify_then_commit(ldv, x, "bf16", False, acc, in_place=False)
    assert st == ldv.STATUS_BAD_ACCEPTED
    g = S.cpu().numpy()
    assert np.all(g[1] == 3.0) and np.all(g[2] == 3.0) and not np.all(g[0] == 3.0)


def test_bad_parent_on_commit(ldv):
    wl = WORKLOADS["tree64"].replace(B=2, H=2, T=10, seed=96)
    x = make_inputs(wl)
    d = to_device(x, "bf16")
    o, u, lp = ldv.verify_tree(d["q"], d["k"], d["v"], d["a"], d["beta"], d["S0"], d["parent"])
    bad = d["parent"].clone()
    bad[0, 5] = 9
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.full_like(d["S0"], 3.0)
    ldv.commit_state(d["k"], u, lp, dev(np.array([4, 4], np.int32)), d["S0"], S_out=out, parent=bad, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == ldv.STATUS_BAD_PARENT
    assert torch.all(out[0] == 3.0) and not torch.all(out[1] == 3.0)


def test_in_place_equals_out_of_place(ldv):
    wl = WORKLOADS["batch256-tree-commit"].replace(B=8, seed=97)
    x = make_inputs(wl)
    S1, _ = verify_then_commit(ldv, x, "bf16", False, x["accepted"], in_place=False)
    S2, _ = verify_then_commit(ldv, x, "bf16", False, x["accepted"], in_place=True)
    assert torch.equal(S1, S2)
