"""HIP verify (chain and tree) against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest

import pins
from gpu_util import DESIGN_TOL, TOL, check, check_logp, dev, host, qkv_torch_dtype, to_device
from workloads import WORKLOADS, bf16_round, make_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ldv():
    import speculative_decoding_verify_amd as m
    return m


def run_verify(ldv, d, chain, status=None):
    if chain:
        return ldv.verify_chain(d["q"], d["k"], d["v"], d["a"], d["beta"], d["S0"], status=status)
    return ldv.verify_tree(d["q"], d["k"], d["v"], d["a"], d["beta"], d["S0"], d["parent"], status=status)


def compare_verify(ldv, orc, x, qkv, chain, name):
    d = to_device(x, qkv)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    o, u, lp = run_verify(ldv, d, chain, st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    ro, ru, _, s = orc.verify(x["q"], x["k"], x["v"], x["a"], x["beta"], x["S0"],
                              None if chain else x["parent"], want_u=True)
    assert s == 0
    check(name + " o", o, ro)
    check(name + " u", u, ru)
    rlp, s = orc.log_decay(x["a"], None if chain else x["parent"])
    assert s == 0
    check_logp(name + " logp", lp, rlp)
    # per (sequence, head) slices, so that a small head cannot hide behind a large one
    go, gu = host(o), host(u)
    for b in range(x["q"].shape[0]):
        for h in range(x["q"].shape[2]):
            assert pins.rel_err(go[b, :, h], ro[b, :, h]) <= DESIGN_TOL
            assert pins.rel_err(gu[b, :, h], ru[b, :, h]) <= DESIGN_TOL
    return o, u, lp


GRID = [
    # D, T, topology, qkv
    (128, 1, "chain", "bf16"), (128, 8, "chain", "bf16"), (128, 16, "chain", "bf16"),
    (128, 17, "tree", "bf16"), (128, 37, "tree", "bf16"), (128, 64, "tree", "bf16"),
    (128, 64, "chain", "bf16"), (128, 20, "tree", "f32"),
    (64, 5, "tree", "bf16"), (64, 33, "tree", "bf16"), (64, 64, "chain", "bf16"),
    (32, 12, "tree", "bf16"), (32, 40, "chain", "f32"), (16, 4, "chain", "f32"), (16, 29, "tree", "bf16"),
    # fp32 q/k/v at every node-block count of d = 128 (hi and lo planes in LDS)
    (128, 9, "chain", "f32"), (128, 33, "tree", "f32"), (128, 64, "tree", "f32"), (64, 64, "chain", "f32"),
]


@pytest.mark.parametrize("D,T,topology,qkv", GRID, ids=lambda v: str(v))
def test_verify_grid(ldv, orc, D, T, topology, qkv):
    wl = WORKLOADS["tree64"].replace(B=3, H=5, D=D, T=T, topology=topology, qkv=qkv,
                                     accept="uniform-node", seed=1000 + D + T)
    x = make_inputs(wl)
    compare_verify(ldv, orc, x, qkv, topology == "chain", "D%d T%d %s %s" % (D, T, topology, qkv))
    if topology == "chain":  # the same chain through the tree entry point
        compare_verify(ldv, orc, x, qkv, False, "D%d T%d chain-as-tree" % (D, T))


@pytest.mark.parametrize("key", list(WORKLOADS))
def test_verify_workload_full_size(ldv, orc, key):
    wl = WORKLOADS[key]
    x = make_inputs(wl, with_gather=False)
    compare_verify(ldv, orc, x, wl.qkv, wl.topology == "chain", key)


def test_golden_fixture_padded(ldv):
    """The hand-worked d = 2 tree, embedded in d = 16 with zero padding (the
    padding rows and columns stay zero through every update)."""
    g, fr = pins.load_golden()
    T, D = len(g["parent"]), 16
    pad = lambda a, shape: np.pad(a, [(0, s - n) for s, n in zip(shape, a.shape)])
    q = pad(fr(g["q"]), (T, D)).reshape(1, T, 1, D).astype(np.float32)
    k = pad(fr(g["k"]), (T, D)).reshape(1, T, 1, D).astype(np.float32)
    v = pad(fr(g["v"]), (T, D)).reshape(1, T, 1, D).astype(np.float32)
    S0 = pad(fr(g["S0"]), (D, D)).reshape(1, 1, D, D).astype(np.float32)
    a = fr(g["a"]).reshape(1, T, 1).astype(np.float32)
    beta = fr(g["beta"]).reshape(1, T, 1).astype(np.float32)
    par = np.array(g["parent"], np.int32).reshape(1, T)
    o, u, lp = ldv.verify_tree(dev(q), dev(k), dev(v), dev(a), dev(beta), dev(S0), dev(par))
    want = np.zeros((T, D))
    want[:, :2] = fr(g["o"])
    check("golden o", host(o)[0, :, 0], want, design_tol=1e-4)
    for n in range(T):
        S = ldv.commit_state(dev(k), u, lp, dev(np.array([n], np.int32)), dev(S0), parent=dev(par))
        wS = np.zeros((D, D))
        wS[:2, :2] = fr(g["states"])[n]
        check("golden S_%d" % n, host(S)[0, 0], wS, design_tol=1e-4)


@pytest.mark.parametrize("case", ["pure-decay", "pure-read", "zero-gate", "overwrite"])
def test_special_cases(ldv, orc, case):
    kw = {"pure-decay": dict(beta=0.0), "pure-read": dict(a=1.0, beta=0.0), "zero-gate": dict(a=0.0),
          "overwrite": dict(beta=1.0)}[case]
    c = pins.random_case(77, 2, 30, 3, 128, 128, "tree", s0_std=0.05, **kw)
    x = {key: c[key] for key in ("q", "k", "v", "a", "beta", "S0", "parent")}
    for key in ("q", "k", "v"):
        x[key] = bf16_round(x[key])
    compare_verify(ldv, orc, x, "bf16", False, case)


def test_forest(ldv, orc):
    wl = WORKLOADS["tree64"].replace(B=2, H=4, T=24, seed=91)
    x = make_inputs(wl)
    x["parent"][0] = np.array([-1, 0, -1, 2, 1, -1] + list(range(5, 23)), np.int32)
    x["parent"][1, 10] = -1
    compare_verify(ldv, orc, x, "bf16", False, "forest")


def test_bad_parent(ldv, orc):
    wl = WORKLOADS["tree64"].replace(B=3, H=2, T=20, seed=92)
    x = make_inputs(wl)
    x["parent"][1, 7] = 7
    d = to_device(x, "bf16")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    o = torch.full((3, 20, 2, 128), 7.0, device="cuda")
    u = torch.full((3, 20, 2, 128), 7.0, device="cuda")
    lp = torch.full((3, 20, 2), 7.0, device="cuda")
    ldv.verify_tree(d["q"], d["k"], d["v"], d["a"], d["beta"], d["S0"], d["parent"], o=o, u=u, logp=lp, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == ldv.STATUS_BAD_PARENT
    assert torch.all(o[1] == 7.0) and torch.all(u[1] == 7.0) and torch.all(lp[1] == 7.0)
    ro, _, s = orc.verify(x["q"], x["k"], x["v"], x["a"], x["beta"], x["S0"], x["parent"])
    assert s == 1
    check("bad-parent others o", host(o)[[0, 2]], ro[[0, 2]])


def test_empty_is_noop(ldv):
    z = torch.zeros(0, device="cuda")
    for B, T, H in [(0, 4, 2), (2, 0, 2), (2, 4, 0)]:
        q = torch.zeros((B, T, H, 128), dtype=torch.bfloat16, device="cuda")
        a = torch.zeros((B, T, H), device="cuda")
        S0 = torch.zeros((B, H, 128, 128), device="cuda")
        par = torch.zeros((B, T), dtype=torch.int32, device="cuda")
        ldv.verify_tree(q, q, q, a, a, S0, par)
        ldv.verify_chain(q, q, q, a, a, S0)
    torch.cuda.synchronize()
    del z


def test_deterministic(ldv):
    wl = WORKLOADS["tree64"].replace(B=4, H=4, seed=93)
    d = to_device(make_inputs(wl), "bf16")
    o1, u1, _ = run_verify(ldv, d, False)
    o2, u2, _ = run_verify(ldv, d, False)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(u1, u2)


def test_unsupported_sizes_raise(ldv):
    q = torch.zeros((1, 65, 1, 128), dtype=torch.bfloat16, device="cuda")
    a = torch.zeros((1, 65, 1), device="cuda")
    S0 = torch.zeros((1, 1, 128, 128), device="cuda")
    with pytest.raises(ldv.LdvError):
        ldv.verify_chain(q, q, q, a, a, S0)
    q = torch.zeros((1, 4, 1, 96), dtype=torch.bfloat16, device="cuda")
    a = torch.zeros((1, 4, 1), device="cuda")
    S0 = torch.zeros((1, 1, 96, 96), device="cuda")
    with pytest.raises(ldv.LdvError):
        ldv.verify_chain(q, q, q, a, a, S0)


@pytest.mark.parametrize("T", [44, 64])
def test_verify_one_round_grid(ldv, orc, T):
    """512 heads at 64 nodes: staged stores on a grid of one round, where the
    waves also lower their issue priority as they advance; with three node
    blocks in use (T = 44) and four (T = 64)."""
    wl = WORKLOADS["tree64"].replace(B=32, H=16, D=128, T=T, seed=4500 + T)
    x = make_inputs(wl, with_gather=False)
    compare_verify(ldv, orc, x, "bf16", False, "one round T%d" % T)


@pytest.mark.parametrize("T,topology,qkv", [(5, "chain", "bf16"), (13, "tree", "bf16"), (16, "tree", "f32"),
                                            (1, "chain", "bf16"), (21, "chain", "bf16"), (29, "tree", "f32"),
                                            (40, "tree", "bf16"), (36, "tree", "f32"), (57, "chain", "bf16"),
                                            (64, "tree", "f32")], ids=lambda v: str(v))
def test_verify_staged_outputs(ldv, orc, T, topology, qkv):
    """On 2048 or more heads the outputs go through LDS and are stored as
    whole rows (16-, 32- and 64-node blocks; at 64 nodes all four node blocks
    at the end, with three or four in use): ragged node counts drop the rows
    past T, and a call without factors writes o alone."""
    wl = WORKLOADS["tree64"].replace(B=32, H=64, D=128, T=T, topology=topology, qkv=qkv,
                                     accept="uniform-node", seed=4400 + T)
    x = make_inputs(wl, with_gather=False)
    chain = topology == "chain"
    compare_verify(ldv, orc, x, qkv, chain, "staged T%d %s %s" % (T, topology, qkv))
    d = to_device(x, qkv)
    if chain:
        o, u, lp = ldv.verify_chain(d["q"], d["k"], d["v"], d["a"], d["beta"], d["S0"], factors=False)
    else:
        o, u, lp = ldv.verify_tree(d["q"], d["k"], d["v"], d["a"], d["beta"], d["S0"], d["parent"], factors=False)
    torch.cuda.synchronize()
    assert u is None and lp is None
    ro, _, s = orc.verify(x["q"], x["k"], x["v"], x["a"], x["beta"], x["S0"], None if chain else x["parent"])
    assert s == 0
    check("staged T%d no factors o" % T, o, ro)
