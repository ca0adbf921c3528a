"""HIP reads of in-block states (from the verify factors) against the fp64
oracle's walk to each position."""
import numpy as np
import pytest

import pins
from gpu_util import check, dev, qkv_torch_dtype
from workloads import WORKLOADS, bf16_round, make_block_read_inputs, make_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ldv():
    import speculative_decoding_verify_amd as m
    return m


def case(seed, B, T, H, D, topology, qkv, P, Qn):
    c = pins.random_case(seed, B, T, H, D, D, topology, s0_std=0.05)
    if qkv == "bf16":
        for key in ("q", "k", "v"):
            c[key] = bf16_round(c[key])
    rng = np.random.default_rng(seed + 7)
    pos = rng.integers(-1, T, size=(B, P)).astype(np.int32)
    pos[0, 0] = -1                 # a read of S0 itself
    if P > 1:
        pos[-1, 1] = pos[-1, 0]    # a duplicate position
    qs = rng.standard_normal((B, P, H, Qn, D)).astype(np.float32)
    qs /= np.linalg.norm(qs, axis=-1, keepdims=True).astype(np.float32)
    if qkv == "bf16":
        qs = bf16_round(qs)
    return c, pos, qs.astype(np.float32)


def gpu_verify(ldv, c, qkv, topology):
    dt = qkv_torch_dtype(qkv)
    q, k, v = (dev(c[key], dt) for key in ("q", "k", "v"))
    a, beta, S0 = dev(c["a"]), dev(c["beta"]), dev(c["S0"])
    par = dev(c["parent"]) if topology == "tree" else None
    if par is None:
        _, u, logp = ldv.verify_chain(q, k, v, a, beta, S0)
    else:
        _, u, logp = ldv.verify_tree(q, k, v, a, beta, S0, par)
    return k, u, logp, S0, par


GRID = [  # D, T, topology, qkv, P, Qn
    (128, 16, "chain", "bf16", 4, 16),
    (128, 64, "tree", "bf16", 5, 13),
    (128, 20, "tree", "f32", 3, 7),
    (128, 33, "chain", "bf16", 2, 32),
    (64, 32, "tree", "bf16", 6, 11),
    (64, 7, "chain", "f32", 1, 64),
    (32, 9, "chain", "f32", 2, 5),
    (32, 48, "tree", "bf16", 3, 3),
    (16, 4, "chain", "f32", 3, 2),
    (16, 64, "tree", "bf16", 2, 40),
    (128, 64, "tree", "f32", 3, 9), (128, 40, "chain", "f32", 2, 17),
]


@pytest.mark.parametrize("D,T,topology,qkv,P,Qn", GRID, ids=lambda v: str(v))
def test_read_grid(ldv, orc, D, T, topology, qkv, P, Qn):
    c, pos, qs = case(5000 + D + T + P, 3, T, 2, D, topology, qkv, P, Qn)
    k, u, logp, S0, par = gpu_verify(ldv, c, qkv, topology)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    o = ldv.read_block_states(k, u, logp, S0, dev(pos), dev(qs, qkv_torch_dtype(qkv)), parent=par, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    ref, s = orc.read_states(c["k"], c["v"], c["a"], c["beta"], c["S0"], pos, qs,
                             c["parent"] if topology == "tree" else None)
    assert s == 0
    check("read D%d T%d %s %s P%d Qn%d" % (D, T, topology, qkv, P, Qn), o, ref, slices=(0, 1, 2))


def test_read_matches_commit_then_gather(ldv):
    """A read at node j equals reading the state that commit forms at j."""
    c, pos, qs = case(5100, 4, 24, 2, 128, "tree", "bf16", 1, 16)
    pos[:, 0] = np.array([0, 5, 23, -1], np.int32)
    k, u, logp, S0, par = gpu_verify(ldv, c, "bf16", "tree")
    o = ldv.read_block_states(k, u, logp, S0, dev(pos), dev(qs, torch.bfloat16), parent=par)
    S = ldv.commit_state(k, u, logp, dev(pos[:, 0].copy()), S0, parent=par)
    slot = torch.arange(4, dtype=torch.int32, device="cuda").reshape(4, 1)
    og, _ = ldv.gather_states(S, slot, dev(qs, torch.bfloat16))
    torch.cuda.synchronize()
    check("read vs commit+gather", o, og.double().cpu().numpy())


def test_read_bad_position_and_parent(ldv):
    c, pos, qs = case(5200, 3, 8, 2, 64, "tree", "bf16", 3, 4)
    pos[0] = [0, 8, -1]
    pos[1] = [-2, 3, 3]
    pos[2] = [-1, -1, -1]
    k, u, logp, S0, _ = gpu_verify(ldv, c, "bf16", "tree")
    par = c["parent"].copy()
    par[2, 5] = 6                  # invalid, but sequence 2 reads only S0
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    o = torch.full((3, 3, 2, 4, 64), 7.0, device="cuda")
    ldv.read_block_states(k, u, logp, S0, dev(pos), dev(qs, torch.bfloat16), parent=dev(par), o=o, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == ldv.STATUS_BAD_POSITION
    assert torch.all(o[0, 1] == 7.0) and torch.all(o[1, 0] == 7.0)
    assert not torch.any(o[0, 0] == 7.0) and not torch.any(o[2] == 7.0)
    # sequence 1 reads nodes: with a bad parent row none of it is written
    par[1, 4] = 4
    st.zero_()
    o.fill_(7.0)
    ldv.read_block_states(k, u, logp, S0, dev(pos), dev(qs, torch.bfloat16), parent=dev(par), o=o, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == ldv.STATUS_BAD_POSITION | ldv.STATUS_BAD_PARENT
    assert torch.all(o[1] == 7.0) and not torch.any(o[2] == 7.0) and not torch.any(o[0, 0] == 7.0)


@pytest.mark.parametrize("key", list(WORKLOADS))
def test_read_workload_full_size(ldv, orc, key):
    """Every workload shape at full size (4 in-block positions x 16 queries
    per sequence, 27B-hybrid: its own P and Qn); every output checked
    against the oracle's walk."""
    wl = WORKLOADS[key]
    x = make_inputs(wl, with_gather=False)
    r = make_block_read_inputs(wl)
    dt = torch.bfloat16 if wl.qkv == "bf16" else torch.float32
    q, k, v = (dev(x[n], dt) for n in ("q", "k", "v"))
    a, beta, S0 = dev(x["a"]), dev(x["beta"]), dev(x["S0"])
    par = dev(x["parent"]) if wl.topology == "tree" else None
    if par is None:
        _, u, logp = ldv.verify_chain(q, k, v, a, beta, S0)
    else:
        _, u, logp = ldv.verify_tree(q, k, v, a, beta, S0, par)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    o = ldv.read_block_states(k, u, logp, S0, dev(r["pos"]), dev(r["queries"], dt), parent=par, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    ref, s = orc.read_states(x["k"], x["v"], x["a"], x["beta"], x["S0"], r["pos"], r["queries"],
                             x["parent"] if wl.topology == "tree" else None)
    assert s == 0
    check("read %s full size" % key, o, ref, slices=(0, 1, 2))
