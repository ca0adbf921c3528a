"""Grids that are not a whole number of XCD units: the block-to-XCD map spreads
groups of eight units and keeps the blocks past the last whole group (and
any part of a unit) in order.  Verify, commit, the in-block read and the
gather on head and position counts that leave such tails, against the
oracle."""
import numpy as np
import pytest

from gpu_util import check, dev, host, to_device
from workloads import WORKLOADS, make_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ldv():
    import speculative_decoding_verify_amd as m
    return m


@pytest.mark.parametrize("B,H,T,topology", [(7, 11, 12, "tree"), (5, 13, 24, "chain"), (9, 7, 40, "tree"),
                                            (3, 37, 5, "chain")], ids=lambda v: str(v))
def test_odd_grids(ldv, orc, B, H, T, topology):
    wl = WORKLOADS["tree64"].replace(B=B, H=H, D=128, T=T, topology=topology, qkv="bf16",
                                     accept="uniform-node", seed=9500 + B * H + T)
    x = make_inputs(wl, with_gather=False)
    chain = topology == "chain"
    par_h = None if chain else x["parent"]
    print("odd grid B%d H%d T%d %s" % (B, H, T, topology), flush=True)
    d = to_device(x, "bf16")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    if chain:
        o, u, lp = ldv.verify_chain(d["q"], d["k"], d["v"], d["a"], d["beta"], d["S0"], status=st)
    else:
        o, u, lp = ldv.verify_tree(d["q"], d["k"], d["v"], d["a"], d["beta"], d["S0"], d["parent"], status=st)
    dpar = None if chain else d["parent"]
    S = ldv.commit_state(d["k"], u, lp, d["accepted"], d["S0"], parent=dpar, status=st)
    rng = np.random.default_rng(B * 100 + H)
    P, Qn = 3, 5
    pos = rng.integers(-1, T, size=(B, P)).astype(np.int32)
    qs = rng.standard_normal((B, P, H, Qn, 128)).astype(np.float32)
    qs = (qs / np.linalg.norm(qs, axis=-1, keepdims=True)).astype(np.float32)
    qb = dev(qs, torch.bfloat16)
    qs = qb.float().cpu().numpy()  # the values the GPU reads
    ro = ldv.read_block_states(d["k"], u, lp, d["S0"], dev(pos), qb, parent=dpar, status=st)
    # a gather over a pool built from the inputs' states, odd slot and position counts
    pool = np.ascontiguousarray(x["S0"][rng.permutation(B)][: max(1, B - 2)])
    slot = rng.integers(0, pool.shape[0], size=(B, P)).astype(np.int32)
    go, gs = ldv.gather_states(dev(pool), dev(slot), qb, want_states=True, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    ref_o, ref_u, _, s = orc.verify(x["q"], x["k"], x["v"], x["a"], x["beta"], x["S0"], par_h, want_u=True)
    assert s == 0
    check("odd verify o", o, ref_o)
    check("odd verify u", u, ref_u)
    ref_S, s = orc.commit(x["k"], x["v"], x["a"], x["beta"], x["S0"], x["accepted"], par_h)
    assert s == 0
    check("odd commit", S, ref_S)
    ref_r, s = orc.read_states(x["k"], x["v"], x["a"], x["beta"], x["S0"], pos, qs, par_h)
    assert s == 0
    check("odd read", ro, ref_r)
    ref_g, ref_s, s = orc.gather(pool, slot, qs)
    assert s == 0
    check("odd gather o", go, ref_g)
    assert np.array_equal(host(gs).astype(np.float32), ref_s)
