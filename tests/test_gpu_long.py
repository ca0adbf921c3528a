"""Chains longer than 64 nodes: chunked verify (each chunk from the state at
the end of the previous one) and commit of any node from S0, against the
oracle's sequential decode and path walk."""
import numpy as np
import pytest

import pins
from gpu_util import TOL, check, check_logp, dev, host, qkv_torch_dtype
from workloads import WORKLOADS, bf16_round, make_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ldv():
    import speculative_decoding_verify_amd as m
    return m


def case(seed, B, T, H, D, qkv):
    c = pins.random_case(seed, B, T, H, D, D, "chain", s0_std=0.05)
    if qkv == "bf16":
        for key in ("q", "k", "v"):
            c[key] = bf16_round(c[key])
    return c


def run(ldv, c, qkv):
    dt = qkv_torch_dtype(qkv)
    t = {key: dev(c[key], dt) for key in ("q", "k", "v")}
    a, beta, S0 = dev(c["a"]), dev(c["beta"]), dev(c["S0"])
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    o, u, logp = ldv.verify_chain_long(t["q"], t["k"], t["v"], a, beta, S0, status=st)
    return t, a, beta, S0, o, u, logp, st


GRID = [  # B, T, H, D, qkv (up to 256 heads: one launch for all chunks; more: a launch per chunk)
    (2, 65, 2, 128, "bf16"),
    (2, 100, 3, 128, "bf16"),
    (3, 129, 2, 64, "f32"),
    (2, 200, 2, 32, "bf16"),
    (1, 150, 2, 16, "f32"),
    (2, 80, 2, 128, "f32"),
    (32, 100, 64, 128, "bf16"),   # 2048 heads: both chunks store through LDS
    (16, 130, 32, 128, "f32"),    # 512 heads, fp32 inputs: staged stores, two in-place chunk ends
    (12, 150, 32, 128, "bf16"),   # 384 heads: a launch per chunk, outputs stored straight
    (8, 200, 32, 64, "bf16"),     # 256 heads at d = 64: all four chunks in one launch
    (2, 140, 2, 64, "bf16"),
    (2, 90, 2, 32, "f32"),
    (2, 70, 3, 16, "bf16"),
]


@pytest.mark.parametrize("B,T,H,D,qkv", GRID, ids=lambda v: str(v))
def test_long_chain_verify_and_commit(ldv, orc, B, T, H, D, qkv):
    c = case(8000 + T + D, B, T, H, D, qkv)
    t, a, beta, S0, o, u, logp, st = run(ldv, c, qkv)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    ref = orc.chain_decode(c["q"], c["k"], c["v"], c["a"], c["beta"], c["S0"])
    check("long chain o B%d T%d H%d D%d %s" % (B, T, H, D, qkv), o, ref)
    # log P from S0 along the whole chain
    lp, s = orc.log_decay(c["a"])
    assert s == 0
    check_logp("long chain logp", logp, lp)
    # commit nodes in every chunk, from S0, with the factors of the whole chain
    for n in sorted({0, 63, 64, T // 2, T - 1}):
        acc = np.full(B, n, dtype=np.int32)
        acc[0] = -1 if n == 0 else acc[0]
        S = ldv.commit_state(t["k"], u, logp, dev(acc), S0)
        torch.cuda.synchronize()
        want, s = orc.commit(c["k"], c["v"], c["a"], c["beta"], c["S0"], acc)
        assert s == 0
        check("long chain commit n=%d" % n, S, want, slices=(0, 1))


def test_long_chain_short_is_verify_chain(ldv):
    """Up to 64 nodes the long form is the ordinary chain verify, bit for bit."""
    c = case(8100, 2, 40, 2, 128, "bf16")
    _, _, _, _, o, u, logp, _ = run(ldv, c, "bf16")
    t = {key: dev(c[key], torch.bfloat16) for key in ("q", "k", "v")}
    o2, u2, lp2 = ldv.verify_chain(t["q"], t["k"], t["v"], dev(c["a"]), dev(c["beta"]), dev(c["S0"]))
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(u, u2) and torch.equal(logp, lp2)


def test_long_chain_gdn_shape(ldv, orc):
    """GDN-1.3B-shaped layer (B16 H16 d128) with a 256-token draft block."""
    wl = WORKLOADS["gdn1.3b-chain"].replace(T=256, seed=41)
    x = make_inputs(wl, with_gather=False)
    t = {key: dev(x[key], torch.bfloat16) for key in ("q", "k", "v")}
    o, u, logp = ldv.verify_chain_long(t["q"], t["k"], t["v"], dev(x["a"]), dev(x["beta"]), dev(x["S0"]))
    torch.cuda.synchronize()
    ref = orc.chain_decode(x["q"], x["k"], x["v"], x["a"], x["beta"], x["S0"])
    check("long chain GDN shape T256", o, ref)


@pytest.mark.parametrize("B,H,D,qkv", [(2, 3, 128, "bf16"), (16, 32, 128, "bf16"), (2, 2, 64, "f32"),
                                       (1, 2, 16, "bf16")], ids=lambda v: str(v))
def test_chunk_end_state(ldv, orc, B, H, D, qkv):
    """Each full chunk but the last also forms the state at its last node, the
    next chunk's base; with two chunks that state (node 63) is what the call
    leaves in S_work.  Checked against the oracle's commit of node 63."""
    c = case(8200 + B + D, B, 100, H, D, qkv)
    dt = qkv_torch_dtype(qkv)
    t = {key: dev(c[key], dt) for key in ("q", "k", "v")}
    S0 = dev(c["S0"])
    work = torch.full_like(S0, 7.0)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    ldv.verify_chain_long(t["q"], t["k"], t["v"], dev(c["a"]), dev(c["beta"]), S0, S_work=work, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    want, s = orc.commit(c["k"], c["v"], c["a"], c["beta"], c["S0"], np.full(B, 63, dtype=np.int32))
    assert s == 0
    check("chunk end state B%d H%d D%d %s" % (B, H, D, qkv), work, want)
    assert np.array_equal(host(S0), c["S0"])  # the committed state is only read


@pytest.mark.parametrize("qkv", ["bf16", "f32"])
def test_long_chain_at_the_length_cap(ldv, orc, qkv):
    """The longest chain the library accepts (LDV_MAX_LONG_T = 8192 nodes, 128
    chunks): log P is an fp32 sum counted from S0, and commit's weights
    exp(log P_n - log P_m) lose precision as |log P| grows; at the cap the
    committed state of the last node and of nodes in early, middle and late
    chunks must still meet the bound."""
    T = ldv.MAX_LONG_T
    c = case(8300, 1, T, 2, 16, qkv)
    t, a, beta, S0, o, u, logp, st = run(ldv, c, qkv)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    ref = orc.chain_decode(c["q"], c["k"], c["v"], c["a"], c["beta"], c["S0"])
    check("chain of %d o" % T, o, ref)
    lp, s = orc.log_decay(c["a"])
    assert s == 0
    check_logp("chain of %d logp" % T, logp, lp)
    for n in (100, T // 2 + 7, T - 1):
        acc = np.array([n], np.int32)
        S = ldv.commit_state(t["k"], u, logp, dev(acc), S0)
        torch.cuda.synchronize()
        want, s = orc.commit(c["k"], c["v"], c["a"], c["beta"], c["S0"], acc)
        assert s == 0
        # the error here comes from the fp32 log P sums, not from the state
        # products, so only the bound itself applies
        check("chain of %d commit n=%d" % (T, n), S, want, design_tol=TOL, slices=(0, 1))
    bad = torch.zeros_like(t["q"])
    q2 = torch.cat([t["q"], bad[:, :1]], dim=1).contiguous()
    with pytest.raises(ldv.LdvError):
        a2 = torch.cat([a, a[:, :1]], dim=1).contiguous()
        ldv.verify_chain_long(q2, q2, q2, a2, a2, S0)
