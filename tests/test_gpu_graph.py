"""The whole path captured in one HIP graph and replayed several times, with
eager work and synchronisation between the replays: every replay must give
the eager results (the kernels clear nothing with memsets and keep no state
between calls, so graph replays are exact repeats)."""
import numpy as np
import pytest

from gpu_util import dev
from workloads import WORKLOADS, make_block_read_inputs, make_inputs, make_select_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ldv():
    import speculative_decoding_verify_amd as m
    return m


def test_graph_replays_match_eager(ldv):
    wl = WORKLOADS["tree64"].replace(B=4, H=4, T=40, seed=51, P=3, R=4, Qn=8, V=5000)
    x = make_inputs(wl)
    r = make_block_read_inputs(wl)
    s = make_select_inputs(wl, x["parent"], x["accepted"])
    bf = torch.bfloat16
    q, k, v = (dev(x[n], bf) for n in ("q", "k", "v"))
    a, beta, par = dev(x["a"]), dev(x["beta"]), dev(x["parent"])
    S0_init = dev(x["S0"])
    pool, slot, gq = dev(x["pool"]), dev(x["slot"]), dev(x["queries"], bf)
    pos, rq = dev(r["pos"]), dev(r["queries"], bf)
    logits, tokens = dev(s["logits"], bf), dev(s["tokens"])
    B, T, H, D = wl.B, wl.T, wl.H, wl.D
    S0 = S0_init.clone()
    o = torch.empty((B, T, H, D), device="cuda")
    u, lp = torch.empty_like(o), torch.empty((B, T, H), device="cuda")
    go = torch.empty((B, wl.P, H, wl.Qn, D), device="cuda")
    ro = torch.empty((B, r["pos"].shape[1], H, 8, D), device="cuda")
    tg = torch.empty((B, T + 1), dtype=torch.int32, device="cuda")
    acc = torch.empty((B,), dtype=torch.int32, device="cuda")
    alen, bonus = torch.empty_like(acc), torch.empty_like(acc)
    Sc = torch.empty_like(S0)
    # packed drafter features: the gather's reads after 4 columns of other
    # features, the in-block reads in bf16
    gf = torch.zeros((B, wl.P, 4 + H * wl.Qn * D), device="cuda")  # columns 0..3 are never written
    rf = torch.empty((B, r["pos"].shape[1], H * 8 * D), device="cuda", dtype=torch.bfloat16)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")

    def path():
        ldv.verify_tree(q, k, v, a, beta, S0, par, o=o, u=u, logp=lp, status=st)
        ldv.read_block_states(k, u, lp, S0, pos, rq, parent=par, o=ro, status=st)
        ldv.select_accepted(logits, tokens, par, target=tg, accepted=acc, accepted_len=alen, bonus=bonus, status=st)
        ldv.commit_state(k, u, lp, acc, S0, S_out=Sc, parent=par, status=st)
        ldv.gather_states(pool, slot, gq, o=go, status=st)
        ldv.gather_states_packed(pool, slot, gq, gf, col=4, status=st)
        ldv.read_block_states_packed(k, u, lp, S0, pos, rq, rf, parent=par, status=st)

    outs = (o, u, lp, ro, tg, acc, alen, bonus, Sc, go, gf, rf)
    path()
    torch.cuda.synchronize()
    want = [t.clone() for t in outs]
    assert int(st.item()) == 0
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        path()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        path()
    for rep in range(4):
        for t in outs:
            t.zero_() if t.dtype != torch.int32 else t.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        for i, (t, w) in enumerate(zip(outs, want)):
            assert torch.equal(t, w), (rep, i)
        # eager work between replays
        ldv.verify_tree(q, k, v, a, beta, S0, par, status=st)
        torch.cuda.synchronize()
    assert int(st.item()) == 0
