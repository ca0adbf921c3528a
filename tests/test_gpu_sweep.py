"""Every draft length T = 1..64, chains and trees, through verify, commit and
the in-block read, against the oracle: covers each kernel shape (one wave of
16 nodes, 32- and 64-node blocks) and every ragged tail between them."""
import numpy as np
import pytest

import pins
from gpu_util import check, dev, qkv_torch_dtype
from workloads import bf16_round

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ldv():
    import speculative_decoding_verify_amd as m
    return m


@pytest.mark.parametrize("topology", ["chain", "tree"])
@pytest.mark.parametrize("D", [32, 128])
def test_every_length(ldv, orc, topology, D):
    B, H = 2, 2
    worst = {}
    for T in range(1, 65):
        c = pins.random_case(9000 + T + D, B, T, H, D, D, topology, s0_std=0.05, max_depth=8, max_fanout=3)
        for key in ("q", "k", "v"):
            c[key] = bf16_round(c[key])
        q, k, v = (dev(c[key], torch.bfloat16) for key in ("q", "k", "v"))
        a, beta, S0 = dev(c["a"]), dev(c["beta"]), dev(c["S0"])
        par = dev(c["parent"]) if topology == "tree" else None
        st = torch.zeros(1, dtype=torch.int32, device="cuda")
        if par is None:
            o, u, lp = ldv.verify_chain(q, k, v, a, beta, S0, status=st)
        else:
            o, u, lp = ldv.verify_tree(q, k, v, a, beta, S0, par, status=st)
        rng = np.random.default_rng(T)
        acc = rng.integers(-1, T, size=B).astype(np.int32)
        S = ldv.commit_state(k, u, lp, dev(acc), S0, parent=par, status=st)
        pos = rng.integers(-1, T, size=(B, 3)).astype(np.int32)
        qs = bf16_round(rng.standard_normal((B, 3, H, 5, D)).astype(np.float32) / np.sqrt(D))
        ro = ldv.read_block_states(k, u, lp, S0, dev(pos), dev(qs, torch.bfloat16), parent=par, status=st)
        torch.cuda.synchronize()
        assert int(st.item()) == 0, (T, int(st.item()))
        parent = c["parent"] if topology == "tree" else None
        ref_o, ref_st = orc.verify(c["q"], c["k"], c["v"], c["a"], c["beta"], c["S0"], parent)[0::2]
        assert ref_st == 0
        ref_S, s1 = orc.commit(c["k"], c["v"], c["a"], c["beta"], c["S0"], acc, parent)
        ref_r, s2 = orc.read_states(c["k"], c["v"], c["a"], c["beta"], c["S0"], pos, qs, parent)
        assert s1 == 0 and s2 == 0
        worst[T] = (check("T%d verify o" % T, o, ref_o), check("T%d commit" % T, S, ref_S),
                    check("T%d read" % T, ro, ref_r))
    print("%s D%d worst over T=1..64: verify %.2e commit %.2e read %.2e" % (
        topology, D, *(max(w[i] for w in worst.values()) for i in range(3))))
