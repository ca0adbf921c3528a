"""Calls enqueued on a stream other than torch's current one: outputs and
scratch that the binding allocates stay reserved until the call's kernels
are done, even when the current stream allocates right after the call."""
import numpy as np
import pytest

from gpu_util import check, dev
from workloads import WORKLOADS, make_inputs, make_select_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ldv():
    import speculative_decoding_verify_amd as m
    return m


def test_side_stream_scratch_and_outputs(ldv, orc):
    wl = WORKLOADS["gdn1.3b-chain"].replace(T=200, seed=4101)
    x = make_inputs(wl, with_gather=False)
    q, k, v = (dev(x[n], torch.bfloat16) for n in ("q", "k", "v"))
    a, beta, S0 = dev(x["a"]), dev(x["beta"]), dev(x["S0"])
    sel = make_select_inputs(WORKLOADS["hybrid27b-chain-gather"].replace(B=8, seed=4102),
                             np.tile(np.arange(-1, 15, dtype=np.int32), (8, 1)), np.full(8, 5, np.int32))
    logits, tokens = dev(sel["logits"], torch.bfloat16), dev(sel["tokens"])
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())  # the inputs are ready before the side stream reads them
    # the long chain's work state and the selection's workspace are dropped
    # when the calls return; the default stream then allocates and writes
    o, u, lp = ldv.verify_chain_long(q, k, v, a, beta, S0, stream=side)
    tg, acc, alen, bonus = ldv.select_accepted(logits, tokens, stream=side)
    junk = [torch.full((1 << 22,), 7.0, device="cuda") for _ in range(8)]
    torch.cuda.synchronize()
    del junk
    ref = orc.chain_decode(x["q"], x["k"], x["v"], x["a"], x["beta"], x["S0"])
    check("side stream long chain o", o, ref)
    rt, racc, ralen, rbonus, rs = orc.select(sel["logits"], sel["tokens"], None)
    assert rs == 0
    assert np.array_equal(tg.cpu().numpy(), rt) and np.array_equal(acc.cpu().numpy(), racc)
    assert np.array_equal(alen.cpu().numpy(), ralen) and np.array_equal(bonus.cpu().numpy(), rbonus)
