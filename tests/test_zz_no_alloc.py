"""The selection entry point that allocates nothing (ldv_select_accepted_noalloc:
its split-row partial results in the library's own per-GPU array) against
ldv_select_accepted with a caller workspace: every output equal (they are
indices), on two calls in a row, the second on a smaller input, so that the
array still holds the first call's entries when the second runs."""
import numpy as np
import pytest

from gpu_util import dev
from workloads import WORKLOADS, make_chain, make_inputs, make_select_inputs, make_tree

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ldv():
    import speculative_decoding_verify_amd as m
    return m


def inputs(seed, B, T, V, dtype, topology):
    wl = WORKLOADS["tree64"].replace(B=B, T=T, V=V, seed=seed, accept="uniform-node", qkv=dtype, topology=topology)
    rng = np.random.default_rng(seed)
    parent = make_chain(B, T) if topology == "chain" else make_tree(rng, B, T, 8, 4)
    accepted = rng.integers(-1, T, size=B).astype(np.int32)
    sel = make_select_inputs(wl, parent, accepted)
    lg = dev(sel["logits"]).to(torch.bfloat16 if dtype == "bf16" else torch.float32)
    return lg, dev(sel["tokens"]), (None if topology == "chain" else dev(parent)), sel, parent


def both(ldv, lg, tok, par):
    B, T1, V = lg.shape
    ws = torch.empty(max(1, ldv.select_workspace_bytes(B, T1 - 1, V)), dtype=torch.uint8, device="cuda")
    ref = ldv.select_accepted(lg, tok, par, workspace=ws)
    outs = [torch.full((B, T1), -7, dtype=torch.int32, device="cuda")] + \
           [torch.full((B,), -7, dtype=torch.int32, device="cuda") for _ in range(3)]
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    got = ldv.select_accepted_noalloc(lg, tok, outs[0], outs[1], parent=par, accepted_len=outs[2], bonus=outs[3],
                                      status=st)
    assert torch.cuda.memory_allocated() == before  # the binding allocated nothing either
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    return [r.cpu().numpy() for r in ref], [g.cpu().numpy() for g in got]


# (B, T, V, dtype, topology): each pair is a large call, then a smaller one
PAIRS = [
    ((64, 16, 151936, "bf16", "chain"), (8, 5, 100003, "f32", "tree")),    # 4352, then 144 scratch entries
    ((16, 64, 151936, "f32", "tree"), (16, 8, 32000, "bf16", "chain")),    # 4160, then rows kept whole
    ((100, 12, 70001, "bf16", "tree"), (3, 2, 65536, "bf16", "chain")),   # 2600, then 18 entries; odd V
]


@pytest.mark.parametrize("first,second", PAIRS, ids=lambda v: str(v))
def test_noalloc_matches_workspace_call(ldv, orc, first, second):
    for k, (B, T, V, dtype, topology) in enumerate((first, second)):
        lg, tok, par, sel, parent = inputs(9100 + 10 * k + B, B, T, V, dtype, topology)
        ref, got = both(ldv, lg, tok, par)
        for name, r, g in zip(("target", "accepted", "accepted_len", "bonus"), ref, got):
            assert np.array_equal(r, g), "%s differs at %s" % (name, (B, T, V, dtype, topology))
        if k == 1:  # the smaller call also against the oracle
            rt, racc, ralen, rbonus, rs = orc.select(sel["logits"], sel["tokens"],
                                                     None if topology == "chain" else parent)
            assert rs == 0
            for r, g in zip((rt, racc, ralen, rbonus), got):
                assert np.array_equal(r, g)


def test_noalloc_rows_split_as_with_a_workspace(ldv):
    """The first call of each pair really splits its rows (the library's
    array is used), and the 27B-hybrid shape needs 4352 of its 6144 entries."""
    assert ldv.select_workspace_bytes(64, 16, 151936) == 64 * 17 * 4 * 8
    for first, _ in PAIRS:
        B, T, V = first[:3]
        assert ldv.select_workspace_bytes(B, T, V) > 0
        assert ldv.select_workspace_bytes(B, T, V) // 8 <= 6144


def test_noalloc_on_a_side_stream(ldv):
    """With a stream passed, the array's address is the one on that stream's
    GPU (here a second stream of the current GPU): the results equal those
    of the workspace call."""
    lg, tok, par, sel, parent = inputs(9300, 64, 16, 151936, "bf16", "chain")
    B, T1, V = lg.shape
    ws = torch.empty(ldv.select_workspace_bytes(B, T1 - 1, V), dtype=torch.uint8, device="cuda")
    ref = ldv.select_accepted(lg, tok, par, workspace=ws)
    outs = [torch.full((B, T1), -7, dtype=torch.int32, device="cuda")] + \
           [torch.full((B,), -7, dtype=torch.int32, device="cuda") for _ in range(3)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    got = ldv.select_accepted_noalloc(lg, tok, outs[0], outs[1], parent=par, accepted_len=outs[2], bonus=outs[3],
                                      stream=side)
    side.synchronize()
    torch.cuda.synchronize()
    for name, r, g in zip(("target", "accepted", "accepted_len", "bonus"), ref, got):
        assert torch.equal(r, g), name
