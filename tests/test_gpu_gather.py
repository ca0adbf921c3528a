"""HIP state gather and read against the fp64 oracle."""
import numpy as np
import pytest

from gpu_util import check, dev, qkv_torch_dtype
from workloads import WORKLOADS, l2_normalise_f32, make_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ldv():
    import speculative_decoding_verify_amd as m
    return m


def case(seed, num_slots, H, D, B, P, Qn, qkv):
    rng = np.random.default_rng(seed)
    pool = (rng.standard_normal((num_slots, H, D, D)) * 0.05).astype(np.float32)
    slot = rng.integers(0, num_slots, size=(B, P)).astype(np.int32)
    qs = l2_normalise_f32(rng.standard_normal((B, P, H, Qn, D)).astype(np.float32))
    if qkv == "bf16":
        from workloads import bf16_round
        qs = bf16_round(qs)
    return pool, slot, qs


GRID = [(128, 16, "bf16"), (128, 20, "bf16"), (128, 1, "f32"), (64, 16, "bf16"), (32, 7, "f32"),
        (16, 16, "bf16"), (16, 33, "f32")]


@pytest.mark.parametrize("D,Qn,qkv", GRID, ids=lambda v: str(v))
def test_gather_grid(ldv, orc, D, Qn, qkv):
    pool, slot, qs = case(3000 + D + Qn, 9, 3, D, 4, 3, Qn, qkv)
    slot[1, 2] = slot[0, 0]  # a duplicate slot
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    o, S = ldv.gather_states(dev(pool), dev(slot), dev(qs, qkv_torch_dtype(qkv)), want_states=True, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    ro, rs, s = orc.gather(pool, slot, qs)
    assert s == 0
    assert np.array_equal(S.cpu().numpy(), rs)
    check("gather D%d Qn%d %s" % (D, Qn, qkv), o, ro, slices=(0, 1, 2))


def test_gather_copy_only_and_read_only(ldv, orc):
    pool, slot, qs = case(3100, 6, 2, 128, 3, 2, 16, "bf16")
    _, S = ldv.gather_states(dev(pool), dev(slot), None, want_states=True)
    o, S2 = ldv.gather_states(dev(pool), dev(slot), dev(qs, torch.bfloat16), want_states=False)
    torch.cuda.synchronize()
    ro, rs, _ = orc.gather(pool, slot, qs)
    assert S2 is None
    assert np.array_equal(S.cpu().numpy(), rs)
    check("gather read-only", o, ro)


def test_gather_bad_slot(ldv):
    pool, slot, qs = case(3200, 5, 2, 64, 2, 3, 4, "bf16")
    slot[0, 1] = 5
    slot[1, 2] = -1
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    o = torch.full((2, 3, 2, 4, 64), 9.0, device="cuda")
    S = torch.full((2, 3, 2, 64, 64), 9.0, device="cuda")
    ldv.gather_states(dev(pool), dev(slot), dev(qs, torch.bfloat16), o=o, states_out=S, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == ldv.STATUS_BAD_SLOT
    assert torch.all(o[0, 1] == 9.0) and torch.all(S[1, 2] == 9.0)
    assert np.array_equal(S[0, 0].cpu().numpy(), pool[slot[0, 0]])


def test_gather_workload_full_size(ldv, orc):
    """The 27B-hybrid-shaped read: 64 sequences x 4 positions x 32 heads of a
    1024-slot pool, 16 queries each; every output checked."""
    wl = WORKLOADS["hybrid27b-chain-gather"]
    x = make_inputs(wl)
    pool = dev(x["pool"])
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    o, S = ldv.gather_states(pool, dev(x["slot"]), dev(x["queries"], torch.bfloat16), want_states=True, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    ro, rs, s = orc.gather(x["pool"], x["slot"], x["queries"])
    assert s == 0
    assert np.array_equal(S.cpu().numpy(), rs)
    check("hybrid27b gather o", o, ro, slices=(0, 1, 2))
