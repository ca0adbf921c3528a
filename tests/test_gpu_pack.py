"""State reads written straight into packed drafter features (gather and
in-block reads): the written columns against the fp64 oracle, every other
element untouched, the plain layout bit-identical to the unpacked o, and
bf16 features equal to the fp32 results rounded to nearest even."""
import numpy as np
import pytest

from gpu_util import check, dev, qkv_torch_dtype
from test_gpu_gather import case as gather_case
from test_gpu_read import case as read_case, gpu_verify

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SENT = 3.25  # exact in bf16 and fp32: marks elements the call must not touch


@pytest.fixture(scope="module")
def ldv():
    import speculative_decoding_verify_amd as m
    return m


def layout(B, P, n, col, tail, rows3d):
    W = col + n + tail
    return ((B, P, W) if rows3d else (B * P, W)), W


def check_packed(name, feat32, featb, ref, B, P, H, Qn, dv, col):
    n = H * Qn * dv
    f = feat32.reshape(B * P, -1)
    fb = featb.reshape(B * P, -1)
    got = f[:, col:col + n].reshape(B, P, H, Qn, dv)
    check(name + " fp32", got, ref)
    # everything outside the written columns keeps its value
    assert torch.all(f[:, :col] == SENT) and torch.all(f[:, col + n:] == SENT)
    assert torch.all(fb[:, :col] == SENT) and torch.all(fb[:, col + n:] == SENT)
    # bf16 features: the same fp32 results, rounded to nearest even
    assert torch.equal(fb[:, col:col + n], f[:, col:col + n].to(torch.bfloat16)), name + " bf16 rounding"


@pytest.mark.parametrize("D,Qn,qkv,col,tail,rows3d", [
    (128, 16, "bf16", 4096, 12, True),   # reads after a block of hidden features
    (128, 5, "f32", 0, 0, False),        # the plain layout
    (64, 20, "bf16", 36, 8, False),
    (16, 3, "bf16", 8, 4, True),
], ids=lambda v: str(v))
def test_gather_packed(ldv, orc, D, Qn, qkv, col, tail, rows3d):
    B, P, H = 4, 3, 3
    pool, slot, qs = gather_case(6000 + D + Qn, 9, H, D, B, P, Qn, qkv)
    q = dev(qs, qkv_torch_dtype(qkv))
    shape, W = layout(B, P, H * Qn * D, col, tail, rows3d)
    f32 = torch.full(shape, SENT, device="cuda")
    fb = torch.full(shape, SENT, device="cuda", dtype=torch.bfloat16)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    ldv.gather_states_packed(dev(pool), dev(slot), q, f32, col=col, status=st)
    ldv.gather_states_packed(dev(pool), dev(slot), q, fb, col=col, status=st)
    o, _ = ldv.gather_states(dev(pool), dev(slot), q)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    ro, _, s = orc.gather(pool, slot, qs)
    assert s == 0
    check_packed("gather packed D%d Qn%d" % (D, Qn), f32, fb, ro, B, P, H, Qn, D, col)
    n = H * Qn * D
    assert torch.equal(f32.reshape(B * P, W)[:, col:col + n].reshape(o.shape), o)  # same kernel, same bits


@pytest.mark.parametrize("D,T,topology,qkv,P,Qn,col,tail", [
    (128, 16, "chain", "bf16", 4, 16, 1024, 4),
    (128, 40, "tree", "bf16", 3, 7, 0, 0),
    (64, 20, "tree", "f32", 2, 9, 12, 20),
    (32, 64, "chain", "bf16", 5, 2, 4, 0),
], ids=lambda v: str(v))
def test_read_packed(ldv, orc, D, T, topology, qkv, P, Qn, col, tail):
    B, H = 3, 2
    c, pos, qs = read_case(6100 + D + T, B, T, H, D, topology, qkv, P, Qn)
    k, u, logp, S0, par = gpu_verify(ldv, c, qkv, topology)
    q = dev(qs, qkv_torch_dtype(qkv))
    shape, W = layout(B, P, H * Qn * D, col, tail, True)
    f32 = torch.full(shape, SENT, device="cuda")
    fb = torch.full(shape, SENT, device="cuda", dtype=torch.bfloat16)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    ldv.read_block_states_packed(k, u, logp, S0, dev(pos), q, f32, col=col, parent=par, status=st)
    ldv.read_block_states_packed(k, u, logp, S0, dev(pos), q, fb, col=col, parent=par, status=st)
    o = ldv.read_block_states(k, u, logp, S0, dev(pos), q, parent=par)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    ref, s = orc.read_states(c["k"], c["v"], c["a"], c["beta"], c["S0"], pos, qs,
                             c["parent"] if topology == "tree" else None)
    assert s == 0
    check_packed("read packed D%d T%d" % (D, T), f32, fb, ref, B, P, H, Qn, D, col)
    n = H * Qn * D
    assert torch.equal(f32.reshape(B * P, W)[:, col:col + n].reshape(o.shape), o)


def test_packed_bad_slot_leaves_rows(ldv):
    """A bad slot: that reading's feature row is left as it was."""
    B, P, H, D, Qn = 2, 2, 2, 64, 4
    pool, slot, qs = gather_case(6200, 5, H, D, B, P, Qn, "bf16")
    slot[1, 0] = 9
    f = torch.full((B, P, 8 + H * Qn * D), SENT, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    ldv.gather_states_packed(dev(pool), dev(slot), dev(qs, torch.bfloat16), f, col=8, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == ldv.STATUS_BAD_SLOT
    assert torch.all(f[1, 0] == SENT) and not torch.any(f[0, 0, 8:] == SENT)


def test_read_staged_large_grid(ldv, orc):
    """A grid of more than 2048 blocks: the in-block read stages its output
    tile in LDS before storing it (plain o and packed features, fp32 and
    bf16); a bad position leaves its row untouched on that path too."""
    B, H, D, T, P, Qn, col = 24, 48, 128, 16, 4, 16, 8   # 24 * 48 heads x 2 value tiles = 2304 blocks
    c, pos, qs = read_case(6300, B, T, H, D, "chain", "bf16", P, Qn)
    k, u, logp, S0, par = gpu_verify(ldv, c, "bf16", "chain")
    q = dev(qs, torch.bfloat16)
    shape, W = layout(B, P, H * Qn * D, col, 4, True)
    f32 = torch.full(shape, SENT, device="cuda")
    fb = torch.full(shape, SENT, device="cuda", dtype=torch.bfloat16)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    ldv.read_block_states_packed(k, u, logp, S0, dev(pos), q, f32, col=col, parent=par, status=st)
    ldv.read_block_states_packed(k, u, logp, S0, dev(pos), q, fb, col=col, parent=par, status=st)
    o = ldv.read_block_states(k, u, logp, S0, dev(pos), q, parent=par, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    ref, s = orc.read_states(c["k"], c["v"], c["a"], c["beta"], c["S0"], pos, qs, None)
    assert s == 0
    check_packed("read staged D%d T%d" % (D, T), f32, fb, ref, B, P, H, Qn, D, col)
    n = H * Qn * D
    assert torch.equal(f32.reshape(B * P, W)[:, col:col + n].reshape(o.shape), o)
    # one bad position: its row keeps the sentinel, every other row is as before
    bad = pos.copy()
    bad[5, 2] = T + 3
    f2 = torch.full(shape, SENT, device="cuda")
    st.zero_()
    ldv.read_block_states_packed(k, u, logp, S0, dev(bad), q, f2, col=col, parent=par, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == ldv.STATUS_BAD_POSITION
    assert torch.all(f2[5, 2] == SENT)
    keep = torch.ones((B, P), dtype=torch.bool, device="cuda")
    keep[5, 2] = False
    assert torch.equal(f2[keep], f32[keep])
