"""HIP greedy accepted-node selection against the oracle: every output is an
index, so every comparison is exact."""
import json
import os

import numpy as np
import pytest

from gpu_util import dev
from workloads import (WORKLOADS, bf16_round, make_chain, make_inputs, make_select_inputs, make_tree)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module")
def ldv():
    import speculative_decoding_verify_amd as m
    return m


def run(ldv, logits, tokens, parent, dtype, split=True):
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    lg = dev(logits).to(torch.bfloat16 if dtype == "bf16" else torch.float32)
    out = ldv.select_accepted(lg, dev(tokens), None if parent is None else dev(parent), status=st, split=split)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in out], int(st.item())


def compare(orc, ldv, logits, tokens, parent, dtype, name, split=True):
    (tg, acc, alen, bonus), st = run(ldv, logits, tokens, parent, dtype, split)
    rt, racc, ralen, rbonus, rs = orc.select(logits, tokens, parent)
    assert st == rs == 0
    assert np.array_equal(tg, rt), name + ": target"
    assert np.array_equal(acc, racc), name + ": accepted"
    assert np.array_equal(alen, ralen), name + ": accepted_len"
    assert np.array_equal(bonus, rbonus), name + ": bonus"
    print("%-32s accepted len mean %.2f" % (name, float(np.mean(alen))), flush=True)


def test_select_golden(ldv, orc):
    with open(os.path.join(GOLDEN, "select_forest6_handworked.json")) as f:
        g = json.load(f)
    logits = np.array([[float(x) for x in row] for row in g["logits"]], dtype=np.float32)[None]
    tokens = np.array([g["tokens"]], dtype=np.int32)
    par = np.array([g["parent"]], dtype=np.int32)
    for dt in ("f32", "bf16"):   # every value of the example is exact in bf16
        (tg, acc, alen, bonus), st = run(ldv, logits, tokens, par, dt)
        assert st == 0
        assert tg[0].tolist() == g["target"]
        assert (int(acc[0]), int(alen[0]), int(bonus[0])) == (g["accepted"], g["accepted_len"], g["bonus"])


GRID = [  # B, T, V, dtype, topology, value kind
    (5, 12, 4, "f32", "tree", "ties"),
    (6, 12, 5, "bf16", "tree", "ties"),
    (7, 64, 1000, "bf16", "tree", "normal"),
    (3, 64, 37, "bf16", "chain", "ties"),        # odd V: rows start off a 16-byte boundary
    (3, 9, 1, "f32", "chain", "normal"),         # V = 1
    (4, 30, 50003, "f32", "tree", "normal"),
    (2, 16, 151936, "bf16", "chain", "normal"),
    (5, 20, 777, "f32", "tree", "specials"),      # NaN, +-inf, signed zeros
]


@pytest.mark.parametrize("B,T,V,dtype,topology,kind", GRID, ids=lambda v: str(v))
def test_select_grid(ldv, orc, B, T, V, dtype, topology, kind):
    rng = np.random.default_rng(7000 + B * T + V)
    par = make_chain(B, T) if topology == "chain" else make_tree(rng, B, T, 6, 3)
    tokens = rng.integers(0, V, size=(B, T)).astype(np.int32)
    if kind == "ties":
        logits = rng.integers(-2, 3, size=(B, T + 1, V)).astype(np.float32)
    else:
        logits = rng.standard_normal((B, T + 1, V)).astype(np.float32)
    if kind == "specials":
        m = rng.random(logits.shape)
        logits[m < 0.05] = np.nan
        logits[(m >= 0.05) & (m < 0.07)] = -np.inf
        logits[(m >= 0.07) & (m < 0.08)] = np.inf
        logits[(m >= 0.08) & (m < 0.1)] = -0.0
        logits[0, 1] = np.nan               # a row of NaN
        logits[1, 0] = -np.inf              # a row of -inf
    # agree with a random root path so that walks go deep
    for b in range(B):
        n = int(rng.integers(0, T))
        path = []
        while n >= 0:
            path.append(n)
            n = int(par[b, n])
        for n in path:
            if kind != "ties" or rng.random() < 0.7:
                logits[b, int(par[b, n]) + 1, tokens[b, n]] = 9.0
    if dtype == "bf16":  # (special values only appear with fp32 logits)
        logits = bf16_round(logits)
    compare(orc, ldv, logits, tokens, par if topology == "tree" else None, dtype,
            "select B%d T%d V%d %s %s %s" % (B, T, V, dtype, topology, kind))
    if topology == "chain":  # an explicit chain parent row gives the same result
        compare(orc, ldv, logits, tokens, par, dtype, "select explicit chain")


@pytest.mark.parametrize("key", ["hybrid27b-chain-gather", "tree64", "gdn1.3b-chain", "batch256-tree-commit"])
def test_select_workload_full_size(ldv, orc, key):
    wl = WORKLOADS[key]
    x = make_inputs(wl, with_gather=False)
    s = make_select_inputs(wl, x["parent"], x["accepted"])
    for split in (True, False):
        compare(orc, ldv, s["logits"], s["tokens"], x["parent"] if wl.topology == "tree" else None, wl.qkv,
                "select %s split=%s" % (key, split), split=split)


SPLIT = [  # B, T, V, dtype, value kind
    (2, 64, 151936, "bf16", "ties"),     # 130 rows in 4 parts each; the walk also combines row 64
    (16, 8, 100003, "bf16", "normal"),   # 144 rows in 3 parts; odd V
    (3, 5, 70000, "f32", "ties"),        # 2 parts; equal maxima in both
    (2, 7, 65579, "f32", "specials"),    # 2 parts; odd V puts rows off 16-byte boundaries
    (1, 3, 98339, "bf16", "ties"),       # 3 parts, the last one shorter
]


@pytest.mark.parametrize("B,T,V,dtype,kind", SPLIT, ids=lambda v: str(v))
def test_select_split_rows(ldv, orc, B, T, V, dtype, kind):
    """Few long rows split over several workgroups (through the workspace)
    give the oracle's result, and the same as one workgroup per row: equal
    maxima in different parts go to the lower index, NaN never wins."""
    assert ldv.select_workspace_bytes(B, T, V) > 0  # the split path runs
    rng = np.random.default_rng(7200 + B * T + V)
    par = make_tree(rng, B, T, 6, 3)
    tokens = rng.integers(0, V, size=(B, T)).astype(np.int32)
    if kind == "ties":
        logits = rng.integers(-2, 3, size=(B, T + 1, V)).astype(np.float32)
    else:
        logits = rng.standard_normal((B, T + 1, V)).astype(np.float32)
    for b in range(B):  # agree along a path so that walks go deep
        n = int(rng.integers(0, T))
        while n >= 0:
            logits[b, int(par[b, n]) + 1, tokens[b, n]] = 9.0
            n = int(par[b, n])
    if kind == "specials":  # (after the path: these rows stay as set here)
        m = rng.random(logits.shape)
        logits[m < 0.05] = np.nan
        logits[(m >= 0.05) & (m < 0.07)] = -np.inf
        logits[(m >= 0.08) & (m < 0.1)] = -0.0
        logits[0, 1] = np.nan                        # a row of NaN
        logits[0, 2] = -np.inf                       # a row of -inf
        logits[0, 3] = -np.inf
        logits[0, 3, V - 5:] = np.nan                # -inf, then NaN in the last part only
        logits[1, 0, :] = -1.0
        logits[1, 0, [V // 2 - 10, V - 1]] = 7.0    # one maximum in each of the two parts
    if dtype == "bf16":
        logits = bf16_round(logits)
    compare(orc, ldv, logits, tokens, par, dtype, "select split B%d T%d V%d %s" % (B, T, V, kind))
    compare(orc, ldv, logits, tokens, par, dtype, "select unsplit B%d T%d V%d %s" % (B, T, V, kind), split=False)


def test_select_bad_parent(ldv, orc):
    rng = np.random.default_rng(7100)
    logits = rng.standard_normal((3, 6, 50)).astype(np.float32)
    tokens = np.argmax(logits[:, :5], axis=-1).astype(np.int32)
    par = make_chain(3, 5)
    par[1, 3] = 3
    (tg, acc, alen, bonus), st = run(ldv, logits, tokens, par, "f32")
    assert st == ldv.STATUS_BAD_PARENT
    assert np.array_equal(tg, np.argmax(logits, axis=-1))
    rt, racc, _, _, rs = orc.select(logits, tokens, par)
    assert rs == 1 and acc[0] == racc[0] == 4 and acc[2] == racc[2] == 4


def test_select_then_commit(ldv, orc):
    """Selection feeds commit on the device: the committed state is the
    oracle's walk state at the oracle's selected node."""
    wl = WORKLOADS["tree64"].replace(B=6, H=4, V=3000, seed=31)
    x = make_inputs(wl, with_gather=False)
    s = make_select_inputs(wl, x["parent"], x["accepted"])
    q, k, v = (dev(x[n]).to(torch.bfloat16) for n in ("q", "k", "v"))
    a, beta, S0, par = dev(x["a"]), dev(x["beta"]), dev(x["S0"]), dev(x["parent"])
    _, u, logp = ldv.verify_tree(q, k, v, a, beta, S0, par)
    _, acc, _, _ = ldv.select_accepted(dev(s["logits"]).to(torch.bfloat16), dev(s["tokens"]), par)
    S = ldv.commit_state(k, u, logp, acc, S0, parent=par)
    torch.cuda.synchronize()
    _, racc, _, _, _ = orc.select(s["logits"], s["tokens"], x["parent"])
    assert np.array_equal(acc.cpu().numpy(), racc)
    ref, st = orc.commit(x["k"], x["v"], x["a"], x["beta"], x["S0"], racc, x["parent"])
    assert st == 0
    from gpu_util import check
    check("select -> commit", S, ref)


def _special_rows(rng, R, V):
    """fp32 rows (uint32 bit patterns) for the edge cases of the argmax rule,
    eight kinds in turn; rows are long enough that every thread of a row
    visits several chunks."""
    x = rng.standard_normal((R, V)).astype(np.float32)
    snan_rows = []
    for r in range(R):
        k = r % 8
        if k == 0:  # NaN, +-inf and -0 scattered: the first +inf wins
            m = rng.random(V)
            x[r, m < 0.05] = np.nan
            x[r, (m >= 0.05) & (m < 0.06)] = -np.inf
            x[r, (m >= 0.06) & (m < 0.0603)] = np.inf
            x[r, (m >= 0.0603) & (m < 0.08)] = -0.0
        elif k == 1:  # NaN, then -inf everywhere: the first -inf
            x[r] = -np.inf
            x[r, :10] = np.nan
        elif k == 2:  # all NaN: 0
            x[r] = np.nan
        elif k == 3:  # one maximum at two places far apart, NaN before the first
            p1, p2 = sorted(int(i) for i in rng.choice(V, 2, replace=False))
            x[r, p1] = x[r, p2] = 50.0
            x[r, :p1:7] = np.nan
        elif k == 4:  # the maximum at the last element
            x[r, V - 1] = 50.0
        elif k == 5:  # the maximum at element 0 and again in the middle
            x[r, 0] = x[r, V // 2] = 50.0
        elif k == 6:  # signalling-NaN patterns around a finite maximum
            x[r, int(rng.integers(0, V))] = 50.0
            snan_rows.append(r)
        else:  # the maximum is zero, -0 first and +0 later
            x[r] = -np.abs(x[r]) - 1.0
            p1, p2 = sorted(int(i) for i in rng.choice(V, 2, replace=False))
            x[r, p1], x[r, p2] = -0.0, 0.0
    return x, snan_rows


@pytest.mark.parametrize("split", [True, False])
@pytest.mark.parametrize("V,dtype", [(50003, "f32"), (151936, "bf16"), (32005, "bf16")])
def test_select_specials_long_rows(ldv, orc, V, dtype, split):
    """Argmax edge cases on rows long enough for full eight-chunk steps:
    NaN (quiet and signalling) never wins, equal values go to the lower
    index across chunks and threads, +0 == -0, rows whose largest value is
    -inf, all-NaN rows; odd V puts every other row off a 16-byte boundary."""
    rng = np.random.default_rng(7100 + V)
    B, T = 2, 7
    x, snan_rows = _special_rows(rng, B * (T + 1), V)
    if dtype == "f32":
        bits = x.view(np.uint32).copy()
        for r in snan_rows:
            idx = rng.choice(V, 200, replace=False)
            bits[r, idx[:100]] = 0x7F800001
            bits[r, idx[100:]] = 0xFF800001
        ref = bits.view(np.float32)
        lg = torch.from_numpy(ref.reshape(B, T + 1, V).copy()).cuda()
    else:
        u = x.view(np.uint32)
        nan = np.isnan(x)
        # round to nearest even on the top 16 bits; NaN kept quiet
        b16 = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
        b16[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
        for r in snan_rows:
            idx = rng.choice(V, 200, replace=False)
            b16[r, idx[:100]] = 0x7F81
            b16[r, idx[100:]] = 0xFF81
        ref = (b16.astype(np.uint32) << 16).view(np.float32)
        lg = torch.from_numpy(b16.view(np.int16).reshape(B, T + 1, V).copy()).cuda().view(torch.bfloat16)
    ref = ref.reshape(B, T + 1, V)
    tokens = rng.integers(0, V, size=(B, T)).astype(np.int32)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    tg, acc, alen, bonus = (t.cpu().numpy() for t in ldv.select_accepted(lg, dev(tokens), None, status=st,
                                                                          split=split))
    rt, racc, ralen, rbonus, rs = orc.select(ref, tokens, None)
    assert int(st.item()) == rs == 0
    assert np.array_equal(tg, rt), "targets %s vs %s" % (tg.ravel()[:16], rt.ravel()[:16])
    assert np.array_equal(acc, racc) and np.array_equal(alen, ralen) and np.array_equal(bonus, rbonus)
    print("select specials V%d %s targets %s" % (V, dtype, tg.ravel().tolist()), flush=True)


@pytest.mark.parametrize("V,dtype", [(32000, "bf16"), (151936, "bf16"), (1000, "f32")], ids=lambda v: str(v))
def test_select_no_draft_nodes(ldv, orc, V, dtype):
    """T = 0: only the committed position's row is read; nothing is accepted
    (accepted -1, length 0) and the bonus token is that row's argmax, as in
    the oracle.  No token array is needed."""
    rng = np.random.default_rng(7900 + V)
    B = 6
    logits = rng.standard_normal((B, 1, V)).astype(np.float32)
    if dtype == "bf16":
        logits = bf16_round(logits)
    tokens = np.zeros((B, 0), np.int32)
    for split in (True, False):
        compare(orc, ldv, logits, tokens, None, dtype, "T=0 V%d split %s" % (V, split), split=split)
    (tg, acc, alen, bonus), _ = run(ldv, logits, tokens, None, dtype)
    assert np.all(acc == -1) and np.all(alen == 0) and np.array_equal(bonus, tg[:, 0])
