"""Seeded input generators: determinism and the stated structure (CPU only)."""
import numpy as np

from workloads import WORKLOADS, bf16_round, make_inputs, make_tree, tree_depths


def test_bf16_round_matches_torch():
    torch = __import__("torch")
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 3
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(bf16_round(x), want)


def test_deterministic():
    wl = WORKLOADS["tiny-chain"]
    a, b = make_inputs(wl), make_inputs(wl)
    for key in a:
        assert np.array_equal(a[key], b[key])


def test_tree_structure():
    rng = np.random.default_rng(3)
    par = make_tree(rng, 50, 64)
    for row in par:
        assert row[0] == -1
        assert all(-1 <= row[n] < n for n in range(64))
        assert all(row[n] >= 0 for n in range(1, 64))
        d = tree_depths(row)
        assert d.max() <= 8
        counts = np.bincount(row[1:], minlength=64)
        assert counts.max() <= 4


def test_small_workload_shapes():
    wl = WORKLOADS["gdn1.3b-chain"].replace(B=2, H=3)
    x = make_inputs(wl)
    assert x["q"].shape == (2, 8, 3, 128) and x["S0"].shape == (2, 3, 128, 128)
    assert np.array_equal(bf16_round(x["q"]), x["q"])
    n = np.linalg.norm(x["k"].astype(np.float64), axis=-1)
    assert np.all(np.abs(n - 1) < 1e-2)
    assert np.all((x["a"] > 0) & (x["a"] < 1)) and np.all((x["beta"] > 0) & (x["beta"] < 1))
    assert np.all((x["accepted"] >= -1) & (x["accepted"] < 8))


def test_gather_inputs():
    wl = WORKLOADS["hybrid27b-chain-gather"].replace(B=3, H=2)
    x = make_inputs(wl)
    assert x["pool"].shape == (48, 2, 128, 128)
    for b in range(3):
        s = x["slot"][b]
        assert len(set(s.tolist())) == 4 and np.all((s >= b * 16) & (s < b * 16 + 16))
    assert x["queries"].shape == (3, 4, 2, 16, 128)


def test_block_read_inputs():
    from workloads import WORKLOADS, make_block_read_inputs
    wl = WORKLOADS["hybrid27b-chain-gather"].replace(B=6)
    r = make_block_read_inputs(wl)
    assert r["pos"].shape == (6, 4) and r["queries"].shape == (6, 4, 32, 16, 128)
    for row in r["pos"]:
        assert len(set(row.tolist())) == 4 and row.min() >= 0 and row.max() < wl.T
    r2 = make_block_read_inputs(wl)
    assert np.array_equal(r["pos"], r2["pos"]) and np.array_equal(r["queries"], r2["queries"])


def test_select_inputs_plant_the_drawn_path():
    from workloads import WORKLOADS, make_inputs, make_select_inputs
    wl = WORKLOADS["tree64"].replace(B=4, V=1000)
    x = make_inputs(wl, with_gather=False)
    s = make_select_inputs(wl, x["parent"], x["accepted"])
    assert s["tokens"].shape == (4, 64) and s["logits"].shape == (4, 65, 1000)
    for b in range(4):
        n = int(x["accepted"][b])
        while n >= 0:
            p = int(x["parent"][b, n])
            assert s["logits"][b, p + 1, s["tokens"][b, n]] == 8.0
            n = p
