"""The fp64 oracle against what the pages and the mathematics fix (CPU only)."""
import numpy as np
import pytest

import pins
from workloads import make_tree, tree_depths


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


@pytest.mark.parametrize("topology,dk,dv", [("tree", 16, 16), ("chain", 8, 12), ("tree", 12, 7)])
def test_closed_form_shapes(orc, topology, dk, dv):
    pins.pin_closed_form(orc, seed=31, B=2, T=17, H=2, dk=dk, dv=dv, topology=topology)


def test_correction_operator_is_nilpotent():
    """G is strictly lower in topological order, so G^D = 0 with D the maximum
    depth in nodes, and sum_{m<D} (-G)^m is the exact inverse of (I + G)
    (Bole page, section IV, Eq. (7): the Neumann sum for the correction)."""
    for seed in range(6):
        c = pins.random_case(100 + seed, 1, 30, 1, 8, 8, "tree", max_depth=6)
        _, _, _, G = pins.closed_form_head(c["q"][0, :, 0], c["k"][0, :, 0], c["v"][0, :, 0],
                                           c["a"][0, :, 0], c["beta"][0, :, 0], c["S0"][0, 0],
                                           c["parent"][0])
        D = int(tree_depths(c["parent"][0]).max())
        assert np.all(np.tril(G, -1) == G)
        assert np.count_nonzero(np.linalg.matrix_power(G, D)) == 0
        neu = sum(np.linalg.matrix_power(-G, m) for m in range(D))
        assert np.max(np.abs((np.eye(30) + G) @ neu - np.eye(30))) <= 1e-13


def test_bad_parent_reported_and_sequence_untouched(orc):
    c = pins.random_case(41, 3, 6, 2, 8, 8, "tree")
    c["parent"][1, 4] = 4          # not an earlier node
    o, _, status = orc.verify(**c)
    assert status == 1
    assert np.all(o[1] == 0) and np.any(o[0] != 0) and np.any(o[2] != 0)
    c["parent"][1, 4] = -2
    assert orc.verify(**c)[2] == 1


def test_bad_accepted_reported(orc):
    c = pins.random_case(42, 3, 6, 2, 8, 8, "tree")
    acc = np.array([5, 6, -2], dtype=np.int32)
    S, status = orc.commit(c["k"], c["v"], c["a"], c["beta"], c["S0"], acc, c["parent"])
    assert status == 2
    assert np.any(S[0] != 0) and np.all(S[1] == 0) and np.all(S[2] == 0)


def test_accepted_minus_one_is_committed_state(orc):
    c = pins.random_case(43, 2, 5, 2, 8, 8, "chain")
    S, status = orc.commit(c["k"], c["v"], c["a"], c["beta"], c["S0"], np.array([-1, -1], np.int32))
    assert status == 0
    assert np.array_equal(S, c["S0"].astype(np.float64))


def test_bad_slot_reported(orc):
    pool = np.ones((4, 2, 16, 16), np.float32)
    slot = np.array([[0, 4], [-1, 3]], np.int32)
    _, st, status = orc.gather(pool, slot, None)
    assert status == 4
    assert np.all(st[0, 0] == 1) and np.all(st[0, 1] == 0) and np.all(st[1, 0] == 0)


def test_forest_roots(orc):
    """Several roots (parent -1) each start from the committed state."""
    c = pins.random_case(44, 1, 6, 1, 8, 8, "tree")
    c["parent"][0] = np.array([-1, 0, -1, 2, -1, 1], np.int32)
    pins.pin_closed_form  # same route as below
    o, _, status = orc.verify(**c)
    assert status == 0
    O, _, _, _ = pins.closed_form_head(c["q"][0, :, 0], c["k"][0, :, 0], c["v"][0, :, 0], c["a"][0, :, 0],
                                       c["beta"][0, :, 0], c["S0"][0, 0], c["parent"][0])
    assert pins.rel_err(o[0, :, 0], O) <= 1e-10


def test_read_bad_position_reported_and_skipped(orc):
    c = pins.random_case(45, 2, 6, 2, 8, 8, "tree")
    pos = np.array([[0, 6, -1], [-2, 5, 2]], np.int32)
    qs = np.ones((2, 3, 2, 2, 8), np.float32)
    o, status = orc.read_states(c["k"], c["v"], c["a"], c["beta"], c["S0"], pos, qs, c["parent"])
    assert status == 8
    assert np.all(o[0, 1] == 0) and np.all(o[1, 0] == 0)
    assert np.any(o[0, 0] != 0) and np.any(o[0, 2] != 0) and np.any(o[1, 1] != 0)


def test_read_parent_checked_only_for_node_positions(orc):
    c = pins.random_case(46, 2, 6, 2, 8, 8, "tree")
    c["parent"][:, 3] = 5                      # invalid in both sequences
    pos = np.array([[-1, -1], [-1, 2]], np.int32)
    qs = np.ones((2, 2, 2, 1, 8), np.float32)
    o, status = orc.read_states(c["k"], c["v"], c["a"], c["beta"], c["S0"], pos, qs, c["parent"])
    assert status == 1
    want = np.einsum("hij,j->hi", c["S0"][0].astype(np.float64), np.ones(8))
    assert np.array_equal(o[0, 0, :, 0], want) and np.array_equal(o[0, 1, :, 0], want)
    assert np.all(o[1] == 0)                   # the whole sequence is skipped


def test_select_bad_parent_leaves_sequence_untouched(orc):
    rng = np.random.default_rng(47)
    logits = rng.standard_normal((3, 5, 9)).astype(np.float32)
    tokens = rng.integers(0, 9, size=(3, 4)).astype(np.int32)
    par = np.tile(np.array([-1, 0, 1, 2], np.int32), (3, 1))
    par[1, 2] = 2
    target, acc, alen, bonus, status = orc.select(logits, tokens, par)
    assert status == 1
    assert np.array_equal(target, np.argmax(logits, axis=-1))
    assert acc[1] == -2 and alen[1] == -2 and bonus[1] == -2
    assert acc[0] >= -1 and acc[2] >= -1
