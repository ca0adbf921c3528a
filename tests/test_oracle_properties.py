"""Property-based checks of the fp64 oracle (CPU only): random small trees,
forests and chains, head sizes and gate regimes drawn by hypothesis, each
checked against explicit matrix products of the recurrence and against the
closed form of the Bole page (section IV, Eq. (2)) with a library solve, and
the greedy selection against its set-based restatement.  The fixed-seed pins
in pins.py cover chosen cases; these widen the net over shapes and gates."""
import numpy as np
import pytest

import pins
from workloads import l2_normalise_f32

hyp = pytest.importorskip("hypothesis")
from hypothesis import HealthCheck, given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402

SETTINGS = dict(max_examples=200, deadline=None, suppress_health_check=[HealthCheck.function_scoped_fixture],
                derandomize=True)


def draw_case(seed, T, dk, dv, topology, gates):
    rng = np.random.default_rng(seed)
    B, H = 2, 2
    S0 = (rng.standard_normal((B, H, dv, dk)) * 0.3).astype(np.float32)
    q = l2_normalise_f32(rng.standard_normal((B, T, H, dk)).astype(np.float32))
    k = l2_normalise_f32(rng.standard_normal((B, T, H, dk)).astype(np.float32))
    v = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    a = (1.0 / (1.0 + np.exp(rng.standard_normal((B, T, H))))).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))).astype(np.float32)
    if gates == "a=1":
        a[:] = 1.0
    elif gates == "beta=0":
        beta[:] = 0.0
    elif gates == "beta=1":
        beta[:] = 1.0
    elif gates == "small a":
        a[:] = 1e-3
    par = np.empty((B, T), dtype=np.int32)
    for b in range(B):
        for n in range(T):
            if topology == "chain":
                par[b, n] = n - 1
            elif topology == "forest":
                par[b, n] = int(rng.integers(-1, n))  # any earlier node, or a new root
            else:
                par[b, n] = -1 if n == 0 else int(rng.integers(0, n))
    return dict(q=q, k=k, v=v, a=a, beta=beta, S0=S0, parent=par)


@settings(**SETTINGS)
@given(T=st.integers(1, 14), dk=st.sampled_from([1, 2, 3, 5, 8]), dv=st.sampled_from([1, 2, 4, 7]),
       topology=st.sampled_from(["tree", "forest", "chain"]),
       gates=st.sampled_from(["random", "a=1", "beta=0", "beta=1", "small a"]),
       seed=st.integers(0, 2 ** 31 - 1))
def test_verify_and_commit_against_matrices_and_closed_form(orc, T, dk, dv, topology, gates, seed):
    c = draw_case(seed, T, dk, dv, topology, gates)
    o, u, states, status = orc.verify(c["q"], c["k"], c["v"], c["a"], c["beta"], c["S0"], c["parent"],
                                      want_states=True, want_u=True)
    assert status == 0
    rng = np.random.default_rng(seed + 1)
    acc = rng.integers(-1, T, size=2).astype(np.int32)
    S, status = orc.commit(c["k"], c["v"], c["a"], c["beta"], c["S0"], acc, c["parent"])
    assert status == 0
    for b in range(2):
        for h in range(2):
            args = [c[x][b, :, h] for x in ("k", "v", "a", "beta")]
            Sbf = pins.brute_force_states(*args, c["S0"][b, h], c["parent"][b])
            assert pins.rel_err(states[b, :, h], Sbf) <= 1e-12
            want_o = np.einsum("nij,nj->ni", Sbf, c["q"][b, :, h].astype(np.float64))
            assert pins.rel_err(o[b, :, h], want_o) <= 1e-12
            want_S = c["S0"][b, h].astype(np.float64) if acc[b] < 0 else Sbf[acc[b]]
            assert pins.rel_err(S[b, h], want_S) <= 1e-12
            O, U, _, _ = pins.closed_form_head(c["q"][b, :, h], c["k"][b, :, h], c["v"][b, :, h], c["a"][b, :, h],
                                               c["beta"][b, :, h], c["S0"][b, h], c["parent"][b])
            assert pins.rel_err(o[b, :, h], O) <= 1e-9
            assert pins.rel_err(u[b, :, h], U) <= 1e-9


@settings(**SETTINGS)
@given(T=st.integers(1, 12), V=st.integers(1, 6), topology=st.sampled_from(["tree", "forest", "chain"]),
       nan_share=st.sampled_from([0.0, 0.1, 0.5]), seed=st.integers(0, 2 ** 31 - 1))
def test_selection_against_sets(orc, T, V, topology, nan_share, seed):
    rng = np.random.default_rng(seed)
    c = draw_case(seed, T, 1, 1, topology, "random")
    par = c["parent"]
    tokens = rng.integers(0, V, size=(2, T)).astype(np.int32)
    logits = rng.integers(-2, 3, size=(2, T + 1, V)).astype(np.float32)
    logits[rng.random(logits.shape) < nan_share] = np.nan
    target, acc, alen, bonus, status = orc.select(logits, tokens, par)
    assert status == 0
    for b in range(2):
        want_t = [pins._argmax_by_keys(logits[b, r]) for r in range(T + 1)]
        assert target[b].tolist() == want_t
        n, d = pins._select_by_sets(want_t, tokens[b].tolist(), par[b])
        assert (int(acc[b]), int(alen[b]), int(bonus[b])) == (n, d, want_t[n + 1])
