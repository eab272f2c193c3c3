"""Pins of the oracle's gating variants (V1, V2, V3) to values and rules the
pages fix: M6.2 §0x05A, §0x06B-§0x06D, §0x06L3-§0x06L4."""
import numpy as np
import pytest

import oracle as O


def _logit(s):
    s = np.asarray(s, dtype=np.float64)
    return np.log(s / (1.0 - s)).astype(np.float32)


# ---- V3 -----------------------------------------------------------------

def test_v3_page_token_t0(golden):
    f = golden("m62_gating_fixtures.json")["v3_t0"]
    z = _logit(f["affinity"])[None, :]
    # the fp32 affinity of these logits reproduces the tabulated affinities
    assert np.allclose(O.sigmoid_f32(z)[0], f["affinity"], atol=2e-7)
    ids, gates, inv = O.route_v3(z, np.array(f["bias"], np.float32), f["k"], f["n_group"], f["topk_group"],
                                 f["route_scale"])
    assert not inv[0]
    assert ids[0].tolist() == f["experts"]
    assert np.allclose(gates[0], f["gates"], atol=6e-7)
    assert abs(gates[0].sum() - f["gate_sum"]) < 1e-9
    # the groups the corrected scores keep, with and without the bias
    corrected = (O.sigmoid_f32(z) + np.array(f["bias"], np.float32)).astype(np.float32)
    _, g = O.group_limited_select(corrected, f["n_group"], f["topk_group"], f["k"], "top2sum")
    assert g[0].tolist() == f["groups_with_bias"]
    _, g0 = O.group_limited_select(O.sigmoid_f32(z), f["n_group"], f["topk_group"], f["k"], "top2sum")
    assert g0[0].tolist() == f["groups_without_bias"]


def test_v3_gates_use_original_not_corrected_scores(golden):
    f = golden("m62_gating_fixtures.json")["v3_t0"]
    s = np.array(f["affinity"])
    b = np.array(f["bias"])
    sel = f["experts"]
    wrong = f["route_scale"] * (s + b)[sel] / (s + b)[sel].sum()
    assert abs(wrong[3] - f["gate_of_expert1_if_corrected_scores_were_reused"]) < 1e-6
    _, gates, _ = O.route_v3(_logit(s)[None, :], b.astype(np.float32), f["k"], f["n_group"], f["topk_group"],
                             f["route_scale"])
    assert abs(gates[0, 3] - wrong[3]) > 0.4


def test_v3_group_statistic_is_top2_sum(golden):
    f = golden("m62_gating_fixtures.json")["v3_t1"]
    top2, mx, tot = f["group_top2_sum"], f["group_max"], f["group_sum_all"]
    # the unique three values of each group with the tabulated statistics, largest first
    rows = [[mx[g], top2[g] - mx[g], tot[g] - top2[g]] for g in range(4)]
    sc = np.array([sum(rows, [])], dtype=np.float32)
    _, g = O.group_limited_select(sc, f["n_group"], f["topk_group"], f["k"], "top2sum")
    assert sorted(g[0].tolist()) == sorted(f["groups_by_top2_sum"])
    _, gmax = O.group_limited_select(sc, f["n_group"], f["topk_group"], f["k"], "max")
    assert sorted(gmax[0].tolist()) == sorted(f["groups_by_max"])
    # expert 0 holds the global maximum but its group is not kept
    ids, _, _ = O.route_v3(_logit(sc[0])[None, :], None, f["k"], f["n_group"], f["topk_group"], 2.5)
    assert 0 not in ids[0].tolist()
    assert int(np.argmax(sc[0])) == 0


def _nearest_f32(x):
    """The fp32 value nearest to the Decimal ``x`` (ties to the even code),
    found among the neighbours of a first guess by exact comparison."""
    from decimal import Decimal
    guess = np.float32(float(x))
    cands = [np.nextafter(guess, np.float32(-np.inf)), guess, np.nextafter(guess, np.float32(np.inf))]
    def key(c):
        return (abs(Decimal(float(c)) - x), int(np.array(c, np.float32).view(np.uint32)) & 1)
    return min(cands, key=key)


def test_v3_affinity_is_the_nearest_fp32_sigmoid():
    """The V3 decision key rounds the exact sigmoid once to fp32: checked
    against a 60-digit decimal evaluation of 1 / (1 + exp(-z)), except where
    the oracle itself reports the rounding as too close to call."""
    from decimal import Decimal, getcontext
    getcontext().prec = 60
    rng = np.random.default_rng(11)
    z = np.concatenate([rng.standard_normal(3000) * 4, [0.0, -0.0, 1e-30, -1e-30, 20.0, -20.0, 88.0, -88.0,
                                                        -103.0, 17.0, -17.0]]).astype(np.float32)
    got = O.sigmoid_f32(z)
    amb, other = O.sigmoid_f32_ambiguous(z)
    assert amb.sum() <= 2
    for zi, g, a in zip(z, got, amb):
        x = Decimal(1) / (Decimal(1) + (-Decimal(float(zi))).exp())
        want = _nearest_f32(x)
        if not a:
            assert g == want, (float(zi), float(g), float(want))
    assert got[z == 0.0].tolist() == [0.5, 0.5]
    assert float(got[z == 20.0][0]) == 1.0                   # 1 - 2e-9 rounds to one in fp32
    # a planted single-rounding mistake (fp32 exp, as a float32 evaluation
    # would do) is caught by the same comparison on some input
    with np.errstate(over="ignore"):
        bad = (np.float32(1) / (np.float32(1) + np.exp(-z))).astype(np.float32)
    assert np.any(bad != got)


def test_v3_ambiguity_report_is_consistent():
    rng = np.random.default_rng(12)
    z = (rng.standard_normal(200000) * 3).astype(np.float32)
    amb, other = O.sigmoid_f32_ambiguous(z)
    s = O.sigmoid_f32(z)
    assert np.array_equal(other[~amb], s[~amb])
    # an ambiguous value's alternative is the adjacent fp32 value
    step = np.abs(other[amb].view(np.int32).astype(np.int64) - s[amb].view(np.int32).astype(np.int64))
    assert np.all(step == 1)
    # a wide window flags more values, a zero window none
    wide, _ = O.sigmoid_f32_ambiguous(z, rel=2.0 ** -30)
    none, _ = O.sigmoid_f32_ambiguous(z, rel=0.0)
    assert wide.sum() > amb.sum() and none.sum() <= amb.sum()
    assert np.all(wide[amb])


# ---- V2 -----------------------------------------------------------------

def test_v2_page_token_t2(golden):
    f = golden("m62_gating_fixtures.json")["v2_t2"]
    sc = np.array([f["scores"]], dtype=np.float64)
    ids, _ = O.group_limited_select(sc, f["n_group"], f["topk_group"], f["k"], "max")
    assert ids[0].tolist() == f["limited_top3"]
    assert abs(sc[0, ids[0]].sum() - f["limited_top3_sum"]) < 1e-12
    assert abs(sc[0, ids[0]].sum() * f["route_scale"] - f["scaled_gate_mass"]) < 1e-9
    gids, _ = O.group_limited_select(sc, 1, 1, f["k"], "max")     # one group: no restriction
    assert gids[0].tolist() == f["global_top3"]
    assert abs(sc[0, gids[0]].sum() - f["global_top3_sum"]) < 1e-12


def test_v2_route_is_softmax_then_group_selection_scaled():
    rng = np.random.default_rng(7)
    z = rng.standard_normal((20, 32)).astype(np.float32)
    ids, gates, inv = O.route_v2(z, 6, 8, 3, 16.0)
    p = np.exp(z.astype(np.float64) - z.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    # same selection as the group rule applied to the probabilities themselves
    ids_p, _ = O.group_limited_select(p, 8, 3, 6, "max")
    assert np.array_equal(ids, ids_p)
    assert np.allclose(gates, 16.0 * np.take_along_axis(p, ids.astype(np.int64), 1), rtol=1e-12)
    # every selected expert lies in at most three groups
    assert all(len(set((ids[t] // 4).tolist())) <= 3 for t in range(20))
    # with one group of everything, V2 selection is the global top-k
    ids1, _, _ = O.route_v2(z, 6, 1, 1, 1.0)
    ids_g, _, _ = O.route_topk(z, 6)
    assert np.array_equal(ids1, ids_g)


# ---- V1 -----------------------------------------------------------------

def test_v1_uniform_logits_closed_form():
    E, k = 64, 6
    ids, gates, _ = O.route_v1(np.zeros((3, E), np.float32), k)
    assert np.array_equal(ids, np.tile(np.arange(k), (3, 1)))   # ties go to the lower expert
    assert np.allclose(gates, 1.0 / E, rtol=1e-15)
    assert np.allclose(gates.sum(1), k / E)


def test_v1_is_renormalised_gate_times_selected_mass():
    rng = np.random.default_rng(3)
    z = rng.standard_normal((50, 64)).astype(np.float32)
    ids1, g1, _ = O.route_v1(z, 6)
    ids0, g0, _ = O.route_topk(z, 6)
    assert np.array_equal(ids1, ids0)
    assert np.all(g1.sum(1) < 1.0)
    assert np.allclose(g1 / g1.sum(1, keepdims=True), g0, rtol=1e-12)
    # the selected mass equals the sum of the k largest softmax probabilities
    p = np.exp(z.astype(np.float64) - z.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    assert np.allclose(g1.sum(1), np.sort(p, 1)[:, -6:].sum(1), rtol=1e-12)


def test_gating_invalid_token_and_bad_geometry():
    z = np.zeros((2, 16), np.float32)
    z[1, 3] = np.nan
    for ids, gates, inv in (O.route_v1(z, 2), O.route_v2(z, 2, 4, 2, 1.0), O.route_v3(z, None, 2, 4, 2, 1.0)):
        assert inv.tolist() == [False, True]
        assert (ids[1] == -1).all() and (gates[1] == 0).all()
    with pytest.raises(ValueError):
        O.group_limited_select(np.zeros((1, 10), np.float32), 4, 2, 2, "max")     # 10 % 4 != 0
    with pytest.raises(ValueError):
        O.group_limited_select(np.zeros((1, 16), np.float32), 4, 1, 5, "max")     # k > experts kept
