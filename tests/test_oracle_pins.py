"""Pins of the CPU oracle against values the pages print and closed forms.

Each test names the page and section its expected values come from; the
values themselves live in ``tests/golden``.
"""
import math

import numpy as np
import pytest
from scipy.special import expit, softmax

import oracle as O


# ---------------------------------------------------------------------------
# M6.6 §0x03A1 / §0x03B / §0x03C3 / §0x04A / §0x04F: eight-route fixture
# ---------------------------------------------------------------------------

def test_eight_route_fixture_output(golden):
    g = golden("m66_eight_route_fixture.json")
    x = np.array(g["hidden"], dtype=np.float64)
    T, k = x.shape[0], g["k"]
    ids = np.array(g["logical_expert"]).reshape(T, k)
    gates = np.array(g["gate"]).reshape(T, k)
    bank = O.scalar_bank(g["scalar_expert"])
    want = np.array(g["expected_output"])
    y_tok = O.moe_layer_token_major(x, ids, gates, bank, 4)
    y_exp, plan = O.moe_layer_expert_major(x, ids, gates, bank, 4)
    np.testing.assert_allclose(y_tok, want, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(y_exp, want, rtol=1e-12, atol=1e-12)
    assert plan.counts.tolist() == g["expected_logical_counts"]


def test_eight_route_fixture_send_layout(golden):
    """Per-source send counts, offsets and order by (destination, physical
    slot, route position), built from the oracle's stable bucket plan."""
    g = golden("m66_eight_route_fixture.json")
    src = np.array(g["source_rank"])
    dst = np.array(g["destination_rank"])
    slot = np.array(g["physical_slot"])
    P, Q = 4, 6
    cm = np.zeros((P, P), dtype=int)
    for p in range(P):
        routes = np.nonzero(src == p)[0]
        plan_d = O.dispatch_plan(dst[routes], P)
        cm[p] = plan_d.sel
        if routes.size == 0:
            continue
        assert plan_d.offsets.tolist() == g["expected_send_offsets"][str(p)]
        # composite key (destination, slot), stable in route order
        plan = O.dispatch_plan(dst[routes] * Q + slot[routes], P * Q)
        order = routes[plan.src[: plan.accepted]]
        assert order.tolist() == g["expected_send_order"][str(p)]
    assert cm.tolist() == g["expected_count_matrix"]


def test_eight_route_fixture_slot_segments(golden):
    """M6.6 §0x03C2/§0x04A: rows per physical slot, in the manifest's slot
    order, n = [2,2,1,1,1,1], o = [0,2,4,5,6,7,8]."""
    g = golden("m66_eight_route_fixture.json")
    plan = O.dispatch_plan(np.array(g["physical_slot"]), 6)
    assert plan.counts.tolist() == g["expected_slot_counts"]
    assert plan.offsets.tolist() == g["expected_slot_offsets"]
    members = [plan.src[a:b].tolist() for a, b in zip(plan.offsets[:-1], plan.offsets[1:])]
    assert members == g["expected_slot_members"]
    # the slot layout executes the same function (replicas of one expert)
    slot_to_expert = {0: 0, 1: 0, 2: 1, 3: 1, 4: 2, 5: 3}
    x = np.array(g["hidden"], dtype=np.float64)
    s = g["scalar_expert"]
    xp = O.gather_rows(x, plan.src, g["k"], plan.accepted)
    z = O.run_segments(xp, plan.offsets[:-1], plan.counts,
                       lambda q, rows: s[slot_to_expert[q]] * rows)
    y = O.combine(z, plan.inv, np.array(g["gate"]), 4, 2)
    np.testing.assert_allclose(y, g["expected_output"], rtol=1e-12)


# ---------------------------------------------------------------------------
# M6.2 §0x03A-§0x03C: logical transpose fixture
# ---------------------------------------------------------------------------

def test_logical_transpose_fixture(golden):
    g = golden("m62_logical_transpose_fixture.json")
    x = np.array(g["hidden"], dtype=np.float64)
    ids = np.array(g["expert"]).reshape(4, 2)
    gates = np.array(g["gate"]).reshape(4, 2)
    bank = O.scalar_bank(g["scalar_expert"])
    y, plan = O.moe_layer_expert_major(x, ids, gates, bank, 4)
    assert plan.counts.tolist() == g["expected_counts"]
    assert plan.offsets.tolist() == g["expected_offsets"]
    assert plan.src.tolist() == g["expected_pi"]
    assert plan.inv.tolist() == g["expected_inverse_pi"]
    np.testing.assert_allclose(y, g["expected_output"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(O.moe_layer_token_major(x, ids, gates, bank, 4),
                               g["expected_output"], rtol=1e-12, atol=1e-12)
    O.check_dispatch(ids, plan, gates)


# ---------------------------------------------------------------------------
# M6.6 §0x04A-§0x04F: row and FLOP ledgers of three representations
# ---------------------------------------------------------------------------

def test_runner_ledgers(golden):
    g = golden("m66_runner_ledgers.json")
    n = g["counts"]
    rows = {
        "grouped": sum(n),
        "padded": O.padded_exec_rows(len(n), g["capacity"], g["align"]),
        "block": O.block_exec_rows(n, g["block_rows"]),
    }
    assert rows == g["expected_rows"]
    for name, r in rows.items():
        assert O.swiglu_flops(r, g["d"], g["d_ff"]) == g["expected_flops"][name]


# ---------------------------------------------------------------------------
# pooled wave §04/§05: capacities, array sizes, drop arithmetic
# ---------------------------------------------------------------------------

def test_pooled_wave_capacities(golden):
    g = golden("pooled_wave_sizes.json")
    A = g["tokens_per_gpu"] * g["top_k"]
    assert A == g["assignments"]
    cs = O.capacity_ceil(*g["sender_factor"], A, g["n_dest"] * g["n_waves"])
    cr = O.capacity_ceil(*g["receiver_factor"], A, g["local_experts"] * g["n_waves"])
    assert cs == g["expected_sender_capacity"]
    assert cr == g["expected_receiver_capacity"]
    gib = 2.0 ** 30
    sizes = {
        "sender_pool_64x3004x3072": 64 * cs * 3072 * 2 / gib,
        "receiver_compact_6x33497x3072": 6 * cr * 3072 * 2 / gib,
        "direct_6x64x1816x3072": 6 * 64 * 1816 * 3072 * 2 / gib,
    }
    for key, want in g["arrays_gib"].items():
        assert round(sizes[key], 2) == want


def test_capacity_ceil_is_exact():
    # a float ceil of 1.10*x can land one above the exact value for round x
    assert O.capacity_ceil(110, 100, 100, 1) == 110
    assert O.capacity_ceil(115, 100, 600, 6) == 115
    assert O.capacity_ceil(1, 1, 7, 2) == 4


def test_drop_rates(golden):
    g = golden("pooled_wave_sizes.json")["drop_percent"]
    T = 10 ** 6
    S = round(T * g["sender"] / 100)
    R = round(T * g["receiver"] / 100)
    s, r, c = O.drop_rates(T, S, R)
    assert round(100 * (s + r), 2) == g["total"]
    # the page prints 13.12 from unrounded run counters; the rounded inputs give 13.127
    assert abs(100 * c - g["conditional_receiver"]) < 0.01


# ---------------------------------------------------------------------------
# a1 route: closed forms and textbook routines
# ---------------------------------------------------------------------------

def test_route_k1_is_first_argmax():
    rng = np.random.default_rng(5)
    z = rng.integers(-3, 3, size=(200, 16)).astype(np.float32)   # many ties
    ids, g, inv = O.route_topk(z, 1)
    assert np.array_equal(ids[:, 0], np.argmax(z, axis=1))
    assert np.all(g == 1.0) and not inv.any()


def test_route_k_equals_E_is_stable_descending_sort():
    rng = np.random.default_rng(6)
    z = rng.integers(-2, 2, size=(100, 9)).astype(np.float32)
    ids, g, _ = O.route_topk(z, 9)
    want = np.argsort(-z, axis=1, kind="stable")
    assert np.array_equal(ids, want)
    p = softmax(z.astype(np.float64), axis=1)
    np.testing.assert_allclose(g, np.take_along_axis(p, want, axis=1), rtol=1e-13)


def test_route_gates_are_renormalised_softmax():
    """Mixtral row of M6.2 §0x06L1: selected softmax mass renormalised to 1."""
    rng = np.random.default_rng(7)
    z = rng.standard_normal((300, 32)).astype(np.float32)
    ids, g, _ = O.route_topk(z, 4)
    p = softmax(z.astype(np.float64), axis=1)
    psel = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    np.testing.assert_allclose(g, psel / psel.sum(1, keepdims=True), rtol=1e-13)
    np.testing.assert_allclose(g.sum(1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(g, softmax(np.take_along_axis(z, ids.astype(np.int64), 1)
                                          .astype(np.float64), axis=1), rtol=1e-12)


def test_route_signed_zero_ties_and_nan():
    z = np.array([[0.0, -0.0, 0.0, -1.0],
                  [-0.0, 0.0, -5.0, -0.0],
                  [1.0, np.nan, 2.0, 3.0],
                  [1.0, np.inf, 2.0, 3.0]], dtype=np.float32)
    ids, g, inv = O.route_topk(z, 3)
    assert ids[0].tolist() == [0, 1, 2]
    assert ids[1].tolist() == [0, 1, 3]
    assert inv.tolist() == [False, False, True, True]
    assert ids[2].tolist() == [-1, -1, -1] and np.all(g[2] == 0)


# ---------------------------------------------------------------------------
# a4/a5 SwiGLU: closed form, element loops, fused-shared identity
# ---------------------------------------------------------------------------

def test_silu_matches_logistic():
    v = np.linspace(-30, 30, 601)
    np.testing.assert_allclose(O.silu(v), v * expit(v), rtol=1e-14, atol=1e-300)


def test_swiglu_closed_form_scalar():
    """d = d_ff = 1: E(x) = w_d * SiLU(w_g x) * (w_u x); swapping gate and up
    or dropping the SiLU gives a different number."""
    x = np.array([[1.5]])
    out = O.swiglu_expert(x, np.array([[0.5]]), np.array([[2.0]]), np.array([[3.0]]))
    s = 0.75 / (1.0 + math.exp(-0.75))
    assert out[0, 0] == pytest.approx(3.0 * s * 3.0, rel=1e-15)


def test_swiglu_element_loops():
    """Non-square shapes catch a transposed operand; explicit loops are the
    textbook definition of each product."""
    rng = np.random.default_rng(8)
    n, d, f = 3, 5, 7
    x = rng.standard_normal((n, d))
    wg, wu = rng.standard_normal((f, d)), rng.standard_normal((f, d))
    wd = rng.standard_normal((d, f))
    want = np.zeros((n, d))
    for r in range(n):
        h = []
        for c in range(f):
            gsum = sum(x[r, i] * wg[c, i] for i in range(d))
            usum = sum(x[r, i] * wu[c, i] for i in range(d))
            h.append(gsum / (1 + math.exp(-gsum)) * usum)
        for o in range(d):
            want[r, o] = sum(h[c] * wd[o, c] for c in range(f))
    np.testing.assert_allclose(O.swiglu_expert(x, wg, wu, wd), want, rtol=1e-12)


def test_fused_shared_experts_identity():
    """M6.2 §0x04C1: the sum of bias-free SwiGLU experts equals one SwiGLU
    with gate/up stacked by rows and down stacked by columns."""
    rng = np.random.default_rng(9)
    d, f, ns = 6, 4, 3
    G = [rng.standard_normal((f, d)) for _ in range(ns)]
    U = [rng.standard_normal((f, d)) for _ in range(ns)]
    D = [rng.standard_normal((d, f)) for _ in range(ns)]
    x = rng.standard_normal((2, d))
    split = sum(O.swiglu_expert(x, G[s], U[s], D[s]) for s in range(ns))
    fused = O.swiglu_expert(x, np.vstack(G), np.vstack(U), np.hstack(D))
    assert np.max(np.abs(split - fused)) < 1e-13


def test_bf16_upcast_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x4049, 0x7F7F, 0x0001], dtype=np.uint16)
    want = [1.0, -1.0, 0.0, -0.0, 3.140625, 3.3895313892515355e38, 9.183549615799121e-41]
    got = O.bf16_to_f64(bits)
    assert got.tolist() == want
    assert math.copysign(1.0, got[3]) == -1.0
