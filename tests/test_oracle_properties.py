"""Property, brute-force and mutation tests of the CPU oracle.

The brute-force helpers here are written as explicit loops over routes, in a
different form from the oracle (which uses a stable sort), so that a
mistake in either shows up as a disagreement.
"""
import numpy as np
import pytest

import oracle as O


# ---------------------------------------------------------------------------
# brute-force references (route-by-route loops)
# ---------------------------------------------------------------------------

def brute_plan(bucket, B, cap):
    bucket = list(bucket)
    R = len(bucket)
    seen = [0] * B
    pos = [-1] * R
    for r, b in enumerate(bucket):
        if 0 <= b < B:
            pos[r] = seen[b]
            seen[b] += 1
    keep = [0 <= b < B and (cap < 0 or pos[r] < cap) for r, b in enumerate(bucket)]
    counts = [sum(1 for r in range(R) if keep[r] and bucket[r] == e) for e in range(B)]
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    inv = [offsets[bucket[r]] + pos[r] if keep[r] else -1 for r in range(R)]
    src = [-1] * R
    for r in range(R):
        if keep[r]:
            src[inv[r]] = r
    return seen, counts, offsets, inv, src


def brute_route(z, k):
    out = []
    for row in z:
        if not np.all(np.isfinite(row)):
            out.append([-1] * k)
            continue
        items = list(range(len(row)))
        # selection sort: largest value, lowest index on ties
        chosen = []
        for _ in range(k):
            best = None
            for e in items:
                if e in chosen:
                    continue
                if best is None or row[e] > row[best]:
                    best = e
            chosen.append(best)
        out.append(chosen)
    return np.array(out)


# ---------------------------------------------------------------------------
# route
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(6))
def test_route_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    T, E = 40, int(rng.integers(2, 12))
    k = int(rng.integers(1, E + 1))
    z = rng.integers(-3, 4, size=(T, E)).astype(np.float32)
    z[rng.random((T, E)) < 0.1] = -0.0
    if seed % 2:
        z[3, 1] = np.nan
    ids, g, inv = O.route_topk(z, k)
    assert np.array_equal(ids, brute_route(z, k))
    live = ~inv
    np.testing.assert_allclose(g[live].sum(1), 1.0, rtol=1e-13)
    assert np.all(g[~live] == 0)


def test_route_invariants():
    rng = np.random.default_rng(3)
    z = rng.standard_normal((500, 64)).astype(np.float32)
    ids, g, _ = O.route_topk(z, 8)
    for t in range(z.shape[0]):
        sel = ids[t]
        assert len(set(sel.tolist())) == 8
        v = z[t, sel]
        assert np.all(np.diff(v) <= 0)                 # non-increasing along j
        rest = np.setdiff1d(np.arange(64), sel)
        assert np.all(z[t, rest] <= v[-1])             # nothing better left out
        assert np.all(np.diff(g[t]) <= 1e-15)


# ---------------------------------------------------------------------------
# dispatch plan
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(10))
def test_plan_brute_force(seed):
    rng = np.random.default_rng(200 + seed)
    B = int(rng.integers(1, 9))
    R = int(rng.integers(0, 60))
    bucket = rng.integers(-1, B, size=R)
    cap = int(rng.integers(-1, 6))
    plan = O.dispatch_plan(bucket, B, cap)
    sel, counts, offsets, inv, src = brute_plan(bucket, B, cap)
    assert plan.sel.tolist() == sel
    assert plan.counts.tolist() == counts
    assert plan.offsets.tolist() == offsets
    assert plan.inv.tolist() == inv
    assert plan.src.tolist() == src
    assert plan.accepted + plan.dropped == R
    O.check_dispatch(bucket, plan, capacity=cap)


def test_plan_bad_ids_are_dropped():
    plan = O.dispatch_plan(np.array([0, 5, -2, 1, -1, 0]), 3)
    assert plan.bad.tolist() == [False, True, True, False, False, False]
    assert plan.inv.tolist() == [0, -1, -1, 2, -1, 1]
    assert plan.dropped == 3


def test_plan_bijection_exercise():
    """"Dispatch and combine" modular orbit: x -> x + a mod m from 0 visits
    every residue for a = 1 (a bijection onto its entries) but only half of
    them for a = 2; the plan checker must reject the second as an inverse."""
    def orbit(m, a):
        x, seen = 0, []
        while x not in seen:
            seen.append(x)
            x = (x + a) % m
        return seen
    assert sorted(orbit(4, 1)) == [0, 1, 2, 3]
    assert len(orbit(4, 2)) == 2
    bucket = np.zeros(4, dtype=int)
    plan = O.dispatch_plan(bucket, 1)
    O.check_dispatch(bucket, plan)
    bad = O.DispatchPlan(**{**plan.__dict__})
    bad.src = np.array((orbit(4, 2) * 2)[:4])
    with pytest.raises(ValueError):
        O.check_dispatch(bucket, bad)


MUTATIONS = [
    ("counts", lambda p: p.counts.__setitem__(0, p.counts[0] + 1)),
    ("offsets", lambda p: p.offsets.__setitem__(2, p.offsets[2] + 1)),
    ("inv", lambda p: p.inv.__setitem__(np.nonzero(p.inv >= 0)[0][0], p.inv[np.nonzero(p.inv >= 0)[0][1]])),
    ("src_dup", lambda p: p.src.__setitem__(1, p.src[0])),
    ("src_swap", lambda p: p.src.__setitem__(slice(0, 2), p.src[1::-1].copy())),
    ("accepted", lambda p: setattr(p, "accepted", p.accepted - 1)),
    ("tail", lambda p: p.src.__setitem__(p.accepted, 0)),
]


@pytest.mark.parametrize("name,mutate", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_plan_mutations_rejected(name, mutate):
    """M6.2 §0x03G rejection list / M6.6 §0x03C3: changing one count,
    offset, inverse entry or order must fail the check."""
    rng = np.random.default_rng(11)
    bucket = rng.integers(0, 4, size=40)
    plan = O.dispatch_plan(bucket, 4, capacity=8)
    O.check_dispatch(bucket, plan, capacity=8)
    bad = O.DispatchPlan(**{k: (v.copy() if isinstance(v, np.ndarray) else v)
                            for k, v in plan.__dict__.items()})
    mutate(bad)
    with pytest.raises(ValueError):
        O.check_dispatch(bucket, bad, capacity=8)


def test_nonfinite_gate_rejected():
    bucket = np.array([0, 1, 0, 1])
    plan = O.dispatch_plan(bucket, 2)
    g = np.array([0.5, 0.5, np.nan, 0.5])
    with pytest.raises(ValueError):
        O.check_dispatch(bucket, plan, g)


# ---------------------------------------------------------------------------
# layer: two layouts, identity experts, capacity
# ---------------------------------------------------------------------------

def _random_layer(seed, T=24, d=8, E=5, k=2, f=6):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    z = rng.standard_normal((T, E)).astype(np.float32)
    ids, g, _ = O.route_topk(z, k)
    W = [(rng.standard_normal((f, d)), rng.standard_normal((f, d)), rng.standard_normal((d, f)))
         for _ in range(E)]
    return x, ids, g, O.swiglu_bank(lambda e: W[e])


@pytest.mark.parametrize("seed", range(4))
def test_two_layouts_agree(seed):
    """M6.2 §0x04D: token-major (repeat + mask) and expert-major (sort +
    segments + scatter) layouts produce the same mixture."""
    x, ids, g, bank = _random_layer(seed)
    y_tok = O.moe_layer_token_major(x, ids, g, bank, 5)
    y_exp, plan = O.moe_layer_expert_major(x, ids, g, bank, 5)
    np.testing.assert_allclose(y_exp, y_tok, rtol=1e-12, atol=1e-12)


def test_capacity_two_layouts_agree():
    x, ids, g, bank = _random_layer(7, T=40)
    cap = 6
    y_exp, plan = O.moe_layer_expert_major(x, ids, g, bank, 5, capacity=cap)
    keep = (plan.inv >= 0).reshape(ids.shape)
    assert plan.dropped > 0
    y_tok = O.moe_layer_token_major(x, ids, g, bank, 5, keep=keep)
    np.testing.assert_allclose(y_exp, y_tok, rtol=1e-12, atol=1e-12)


def test_identity_experts_reproduce_tokens():
    """Identity experts with renormalised gates return each token itself; with
    drops they return the kept gate mass times the token (no renormalisation
    after a drop, M6.2 §0x05D reading)."""
    x, ids, g, _ = _random_layer(8, T=50)
    ident = lambda e, rows: rows
    y, _ = O.moe_layer_expert_major(x, ids, g, ident, 5)
    np.testing.assert_allclose(y, x, rtol=1e-13)
    y, plan = O.moe_layer_expert_major(x, ids, g, ident, 5, capacity=7)
    keep = (plan.inv >= 0).reshape(ids.shape)
    np.testing.assert_allclose(y, (g * keep).sum(1)[:, None] * x, rtol=1e-13, atol=1e-15)


def test_gate_after_expert():
    """M6.6 §0x0AE: the gate scales the expert output, E(g h) != g E(h)."""
    sq = lambda e, rows: rows ** 2
    x = np.array([[2.0]])
    ids = np.array([[0, 1]])
    g = np.array([[0.25, 0.75]])
    y, _ = O.moe_layer_expert_major(x, ids, g, sq, 2)
    assert y[0, 0] == pytest.approx(4.0)


def test_combine_window_and_accumulate():
    z = np.arange(12, dtype=np.float64).reshape(6, 2)
    idx = np.array([0, 7, 3, -1, 9, 2])
    g = np.array([1.0, 2.0, 3.0, 4.0, 5.0, 6.0])
    y = O.combine(z[0:4], idx, g, 3, 2, lo=0, hi=4)
    y = O.combine(z[4:6] * 0 + z[0:2], idx, g, 3, 2, lo=8, hi=10, y=y)
    want = np.zeros((3, 2))
    want[0] = 1 * z[0]
    want[1] = 3 * z[3]
    want[2] = 5 * z[1] + 6 * z[2]
    np.testing.assert_allclose(y, want)


# ---------------------------------------------------------------------------
# pool pack and receiver compaction
# ---------------------------------------------------------------------------

def brute_pack(x, ids, epd, D, W, P):
    """Route-by-route pack.  Header: as many full-width rows as the P ids need
    (at least one); data row ``row`` sits below them."""
    T, k = ids.shape
    d = x.shape[1]
    H = 1
    while H * d < P:
        H += 1
    pools = np.zeros((W, D, P + H, d), dtype=np.uint16)
    pools[:, :, :H, :] = 0xFFFF
    loc = [-1] * (T * k)
    ordinal = [0] * D
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            if not 0 <= e < D * epd:
                continue
            dst, l = e // epd, e % epd
            o = ordinal[dst]
            ordinal[dst] += 1
            w, row = o % W, o // W
            if row >= P:
                continue
            pools[w, dst, H + row] = x[t]
            pools[w, dst, row // d, row % d] = l
            loc[t * k + j] = (w * D + dst) * (P + H) + H + row
    return pools, loc, ordinal


@pytest.mark.parametrize("seed", range(8))
def test_pool_pack_brute_force(seed):
    rng = np.random.default_rng(300 + seed)
    epd, D, W = 3, 4, int(rng.integers(1, 4))
    # pools of up to three header rows (d = 8 ids per header row)
    P = int(rng.integers(1, 5)) if seed < 4 else int(rng.integers(9, 21))
    T, k, d = 30 if seed >= 4 else 9, 2, 8
    ids = rng.integers(-1, D * epd, size=(T, k))
    x = rng.integers(0, 2 ** 16, size=(T, d)).astype(np.uint16)
    pk = O.pool_pack(x, ids, epd, D, W, P)
    pools, loc, ordinal = brute_pack(x, ids, epd, D, W, P)
    assert np.array_equal(pk["pools"], pools)
    assert pk["route_loc"].tolist() == loc
    assert pk["dest_counts"].tolist() == ordinal
    assert pk["sender_dropped"] == T * k - sum(1 for v in loc if v >= 0)


def test_pool_pack_invariants():
    rng = np.random.default_rng(9)
    epd, D, W, P = 6, 8, 3, 40
    T, k, d = 200, 4, 48
    z = rng.standard_normal((T, D * epd)).astype(np.float32)
    z[:, :6] += 2.0          # one hot destination overflows
    ids, _, _ = O.route_topk(z, k)
    x = rng.integers(0, 2 ** 16, size=(T, d)).astype(np.uint16)
    pk = O.pool_pack(x, ids, epd, D, W, P)
    loc = pk["route_loc"]
    live = loc[loc >= 0]
    assert np.unique(live).size == live.size                 # each slot used once
    n = pk["dest_counts"]
    assert pk["sender_dropped"] == int(np.maximum(0, n - W * P).sum())
    pools = pk["pools"].reshape(-1, d)
    r = np.nonzero(loc >= 0)[0]
    assert np.array_equal(pools[loc[r]], x[r // k])           # payload rows
    hdr = pk["pools"][:, :, 0, :]
    w_idx, dst, row = pk["wave"][r], pk["dest"][r], pk["row"][r]
    assert np.array_equal(hdr[w_idx, dst, row], (ids.reshape(-1)[r] % epd))
    for dd in range(D):                                       # waves balanced
        per_wave = [(hdr[w, dd, :P] != 0xFFFF).sum() for w in range(W)]
        assert max(per_wave) - min(per_wave) <= 1
    assert np.all(hdr[:, :, P:] == 0xFFFF)


def brute_compact(pools, L, cap, P, rotation=0):
    """Row-by-row compaction, sources visited from ``rotation`` onward."""
    S, P1, d = pools.shape
    H = P1 - P
    comp = np.zeros((L, cap, d), dtype=np.uint16)
    cnt = [0] * L
    slot = [-1] * (S * P1)
    for v in range(S):
        s = (rotation + v) % S
        for i in range(P):
            h = int(pools[s, i // d, i % d])
            if h >= L:
                continue
            q = cnt[h]
            cnt[h] += 1
            if q < cap:
                comp[h, q] = pools[s, H + i]
                slot[s * P1 + H + i] = h * cap + q
    return comp, cnt, slot


@pytest.mark.parametrize("seed", range(8))
def test_recv_compact_brute_force(seed):
    rng = np.random.default_rng(400 + seed)
    S, d, L = 5, 8, 3
    P = 6 if seed < 4 else int(rng.integers(9, 21))          # one to three header rows
    H = -(-P // d)
    rotation = 0 if seed % 2 == 0 else int(rng.integers(1, S))
    cap = int(rng.integers(1, 9))
    pools = rng.integers(0, 2 ** 16, size=(S, P + H, d)).astype(np.uint16)
    hdr = rng.integers(0, L + 1, size=(S, P))
    hdr[hdr == L] = 0xFFFF
    hdr[0, 0] = 7                                             # bad id
    flat = np.full((S, H * d), 0xFFFF, dtype=np.uint16)
    flat[:, :P] = hdr
    pools[:, :H, :] = flat.reshape(S, H, d)
    rc = O.recv_compact(pools, L, cap, rotation=rotation)
    comp, cnt, slot = brute_compact(pools, L, cap, P, rotation)
    assert np.array_equal(rc["compact"], comp)
    assert rc["arrived"].tolist() == cnt
    assert rc["counts"].tolist() == [min(c, cap) for c in cnt]
    assert rc["row_slot"].tolist() == slot
    assert rc["recv_dropped"] == sum(max(0, c - cap) for c in cnt)
    assert rc["bad_header"] == 1


def test_loopback_identity_experts():
    """Sender pack -> receiver compaction -> identity experts -> expand ->
    sender combine returns each token scaled by the gate mass that survived
    both the sender and the receiver capacity."""
    rng = np.random.default_rng(12)
    epd, D, W, P, cap = 3, 4, 2, 6, 9
    T, k, d = 30, 2, 8
    z = rng.standard_normal((T, D * epd)).astype(np.float32)
    ids, g, _ = O.route_topk(z, k)
    xf = rng.standard_normal((T, d)).astype(np.float32)
    bits = (xf.view(np.uint32) >> 16).astype(np.uint16)       # truncation is fine here
    y, det = O.loopback_layer(bits, ids, g, lambda e, rows: rows, epd, D, W, P, cap)
    loc = det["pack"]["route_loc"]
    kept = np.zeros(T * k, dtype=bool)
    P1 = P + O.header_rows(P, d)
    for w, rc in enumerate(det["waves"]):
        lo = w * D * P1
        inwave = (loc >= lo) & (loc < lo + D * P1)
        kept |= inwave & (rc["row_slot"][np.where(inwave, loc - lo, 0)] >= 0)
    mass = (g.reshape(-1) * kept).reshape(T, k).sum(1)
    np.testing.assert_allclose(y, mass[:, None] * O.bf16_to_f64(bits), rtol=1e-13)
    sent = int((loc >= 0).sum())
    arrived = sum(int(rc["arrived"].sum()) for rc in det["waves"])
    assert sent == arrived
    acc = sum(int(rc["counts"].sum()) for rc in det["waves"])
    assert acc + sum(rc["recv_dropped"] for rc in det["waves"]) == arrived


def test_rotation_moves_overflow_to_the_last_visited_source():
    """Pooled wave §07: with the fixed order, receiver overflow always falls
    on the last sources; a rotation makes the last visited source take it."""
    S, P, d, L, cap = 4, 5, 8, 2, 12
    pools = np.zeros((S, P + 1, d), dtype=np.uint16)
    pools[:, 0, :] = 0xFFFF
    pools[:, 0, :P] = 0                                       # every row wants local expert 0
    for rot in range(S):
        rc = O.recv_compact(pools, L, cap, rotation=rot)
        dropped_src = {s for s in range(S) for i in range(P) if rc["row_slot"][s * (P + 1) + 1 + i] < 0}
        # 20 rows, 12 accepted: the last 8 visited rows (sources rot-1 and rot-2, wrapping) are dropped
        assert dropped_src == {(rot - 1) % S, (rot - 2) % S}
        assert rc["recv_dropped"] == S * P - cap
        assert rc["counts"].tolist() == [cap, 0]


def test_two_wave_profile_geometry():
    """Pooled wave §04/§05: at two waves the sender pool grows to
    ceil(1.10 * 524288 / 64 / 2) rows, which needs two header rows at
    d = 3072, and the receiver array to ceil(1.15 * 524288 / 6 / 2)."""
    P2 = O.capacity_ceil(110, 100, 524288, 64 * 2)
    assert P2 == 4506 and O.header_rows(P2, 3072) == 2
    assert O.capacity_ceil(115, 100, 524288, 6 * 2) == 50245
    P3 = O.capacity_ceil(110, 100, 524288, 64 * 3)
    assert P3 == 3004 and O.header_rows(P3, 3072) == 1
    assert O.pool_rows_of(P2 + 2, 3072) == P2 and O.pool_rows_of(P3 + 1, 3072) == P3
    # both profiles hold the same number of incoming rows per receiver
    assert 2 * 64 * P2 == 3 * 64 * P3


def test_loopback_identity_experts_two_header_rows():
    rng = np.random.default_rng(13)
    epd, D, W, P, cap = 3, 4, 2, 19, 40                       # 19 ids need three 8-wide header rows
    T, k, d = 60, 2, 8
    z = rng.standard_normal((T, D * epd)).astype(np.float32)
    ids, g, _ = O.route_topk(z, k)
    bits = rng.integers(0, 2 ** 15, size=(T, d)).astype(np.uint16)
    y, det = O.loopback_layer(bits, ids, g, lambda e, rows: rows, epd, D, W, P, cap)
    loc = det["pack"]["route_loc"]
    H = O.header_rows(P, d)
    assert H == 3
    kept = np.zeros(T * k, dtype=bool)
    for w, rc in enumerate(det["waves"]):
        lo = w * D * (P + H)
        inwave = (loc >= lo) & (loc < lo + D * (P + H))
        kept |= inwave & (rc["row_slot"][np.where(inwave, loc - lo, 0)] >= 0)
    mass = (g.reshape(-1) * kept).reshape(T, k).sum(1)
    np.testing.assert_allclose(y, O.bf16_to_f64(bits) * mass[:, None], rtol=1e-12, atol=1e-300)
