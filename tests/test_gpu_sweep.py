"""Seeded random sweep of small shapes for the GPU path against the oracle.

Each case draws its sizes from a seeded generator (printed on failure), so
that shapes no hand-written case names (odd expert counts, widths of 8, k
up to 16, capacities below and above the mean load, ragged pools) are run
through the same bit-exact and 2e-2 checks as the fixed cases."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle as O
import workloads as W
from tests.helpers import as_f64, assert_rows_close, to_gpu, to_np
from tests.test_gpu_ops import _gates_close, _v3_exact

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ge():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import grouped_expert_amd as ge
    return ge


@pytest.mark.parametrize("seed", range(24))
def test_route_permute_combine_sweep(ge, seed):
    rng = np.random.default_rng(1000 + seed)
    E = int(rng.choice([2, 3, 8, 31, 64, 129, 384, 1024]))
    k = int(rng.integers(1, min(E, 16) + 1))
    T = int(rng.integers(0, 700))
    d = int(rng.choice([8, 16, 72, 256, 520]))
    cap = int(rng.choice([-1, 0, max(1, T * k // E), 3 * T * k // E + 1]))
    dt = str(rng.choice(["f32", "bf16"]))
    case = dict(seed=seed, E=E, k=k, T=T, d=d, cap=cap, dt=dt)
    z = rng.standard_normal((T, E)).astype(np.float32)
    if T and rng.random() < 0.5:
        z[rng.integers(0, T), :] = 0.0                        # a token with all-equal logits (ties)
    x32 = rng.standard_normal((T, d)).astype(np.float32)
    x = W.f32_to_bf16_bits(x32) if dt == "bf16" else x32
    flags = ge.new_flags("cuda")
    zt = to_gpu(z) if T else torch.empty((0, E), device="cuda")
    ids, g = ge.route_topk(zt, k, flags=flags)
    want_ids, want_g, _ = O.route_topk(z, k)
    assert np.array_equal(to_np(ids), want_ids), case
    assert np.all(np.abs(to_np(g).astype(np.float64) - want_g) <= 1e-5 * np.abs(want_g) + 1e-7), case
    xt = to_gpu(x) if T else torch.empty((0, d), dtype=torch.bfloat16 if dt == "bf16" else torch.float32,
                                         device="cuda")
    plan = ge.permute(xt, ids, E, cap, flags=flags)
    want = O.dispatch_plan(want_ids.reshape(-1), E, cap)
    assert np.array_equal(to_np(plan["inv"]), want.inv), case
    assert np.array_equal(to_np(plan["counts"]), want.counts), case
    assert np.array_equal(to_np(plan["offsets"]), want.offsets), case
    assert int(to_np(plan["dropped"])[0]) == want.dropped, case
    A = want.accepted
    if A:
        assert np.array_equal(to_np(plan["x_perm"])[:A], x[want.src[:A] // k]), case
    y = ge.unpermute_combine(plan["x_perm"], plan["inv"], g, T, k, flags=flags)
    want_y = O.combine(O.to_f64(x)[want.src[:A] // k] if A else np.zeros((0, d)), want.inv, want_g, T, k)
    if T:
        assert_rows_close(to_np(y).astype(np.float64), want_y, tol=1e-5, what=str(case))
    assert int(to_np(flags)[0]) == 0, case


@pytest.mark.parametrize("seed", range(16))
def test_pack_compact_sweep(ge, seed):
    rng = np.random.default_rng(2000 + seed)
    epd = int(rng.integers(1, 7))
    D = int(rng.choice([1, 3, 8, 17]))
    E = epd * D
    k = int(rng.integers(1, min(E, 8) + 1))
    T = int(rng.integers(1, 900))
    Wv = int(rng.integers(1, 4))
    d = int(rng.choice([8, 64, 200, 512]))
    P = int(rng.integers(0, 2 * T * k // max(1, D * Wv) + 3))
    payload = rng.choice([None, "row", "b128"]) if d % 8 == 0 else None
    case = dict(seed=seed, epd=epd, D=D, k=k, T=T, Wv=Wv, d=d, P=P, payload=payload)
    z = rng.standard_normal((T, E)).astype(np.float32)
    ids, _, _ = O.route_topk(z, k)
    x16 = W.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    rows = x16 if payload is None else O.quantize_fp8_rows(O.to_f64(x16).astype(np.float32), payload)
    flags = ge.new_flags("cuda")
    out = ge.pool_pack(to_gpu(x16), to_gpu(ids), E, epd, D, Wv, P, flags=flags, payload=payload, d=d)
    pk = O.pool_pack(rows, ids, epd, D, Wv, P)
    assert np.array_equal(to_np(out["pools"]), pk["pools"]), case
    assert np.array_equal(to_np(out["route_loc"]), pk["route_loc"]), case
    assert int(to_np(out["sender_dropped"])[0]) == pk["sender_dropped"], case
    cap = int(rng.integers(0, P * D + 2))
    for w in range(Wv):
        rot = int(rng.integers(0, D))
        rc = ge.recv_compact(out["pools"][w], epd, cap, flags=flags, rotation=rot, payload=payload, d=d)
        want = O.recv_compact(pk["pools"][w], epd, cap, rotation=rot,
                              **({} if payload is None else dict(record=(d, payload))))
        counts = to_np(rc["counts"])
        assert np.array_equal(counts, want["counts"]), case
        assert np.array_equal(to_np(rc["row_slot"]), want["row_slot"]), case
        assert int(to_np(rc["recv_dropped"])[0]) == want["recv_dropped"], case
        got = to_np(rc["compact"])
        for h in range(epd):
            assert np.array_equal(got[h, :counts[h]], want["compact"][h, :counts[h]]), (case, w, h)
    assert int(to_np(flags)[0]) == 0, case


@pytest.mark.parametrize("seed", range(12))
def test_grouped_swiglu_sweep(ge, seed):
    rng = np.random.default_rng(3000 + seed)
    E = int(rng.choice([1, 5, 16, 40]))
    d = int(rng.choice([64, 128, 192, 320]))
    d_ff = int(rng.choice([64, 128, 256, 384]))
    top = min(int(rng.choice([3, 40, 300, 900])), 4000 // E + 1)       # the fp64 oracle stays fast
    counts = rng.integers(0, top, size=E).astype(np.int32)
    gaps = rng.integers(0, 5, size=E).astype(np.int32)
    starts = (np.cumsum(counts + gaps) - counts).astype(np.int32)
    rows = int(starts[-1] + counts[-1] + rng.integers(0, 9))
    zdt = str(rng.choice(["f32", "bf16"]))
    case = dict(seed=seed, E=E, d=d, d_ff=d_ff, rows=rows, zdt=zdt, counts=counts.tolist())
    x = W.f32_to_bf16_bits(rng.standard_normal((rows, d)).astype(np.float32))
    ws = [W.f32_to_bf16_bits((0.05 * rng.standard_normal(s)).astype(np.float32))
          for s in [(E, d_ff, d), (E, d_ff, d), (E, d, d_ff)]]
    flags = ge.new_flags("cuda")
    zt = torch.float32 if zdt == "f32" else torch.bfloat16
    z0 = torch.zeros((rows, d), dtype=zt, device="cuda")
    z = ge.grouped_swiglu(to_gpu(x), to_gpu(starts), to_gpu(counts), *[to_gpu(w) for w in ws], z=z0, flags=flags)
    want = O.run_segments(x, starts, counts, O.swiglu_bank(lambda e: (ws[0][e], ws[1][e], ws[2][e])))
    assert_rows_close(as_f64(z), want, what=str(case))
    covered = np.zeros(rows, bool)
    for s, c in zip(starts, counts):
        covered[s:s + c] = True
    assert np.all(as_f64(z)[~covered] == 0), case                   # rows outside every segment untouched
    assert int(to_np(flags)[0]) == 0, case


@pytest.mark.parametrize("seed", range(8))
def test_grouped_swiglu_backward_sweep(ge, seed):
    rng = np.random.default_rng(4000 + seed)
    E = int(rng.choice([1, 3, 12]))
    d = int(rng.choice([64, 192, 256]))
    d_ff = int(rng.choice([64, 128, 320]))
    top = min(int(rng.choice([2, 70, 500, 1100])), 3000 // E + 1)
    counts = rng.integers(0, top, size=E).astype(np.int32)
    gaps = rng.integers(0, 4, size=E).astype(np.int32)
    starts = (np.cumsum(counts + gaps) - counts).astype(np.int32)
    rows = int(starts[-1] + counts[-1] + rng.integers(0, 5))
    dxdt = torch.float32 if rng.random() < 0.5 else torch.bfloat16
    case = dict(seed=seed, E=E, d=d, d_ff=d_ff, rows=rows, counts=counts.tolist(), dx=str(dxdt))
    x = W.f32_to_bf16_bits(rng.standard_normal((rows, d)).astype(np.float32))
    dz = W.f32_to_bf16_bits(rng.standard_normal((rows, d)).astype(np.float32))
    ws = [W.f32_to_bf16_bits((0.05 * rng.standard_normal(s)).astype(np.float32))
          for s in [(E, d_ff, d), (E, d_ff, d), (E, d, d_ff)]]
    flags = ge.new_flags("cuda")
    dx0 = torch.zeros((rows, d), dtype=dxdt, device="cuda")
    out = ge.grouped_swiglu_backward(to_gpu(x), to_gpu(dz), to_gpu(starts), to_gpu(counts),
                                     *[to_gpu(w) for w in ws], dx=dx0, flags=flags)
    torch.cuda.synchronize()
    assert int(to_np(flags)[0]) == 0, case
    want_dx, grads = O.run_segments_backward(x, O.to_f64(dz), starts, counts,
                                             O.swiglu_bank_backward(lambda e: (ws[0][e], ws[1][e], ws[2][e])))
    covered = np.zeros(rows, bool)
    for s, c in zip(starts, counts):
        covered[s:s + c] = True
    got_dx = as_f64(out["dx"])
    if covered.any():
        assert_rows_close(got_dx[covered], want_dx[covered], what=f"dx {case}")
    assert np.all(got_dx[~covered] == 0), case
    for e in range(E):
        for name, i in (("dw_gate", 0), ("dw_up", 1), ("dw_down", 2)):
            got = to_np(out[name][e]).astype(np.float64)
            if grads[e] is None:
                assert np.all(got == 0), (case, e, name)
            else:
                assert_rows_close(got, grads[e][i], what=f"{name}[{e}] {case}")


@pytest.mark.parametrize("seed", range(10))
def test_grouped_router_sweep(ge, seed):
    """V2 (group-limited softmax) and V3 (sigmoid + bias, top-two group
    scores) on random group geometries."""
    rng = np.random.default_rng(5000 + seed)
    n_group = int(rng.choice([1, 2, 4, 8]))
    per = int(rng.choice([2, 4, 16, 32]))
    E = n_group * per
    topk_group = int(rng.integers(1, n_group + 1))
    k = int(rng.integers(1, min(topk_group * per, 16) + 1))
    T = int(rng.integers(1, 400))
    scale = float(rng.choice([1.0, 2.5, 16.0]))
    case = dict(seed=seed, E=E, n_group=n_group, topk_group=topk_group, k=k, T=T, scale=scale)
    z = rng.standard_normal((T, E)).astype(np.float32)
    bias = (0.1 * rng.standard_normal(E)).astype(np.float32)
    flags = ge.new_flags("cuda")
    ids2, g2 = ge.route_topk_grouped(to_gpu(z), k, ge.MOE_GATING_SOFTMAX_GROUP_LIMITED, n_group, topk_group, scale,
                                     flags=flags)
    want2 = O.route_v2(z, k, n_group, topk_group, scale)
    assert np.array_equal(to_np(ids2), want2[0]), case
    assert np.all(np.abs(to_np(g2).astype(np.float64) - want2[1]) <= 1e-5 * np.abs(want2[1]) + 1e-7), case
    ids3, g3 = ge.route_topk_grouped(to_gpu(z), k, ge.MOE_GATING_SIGMOID_BIAS_GROUP_TOP2, n_group, topk_group,
                                     scale, bias=to_gpu(bias), flags=flags)
    _v3_exact(z, bias, to_np(ids3), to_np(g3), k, n_group, topk_group, scale)
    assert int(to_np(flags)[0]) == 0, case
