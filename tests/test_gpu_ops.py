"""GPU parity of each C-ABI call against the CPU oracle, at sizes the oracle
finishes in seconds that still span several tiles and ragged tails, plus the
degenerate cases (empty inputs, capacity 0, invalid ids, NaN logits).

Integer outputs are compared bit-exactly; floating-point outputs by the
per-row relative error rule of ``tests/helpers.py`` (2e-2 against fp64)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle as O
from tests.helpers import as_f64, assert_rows_close, row_rel_err, to_gpu, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ge():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import grouped_expert_amd as ge
    return ge


def _bf16(a32):
    import workloads as W
    return W.f32_to_bf16_bits(a32)


# ---------------------------------------------------------------------------
# route
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (300, 8, 2), (257, 128, 8), (190, 384, 8), (70, 1024, 16),
                                   (64, 65, 5), (0, 16, 2)])
def test_route_topk(ge, T, E, k):
    rng = np.random.default_rng(T * 7 + E)
    z = rng.standard_normal((T, E)).astype(np.float32)
    if T > 10:
        z[:5] = np.round(z[:5])                      # ties
        z[5, : min(E, 3)] = -0.0
        z[6, :] = 0.0
        z[7, E // 2] = np.nan
        z[8, 0] = np.inf
    flags = ge.new_flags("cuda")
    ids, w = ge.route_topk(to_gpu(z), k, flags=flags)
    rid, rg, inv = O.route_topk(z, k)
    assert np.array_equal(to_np(ids), rid)
    gw = to_np(w).astype(np.float64)
    assert np.all(np.abs(gw - rg) <= 1e-5 * np.maximum(rg, 1e-30) + 1e-7)
    assert (int(to_np(flags)[0]) & 2 != 0) == bool(inv.any())


def _route_inputs(T, E, seed):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((T, E)).astype(np.float32)
    if T > 10:
        z[:3] = np.round(z[:3])                      # ties
        z[3, :] = 0.0
        z[4, E // 2] = np.nan
    return z


def _gates_close(gw, rg):
    gw = np.asarray(gw, dtype=np.float64)
    return np.all(np.abs(gw - rg) <= 1e-5 * np.abs(rg) + 1e-7)


@pytest.mark.parametrize("T,E,k", [(300, 64, 6), (257, 128, 8), (190, 384, 8), (40, 1024, 16), (1, 8, 2)])
def test_route_topk_v1(ge, T, E, k):
    z = _route_inputs(T, E, T + E)
    flags = ge.new_flags("cuda")
    ids, w = ge.route_topk(to_gpu(z), k, gating=ge.binding.MOE_GATING_SOFTMAX_TOPK, flags=flags)
    rid, rg, inv = O.route_v1(z, k)
    assert np.array_equal(to_np(ids), rid)
    assert _gates_close(to_np(w), rg)
    assert (int(to_np(flags)[0]) & 2 != 0) == bool(inv.any())


@pytest.mark.parametrize("T,E,k,ng,tg,scale", [(300, 160, 6, 8, 3, 16.0), (257, 64, 4, 4, 2, 1.0),
                                              (120, 256, 8, 8, 4, 2.0), (64, 1024, 16, 64, 5, 1.0),
                                              (33, 16, 3, 1, 1, 1.0),
                                              # 16 lanes per token: groups of 16, 32 and 64 experts
                                              (301, 256, 16, 16, 5, 1.0), (77, 128, 5, 8, 2, 2.0),
                                              (130, 256, 7, 4, 2, 1.0), (45, 128, 6, 4, 3, 1.0)])
def test_route_grouped_v2(ge, T, E, k, ng, tg, scale):
    z = _route_inputs(T, E, 3 * T + E)
    flags = ge.new_flags("cuda")
    ids, w = ge.route_topk_grouped(to_gpu(z), k, ge.binding.MOE_GATING_SOFTMAX_GROUP_LIMITED, ng, tg, scale,
                                   flags=flags)
    rid, rg, inv = O.route_v2(z, k, ng, tg, scale)
    assert np.array_equal(to_np(ids), rid)
    assert _gates_close(to_np(w), rg)
    assert (int(to_np(flags)[0]) & 2 != 0) == bool(inv.any())


def _v3_exact(z, bias, gids, gw, k, ng, tg, scale):
    """V3 ids must equal the oracle's exactly, token by token.  The one
    exception is a token holding a logit whose fp64 sigmoid lies within
    2^-45 of an fp32 rounding midpoint (the oracle names these): there the
    ids (and gates) must equal the oracle's under one of the two roundings of
    each such value.  Returns the excepted tokens."""
    z = np.asarray(z, np.float32)
    rid, rg, inv = O.route_v3(z, bias, k, ng, tg, scale)
    amb, other = O.sigmoid_f32_ambiguous(z)
    amb &= np.isfinite(z)
    named = np.nonzero(amb.any(axis=1))[0]
    plain = np.ones(z.shape[0], dtype=bool)
    plain[named] = False
    assert np.array_equal(gids[plain], rid[plain])
    assert _gates_close(gw[plain], rg[plain])
    base = O.sigmoid_f32(z)
    for t in named:
        cols = np.nonzero(amb[t])[0]
        assert cols.size <= 4, (t, cols)
        ok = False
        for m in range(1 << cols.size):
            s32 = base[t:t + 1].copy()
            for i, c in enumerate(cols):
                if (m >> i) & 1:
                    s32[0, c] = other[t, c]
            ids_t, g_t, _ = O.route_v3(z[t:t + 1], bias, k, ng, tg, scale, affinity32=s32)
            if np.array_equal(gids[t], ids_t[0]) and _gates_close(gw[t:t + 1], g_t):
                ok = True
                break
        assert ok, f"token {t}: ids {gids[t].tolist()} match neither rounding of logits {cols.tolist()}"
    return inv, named.tolist()


@pytest.mark.parametrize("T,E,k,ng,tg,scale", [(300, 256, 8, 8, 4, 2.5), (200, 64, 6, 8, 3, 1.0),
                                              (100, 384, 8, 16, 4, 2.5), (40, 12, 4, 4, 2, 2.5),
                                              # 16 lanes per token: groups of 16, 32 and 64 experts
                                              (257, 256, 16, 16, 6, 2.5), (99, 128, 8, 8, 4, 1.0),
                                              (150, 256, 8, 4, 2, 2.5), (61, 128, 3, 4, 1, 1.0)])
def test_route_grouped_v3(ge, T, E, k, ng, tg, scale):
    z = _route_inputs(T, E, 5 * T + E)
    bias = (0.05 * np.random.default_rng(E).standard_normal(E)).astype(np.float32)
    flags = ge.new_flags("cuda")
    ids, w = ge.route_topk_grouped(to_gpu(z), k, ge.binding.MOE_GATING_SIGMOID_BIAS_GROUP_TOP2, ng, tg, scale,
                                   bias=to_gpu(bias), flags=flags)
    inv, named = _v3_exact(z, bias, to_np(ids), to_np(w), k, ng, tg, scale)
    assert (int(to_np(flags)[0]) & 2 != 0) == bool(inv.any())
    if named:
        print(f"V3 tokens with an ambiguous fp32 affinity (either rounding accepted): {named}")


def test_route_grouped_page_tokens(ge, golden):
    g = golden("m62_gating_fixtures.json")
    f = g["v3_t0"]
    s = np.array(f["affinity"], dtype=np.float64)
    z = np.log(s / (1 - s)).astype(np.float32)[None, :]
    ids, w = ge.route_topk_grouped(to_gpu(z), f["k"], ge.binding.MOE_GATING_SIGMOID_BIAS_GROUP_TOP2, f["n_group"],
                                   f["topk_group"], f["route_scale"], bias=to_gpu(np.array(f["bias"], np.float32)))
    assert to_np(ids)[0].tolist() == f["experts"]
    assert np.allclose(to_np(w)[0], f["gates"], atol=2e-6)
    v = g["v2_t2"]
    zs = np.log(np.array([v["scores"]], dtype=np.float64)).astype(np.float32)
    ids2, _ = ge.route_topk_grouped(to_gpu(zs), v["k"], ge.binding.MOE_GATING_SOFTMAX_GROUP_LIMITED, v["n_group"],
                                    v["topk_group"], v["route_scale"])
    assert to_np(ids2)[0].tolist() == v["limited_top3"]


# ---------------------------------------------------------------------------
# permute
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T,k,E,cap,dt", [(256, 2, 8, -1, "f32"), (1000, 8, 128, -1, "bf16"),
                                          (999, 8, 128, 40, "bf16"), (64, 8, 384, -1, "bf16"),
                                          (3000, 4, 1024, 7, "bf16"), (500, 3, 5, 0, "bf16"),
                                          (0, 2, 4, -1, "bf16"), (40000, 8, 64, 4000, "bf16")])
def test_permute(ge, T, k, E, cap, dt):
    rng = np.random.default_rng(T + E + k)
    d = 64
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    if T > 20:
        ids[3, 0] = -1
        ids[4, 1] = E + 3
        ids[5, 0] = -7
    x32 = rng.standard_normal((T, d)).astype(np.float32)
    x = x32 if dt == "f32" else _bf16(x32)
    flags = ge.new_flags("cuda")
    out = ge.permute(to_gpu(x) if T else torch.empty((0, d), device="cuda", dtype=torch.float32 if dt == "f32"
                                                    else torch.bfloat16),
                     to_gpu(ids) if T else torch.empty((0, k), dtype=torch.int32, device="cuda"),
                     E, cap, flags=flags)
    plan = O.dispatch_plan(ids, E, cap)
    assert to_np(out["sel"]).tolist() == plan.sel.tolist()
    assert to_np(out["counts"]).tolist() == plan.counts.tolist()
    assert to_np(out["offsets"]).tolist() == plan.offsets.tolist()
    assert to_np(out["inv"]).tolist() == plan.inv.tolist()
    assert to_np(out["src"]).tolist() == plan.src.tolist()
    assert int(to_np(out["dropped"])[0]) == plan.dropped
    A = plan.accepted
    xp = to_np(out["x_perm"])[:A]
    assert np.array_equal(xp, O.gather_rows(x, plan.src, k, A))
    assert (int(to_np(flags)[0]) & 1 != 0) == bool(plan.bad.any())


# ---------------------------------------------------------------------------
# grouped SwiGLU
# ---------------------------------------------------------------------------

def _segments(rng, E, rows, mode):
    if mode == "packed":
        counts = rng.multinomial(rows, rng.dirichlet(np.ones(E) * 0.3))
        counts[rng.integers(0, E)] = 0
        starts = np.concatenate([[0], np.cumsum(counts)[:-1]])
    else:   # static arrays with gaps
        cap = rows // E
        counts = rng.integers(0, cap + 1, size=E)
        counts[0] = cap
        starts = np.arange(E) * cap
    return starts.astype(np.int32), counts.astype(np.int32)


@pytest.mark.parametrize("E,rows,d,d_ff,dt,zdt,mode", [
    (8, 512, 128, 256, "f32", "f32", "packed"),
    (6, 900, 256, 128, "bf16", "f32", "static"),
    (5, 700, 128, 192, "bf16", "bf16", "packed"),
    (16, 300, 384, 64, "bf16", "bf16", "packed"),
    (3, 1, 128, 64, "bf16", "f32", "packed"),
    (2, 2100, 128, 128, "bf16", "f32", "static"),       # >= 768 rows per expert: 256-row tiles
    (3, 2400, 192, 256, "bf16", "bf16", "packed"),     # 256-row tiles, odd slice count (d / 64 = 3)
    (2, 1700, 320, 192, "bf16", "f32", "static"),      # 256-row tiles, odd slice counts, partial N-tiles
    # 256-row tiles with 6 slices per down tile and more tiles than CUs: the
    # persistent register-staged down kernel, several tiles per workgroup,
    # ragged segment ends and a partial last N-tile
    (3, 70000, 320, 384, "bf16", "f32", "static"),
    # both launches persistent (d / 64 = 6 gate/up slices), a partial last
    # down N-tile
    (3, 70000, 384, 384, "bf16", "f32", "static"),
    # persistent gate/up tiles with a partial last N-tile (d_ff = 448)
    (2, 60000, 384, 448, "bf16", "bf16", "packed"),
    # 128-row tiles with K / 64 a multiple of 4 and at least 6 for both
    # products: the weight rows through four register stages, persistent;
    # several tiles per workgroup in the second case.  (d = 256, 4 slices,
    # is below the weight loads' lead: the DMA-ring tiles.)
    (8, 2000, 512, 512, "bf16", "f32", "packed"),
    (64, 40000, 512, 512, "bf16", "bf16", "packed"),
    (64, 40000, 256, 512, "bf16", "bf16", "packed"),
])
def test_grouped_swiglu(ge, E, rows, d, d_ff, dt, zdt, mode):
    rng = np.random.default_rng(rows + E)
    starts, counts = _segments(rng, E, rows, mode)
    x32 = rng.standard_normal((rows, d)).astype(np.float32)
    ws = [(0.05 * rng.standard_normal(s)).astype(np.float32) for s in
          [(E, d_ff, d), (E, d_ff, d), (E, d, d_ff)]]
    if dt == "bf16":
        x = _bf16(x32)
        ws = [_bf16(w) for w in ws]
    else:
        x = x32
    zt = torch.float32 if zdt == "f32" else torch.bfloat16
    z0 = torch.zeros((rows, d), dtype=zt, device="cuda")
    flags = ge.new_flags("cuda")
    z = ge.grouped_swiglu(to_gpu(x), to_gpu(starts), to_gpu(counts), *[to_gpu(w) for w in ws], z=z0, flags=flags)
    bank = O.swiglu_bank(lambda e: (ws[0][e], ws[1][e], ws[2][e]))
    want = O.run_segments(x, starts, counts, bank)
    got = as_f64(z)
    covered = np.zeros(rows, bool)
    for s, c in zip(starts, counts):
        covered[s:s + c] = True
    assert_rows_close(got[covered], want[covered], what="swiglu")
    assert np.all(got[~covered] == 0)
    assert int(to_np(flags)[0]) == 0


@pytest.mark.parametrize("E,rows,d,d_ff,dt,zdt,mode", [
    (8, 512, 128, 256, "f32", "f32", "packed"),          # fp32 FMA path
    (16, 300, 384, 64, "bf16", "bf16", "packed"),        # 32-row tiles
    (5, 700, 128, 192, "bf16", "f32", "packed"),         # 128-row tiles
    (2, 2100, 128, 128, "bf16", "f32", "static"),        # 256-row tiles, direct fp32 stores
    (3, 2400, 192, 256, "bf16", "bf16", "packed"),       # 256-row tiles, stores staged through LDS
    (3, 70000, 320, 384, "bf16", "f32", "packed"),       # persistent register-staged down tiles
    (3, 70000, 384, 384, "bf16", "f32", "packed"),       # both launches persistent
    (8, 2000, 512, 512, "bf16", "f32", "packed"),        # 128-row register-staged tiles, fp32 through the map
    (64, 40000, 512, 768, "bf16", "bf16", "static"),     # the same, bf16, several tiles per workgroup
])
def test_grouped_swiglu_row_map(ge, E, rows, d, d_ff, dt, zdt, mode):
    """With z_rows, row i of the result lands in z row z_rows[i]: the rows
    equal the unmapped call's bit for bit (and the oracle's within the
    tolerance); rows mapped to -1 or past the end of z are not stored, and
    z rows no segment row maps to keep their contents."""
    rng = np.random.default_rng(rows + 7 * E)
    starts, counts = _segments(rng, E, rows, mode)
    x32 = rng.standard_normal((rows, d)).astype(np.float32)
    ws = [(0.05 * rng.standard_normal(s)).astype(np.float32) for s in
          [(E, d_ff, d), (E, d_ff, d), (E, d, d_ff)]]
    if dt == "bf16":
        x = _bf16(x32)
        ws = [_bf16(w) for w in ws]
    else:
        x = x32
    zt = torch.float32 if zdt == "f32" else torch.bfloat16
    n_out = rows + 37
    zmap = rng.permutation(n_out)[:rows].astype(np.int32)
    zmap[rng.choice(rows, size=rows // 10, replace=False)] = -1
    zmap[rng.choice(rows, size=rows // 20, replace=False)] = n_out + 5       # out of range: dropped
    gw = [to_gpu(w) for w in ws]
    flags = ge.new_flags("cuda")
    plain = ge.grouped_swiglu(to_gpu(x), to_gpu(starts), to_gpu(counts), *gw,
                              z=torch.zeros((rows, d), dtype=zt, device="cuda"), flags=flags)
    mapped = torch.full((n_out, d), 7.0, dtype=zt, device="cuda")
    ge.grouped_swiglu(to_gpu(x), to_gpu(starts), to_gpu(counts), *gw, z=mapped, z_rows=to_gpu(zmap), flags=flags)
    torch.cuda.synchronize()
    assert int(to_np(flags)[0]) == 0
    covered = np.zeros(rows, bool)
    for s0, c in zip(starts, counts):
        covered[s0:s0 + c] = True
    live = covered & (zmap >= 0) & (zmap < n_out)
    got, ref = as_f64(mapped), as_f64(plain)
    assert np.array_equal(got[zmap[live]], ref[live])
    untouched = np.ones(n_out, bool)
    untouched[zmap[live]] = False
    assert np.all(got[untouched] == 7.0)
    want = O.run_segments(x, starts, counts, O.swiglu_bank(lambda e: (ws[0][e], ws[1][e], ws[2][e])))
    assert_rows_close(got[zmap[live]], want[live], what="swiglu through the row map")


def test_grouped_swiglu_bad_segment_flag(ge):
    rng = np.random.default_rng(1)
    E, rows, d, d_ff = 3, 256, 128, 64
    x = _bf16(rng.standard_normal((rows, d)).astype(np.float32))
    ws = [_bf16((0.05 * rng.standard_normal(s)).astype(np.float32)) for s in
          [(E, d_ff, d), (E, d_ff, d), (E, d, d_ff)]]
    starts = np.array([0, 100, 250], np.int32)
    counts = np.array([100, 100, 50], np.int32)      # last one overruns rows
    flags = ge.new_flags("cuda")
    z = ge.grouped_swiglu(to_gpu(x), to_gpu(starts), to_gpu(counts), *[to_gpu(w) for w in ws],
                          z=torch.zeros((rows, d), dtype=torch.float32, device="cuda"), flags=flags)
    assert int(to_np(flags)[0]) & 16
    counts_ok = counts.copy()
    counts_ok[2] = 0
    want = O.run_segments(x, starts, counts_ok, O.swiglu_bank(lambda e: (ws[0][e], ws[1][e], ws[2][e])))
    assert_rows_close(as_f64(z)[:200], want[:200], what="swiglu")
    assert np.all(as_f64(z)[200:] == 0)


# ---------------------------------------------------------------------------
# combine
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T,k,d,zdt,window,acc", [(100, 2, 128, "f32", None, False),
                                                  (333, 8, 2048, "bf16", None, True),
                                                  (50, 1, 3072, "f32", (40, 90), False),
                                                  (0, 4, 64, "bf16", None, False),
                                                  (77, 8, 24, "bf16", (10, 200), True)])
def test_unpermute_combine(ge, T, k, d, zdt, window, acc):
    rng = np.random.default_rng(T + d)
    nz = 256
    z32 = rng.standard_normal((nz, d)).astype(np.float32)
    z = z32 if zdt == "f32" else _bf16(z32)
    idx = rng.integers(-1, nz, size=T * k).astype(np.int32)
    g = rng.random(T * k).astype(np.float32)
    lo, hi = window if window else (0, nz)
    y0 = rng.standard_normal((T, d)).astype(np.float32)
    flags = ge.new_flags("cuda")
    zt = to_gpu(z[lo:hi] if window else z)
    y = to_gpu(y0.copy()) if acc else None
    out = ge.unpermute_combine(zt, to_gpu(idx) if T else torch.empty(0, dtype=torch.int32, device="cuda"),
                               to_gpu(g) if T else None, T, k, lo=lo, hi=hi, y=y, accumulate=acc, flags=flags)
    want = O.combine(z[lo:hi], idx, g, T, k, lo=lo, hi=hi, y=y0.astype(np.float64).copy() if acc else None)
    if T:
        assert_rows_close(to_np(out), want, tol=1e-5, what="combine")
    assert int(to_np(flags)[0]) == 0


@pytest.mark.parametrize("zdt,rdt", [("f32", "f32"), ("bf16", "bf16"), ("f32", "bf16"), ("bf16", "f32")])
@pytest.mark.parametrize("n,nz,d", [(1000, 300, 3072), (77, 5, 8), (3, 0, 64), (0, 4, 16)])
def test_expand_rows(ge, zdt, rdt, n, nz, d):
    """Expansion of static-array rows to pool rows: a copy (exact), a widening
    (exact) or a rounding to bf16 (nearest even, bit-exact)."""
    rng = np.random.default_rng(n + nz + d)
    z32 = rng.standard_normal((max(nz, 1), d)).astype(np.float32)[:nz]
    z = z32 if zdt == "f32" else _bf16(z32)
    slot = rng.integers(-1, max(nz, 1), size=n).astype(np.int32) if nz else np.full(n, -1, np.int32)
    flags = ge.new_flags("cuda")
    zt = to_gpu(z) if nz else torch.empty((0, d), dtype=torch.float32 if zdt == "f32" else torch.bfloat16,
                                          device="cuda")
    st = to_gpu(slot) if n else torch.empty(0, dtype=torch.int32, device="cuda")
    ret = ge.expand_rows(zt, st, ret_dtype=torch.float32 if rdt == "f32" else torch.bfloat16, flags=flags)
    want = O.expand_rows(z if nz else np.zeros((0, d), np.float32), slot.astype(np.int64))
    got = to_np(ret)
    assert got.shape == (n, d) and int(to_np(flags)[0]) == 0
    if rdt == "bf16":
        assert np.array_equal(got, _bf16(want.astype(np.float32)))      # nearest-even of an exact value
    else:
        assert np.array_equal(got.astype(np.float64), want)


def test_expand_rows_bad_slot_flag(ge):
    z = to_gpu(np.ones((4, 8), np.float32))
    flags = ge.new_flags("cuda")
    ret = ge.expand_rows(z, to_gpu(np.array([0, -5, 4, 3, -1], np.int32)), ret_dtype=torch.bfloat16, flags=flags)
    assert int(to_np(flags)[0]) == 8
    assert (as_f64(ret) == np.array([[1.0] * 8, [0.0] * 8, [0.0] * 8, [1.0] * 8, [0.0] * 8])).all()


def test_combine_bad_index_flag(ge):
    z = to_gpu(np.ones((4, 8), np.float32))
    idx = to_gpu(np.array([0, -5, 1, 2], np.int32))
    flags = ge.new_flags("cuda")
    y = ge.unpermute_combine(z, idx, None, 2, 2, flags=flags)
    assert int(to_np(flags)[0]) == 8
    assert to_np(y).tolist() == [[1.0] * 8, [2.0] * 8]


# ---------------------------------------------------------------------------
# pooled-wave pack and receiver compaction
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T,k,epd,D,W,P,d,wave", [(200, 4, 6, 8, 3, 40, 64, -1),
                                                  (500, 8, 3, 16, 2, 100, 128, -1),
                                                  (500, 8, 3, 16, 2, 100, 128, 1),
                                                  (64, 2, 1, 4, 1, 0, 8, -1),
                                                  (0, 2, 2, 3, 3, 5, 8, -1),
                                                  (3000, 8, 6, 64, 3, 30, 64, 2),
                                                  (400, 4, 3, 8, 2, 30, 8, -1),      # four header rows
                                                  (3000, 8, 6, 16, 2, 150, 64, 1),   # three header rows
                                                  (900, 8, 2, 8, 2, 129, 128, -1)])  # two, second one 1 id
def test_pool_pack(ge, T, k, epd, D, W, P, d, wave):
    rng = np.random.default_rng(T + D + P)
    E = D * epd
    z = rng.standard_normal((max(T, 1), E)).astype(np.float32)[:T]
    z[:, :epd] += 1.5
    ids = O.route_topk(z, k)[0] if T else np.zeros((0, k), np.int32)
    if T > 10:
        ids[2, 0] = -1
        ids[3, 1] = E + 5
    x = _bf16(rng.standard_normal((T, d)).astype(np.float32))
    flags = ge.new_flags("cuda")
    out = ge.pool_pack(to_gpu(x) if T else torch.empty((0, d), dtype=torch.bfloat16, device="cuda"),
                       to_gpu(ids) if T else torch.empty((0, k), dtype=torch.int32, device="cuda"),
                       E, epd, D, W, P, wave=wave, flags=flags)
    pk = O.pool_pack(x, ids, epd, D, W, P)
    want_pools = pk["pools"] if wave < 0 else pk["pools"][wave]
    assert np.array_equal(to_np(out["pools"]), want_pools)
    assert to_np(out["route_loc"]).tolist() == pk["route_loc"].tolist()
    assert to_np(out["dest_counts"]).tolist() == pk["dest_counts"].tolist()
    assert int(to_np(out["sender_dropped"])[0]) == pk["sender_dropped"]
    assert (int(to_np(flags)[0]) & 1 != 0) == bool(pk["bad"].any())


@pytest.mark.parametrize("S,P,d,L,cap,rot", [(8, 40, 64, 6, 30, 0), (64, 100, 128, 6, 700, 0), (5, 6, 8, 3, 0, 0),
                                             (3, 0, 8, 2, 4, 0), (40, 200, 256, 17, 100, 0),
                                             (8, 40, 64, 6, 30, 5),             # rotated source order
                                             (7, 30, 8, 3, 25, 6),              # four header rows, rotated
                                             (33, 129, 128, 6, 300, 1),         # two header rows
                                             (1, 20, 8, 2, 3, 0)])
def test_recv_compact(ge, S, P, d, L, cap, rot):
    rng = np.random.default_rng(S * P + L + rot)
    H = O.header_rows(P, d)
    pools = rng.integers(0, 2 ** 16, size=(S, P + H, d)).astype(np.uint16)
    p = (np.arange(1, L + 1) ** -1.1)
    hdr = rng.choice(L, size=(S, P), p=p / p.sum()).astype(np.uint16)
    if P > 3:
        hdr[1 % S, 2] = 0xFFFF
        hdr[0, 3] = L + 1                         # bad id
    flat = np.full((S, H * d), 0xFFFF, dtype=np.uint16)
    flat[:, :P] = hdr
    pools[:, :H, :] = flat.reshape(S, H, d)
    flags = ge.new_flags("cuda")
    compact0 = torch.zeros((L, cap, d), dtype=torch.bfloat16, device="cuda")
    out = ge.recv_compact(to_gpu(pools), L, cap, compact=compact0, flags=flags, rotation=rot)
    rc = O.recv_compact(pools, L, cap, rotation=rot)
    assert np.array_equal(to_np(out["compact"]), rc["compact"])
    assert to_np(out["counts"]).tolist() == rc["counts"].tolist()
    assert to_np(out["arrived"]).tolist() == rc["arrived"].tolist()
    assert to_np(out["row_slot"]).tolist() == rc["row_slot"].tolist()
    assert int(to_np(out["recv_dropped"])[0]) == rc["recv_dropped"]
    assert (int(to_np(flags)[0]) & 4 != 0) == (rc["bad_header"] > 0)
    # the same call with the slot map and the return rows of the fused receiver
    for rdt in (torch.float32, torch.bfloat16):
        ret = torch.full((S * (P + H), d), 3.0, dtype=rdt, device="cuda")
        slot_row = torch.full((L * cap,), -7, dtype=torch.int32, device="cuda")
        out2 = ge.recv_compact(to_gpu(pools), L, cap, compact=compact0, rotation=rot, slot_row=slot_row, ret=ret)
        row_slot = rc["row_slot"]
        assert to_np(out2["row_slot"]).tolist() == row_slot.tolist()
        want = np.full(L * cap, -7, dtype=np.int64)
        acc = np.nonzero(row_slot >= 0)[0]
        want[row_slot[acc]] = acc                               # the inverse of row_slot
        assert to_np(slot_row).tolist() == want.tolist()
        r = as_f64(ret)
        assert np.all(r[row_slot < 0] == 0) and np.all(r[row_slot >= 0] == 3.0)


# ---------------------------------------------------------------------------
# chained: identity check through permute + combine (no GEMM)
# ---------------------------------------------------------------------------

def test_permute_combine_identity(ge):
    """combine(permute(x)) with Z = X_perm and renormalised gates gives x
    back; with a capacity it gives the kept gate mass times x."""
    rng = np.random.default_rng(4)
    T, E, k, d = 1500, 32, 4, 256
    z = rng.standard_normal((T, E)).astype(np.float32)
    x32 = rng.standard_normal((T, d)).astype(np.float32)
    x = to_gpu(x32)
    for cap in (-1, 150):
        ids, g = ge.route_topk(to_gpu(z), k)
        plan = ge.permute(x, ids, E, cap)
        y = ge.unpermute_combine(plan["x_perm"], plan["inv"], g, T, k)
        keep = (to_np(plan["inv"]) >= 0).reshape(T, k)
        mass = (to_np(g).astype(np.float64) * keep).sum(1)
        assert row_rel_err(to_np(y), mass[:, None] * x32) < 1e-5
