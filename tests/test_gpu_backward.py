"""GPU parity of the backward of the transpose against the fp64 oracle.

Route and gate gradients (moe_combine_backward), the expert backward over
ragged segments (moe_grouped_swiglu_backward: route-input and weight
gradients) and the whole layer backward, at sizes that span several tiles
of every tiling with ragged tails, empty experts and dropped routes.

Tolerances: rows compare with the 2e-2 per-row relative rule; a value that
is a single product rounded to bf16 is within 2^-8 of it; a gate gradient
is a dot product of d terms whose z factor is rounded to bf16 at most once,
so its error is below 2^-8 * sum |dy_i z_i| (4e-3 used)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle as O
import workloads as W
from tests.helpers import as_f64, assert_rows_close, to_gpu, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ge():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import grouped_expert_amd as ge
    return ge


def _bf16(a32):
    return W.f32_to_bf16_bits(a32)


def _segments(rng, E, rows, mode):
    if mode == "packed":
        counts = rng.multinomial(rows, rng.dirichlet(np.ones(E) * 0.3)) if rows else np.zeros(E, np.int64)
        if rows:
            counts[rng.integers(0, E)] = 0
        starts = np.concatenate([[0], np.cumsum(counts)[:-1]])
    else:   # static arrays with gaps
        cap = rows // E
        counts = rng.integers(0, cap + 1, size=E)
        counts[0] = cap
        starts = np.arange(E) * cap
    return starts.astype(np.int32), counts.astype(np.int32)


def _dot_bound(dy, z, idx, T, k):
    """sum_i |dy[t, i] z[p, i]| per route (0 where no row)."""
    idx = np.asarray(idx).reshape(T, k)
    out = np.zeros((T, k))
    for j in range(k):
        t = np.nonzero(idx[:, j] >= 0)[0]
        out[t, j] = np.abs(dy[t] * z[idx[t, j]]).sum(axis=1)
    return out


@pytest.mark.parametrize("T,k,d,zdt,dzdt", [(300, 4, 256, "bf16", "bf16"), (77, 8, 2048, "bf16", "f32"),
                                            (50, 2, 3072, "f32", "bf16"), (130, 1, 64, "f32", "f32"),
                                            (0, 2, 64, "bf16", "bf16")])
def test_combine_backward(ge, T, k, d, zdt, dzdt):
    rng = np.random.default_rng(T + d + k)
    rows = T * k
    perm = rng.permutation(rows)
    idx = perm.astype(np.int32)
    if T > 4:
        idx[rng.choice(rows, size=rows // 7, replace=False)] = -1      # dropped routes
    z32 = rng.standard_normal((rows, d)).astype(np.float32)
    z = z32 if zdt == "f32" else _bf16(z32)
    g = rng.random(rows).astype(np.float32)
    dy = rng.standard_normal((T, d)).astype(np.float32)
    flags = ge.new_flags("cuda")
    dz0 = torch.zeros((rows, d), dtype=torch.float32 if dzdt == "f32" else torch.bfloat16, device="cuda")
    mk = lambda a, dt: to_gpu(a) if a.size else torch.empty(a.shape, dtype=dt, device="cuda")
    dz, dg = ge.combine_backward(mk(dy, torch.float32), mk(z, torch.float32 if zdt == "f32" else torch.bfloat16),
                                 mk(idx, torch.int32), mk(g, torch.float32), k, dz=dz0, flags=flags)
    want_dz, want_dg = O.combine_backward(dy, z, idx, g, T, k)
    assert int(to_np(flags)[0]) == 0
    got_dz = as_f64(dz)
    live = np.zeros(rows, bool)
    live[idx[idx >= 0]] = True
    if dzdt == "f32":
        assert np.allclose(got_dz[live], want_dz[live], rtol=1e-6, atol=0)
    else:
        assert np.all(np.abs(got_dz[live] - want_dz[live]) <= 2.0 ** -8 * np.abs(want_dz[live]))
    assert np.all(got_dz[~live] == 0)                                  # rows no route points to: untouched
    bound = _dot_bound(dy.astype(np.float64), O.to_f64(z), idx, T, k)
    assert np.all(np.abs(to_np(dg).astype(np.float64) - want_dg) <= 1e-5 * bound + 1e-30)
    assert np.all(to_np(dg)[idx.reshape(T, k) < 0] == 0)


def test_combine_backward_bad_index_flag(ge):
    z = to_gpu(_bf16(np.ones((4, 8), np.float32)))
    idx = to_gpu(np.array([0, -5, 3, 9], np.int32))
    flags = ge.new_flags("cuda")
    dz, dg = ge.combine_backward(to_gpu(np.ones((2, 8), np.float32)), z, idx,
                                 to_gpu(np.full(4, 0.5, np.float32)), 2, flags=flags)
    assert int(to_np(flags)[0]) == 8
    assert to_np(dg).tolist() == [[8.0, 0.0], [8.0, 0.0]]


@pytest.mark.parametrize("saved", [False, True])
@pytest.mark.parametrize("E,rows,d,d_ff,mode,dxdt", [
    (5, 700, 128, 192, "packed", "f32"),       # 128-row tiles
    (16, 300, 384, 64, "packed", "bf16"),      # 32-row tiles
    (3, 1, 128, 64, "packed", "f32"),
    (3, 0, 128, 64, "packed", "f32"),          # no rows: every weight gradient zero
    (2, 2100, 128, 128, "static", "f32"),      # 256-row tiles, segments with gaps
    (3, 2400, 192, 256, "packed", "bf16"),     # 256-row tiles, odd slice count
    (2, 1700, 320, 192, "static", "f32"),      # partial M- and N-tiles everywhere
])
def test_grouped_swiglu_backward(ge, E, rows, d, d_ff, mode, dxdt, saved):
    """Expert backward against the oracle, with G, U and H recomputed, or
    (saved) taken from the activations a forward call of the same rows and
    segments saved; that forward's z must not change when it saves them."""
    rng = np.random.default_rng(rows + E + d)
    starts, counts = _segments(rng, E, rows, mode)
    x = _bf16(rng.standard_normal((rows, d)).astype(np.float32))
    dz = _bf16(rng.standard_normal((rows, d)).astype(np.float32))
    ws = [_bf16((0.05 * rng.standard_normal(s)).astype(np.float32)) for s in
          [(E, d_ff, d), (E, d_ff, d), (E, d, d_ff)]]
    flags = ge.new_flags("cuda")
    dx0 = torch.zeros((rows, d), dtype=torch.float32 if dxdt == "f32" else torch.bfloat16, device="cuda")
    mk = lambda a: to_gpu(a) if a.size else torch.empty((0, d), dtype=torch.bfloat16, device="cuda")
    gws = [to_gpu(w) for w in ws]
    act = None
    if saved and rows > 0:
        act = ge.new_act(rows, d_ff, "cuda")
        z_plain = ge.grouped_swiglu(mk(x), to_gpu(starts), to_gpu(counts), *gws, z_dtype=torch.float32,
                                    z=torch.zeros((rows, d), dtype=torch.float32, device="cuda"), flags=flags)
        z_saved = ge.grouped_swiglu(mk(x), to_gpu(starts), to_gpu(counts), *gws, z_dtype=torch.float32,
                                    z=torch.zeros((rows, d), dtype=torch.float32, device="cuda"), flags=flags,
                                    act=act)
        assert torch.equal(z_plain, z_saved)
    out = ge.grouped_swiglu_backward(mk(x), mk(dz), to_gpu(starts), to_gpu(counts), *gws,
                                     dx=dx0, flags=flags, act=act)
    torch.cuda.synchronize()
    assert int(to_np(flags)[0]) == 0
    bwd = O.swiglu_bank_backward(lambda e: (ws[0][e], ws[1][e], ws[2][e]))
    want_dx, grads = O.run_segments_backward(x, O.to_f64(dz), starts, counts, bwd)
    covered = np.zeros(rows, bool)
    for s, c in zip(starts, counts):
        covered[s:s + c] = True
    got_dx = as_f64(out["dx"])
    if covered.any():
        assert_rows_close(got_dx[covered], want_dx[covered], what="route-input gradient")
    assert np.all(got_dx[~covered] == 0)
    if act is not None:
        _check_saved_planes(act, x, ws, starts, counts, d_ff)
    for e in range(E):
        for name, i in (("dw_gate", 0), ("dw_up", 1), ("dw_down", 2)):
            got = to_np(out[name][e]).astype(np.float64)
            if grads[e] is None:
                assert np.all(got == 0), (e, name)
            elif act is not None and name == "dw_gate":
                s, c = starts[e], counts[e]
                _check_dw_gate_saved(got, grads[e][0], O.to_f64(x[s:s + c]), O.to_f64(dz[s:s + c]),
                                     *(O.to_f64(w[e]) for w in ws))
            else:
                assert_rows_close(got, grads[e][i], what=f"{name}[{e}]")


def _expert_terms(xe, wg, wu):
    """fp64 G, U of an expert's rows, with the sums of magnitudes that bound
    their fp32 accumulation."""
    return xe @ wg.T, xe @ wu.T, np.abs(xe) @ np.abs(wg.T), np.abs(xe) @ np.abs(wu.T)


def _check_saved_planes(act, x, ws, starts, counts, d_ff):
    """The saved planes hold bf16 G | U (one rounding to 8 significant bits of
    an fp32 sum: within 2^-8 of the value, plus the fp32 accumulation error,
    below 1e-4 of the sum of magnitudes at these depths) and bf16
    H = silu(G) U (one rounding of the fp32 product, whose factors carry the
    accumulation errors; |silu'| < 1.1)."""
    rows = x.shape[0]
    a = as_f64(act)
    GU = a[:rows * 2 * d_ff].reshape(rows, 2 * d_ff)
    H = a[rows * 2 * d_ff:].reshape(rows, d_ff)
    for e, (s, c) in enumerate(zip(starts, counts)):
        if c == 0:
            continue
        g, u, ag, au = _expert_terms(O.to_f64(x[s:s + c]), O.to_f64(ws[0][e]), O.to_f64(ws[1][e]))
        for what, got, want, mag in (("G", GU[s:s + c, :d_ff], g, ag), ("U", GU[s:s + c, d_ff:], u, au)):
            r = np.abs(got - want) / (2.0 ** -8 * np.abs(want) + 1e-4 * mag)
            i, j = np.unravel_index(np.argmax(r), r.shape)
            assert r[i, j] <= 1, (what, e, s + i, j, got[i, j], want[i, j], int((r > 1).sum()))
        h = O.silu(g) * u
        hb = (2.0 ** -8 + 1e-5) * np.abs(h) + 1e-4 * (1.1 * ag * np.abs(u) + au * np.abs(O.silu(g)) + 1.1 * ag * au)
        assert np.all(np.abs(H[s:s + c] - h) <= hb), e


def _check_dw_gate_saved(got, want, xe, dze, wg, wu, wd, dz_rounded=False):
    """dW_g from saved bf16 G: dG = dH U silu'(G) with silu' evaluated at the
    rounded G, whose error 2^-8 |G| moves silu' by at most 2^-9 |G| (|silu''|
    <= 1/2); dH, U and dG itself are rounded to bf16 once each (2^-8 each).
    So per element |dG - dG*| <= 2^-6 |dG*| + 2^-8 |dH U G| (both twice
    what is needed for margin), and
    |dW_g - dW_g*|[j, i] <= sum_r |x[r, i]| that bound.  Near silu'(g) = 0 the
    second term is not small against dG itself, which makes the row rule unfit
    for experts of a row or two.  With dz_rounded the route gradients were
    rounded to bf16 once more (2^-8 of sum |dZ| |W_d| added to dH's error)."""
    g, u, ag, au = _expert_terms(xe, wg, wu)
    dh = dze @ wd
    dg = dh * u * O.silu_grad(g)
    per = 2.0 ** -6 * np.abs(dg) + 2.0 ** -8 * np.abs(dh * u * g) + 1e-4 * np.abs(dh) * (ag + au)
    if dz_rounded:
        per += 2.0 ** -8 * (np.abs(dze) @ np.abs(wd)) * np.abs(u * O.silu_grad(g))
    bound = per.T @ np.abs(xe)
    assert np.all(np.abs(got - want) <= bound + 1e-30), e


@pytest.mark.parametrize("save_act", [False, True])
@pytest.mark.parametrize("T,E,k,d,d_ff,cap", [(300, 16, 4, 256, 128, -1), (700, 8, 2, 128, 192, 150),
                                              (64, 32, 8, 192, 64, -1)])
def test_layer_backward(ge, T, E, k, d, d_ff, cap, save_act):
    """Layer backward from the forward's saved state against the oracle:
    token gradients, gate gradients (0 for dropped routes) and every
    expert's weight gradients; with save_act the forward also saved the
    experts' activations and the backward reads them."""
    rng = np.random.default_rng(T + E)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    x = _bf16(rng.standard_normal((T, d)).astype(np.float32))
    ws = [_bf16((0.05 * rng.standard_normal(s)).astype(np.float32)) for s in
          [(E, d_ff, d), (E, d_ff, d), (E, d, d_ff)]]
    dy = rng.standard_normal((T, d)).astype(np.float32)
    flags = ge.new_flags("cuda")
    gw = [to_gpu(w) for w in ws]
    y, st = ge.moe_layer(to_gpu(x), to_gpu(logits), *gw, k, cap, flags=flags, save_act=save_act)
    assert (st["act"] is not None) == save_act
    dx, gr = ge.moe_layer_backward(to_gpu(dy), to_gpu(x), st, *gw, flags=flags)
    torch.cuda.synchronize()
    assert int(to_np(flags)[0]) == 0
    ids, gates, _ = O.route_topk(logits, k)
    assert np.array_equal(to_np(st["ids"]), ids)
    bank = O.swiglu_bank(lambda e: (ws[0][e], ws[1][e], ws[2][e]))
    bwd = O.swiglu_bank_backward(lambda e: (ws[0][e], ws[1][e], ws[2][e]))
    want = O.moe_layer_backward(x, ids, gates.astype(np.float64), bank, bwd, E, dy.astype(np.float64), cap)
    assert np.array_equal(to_np(st["plan"]["inv"]), want["plan"].inv)
    if cap > 0:
        assert want["plan"].dropped > 0
    assert_rows_close(to_np(dx), want["dx"], what="token gradient")
    bound = _dot_bound(dy.astype(np.float64), want["z"], want["plan"].inv, T, k)
    assert np.all(np.abs(to_np(gr["dgates"]).astype(np.float64) - want["dgates"]) <= 4e-3 * bound + 1e-30)
    xp = O.gather_rows(x, want["plan"].src, k, want["plan"].accepted)
    for e in range(E):
        for name, i in (("dw_gate", 0), ("dw_up", 1), ("dw_down", 2)):
            got = to_np(gr[name][e]).astype(np.float64)
            if want["grads"][e] is None:
                assert np.all(got == 0), (e, name)
            elif save_act and name == "dw_gate":
                s, c = want["plan"].offsets[e], want["plan"].counts[e]
                _check_dw_gate_saved(got, want["grads"][e][0], O.to_f64(xp[s:s + c]), want["dz"][s:s + c],
                                     *(O.to_f64(w[e]) for w in ws), dz_rounded=True)
            else:
                assert_rows_close(got, want["grads"][e][i], what=f"{name}[{e}]")
