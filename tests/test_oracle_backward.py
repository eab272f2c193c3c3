"""Pins of the oracle's backward of the transpose (CPU only).

The page's toy values (M6.2 §0x03D), a direct token-major evaluation written
out route by route, central finite differences of the forward oracle, and a
closed form at width one.  Mutation checks plant plausible mistakes in the
oracle (on the CPU) and show that these pins catch them."""
import numpy as np
import pytest

import oracle as O
import oracle.moe_oracle as OM


def _toy(golden):
    f = golden("m62_logical_transpose_fixture.json")
    x = np.array(f["hidden"], dtype=np.float64)
    k = f["k"]
    ids = np.array(f["expert"], dtype=np.int64).reshape(-1, k)
    gates = np.array(f["gate"], dtype=np.float64).reshape(-1, k)
    return x, ids, gates, f["scalar_expert"]


def test_toy_backward_matches_page(golden):
    """M6.2 §0x03D: all-ones upstream gradient on the 0x03A toy."""
    want = golden("m62_backward_fixture.json")
    x, ids, gates, s = _toy(golden)
    out = O.moe_layer_backward(x, ids, gates, O.scalar_bank(s), O.scalar_bank_backward(s), len(s),
                               np.ones_like(x))
    assert np.allclose(out["dgates"].reshape(-1), want["expected_gate_grad"], rtol=0, atol=1e-12)
    assert np.allclose([g[0] for g in out["grads"]], want["expected_expert_scalar_grad"], rtol=0, atol=1e-12)
    fac = np.array(want["expected_token_grad_factor"])
    assert np.allclose(out["dx"], fac[:, None] * np.ones((1, 3)), rtol=0, atol=1e-12)


def test_toy_direct_equals_transposed(golden):
    """M6.2 §0x03D: the direct (token-major) and transposed token gradients
    agree; written out route by route with a random upstream gradient."""
    x, ids, gates, s = _toy(golden)
    rng = np.random.default_rng(0)
    dy = rng.standard_normal(x.shape)
    out = O.moe_layer_backward(x, ids, gates, O.scalar_bank(s), O.scalar_bank_backward(s), len(s), dy)
    T, k = ids.shape
    dx = np.zeros_like(x)
    dg = np.zeros((T, k))
    ds = np.zeros(len(s))
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            dx[t] += gates[t, j] * s[e] * dy[t]
            dg[t, j] = float(np.dot(dy[t], s[e] * x[t]))
            ds[e] += gates[t, j] * float(np.dot(dy[t], x[t]))
    assert np.allclose(out["dx"], dx, rtol=1e-13, atol=1e-13)
    assert np.allclose(out["dgates"], dg, rtol=1e-13, atol=1e-13)
    assert np.allclose([g[0] for g in out["grads"]], ds, rtol=1e-13, atol=1e-13)


def _fd(f, theta, h=1e-6):
    """Central differences of the scalar function f at every entry of theta."""
    g = np.zeros_like(theta)
    it = np.nditer(theta, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = theta[i]
        theta[i] = old + h
        fp = f()
        theta[i] = old - h
        fm = f()
        theta[i] = old
        g[i] = (fp - fm) / (2 * h)
    return g


def _close(a, b, tol=1e-7):
    scale = max(1.0, float(np.abs(b).max()))
    return float(np.abs(a - b).max()) <= tol * scale


def _swiglu_case(seed, n=5, d=4, d_ff=3):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((n, d)), rng.standard_normal((d_ff, d)), rng.standard_normal((d_ff, d)),
            rng.standard_normal((d, d_ff)), rng.standard_normal((n, d)))


@pytest.mark.parametrize("seed", [1, 2])
def test_swiglu_backward_finite_differences(seed):
    x, wg, wu, wd, dz = _swiglu_case(seed)
    loss = lambda: float((dz * O.swiglu_expert(x, wg, wu, wd)).sum())
    dx, (dwg, dwu, dwd) = O.swiglu_expert_backward(x, dz, wg, wu, wd)
    for got, theta in ((dx, x), (dwg, wg), (dwu, wu), (dwd, wd)):
        assert got.shape == theta.shape
        assert _close(got, _fd(loss, theta))


def test_swiglu_backward_width_one_closed_form():
    """d = d_ff = 1: z = c SiLU(a x) (b x), so dz/dx = c (a SiLU'(a x) b x +
    SiLU(a x) b), with SiLU'(v) = sigma(v) + v sigma(v) (1 - sigma(v))."""
    a, b, c, xv = 0.7, -1.3, 0.9, 1.1
    sig = 1.0 / (1.0 + np.exp(-a * xv))
    silu = a * xv * sig
    dsilu = sig + a * xv * sig * (1.0 - sig)
    dx, (dwg, dwu, dwd) = O.swiglu_expert_backward(np.array([[xv]]), np.array([[1.0]]), np.array([[a]]),
                                                   np.array([[b]]), np.array([[c]]))
    assert np.isclose(dx[0, 0], c * (a * dsilu * b * xv + silu * b), rtol=1e-14)
    assert np.isclose(dwg[0, 0], c * dsilu * xv * b * xv, rtol=1e-14)
    assert np.isclose(dwu[0, 0], c * silu * xv, rtol=1e-14)
    assert np.isclose(dwd[0, 0], silu * b * xv, rtol=1e-14)


def _layer_case(seed, capacity):
    rng = np.random.default_rng(seed)
    T, E, k, d, d_ff = 7, 3, 2, 4, 3
    z = rng.standard_normal((T, E)).astype(np.float32)
    ids, gates, _ = O.route_topk(z, k)
    gates = gates.astype(np.float64)
    x = rng.standard_normal((T, d))
    W = [[rng.standard_normal((d_ff, d)), rng.standard_normal((d_ff, d)), rng.standard_normal((d, d_ff))]
         for _ in range(E)]
    dy = rng.standard_normal((T, d))
    return ids, gates, x, W, dy, E, capacity


@pytest.mark.parametrize("capacity", [-1, 4])
def test_layer_backward_finite_differences(capacity):
    """Gate, token and weight gradients of the whole layer against central
    differences of the forward oracle (ids fixed; capacity 4 drops routes)."""
    ids, gates, x, W, dy, E, cap = _layer_case(3, capacity)
    bank = lambda e, rows: O.swiglu_expert(rows, *W[e])
    bwd = lambda e, rows, dz: O.swiglu_expert_backward(rows, dz, *W[e])
    loss = lambda: float((dy * O.moe_layer_expert_major(x, ids, gates, bank, E, cap)[0]).sum())
    out = O.moe_layer_backward(x, ids, gates, bank, bwd, E, dy, cap)
    if cap > 0:
        assert out["plan"].dropped > 0
        assert np.all(out["dgates"][out["plan"].inv.reshape(ids.shape) < 0] == 0)
    assert _close(out["dx"], _fd(loss, x))
    assert _close(out["dgates"], _fd(loss, gates))
    for e in range(E):
        if out["grads"][e] is None:
            continue
        for got, theta in zip(out["grads"][e], W[e]):
            assert _close(got, _fd(loss, theta))


def test_mutations_are_caught(monkeypatch):
    """A SiLU' without the v (1 - sigma) term, or route gradients without the
    gate factor, fail the finite-difference pins."""
    ids, gates, x, W, dy, E, cap = _layer_case(4, -1)
    bank = lambda e, rows: O.swiglu_expert(rows, *W[e])
    bwd = lambda e, rows, dz: O.swiglu_expert_backward(rows, dz, *W[e])
    loss = lambda: float((dy * O.moe_layer_expert_major(x, ids, gates, bank, E, cap)[0]).sum())
    fd = _fd(loss, x)
    assert _close(O.moe_layer_backward(x, ids, gates, bank, bwd, E, dy)["dx"], fd)

    with monkeypatch.context() as m:
        m.setattr(OM, "silu_grad", lambda v: 1.0 / (1.0 + np.exp(-v)))
        assert not _close(O.moe_layer_backward(x, ids, gates, bank, bwd, E, dy)["dx"], fd)
    real = OM.combine_backward

    def no_gate(dy_, z_, idx_, gates_, T_, k_):
        return real(dy_, z_, idx_, np.ones_like(gates_), T_, k_)
    with monkeypatch.context() as m:
        m.setattr(OM, "combine_backward", no_gate)
        assert not _close(OM.moe_layer_backward(x, ids, gates, bank, bwd, E, dy)["dx"], fd)


def test_combine_backward_skips_dropped_routes():
    z = np.arange(12, dtype=np.float64).reshape(3, 4)
    idx = np.array([2, -1, 0, 1])
    g = np.array([0.5, 0.25, 2.0, 1.0])
    dy = np.array([[1.0, 0, 0, 0], [0, 1.0, 0, 0]])
    dz, dg = O.combine_backward(dy, z, idx, g, 2, 2)
    assert dg.tolist() == [[8.0, 0.0], [1.0, 5.0]]
    assert dz.tolist() == [[0, 2.0, 0, 0], [0, 1.0, 0, 0], [0.5, 0, 0, 0]]
