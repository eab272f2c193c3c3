"""GPU parity of the fp8 dispatch payload against the oracle.

Codes, scales and padding of every record are compared bit-exactly (every
step of the quantization is one correctly rounded fp32 operation on both
sides); dequantized bf16 rows bit-exactly; records moved by the permute, the
sender pack and the receiver compaction (which dequantizes) bit-exactly."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle as O
import workloads as W
from tests.helpers import to_gpu, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ge():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import grouped_expert_amd as ge
    return ge


def _rows(rng, n, d, zero_row=True):
    x = (rng.standard_normal((n, d)) * 10.0 ** rng.uniform(-3, 2, (n, 1))).astype(np.float32)
    if zero_row and n > 2:
        x[1] = 0.0
    return x


def test_e4m3_encoder_on_the_gpu(ge):
    """Rows whose largest magnitude is 448 quantize with scale 1, so their
    codes are the encoder applied to the values themselves: midpoints
    between neighbouring codes (ties), subnormals, random values."""
    mags = O.fp8_e4m3_decode(np.arange(127, dtype=np.uint8)).astype(np.float64)
    mids = (mags[:-1] + mags[1:]) / 2.0
    rng = np.random.default_rng(0)
    vals = np.concatenate([mags, mids, rng.uniform(0, 448, 3000), 2.0 ** rng.uniform(-12, -6, 2000),
                           np.nextafter(mids.astype(np.float32), np.float32(0)),
                           np.nextafter(mids.astype(np.float32), np.float32(1e9))]).astype(np.float32)
    vals = vals * np.where(rng.random(vals.size) < 0.5, -1, 1).astype(np.float32)
    d = 128
    n = -(-vals.size // (d - 1))
    flat = np.zeros(n * (d - 1), np.float32)
    flat[:vals.size] = vals
    x = np.zeros((n, d), np.float32)
    x[:, 0] = 448.0
    x[:, 1:] = flat.reshape(n, d - 1)
    for mode in ("row", "b128"):
        rec = to_np(ge.quantize_fp8(to_gpu(x), mode))
        want = O.quantize_fp8_rows(x, mode)
        assert np.array_equal(rec, want), mode
        assert np.array_equal(rec[:, 1:d].reshape(-1)[:vals.size], O.fp8_e4m3_encode(vals))


@pytest.mark.parametrize("n,d,xdt,mode", [(300, 3072, "bf16", "b128"), (300, 3072, "bf16", "row"),
                                          (77, 200, "f32", "b128"), (64, 64, "f32", "row"),
                                          (5, 7168, "bf16", "b128"), (0, 128, "bf16", "row")])
def test_quantize_dequantize(ge, n, d, xdt, mode):
    rng = np.random.default_rng(n + d)
    x32 = _rows(rng, n, d)
    x = W.f32_to_bf16_bits(x32) if xdt == "bf16" else x32
    xv = O.to_f64(x).astype(np.float32)
    flags = ge.new_flags("cuda")
    xt = to_gpu(x) if n else torch.empty((0, d), dtype=torch.bfloat16 if xdt == "bf16" else torch.float32,
                                         device="cuda")
    rec = ge.quantize_fp8(xt, mode, flags=flags)
    want = O.quantize_fp8_rows(xv, mode)
    assert rec.shape == (n, ge.row_bytes(d, mode)) == want.shape
    assert np.array_equal(to_np(rec), want)
    back16 = ge.dequantize_fp8(rec, d, mode, out_dtype=torch.bfloat16)
    back32 = ge.dequantize_fp8(rec, d, mode, out_dtype=torch.float32)
    deq = O.dequantize_fp8_rows(want, d, mode)
    assert np.array_equal(to_np(back16), O.f32_to_bf16_rne(deq))
    assert np.array_equal(to_np(back32), deq)
    assert int(to_np(flags)[0]) == 0


def test_quantize_nonfinite_group_flag(ge):
    x = np.ones((2, 256), np.float32)
    x[0, 130] = np.nan                       # second 128-value group of row 0
    flags = ge.new_flags("cuda")
    rec = to_np(ge.quantize_fp8(to_gpu(x), "b128", flags=flags))
    assert int(to_np(flags)[0]) == 32
    assert np.array_equal(rec, O.quantize_fp8_rows(x, "b128"))
    assert np.all(rec[0, 128:256] == 0) and np.all(rec[0, :128] == 0x7E)


@pytest.mark.parametrize("mode", ["row", "b128"])
def test_permute_moves_whole_records(ge, mode):
    rng = np.random.default_rng(7)
    T, E, k, d = 500, 16, 4, 384
    rec = O.quantize_fp8_rows(_rows(rng, T, d), mode)
    ids, _, _ = O.route_topk(rng.standard_normal((T, E)).astype(np.float32), k)
    plan = ge.permute(to_gpu(rec), to_gpu(ids), E, 100, payload=mode, d=d)
    want = O.dispatch_plan(ids, E, 100)
    A = want.accepted
    assert np.array_equal(to_np(plan["inv"]), want.inv)
    assert np.array_equal(to_np(plan["x_perm"])[:A], rec[want.src[:A] // k])


@pytest.mark.parametrize("T,k,epd,D,Wv,P,d,mode,fused", [(400, 4, 3, 8, 2, 30, 128, "row", False),
                                                         (400, 4, 3, 8, 2, 30, 128, "row", True),
                                                         (3000, 8, 6, 64, 3, 30, 256, "b128", False),
                                                         (3000, 8, 6, 64, 3, 30, 256, "b128", True),
                                                         (900, 8, 2, 8, 2, 200, 200, "b128", True),
                                                         (900, 8, 2, 8, 2, 200, 64, "b128", False)])
def test_pool_pack_and_compact_fp8(ge, T, k, epd, D, Wv, P, d, mode, fused):
    """Records packed as they are, or bf16 rows quantized by the pack itself
    (fused): the same pools either way.  d = 200 has a short last group and
    d = 64 needs several header rows."""
    rng = np.random.default_rng(T + P)
    E = D * epd
    z = rng.standard_normal((T, E)).astype(np.float32)
    z[:, :epd] += 1.5
    ids, _, _ = O.route_topk(z, k)
    x16 = W.f32_to_bf16_bits(_rows(rng, T, d))
    rec = O.quantize_fp8_rows(O.to_f64(x16).astype(np.float32), mode)
    flags = ge.new_flags("cuda")
    out = ge.pool_pack(to_gpu(x16 if fused else rec), to_gpu(ids), E, epd, D, Wv, P, flags=flags, payload=mode,
                       d=d)
    pk = O.pool_pack(rec, ids, epd, D, Wv, P)
    assert np.array_equal(to_np(out["pools"]), pk["pools"])
    assert np.array_equal(to_np(out["route_loc"]), pk["route_loc"])
    cap = max(1, P * D // (2 * epd))
    for w in range(Wv):
        rot = w % D
        rc = ge.recv_compact(out["pools"][w], epd, cap, flags=flags, rotation=rot, payload=mode, d=d)
        want = O.recv_compact(pk["pools"][w], epd, cap, rotation=rot, record=(d, mode))
        counts = to_np(rc["counts"])
        assert np.array_equal(counts, want["counts"])
        assert np.array_equal(to_np(rc["row_slot"]), want["row_slot"])
        got = to_np(rc["compact"])
        for h in range(epd):
            assert np.array_equal(got[h, :counts[h]], want["compact"][h, :counts[h]]), (w, h)
    assert int(to_np(flags)[0]) == 0
