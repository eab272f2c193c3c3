"""Pins of the oracle's FP8 dispatch payload (CPU only).

The page's byte ledger (M6.2 §0x0AB), the E4M3 format's own values (bias 7,
3 mantissa bits, subnormals, 448 maximum, 0x7F NaN), rounding checked
against an independent bit-level encoder, quantization error bounds, and the
scale-ownership rule of M6.2 §0x0AC with a planted violation."""
import numpy as np
import pytest

import oracle as O


def test_payload_ledger_matches_page(golden):
    f = golden("m62_fp8_payload_fixture.json")
    R = f["rows"]
    for row in f["table"]:
        d = row["d"]
        assert O.fp8_payload_bytes(R, d, None) == row["bf16"]
        assert O.fp8_payload_bytes(R, d, "row") == row["fp8_row"]
        assert O.fp8_payload_bytes(R, d, "b128") == row["fp8_b128"]
    # the d = 3 row: the scales make the fp8 payload larger than bf16
    assert O.fp8_payload_bytes(R, 3, "row") > O.fp8_payload_bytes(R, 3, None)


def test_e4m3_format_values():
    """Values fixed by the format definition."""
    dec = lambda c: float(O.fp8_e4m3_decode(np.array([c], np.uint8))[0])
    assert dec(0x7E) == 448.0 and dec(0xFE) == -448.0
    assert np.isnan(dec(0x7F)) and np.isnan(dec(0xFF))
    assert dec(0x01) == 2.0 ** -9 and dec(0x07) == 7 * 2.0 ** -9       # subnormals
    assert dec(0x08) == 2.0 ** -6                                       # smallest normal
    assert dec(0x38) == 1.0 and dec(0x30) == 0.5 and dec(0xC0) == -2.0
    assert dec(0x00) == 0.0 and dec(0x80) == 0.0
    enc = lambda v: int(O.fp8_e4m3_encode(np.array([v], np.float32))[0])
    assert enc(1.0625) == 0x38            # halfway between 1.0 (even code) and 1.125
    assert enc(1.1875) == 0x3A            # halfway between 1.125 and 1.25 (even code)
    assert enc(500.0) == 0x7E and enc(-1e30) == 0xFE and enc(np.inf) == 0x7E
    assert enc(2.0 ** -10) == 0x00        # half the smallest subnormal ties to zero
    assert enc(1.5 * 2.0 ** -9) == 0x02   # 1.5 subnormal units tie to the even code 2
    assert enc(-0.0) == 0x80 and enc(np.nan) == 0x7F


def test_e4m3_round_trip_every_code():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    v = O.fp8_e4m3_decode(codes)
    back = O.fp8_e4m3_encode(v)
    same = (back == codes) | ((codes & 0x7F) == 0)      # +-0 keep their sign bit
    assert np.all(same)


def _bitwise_e4m3(v):
    """Independent encoder on the fp32 bit pattern: shift the significand to
    the E4M3 grid and round half to even on the dropped bits."""
    out = []
    for x in np.asarray(v, np.float32):
        u = int(np.array([x], np.float32).view(np.uint32)[0])
        sign = (u >> 31) << 7
        ax = abs(float(x))
        if ax >= 448.0:
            out.append(sign | 0x7E)
            continue
        e = ((u >> 23) & 0xFF) - 127
        m = (u & 0x7FFFFF) | (0x800000 if ((u >> 23) & 0xFF) else 0)
        if ((u >> 23) & 0xFF) == 0:
            e = -126
        shift = 20 if e >= -6 else 20 + (-6 - e)      # keep 3 fraction bits (fewer below 2^-6)
        if shift >= 32:
            q = 0
        else:
            q = m >> shift
            rem = m & ((1 << shift) - 1)
            half = 1 << (shift - 1)
            if rem > half or (rem == half and (q & 1)):
                q += 1
        if e >= -6:
            # q holds 1.mmm (with carry) at exponent e
            if q >= 16:
                q >>= 1
                e += 1
            code = ((e + 7) << 3) | (q & 7)
        else:
            code = q                                   # subnormal count of 2^-9 units (may carry to 8)
        out.append(sign | min(code, 0x7E))
    return np.array(out, np.uint8)


def test_e4m3_encode_matches_bitwise_encoder():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(4000) * 10.0 ** rng.uniform(-4, 2.8, 4000),
                        (O.fp8_e4m3_decode(np.arange(126, dtype=np.uint8)).astype(np.float64)
                         + O.fp8_e4m3_decode(np.arange(1, 127, dtype=np.uint8))) / 2.0]).astype(np.float32)
    assert np.array_equal(O.fp8_e4m3_encode(v), _bitwise_e4m3(v))


@pytest.mark.parametrize("mode", ["row", "b128"])
def test_quantize_bounds_and_layout(mode):
    rng = np.random.default_rng(1)
    n, d = 40, 384
    x = (rng.standard_normal((n, d)) * rng.uniform(0.01, 10, (n, 1))).astype(np.float32)
    x[3] = 0.0                                            # an all-zero row
    rec = O.quantize_fp8_rows(x, mode)
    G, W = O.fp8_record_layout(d, mode)
    assert rec.shape == (n, W) and W % 128 == 0 and d + 4 * G <= W < d + 4 * G + 128
    assert np.all(rec[:, d + 4 * G:] == 0)                # padding
    scales = np.ascontiguousarray(rec[:, d:d + 4 * G]).view(np.float32)
    width = d if mode == "row" else 128
    amax = np.abs(x.reshape(n, G, width)).max(axis=2)
    assert np.array_equal(scales, (amax / np.float32(448)).astype(np.float32))
    back = O.dequantize_fp8_rows(rec, d, mode)
    err = np.abs(back.astype(np.float64) - x)
    per_col = np.repeat(amax, width, axis=1).astype(np.float64)
    # E4M3 keeps 3 fraction bits: half a unit in the last place is 2^-4 relative
    # for normal values; below 2^-6 (scaled) the absolute step is 2^-9 * scale
    assert np.all(err <= np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * per_col / 448 * 1.01) + 1e-30)
    # each group's largest magnitude maps to the top of the range
    top = np.abs(O.fp8_e4m3_decode(rec[:, :d])).reshape(n, G, width).max(axis=2)
    assert np.all((top == 448.0) | (amax == 0))
    assert np.all(back[3] == 0) and np.all(scales[3] == 0)


def test_scales_travel_with_their_rows():
    """M6.2 §0x0AC: permuting records moves data and scales together, so
    dequantize(permute(q)) = permute(dequantize(q)); permuting only the data
    while the scales stay token-major (the page's failure case) does not."""
    rng = np.random.default_rng(2)
    n, d = 12, 256
    x = (rng.standard_normal((n, d)) * rng.uniform(0.1, 50, (n, 1))).astype(np.float32)
    rec = O.quantize_fp8_rows(x, "b128")
    perm = rng.permutation(n)
    assert np.array_equal(O.dequantize_fp8_rows(rec[perm], d, "b128"), O.dequantize_fp8_rows(rec, d, "b128")[perm])
    wrong = rec.copy()
    wrong[:, :d] = rec[perm, :d]                          # data permuted, scales left in token order
    assert not np.allclose(O.dequantize_fp8_rows(wrong, d, "b128"), O.dequantize_fp8_rows(rec, d, "b128")[perm])


def test_fp8_pools_round_trip_through_compaction():
    """Records packed into pools and compacted give the dequantized rows, in
    bf16, at the same slots as the bf16 payload's rows."""
    rng = np.random.default_rng(3)
    T, k, epd, D, Wv, P, cap, d = 120, 4, 3, 4, 2, 30, 25, 128
    z = rng.standard_normal((T, epd * D)).astype(np.float32)
    ids, _, _ = O.route_topk(z, k)
    x = O.f32_to_bf16_rne(rng.standard_normal((T, d)).astype(np.float32))
    rec = O.quantize_fp8_rows(O.to_f64(x).astype(np.float32), "row")
    pk16 = O.pool_pack(x, ids, epd, D, Wv, P)
    pk8 = O.pool_pack(rec, ids, epd, D, Wv, P)
    assert np.array_equal(pk16["route_loc"] >= 0, pk8["route_loc"] >= 0)
    H8 = O.header_rows_bytes(P, rec.shape[1])
    assert pk8["pools"].shape == (Wv, D, P + H8, rec.shape[1])
    for w in range(Wv):
        a = O.recv_compact(pk16["pools"][w], epd, cap)
        b = O.recv_compact(pk8["pools"][w], epd, cap, record=(d, "row"))
        assert np.array_equal(a["counts"], b["counts"])
        want = O.f32_to_bf16_rne(O.dequantize_fp8_rows(rec, d, "row"))
        src = {}
        for r in np.nonzero(pk8["route_loc"] >= 0)[0]:
            src[int(pk8["route_loc"][r])] = r // k
        lo = w * D * (P + H8)
        for i, slot in enumerate(b["row_slot"]):
            if slot >= 0:
                h, q = divmod(int(slot), cap)
                assert np.array_equal(b["compact"][h, q], want[src[lo + i]])


def test_f32_to_bf16_rne():
    v = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 0.0], np.float32)
    got = O.f32_to_bf16_rne(v)
    back = (got.astype(np.uint32) << 16).view(np.float32)
    assert back.tolist() == [1.0, 1.0, 1.0 + 2.0 ** -6, -2.5, 0.0]    # ties to even
