"""The C-ABI library loads, exports every function ``include/moe.h``
declares, and rejects bad arguments on the host before touching the GPU
(these calls return before any HIP call, so they run without a GPU)."""
import ctypes

import pytest

from grouped_expert_amd import binding as B

lib = B.lib
NULL = None
EINVAL, EUNSUP, EWS = -1, -2, -3


def test_exports_every_header_symbol():
    names = B.header_functions()
    assert len(names) == 23
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(B._SIGS)


def test_strerror_and_version():
    assert B.strerror(0) == "ok"
    assert B.strerror(-3).startswith("workspace")
    assert B.strerror(12345) == "unknown status"
    assert lib.moe_version() >= 100


def _fake(n=1):
    # host buffer addresses: never dereferenced because validation fails first
    buf = (ctypes.c_char * (64 * n))()
    return ctypes.c_void_p((ctypes.addressof(buf) + 15) & ~15), buf


def test_route_validation():
    p, _keep = _fake()
    assert lib.moe_route_topk(p, 10, 8, 0, 0, p, p, NULL, NULL) == EINVAL         # k < 1
    assert lib.moe_route_topk(p, 10, 8, 9, 0, p, p, NULL, NULL) == EINVAL         # k > E
    assert lib.moe_route_topk(p, 10, 2000, 2, 0, p, p, NULL, NULL) == EINVAL      # E too large
    assert lib.moe_route_topk(p, 10, 32, 17, 0, p, p, NULL, NULL) == EINVAL       # k > 16
    assert lib.moe_route_topk(p, 10, 8, 2, 7, p, p, NULL, NULL) == EUNSUP         # unknown gating
    assert lib.moe_route_topk(NULL, 10, 8, 2, 0, p, p, NULL, NULL) == EINVAL      # null logits
    assert lib.moe_route_topk(NULL, 0, 8, 2, 0, NULL, NULL, NULL, NULL) == 0      # empty batch
    assert lib.moe_route_topk(NULL, 0, 8, 2, 1, NULL, NULL, NULL, NULL) == 0      # V1 accepted
    assert lib.moe_route_topk(p, 10, 8, 2, 2, p, p, NULL, NULL) == EUNSUP         # V2 needs the grouped call


def test_route_grouped_validation():
    p, _keep = _fake()
    f = lib.moe_route_topk_grouped
    V2, V3 = 2, 3
    ok = [p, 10, 256, 8, V3, 8, 4, 2.5, p, p, p, NULL, NULL]
    assert f(NULL, 0, *ok[2:]) == 0                                           # empty batch, valid geometry
    for i, v, want in [(4, 0, EUNSUP),          # plain softmax gating belongs to moe_route_topk
                       (4, 1, EUNSUP),
                       (5, 0, EINVAL),          # n_group < 1
                       (5, 65, EINVAL),         # more groups than lanes
                       (5, 7, EINVAL),          # 256 % 7 != 0
                       (6, 0, EINVAL),          # topk_group < 1
                       (6, 9, EINVAL),          # topk_group > n_group
                       (3, 17, EINVAL),         # k > 16
                       (7, float("inf"), EINVAL)]:
        bad = list(ok); bad[i] = v
        assert f(*bad) == want, (i, v)
    bad = list(ok); bad[5] = 128; bad[6] = 2; bad[3] = 8                       # 2 experts per group, keep 2: k <= 4
    assert f(*bad) == EINVAL
    bad = list(ok); bad[4] = V2                                                 # bias is V3-only
    assert f(*bad) == EINVAL
    bad = list(ok); bad[2] = 8; bad[5] = 8; bad[6] = 4; bad[3] = 2              # V3 needs >= 2 experts per group
    assert f(*bad) == EINVAL
    bad = list(ok); bad[0] = NULL                                               # null logits
    assert f(*bad) == EINVAL


def test_permute_validation():
    p, _keep = _fake()
    ws = lib.moe_permute_workspace(100, 8, 128)
    assert ws > 0
    args = [p, 1, 100, 64, p, 8, 128, -1, p, p, p, p, p, p, p, p, ws, NULL, NULL]
    bad = list(args); bad[7] = -2                                   # capacity < -1
    assert lib.moe_permute(*bad) == EINVAL
    bad = list(args); bad[16] = ws - 1                              # workspace too small
    assert lib.moe_permute(*bad) == EWS
    bad = list(args); bad[15] = NULL                                # no workspace
    assert lib.moe_permute(*bad) == EWS
    bad = list(args); bad[3] = 60                                   # bf16 row not 16-byte multiple
    assert lib.moe_permute(*bad) == EINVAL
    bad = list(args); bad[1] = 5                                    # unknown dtype
    assert lib.moe_permute(*bad) == EINVAL
    bad = list(args); bad[13] = NULL                                # offsets required
    assert lib.moe_permute(*bad) == EINVAL
    q = ctypes.c_void_p(p.value + 4)
    bad = list(args); bad[0] = q                                    # misaligned rows
    assert lib.moe_permute(*bad) == EINVAL


def test_swiglu_validation():
    p, _keep = _fake()
    ws = lib.moe_grouped_swiglu_workspace(1000, 8, 256, 1)
    assert ws >= 1000 * 256 * 2
    args = [p, 1, 128, 256, 8, p, p, 1000, p, p, p, p, 1, NULL, 0, NULL, p, ws, NULL, NULL]
    assert lib.moe_grouped_swiglu(*args[:17], ws - 1, NULL, NULL) == EWS
    q = ctypes.c_void_p(p.value + 2)
    bad = list(args); bad[13] = q; bad[14] = 10                     # misaligned row map
    assert lib.moe_grouped_swiglu(*bad) == EINVAL
    bad = list(args); bad[13] = p; bad[14] = -1                     # negative z rows
    assert lib.moe_grouped_swiglu(*bad) == EINVAL
    bad = list(args); bad[13] = p; bad[14] = 1 << 31                # z rows past int32 indexes
    assert lib.moe_grouped_swiglu(*bad) == EUNSUP
    bad = list(args); bad[2] = 100                                  # d not a multiple of 64
    assert lib.moe_grouped_swiglu(*bad) == EUNSUP
    bad = list(args); bad[1] = 0; bad[12] = 1                       # fp32 in, bf16 out
    assert lib.moe_grouped_swiglu(*bad) == EUNSUP
    bad = list(args); bad[8] = NULL                                 # no gate weights
    assert lib.moe_grouped_swiglu(*bad) == EINVAL
    bad = list(args); bad[4] = 0                                    # no experts
    assert lib.moe_grouped_swiglu(*bad) == EINVAL
    bad = list(args); bad[1] = 0; bad[15] = p                       # saved activations on the fp32 path
    assert lib.moe_grouped_swiglu(*bad) == EUNSUP
    bad = list(args); bad[15] = ctypes.c_void_p(p.value + 2)        # misaligned saved activations
    assert lib.moe_grouped_swiglu(*bad) == EINVAL


def test_combine_validation():
    p, _keep = _fake()
    assert lib.moe_unpermute_combine(p, 1, 60, p, 0, 10, NULL, 10, 2, p, 0, NULL, NULL) == EINVAL   # d % 8
    assert lib.moe_unpermute_combine(p, 0, 64, p, 5, 2, NULL, 10, 2, p, 0, NULL, NULL) == EINVAL    # hi < lo
    assert lib.moe_unpermute_combine(p, 0, 64, NULL, 0, 2, NULL, 10, 2, p, 0, NULL, NULL) == EINVAL  # idx
    assert lib.moe_unpermute_combine(p, 0, 64, p, 0, 2, NULL, 0, 2, p, 0, NULL, NULL) == 0          # empty


def test_pool_pack_validation():
    p, _keep = _fake()
    ws = lib.moe_pool_pack_workspace(100, 8, 64)
    args = [p, 1, 1, 100, 3072, p, 8, 384, 6, 64, 3, 3004, -1, p, p, p, p, p, ws, NULL, NULL]
    bad = list(args); bad[7] = 385                                  # E > n_dest * epd
    assert lib.moe_pool_pack(*bad) == EINVAL
    bad = list(args); bad[11] = 1 << 30                             # pool rows past the int32 route locations
    assert lib.moe_pool_pack(*bad) == EUNSUP
    bad = list(args); bad[11] = -1                                  # negative pool rows
    assert lib.moe_pool_pack(*bad) == EINVAL
    bad = list(args); bad[12] = 3                                   # wave out of range
    assert lib.moe_pool_pack(*bad) == EINVAL
    bad = list(args); bad[18] = 8                                   # workspace too small
    assert lib.moe_pool_pack(*bad) == EWS
    bad = list(args); bad[1] = 0; bad[2] = 0                        # fp32 rows are not a dispatch payload
    assert lib.moe_pool_pack(*bad) == EINVAL
    bad = list(args); bad[1] = 3; bad[2] = 1                        # records cannot be widened back to bf16
    assert lib.moe_pool_pack(*bad) == EINVAL
    bad = list(args); bad[1] = 3; bad[2] = 2                        # nor turned into the other record kind
    assert lib.moe_pool_pack(*bad) == EINVAL
    for xd, pd in ((3, 3), (1, 2), (1, 3)):                         # accepted pairs (then: too many rows)
        bad = list(args); bad[1] = xd; bad[2] = pd; bad[11] = 1 << 30
        assert lib.moe_pool_pack(*bad) == EUNSUP


def test_recv_compact_validation():
    p, _keep = _fake()
    ws = lib.moe_recv_compact_workspace(64, 3004, 6)
    args = [p, 1, 64, 3004, 3072, 6, 33497, 0, p, p, p, p, p, NULL, NULL, 0, p, ws, NULL, NULL]
    bad = list(args); bad[6] = -1                                   # negative capacity
    assert lib.moe_recv_compact(*bad) == EINVAL
    bad = list(args); bad[5] = 0                                    # no local experts
    assert lib.moe_recv_compact(*bad) == EINVAL
    bad = list(args); bad[7] = 64                                   # rotation past the last source
    assert lib.moe_recv_compact(*bad) == EINVAL
    bad = list(args); bad[7] = -1                                   # negative rotation
    assert lib.moe_recv_compact(*bad) == EINVAL
    bad = list(args); bad[17] = 0                                   # workspace
    assert lib.moe_recv_compact(*bad) == EWS
    bad = list(args); bad[14] = p; bad[15] = 2                      # return rows must be fp32 or bf16
    assert lib.moe_recv_compact(*bad) == EINVAL
    bad = list(args); bad[14] = ctypes.c_void_p(p.value + 4); bad[15] = 0   # misaligned return rows
    assert lib.moe_recv_compact(*bad) == EINVAL
    bad = list(args); bad[13] = ctypes.c_void_p(p.value + 2)         # misaligned slot map
    assert lib.moe_recv_compact(*bad) == EINVAL
    bad = list(args); bad[3] = 1 << 26                              # pool rows past int32 row indexes
    assert lib.moe_recv_compact(*bad) == EUNSUP
    bad = list(args); bad[1] = 7                                    # unknown pool dtype
    assert lib.moe_recv_compact(*bad) == EINVAL


def test_fp8_record_widths_and_validation():
    assert lib.moe_row_bytes(1, 3072) == 6144 and lib.moe_row_bytes(0, 3) == 12
    assert lib.moe_row_bytes(2, 3072) == 3200            # 3072 codes + 4 + 124 padding
    assert lib.moe_row_bytes(3, 3072) == 3200            # 3072 codes + 24 scales + 104 padding
    assert lib.moe_row_bytes(3, 7168) == 7424            # 7168 + 4 * 56 = 7392, to whole 128-byte lines
    assert lib.moe_row_bytes(2, 124) == 128 and lib.moe_row_bytes(2, 125) == 256
    assert lib.moe_row_bytes(9, 64) == 0 and lib.moe_row_bytes(1, 0) == 0
    p, _keep = _fake()
    assert lib.moe_quantize_fp8(p, 1, 10, 64, 1, p, NULL, NULL) == EINVAL      # record dtype must be fp8
    assert lib.moe_quantize_fp8(p, 2, 10, 64, 2, p, NULL, NULL) == EINVAL      # input must be bf16 / fp32
    assert lib.moe_quantize_fp8(p, 1, 10, 12, 2, p, NULL, NULL) == EINVAL      # d % 8
    assert lib.moe_quantize_fp8(NULL, 1, 0, 64, 3, NULL, NULL, NULL) == 0      # nothing to do
    assert lib.moe_dequantize_fp8(p, 1, 10, 64, p, 1, NULL, NULL) == EINVAL    # records must be fp8
    assert lib.moe_dequantize_fp8(p, 3, 10, 64, p, 2, NULL, NULL) == EINVAL    # output bf16 / fp32
    assert lib.moe_dequantize_fp8(NULL, 3, 0, 64, NULL, 1, NULL, NULL) == 0


def test_expand_rows_validation():
    p, _keep = _fake()
    args = [p, 1, 3072, p, 100, 50, p, 0, NULL, NULL]
    bad = list(args); bad[1] = 2                                    # unknown z dtype
    assert lib.moe_expand_rows(*bad) == EINVAL
    bad = list(args); bad[7] = 5                                    # unknown return dtype
    assert lib.moe_expand_rows(*bad) == EINVAL
    bad = list(args); bad[2] = 12                                   # d not a multiple of 8
    assert lib.moe_expand_rows(*bad) == EINVAL
    bad = list(args); bad[4] = 1 << 40                              # more rows than one launch holds
    assert lib.moe_expand_rows(*bad) == EUNSUP
    bad = list(args); bad[6] = NULL                                 # no output
    assert lib.moe_expand_rows(*bad) == EINVAL
    assert lib.moe_expand_rows(NULL, 0, 64, NULL, 0, 0, NULL, 1, NULL, NULL) == 0   # nothing to do


def test_workspace_queries_reject_bad_sizes():
    assert lib.moe_permute_workspace(-1, 8, 8) == 0
    assert lib.moe_permute_workspace(10, 8, 5000) == 0
    assert lib.moe_grouped_swiglu_workspace(10, 8, 64, 7) == 0
    assert lib.moe_pool_pack_workspace(10, 0, 8) == 0
    assert lib.moe_recv_compact_workspace(4, 4, 0) == 0


def test_record_widths_agree_with_the_oracle_layout():
    """The library's record width and the oracle's record layout are written
    independently; they must agree for every width and scale layout."""
    import oracle as O
    for d in list(range(8, 1025, 8)) + [2048, 3072, 4096, 7168, 8192]:
        for code, mode in ((2, "row"), (3, "b128")):
            assert lib.moe_row_bytes(code, d) == O.fp8_record_layout(d, mode)[1], (d, mode)
        assert lib.moe_row_bytes(1, d) == 2 * d and lib.moe_row_bytes(0, d) == 4 * d


def test_pool_geometry_agrees_with_the_oracle():
    """The library's pool geometry (header rows, pool height, and its inverse)
    against the oracle's header-row rule, written independently, for bf16
    rows and both fp8 record layouts."""
    import oracle as O
    for d in (8, 64, 136, 1024, 3072, 7168):
        for code, payload in ((1, None), (2, "row"), (3, "b128")):
            rb = lib.moe_row_bytes(code, d)
            for P in (0, 1, 2, 3, rb // 2 - 1, rb // 2, rb // 2 + 1, 3004, 4506, 24030, 33497):
                h, ph = B.pool_geometry(P, d, payload)
                assert h == O.header_rows_bytes(P, rb), (d, payload, P)
                assert ph == P + h
                assert B.pool_rows_of_height(ph, d, payload) == P
    # the pages' sizes: one header row for 3004-row pools, two for 4506 rows
    assert B.pool_geometry(3004, 3072) == (1, 3005)
    assert B.pool_geometry(4506, 3072) == (2, 4508)
    h = ctypes.c_int64()
    assert lib.moe_pool_geometry(1, 3072, -1, ctypes.byref(h), ctypes.byref(h)) == EINVAL
    assert lib.moe_pool_geometry(9, 3072, 10, ctypes.byref(h), ctypes.byref(h)) == EINVAL
    assert lib.moe_pool_geometry(1, 12, 10, ctypes.byref(h), ctypes.byref(h)) == EINVAL
    assert lib.moe_pool_rows_of_height(1, 3072, 0, ctypes.byref(h)) == EINVAL


def test_permute_noalloc_validation():
    """Host checks of the no-allocation permute: the permute's own argument
    rules, and MOE_ESCRATCH (before any HIP call) when the rank table would
    not fit the static scratch."""
    p, _keep = _fake()
    ESCRATCH = B.MOE_ESCRATCH
    assert lib.moe_permute_noalloc(p, 1, 10, 8, p, 0, 8, -1, p, p, p, p, p, p, p, NULL, NULL) == EINVAL   # k < 1
    assert lib.moe_permute_noalloc(p, 1, 10, 8, p, 2, 8, -2, p, p, p, p, p, p, p, NULL, NULL) == EINVAL   # capacity
    assert lib.moe_permute_noalloc(p, 1, 10, 8, p, 2, 8, -1, p, p, p, p, NULL, p, p, NULL, NULL) == EINVAL
    big_T, k, E = 1 << 20, 8, 1024
    assert lib.moe_permute_workspace(big_T, k, E) > B.PERMUTE_NOALLOC_SCRATCH_BYTES
    assert lib.moe_permute_noalloc(p, 1, big_T, 8, p, k, E, -1, NULL, p, p, p, p, p, p, NULL, NULL) == ESCRATCH
    assert "scratch" in B.strerror(ESCRATCH)
