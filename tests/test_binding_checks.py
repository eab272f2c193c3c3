"""Host-side argument checks of the Python binding (no GPU needed): tensors
whose shape or dtype disagrees with the sizes handed to the kernels are
refused before any call, since the kernels would index past them."""
import pytest

torch = pytest.importorskip("torch")
ge = pytest.importorskip("grouped_expert_amd")


def _weights(E=4, d=64, d_ff=128, dt=torch.bfloat16):
    return (torch.zeros((E, d_ff, d), dtype=dt), torch.zeros((E, d_ff, d), dtype=dt),
            torch.zeros((E, d, d_ff), dtype=dt))


def test_grouped_swiglu_checks_weight_shapes_and_dtypes():
    x = torch.zeros((32, 64), dtype=torch.bfloat16)
    wg, wu, wd = _weights()
    s = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError, match="w_up"):
        ge.grouped_swiglu(x, s, s, wg, wu[:, :64], wd)
    with pytest.raises(ValueError, match="w_down"):
        ge.grouped_swiglu(x, s, s, wg, wu, wd.transpose(1, 2).contiguous())
    with pytest.raises(ValueError, match="w_gate"):
        ge.grouped_swiglu(x, s, s, wg.float(), wu, wd)
    with pytest.raises(ValueError, match="seg_count"):
        ge.grouped_swiglu(x, s, s.long(), wg, wu, wd)
    with pytest.raises(ValueError, match="seg_start"):
        ge.grouped_swiglu(x, s[:3], s, wg, wu, wd)
    with pytest.raises(ValueError, match="z"):
        ge.grouped_swiglu(x, s, s, wg, wu, wd, z=torch.zeros((31, 64)))
    with pytest.raises(ValueError, match="GPU"):                # well-formed, but on the host
        ge.grouped_swiglu(x, s, s, wg, wu, wd)


def test_combine_checks_indices_gates_window_and_flags():
    z = torch.zeros((40, 64), dtype=torch.bfloat16)
    idx = torch.zeros((10, 4), dtype=torch.int32)
    g = torch.zeros((10, 4))
    with pytest.raises(ValueError, match="idx"):
        ge.unpermute_combine(z, idx.long(), g, 10, 4)
    with pytest.raises(ValueError, match="gates"):
        ge.unpermute_combine(z, idx, g[:, :3], 10, 4)
    with pytest.raises(ValueError, match="window"):
        ge.unpermute_combine(z, idx, g, 10, 4, lo=0, hi=41)
    with pytest.raises(ValueError, match="y"):
        ge.unpermute_combine(z, idx, g, 10, 4, y=torch.zeros((10, 63)))
    with pytest.raises(ValueError, match="flags"):
        ge.unpermute_combine(z, idx, g, 10, 4, flags=torch.zeros(1, dtype=torch.int64))


def test_router_permute_and_pack_check_dtypes():
    with pytest.raises(ValueError, match="logits"):
        ge.route_topk(torch.zeros((8, 16), dtype=torch.bfloat16), 2)
    with pytest.raises(ValueError, match="bias"):
        ge.route_topk_grouped(torch.zeros((8, 16)), 2, ge.MOE_GATING_SIGMOID_BIAS_GROUP_TOP2, 4, 2, 1.0,
                              bias=torch.zeros(15))
    with pytest.raises(ValueError, match="topk_ids"):
        ge.permute(torch.zeros((8, 64), dtype=torch.bfloat16), torch.zeros((8, 2)), 16)
    with pytest.raises(ValueError, match="x"):
        ge.permute(torch.zeros((7, 64), dtype=torch.bfloat16), torch.zeros((8, 2), dtype=torch.int32), 16)
    with pytest.raises(ValueError, match="topk_ids"):
        ge.pool_pack(torch.zeros((8, 64), dtype=torch.bfloat16), torch.zeros((8, 2), dtype=torch.int64), 12, 6, 2,
                     2, 10)


def test_backward_and_fp8_check_shapes():
    x = torch.zeros((32, 64), dtype=torch.bfloat16)
    wg, wu, wd = _weights()
    s = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError, match="dz"):
        ge.grouped_swiglu_backward(x, torch.zeros((32, 64)), s, s, wg, wu, wd)
    with pytest.raises(ValueError, match="dy"):
        ge.combine_backward(torch.zeros((8, 64), dtype=torch.bfloat16), x, torch.zeros(16, dtype=torch.int32),
                            torch.zeros(16), 2)
    with pytest.raises(ValueError, match="rec"):
        ge.dequantize_fp8(torch.zeros((4, 100), dtype=torch.uint8), 64, "b128")
    with pytest.raises(ValueError, match="ret"):
        ge.expand_rows(torch.zeros((10, 64)), torch.zeros(12, dtype=torch.int32), ret=torch.zeros((11, 64)))
