"""Shared helpers of the GPU parity tests (host-side marshalling and the
comparison rule).  Nothing here computes the layer."""
import numpy as np
import torch


def dev():
    return torch.device("cuda:0")


def to_gpu(a: np.ndarray) -> torch.Tensor:
    """numpy -> device tensor; uint16 arrays are bf16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(dev()).view(torch.bfloat16)
    return torch.from_numpy(a).to(dev())


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def as_f64(t) -> np.ndarray:
    a = to_np(t) if isinstance(t, torch.Tensor) else np.asarray(t)
    return bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


REL_TOL = 2e-2   # max relative error against the fp64 oracle (bf16 inputs, fp32 accumulate)


def row_rel_err(got: np.ndarray, want: np.ndarray) -> float:
    """Per output row: max |got - want| / max |want|; the worst row is
    returned.  Rows the oracle makes exactly zero must be exactly zero
    (reported as inf otherwise)."""
    got = np.asarray(got, np.float64).reshape(want.shape[0], -1)
    want = np.asarray(want, np.float64).reshape(want.shape[0], -1)
    scale = np.abs(want).max(axis=1)
    err = np.abs(got - want).max(axis=1)
    zero = scale == 0
    if np.any(err[zero] != 0):
        return float("inf")
    if np.all(zero):
        return 0.0
    return float((err[~zero] / scale[~zero]).max())


def assert_rows_close(got, want, tol=REL_TOL, what=""):
    e = row_rel_err(got, want)
    assert e <= tol, f"{what}: max row relative error {e:.3e} > {tol}"
    return e
