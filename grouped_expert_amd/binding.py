"""Thin ctypes binding of ``libgrouped_expert_amd.so``.

Argument marshalling only: every step of the layer runs in the library's
HIP kernels.  PyTorch provides device memory and the current HIP stream.
The functions keep the C names without the ``moe_`` prefix, allocate their
outputs (and the workspaces the library asks for) as torch tensors on the
input's device, and raise :class:`MoEError` on a negative status.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgrouped_expert_amd.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "moe.h")

MOE_F32, MOE_BF16, MOE_FP8_ROW, MOE_FP8_B128 = 0, 1, 2, 3
MOE_ESCRATCH = -5
PERMUTE_NOALLOC_SCRATCH_BYTES = 4 << 20
FP8_CODES = {"row": MOE_FP8_ROW, "b128": MOE_FP8_B128}
MOE_GATING_SOFTMAX_TOPK_RENORM = 0
MOE_GATING_SOFTMAX_TOPK = 1                 # V1
MOE_GATING_SOFTMAX_GROUP_LIMITED = 2        # V2
MOE_GATING_SIGMOID_BIAS_GROUP_TOP2 = 3      # V3
FLAG_BAD_EXPERT, FLAG_NONFINITE_LOGIT, FLAG_BAD_HEADER, FLAG_BAD_INDEX, FLAG_BAD_SEGMENT = 1, 2, 4, 8, 16
FLAG_NONFINITE_INPUT = 32


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {msg} (status {status})")
        self.status = status


_i32, _i64, _sz, _p = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p

_SIGS = {
    "moe_strerror": (ctypes.c_char_p, [_i32]),
    "moe_version": (ctypes.c_int, []),
    "moe_route_topk": (ctypes.c_int, [_p, _i64, _i32, _i32, _i32, _p, _p, _p, _p]),
    "moe_route_topk_grouped": (ctypes.c_int, [_p, _i64, _i32, _i32, _i32, _i32, _i32, ctypes.c_float, _p, _p, _p,
                                              _p, _p]),
    "moe_permute_workspace": (_sz, [_i64, _i32, _i32]),
    "moe_permute": (ctypes.c_int, [_p, _i32, _i64, _i32, _p, _i32, _i32, _i64, _p, _p, _p, _p, _p, _p, _p,
                                   _p, _sz, _p, _p]),
    "moe_permute_noalloc": (ctypes.c_int, [_p, _i32, _i64, _i32, _p, _i32, _i32, _i64, _p, _p, _p, _p, _p, _p,
                                           _p, _p, _p]),
    "moe_grouped_swiglu_workspace": (_sz, [_i64, _i32, _i32, _i32]),
    "moe_grouped_swiglu": (ctypes.c_int, [_p, _i32, _i32, _i32, _i32, _p, _p, _i64, _p, _p, _p, _p, _i32, _p,
                                          _i64, _p, _p, _sz, _p, _p]),
    "moe_unpermute_combine": (ctypes.c_int, [_p, _i32, _i32, _p, _i64, _i64, _p, _i64, _i32, _p, _i32, _p, _p]),
    "moe_combine_backward": (ctypes.c_int, [_p, _i64, _i32, _p, _i32, _i64, _p, _p, _i32, _p, _i32, _p, _p, _p]),
    "moe_grouped_swiglu_backward_workspace": (_sz, [_i64, _i32, _i32, _i32]),
    "moe_grouped_swiglu_backward": (ctypes.c_int, [_p, _i32, _i32, _i32, _p, _p, _i64, _p, _p, _p, _p, _p, _p,
                                                   _i32, _p, _p, _p, _p, _sz, _p, _p]),
    "moe_pool_pack_workspace": (_sz, [_i64, _i32, _i32]),
    "moe_pool_pack": (ctypes.c_int, [_p, _i32, _i32, _i64, _i32, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _p,
                                     _p, _p, _p, _p, _sz, _p, _p]),
    "moe_row_bytes": (_sz, [_i32, _i32]),
    "moe_pool_geometry": (ctypes.c_int, [_i32, _i32, _i64, _p, _p]),
    "moe_pool_rows_of_height": (ctypes.c_int, [_i32, _i32, _i64, _p]),
    "moe_quantize_fp8": (ctypes.c_int, [_p, _i32, _i64, _i32, _i32, _p, _p, _p]),
    "moe_dequantize_fp8": (ctypes.c_int, [_p, _i32, _i64, _i32, _p, _i32, _p, _p]),
    "moe_recv_compact_workspace": (_sz, [_i32, _i32, _i32]),
    "moe_expand_rows": (ctypes.c_int, [_p, _i32, _i32, _p, _i64, _i64, _p, _i32, _p, _p]),
    "moe_recv_compact": (ctypes.c_int, [_p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _p, _p,
                                        _p, _i32, _p, _sz, _p, _p]),
}


def header_functions(path: str = HEADER):
    """Names of the functions declared in ``include/moe.h``."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with grouped_expert_amd.build.build() "
                          "(or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = load_library()


def strerror(status: int) -> str:
    return lib.moe_strerror(status).decode()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise MoEError(fn, status, strerror(status))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need_gpu(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _expect(name: str, t: Optional[torch.Tensor], shape=None, dtype=None, numel: Optional[int] = None) -> None:
    """Host-side check of a tensor the kernels will index by the sizes they
    were given: a wrong shape or dtype would make them read or write outside
    it.  ``shape`` entries of None are free."""
    if t is None:
        return
    if dtype is not None:
        allowed = dtype if isinstance(dtype, tuple) else (dtype,)
        if t.dtype not in allowed:
            raise ValueError(f"{name}: dtype {t.dtype}, expected {' or '.join(str(a) for a in allowed)}")
    if shape is not None:
        if t.dim() != len(shape) or any(s is not None and int(a) != int(s) for a, s in zip(t.shape, shape)):
            raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name}: {t.numel()} elements, expected {numel}")


_FLOATS = (torch.float32, torch.bfloat16)


def _segments_ok(seg_start: torch.Tensor, seg_count: torch.Tensor, E: int) -> None:
    """int32 vectors of at least E entries (the kernels read the first E; an
    offsets vector with its sentinel serves as seg_start)."""
    for name, t in (("seg_start", seg_start), ("seg_count", seg_count)):
        _expect(name, t, (None,), torch.int32)
        if t.numel() < E:
            raise ValueError(f"{name}: {t.numel()} entries, expected at least {E}")


def _flags_ok(flags: Optional[torch.Tensor]) -> None:
    _expect("flags", flags, dtype=(torch.int32,))
    if flags is not None and flags.numel() < 1:
        raise ValueError("flags: needs one element")


def _ws(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def new_flags(device) -> torch.Tensor:
    return torch.zeros(1, dtype=torch.int32, device=device)


# ---------------------------------------------------------------------------

def route_topk(logits: torch.Tensor, k: int, gating: int = MOE_GATING_SOFTMAX_TOPK_RENORM,
               flags: Optional[torch.Tensor] = None):
    """Returns ``(topk_ids int32 [T,k], topk_w fp32 [T,k])``."""
    _expect("logits", logits, (None, None), torch.float32)
    _flags_ok(flags)
    _need_gpu(logits, flags)
    T, E = logits.shape
    ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _check("moe_route_topk", lib.moe_route_topk(_ptr(logits), T, E, k, gating, _ptr(ids), _ptr(w), _ptr(flags),
                                                _stream(logits.device)))
    return ids, w


def route_topk_grouped(logits: torch.Tensor, k: int, gating: int, n_group: int, topk_group: int,
                       route_scale: float, bias: Optional[torch.Tensor] = None,
                       flags: Optional[torch.Tensor] = None):
    """Group-restricted router (V2 / V3).  Returns ``(topk_ids, topk_w)``."""
    _expect("logits", logits, (None, None), torch.float32)
    _expect("bias", bias, (logits.shape[1],), torch.float32)
    _flags_ok(flags)
    _need_gpu(logits, bias, flags)
    T, E = logits.shape
    ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _check("moe_route_topk_grouped",
           lib.moe_route_topk_grouped(_ptr(logits), T, E, k, gating, n_group, topk_group, float(route_scale),
                                      _ptr(bias), _ptr(ids), _ptr(w), _ptr(flags), _stream(logits.device)))
    return ids, w


def permute(x: Optional[torch.Tensor], topk_ids: torch.Tensor, E: int, capacity: int = -1,
            materialize: bool = True, flags: Optional[torch.Tensor] = None, payload: Optional[str] = None,
            d: Optional[int] = None):
    """``topk_ids`` is ``[T, k]``.  Returns a dict with x_perm (None when not
    materialised), src, inv, sel, counts, offsets, dropped.  With ``payload``
    "row" / "b128", ``x`` holds fp8 records of rows ``d`` wide and x_perm
    receives whole records."""
    _expect("topk_ids", topk_ids, (None, None), torch.int32)
    _flags_ok(flags)
    if materialize or x is not None:
        if x is None:
            raise ValueError("x: required to materialise x_perm")
        _expect("x", x, (topk_ids.shape[0], None), _FLOATS if payload is None else torch.uint8)
    _need_gpu(x, topk_ids, flags)
    T, k = topk_ids.shape
    dev = topk_ids.device
    R = T * k
    xp = None
    if materialize:
        xp = torch.empty((R, x.shape[1]), dtype=x.dtype, device=dev)
    src = torch.empty(R, dtype=torch.int32, device=dev)
    inv = torch.empty(R, dtype=torch.int32, device=dev)
    sel = torch.empty(E, dtype=torch.int32, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    dropped = torch.empty(1, dtype=torch.int32, device=dev)
    nbytes = lib.moe_permute_workspace(T, k, E)
    ws = _ws(nbytes, dev)
    if payload is not None:
        dt, dd = FP8_CODES[payload], d
        assert x.dtype == torch.uint8 and x.shape[1] == row_bytes(d, payload), "fp8 payload: x holds records"
    else:
        dt, dd = (_dtype_code(x), x.shape[1]) if x is not None else (MOE_BF16, 0)
    _check("moe_permute", lib.moe_permute(_ptr(x), dt, T, dd, _ptr(topk_ids), k, E,
                                          capacity, _ptr(xp), _ptr(src), _ptr(inv), _ptr(sel), _ptr(counts),
                                          _ptr(offsets), _ptr(dropped), _ptr(ws), ws.numel(), _ptr(flags),
                                          _stream(dev)))
    return dict(x_perm=xp, src=src, inv=inv, sel=sel, counts=counts, offsets=offsets, dropped=dropped)


def permute_noalloc(x: Optional[torch.Tensor], topk_ids: torch.Tensor, E: int, capacity: int = -1,
                    out: Optional[dict] = None, flags: Optional[torch.Tensor] = None):
    """:func:`permute` through the entry point that allocates nothing (its
    rank table is the library's static per-GPU scratch).  ``out`` may hold
    preallocated outputs (keys of :func:`permute`'s result); missing ones are
    allocated here, by torch, before the call."""
    _expect("topk_ids", topk_ids, (None, None), torch.int32)
    _flags_ok(flags)
    _need_gpu(x, topk_ids, flags)
    T, k = topk_ids.shape
    dev = topk_ids.device
    R = T * k
    o = dict(out or {})
    if x is not None:
        _expect("x", x, (T, None), _FLOATS)
        o.setdefault("x_perm", torch.empty((R, x.shape[1]), dtype=x.dtype, device=dev))
        _expect("x_perm", o["x_perm"], (R, x.shape[1]), x.dtype)
    for name, n in (("src", R), ("inv", R), ("sel", E), ("counts", E), ("offsets", E + 1), ("dropped", 1)):
        o.setdefault(name, torch.empty(n, dtype=torch.int32, device=dev))
        _expect(name, o[name], None, torch.int32, n)
    dt, dd = (_dtype_code(x), x.shape[1]) if x is not None else (MOE_BF16, 0)
    _check("moe_permute_noalloc", lib.moe_permute_noalloc(
        _ptr(x), dt, T, dd, _ptr(topk_ids), k, E, capacity, _ptr(o.get("x_perm")), _ptr(o["src"]), _ptr(o["inv"]),
        _ptr(o["sel"]), _ptr(o["counts"]), _ptr(o["offsets"]), _ptr(o["dropped"]), _ptr(flags), _stream(dev)))
    o.setdefault("x_perm", None)
    return o


def grouped_swiglu(x: torch.Tensor, seg_start: torch.Tensor, seg_count: torch.Tensor, w_gate: torch.Tensor,
                   w_up: torch.Tensor, w_down: torch.Tensor, z_dtype=torch.float32,
                   z: Optional[torch.Tensor] = None, flags: Optional[torch.Tensor] = None,
                   z_rows: Optional[torch.Tensor] = None, act: Optional[torch.Tensor] = None):
    """Runs expert ``e`` on rows ``[seg_start[e], seg_start[e]+seg_count[e])``
    of ``x``; returns ``z`` (rows outside every segment are left as allocated).

    With ``act`` (bf16, :func:`new_act` of ``x``'s rows and ``d_ff``) the call
    also saves the activations :func:`grouped_swiglu_backward` can take.

    With ``z_rows`` (int32 ``[rows]``, e.g. ``recv_compact``'s ``slot_row``)
    row ``i`` of the result is stored as row ``z_rows[i]`` of ``z``, which
    must then be given (any row count); rows mapped outside it are dropped."""
    _expect("x", x, (None, None), _FLOATS)
    rows, d = x.shape
    _expect("w_gate", w_gate, (None, None, d), x.dtype)
    E, d_ff, _ = w_gate.shape
    _expect("w_up", w_up, (E, d_ff, d), x.dtype)
    _expect("w_down", w_down, (E, d, d_ff), x.dtype)
    _segments_ok(seg_start, seg_count, E)
    if z_rows is not None:
        if z is None:
            raise ValueError("z_rows needs the output z")
        _expect("z_rows", z_rows, (rows,), torch.int32)
        _expect("z", z, (None, d), _FLOATS)
    else:
        _expect("z", z, (rows, d), _FLOATS)
    if act is not None:
        _expect("act", act, (3 * rows * d_ff,), torch.bfloat16)
        if x.dtype != torch.bfloat16:
            raise ValueError("act: saved activations need the bf16 path")
    _flags_ok(flags)
    _need_gpu(x, seg_start, seg_count, w_gate, w_up, w_down, z, flags, z_rows, act)
    dev = x.device
    if z is None:
        z = torch.empty((rows, d), dtype=z_dtype, device=dev)
    dt = _dtype_code(x)
    ws = _ws(lib.moe_grouped_swiglu_workspace(rows, E, d_ff, dt), dev)
    _check("moe_grouped_swiglu", lib.moe_grouped_swiglu(
        _ptr(x), dt, d, d_ff, E, _ptr(seg_start), _ptr(seg_count), rows, _ptr(w_gate), _ptr(w_up), _ptr(w_down),
        _ptr(z), _dtype_code(z), _ptr(z_rows), z.shape[0] if z_rows is not None else 0, _ptr(act), _ptr(ws),
        ws.numel(), _ptr(flags), _stream(dev)))
    return z


def new_act(rows: int, d_ff: int, device) -> torch.Tensor:
    """Buffer for the saved activations of :func:`grouped_swiglu` (G | U, then
    H: ``3 * rows * d_ff`` bf16)."""
    return torch.empty(3 * rows * d_ff, dtype=torch.bfloat16, device=device)


def unpermute_combine(z: torch.Tensor, idx: torch.Tensor, gates: Optional[torch.Tensor], T: int, k: int,
                      lo: int = 0, hi: Optional[int] = None, y: Optional[torch.Tensor] = None,
                      accumulate: bool = False, flags: Optional[torch.Tensor] = None):
    """``y[t] (+)= sum_j g[t,j] z[idx[t,j] - lo]`` over routes inside ``[lo, hi)``."""
    _expect("z", z, (None, None), _FLOATS)
    d = z.shape[-1]
    if hi is None:
        hi = lo + z.shape[0]
    if hi - lo > z.shape[0]:
        raise ValueError(f"z: {z.shape[0]} rows, window [lo, hi) needs {hi - lo}")
    _expect("idx", idx, None, torch.int32, T * k)
    _expect("gates", gates, None, torch.float32, T * k)
    _expect("y", y, (T, d), torch.float32)
    _flags_ok(flags)
    _need_gpu(z, idx, gates, y, flags)
    dev = idx.device
    if y is None:
        y = torch.empty((T, d), dtype=torch.float32, device=dev)
        accumulate = False
    _check("moe_unpermute_combine", lib.moe_unpermute_combine(
        _ptr(z), _dtype_code(z), d, _ptr(idx), lo, hi, _ptr(gates), T, k, _ptr(y), int(accumulate), _ptr(flags),
        _stream(dev)))
    return y


def row_bytes(d: int, payload: Optional[str] = None) -> int:
    """Bytes of one dispatched row: bf16 (payload None) or an fp8 record
    ("row": one fp32 scale per row, "b128": one per 128 values)."""
    return int(lib.moe_row_bytes(MOE_BF16 if payload is None else FP8_CODES[payload], d))


def _row_code(payload: Optional[str]) -> int:
    return MOE_BF16 if payload is None else FP8_CODES[payload]


def pool_geometry(pool_rows: int, d: int, payload: Optional[str] = None):
    """``(header_rows, pool_height)`` of a pool as the library lays it out."""
    h, ph = ctypes.c_int64(), ctypes.c_int64()
    _check("moe_pool_geometry", lib.moe_pool_geometry(_row_code(payload), d, int(pool_rows), ctypes.byref(h),
                                                      ctypes.byref(ph)))
    return int(h.value), int(ph.value)


def header_rows(pool_rows: int, d: int, payload: Optional[str] = None) -> int:
    """Header rows of a pool (the library's geometry query)."""
    return pool_geometry(pool_rows, d, payload)[0]


def pool_height(pool_rows: int, d: int, payload: Optional[str] = None) -> int:
    """Rows of one pool: data rows plus header rows (the library's query)."""
    return pool_geometry(pool_rows, d, payload)[1]


def pool_rows_of_height(height: int, d: int, payload: Optional[str] = None) -> int:
    """Data rows of a pool that is ``height`` rows tall (the library's query)."""
    p = ctypes.c_int64()
    st = lib.moe_pool_rows_of_height(_row_code(payload), d, int(height), ctypes.byref(p))
    if st != 0:
        raise ValueError(f"no pool of row width {d} is {height} rows tall")
    return int(p.value)


def quantize_fp8(x: torch.Tensor, payload: str = "b128", rec: Optional[torch.Tensor] = None,
                 flags: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Rows ``[n, d]`` (bf16 or fp32) to fp8 records ``uint8 [n, row_bytes]``."""
    _expect("x", x, (None, None), _FLOATS)
    n, d = x.shape
    _expect("rec", rec, (n, row_bytes(d, payload)), torch.uint8)
    _flags_ok(flags)
    _need_gpu(x, rec, flags)
    if rec is None:
        rec = torch.empty((n, row_bytes(d, payload)), dtype=torch.uint8, device=x.device)
    _check("moe_quantize_fp8", lib.moe_quantize_fp8(_ptr(x), _dtype_code(x), n, d, FP8_CODES[payload], _ptr(rec),
                                                     _ptr(flags), _stream(x.device)))
    return rec


def dequantize_fp8(rec: torch.Tensor, d: int, payload: str = "b128", out_dtype: torch.dtype = torch.bfloat16,
                   out: Optional[torch.Tensor] = None, flags: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp8 records back to ``[n, d]`` rows of ``out_dtype``."""
    _expect("rec", rec, (None, row_bytes(d, payload)), torch.uint8)
    n = rec.shape[0]
    _expect("out", out, (n, d), _FLOATS)
    _flags_ok(flags)
    _need_gpu(rec, out, flags)
    if out is None:
        out = torch.empty((n, d), dtype=out_dtype, device=rec.device)
    _check("moe_dequantize_fp8", lib.moe_dequantize_fp8(_ptr(rec), FP8_CODES[payload], n, d, _ptr(out),
                                                         _dtype_code(out), _ptr(flags), _stream(rec.device)))
    return out


def combine_backward(dy: torch.Tensor, z: torch.Tensor, idx: torch.Tensor, gates: torch.Tensor, k: int,
                     dz_dtype: torch.dtype = torch.bfloat16, dz: Optional[torch.Tensor] = None,
                     flags: Optional[torch.Tensor] = None):
    """Route gradients ``dz[idx[r]] = g_r dy[t]`` and gate gradients
    ``<dy[t], z[idx[r]]>``; returns ``(dz, dgates [T, k])``."""
    _expect("dy", dy, (None, None), torch.float32)
    T, d = dy.shape
    _expect("z", z, (None, d), _FLOATS)
    rows = z.shape[0]
    _expect("idx", idx, None, torch.int32, T * k)
    _expect("gates", gates, None, torch.float32, T * k)
    _expect("dz", dz, (rows, d), _FLOATS)
    _flags_ok(flags)
    _need_gpu(dy, z, idx, gates, dz, flags)
    if dz is None:
        dz = torch.empty((rows, d), dtype=dz_dtype, device=dy.device)
    dg = torch.empty((T, k), dtype=torch.float32, device=dy.device)
    _check("moe_combine_backward", lib.moe_combine_backward(
        _ptr(dy), T, d, _ptr(z), _dtype_code(z), rows, _ptr(idx), _ptr(gates), k, _ptr(dz), _dtype_code(dz),
        _ptr(dg), _ptr(flags), _stream(dy.device)))
    return dz, dg


def grouped_swiglu_backward(x: torch.Tensor, dz: torch.Tensor, seg_start: torch.Tensor, seg_count: torch.Tensor,
                            w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor,
                            dx_dtype: torch.dtype = torch.float32, dx: Optional[torch.Tensor] = None,
                            flags: Optional[torch.Tensor] = None, act: Optional[torch.Tensor] = None):
    """Expert backward over the segments; returns a dict with dx (route-input
    gradients, rows of x), dw_gate, dw_up, dw_down (fp32).  With ``act`` (the
    activations a :func:`grouped_swiglu` call saved for the same ``x`` and
    segments) G, U and H are taken from it instead of recomputed."""
    _expect("x", x, (None, None), torch.bfloat16)
    rows, d = x.shape
    _expect("dz", dz, (rows, d), torch.bfloat16)
    _expect("w_gate", w_gate, (None, None, d), torch.bfloat16)
    E, d_ff, _ = w_gate.shape
    _expect("w_up", w_up, (E, d_ff, d), torch.bfloat16)
    _expect("w_down", w_down, (E, d, d_ff), torch.bfloat16)
    _segments_ok(seg_start, seg_count, E)
    _expect("dx", dx, (rows, d), _FLOATS)
    if act is not None:
        _expect("act", act, (3 * rows * d_ff,), torch.bfloat16)
    _flags_ok(flags)
    _need_gpu(x, dz, seg_start, seg_count, w_gate, w_up, w_down, dx, flags, act)
    dev = x.device
    if dx is None:
        dx = torch.empty((rows, d), dtype=dx_dtype, device=dev)
    dwg = torch.empty((E, d_ff, d), dtype=torch.float32, device=dev)
    dwu = torch.empty((E, d_ff, d), dtype=torch.float32, device=dev)
    dwd = torch.empty((E, d, d_ff), dtype=torch.float32, device=dev)
    ws = _ws(lib.moe_grouped_swiglu_backward_workspace(rows, E, d, d_ff), dev)
    _check("moe_grouped_swiglu_backward", lib.moe_grouped_swiglu_backward(
        _ptr(x), d, d_ff, E, _ptr(seg_start), _ptr(seg_count), rows, _ptr(w_gate), _ptr(w_up), _ptr(w_down),
        _ptr(dz), _ptr(act), _ptr(dx), _dtype_code(dx), _ptr(dwg), _ptr(dwu), _ptr(dwd), _ptr(ws), ws.numel(),
        _ptr(flags), _stream(dev)))
    return dict(dx=dx, dw_gate=dwg, dw_up=dwu, dw_down=dwd)


def expand_rows(z: torch.Tensor, row_slot: torch.Tensor, ret_dtype: torch.dtype = torch.float32,
                ret: Optional[torch.Tensor] = None, flags: Optional[torch.Tensor] = None):
    """``ret[i] = z[row_slot[i]]`` (converted) or a zero row; returns ``ret``."""
    _expect("z", z, None, _FLOATS)
    _expect("row_slot", row_slot, None, torch.int32)
    d = z.shape[-1]
    n_slots = z.numel() // d
    n = row_slot.numel()
    _expect("ret", ret, None, _FLOATS, n * d)
    _flags_ok(flags)
    _need_gpu(z, row_slot, ret, flags)
    if ret is None:
        ret = torch.empty((n, d), dtype=ret_dtype, device=row_slot.device)
    _check("moe_expand_rows", lib.moe_expand_rows(
        _ptr(z), _dtype_code(z), d, _ptr(row_slot), n, n_slots, _ptr(ret), _dtype_code(ret), _ptr(flags),
        _stream(row_slot.device)))
    return ret


def pool_pack(x: torch.Tensor, topk_ids: torch.Tensor, E: int, experts_per_dest: int, n_dest: int, n_waves: int,
              pool_rows: int, wave: int = -1, pools: Optional[torch.Tensor] = None,
              flags: Optional[torch.Tensor] = None, payload: Optional[str] = None, d: Optional[int] = None):
    """Returns a dict with pools, route_loc, dest_counts, sender_dropped.

    ``x`` is bf16 ``[T, d]`` (pools bf16 ``[..., PH, d]``).  With ``payload``
    "row" / "b128" the pools hold fp8 records (uint8 ``[..., PH, row_bytes]``)
    and ``x`` is either those records (``uint8 [T, row_bytes]`` of rows ``d``
    wide) or bf16 rows that the pack quantizes on the way."""
    _expect("x", x, (None, None), (torch.bfloat16, torch.uint8))
    _expect("topk_ids", topk_ids, (x.shape[0], None), torch.int32)
    _flags_ok(flags)
    _need_gpu(x, topk_ids, pools, flags)
    T = x.shape[0]
    if payload is None:
        d = x.shape[1]
        code, last, pdt = MOE_BF16, d, torch.bfloat16
    else:
        code, last, pdt = FP8_CODES[payload], row_bytes(d, payload), torch.uint8
        if x.dtype == torch.bfloat16:
            d = x.shape[1] if d is None else d
            assert x.shape[1] == d
        else:
            assert x.dtype == torch.uint8 and x.shape[1] == last, "fp8 payload: x holds records or bf16 rows"
    xcode = MOE_BF16 if x.dtype == torch.bfloat16 else code
    k = topk_ids.shape[-1]
    dev = x.device
    PH = pool_height(pool_rows, d, payload)
    shape = (n_waves, n_dest, PH, last) if wave < 0 else (n_dest, PH, last)
    if pools is None:
        pools = torch.empty(shape, dtype=pdt, device=dev)
    _expect("pools", pools, shape, pdt)
    route_loc = torch.empty(T * k, dtype=torch.int32, device=dev)
    dest_counts = torch.empty(n_dest, dtype=torch.int32, device=dev)
    dropped = torch.empty(1, dtype=torch.int32, device=dev)
    ws = _ws(lib.moe_pool_pack_workspace(T, k, n_dest), dev)
    _check("moe_pool_pack", lib.moe_pool_pack(
        _ptr(x), xcode, code, T, d, _ptr(topk_ids), k, E, experts_per_dest, n_dest, n_waves, pool_rows, wave, _ptr(pools),
        _ptr(route_loc), _ptr(dest_counts), _ptr(dropped), _ptr(ws), ws.numel(), _ptr(flags), _stream(dev)))
    return dict(pools=pools, route_loc=route_loc, dest_counts=dest_counts, sender_dropped=dropped)


def recv_compact(pools_in: torch.Tensor, n_local: int, cap: int, compact: Optional[torch.Tensor] = None,
                 flags: Optional[torch.Tensor] = None, rotation: int = 0, payload: Optional[str] = None,
                 d: Optional[int] = None, slot_row: Optional[torch.Tensor] = None,
                 ret: Optional[torch.Tensor] = None):
    """Returns a dict with compact [n_local, cap, d] (bf16), counts, arrived, row_slot, recv_dropped
    (and slot_row when asked for).

    ``pools_in`` is ``[n_src, pool_height, d]`` bf16, or with ``payload``
    "row" / "b128" fp8 records ``uint8 [n_src, pool_height, row_bytes]`` of
    rows ``d`` wide (dequantized into ``compact``); sources are visited from
    ``rotation`` onwards.  ``slot_row`` (int32 ``[n_local*cap]``, or True to
    allocate it) receives the pool row of every filled slot; ``ret``
    (``[n_src*pool_height, d]`` fp32 or bf16) gets zero rows wherever
    ``row_slot`` is -1, for a grouped SwiGLU that stores its results through
    ``z_rows=slot_row`` into the same ``ret``."""
    _expect("pools_in", pools_in, (None, None, None), torch.bfloat16 if payload is None else torch.uint8)
    _flags_ok(flags)
    _need_gpu(pools_in, compact, flags)
    S, P1 = pools_in.shape[0], pools_in.shape[1]
    if payload is None:
        d = pools_in.shape[2]
        code = MOE_BF16
    else:
        code = FP8_CODES[payload]
        assert pools_in.dtype == torch.uint8 and pools_in.shape[2] == row_bytes(d, payload)
    P = pool_rows_of_height(P1, d, payload)
    dev = pools_in.device
    if compact is None:
        compact = torch.empty((n_local, cap, d), dtype=torch.bfloat16, device=dev)
    _expect("compact", compact, None, torch.bfloat16, n_local * cap * d)
    counts = torch.empty(n_local, dtype=torch.int32, device=dev)
    arrived = torch.empty(n_local, dtype=torch.int32, device=dev)
    row_slot = torch.empty(S * P1, dtype=torch.int32, device=dev)
    dropped = torch.empty(1, dtype=torch.int32, device=dev)
    if slot_row is True:
        slot_row = torch.empty(n_local * cap, dtype=torch.int32, device=dev)
    _expect("slot_row", slot_row, None, torch.int32, n_local * cap)
    _expect("ret", ret, (S * P1, d), _FLOATS)
    _need_gpu(slot_row, ret)
    ws = _ws(lib.moe_recv_compact_workspace(S, P, n_local), dev)
    _check("moe_recv_compact", lib.moe_recv_compact(
        _ptr(pools_in), code, S, P, d, n_local, cap, rotation, _ptr(compact), _ptr(counts), _ptr(arrived),
        _ptr(row_slot), _ptr(dropped), _ptr(slot_row), _ptr(ret), _dtype_code(ret) if ret is not None else 0,
        _ptr(ws), ws.numel(), _ptr(flags), _stream(dev)))
    out = dict(compact=compact, counts=counts, arrived=arrived, row_slot=row_slot, recv_dropped=dropped)
    if slot_row is not None:
        out["slot_row"] = slot_row
    return out
