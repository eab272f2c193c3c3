"""The layer as a chain of library calls (marshalling only).

``moe_layer`` is one pass of the routed-expert layer on a token batch:
route -> permute -> grouped SwiGLU -> un-permute/combine, all on the current
stream with no host synchronisation ("M6.6 - MoE Runtime Systems", 0x0CC
forward blueprint, reduced to one GPU).  ``loopback_wave`` is one wave of
the pooled-wave receiver path fed with a sender's pools ("Fixed pooled-wave
all-to-all for the 8-of-384 MoE", 03): compaction -> batched SwiGLU over the
static arrays, its results stored straight into pool rows (compaction zeroes
the rows without a slot) -> sender combine into the FP32 accumulator.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import binding as B


def moe_layer(x: torch.Tensor, logits: torch.Tensor, w_gate: torch.Tensor, w_up: torch.Tensor,
              w_down: torch.Tensor, k: int, capacity: int = -1, z_dtype: Optional[torch.dtype] = None,
              flags: Optional[torch.Tensor] = None, save_act: bool = False):
    """Returns ``(y fp32 [T, d], state)`` where state holds the intermediate
    routing and dispatch tensors; with ``save_act`` (bf16) also the experts'
    activations for :func:`moe_layer_backward`, which then reads each weight
    once instead of recomputing the gate/up product."""
    E = w_gate.shape[0]
    T = x.shape[0]
    if z_dtype is None:
        z_dtype = torch.float32 if x.dtype == torch.float32 else torch.bfloat16
    ids, gates = B.route_topk(logits, k, flags=flags)
    plan = B.permute(x, ids, E, capacity, flags=flags)
    act = B.new_act(plan["x_perm"].shape[0], w_gate.shape[1], x.device) if save_act else None
    z = B.grouped_swiglu(plan["x_perm"], plan["offsets"], plan["counts"], w_gate, w_up, w_down,
                         z_dtype=z_dtype, flags=flags, act=act)
    y = B.unpermute_combine(z, plan["inv"], gates, T, k, flags=flags)
    return y, dict(ids=ids, gates=gates, plan=plan, z=z, act=act)


def moe_layer_backward(dy: torch.Tensor, x: torch.Tensor, state: dict, w_gate: torch.Tensor, w_up: torch.Tensor,
                       w_down: torch.Tensor, flags: Optional[torch.Tensor] = None):
    """Backward of :func:`moe_layer` from its saved state ("M6.2 - Expert
    Parallelism and DeepSeek MoE", 0x03D: the permutation, the inverse map,
    the gates, the segments and the expert outputs are backward state):
    route and gate gradients, the expert backward over the segments, then the
    route-input gradients summed by origin token through the inverse map.

    Returns ``(dx fp32 [T, d], grads)`` with ``grads`` holding ``dgates``
    ``[T, k]``, ``dw_gate``, ``dw_up``, ``dw_down`` (fp32) and the
    intermediate ``dz`` / ``dx_rows``."""
    plan = state["plan"]
    T, k = state["ids"].shape
    dz, dg = B.combine_backward(dy, state["z"], plan["inv"], state["gates"], k, dz_dtype=x.dtype, flags=flags)
    bw = B.grouped_swiglu_backward(plan["x_perm"], dz, plan["offsets"], plan["counts"], w_gate, w_up, w_down,
                                   flags=flags, act=state.get("act"))
    dx = B.unpermute_combine(bw["dx"], plan["inv"], None, T, k, flags=flags)
    return dx, dict(dgates=dg, dw_gate=bw["dw_gate"], dw_up=bw["dw_up"], dw_down=bw["dw_down"], dz=dz,
                    dx_rows=bw["dx"])


def loopback_wave(pools_w: torch.Tensor, wave: int, n_waves: int, route_loc: torch.Tensor, gates: torch.Tensor,
                  T: int, k: int, w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor, cap: int,
                  y: torch.Tensor, flags: Optional[torch.Tensor] = None, bufs: Optional[dict] = None,
                  rotation: int = 0, ret_dtype: torch.dtype = torch.float32, payload: Optional[str] = None):
    """One wave of the receiver path; adds the wave's contributions into ``y``.
    Returns ``(rc, ret)``: the compaction's outputs and the return rows
    ``[n_src * pool_height, d]`` in pool-row order.

    ``pools_w`` is ``[n_src, pool_height, d]`` (one wave's pools, header rows
    included).  ``bufs`` may hold preallocated ``compact``/``slot_row``/``ret``
    tensors to reuse; ``rotation`` is the receiver's first source.  With
    ``ret_dtype`` bf16 the expert rows leave the GEMM as bf16 and the return
    buffer is bf16 ("M6.6 - MoE Runtime Systems", 0x0AE); the combine still
    accumulates in FP32.  With ``payload`` "row" / "b128" the pools hold fp8
    records and the compaction dequantizes them ("M6.2", 0x0AC)."""
    S, P1 = pools_w.shape[0], pools_w.shape[1]
    L = w_gate.shape[0]
    d = w_down.shape[1]
    bufs = {} if bufs is None else bufs
    ret = bufs.get("ret")
    if ret is None:
        ret = torch.empty((S * P1, d), dtype=ret_dtype, device=pools_w.device)
    rc = B.recv_compact(pools_w, L, cap, compact=bufs.get("compact"), flags=flags, rotation=rotation,
                        payload=payload, d=d, slot_row=bufs.get("slot_row", True), ret=ret)
    starts = torch.arange(L, dtype=torch.int32, device=pools_w.device) * cap
    B.grouped_swiglu(rc["compact"].view(L * cap, d), starts, rc["counts"], w_gate, w_up, w_down,
                     z=ret, z_rows=rc["slot_row"], flags=flags)
    lo = wave * S * P1
    B.unpermute_combine(ret, route_loc, gates, T, k, lo=lo, hi=lo + S * P1, y=y, accumulate=True, flags=flags)
    return rc, ret
