"""CPU oracle of the single-GPU MoE routed-expert layer (fp64, numpy).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import, call or execute this file.
It shares no code with the HIP library and imports nothing from it.

Sources (page title, then section):

* "M6.6 - MoE Runtime Systems: Placement, Dispatch, Kernels, and Topology"
  (cited as *M6.6*): §0x03A router-side tensors, §0x03B count / prefix /
  stable permute, §0x03C3 inverse composition and weighted scatter-add
  combine, §0x04A SwiGLU expert and its FLOP count, §0x04B-§0x04F row
  ledgers, §0x0AE dtype roles, §0x0CD route and combine assertions.
* "M6.2 - Expert Parallelism and DeepSeek MoE" (cited as *M6.2*): §0x01C
  capacity, §0x03B count / prefix / permute, §0x03C forward transpose,
  §0x03G executable logical transpose and its rejection list, §0x04D the two
  layouts (token-major repeat vs expert-major sort), §0x06L1 family table
  (Mixtral row: FP32 softmax, top-k, renormalise to one),
  §0x03D backward as the reverse semantic transpose.
* "Fixed pooled-wave all-to-all for the 8-of-384 MoE" (cited as *pooled
  wave*): §02 pools and stripe rule, §03 one wave, §04 capacities, §05 drop
  metrics, §07 fixed source order on the receiver.
* "Dispatch and combine: preserve token identity across expert ranks"
  (cited as *dispatch and combine*): keep the inverse map; bijection.

Every floating-point value is computed in float64 from the exact stored
input values (fp32 and bf16 upcast without rounding).  Integer results are
unique given the readings below, so they are compared bit-exactly.

Readings where the pages leave a step open (each is also listed in the design
notes):

* Selection is done on the fp32 logits (softmax is monotone); equal values
  (-0.0 == +0.0) rank the lower expert index first.
* A token with any non-finite logit is invalid: all of its slots get expert
  id -1 and weight 0 (id -1 is the "no route" sentinel downstream).
* Inside a segment routes keep route order ``r = t*k + j``; a capacity keeps
  the first ``C`` routes of an expert in that order and drops the rest.
* A dropped route contributes nothing; the gates are never renormalised
  after a drop.
* Pooled-wave stripe: a route's ordinal among this sender's routes to the
  same destination is its destination rank; ``wave = rank mod n_waves``,
  ``pool row = rank div n_waves``.  Expert ``e`` lives on destination
  ``e div experts_per_dest`` as local expert ``e mod experts_per_dest``.
* Header row: row 0 of each pool; element ``i`` is the 16-bit local expert id
  of data row ``i`` (pool row ``1 + i``) or 0xFFFF when that row is empty;
  elements past ``pool_rows`` are 0xFFFF.  Empty data rows are zero.  (This
  bit format is not printed on the pages: parity unpinned by them.)
* Receiver order is (source pool, row) ascending; a local expert keeps its
  first ``cap`` arrivals.  Rows the receiver drops return as zero rows.
"""
from __future__ import annotations

import dataclasses
from typing import Callable, Optional, Tuple

import numpy as np

__all__ = [
    "HEADER_EMPTY", "bf16_to_f64", "to_f64",
    "route_topk", "route_v1", "group_limited_select", "route_v2", "sigmoid_f32", "sigmoid_f32_ambiguous",
    "route_v3",
    "DispatchPlan", "dispatch_plan", "check_dispatch",
    "gather_rows", "silu", "swiglu_expert", "swiglu_bank", "scalar_bank", "run_segments",
    "combine", "moe_layer_token_major", "moe_layer_expert_major",
    "combine_backward", "silu_grad", "swiglu_expert_backward", "swiglu_bank_backward",
    "scalar_bank_backward", "run_segments_backward", "moe_layer_backward",
    "header_rows", "header_rows_bytes", "pool_rows_of", "pool_rows_of_bytes", "pool_pack", "recv_compact",
    "expand_rows", "loopback_layer",
    "FP8_E4M3_MAX", "FP8_MODES", "fp8_e4m3_decode", "fp8_e4m3_encode", "fp8_record_layout", "fp8_payload_bytes",
    "quantize_fp8_rows", "dequantize_fp8_rows", "f32_to_bf16_rne",
    "capacity_ceil", "drop_rates", "swiglu_flops", "padded_exec_rows",
    "block_exec_rows",
]

HEADER_EMPTY = 0xFFFF


# ----------------------------------------------------------------------------
# exact upcasts
# ----------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns: the pattern is the top half of an
    IEEE binary32 word, so shifting it up and reinterpreting is exact."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def to_f64(a: np.ndarray) -> np.ndarray:
    """fp32 arrays and bf16 bit arrays (uint16) to exact float64."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_to_f64(a)
    return a.astype(np.float64)


# ----------------------------------------------------------------------------
# a1: router top-k with softmax-renormalised gates
# ----------------------------------------------------------------------------

def route_topk(logits: np.ndarray, k: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Softmax over all experts, keep the top ``k``, renormalise the kept mass.

    M6.2 §0x06L1 (Mixtral row): FP32 softmax over all experts, top-2,
    selected probabilities renormalised to one.  M6.6 §0x0AE: logits and
    the top-k comparison are FP32.  M6.6 §0x03A: the router emits
    ``topk_ids [T,k]`` and ``topk_weights [T,k]``.

    Returns ``(ids int32 [T,k], gates float64 [T,k], invalid bool [T])``.
    """
    z = np.asarray(logits, dtype=np.float32)
    T, E = z.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    invalid = ~np.isfinite(z).all(axis=1)
    zc = (z + np.float32(0.0)).astype(np.float64)   # -0.0 becomes +0.0
    expert = np.broadcast_to(np.arange(E), (T, E))
    # lexsort: last key is primary.  Descending logit, then ascending expert.
    order = np.lexsort((expert, -zc), axis=-1)
    ids = order[:, :k].astype(np.int32)

    # softmax over all E experts in float64, then select and renormalise
    zz = np.where(invalid[:, None], 0.0, zc)
    m = zz.max(axis=1, keepdims=True)
    p = np.exp(zz - m)
    p /= p.sum(axis=1, keepdims=True)
    psel = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    gates = psel / psel.sum(axis=1, keepdims=True)

    ids[invalid] = -1
    gates[invalid] = 0.0
    return ids, gates, invalid


# ----------------------------------------------------------------------------
# a1 gating variants: V1 (no renormalisation), V2 (group-limited greedy on
# softmax, scaled), V3 (sigmoid affinity, selection bias, group top-2 sums,
# renormalised original affinities, scaled)
# ----------------------------------------------------------------------------

def _softmax64(z32: np.ndarray) -> np.ndarray:
    zz = z32.astype(np.float64)
    m = zz.max(axis=1, keepdims=True)
    p = np.exp(zz - m)
    return p / p.sum(axis=1, keepdims=True)


def route_v1(logits: np.ndarray, k: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Softmax over all experts, keep the top ``k``, no renormalisation.

    M6.2 §0x04D (released DeepSeekMoE checkpoint: softmax scores, top-6,
    norm_topk_prob false) and §0x06L3-§0x06L4 (V1 keeps the selected full
    probability mass, scale 1: selected sums 0.70 / 0.75 in the reduced
    fixture).  Selection is that of ``route_topk``; only the gates differ.
    """
    ids, _, invalid = route_topk(logits, k)
    z = np.asarray(logits, dtype=np.float32)
    p = _softmax64(np.where(invalid[:, None], np.float32(0), z))
    gates = np.take_along_axis(p, np.maximum(ids, 0).astype(np.int64), axis=1)
    gates[invalid] = 0.0
    return ids, gates, invalid


def _top2_sum_f32(v: np.ndarray) -> np.float32:
    """Sum of the two largest values, added in fp32 (larger + smaller)."""
    srt = np.sort(v.astype(np.float32))[::-1]
    return np.float32(srt[0] + srt[1])


def group_limited_select(scores: np.ndarray, n_group: int, topk_group: int, k: int,
                         group_stat: str) -> Tuple[np.ndarray, np.ndarray]:
    """Group-restricted top-k on selection scores ``[T, E]``.

    M6.2 §0x05A-§0x05B (V2: score each contiguous group by its best expert,
    keep ``topk_group`` groups, mask the others, then take ``k`` experts from
    the survivors) and §0x06B-§0x06C (V3: score a group by the sum of its two
    largest corrected scores, keep ``topk_group`` groups, then top-``k``).
    Groups are contiguous expert-id ranges of ``E / n_group``.  Groups and
    experts are ranked by descending score, ties to the lower index; the
    expert top-k ranges over the experts of the kept groups only.

    ``group_stat``: ``"max"`` or ``"top2sum"`` (the latter added in fp32,
    the precision the scores are given in).  Returns ``(ids int32 [T,k],
    groups int32 [T,topk_group])``, both in rank order.
    """
    sc = np.asarray(scores)
    T, E = sc.shape
    if E % n_group or not 1 <= topk_group <= n_group or k > topk_group * (E // n_group):
        raise ValueError("bad group geometry")
    gs = E // n_group
    ids = np.empty((T, k), dtype=np.int32)
    groups = np.empty((T, topk_group), dtype=np.int32)
    for t in range(T):
        row = sc[t]
        stat = []
        for g in range(n_group):
            members = row[g * gs:(g + 1) * gs]
            stat.append(float(members.max()) if group_stat == "max" else float(_top2_sum_f32(members)))
        g_order = sorted(range(n_group), key=lambda g: (-stat[g], g))[:topk_group]
        groups[t] = g_order
        eligible = [e for g in g_order for e in range(g * gs, (g + 1) * gs)]
        e_order = sorted(eligible, key=lambda e: (-float(row[e]), e))[:k]
        ids[t] = e_order
    return ids, groups


def route_v2(logits: np.ndarray, k: int, n_group: int, topk_group: int,
             route_scale: float) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """V2: FP32 softmax over all experts, group-limited greedy, no
    renormalisation, gates scaled by ``route_scale`` (M6.2 §0x05B: 8 groups,
    keep 3, top-6, scale 16).  Softmax is strictly monotone, so ranking groups
    by their best probability and experts by probability equals ranking by
    the fp32 logits; the selection is taken on the logits (-0.0 == +0.0)."""
    z = np.asarray(logits, dtype=np.float32)
    invalid = ~np.isfinite(z).all(axis=1)
    zc = np.where(invalid[:, None], np.float32(0), z + np.float32(0.0)).astype(np.float64)
    ids, _ = group_limited_select(zc, n_group, topk_group, k, "max")
    p = _softmax64(zc.astype(np.float32))
    gates = np.take_along_axis(p, ids.astype(np.int64), axis=1) * route_scale
    ids[invalid] = -1
    gates[invalid] = 0.0
    return ids, gates, invalid


def sigmoid_f32(z: np.ndarray) -> np.ndarray:
    """The V3 affinity as a decision key: the sigmoid ``1 / (1 + exp(-z))``
    evaluated in fp64 and rounded once to fp32 (nearest, ties to even).

    M6.2 §0x06I makes the selection from sigmoid scores plus an FP32
    correction bias, so the corrected score is an fp32 value; the pages leave
    open how the fp32 affinity itself is obtained.  Reading: the fp32 value
    nearest to the sigmoid.  Evaluated in fp64 (relative error near 2^-52),
    that rounding is exact unless the sigmoid lies within about 2^-45 of an
    fp32 rounding midpoint (``sigmoid_f32_ambiguous``)."""
    z64 = np.asarray(z, dtype=np.float32).astype(np.float64)
    with np.errstate(over="ignore"):
        return (1.0 / (1.0 + np.exp(-z64))).astype(np.float32)


def sigmoid_f32_ambiguous(z: np.ndarray, rel: float = 2.0 ** -45) -> Tuple[np.ndarray, np.ndarray]:
    """Where rounding the fp64 sigmoid to fp32 is not determined by an fp64
    evaluation: the value lies within ``rel`` (relative) of the midpoint
    between two adjacent fp32 values.  Returns ``(mask, other)``: ``other``
    holds the fp32 neighbour on the far side of that midpoint (equal to
    ``sigmoid_f32`` where ``mask`` is false)."""
    z64 = np.asarray(z, dtype=np.float32).astype(np.float64)
    with np.errstate(over="ignore"):
        s64 = 1.0 / (1.0 + np.exp(-z64))
    s32 = s64.astype(np.float32)
    up = np.nextafter(s32, np.float32(np.inf))
    dn = np.nextafter(s32, np.float32(-np.inf))
    other = np.where(s64 >= s32.astype(np.float64), up, dn).astype(np.float32)
    mid = (s32.astype(np.float64) + other.astype(np.float64)) / 2.0     # exact in fp64
    mask = np.abs(s64 - mid) <= rel * np.abs(s64)
    return mask, np.where(mask, other, s32)


def route_v3(logits: np.ndarray, bias: Optional[np.ndarray], k: int, n_group: int, topk_group: int,
             route_scale: float, affinity32: Optional[np.ndarray] = None
             ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """V3: sigmoid affinity ``s``, corrected score ``s + b`` (fp32) decides
    groups (sum of each group's two largest corrected scores) and experts;
    the gates return to the original affinities of the selected experts,
    renormalised and scaled by ``route_scale`` (M6.2 §0x06A-§0x06D, §0x06I:
    8 groups of 32, keep 4, top-8, scale 2.5).

    Decisions use the fp32 affinity of ``sigmoid_f32`` (or ``affinity32``
    when given, e.g. the other rounding of an ambiguous value) plus the fp32
    bias, added in fp32; gates use the fp64 sigmoid of the logits.
    """
    z = np.asarray(logits, dtype=np.float32)
    T, E = z.shape
    b = np.zeros(E, np.float32) if bias is None else np.asarray(bias, dtype=np.float32)
    s32 = sigmoid_f32(z) if affinity32 is None else np.asarray(affinity32, dtype=np.float32)
    corrected = (s32 + b[None, :]).astype(np.float32)
    invalid = ~(np.isfinite(z).all(axis=1) & np.isfinite(corrected).all(axis=1))
    corrected = np.where(invalid[:, None], np.float32(0), corrected)
    ids, _ = group_limited_select(corrected, n_group, topk_group, k, "top2sum")
    s64 = 1.0 / (1.0 + np.exp(-np.where(invalid[:, None], 0.0, z.astype(np.float64))))
    ssel = np.take_along_axis(s64, ids.astype(np.int64), axis=1)
    gates = route_scale * ssel / ssel.sum(axis=1, keepdims=True)
    ids[invalid] = -1
    gates[invalid] = 0.0
    return ids, gates, invalid


# ----------------------------------------------------------------------------
# a2: count, exclusive prefix, stable permutation, capacity, inverse
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class DispatchPlan:
    sel: np.ndarray       # [B] routes that selected each bucket (before capacity)
    counts: np.ndarray    # [B] accepted routes per bucket
    offsets: np.ndarray   # [B+1] exclusive prefix of counts, offsets[B] = accepted
    pos: np.ndarray       # [R] rank of the route inside its bucket (route order), -1 if no bucket
    inv: np.ndarray       # [R] packed position of the route, -1 if dropped
    src: np.ndarray       # [R] route at each packed position, -1 past the accepted total
    accepted: int
    dropped: int
    bad: np.ndarray       # [R] bucket id outside [-1, B)


def _exclusive_prefix(c: np.ndarray) -> np.ndarray:
    o = np.zeros(c.size + 1, dtype=np.int64)
    np.cumsum(c, out=o[1:])
    return o


def dispatch_plan(bucket: np.ndarray, n_buckets: int, capacity: int = -1) -> DispatchPlan:
    """Group routes by bucket with a stable order and keep the inverse map.

    M6.2 §0x03B: ``c_e`` counts routes of expert ``e``; ``o`` is the exclusive
    prefix with ``o_{E} = R``; ``pi`` is the stable argsort of route ids by
    ``(expert, route_id)``; ``inverse_pi[pi[j]] = j``.  M6.2 §0x01C: a
    capacity ``C`` bounds each expert's buffer and the overflow is dropped
    (first ``C`` routes in route order are kept).  M6.6 §0x0CD: accepted plus
    dropped equals ``T*k`` and the counts sum to the accepted total.

    ``bucket`` lists one bucket id per route in route order; -1 means "no
    route" (dropped, not an error); ids below -1 or at least ``n_buckets``
    are bad (dropped and reported in ``bad``).
    """
    b = np.asarray(bucket).reshape(-1).astype(np.int64)
    R = b.size
    valid = (b >= 0) & (b < n_buckets)
    bad = (b < -1) | (b >= n_buckets)
    route_id = np.arange(R, dtype=np.int64)

    sel = np.bincount(b[valid], minlength=n_buckets).astype(np.int64)
    sel_off = _exclusive_prefix(sel)
    # stable argsort by (bucket, route id); routes without a bucket sort last
    key = np.where(valid, b, n_buckets)
    order = np.argsort(key, kind="stable")
    n_valid = int(valid.sum())
    pos = np.full(R, -1, dtype=np.int64)
    first = order[:n_valid]
    pos[first] = np.arange(n_valid) - sel_off[b[first]]

    keep = valid if capacity < 0 else valid & (pos < capacity)
    counts = np.bincount(b[keep], minlength=n_buckets).astype(np.int64)
    offsets = _exclusive_prefix(counts)
    inv = np.full(R, -1, dtype=np.int64)
    inv[keep] = offsets[b[keep]] + pos[keep]
    src = np.full(R, -1, dtype=np.int64)
    src[inv[keep]] = route_id[keep]
    accepted = int(keep.sum())
    return DispatchPlan(sel=sel, counts=counts, offsets=offsets, pos=pos, inv=inv,
                        src=src, accepted=accepted, dropped=R - accepted, bad=bad)


def check_dispatch(bucket: np.ndarray, plan: DispatchPlan, gates: Optional[np.ndarray] = None,
                   capacity: int = -1) -> None:
    """Reject an inconsistent dispatch plan (raises ``ValueError``).

    M6.2 §0x03G rejection list: non-bijective permutation, count/offset
    mismatch, duplicate route identity, nonfinite gate.  M6.6 §0x0CD:
    accepted + dropped = expected routes; counts sum to accepted.
    "Dispatch and combine": the inverse must be a real bijection over its
    entries.
    """
    b = np.asarray(bucket).reshape(-1).astype(np.int64)
    R = b.size
    B = plan.counts.size
    A = plan.accepted
    if plan.accepted + plan.dropped != R:
        raise ValueError("accepted + dropped != routes")
    if int(plan.counts.sum()) != A or int(plan.offsets[-1]) != A:
        raise ValueError("counts/offsets do not sum to the accepted total")
    if plan.offsets[0] != 0 or np.any(np.diff(plan.offsets) != plan.counts):
        raise ValueError("offsets are not the exclusive prefix of counts")
    if capacity >= 0 and np.any(plan.counts > capacity):
        raise ValueError("a bucket exceeds its capacity")
    if np.any(plan.counts > plan.sel):
        raise ValueError("more accepted than selected routes")
    head = plan.src[:A]
    if np.any(head < 0) or np.any(head >= R) or np.any(plan.src[A:] != -1):
        raise ValueError("src has holes or stray entries")
    if np.unique(head).size != A:
        raise ValueError("duplicate route identity in src")
    if np.any(plan.inv[head] != np.arange(A)):
        raise ValueError("inv is not the inverse of src")
    if int((plan.inv >= 0).sum()) != A:
        raise ValueError("inv marks a different number of routes")
    for e in range(B):
        seg = head[plan.offsets[e]:plan.offsets[e + 1]]
        if np.any(b[seg] != e):
            raise ValueError("a route sits in another bucket's segment")
        if np.any(np.diff(seg) <= 0):
            raise ValueError("segment is not in route order")
    if gates is not None:
        g = np.asarray(gates, dtype=np.float64).reshape(-1)
        if not np.all(np.isfinite(g[head])):
            raise ValueError("nonfinite gate on an accepted route")


def gather_rows(x: np.ndarray, src: np.ndarray, k: int, accepted: int) -> np.ndarray:
    """Packed rows ``X_perm[p] = X[src[p] div k]`` for ``p < accepted``
    (M6.6 §0x03A: route rows are gathered from hidden states)."""
    return np.asarray(x)[np.asarray(src[:accepted]) // k]


# ----------------------------------------------------------------------------
# a4/a5: SwiGLU expert over ragged segments
# ----------------------------------------------------------------------------

def silu(v: np.ndarray) -> np.ndarray:
    """SiLU(v) = v * sigmoid(v) = v / (1 + exp(-v))."""
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def swiglu_expert(x: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """M6.6 §0x04A: ``E(X) = (SiLU(X W_g^T) (.) X W_u^T) W_2^T``, bias-free
    (M6.2 §0x04C1 writes the same bias-free form per expert)."""
    g = x @ wg.T
    u = x @ wu.T
    return (silu(g) * u) @ wd.T


ExpertFn = Callable[[int, np.ndarray], np.ndarray]
"""An expert bank: ``f(e, rows_f64) -> outputs_f64`` for expert ``e``."""


def swiglu_bank(weights: Callable[[int], Tuple[np.ndarray, np.ndarray, np.ndarray]]) -> ExpertFn:
    """Expert bank of bias-free SwiGLU experts; ``weights(e)`` returns the
    stored ``(W_g [d_ff,d], W_u [d_ff,d], W_d [d,d_ff])`` (fp32 or bf16 bits)."""
    def run(e: int, x: np.ndarray) -> np.ndarray:
        wg, wu, wd = (to_f64(w) for w in weights(e))
        return swiglu_expert(x, wg, wu, wd)
    return run


def scalar_bank(scales) -> ExpertFn:
    """Teaching experts ``E_e(x) = s_e x`` (M6.6 §0x04A; M6.2 §0x03C)."""
    s = [float(v) for v in scales]
    return lambda e, x: s[e] * x


def run_segments(rows: np.ndarray, seg_start: np.ndarray, seg_count: np.ndarray,
                 expert: ExpertFn, out: Optional[np.ndarray] = None) -> np.ndarray:
    """Run expert ``e`` on ``rows[seg_start[e] : seg_start[e]+seg_count[e]]``.

    M6.6 §0x04C: one problem per non-empty segment, with the segment's own
    expert (zero-row experts are skipped without shifting the binding of
    later segments).  Rows outside every segment stay zero in a fresh output.
    """
    x = to_f64(rows)
    for e in range(len(seg_count)):
        n = int(seg_count[e])
        if n == 0:
            continue
        s = int(seg_start[e])
        z = expert(e, x[s:s + n])
        if out is None:
            out = np.zeros((x.shape[0], z.shape[1]), dtype=np.float64)
        out[s:s + n] = z
    if out is None:
        out = np.zeros_like(x)
    return out


# ----------------------------------------------------------------------------
# a6: un-permute and gate-weighted combine
# ----------------------------------------------------------------------------

def combine(z_rows: np.ndarray, idx: np.ndarray, gates: Optional[np.ndarray], T: int, k: int,
            lo: int = 0, hi: Optional[int] = None, y: Optional[np.ndarray] = None) -> np.ndarray:
    """Weighted scatter-add back to token rows over the semantic key.

    M6.6 §0x03C3: ``y_t = sum_{r: origin(r)=t} g_r z_r``, with ``z_r`` read
    through the inverse map; M6.6 §0x0CD: gather by the inverse permutation,
    multiply by the route's gate, scatter-add by origin token.  Route
    ``r = t*k + j`` reads row ``idx[r] - lo`` of ``z_rows`` when
    ``lo <= idx[r] < hi``; other routes (dropped, -1, or outside the window)
    add nothing.  Slots are added in ascending ``j``.  ``gates`` None means
    weight 1.  ``y`` (float64) is accumulated into when given.
    """
    z = to_f64(z_rows)
    if hi is None:
        hi = lo + z.shape[0]
    idx = np.asarray(idx, dtype=np.int64).reshape(T, k)
    g = np.ones((T, k)) if gates is None else np.asarray(gates, dtype=np.float64).reshape(T, k)
    if y is None:
        y = np.zeros((T, z.shape[1]), dtype=np.float64)
    for j in range(k):
        i = idx[:, j]
        live = (i >= lo) & (i < hi)
        t = np.nonzero(live)[0]
        y[t] += g[t, j, None] * z[i[t] - lo]
    return y


def moe_layer_token_major(x: np.ndarray, ids: np.ndarray, gates: np.ndarray,
                          expert: ExpertFn, E: int,
                          keep: Optional[np.ndarray] = None) -> np.ndarray:
    """The semantic definition, evaluated token-major.

    M6.6 §0x0AE: ``y_t = sum_j g_{t,j} E_{e_{t,j}}(h_t)``.  Layout as in the
    DeepSeekMoE training branch (M6.2 §0x04D): repeat every token ``k`` times,
    run each expert on its masked rows, reshape to ``[T,k,d]`` and take the
    gate-weighted sum.  ``keep`` (bool ``[T,k]``) removes dropped routes.
    """
    xf = to_f64(x)
    T, k = ids.shape
    flat = ids.reshape(-1)
    live = flat >= 0 if keep is None else (flat >= 0) & keep.reshape(-1)
    routed_x = np.repeat(xf, k, axis=0)
    routed_y = None
    for e in range(E):
        mask = live & (flat == e)
        if not mask.any():
            continue
        z = expert(e, routed_x[mask])
        if routed_y is None:
            routed_y = np.zeros((T * k, z.shape[1]))
        routed_y[mask] = z
    if routed_y is None:
        return np.zeros_like(xf)
    g = np.where(live.reshape(T, k), np.asarray(gates, dtype=np.float64), 0.0)
    return (routed_y.reshape(T, k, -1) * g[..., None]).sum(axis=1)


def moe_layer_expert_major(x: np.ndarray, ids: np.ndarray, gates: np.ndarray,
                           expert: ExpertFn, E: int, capacity: int = -1):
    """The same layer evaluated expert-major (M6.2 §0x03G): count, prefix,
    stable permutation, gather, run each segment, gather back through the
    inverse, weighted scatter-add.  Returns ``(y, plan)``."""
    T, k = ids.shape
    plan = dispatch_plan(ids, E, capacity)
    xp = gather_rows(x, plan.src, k, plan.accepted)
    z = run_segments(xp, plan.offsets[:-1], plan.counts, expert)
    y = combine(z, plan.inv, gates, T, k)
    return y, plan


# ----------------------------------------------------------------------------
# backward of the transpose (M6.2 §0x03D)
# ----------------------------------------------------------------------------

ExpertBwd = Callable[[int, np.ndarray, np.ndarray], Tuple[np.ndarray, tuple]]
"""Expert backward: ``f(e, rows_f64, dz_f64) -> (dx_f64, parameter_grads)``."""


def combine_backward(dy: np.ndarray, z_rows: np.ndarray, idx: np.ndarray, gates: np.ndarray,
                     T: int, k: int):
    """Reverse of :func:`combine` (M6.2 §0x03D): an accepted route ``r`` of
    token ``t`` whose row is ``p = idx[r]`` receives ``Zbar_p = g_r Ybar_t``
    and the gate gradient ``gbar_r = <Ybar_t, Z_p>``.  Routes without a row
    (``idx = -1``) get ``gbar = 0`` and write nothing.

    Returns ``(dz [rows, d] float64, zero where no route points, dgates
    [T, k] float64)``.
    """
    dyf = np.asarray(dy, dtype=np.float64)
    z = to_f64(z_rows)
    idx = np.asarray(idx, dtype=np.int64).reshape(T, k)
    g = np.asarray(gates, dtype=np.float64).reshape(T, k)
    dz = np.zeros_like(z)
    dg = np.zeros((T, k))
    for j in range(k):
        t = np.nonzero(idx[:, j] >= 0)[0]
        p = idx[t, j]
        dz[p] = g[t, j, None] * dyf[t]
        dg[t, j] = np.einsum("ij,ij->i", dyf[t], z[p])
    return dz, dg


def silu_grad(v: np.ndarray) -> np.ndarray:
    """d SiLU / dv = sigma(v) (1 + v (1 - sigma(v)))."""
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-v))
    return s * (1.0 + v * (1.0 - s))


def swiglu_expert_backward(x: np.ndarray, dz: np.ndarray, wg: np.ndarray, wu: np.ndarray,
                           wd: np.ndarray):
    """Reverse of :func:`swiglu_expert` (chain rule through M6.6 §0x04A):
    with ``G = X W_g^T``, ``U = X W_u^T``, ``H = SiLU(G) (.) U``,
    ``Z = H W_d^T``:  ``Hbar = Zbar W_d``, ``W_d bar = Zbar^T H``,
    ``Gbar = Hbar (.) U (.) SiLU'(G)``, ``Ubar = Hbar (.) SiLU(G)``,
    ``Xbar = Gbar W_g + Ubar W_u``, ``W_g bar = Gbar^T X``,
    ``W_u bar = Ubar^T X``.  Returns ``(dx, (dwg, dwu, dwd))``."""
    g = x @ wg.T
    u = x @ wu.T
    h = silu(g) * u
    dh = dz @ wd
    dwd = dz.T @ h
    dg = dh * u * silu_grad(g)
    du = dh * silu(g)
    dx = dg @ wg + du @ wu
    return dx, (dg.T @ x, du.T @ x, dwd)


def swiglu_bank_backward(weights: Callable[[int], Tuple[np.ndarray, np.ndarray, np.ndarray]]) -> ExpertBwd:
    """Backward of :func:`swiglu_bank` with the same stored weights."""
    def run(e: int, x: np.ndarray, dz: np.ndarray):
        wg, wu, wd = (to_f64(w) for w in weights(e))
        return swiglu_expert_backward(x, dz, wg, wu, wd)
    return run


def scalar_bank_backward(scales) -> ExpertBwd:
    """Backward of :func:`scalar_bank`: ``Xbar = s_e Zbar`` and
    ``s_e bar = sum <Zbar, X>`` over the expert's rows (M6.2 §0x03D toy)."""
    s = [float(v) for v in scales]
    return lambda e, x, dz: (s[e] * dz, (float((dz * x).sum()),))


def run_segments_backward(rows: np.ndarray, dz: np.ndarray, seg_start: np.ndarray,
                          seg_count: np.ndarray, expert_bwd: ExpertBwd):
    """Expert backward per non-empty segment (the segmentation is backward
    state, M6.2 §0x03D).  Returns ``(dx_rows, grads)`` with ``grads[e]`` the
    expert's parameter gradients, or None for a zero-row expert."""
    x = to_f64(rows)
    dzf = np.asarray(dz, dtype=np.float64)
    dx = np.zeros_like(x)
    grads = []
    for e in range(len(seg_count)):
        n = int(seg_count[e])
        if n == 0:
            grads.append(None)
            continue
        s0 = int(seg_start[e])
        dx[s0:s0 + n], ge = expert_bwd(e, x[s0:s0 + n], dzf[s0:s0 + n])
        grads.append(ge)
    return dx, grads


def moe_layer_backward(x: np.ndarray, ids: np.ndarray, gates: np.ndarray, expert: ExpertFn,
                       expert_bwd: ExpertBwd, E: int, dy: np.ndarray, capacity: int = -1):
    """Backward of the layer, expert-major (M6.2 §0x03D): the forward state
    (permutation, origin record through the inverse map, gates, segments and
    the expert outputs ``Z``) is rematerialised; the route gradients and gate
    gradients come from :func:`combine_backward`; each segment runs its
    expert backward; the route-input gradients are summed by origin token
    through the inverse map (:func:`combine` with unit weights).

    Returns a dict with ``dx [T, d]``, ``dgates [T, k]`` (0 for dropped
    routes), ``grads`` (per expert, None when it has no rows) and the
    intermediate ``plan``, ``z``, ``dz``, ``dx_rows``.
    """
    T, k = ids.shape
    plan = dispatch_plan(ids, E, capacity)
    xp = gather_rows(x, plan.src, k, plan.accepted)
    z = run_segments(xp, plan.offsets[:-1], plan.counts, expert)
    dz, dg = combine_backward(dy, z, plan.inv, gates, T, k)
    dx_rows, grads = run_segments_backward(xp, dz, plan.offsets[:-1], plan.counts, expert_bwd)
    dx = combine(dx_rows, plan.inv, None, T, k)
    return dict(dx=dx, dgates=dg, grads=grads, plan=plan, z=z, dz=dz, dx_rows=dx_rows)


# ----------------------------------------------------------------------------
# FP8 dispatch payload (M6.2 §0x0AA-§0x0AC)
# ----------------------------------------------------------------------------

FP8_E4M3_MAX = 448.0


def _e4m3_magnitudes() -> np.ndarray:
    """Values of the 127 non-negative finite E4M3 codes 0x00..0x7E (4-bit
    exponent with bias 7, 3-bit mantissa, exponent field 0 subnormal; code
    0x7F is NaN and there are no infinities), in code order (increasing)."""
    c = np.arange(127)
    e, m = c >> 3, c & 7
    return np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))


def fp8_e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """E4M3 codes to float32 (exact)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    mag = c & 0x7F
    v = np.where(mag == 0x7F, np.nan, _e4m3_magnitudes()[np.minimum(mag, 126)])
    return np.where(c & 0x80, -v, v).astype(np.float32)


def fp8_e4m3_encode(v: np.ndarray) -> np.ndarray:
    """float32 to E4M3 by round to nearest, ties to the even code, saturating
    at +-448 (the format has no infinity); NaN gives 0x7F with the sign.  The
    sign bit is copied from the input, zeros and underflow included."""
    a32 = np.asarray(v, dtype=np.float32)
    a = np.abs(a32.astype(np.float64))
    mags = _e4m3_magnitudes()
    hi = np.clip(np.searchsorted(mags, a, side="left"), 1, 126)      # mags[hi-1] < a <= mags[hi]
    lo = hi - 1
    dlo, dhi = a - mags[lo], mags[hi] - a
    code = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    code = np.where(a >= FP8_E4M3_MAX, 126, code)
    code = np.where(a <= 0.0, 0, code)
    code = np.where(np.isnan(a), 0x7F, code)
    return (code | np.where(np.signbit(a32), 0x80, 0)).astype(np.uint8)


FP8_MODES = ("row", "b128")


def fp8_record_layout(d: int, mode: str) -> Tuple[int, int]:
    """``(G, W)``: scales per row (one, or one per 128 values, M6.2 §0x0AB)
    and the record width in bytes: ``d`` fp8 bytes, then ``G`` fp32 scales,
    zero padding to a multiple of 128 bytes (whole cache lines: the layout is
    the library's choice, the pages fix only that scales travel with their
    row)."""
    if mode not in FP8_MODES:
        raise ValueError(mode)
    G = 1 if mode == "row" else -(-int(d) // 128)
    return G, -(-(int(d) + 4 * G) // 128) * 128


def fp8_payload_bytes(R: int, d: int, mode: Optional[str]) -> int:
    """Logical payload bytes of ``R`` rows (M6.2 §0x0AB): bf16 data
    ``2 R d``; fp8 data plus fp32 scales ``R d + 4 R G``.  No padding,
    alignment or transport metadata."""
    if mode is None:
        return 2 * R * d
    G = fp8_record_layout(d, mode)[0]
    return R * d + 4 * R * G


def quantize_fp8_rows(x: np.ndarray, mode: str) -> np.ndarray:
    """Rows (exact fp32 values, e.g. bf16 inputs) to fp8 records.

    M6.2 §0x0AC: quantization yields data plus its scales, owned by the same
    row.  Per scale group (the row, or 128 consecutive values): ``a`` = the
    largest magnitude; ``scale = fp32(a / 448)``, ``inv = fp32(448 / a)``,
    code ``= E4M3(fp32(x * inv))``; a group with ``a = 0`` gets scale 0 and
    zero codes.  (The pages fix no scale rule: this max-to-448 rule, with
    every step one correctly rounded fp32 operation, is the reading; a group
    holding NaN or infinity is stored like an all-zero group.)
    Returns uint8 ``[n, W]``.
    """
    xf = np.asarray(x, dtype=np.float32)
    n, d = xf.shape
    G, Wb = fp8_record_layout(d, mode)
    width = d if mode == "row" else 128
    rec = np.zeros((n, Wb), dtype=np.uint8)
    scales = np.zeros((n, G), dtype=np.float32)
    for g in range(G):
        c0, c1 = g * width, min(d, (g + 1) * width)
        blk = xf[:, c0:c1]
        amax = np.abs(blk).max(axis=1) if n else np.zeros(0, np.float32)
        live = np.isfinite(amax) & (amax > 0)         # zero or non-finite groups store zeros
        safe = np.where(live, amax, np.float32(1.0)).astype(np.float32)
        scale = np.where(live, safe / np.float32(FP8_E4M3_MAX), np.float32(0.0)).astype(np.float32)
        inv = (np.float32(FP8_E4M3_MAX) / safe).astype(np.float32)
        q = fp8_e4m3_encode((blk * inv[:, None]).astype(np.float32))
        rec[:, c0:c1] = np.where(live[:, None], q, 0)
        scales[:, g] = scale
    rec[:, d:d + 4 * G] = scales.view(np.uint8).reshape(n, 4 * G)
    return rec


def dequantize_fp8_rows(rec: np.ndarray, d: int, mode: str) -> np.ndarray:
    """fp8 records to fp32 rows: ``fp32(decode(code) * scale)`` with the scale
    of the value's group read from the same record (M6.2 §0x0AC)."""
    r = np.ascontiguousarray(rec, dtype=np.uint8)
    G, Wb = fp8_record_layout(d, mode)
    if r.shape[-1] != Wb:
        raise ValueError("record width")
    r = r.reshape(-1, Wb)
    scales = np.ascontiguousarray(r[:, d:d + 4 * G]).view(np.float32)
    width = d if mode == "row" else 128
    per_col = scales[:, np.arange(d) // width]
    return (fp8_e4m3_decode(r[:, :d]) * per_col).astype(np.float32)


def f32_to_bf16_rne(a: np.ndarray) -> np.ndarray:
    """float32 to bf16 bits, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


# ----------------------------------------------------------------------------
# a7: pooled-wave sender pack
# ----------------------------------------------------------------------------

def header_rows_bytes(pool_rows: int, row_bytes: int) -> int:
    """Full-width header rows of a pool whose rows are ``row_bytes`` wide:
    one 16-bit id per data row, ``row_bytes / 2`` ids per header row, at
    least one (pooled wave §02 uses one row for 3004 ids in 6144-byte bf16
    rows; more rows are the configurable-header variant)."""
    return max(1, -(-2 * int(pool_rows) // int(row_bytes)))


def header_rows(pool_rows: int, d: int) -> int:
    """Header rows of a pool of bf16 rows ``d`` values wide (the two-wave
    profile of §05 needs 4506 ids per pool: two rows at d = 3072)."""
    return header_rows_bytes(pool_rows, 2 * int(d))


def pool_rows_of_bytes(pool_height: int, row_bytes: int) -> int:
    """The ``pool_rows`` whose pool has ``pool_height`` rows (data rows plus
    their header rows); unique because the height grows with pool_rows."""
    for h in range(1, pool_height + 1):
        p = pool_height - h
        if header_rows_bytes(p, row_bytes) == h:
            return p
    raise ValueError("no pool_rows gives this pool height")


def pool_rows_of(pool_height: int, d: int) -> int:
    """:func:`pool_rows_of_bytes` for bf16 rows ``d`` values wide."""
    return pool_rows_of_bytes(pool_height, 2 * int(d))


def _row_bytes(a: np.ndarray) -> np.ndarray:
    """Rows of bf16 bits (uint16) or of fp8 records (uint8) as bytes."""
    a = np.ascontiguousarray(a)
    if a.dtype not in (np.uint16, np.uint8):
        raise TypeError("rows are bf16 bits (uint16) or fp8 records (uint8)")
    return a.view(np.uint8).reshape(a.shape[:-1] + (a.shape[-1] * a.itemsize,))


def pool_pack(x_bits: np.ndarray, ids: np.ndarray, experts_per_dest: int, n_dest: int,
              n_waves: int, pool_rows: int, *, with_pools: bool = True, E: Optional[int] = None):
    """Pack one sender's routes into fixed destination pools.

    Pooled wave §02: expert id gives a destination and a local expert id;
    the stripe rule takes the page's rank modulo three as the wave and the
    rank divided by three as the pool row, with the rank read as the route's
    ordinal among this sender's routes to that destination (generalised to
    ``n_waves``: the two-wave profile of §05); each destination gets
    ``pool_rows`` rows per wave and extra rows are dropped; the first
    full-width rows of a pool carry the packed local expert ids (element ``i``
    of the header, row ``i // d`` column ``i % d``, holds data row ``i``'s id;
    ``H = header_rows(pool_rows, d)``, one at the pages' sizes).  §03: pool
    shape ``[n_dest, pool_rows + H, d]`` per wave.

    Returns a dict with ``pools`` (uint16 ``[n_waves, n_dest, pool_rows+H, d]``,
    or None when ``with_pools`` is False), ``route_loc`` (int64 ``[T*k]``:
    flat pool row ``(w*n_dest + dest)*(pool_rows+H) + H + row`` or -1),
    ``dest_counts`` (routes per destination before the cap),
    ``sender_dropped`` (routes not placed, including "no route" ids) and the
    per-route ``wave``/``row``/``dest``/``local``; ``bad`` marks expert ids
    that are neither -1 nor below ``E`` (default ``n_dest*experts_per_dest``).
    """
    T, k = ids.shape
    e = np.asarray(ids, dtype=np.int64).reshape(-1)
    n_exp = n_dest * experts_per_dest if E is None else E
    valid = (e >= 0) & (e < n_exp)
    dest = np.where(valid, e // experts_per_dest, -1)
    local = np.where(valid, e % experts_per_dest, -1)
    plan = dispatch_plan(dest, n_dest)
    rank = plan.pos
    wave = np.where(valid, rank % n_waves, -1)
    row = np.where(valid, rank // n_waves, -1)
    acc = valid & (row < pool_rows)
    xa = np.asarray(x_bits)
    x8 = _row_bytes(xa)
    rb = x8.shape[1]
    H = header_rows_bytes(pool_rows, rb)
    P1 = pool_rows + H
    route_loc = np.where(acc, (wave * n_dest + dest) * P1 + H + row, -1)
    pools = None
    if with_pools:
        n_pools = n_waves * n_dest
        p8 = np.zeros((n_pools, P1, rb), dtype=np.uint8)
        p8[:, :H, :] = 0xFF                              # 0xFFFF ids: empty
        r = np.nonzero(acc)[0]
        p8.reshape(-1, rb)[route_loc[r]] = x8[r // k]    # rows indexed like route_loc
        hdr = p8.reshape(n_pools, P1 * rb)[:, :H * rb].view(np.uint16)   # little-endian 16-bit ids
        hdr[wave[r] * n_dest + dest[r], row[r]] = local[r].astype(np.uint16)
        pools = p8.reshape(n_waves, n_dest, P1, rb)
        if xa.dtype == np.uint16:
            pools = pools.view(np.uint16)
    return dict(pools=pools, route_loc=route_loc, dest_counts=plan.sel,
                sender_dropped=int(e.size - acc.sum()), wave=wave, row=row,
                dest=dest, local=local, accepted=acc, bad=(e < -1) | (e >= n_exp))


# ----------------------------------------------------------------------------
# a8: receiver compaction into static per-expert arrays
# ----------------------------------------------------------------------------

def recv_compact(pools: np.ndarray, n_local: int, cap: int, *, with_rows: bool = True, rotation: int = 0,
                 record: Optional[Tuple[int, str]] = None):
    """Group one wave's incoming rows into ``[n_local, cap, d]`` arrays.

    Pooled wave §02/§03: the receiver reads each row's local expert id from
    the header rows and groups rows into six static expert arrays, dropping
    rows above the receiver capacity; §07: rows keep a fixed source order
    (source pool, then row) and overflow does not look at router scores.
    ``rotation`` is the per-receiver rotation proposed in §07: sources are
    visited in the order ``rotation, rotation+1, ..., n_src-1, 0, ...`` so
    that overflow does not always fall on the same last source (0 = the
    fixed order).  The pool height is ``pool_rows + header_rows(pool_rows, d)``.
    ``record = (d, mode)`` says that the pools hold fp8 records (uint8 rows,
    see :func:`quantize_fp8_rows`); the compaction then dequantizes the
    accepted rows with the scales stored in the same record (M6.2 §0x0AC)
    and the compact arrays hold bf16 bits.

    Returns a dict with ``compact`` (uint16 ``[n_local, cap, d]``, rows past
    ``counts[h]`` zero; None when ``with_rows`` is False), ``counts``,
    ``arrived``, ``row_slot`` (int64 ``[n_src*(pool_rows+H)]``: ``h*cap + q``
    or -1; header rows -1), ``recv_dropped`` and ``bad_header`` (count of
    header ids that are neither a local id nor 0xFFFF).
    """
    pools = np.asarray(pools)
    p8 = _row_bytes(pools)
    S, P1, rb = p8.shape
    P = pool_rows_of_bytes(P1, rb)
    H = P1 - P
    d = pools.shape[2] if record is None else int(record[0])
    if not 0 <= rotation < max(S, 1):
        raise ValueError("rotation must be in [0, n_src)")
    order = (np.arange(S) + rotation) % S if S else np.arange(0)
    # ids in visiting order: source order[v], then data row i
    h = np.ascontiguousarray(p8[order, :H, :]).reshape(S, H * rb).view(np.uint16)[:, :P]
    h = h.astype(np.int64).reshape(-1)
    valid = h < n_local
    bad = (h != HEADER_EMPTY) & ~valid
    plan = dispatch_plan(np.where(valid, h, -1), n_local, capacity=cap)
    q = plan.pos
    acc = plan.inv >= 0
    v_idx, i_idx = np.divmod(np.arange(S * P), P)
    s_idx = order[v_idx] if S else v_idx
    row_slot = np.full(S * P1, -1, dtype=np.int64)
    row_slot[s_idx * P1 + H + i_idx] = np.where(acc, h * cap + q, -1)
    compact = None
    if with_rows:
        compact = np.zeros((n_local, cap, d), dtype=np.uint16)
        r = np.nonzero(acc)[0]
        if record is None:
            compact[h[r], q[r]] = pools[s_idx[r], H + i_idx[r]]
        else:
            rows = dequantize_fp8_rows(p8[s_idx[r], H + i_idx[r]], d, record[1])
            compact[h[r], q[r]] = f32_to_bf16_rne(rows)
    return dict(compact=compact, counts=plan.counts, arrived=plan.sel, row_slot=row_slot,
                recv_dropped=int(plan.sel.sum() - plan.counts.sum()),
                bad_header=int(bad.sum()))


def expand_rows(z_static: np.ndarray, row_slot: np.ndarray) -> np.ndarray:
    """Return buffer in pool-row order: ``ret[i] = z[row_slot[i]]`` or zeros
    (header, empty and receiver-dropped rows; M6.6 §0x04B: padding never
    reaches combine).  Same as :func:`combine` with one slot and unit
    weights."""
    n = row_slot.size
    return combine(z_static, row_slot, None, n, 1)


def loopback_layer(x_bits: np.ndarray, ids: np.ndarray, gates: np.ndarray, expert: ExpertFn,
                   experts_per_dest: int, n_dest: int, n_waves: int, pool_rows: int,
                   recv_cap: int, payload: Optional[str] = None):
    """One sender's pools fed back as one receiver's incoming pools.

    A single-GPU stand-in for the fixed exchange: the sender's wave-``w``
    pools (one per destination) are read as the ``n_dest`` source pools of a
    receiver whose ``experts_per_dest`` local experts serve every local id.
    Pooled wave §03: per wave, compaction, one batched SwiGLU over the local
    experts, expansion back to pool rows, and the waves add into one FP32
    accumulator through the sender's route locations.  The result equals the
    layer in which expert ``e`` uses local expert ``e mod experts_per_dest``'s
    weights and routes dropped by the sender or the receiver add nothing.
    ``payload`` "row" / "b128" sends fp8 records (M6.2 §0x0AB-§0x0AC): each
    token row is quantized once, the records travel in the pools and the
    receiver dequantizes them into its bf16 arrays.
    Returns ``(y [T,d] float64, details)``.
    """
    T, k = ids.shape
    d = np.asarray(x_bits).shape[1]
    rows = x_bits if payload is None else quantize_fp8_rows(to_f64(x_bits).astype(np.float32), payload)
    pk = pool_pack(rows, ids, experts_per_dest, n_dest, n_waves, pool_rows)
    P1 = pool_rows + header_rows_bytes(pool_rows, _row_bytes(np.asarray(rows[:1])).shape[1])
    y = np.zeros((T, d))
    waves = []
    for w in range(n_waves):
        rc = recv_compact(pk["pools"][w], experts_per_dest, recv_cap,
                          record=None if payload is None else (d, payload))
        starts = np.arange(experts_per_dest) * recv_cap
        z = run_segments(rc["compact"].reshape(-1, d), starts, rc["counts"], expert)
        ret = expand_rows(z, rc["row_slot"])
        lo = w * n_dest * P1
        combine(ret, pk["route_loc"], gates, T, k, lo=lo, hi=lo + n_dest * P1, y=y)
        waves.append(rc)
    return y, dict(pack=pk, waves=waves)


# ----------------------------------------------------------------------------
# ledgers and capacities
# ----------------------------------------------------------------------------

def capacity_ceil(factor_num: int, factor_den: int, assignments: int, parts: int) -> int:
    """``ceil(c_f * assignments / parts)`` with ``c_f = factor_num/factor_den``
    in exact integer arithmetic (M6.2 §0x01C; pooled wave §04)."""
    num = factor_num * assignments
    den = factor_den * parts
    return -(-num // den)


def drop_rates(assignments: int, sender_dropped: int, recv_dropped: int):
    """Pooled wave §05: additive rates ``S/T`` and ``R/T`` and the
    conditional receiver rate ``R/(T-S)``."""
    T, S, R = float(assignments), float(sender_dropped), float(recv_dropped)
    return S / T, R / T, (R / (T - S) if T > S else 0.0)


def swiglu_flops(rows: int, d: int, d_ff: int) -> int:
    """M6.6 §0x04A: three matmuls, ``2 n d d_ff`` each, ``6 n d d_ff`` total."""
    return 6 * rows * d * d_ff


def padded_exec_rows(n_slots: int, capacity: int, align: int) -> int:
    """M6.6 §0x04B: ``C_exec = a * ceil(C / a)`` rows for each physical slot."""
    return n_slots * align * (-(-capacity // align))


def block_exec_rows(counts, block_rows: int) -> int:
    """M6.6 §0x04D: every expert rounded up to whole row blocks."""
    return int(sum(block_rows * (-(-int(n) // block_rows)) for n in counts))
