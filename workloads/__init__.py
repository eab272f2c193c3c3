"""Seeded synthetic inputs for the routed-expert layer.

This module only draws random numbers and lays them out in the storage
formats the library consumes.  It contains none of the layer's arithmetic:
no routing, no permutation, no expert math.  Both the HIP path (through the
tests and the benchmark) and the CPU oracle consume exactly the bytes made
here, so a parity test compares two independent computations on identical
inputs.

Storage conventions
-------------------
* fp32 tensors are ``numpy.float32``.
* bf16 tensors are raw 16-bit patterns in ``numpy.uint16`` (the upper half of
  the float32 bit pattern after round-to-nearest-even), which is the byte
  layout of ``torch.bfloat16``.

Random streams
--------------
Every tensor (and every expert's weight triple) has its own
``numpy.random.SeedSequence(entropy=seed, spawn_key=(tag, index))`` stream, so
tensors can be generated lazily, in any order, or in parallel threads and
still produce the same bytes.

Workloads
---------
The five named workloads follow the shapes of the pages' 8-of-384 design
("Fixed pooled-wave all-to-all for the 8-of-384 MoE", §02-§04: 65,536 tokens
per GPU, top-8 of 384 experts, six experts per GPU, three waves, latent width
3072) plus a tiny fp32 layer and a mid-size bf16 layer.  Trained router
statistics are not available, so router logits are Gaussian (or uniform)
with an additive Zipf-shaped per-expert bias ``(e+1)^-1.1``.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os
from typing import Optional, Tuple

import numpy as np

# Stream tags (part of the seed; never change without regenerating goldens).
_TAG_LOGITS = 1
_TAG_TOKENS = 2
_TAG_WEIGHTS = 3
_TAG_RECV_IDS = 4
_TAG_RECV_ROWS = 5
_TAG_BIAS = 6
_TAG_DY = 7

HEADER_EMPTY = 0xFFFF


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and distribution recipe of one synthetic workload."""

    name: str
    seed: int
    dtype: str                 # "f32" or "bf16" for activations and weights
    T: int = 0                 # tokens
    d: int = 0                 # expert input / output width
    E: int = 0                 # routed experts
    k: int = 0                 # experts per token
    d_ff: int = 0              # SwiGLU intermediate width
    capacity: int = -1         # per-expert capacity, -1 = dropless
    logits: str = "normal"     # "uniform" or "normal"
    zipf_bias: float = 0.0     # exponent s of the additive (e+1)^-s bias, 0 = none
    x_std: float = 0.02
    w_std: float = 0.02
    # pooled-wave geometry (sender pack / receiver share)
    experts_per_dest: int = 0
    n_dest: int = 0
    n_waves: int = 0
    pool_rows: int = 0
    n_src: int = 0
    n_local: int = 0
    recv_cap: int = 0
    recv_zipf: float = 0.0
    ret_dtype: str = "f32"     # receiver return rows: "f32" or "bf16"
    train: bool = False        # a step is the layer forward plus its backward (upstream gradient ~ N(0, 1))
    payload: Optional[str] = None   # dispatched rows: None = bf16, "row" / "b128" = fp8 records
    # group-restricted router (gating variants)
    gating: int = 0            # 0 softmax-renorm, 1 V1, 2 V2, 3 V3 (the library's moe_gating ids)
    n_group: int = 0
    topk_group: int = 0
    route_scale: float = 1.0
    bias_std: float = 0.0      # V3 selection bias ~ N(0, bias_std), its own stream

    @property
    def R(self) -> int:
        return self.T * self.k


TINY = Workload(name="tiny_fp32", seed=0, dtype="f32", T=256, d=128, E=8, k=2,
                d_ff=256, logits="uniform", x_std=0.02, w_std=0.02)
MID = Workload(name="mid_bf16", seed=1, dtype="bf16", T=2048, d=2048, E=128, k=8,
               d_ff=768, logits="normal", zipf_bias=1.1, x_std=0.02, w_std=0.02)
RECV = Workload(name="recv_share_bf16", seed=2, dtype="bf16", d=3072, d_ff=1536,
                E=6, n_src=64, pool_rows=3004, n_waves=3, n_local=6, recv_cap=33497,
                recv_zipf=1.1, x_std=1.0, w_std=0.02)
SEND = Workload(name="sender_pack_bf16", seed=3, dtype="bf16", T=65536, d=3072,
                E=384, k=8, logits="normal", zipf_bias=1.1, x_std=1.0,
                experts_per_dest=6, n_dest=64, n_waves=3, pool_rows=3004)
# The two-wave profile (pooled wave 05): the same incoming rows per receiver in
# two waves, so each pool holds ceil(1.10 * 524288 / 128) rows (two header
# rows at d = 3072) and each receiver array ceil(1.15 * 524288 / 12) rows.
RECV_2W = Workload(name="recv_share_2w_bf16", seed=2, dtype="bf16", d=3072, d_ff=1536,
                   E=6, n_src=64, pool_rows=4506, n_waves=2, n_local=6, recv_cap=50245,
                   recv_zipf=1.1, x_std=1.0, w_std=0.02)
# The mid layer as a training step: forward, then the backward of the
# transpose ("M6.2", 0x03D) with an N(0, 1) fp32 upstream gradient.
MID_TRAIN = dataclasses.replace(MID, name="mid_bf16_train", train=True)

# The receiver share with bf16 return rows ("M6.6", 0x0AE: the returned row is
# BF16): the expert GEMM stores bf16 and the return buffer is bf16.
RECV_RET16 = dataclasses.replace(RECV, name="recv_share_ret_bf16", ret_dtype="bf16")
# fp8 dispatch records with one fp32 scale per 128 values ("M6.2", 0x0AB):
# the sender quantizes each token row once and packs records; the receiver
# compacts records and dequantizes them into its bf16 arrays.
SEND_FP8 = dataclasses.replace(SEND, name="sender_pack_fp8", payload="b128")
RECV_FP8 = dataclasses.replace(RECV, name="recv_share_fp8", payload="b128")
SEND_2W = Workload(name="sender_pack_2w_bf16", seed=3, dtype="bf16", T=65536, d=3072,
                   E=384, k=8, logits="normal", zipf_bias=1.1, x_std=1.0,
                   experts_per_dest=6, n_dest=64, n_waves=2, pool_rows=4506)
DECODE = Workload(name="decode_bf16", seed=4, dtype="bf16", T=64, d=3072, E=384,
                  k=8, d_ff=1536, logits="normal", x_std=1.0, w_std=0.02)

# The V3 router at the pages' released shape ("M6.2", 0x06I: 256 experts in
# 8 groups, keep 4, top-8, route scale 2.5) over the sender's 65,536 tokens.
ROUTER_V3 = Workload(name="router_v3_f32", seed=5, dtype="f32", T=65536, E=256, k=8, logits="normal",
                     gating=3, n_group=8, topk_group=4, route_scale=2.5, bias_std=0.05)

WORKLOADS = {w.name: w for w in (TINY, MID, RECV, SEND, DECODE, ROUTER_V3, RECV_2W, SEND_2W, RECV_RET16,
                                 MID_TRAIN, SEND_FP8, RECV_FP8)}


def scaled(w: Workload, **changes) -> Workload:
    """A copy of ``w`` with some fields replaced (smaller parity cases)."""
    return dataclasses.replace(w, **changes)


# ----------------------------------------------------------------------------
# storage helpers
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return the bits.

    Inputs here are finite, so no NaN special case is needed.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _rng(seed: int, tag: int, index: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence(entropy=seed, spawn_key=(tag, index))
    return np.random.Generator(np.random.PCG64(ss))


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    out = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def _store(a32: np.ndarray, dtype: str) -> np.ndarray:
    return a32 if dtype == "f32" else f32_to_bf16_bits(a32)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


# ----------------------------------------------------------------------------
# generators
# ----------------------------------------------------------------------------

def router_logits(w: Workload) -> np.ndarray:
    """fp32 router logits ``[T, E]``: uniform [0,1) or N(0,1) plus Zipf bias."""
    rng = _rng(w.seed, _TAG_LOGITS)
    if w.logits == "uniform":
        z = rng.random(size=(w.T, w.E), dtype=np.float32)
    else:
        z = rng.standard_normal(size=(w.T, w.E), dtype=np.float32)
    if w.zipf_bias:
        bias = (np.arange(1, w.E + 1, dtype=np.float64) ** (-w.zipf_bias)).astype(np.float32)
        z += bias[None, :]
    return z


def router_bias(w: Workload) -> np.ndarray:
    """fp32 per-expert selection bias ``[E]`` ~ N(0, bias_std)."""
    return _normal(_rng(w.seed, _TAG_BIAS), (w.E,), w.bias_std) if w.bias_std else np.zeros(w.E, np.float32)


def tokens(w: Workload) -> np.ndarray:
    """Token rows ``[T, d]`` (fp32, or bf16 bits).  Blocks of 4096 rows have
    their own streams and are drawn in parallel threads."""
    chunk = 4096
    out = np.empty((w.T, w.d), dtype=np.float32 if w.dtype == "f32" else np.uint16)

    def one(i):
        t0, t1 = i * chunk, min(w.T, (i + 1) * chunk)
        out[t0:t1] = _store(_normal(_rng(w.seed, _TAG_TOKENS, i), (t1 - t0, w.d), w.x_std), w.dtype)

    with _cf.ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range((w.T + chunk - 1) // chunk)))
    return out


def upstream_grad(w: Workload) -> np.ndarray:
    """fp32 upstream gradient ``[T, d]`` of the layer output ~ N(0, 1)."""
    return _normal(_rng(w.seed, _TAG_DY), (w.T, w.d), 1.0)


def expert_weights(w: Workload, e: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """One expert's ``(W_gate [d_ff,d], W_up [d_ff,d], W_down [d,d_ff])``."""
    rng = _rng(w.seed, _TAG_WEIGHTS, e)
    wg = _store(_normal(rng, (w.d_ff, w.d), w.w_std), w.dtype)
    wu = _store(_normal(rng, (w.d_ff, w.d), w.w_std), w.dtype)
    wd = _store(_normal(rng, (w.d, w.d_ff), w.w_std), w.dtype)
    return wg, wu, wd


def all_expert_weights(w: Workload, n_experts: Optional[int] = None):
    """Stacked weights ``W_gate, W_up [E,d_ff,d]`` and ``W_down [E,d,d_ff]``.

    Experts are generated in parallel threads from their own streams.
    """
    E = w.E if n_experts is None else n_experts
    st = np.float32 if w.dtype == "f32" else np.uint16
    wg = np.empty((E, w.d_ff, w.d), dtype=st)
    wu = np.empty((E, w.d_ff, w.d), dtype=st)
    wd = np.empty((E, w.d, w.d_ff), dtype=st)

    def one(e):
        wg[e], wu[e], wd[e] = expert_weights(w, e)

    with _cf.ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(E)))
    return wg, wu, wd


def recv_local_ids(w: Workload, wave: int) -> np.ndarray:
    """Local expert id ``[n_src, pool_rows]`` of every incoming row of a wave,
    drawn from the skewed multinomial ``p_l ~ (l+1)^-s``."""
    rng = _rng(w.seed, _TAG_RECV_IDS, wave)
    p = np.arange(1, w.n_local + 1, dtype=np.float64) ** (-w.recv_zipf)
    p /= p.sum()
    return rng.choice(w.n_local, size=(w.n_src, w.pool_rows), p=p).astype(np.uint16)


def recv_header_rows(w: Workload) -> int:
    """Header rows per incoming pool: ``d`` 16-bit ids per row, at least one."""
    return max(1, -(-w.pool_rows // w.d))


def recv_pools(w: Workload, wave: int, ids: Optional[np.ndarray] = None) -> np.ndarray:
    """Incoming bf16 pools ``[n_src, H + pool_rows, d]`` for one wave.

    The first ``H = recv_header_rows(w)`` rows of each pool are the header:
    element ``i`` of the flattened header holds the 16-bit local expert id of
    data row ``i`` (stored at pool row ``H + i``); elements past ``pool_rows``
    hold 0xFFFF.  Every data row of this workload is occupied.  ``ids`` may
    override the drawn ids (0xFFFF marks an empty row).
    """
    if ids is None:
        ids = recv_local_ids(w, wave)
    H = recv_header_rows(w)
    pools = np.empty((w.n_src, H + w.pool_rows, w.d), dtype=np.uint16)
    hdr = pools[:, :H, :].reshape(w.n_src, H * w.d)
    hdr[:] = HEADER_EMPTY
    hdr[:, : w.pool_rows] = ids
    pools[:, :H, :] = hdr.reshape(w.n_src, H, w.d)
    base = _rng(w.seed, _TAG_RECV_ROWS, wave)
    seeds = base.integers(0, 2**63 - 1, size=w.n_src)

    def one(s):
        r = np.random.Generator(np.random.PCG64(int(seeds[s])))
        pools[s, H:, :] = f32_to_bf16_bits(_normal(r, (w.pool_rows, w.d), w.x_std))

    with _cf.ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(w.n_src)))
    return pools
