"""Seeded synthetic inputs shaped like Wan2.1/2.2 video-latent attention.

This module holds no part of the attention method: it only draws numbers.
Both the HIP path (through the tests and the benchmark) and the CPU oracle
(through the tests) take their inputs from here, so that the two sides see
the same bits.

Generator (counter based, so any slice can be drawn on its own):

* ``key(seed, tid) = seed * G + tid * 0xD1B54A32D192ED03  (mod 2**64)`` with
  ``G = 0x9E3779B97F4A7C15``;
* for flat index ``n`` the state is ``key + (n + 1) * G``, passed through the
  SplitMix64 finaliser (Steele, Lea, Flood, "Fast splittable pseudorandom
  number generators", OOPSLA 2014);
* the high and low 32-bit halves give ``u1, u2 = (h + 0.5) / 2**32`` in (0, 1);
* Box-Muller in float64: ``sqrt(-2 ln u1) * cos(2 pi u2)``;
* values are scaled/shifted in float64, rounded to float32 (nearest even),
  then to bfloat16 (nearest even).

Tensor ids: Q = 1, K noise = 2, K per-channel offset = 3, V = 4, W = 5,
outlier-channel pick = 6; linear layers (W8A8): activations = 7, weights = 8.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

_G = np.uint64(0x9E3779B97F4A7C15)
_G2 = np.uint64(0xD1B54A32D192ED03)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

TID_Q, TID_KNOISE, TID_KOFF, TID_V, TID_W, TID_OUTLIER = 1, 2, 3, 4, 5, 6
TID_LIN_X, TID_LIN_W = 7, 8
TID_DOUT = 9  # output gradient of the backward pass

_CHUNK = 1 << 22


def _key(seed: int, tid: int) -> np.uint64:
    return np.uint64((seed * 0x9E3779B97F4A7C15 + tid * 0xD1B54A32D192ED03) & (2**64 - 1))


def _mix(z: np.ndarray) -> np.ndarray:
    z ^= z >> np.uint64(30)
    z *= _M1
    z ^= z >> np.uint64(27)
    z *= _M2
    z ^= z >> np.uint64(31)
    return z


def raw_u64(seed: int, tid: int, start: int, count: int) -> np.ndarray:
    """SplitMix64 outputs for flat indices [start, start + count)."""
    with np.errstate(over="ignore"):
        n = np.arange(start + 1, start + count + 1, dtype=np.uint64)
        z = _key(seed, tid) + n * _G
        return _mix(z)


def _normal_chunk(seed, tid, start, count):
    z = raw_u64(seed, tid, start, count)
    u1 = ((z >> np.uint64(32)).astype(np.float64) + 0.5) * (1.0 / 4294967296.0)
    u2 = ((z & np.uint64(0xFFFFFFFF)).astype(np.float64) + 0.5) * (1.0 / 4294967296.0)
    return np.sqrt(-2.0 * np.log(u1)) * np.cos((2.0 * np.pi) * u2)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> float32 (nearest even) -> bfloat16 bits (nearest even)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
    r = np.where(nan, (u >> np.uint32(16)) | np.uint32(0x40), r)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def normal_bf16(seed: int, tid: int, count: int, start: int = 0, std: float = 1.0,
                add: np.ndarray | None = None, add_period: int = 0) -> np.ndarray:
    """bf16 bits of ``std * N(0,1) [+ add[(index // add_period?)]]`` for a flat range.

    ``add``: optional float64 vector added before rounding; element ``n`` of the
    output gets ``add[n % len(add)]`` when ``add_period == 0`` (per-channel
    offsets broadcast along rows), else ``add[(n // add_period) % len(add)]``.
    """
    out = np.empty(count, dtype=np.uint16)

    def work(lo):
        hi = min(count, lo + _CHUNK)
        v = _normal_chunk(seed, tid, start + lo, hi - lo) * std
        if add is not None:
            idx = np.arange(start + lo, start + hi, dtype=np.int64)
            if add_period:
                idx //= add_period
            v += add[idx % len(add)]
        out[lo:hi] = f64_to_bf16_bits(v)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(0, count, _CHUNK)))
    return out


@dataclass(frozen=True)
class Workload:
    """One synthetic SageSLA problem (shapes, sparsity, value distributions)."""
    name: str
    B: int
    H: int
    N: int
    d: int
    topk: float
    use_linear: int = 1
    koff_std: float = 2.0          # per-channel K offset ~ N(0, koff_std**2)
    outlier_frac: float = 0.0      # fraction of channels whose offset is scaled
    outlier_scale: float = 1.0
    seed: int = 0
    q_std: float = 1.0             # Q ~ N(0, q_std**2) (sharper attention when > 1)

    @property
    def T(self) -> int:
        return (self.N + 63) // 64

    def heads(self):
        return [(b, h) for b in range(self.B) for h in range(self.H)]


# The workloads: a tiny case, three Wan-shaped self-attention layers
# (latent 21 frames x 30 x 52 for 480P, 21 x 45 x 80 for 720P), a dense
# INT8 stress case with outlier K channels, and the 720P layer's per-GPU share
# under head sharding.
WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 1024, 64, 0.25),
    "wan1.3b-480p": Workload("wan1.3b-480p", 1, 12, 21 * 30 * 52, 128, 0.10),
    "wan14b-480p": Workload("wan14b-480p", 1, 40, 21 * 30 * 52, 128, 0.10),
    "wan14b-720p": Workload("wan14b-720p", 1, 40, 21 * 45 * 80, 128, 0.10),
    "dense-outlier": Workload("dense-outlier", 2, 12, 21 * 30 * 52, 128, 1.0, use_linear=0,
                              koff_std=4.0, outlier_frac=0.01, outlier_scale=20.0),
    # One GPU's share of the 720P layer when its 40 heads are split over 8
    # GPUs: 5 heads.  The generators are keyed by the flat element index, so
    # these are exactly heads 0..4 of "wan14b-720p".
    "wan14b-720p-shard8": Workload("wan14b-720p-shard8", 1, 5, 21 * 45 * 80, 128, 0.10),
}


def k_offsets(wl: Workload, b: int, h: int) -> np.ndarray:
    """float64 per-channel K offset of head (b, h), shared by all its tokens."""
    d = wl.d
    head = b * wl.H + h
    z = _normal_chunk(wl.seed, TID_KOFF, head * d, d) * wl.koff_std
    n_out = int(round(wl.outlier_frac * d))
    if n_out:
        picks = raw_u64(wl.seed, TID_OUTLIER, 0, 4 * n_out + 4)
        chosen = []
        for p in picks:
            c = int(p % np.uint64(d))
            if c not in chosen:
                chosen.append(c)
            if len(chosen) == n_out:
                break
        z[chosen] *= wl.outlier_scale
    return z


def head_inputs(wl: Workload, b: int, h: int):
    """bf16 bits of Q, K, V for one head, each [N, d] (uint16)."""
    n = wl.N * wl.d
    start = (b * wl.H + h) * n
    q = normal_bf16(wl.seed, TID_Q, n, start, std=wl.q_std)
    k = normal_bf16(wl.seed, TID_KNOISE, n, start, add=k_offsets(wl, b, h))
    v = normal_bf16(wl.seed, TID_V, n, start)
    return q.reshape(wl.N, wl.d), k.reshape(wl.N, wl.d), v.reshape(wl.N, wl.d)


def proj_weight(wl: Workload) -> np.ndarray:
    """bf16 bits of the d x d projection, entries ~ N(0, 1/d), [d_out, d_in]."""
    return normal_bf16(wl.seed, TID_W, wl.d * wl.d, std=1.0 / np.sqrt(wl.d)).reshape(wl.d, wl.d)


def all_inputs(wl: Workload):
    """bf16 bits of Q, K, V as [B, H, N, d] and W as [d, d]."""
    shape = (wl.B, wl.H, wl.N, wl.d)
    n = wl.B * wl.H * wl.N * wl.d
    q = normal_bf16(wl.seed, TID_Q, n, std=wl.q_std)
    offs = np.concatenate([k_offsets(wl, b, h) for b, h in wl.heads()])
    # offset of head e, channel c sits at offs[e * d + c]; flat index n of K
    # belongs to head n // (N d) and channel n % d.
    k = np.empty(n, dtype=np.uint16)
    per_head = wl.N * wl.d
    for e in range(wl.B * wl.H):
        k[e * per_head:(e + 1) * per_head] = normal_bf16(
            wl.seed, TID_KNOISE, per_head, e * per_head, add=offs[e * wl.d:(e + 1) * wl.d])
    v = normal_bf16(wl.seed, TID_V, n)
    return q.reshape(shape), k.reshape(shape), v.reshape(shape), proj_weight(wl)


def grad_output(wl: Workload) -> np.ndarray:
    """bf16 bits of the output gradient dO [B, H, N, d], N(0, 1) per element
    (the backward pass's seeded stand-in for a training loss's gradient)."""
    n = wl.B * wl.H * wl.N * wl.d
    return normal_bf16(wl.seed, TID_DOUT, n).reshape(wl.B, wl.H, wl.N, wl.d)


# ---- linear layers around attention (W8A8 GEMM inputs) ----------------------

@dataclass(frozen=True)
class LinearWorkload:
    """Y = X W^T with X [M, K] (tokens x input features), W [N, K] ([out, in])."""
    name: str
    M: int
    N: int
    K: int
    seed: int = 0
    x_std: float = 1.0


# Wan2.1-14B: model width 5120 (40 heads x 128), 720P latents 21x45x80 tokens.
LINEAR_WORKLOADS = {
    "wan14b-720p-qkv": LinearWorkload("wan14b-720p-qkv", 21 * 45 * 80, 3 * 5120, 5120),
    "wan14b-720p-o": LinearWorkload("wan14b-720p-o", 21 * 45 * 80, 5120, 5120),
    "small": LinearWorkload("small", 300, 200, 384, seed=3),
}


def linear_inputs(lw: LinearWorkload):
    """bf16 bits of X [M, K] ~ N(0, x_std^2) and W [N, K] ~ N(0, 1/K)."""
    x = normal_bf16(lw.seed, TID_LIN_X, lw.M * lw.K, std=lw.x_std).reshape(lw.M, lw.K)
    w = normal_bf16(lw.seed, TID_LIN_W, lw.N * lw.K, std=1.0 / np.sqrt(lw.K)).reshape(lw.N, lw.K)
    return x, w
