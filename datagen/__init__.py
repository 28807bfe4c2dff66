"""Seeded synthetic inputs for the int4 (q4f16_1) decode path.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark. It only draws random numbers and rounds them to the storage types;
it holds none of the method's arithmetic (no packing, no dequantisation, no
matmul, no normalisation).

Distributions follow the workloads described on the Zero-TVM pages and the
q4f16_1 format (Zero TVM Documentation, "Q4F16 quantization format"):

* 4-bit codes: uniform integers in [0, 15], one per weight, as ``uint8[N][K]``.
  Packing them into ``uint32`` words is the method's job, not this module's.
* scales: uniform in [0.005, 0.05], rounded to IEEE binary16 (round to nearest
  even), one per 32-element K-group, ``float16[N][K/32]``.
* activations: standard normal, rounded to binary16.
* RMSNorm gammas: normal with mean 1 and std 0.1, rounded to binary16.
* MoE routing: per token, ``topk`` distinct expert ids drawn uniformly without
  replacement, and routing weights equal to the softmax of ``topk`` standard
  normal logits, rounded to binary16. The router itself is not part of the
  method under test; these are inputs.

Every generator takes an explicit integer seed and uses numpy's PCG64 bit
generator, so the same seed yields the same bytes on any host with this numpy.
"""
from __future__ import annotations

import numpy as np

#: Base of the per-tensor seed scheme: seed = BASE + 1000 * workload + tensor.
SEED_BASE = 0x51A7E5EED

#: Scale distribution bounds.
SCALE_LO = 0.005
SCALE_HI = 0.05

#: Quantisation group length along K.
GROUP = 32


def seed_for(workload: int, tensor: int) -> int:
    """Deterministic seed for tensor number ``tensor`` of workload ``workload``."""
    return SEED_BASE + 1000 * int(workload) + int(tensor)


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(int(seed)))


def codes(seed: int, n: int, k: int) -> np.ndarray:
    """Uniform 4-bit codes in [0, 15] as ``uint8[n][k]``."""
    return _rng(seed).integers(0, 16, size=(n, k), dtype=np.uint8)


def words(seed: int, n: int, k: int) -> np.ndarray:
    """Uniform random 32-bit words ``uint32[n][k // 8]``.

    Every 4-bit field of a uniform random word is an independent uniform code in
    [0, 15], whatever the field order, so these words are a draw of ``n * k``
    uniform codes already in packed form. Used for the large workloads, where
    drawing one byte per code would dominate the set-up time.
    """
    if k % 8:
        raise ValueError(f"K={k} is not a multiple of 8")
    count = n * (k // 8)
    raw = _rng(seed).bit_generator.random_raw((count + 1) // 2).astype("<u8")
    return raw.view("<u4")[:count].reshape(n, k // 8).copy()


def scales(seed: int, n: int, k: int) -> np.ndarray:
    """One binary16 scale per 32-element K-group: ``float16[n][k // 32]``."""
    if k % GROUP:
        raise ValueError(f"K={k} is not a multiple of {GROUP}")
    u = _rng(seed).uniform(SCALE_LO, SCALE_HI, size=(n, k // GROUP))
    return u.astype(np.float16)


def normal_f16(seed: int, shape, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    """Normal draws rounded to binary16."""
    v = _rng(seed).normal(mean, std, size=shape)
    return v.astype(np.float16)


def activations(seed: int, m: int, k: int) -> np.ndarray:
    """``m`` independent f16 activation rows of length ``k`` drawn from N(0, 1)."""
    return normal_f16(seed, (m, k))


def gammas(seed: int, count: int, d: int) -> np.ndarray:
    """``count`` RMSNorm weight vectors of length ``d`` drawn from N(1, 0.1)."""
    return normal_f16(seed, (count, d), 1.0, 0.1)


def routing(seed: int, t: int, n_experts: int, topk: int):
    """Synthetic MoE routing for ``t`` tokens.

    Returns ``(ids int32[t][topk], weights float16[t][topk])``. Ids are
    distinct per token, drawn uniformly without replacement; weights are the
    softmax of ``topk`` N(0, 1) logits, computed in float64 and rounded to
    binary16.
    """
    if topk > n_experts:
        raise ValueError("topk exceeds the number of experts")
    r = _rng(seed)
    ids = np.empty((t, topk), dtype=np.int32)
    for i in range(t):
        ids[i] = r.choice(n_experts, size=topk, replace=False)
    logits = r.normal(0.0, 1.0, size=(t, topk))
    e = np.exp(logits - logits.max(axis=1, keepdims=True))
    w = e / e.sum(axis=1, keepdims=True)
    return ids, w.astype(np.float16)


def routing_pool(seed: int, count: int, t: int, n_experts: int, topk: int):
    """``count`` independent routings of ``t`` tokens (for cycling in a benchmark)."""
    out = [routing(seed + 7919 * i, t, n_experts, topk) for i in range(count)]
    ids = np.stack([o[0] for o in out])
    w = np.stack([o[1] for o in out])
    return ids, w


def logits(seed: int, m: int, n: int, ties: bool = False, special: bool = False) -> np.ndarray:
    """``m`` rows of ``n`` float32 logits drawn from N(0, 3^2).

    ties: values rounded to multiples of 1/2, so a row's maximum is often shared
    by several positions. special: each row also gets -0.0, +0.0, -inf and +inf
    at random positions, and every third row a NaN or two.
    """
    r = _rng(seed)
    v = r.normal(0.0, 3.0, size=(m, n))
    if ties:
        v = np.round(v * 2.0) / 2.0
    v = v.astype(np.float32)
    if special:
        for i in range(m):
            pos = r.integers(0, n, size=4)
            v[i, pos] = np.array([-0.0, 0.0, -np.inf, np.inf], np.float32)
            if i % 3 == 2:
                v[i, r.integers(0, n, size=2)] = np.nan
    return v


def q4_matrix(seed: int, n: int, k: int):
    """Codes and scales of one int4 weight matrix (two seeds derived from ``seed``)."""
    return codes(seed, n, k), scales(seed + 500, n, k)
