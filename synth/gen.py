"""Counter-free, substream-per-tensor generators (numpy PCG64 + SeedSequence).

Every named tensor draws from its own substream
``SeedSequence(entropy=seed, spawn_key=(TAG[name], *index))`` so that one unit
(e.g. one (batch, kv-head) slice) can be regenerated on its own, bit for bit,
without drawing the whole tensor.  Normal values are sampled in float32 and
rounded to bfloat16 with round-to-nearest-even on the bit patterns.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

TAG = {
    "k": 1, "v": 2, "q": 3, "k_new": 4, "v_new": 5, "w_vocab": 6,
    "keep": 7, "pages": 8, "draft_ids": 9, "misc": 10, "q_resample": 11,
    "model": 12, "prompt": 13, "plant": 14,
}


def threads_default() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def rng(seed: int, tag: str, *index: int) -> np.random.Generator:
    key = (TAG[tag],) + tuple(int(i) for i in index)
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy=int(seed), spawn_key=key)))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bit patterns.

    Inputs are finite (the generators never produce NaN or Inf)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def normal_f32(seed: int, tag: str, index: tuple, shape, std: float = 1.0) -> np.ndarray:
    g = rng(seed, tag, *index)
    out = np.empty(shape, dtype=np.float32)
    g.standard_normal(out=out, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def normal_bf16(seed: int, tag: str, shape, unit_dims: int = 2, std: float = 1.0,
                threads: int | None = None) -> np.ndarray:
    """N(0, std^2) sampled in float32, rounded to bf16; one substream per index of the
    leading ``unit_dims`` dimensions.  Returns uint16 bit patterns of ``shape``."""
    shape = tuple(int(s) for s in shape)
    lead = shape[:unit_dims]
    inner = shape[unit_dims:]
    out = np.empty(shape, dtype=np.uint16)
    units = list(np.ndindex(*lead)) if lead else [()]

    def one(idx):
        out[idx] = f32_to_bf16_bits(normal_f32(seed, tag, idx, inner, std))

    n = threads or threads_default()
    if len(units) == 1 or n == 1:
        for u in units:
            one(u)
    else:
        with ThreadPoolExecutor(n) as ex:
            list(ex.map(one, units))
    return out


def uniform_f32(seed: int, tag: str, index: tuple, shape, lo: float = 0.0, hi: float = 1.0) -> np.ndarray:
    g = rng(seed, tag, *index)
    return g.uniform(lo, hi, size=shape).astype(np.float32)


def kept_subset(seed: int, b: int, h: int, L: int, M: int) -> np.ndarray:
    """Sorted int32 indices of the kept tokens of one (batch, kv-head).

    Keeping the top-M of i.i.d. continuous importance scores selects a uniformly
    random M-subset of [0, L); this draws that subset directly."""
    g = rng(seed, "keep", b, h)
    idx = g.choice(L, size=M, replace=False)
    idx.sort()
    return idx.astype(np.int32)


def page_permutation(seed: int, n_pages: int) -> np.ndarray:
    """A seeded permutation of page slots: logical page i lives in slot perm[i]."""
    return rng(seed, "pages").permutation(n_pages).astype(np.int32)
