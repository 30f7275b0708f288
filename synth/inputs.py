"""Seeded inputs of a single-layer workload, as numpy arrays.

Layouts (row-major):
  context K/V   bf16 bits [B, Hkv, L, D]       one substream per (b, kv-head)
  new rows K/V  bf16 bits [B, Hkv, n_q, D]     rows of positions L .. L+k
  queries       bf16 bits [B, Hq, n_q, D]      one substream per (b, position, attempt)
  vocab matrix  fp32 [Hq*D, vocab]             N(0, 1/(Hq*D)), substream per 256-row block
  kept indices  int32 [B, Hkv, n_keep]         sorted (token_drop only)
  page table    int32 [B, ceil((L+n_q)/page)]  context pages shuffled over the pool
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import Workload
from .gen import (f32_to_bf16_bits, kept_subset, normal_bf16, normal_f32,
                  page_permutation, threads_default)


def context_kv(w: Workload, which: str) -> np.ndarray:
    assert which in ("k", "v")
    return normal_bf16(w.seed, which, (w.B, w.Hkv, w.L, w.D), unit_dims=2)


def context_kv_unit(w: Workload, which: str, b: int, h: int) -> np.ndarray:
    """[L, D] slice of ``context_kv`` regenerated alone (identical bits)."""
    return f32_to_bf16_bits(normal_f32(w.seed, which, (b, h), (w.L, w.D)))


def context_kv_seqs(w: Workload, which: str, seqs) -> np.ndarray:
    """[len(seqs), Hkv, L, D] rows of ``context_kv`` for the listed sequences only
    (identical bits; one substream per (b, kv-head), drawn in parallel)."""
    seqs = [int(b) for b in seqs]
    out = np.empty((len(seqs), w.Hkv, w.L, w.D), dtype=np.uint16)

    def one(ih):
        i, h = ih
        out[i, h] = context_kv_unit(w, which, seqs[i], h)

    with ThreadPoolExecutor(threads_default()) as ex:
        list(ex.map(one, [(i, h) for i in range(len(seqs)) for h in range(w.Hkv)]))
    return out


def new_rows(w: Workload, which: str) -> np.ndarray:
    assert which in ("k", "v")
    return normal_bf16(w.seed, which + "_new", (w.B, w.Hkv, w.n_q, w.D), unit_dims=2)


def query_position(w: Workload, b: int, j: int, attempt: int = 0) -> np.ndarray:
    """[Hq, D] bf16 bits of the query vectors of position j of sequence b."""
    return f32_to_bf16_bits(normal_f32(w.seed, "q", (b, j, attempt), (w.Hq, w.D)))


def queries(w: Workload, attempts: np.ndarray | None = None) -> np.ndarray:
    out = np.empty((w.B, w.Hq, w.n_q, w.D), dtype=np.uint16)
    for b in range(w.B):
        for j in range(w.n_q):
            a = 0 if attempts is None else int(attempts[b, j])
            out[b, :, j, :] = query_position(w, b, j, a)
    return out


def vocab_matrix(w: Workload) -> np.ndarray:
    rows = w.Hq * w.D
    out = np.empty((rows, w.vocab), dtype=np.float32)
    blk = 256

    def one(i):
        r0 = i * blk
        r1 = min(rows, r0 + blk)
        out[r0:r1] = normal_f32(w.seed, "w_vocab", (i,), (r1 - r0, w.vocab), std=w.w_std)

    nblk = (rows + blk - 1) // blk
    with ThreadPoolExecutor(threads_default()) as ex:
        list(ex.map(one, range(nblk)))
    return out


def keep_indices(w: Workload) -> np.ndarray:
    out = np.empty((w.B, w.Hkv, w.n_keep), dtype=np.int32)
    for b in range(w.B):
        for h in range(w.Hkv):
            out[b, h] = kept_subset(w.seed, b, h, w.L, w.n_keep)
    return out


def pages_per_seq(w: Workload) -> int:
    return (w.L + w.n_q + w.page_tokens - 1) // w.page_tokens


def page_table(w: Workload) -> tuple[np.ndarray, int]:
    """Shuffled table for the whole context pages of every sequence, then one
    fresh slot per page that holds new rows (those pages live only on the
    device; with L not a multiple of the page size the first of them also holds
    the last context rows).  Returns (table [B, pages_per_seq], total slots)."""
    ctx_pages = w.L // w.page_tokens
    n_ctx = w.B * ctx_pages
    perm = page_permutation(w.seed, n_ctx)
    pps = pages_per_seq(w)
    extra = pps - ctx_pages
    tab = np.empty((w.B, pps), dtype=np.int32)
    tab[:, :ctx_pages] = perm.reshape(w.B, ctx_pages)
    tab[:, ctx_pages:] = n_ctx + np.arange(w.B * extra, dtype=np.int32).reshape(w.B, extra)
    return tab, n_ctx + w.B * extra
