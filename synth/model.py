"""Seeded weights, prompt and rotary tables of the tiny decoder (data only).

Every matrix draws from its own substream (tag "model", index (layer + 1,
matrix)) in float32 and is rounded to bfloat16.  Standard deviations are
1/sqrt(fan_in) (W_q: q_gain/sqrt(fan_in)); RMSNorm gains are 1 + N(0, 0.1^2);
the embedding is N(0, 1).

Successor plant: a seeded permutation succ of the vocabulary; column v of the
vocabulary head gets plant * e / d added, where e is the embedding row
of pred(v) = succ^-1(v) scaled to unit RMS.  Through the residual stream the
final hidden state of a position holding token t keeps a component along that
embedding row, so the logit of succ(t) is raised by about plant times the
cosine between the two, which keeps the greedy top-1 margins away from zero.

Rotary tables: angle(pos, i) = pos * theta^(-2 i / D) for i < D/2, evaluated in
float64 and rounded to float32; the same tables serve both sides.
"""
from __future__ import annotations

import numpy as np

from .configs import TinyLM
from .gen import f32_to_bf16_bits, normal_f32, rng

LAYER_MATS = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down", "attn_norm", "ffn_norm")


def _mat(cfg: TinyLM, idx: tuple, shape, std: float) -> np.ndarray:
    return f32_to_bf16_bits(normal_f32(cfg.seed, "model", idx, shape, std))


def _gain(cfg: TinyLM, idx: tuple, n: int) -> np.ndarray:
    return f32_to_bf16_bits(np.float32(1.0) + normal_f32(cfg.seed, "model", idx, (n,), 0.1))


def successor(cfg: TinyLM) -> np.ndarray:
    return rng(cfg.seed, "plant").permutation(cfg.vocab).astype(np.int64)


def weights(cfg: TinyLM) -> dict:
    """bf16 bit patterns (uint16) of every parameter; per-layer entries are lists."""
    d, F, V = cfg.d_model, cfg.ffn, cfg.vocab
    qd, kd = cfg.Hq * cfg.D, cfg.Hkv * cfg.D
    W = {"embed": _mat(cfg, (0, 0), (V, d), 1.0)}
    for name in LAYER_MATS:
        W[name] = []
    for l in range(cfg.n_layers):
        i = l + 1
        W["wq"].append(_mat(cfg, (i, 0), (d, qd), cfg.q_gain / np.sqrt(d)))
        W["wk"].append(_mat(cfg, (i, 1), (d, kd), 1.0 / np.sqrt(d)))
        W["wv"].append(_mat(cfg, (i, 2), (d, kd), 1.0 / np.sqrt(d)))
        W["wo"].append(_mat(cfg, (i, 3), (qd, d), 1.0 / np.sqrt(qd)))
        W["w_gate"].append(_mat(cfg, (i, 4), (d, F), 1.0 / np.sqrt(d)))
        W["w_up"].append(_mat(cfg, (i, 5), (d, F), 1.0 / np.sqrt(d)))
        W["w_down"].append(_mat(cfg, (i, 6), (F, d), 1.0 / np.sqrt(F)))
        W["attn_norm"].append(_gain(cfg, (i, 7), d))
        W["ffn_norm"].append(_gain(cfg, (i, 8), d))
    W["final_norm"] = _gain(cfg, (cfg.n_layers + 1, 0), d)
    head = normal_f32(cfg.seed, "model", (cfg.n_layers + 1, 1), (d, V), 1.0 / np.sqrt(d))
    if cfg.plant:
        e = (W["embed"].astype(np.uint32) << np.uint32(16)).view(np.float32)      # [V, d] exact
        rms = np.sqrt(np.mean(e.astype(np.float64) ** 2, axis=1, keepdims=True))
        unit = (e / rms).astype(np.float32)                                          # unit-RMS rows
        pred = np.argsort(successor(cfg))                                           # pred[succ[t]] = t
        head += np.float32(cfg.plant / d) * unit[pred].T
    W["lm_head"] = f32_to_bf16_bits(head)
    return W


def prompt(cfg: TinyLM, request: int = 0) -> np.ndarray:
    """Prompt ids of request `request` (request 0 is the configuration's own prompt)."""
    g = rng(cfg.seed, "prompt") if request == 0 else rng(cfg.seed, "prompt", request)
    return g.integers(0, cfg.vocab, size=cfg.prompt).astype(np.int64)


def rope_tables(cfg: TinyLM, n_pos: int | None = None):
    """cos, sin float32 [n_pos, D/2]."""
    n = cfg.L_cap if n_pos is None else n_pos
    half = cfg.D // 2
    inv = cfg.rope_theta ** (-2.0 * np.arange(half, dtype=np.float64) / cfg.D)
    ang = np.arange(n, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
