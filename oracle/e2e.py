"""fp64 reference of the end-to-end draft-then-verify loop on a tiny decoder (test infrastructure only).

[VC Core Algorithm] drafting runs the target model itself over a compressed
cache KV_comp; one forward pass over the full cache KV_full checks the k
drafts together; the drafts before the first one that differs from the
verifier's greedy token are kept, followed by the verifier's token at that
position, and the next round starts from there.  [VC Experimental Results]
with greedy decoding the loop emits exactly what the target model emits with
its full cache.

Model (the pages name none; readings):
  * Llama-style pre-norm decoder: x += O(attn(RMSNorm(x))); x += SwiGLU(RMSNorm(x));
    logits = RMSNorm(x) @ W_head.  RMSNorm(x) = x / sqrt(mean(x^2) + eps) * gain.
    SwiGLU(a) = (silu(a W_gate) * (a W_up)) W_down, silu(u) = u / (1 + e^-u).
  * Rotary positions on q and k, pairing channel i with i + D/2, from given
    cos/sin tables (data).
  * The attention operands are bf16: q, and the k and v rows written to the
    cache, are rounded to bf16 (nearest even) right after the projections
    (q and k after the rotation); attention outputs stay unrounded.
  * Query head h reads KV head floor(h * Hkv / Hq); scale 1/sqrt(D).
  * Draft cache: the prompt's K/V rows quantised with the asymmetric group
    quantiser (all prompt rows); generated rows stay exact (bf16) in a tail.
    Each round appends the verify-computed rows of the accepted positions (the
    pending token plus the accepted drafts) to the tail; rows the draft wrote
    for its own positions in that round are dropped.
  * The first generated token is the argmax of the prompt's last-position logits.
All arithmetic is float64 apart from the bf16 roundings stated above.
"""
from __future__ import annotations

import numpy as np

from . import vc_oracle as O


# ----------------------------------------------------------------------------
# elementwise pieces
# ----------------------------------------------------------------------------


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), returned as
    float64.  Direct from float64 (one rounding): keep the top 8 significant
    bits, i.e. round away the low 45 bits of the 52-bit fraction.  Finite normal
    inputs only (the model's activations are far from bf16's range limits)."""
    u = np.ascontiguousarray(x, dtype=np.float64).view(np.uint64)
    lsb = (u >> np.uint64(45)) & np.uint64(1)
    r = (u + np.uint64((1 << 44) - 1) + lsb) & ~np.uint64((1 << 45) - 1)
    return r.view(np.float64)


def rmsnorm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * gain


def silu(u: np.ndarray) -> np.ndarray:
    return u / (1.0 + np.exp(-u))


def rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate channel pairs (i, i + D/2) of x [..., n, D] by the angles whose
    cosines and sines are cos/sin [n, D/2] (one row per position)."""
    half = x.shape[-1] // 2
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * cos - b * sin, b * cos + a * sin], axis=-1)


# ----------------------------------------------------------------------------
# the model
# ----------------------------------------------------------------------------


class Model:
    """Weights as float64 (exact copies of the bf16 parameters)."""

    def __init__(self, cfg, W: dict, cos: np.ndarray, sin: np.ndarray):
        self.cfg = cfg
        f = O.bf16_to_f64
        self.embed = f(W["embed"])
        self.layers = []
        for l in range(cfg.n_layers):
            self.layers.append({name: f(W[name][l]) for name in
                                ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down", "attn_norm", "ffn_norm")})
        self.final_norm = f(W["final_norm"])
        self.head = f(W["lm_head"])
        self.cos = np.asarray(cos, dtype=np.float64)
        self.sin = np.asarray(sin, dtype=np.float64)
        self.scale = O.scale_for(cfg.D)

    def project(self, l: int, x: np.ndarray, pos: np.ndarray):
        """Hidden rows x [n, d] at positions pos [n] -> bf16-rounded q [Hq, n, D],
        k [Hkv, n, D], v [Hkv, n, D]."""
        c, P = self.cfg, self.layers[l]
        a = rmsnorm(x, P["attn_norm"], c.eps)
        n = x.shape[0]
        q = (a @ P["wq"]).reshape(n, c.Hq, c.D).transpose(1, 0, 2)
        k = (a @ P["wk"]).reshape(n, c.Hkv, c.D).transpose(1, 0, 2)
        v = (a @ P["wv"]).reshape(n, c.Hkv, c.D).transpose(1, 0, 2)
        cs, sn = self.cos[pos], self.sin[pos]
        return round_bf16(rope(q, cs, sn)), round_bf16(rope(k, cs, sn)), round_bf16(v)

    def finish_layer(self, l: int, x: np.ndarray, o: np.ndarray) -> np.ndarray:
        """Residual update of x [n, d] with the attention output o [Hq, n, D], then the feed-forward block."""
        c, P = self.cfg, self.layers[l]
        n = x.shape[0]
        x = x + o.transpose(1, 0, 2).reshape(n, c.Hq * c.D) @ P["wo"]
        a = rmsnorm(x, P["ffn_norm"], c.eps)
        return x + (silu(a @ P["w_gate"]) * (a @ P["w_up"])) @ P["w_down"]

    def logits(self, x: np.ndarray) -> np.ndarray:
        return rmsnorm(x, self.final_norm, self.cfg.eps) @ self.head

    def heads_of(self, h: int) -> slice:
        g = self.cfg.g
        assert all(O.gqa_kv_head(i, self.cfg.Hq, self.cfg.Hkv) == h for i in range(h * g, (h + 1) * g))
        return slice(h * g, (h + 1) * g)


class Cache:
    """Full (exact) cache of every layer: K, V [Hkv, L_cap, D] (bf16 values)."""

    def __init__(self, cfg):
        self.K = [np.zeros((cfg.Hkv, cfg.L_cap, cfg.D)) for _ in range(cfg.n_layers)]
        self.V = [np.zeros((cfg.Hkv, cfg.L_cap, cfg.D)) for _ in range(cfg.n_layers)]


def causal_pass(m: Model, cache: Cache, tokens: np.ndarray, start: int, chunk: int = 512) -> np.ndarray:
    """Run positions start .. start + n - 1 (tokens [n]) through every layer in
    one causal pass over the full cache, writing their K/V rows first.  This is
    the verify pass ([VC Core Algorithm]) and, with start = 0, the prefill.
    Query rows are taken in chunks (each row's attention is computed whole);
    returns the final hidden rows [n, d]."""
    c = m.cfg
    n = len(tokens)
    pos = np.arange(start, start + n)
    x = m.embed[tokens]
    for l in range(c.n_layers):
        q, k, v = m.project(l, x, pos)
        cache.K[l][:, start:start + n] = k
        cache.V[l][:, start:start + n] = v
        o = np.zeros((c.Hq, n, c.D))
        for h in range(c.Hkv):
            hs = m.heads_of(h)
            for c0 in range(0, n, chunk):
                c1 = min(n, c0 + chunk)
                o[hs, c0:c1] = O.verify_attention_unit(q[hs, c0:c1], cache.K[l][h, :start + c1],
                                                       cache.V[l][h, :start + c1], start + c0, m.scale)
        x = m.finish_layer(l, x, o)
    return x


def decode_step(m: Model, cache: Cache, token: int, pos: int) -> np.ndarray:
    """One position through every layer, attending to full-cache rows [0, pos]
    (its own row written first).  Returns the final hidden row [1, d]."""
    c = m.cfg
    x = m.embed[[token]]
    for l in range(c.n_layers):
        q, k, v = m.project(l, x, np.array([pos]))
        cache.K[l][:, pos] = k[:, 0]
        cache.V[l][:, pos] = v[:, 0]
        o = np.zeros((c.Hq, 1, c.D))
        for h in range(c.Hkv):
            hs = m.heads_of(h)
            kc, vc = O.draft_kv_rows("identity", k_full=cache.K[l][h], v_full=cache.V[l][h], L=pos + 1)
            o[hs, 0] = O.draft_attention_unit(q[hs, 0], kc, vc, m.scale)
        x = m.finish_layer(l, x, o)
    return x


def prefill(m: Model, cache: Cache, prompt: np.ndarray):
    """Prompt through the model; returns the last position's logits [V]."""
    x = causal_pass(m, cache, np.asarray(prompt), 0)
    return m.logits(x[-1:])[0]


def greedy_decode(m: Model, prompt: np.ndarray, n_gen: int, cache: Cache | None = None,
                  first_logits: np.ndarray | None = None):
    """Plain greedy decoding with the full cache.  Returns (tokens [n_gen],
    top-1 logits [n_gen], top-2 margins [n_gen]).  cache/first_logits may carry
    an already computed prefill (the cache is extended in place)."""
    P = len(prompt)
    if cache is None:
        cache = Cache(m.cfg)
        first_logits = prefill(m, cache, prompt)
    lg = first_logits
    toks, top, marg = [], [], []
    for i in range(n_gen):
        t = O.argmax_first(lg)
        toks.append(t)
        top.append(float(lg[t]))
        marg.append(O.top2_margin(lg))
        if i + 1 < n_gen:
            lg = m.logits(decode_step(m, cache, t, P + i))[0]
    return np.array(toks), np.array(top), np.array(marg)


# ----------------------------------------------------------------------------
# the draft-then-verify loop
# ----------------------------------------------------------------------------


class DraftCache:
    """Dequantised prompt rows of every (layer, kv-head): the lossy KV_comp.
    exact=True keeps the rows as they are (the identity compressor)."""

    def __init__(self, m: Model, cache: Cache, P: int, exact: bool = False):
        c = m.cfg
        self.kd, self.vd = [], []
        for l in range(c.n_layers):
            kl, vl = [], []
            for h in range(c.Hkv):
                if exact:
                    kl.append(cache.K[l][h, :P].copy())
                    vl.append(cache.V[l][h, :P].copy())
                    continue
                kf = cache.K[l][h, :P].astype(np.float32)     # exact: rows are bf16 values
                vf = cache.V[l][h, :P].astype(np.float32)
                kc, ks, kz = O.quantize_k(kf, c.bits)
                vc, vs, vz = O.quantize_v(vf, c.bits)
                kl.append(O.dequant_k(kc, ks, kz))
                vl.append(O.dequant_v(vc, vs, vz))
            self.kd.append(kl)
            self.vd.append(vl)


def draft_step(m: Model, cache: Cache, dc: DraftCache, P: int, ctx: int, rows_k, rows_v, token: int,
               pos: int) -> np.ndarray:
    """One draft position: attends to the compressed prompt, the exact tail
    (full-cache rows P .. ctx-1 committed by earlier rounds) and this round's
    draft rows (rows_k/rows_v [l][h] lists, extended in place with its own)."""
    c = m.cfg
    x = m.embed[[token]]
    for l in range(c.n_layers):
        q, k, v = m.project(l, x, np.array([pos]))
        o = np.zeros((c.Hq, 1, c.D))
        for h in range(c.Hkv):
            rows_k[l][h].append(k[h, 0])
            rows_v[l][h].append(v[h, 0])
            tail_k = np.concatenate([cache.K[l][h, P:ctx], np.array(rows_k[l][h])])
            tail_v = np.concatenate([cache.V[l][h, P:ctx], np.array(rows_v[l][h])])
            kc, vc = O.draft_kv_rows("quant", k_deq=dc.kd[l][h], v_deq=dc.vd[l][h], tail_k=tail_k, tail_v=tail_v)
            hs = m.heads_of(h)
            o[hs, 0] = O.draft_attention_unit(q[hs, 0], kc, vc, m.scale)
        x = m.finish_layer(l, x, o)
    return x


def vericache_decode(m: Model, prompt: np.ndarray, n_gen: int, cache: Cache | None = None,
                     first_logits: np.ndarray | None = None, exact_draft: bool = False):
    """Greedy generation by the draft-then-verify loop.  Returns (tokens
    [n_gen], per-round accepted draft counts, per-round draft tokens).
    exact_draft: draft from an uncompressed copy of the prompt rows."""
    c = m.cfg
    P = len(prompt)
    if cache is None:
        cache = Cache(c)
        first_logits = prefill(m, cache, prompt)
    dc = DraftCache(m, cache, P, exact=exact_draft)
    pending = O.argmax_first(first_logits)
    out = [pending]
    ctx = P                          # position of the pending token = rows in the cache
    accepted, drafted = [], []
    while len(out) < n_gen:
        rows_k = [[[] for _ in range(c.Hkv)] for _ in range(c.n_layers)]
        rows_v = [[[] for _ in range(c.Hkv)] for _ in range(c.n_layers)]
        d, tok = [], pending
        for j in range(c.k):
            x = draft_step(m, cache, dc, P, ctx, rows_k, rows_v, tok, ctx + j)
            tok = O.argmax_first(m.logits(x)[0])
            d.append(tok)
        x = causal_pass(m, cache, np.array([pending] + d), ctx)
        lg = m.logits(x)
        y = np.array([O.argmax_first(r) for r in lg])
        emitted, n = O.accept(np.array(d), y)
        out.extend(int(t) for t in emitted[:n + 1])
        accepted.append(n)
        drafted.append(d)
        ctx += n + 1                 # rows ctx .. ctx+n (pending + n drafts) stay; later rows are rewritten
        pending = int(emitted[n])
    return np.array(out[:n_gen]), accepted, drafted
