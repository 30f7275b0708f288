"""Pins of the end-to-end oracle (the tiny decoder and its draft-then-verify
loop) to facts that do not come from the oracle itself: hand-derived values,
library special cases, closed forms, invariants of the model and the pages'
losslessness claim, and a planted model whose greedy output is known.

Each ``pin_*`` takes the function it checks as an argument, so that
``test_e2e_pins_catch_planted_mistakes`` can hand it a deliberately broken
copy (the mistake lives in this CPU test only) and confirm that the pin fails.
"""
import numpy as np
import pytest

import oracle.e2e as E
import oracle.vc_oracle as O
from synth import configs as C
from synth import model as M


def _model(cfg):
    W = M.weights(cfg)
    cos, sin = M.rope_tables(cfg)
    return E.Model(cfg, W, cos, sin), M.prompt(cfg)


# ------------------------------------------------------------ elementwise ---

def pin_round_bf16(round_bf16):
    # hand values: bf16 keeps 7 fraction bits, so the spacing on [1, 2) is 2^-7
    x = np.array([1 + 2 ** -8,               # halfway 1 | 1+2^-7 -> even (1)
                  1 + 3 * 2 ** -8,           # halfway 1+2^-7 | 1+2^-6 -> even (1+2^-6)
                  1 + 2 ** -8 + 2 ** -40,    # just above halfway -> up
                  -(1 + 2 ** -8),            # sign symmetric
                  3.0, 2 ** -100 * 1.75])
    want = [1.0, 1 + 2 ** -6, 1 + 2 ** -7, -1.0, 3.0, 2 ** -100 * 1.75]
    assert list(round_bf16(x)) == want
    # fp32 inputs: the single rounding is what torch's fp32 -> bf16 conversion does
    torch = pytest.importorskip("torch")
    r = np.random.default_rng(3).standard_normal(20000).astype(np.float32) * 10.0
    ref = torch.from_numpy(r).to(torch.bfloat16).float().numpy().astype(np.float64)
    assert np.array_equal(round_bf16(r.astype(np.float64)), ref)


def test_round_bf16():
    pin_round_bf16(E.round_bf16)


def pin_rmsnorm(rmsnorm):
    eps = 1e-5
    g = np.linspace(0.5, 1.5, 16)
    for cval in (3.0, -0.25, 1e-3):
        x = np.full((2, 16), cval)
        want = np.broadcast_to(cval / np.sqrt(cval * cval + eps) * g, x.shape)
        np.testing.assert_allclose(rmsnorm(x, g, eps), want, rtol=1e-14)
    # scale invariance away from eps: rmsnorm(a x) == sign(a) rmsnorm(x) for |x| >> sqrt(eps)
    x = np.random.default_rng(1).standard_normal((3, 16)) * 100
    np.testing.assert_allclose(rmsnorm(7 * x, g, 0.0), rmsnorm(x, g, 0.0), rtol=1e-13)


def test_rmsnorm():
    pin_rmsnorm(E.rmsnorm)


def pin_silu(silu):
    u = np.linspace(-30, 30, 121)
    assert silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(silu(u) - silu(-u), u, atol=1e-12)          # silu(u) - silu(-u) = u
    np.testing.assert_allclose(silu(np.array([2.0])), 2.0 / (1.0 + np.exp(-2.0)), rtol=1e-15)
    np.testing.assert_allclose(silu(np.array([40.0])), 40.0, rtol=1e-15)


def test_silu():
    pin_silu(E.silu)


def pin_rope(rope):
    D = 8
    rng = np.random.default_rng(5)
    theta = 10000.0
    inv = theta ** (-2.0 * np.arange(D // 2) / D)
    tab = lambda p: (np.cos(np.outer(p, inv)), np.sin(np.outer(p, inv)))  # noqa: E731
    # position 0 is the identity
    x = rng.standard_normal((1, D))
    c0, s0 = tab(np.array([0]))
    np.testing.assert_array_equal(rope(x, c0, s0), x)
    # hand example: channel 0 pairs with channel D/2, rotated by the position's angle
    e = np.zeros((1, D))
    e[0, 0] = 1.0
    c, s = tab(np.array([1]))
    got = rope(e, c, s)[0]
    want = np.zeros(D)
    want[0], want[D // 2] = np.cos(1.0), np.sin(1.0)
    np.testing.assert_allclose(got, want, atol=1e-15)
    # norms are kept and q.k depends only on the offset between the positions
    q, k = rng.standard_normal((1, D)), rng.standard_normal((1, D))
    dots = []
    for m, n in ((5, 2), (13, 10), (1003, 1000)):
        cm, sm = tab(np.array([m]))
        cn, sn = tab(np.array([n]))
        qm, kn = rope(q, cm, sm), rope(k, cn, sn)
        np.testing.assert_allclose(np.linalg.norm(qm), np.linalg.norm(q), rtol=1e-13)
        dots.append(float(qm[0] @ kn[0]))
    np.testing.assert_allclose(dots, dots[0], rtol=1e-10)


def test_rope():
    pin_rope(E.rope)


# ------------------------------------------------------------------ model ---

def test_prefill_last_logits_equal_incremental_decode():
    """The causal pass over P tokens (verify code path, chunked rows) and a pass
    over P-1 tokens followed by one decode step (decode code path) give the same
    last-position logits: pins the causal mask, positions and cache writes."""
    cfg = C.LM_SMALL.with_(prompt=96)
    m, p = _model(cfg)
    a = E.Cache(cfg)
    la = E.prefill(m, a, p)
    b = E.Cache(cfg)
    E.causal_pass(m, b, p[:-1], 0, chunk=7)
    lb = m.logits(E.decode_step(m, b, int(p[-1]), len(p) - 1))[0]
    np.testing.assert_allclose(la, lb, rtol=0, atol=1e-9 * np.abs(la).max())
    for l in range(cfg.n_layers):
        np.testing.assert_array_equal(a.K[l][:, :96], b.K[l][:, :96])
        np.testing.assert_array_equal(a.V[l][:, :96], b.V[l][:, :96])


def test_planted_model_follows_successor_chain():
    """All block weights zero: attention and feed-forward add nothing, the final
    hidden state is the token's embedding and a head made only of the planted
    columns picks succ(t).  Greedy decoding must walk the successor chain."""
    cfg = C.LM_SMALL.with_(prompt=64, n_gen=24, plant=5.0)
    W = M.weights(cfg)
    for name in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"):
        W[name] = [np.zeros_like(w) for w in W[name]]
    from synth.gen import f32_to_bf16_bits
    e = O.bf16_to_f64(W["embed"])
    succ = M.successor(cfg)
    head = np.zeros((cfg.d_model, cfg.vocab))
    head[:, succ] = (e / np.sqrt(np.mean(e * e, axis=1, keepdims=True))).T
    W["lm_head"] = f32_to_bf16_bits(head.astype(np.float32))
    cos, sin = M.rope_tables(cfg)
    m = E.Model(cfg, W, cos, sin)
    p = M.prompt(cfg)
    toks, _, marg = E.greedy_decode(m, p, cfg.n_gen)
    chain = [int(succ[p[-1]])]
    for _ in range(cfg.n_gen - 1):
        chain.append(int(succ[chain[-1]]))
    assert list(toks) == chain
    assert marg.min() > 0


# ------------------------------------------------------------------- loop ---

def pin_loop_lossless(vericache_decode, greedy_decode, cfg):
    """[VC Experimental Results] the loop's greedy output equals full-cache
    greedy decoding; [VC Core Algorithm] at least one draft is rejected (the
    rollback path runs) and every round emits n + 1 tokens."""
    m, p = _model(cfg)
    tg, _, marg = greedy_decode(m, p, cfg.n_gen)
    tv, acc, drafted = vericache_decode(m, p, cfg.n_gen)
    assert list(tv) == list(tg)
    assert min(acc) < cfg.k, "no rejected draft: rollback untested"
    assert 1 + sum(a + 1 for a in acc) >= cfg.n_gen
    for n, d in zip(acc, drafted):
        assert len(d) == cfg.k and 0 <= n <= cfg.k


def test_loop_equals_greedy_small():
    pin_loop_lossless(E.vericache_decode, E.greedy_decode, C.LM_SMALL)


def test_identity_compressor_accepts_every_draft():
    """An exact draft cache makes draft and verify compute the same model, so
    every round accepts all k drafts plus the bonus token."""
    cfg = C.LM_SMALL
    m, p = _model(cfg)
    tg, _, _ = E.greedy_decode(m, p, cfg.n_gen)
    tv, acc, _ = E.vericache_decode(m, p, cfg.n_gen, exact_draft=True)
    assert list(tv) == list(tg)
    assert all(a == cfg.k for a in acc)


# ---------------------------------------------------------------- mutants ---

def test_e2e_pins_catch_planted_mistakes():
    def bf16_truncate(x):
        u = np.ascontiguousarray(x, dtype=np.float64).view(np.uint64)
        return (u & ~np.uint64((1 << 45) - 1)).view(np.float64)

    def rms_no_mean(x, g, eps):
        return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps) * g

    def silu_wrong(u):
        return u / (1.0 + np.exp(u))

    def rope_adjacent_pairs(x, cos, sin):
        a, b = x[..., 0::2], x[..., 1::2]
        out = np.empty_like(x)
        out[..., 0::2] = a * cos - b * sin
        out[..., 1::2] = b * cos + a * sin
        return out

    def rope_sign(x, cos, sin):
        half = x.shape[-1] // 2
        a, b = x[..., :half], x[..., half:]
        return np.concatenate([a * cos - b * sin, b * cos - a * sin], axis=-1)

    for pin, bad in ((pin_round_bf16, bf16_truncate), (pin_rmsnorm, rms_no_mean), (pin_silu, silu_wrong),
                     (pin_rope, rope_adjacent_pairs), (pin_rope, rope_sign)):
        with pytest.raises(AssertionError):
            pin(bad)

    # a loop that keeps the draft's own rows instead of the verified ones, or that
    # drops the bonus token, must break losslessness or the emitted count
    def loop_keep_draft_rows(m, prompt, n_gen):
        cache = E.Cache(m.cfg)
        first = E.prefill(m, cache, prompt)
        orig = E.causal_pass

        def verify_without_write(mm, cc, toks, start, chunk=512):
            saved = [(k[:, start:start + len(toks)].copy(), v[:, start:start + len(toks)].copy())
                     for k, v in zip(cc.K, cc.V)]
            x = orig(mm, cc, toks, start, chunk)
            for (k, v), K, V in zip(saved, cc.K, cc.V):
                K[:, start:start + len(toks)] = k     # verified rows discarded
                V[:, start:start + len(toks)] = v
            return x
        E.causal_pass = verify_without_write
        try:
            return E.vericache_decode(m, prompt, n_gen, cache=cache, first_logits=first)
        finally:
            E.causal_pass = orig

    with pytest.raises(AssertionError):
        pin_loop_lossless(loop_keep_draft_rows, E.greedy_decode, C.LM_SMALL)
