"""Pins of the fp64 oracle to facts that do not come from the oracle itself:
closed forms, invariants, brute force on tiny inputs and hand-derived values.

Each ``pin_*`` takes the oracle functions it checks as arguments, so that
``test_pins_catch_planted_mistakes`` can hand it a deliberately broken copy
(the mistake lives in this CPU test only) and confirm the pin fails.
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle.vc_oracle as O
from oracle import round as R
from synth import configs as C
from synth import gen as G
from synth import inputs as I

GOLD = __import__("os").path.join(__import__("os").path.dirname(__file__), "golden")


# ---------------------------------------------------------------- formats ---

def test_bf16_conversions():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x4049], dtype=np.uint16)
    want = [1.0, -2.0, 1.0 + 2 ** -7, 0.0, -0.0, 3.140625]
    assert list(O.bf16_to_f64(bits)) == want
    # round to nearest even on the fp32 -> bf16 step of the generator
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8) - 2 ** -20], dtype=np.float32)
    assert list(G.f32_to_bf16_bits(x)) == [0x3F80, 0x3F82, 0xBF81]


# ---------------------------------------------------------- quantisation ---

def pin_quant_brute_force(quantize_groups, dequant_groups, bits, seed=0, ngroups=400):
    """Every code is the nearest grid point of its value except at (near-)ties,
    and values outside [z, z + qmax s] clamp to the end codes; the dequantised
    value is within s/2 (plus fp32 rounding) inside the range."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((ngroups, 32)).astype(np.float32) * rng.uniform(0.01, 4, (ngroups, 1)).astype(np.float32)
    x = O.bf16_to_f64(G.f32_to_bf16_bits(x)).astype(np.float32)
    codes, s, z = quantize_groups(x, bits)
    qmax = (1 << bits) - 1
    deq = dequant_groups(codes, s, z)
    for gi in range(ngroups):
        S = Fraction(float(s[gi]))
        Z = Fraction(float(z[gi]))
        assert S > 0
        for i in range(32):
            X = Fraction(float(x[gi, i]))
            dist = [abs(X - (c * S + Z)) for c in range(qmax + 1)]
            best = min(range(qmax + 1), key=lambda c: dist[c])
            c = int(codes[gi, i])
            if c != best:
                # allowed only where two grid points are (almost) equally near
                assert abs(dist[c] - dist[best]) <= S * Fraction(1, 1 << 18), (gi, i, c, best)
            lo, hi = Z, Z + qmax * S
            if lo <= X <= hi:
                assert abs(X - Fraction(float(deq[gi, i]))) <= S / 2 * (1 + Fraction(1, 1 << 18)) + abs(X) * Fraction(1, 1 << 23)
            elif X < lo:
                assert c == 0
            else:
                assert c == qmax


def _dequant_groups(codes, s, z):
    return O.f64_to_f32_rn(codes.astype(np.float64) * O.f16_to_f64(s)[..., None] + O.f16_to_f64(z)[..., None])


@pytest.mark.parametrize("bits", [2, 4])
def test_quant_brute_force(bits):
    pin_quant_brute_force(O.quantize_groups, _dequant_groups, bits)


@pytest.mark.parametrize("bits", [2, 4])
def test_quant_grid_values_exact(bits):
    qmax = (1 << bits) - 1
    rng = np.random.default_rng(5)
    for s_val, z_val in [(0.25, -1.0), (0.0625, 3.5), (1.5, -7.0), (2.0 ** -6, 0.0)]:
        c = rng.integers(0, qmax + 1, 32)
        c[0], c[1] = 0, qmax
        x = (z_val + c * s_val).astype(np.float32)
        codes, s, z = O.quantize_groups(x[None], bits)
        assert float(s[0]) == s_val and float(z[0]) == z_val
        assert (codes[0] == c).all()
        assert (_dequant_groups(codes, s, z)[0] == x).all()


def test_quant_constant_group():
    x = np.full((1, 32), 0.7109375, dtype=np.float32)
    codes, s, z = O.quantize_groups(x, 2)
    assert float(s[0]) == 0.0 and (codes == 0).all()
    assert (_dequant_groups(codes, s, z) == x).all()


def test_quant_golden_hand_example():
    """tests/golden/quant_ramp_int4.txt: the ramp 0..31, 4-bit, derived by hand
    (see the derivation lines in the file)."""
    lines = [l for l in open(f"{GOLD}/quant_ramp_int4.txt") if l.strip() and not l.startswith("#")]
    kv = dict(l.split("=", 1) for l in lines)
    x = np.arange(32, dtype=np.float32)
    codes, s, z = O.quantize_groups(x[None], 4)
    assert float(s[0]) == float(kv["scale"])
    assert float(z[0]) == float(kv["zero"])
    assert list(codes[0]) == [int(t) for t in kv["codes"].split()]


def test_quant_k_v_grouping_axes():
    """K groups run over 32 tokens of one channel; V groups over 32 channels of one token."""
    n, D = 64, 64
    k = np.zeros((n, D), np.float32)
    k[:32, 5] = np.arange(32)          # one K group: channel 5, tokens 0..31
    kc, ks, kz = O.quantize_k(k, 4)
    assert ks.shape == (2, D) and float(ks[0, 5]) > 0 and (ks[1] == 0).all()
    assert (np.delete(ks[0], 5) == 0).all()
    v = np.zeros((n, D), np.float32)
    v[7, 32:64] = np.arange(32)        # one V group: token 7, channels 32..63
    vc, vs, vz = O.quantize_v(v, 4)
    assert vs.shape == (n, 2) and float(vs[7, 1]) > 0
    assert float(vs.sum()) == float(vs[7, 1])


def test_quant_blocks_are_independent():
    """What makes a rolled-over cache equal a one-shot one: every group, and
    every packed byte and metadata word, depends on the rows of its own
    32-token block only, so the cache of rows [0, n) is the concatenation of the
    caches of its blocks."""
    rng = np.random.default_rng(7)
    n, D, bits = 128, 64, 2
    k = (rng.standard_normal((n, D)) * rng.uniform(0.1, 4, (n, 1))).astype(np.float32)
    v = (rng.standard_normal((n, D)) * rng.uniform(0.1, 4, (1, D))).astype(np.float32)
    c, s, z = O.quantize_k(k, bits)
    cv, sv, zv = O.quantize_v(v, bits)
    kb = [O.quantize_k(k[i:i + 32], bits) for i in range(0, n, 32)]
    vb = [O.quantize_v(v[i:i + 32], bits) for i in range(0, n, 32)]
    assert np.array_equal(O.pack_codes(c, bits), np.concatenate([O.pack_codes(b[0], bits) for b in kb]))
    assert np.array_equal(s, np.concatenate([b[1] for b in kb])) and np.array_equal(z, np.concatenate([b[2] for b in kb]))
    assert np.array_equal(O.pack_codes(cv, bits), np.concatenate([O.pack_codes(b[0], bits) for b in vb]))
    assert np.array_equal(sv, np.concatenate([b[1] for b in vb])) and np.array_equal(zv, np.concatenate([b[2] for b in vb]))
    # and a block's K groups do see all of its 32 rows: changing one row moves them
    k2 = k.copy()
    k2[40] += 100.0
    assert not np.array_equal(O.quantize_k(k2, bits)[1][1], s[1])
    assert np.array_equal(O.quantize_k(k2, bits)[1][0], s[0])


def test_pack_codes_bit_layout():
    c4 = np.array([[1, 2, 3, 4, 15, 0, 9, 10]], np.uint8)
    assert list(O.pack_codes(c4, 4)[0]) == [0x21, 0x43, 0x0F, 0xA9]
    c2 = np.array([[1, 2, 3, 0, 3, 3, 3, 3]], np.uint8)
    assert list(O.pack_codes(c2, 2)[0]) == [0b00111001, 0xFF]


def test_dequant_fraction_exact():
    rng = np.random.default_rng(2)
    codes = rng.integers(0, 16, (64, 64)).astype(np.uint8)
    s = rng.uniform(0.01, 1, (2, 64)).astype(np.float16)
    z = rng.uniform(-3, 0, (2, 64)).astype(np.float16)
    d = O.dequant_k(codes, s, z)
    for (t, c) in [(0, 0), (31, 63), (32, 1), (63, 17)]:
        exact = int(codes[t, c]) * Fraction(float(s[t // 32, c])) + Fraction(float(z[t // 32, c]))
        assert d[t, c] == float(np.float32(float(exact)))


def pin_dequant_v(dequant_v):
    """V dequantisation against exact fractions: value (t, c) takes the fp16 pair
    of group c // 32 of its own token t, and code * s + z is rounded once to
    fp32.  The scales carry a full 11-bit significand, so for most codes the
    exact value needs more than 11 bits: an fp16 rounding of the result, or of
    the product alone, shows; a pair taken from another group or token shows."""
    n, D = 3, 96
    codes = (np.arange(n * D).reshape(n, D) * 7 % 16).astype(np.uint8)
    s = np.array([[1 + 2 ** -10, 0.3330078125, 3.0009765625],
                  [0.0999755859375, 1.2001953125, 0.0],
                  [5.00390625, 2 ** -14 * 1.5, 0.7001953125]], np.float16)
    z = np.array([[-1.0009765625, 0.5, -7.25],
                  [2.001953125, -0.0999755859375, 1.5],
                  [-3.0, 0.0, 6.00390625]], np.float16)
    d = dequant_v(codes, s, z)
    assert d.shape == (n, D)
    for t in range(n):
        for c in range(D):
            exact = int(codes[t, c]) * Fraction(float(s[t, c // 32])) + Fraction(float(z[t, c // 32]))
            assert d[t, c] == float(np.float32(float(exact))), (t, c)
    # hand values: t 0, c 1 (code 7, group 0): 7 (1 + 2^-10) - 1.0009765625 = 6 + 7 2^-10 - 2^-10 = 6.005859375
    assert d[0, 1] == 6.005859375
    # t 1, c 70 (code (96 + 70) 7 % 16 = 10, group 2, s = 0): exactly the zero point 1.5
    assert d[1, 70] == 1.5


def test_dequant_v_pin():
    pin_dequant_v(O.dequant_v)


def pin_logits(logits):
    """Logits of one position: the head outputs concatenated head by head, then
    times W.  A 2-head, 2-channel example worked by hand, where the head-major
    order is visible, and a random one against the sum over heads of each
    head's output times its own D rows of W (a block decomposition of the same
    product)."""
    o = np.array([[1.0, 2.0], [3.0, 4.0]])
    W = np.array([[1.0, 0.0, 0.0], [0.0, 1.0, 0.0], [0.0, 0.0, 1.0], [1.0, 1.0, 1.0]])
    # concat = [1, 2, 3, 4]: column v is x_v + 4
    assert list(logits(o, W)) == [5.0, 6.0, 7.0]
    rng = np.random.default_rng(23)
    Hq, D, V = 3, 4, 5
    o = rng.standard_normal((Hq, D))
    W = rng.standard_normal((Hq * D, V))
    want = sum(o[h] @ W[h * D:(h + 1) * D] for h in range(Hq))
    got = logits(o, W)
    assert got.shape == (V,)
    assert np.allclose(got, want, atol=1e-13, rtol=0)


def test_logits_pin():
    pin_logits(O.logits)


def test_dequant_v_and_logits_pins_catch_planted_mistakes():
    def dv_swapped(codes, s, z):
        return O.dequant_v(codes, z, s)

    def dv_f16_round(codes, s, z):
        sf = np.repeat(O.f16_to_f64(s), 32, axis=1)
        zf = np.repeat(O.f16_to_f64(z), 32, axis=1)
        return (codes * sf + zf).astype(np.float16).astype(np.float64)

    def dv_f16_product(codes, s, z):
        sf = np.repeat(O.f16_to_f64(s), 32, axis=1)
        zf = np.repeat(O.f16_to_f64(z), 32, axis=1)
        return O.f64_to_f32_rn((codes * sf).astype(np.float16).astype(np.float64) + zf)

    def dv_interleaved_groups(codes, s, z):
        # channel c in group c % (D/32) instead of c // 32
        sf = np.tile(O.f16_to_f64(s), (1, 32))
        zf = np.tile(O.f16_to_f64(z), (1, 32))
        return O.f64_to_f32_rn(codes * sf + zf)

    def dv_first_token_pairs(codes, s, z):
        # every token reads the pairs of token 0 (a group per channel range, not per token)
        return O.dequant_v(codes, np.repeat(s[:1], len(s), 0), np.repeat(z[:1], len(z), 0))

    for bad in (dv_swapped, dv_f16_round, dv_f16_product, dv_interleaved_groups, dv_first_token_pairs):
        with pytest.raises(AssertionError):
            pin_dequant_v(bad)

    def lg_channel_major(o, W):
        return o.T.reshape(-1) @ W

    def lg_heads_reversed(o, W):
        return o[::-1].reshape(-1) @ W

    def lg_mean_of_heads(o, W):
        D = o.shape[1]
        return sum(o[h] @ W[h * D:(h + 1) * D] for h in range(o.shape[0])) / o.shape[0]

    for bad in (lg_channel_major, lg_heads_reversed, lg_mean_of_heads):
        with pytest.raises(AssertionError):
            pin_logits(bad)


def pin_draft_lse(lse):
    """The log-sum-exp of the draft scores: one key gives its scaled score
    exactly; n equal keys give ln n plus that score; a random case equals the
    sum of exponentials written out with math.fsum; no key gives -inf."""
    q = np.array([[1.0, 2.0], [-0.5, 0.25]])
    k1 = np.array([[3.0, -1.0]])
    # scores 0.5 (1*3 - 2*1) = 0.5 and 0.5 (-1.5 - 0.25) = -0.875
    assert list(lse(q, k1, 0.5)) == [0.5, -0.875]
    kn = np.repeat(k1, 5, axis=0)
    assert np.allclose(lse(q, kn, 0.5), [0.5 + math.log(5), -0.875 + math.log(5)], atol=1e-15, rtol=0)
    rng = np.random.default_rng(31)
    q = rng.standard_normal((3, 8))
    keys = rng.standard_normal((11, 8))
    want = [math.log(math.fsum(math.exp(0.3 * float(q[i] @ keys[t])) for t in range(11))) for i in range(3)]
    assert np.allclose(lse(q, keys, 0.3), want, atol=1e-13, rtol=0)
    assert list(lse(q, keys[:0], 0.3)) == [-np.inf] * 3


def test_draft_lse_pin():
    pin_draft_lse(O.draft_lse_unit)


def test_draft_lse_pin_catches_planted_mistakes():
    def lse_log2(q, keys, scale):
        return O.draft_lse_unit(q, keys, scale) / math.log(2)

    def lse_unscaled(q, keys, scale):
        return O.draft_lse_unit(q, keys, 1.0)

    def lse_max_only(q, keys, scale):
        return (q @ keys.T * scale).max(axis=1) if len(keys) else np.full(len(q), -np.inf)

    def lse_mean(q, keys, scale):
        return O.draft_lse_unit(q, keys, scale) - (math.log(len(keys)) if len(keys) else 0.0)

    for bad in (lse_log2, lse_unscaled, lse_max_only, lse_mean):
        with pytest.raises(AssertionError):
            pin_draft_lse(bad)


# -------------------------------------------------------------- attention ---

def pin_attention_closed_forms(attn):
    rng = np.random.default_rng(11)
    D = 16
    q = rng.standard_normal((3, D))
    v = rng.standard_normal((9, D))
    # all-equal keys: uniform weights -> mean of V
    kk = np.tile(rng.standard_normal(D), (9, 1))
    assert np.allclose(attn(q, kk, v, 0.25), v.mean(0)[None], atol=1e-14, rtol=0)
    # one key -> that value row
    assert np.allclose(attn(q, kk[:1], v[:1], 0.25), v[:1], atol=1e-15, rtol=0)
    # one key far ahead of the others -> its row within e^-40
    k2 = rng.standard_normal((9, D)) * 0.01
    k2[4] = q[0] * (60.0 / (q[0] @ q[0]))
    o = attn(q[:1], k2, v, 1.0)
    assert np.abs(o[0] - v[4]).max() < 9 * math.exp(-40) * np.abs(v).max()
    # a constant added to every score of a row leaves the output unchanged
    base = attn(q[:1], k2, v, 0.3)
    shift = k2 + 5.0 * q[0] / (q[0] @ q[0])
    assert np.allclose(attn(q[:1], shift, v, 0.3), base, atol=1e-12, rtol=0)
    # explicit formula with math.fsum for n <= 4
    for n in range(1, 5):
        kk = rng.standard_normal((n, D))
        vv = rng.standard_normal((n, D))
        qq = rng.standard_normal((1, D))
        sc = [math.fsum(qq[0, d] * kk[t, d] for d in range(D)) * 0.5 for t in range(n)]
        m = max(sc)
        e = [math.exp(x - m) for x in sc]
        den = math.fsum(e)
        want = [math.fsum(e[t] * vv[t, d] for t in range(n)) / den for d in range(D)]
        assert np.allclose(attn(qq, kk, vv, 0.5)[0], want, atol=1e-14, rtol=0)


def test_attention_closed_forms():
    pin_attention_closed_forms(O.softmax_attention)


def test_gqa_mapping():
    assert [O.gqa_kv_head(h, 8, 2) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]
    assert [O.gqa_kv_head(h, 4, 1) for h in range(4)] == [0] * 4
    assert [O.gqa_kv_head(h, 64, 8) for h in (0, 7, 8, 63)] == [0, 0, 1, 7]


def pin_verify(verify, attn):
    """Verify position j == a decode step over context + new rows 0..j (two code
    paths), is unchanged bitwise when later rows change, and n_q = 1 on the full
    cache equals identity decode."""
    rng = np.random.default_rng(3)
    g, nq, D, L = 3, 5, 16, 23
    q = rng.standard_normal((g, nq, D))
    k = rng.standard_normal((L + nq, D))
    v = rng.standard_normal((L + nq, D))
    out = verify(q, k, v, L, 0.25)
    for j in range(nq):
        dec = attn(q[:, j], k[:L + j + 1], v[:L + j + 1], 0.25)
        assert np.allclose(out[:, j], dec, atol=1e-13, rtol=0), j
    for j in range(nq):
        k2, v2 = k.copy(), v.copy()
        k2[L + j + 1:] += 7.0
        v2[L + j + 1:] -= 3.0
        out2 = verify(q, k2, v2, L, 0.25)
        assert np.array_equal(out2[:, j], out[:, j]), j
    # brute force with explicit loops for one position
    j = 2
    for h in range(g):
        sc = [math.fsum(q[h, j, d] * k[t, d] for d in range(D)) * 0.25 for t in range(L + j + 1)]
        m = max(sc)
        e = [math.exp(x - m) for x in sc]
        den = math.fsum(e)
        want = [math.fsum(e[t] * v[t, d] for t in range(L + j + 1)) / den for d in range(D)]
        assert np.allclose(out[h, j], want, atol=1e-13, rtol=0)


def test_verify_pins():
    pin_verify(O.verify_attention_unit, O.softmax_attention)


def test_draft_kinds_agree():
    """token_drop keeping every index == identity == verify position 0 (n_q = 1)."""
    rng = np.random.default_rng(4)
    L, D = 40, 16
    k = rng.standard_normal((L + 1, D))
    v = rng.standard_normal((L + 1, D))
    q = rng.standard_normal((2, D))
    kc1, vc1 = O.draft_kv_rows("token_drop", k_full=k, v_full=v, keep_idx=np.arange(L),
                               tail_k=k[L:], tail_v=v[L:])
    kc2, vc2 = O.draft_kv_rows("identity", k_full=k, v_full=v, L=L, tail_k=k[L:], tail_v=v[L:])
    a = O.draft_attention_unit(q, kc1, vc1, 0.25)
    b = O.draft_attention_unit(q, kc2, vc2, 0.25)
    c = O.verify_attention_unit(q[:, None], k, v, L, 0.25)[:, 0]
    assert np.array_equal(a, b)
    assert np.allclose(a, c, atol=1e-13, rtol=0)
    # dropping a row changes the result (the index set is honoured)
    kc3, vc3 = O.draft_kv_rows("token_drop", k_full=k, v_full=v, keep_idx=np.arange(1, L),
                               tail_k=k[L:], tail_v=v[L:])
    assert not np.allclose(O.draft_attention_unit(q, kc3, vc3, 0.25), a)


# ------------------------------------------------------------- acceptance ---

def pin_accept(accept_fn, argmax_fn):
    assert argmax_fn(np.array([1.0, 3.0, 3.0, -1.0])) == 1
    assert argmax_fn(np.array([-5.0, -5.0])) == 0
    # brute force over all binary draft/verify strings of length <= 4
    for k in range(0, 5):
        for d in itertools.product([0, 1], repeat=k):
            for y in itertools.product([0, 1], repeat=k + 1):
                out, n = accept_fn(np.array(d, dtype=np.int64), np.array(y, dtype=np.int64))
                lcp = 0
                while lcp < k and d[lcp] == y[lcp]:
                    lcp += 1
                assert n == lcp
                assert list(out[:n]) == list(d[:n]) and out[n] == y[n]
                assert (out[n + 1:] == -1).all() and len(out) == k + 1
    # identity drafts accept everything plus the bonus token
    y = np.array([5, 9, 2, 7, 1])
    out, n = accept_fn(y[:4].copy(), y)
    assert n == 4 and list(out) == [5, 9, 2, 7, 1]
    # a mismatch forced at i gives exactly i accepted drafts
    for i in range(4):
        d = y[:4].copy()
        d[i] = (d[i] + 1) % 10
        out, n = accept_fn(d, y)
        assert n == i and list(out[:i + 1]) == list(y[:i + 1])


def test_accept_pins():
    pin_accept(O.accept, O.argmax_first)


def test_prefetch_expected():
    """Hand-checked gathers: pages come out in (sequence, page) order from the
    slots the table names; a token range maps to the pages that hold it."""
    host = np.arange(8 * 4, dtype=np.uint8).reshape(8, 4) + 100
    table = np.array([[3, 0, 6, 1], [2, 7, 4, 5]], dtype=np.int32)
    out = O.prefetch_expected(host, table, [1], 16, 40, 16)   # tokens 16..39 -> pages 1, 2 of seq 1
    assert np.array_equal(out, host[[7, 4]])
    out = O.prefetch_expected(host, table, [1, 0], 0, 64, 16)
    assert np.array_equal(out, host[[2, 7, 4, 5, 3, 0, 6, 1]])
    out = O.prefetch_expected(host, table, [0], 17, 18, 16)    # one token -> its page only
    assert np.array_equal(out, host[[0]])
    assert O.prefetch_expected(host, table, [0], 5, 5, 16).shape == (0, 4)


# ------------------------------------------------------------ whole round ---

def _tiny_round(w, b=0):
    K = I.context_kv(w, "k")[b]
    V = I.context_kv(w, "v")[b]
    Kn = I.new_rows(w, "k")[b]
    Vn = I.new_rows(w, "v")[b]
    W = I.vocab_matrix(w)
    keep = I.keep_indices(w)[b] if w.kind == "token_drop" else None
    return K, V, Kn, Vn, W, keep


def test_round_identity_accepts_all():
    """An exact (identity) compressor drafts exactly what verify predicts: n = k."""
    w = C.TINY.with_(kind="identity")
    K, V, Kn, Vn, W, _ = _tiny_round(w)
    attempts, Q, r = R.plant_margins(w, 0, K, V, Kn, Vn, W)
    assert r["n_accept"] == w.k
    assert list(r["out_ids"]) == list(r["verify_ids"])


def test_round_quant_consistent():
    w = C.TINY
    K, V, Kn, Vn, W, _ = _tiny_round(w)
    attempts, Q, r = R.plant_margins(w, 0, K, V, Kn, Vn, W)
    n = r["n_accept"]
    assert 0 <= n <= w.k
    assert list(r["out_ids"][:n]) == list(r["draft_ids"][:n])
    assert r["out_ids"][n] == r["verify_ids"][n]
    # int4 draft output is close to, but not equal to, the exact draft
    wi = w.with_(kind="identity")
    ex = R.unit_draft(wi, K[0], V[0], Kn[0], Vn[0], Q[:4])
    rel = np.linalg.norm(r["draft_out"][:4] - ex) / np.linalg.norm(ex)
    assert 1e-4 < rel < 0.3


def test_round_token_drop_small():
    w = C.TINY.with_(kind="token_drop", keep_frac=0.25)
    K, V, Kn, Vn, W, keep = _tiny_round(w)
    assert keep.shape == (1, 128) and (np.diff(keep[0]) > 0).all()
    Q = I.queries(w)[0]
    r = R.sequence_round(w, 0, K, V, Kn, Vn, Q, W, keep=keep)
    # against a direct gather written out here
    sc = O.scale_for(w.D)
    kf, vf = O.bf16_to_f64(K[0]), O.bf16_to_f64(V[0])
    j = 3
    keys = np.concatenate([kf[keep[0]], O.bf16_to_f64(Kn[0, :j + 1])])
    vals = np.concatenate([vf[keep[0]], O.bf16_to_f64(Vn[0, :j + 1])])
    want = O.softmax_attention(O.bf16_to_f64(Q[:, j]), keys, vals, sc)
    assert np.allclose(r["draft_out"][:, j], want, atol=1e-14, rtol=0)


# ---------------------------------------- the pins catch planted mistakes ---

def test_pins_catch_planted_mistakes():
    def attn_no_scale(q, k, v, scale):
        return O.softmax_attention(q, k, v, 1.0)

    def attn_transposed_pv(q, k, v, scale):
        s = (q @ k.T) * scale
        p = np.exp(s - s.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        return (p @ v[::-1])

    def verify_off_by_one(q, k, v, L, scale):
        return O.verify_attention_unit(q, k, v, L - 1, scale)

    def verify_no_mask(q, k, v, L, scale):
        g, nq, D = q.shape
        return np.stack([O.softmax_attention(q[:, j], k[:L + nq], v[:L + nq], scale) for j in range(nq)], 1)

    def accept_no_bonus(d, y):
        out, n = O.accept(d, y)
        out = out.copy()
        out[n] = -1
        return out, n

    def accept_counts_all_matches(d, y):
        n = int(sum(int(a) == int(b) for a, b in zip(d, y)))
        out = np.full(len(d) + 1, -1)
        out[:n] = d[:n]
        out[n] = y[n]
        return out, n

    def argmax_last(x):
        return int(len(x) - 1 - np.argmax(x[::-1]))

    def quant_floor(x, bits):
        c, s, z = O.quantize_groups(x, bits)
        xf = np.asarray(x, np.float32)
        q = np.floor((xf - z.astype(np.float32)[..., None]) / s.astype(np.float32)[..., None])
        return np.clip(q, 0, (1 << bits) - 1).astype(np.uint8), s, z

    def dequant_swapped(codes, s, z):
        return _dequant_groups(codes, z, s)

    for bad in (attn_no_scale, attn_transposed_pv):
        with pytest.raises(AssertionError):
            pin_attention_closed_forms(bad)
    for bad in (verify_off_by_one, verify_no_mask):
        with pytest.raises(AssertionError):
            pin_verify(bad, O.softmax_attention)
    with pytest.raises(AssertionError):
        pin_accept(accept_no_bonus, O.argmax_first)
    with pytest.raises(AssertionError):
        pin_accept(accept_counts_all_matches, O.argmax_first)
    with pytest.raises(AssertionError):
        pin_accept(O.accept, argmax_last)
    with pytest.raises(AssertionError):
        pin_quant_brute_force(quant_floor, _dequant_groups, 4, ngroups=50)
    with pytest.raises(AssertionError):
        pin_quant_brute_force(O.quantize_groups, dequant_swapped, 4, ngroups=50)


# ---------------------------------------------------------------------------
# token selection: the defining property of the kept set, checked directly


def pin_select_top_m(select):
    """The kept set S (|S| = M) is defined by: every kept score >= every dropped
    score (as real numbers), and at the boundary value v = min kept score every
    kept index with score v is lower than every dropped index with score v; the
    list is ascending.  Checked on random rows with heavy ties, signed zeros and
    infinities, plus closed cases."""
    rng = np.random.default_rng(17)
    pool = np.array([-np.inf, -2.5, -0.0, 0.0, 0.75, 0.75, 3.0, np.inf])
    for trial in range(300):
        L = int(rng.integers(1, 40))
        s = pool[rng.integers(0, len(pool), L)] if trial % 2 else rng.standard_normal(L).round(1)
        M = int(rng.integers(0, L + 1))
        got = np.asarray(select(s, M))
        assert got.shape == (M,) and got.dtype == np.int32, (trial, got)
        assert np.all(np.diff(got) > 0), ("ascending, unique", trial, got)
        if M == 0:
            continue
        kept = np.zeros(L, bool)
        kept[got] = True
        ks, ds = s[kept], s[~kept]
        if ds.size:
            assert ks.min() >= ds.max(), ("kept >= dropped", trial, s, got)
            v = ks.min()
            ki = np.flatnonzero(kept & (s == v))
            di = np.flatnonzero(~kept & (s == v))
            if di.size:
                assert ki.max() < di.min(), ("ties to the lower index", trial, s, got)
    # closed cases
    s = np.array([0.5, 2.0, -1.0, 2.0, 0.5, 7.0])
    assert list(select(s, 3)) == [1, 3, 5]
    assert list(select(s, 4)) == [0, 1, 3, 5]
    assert list(select(s, 0)) == []
    assert list(select(s, 6)) == [0, 1, 2, 3, 4, 5]
    assert list(select(np.zeros(9), 4)) == [0, 1, 2, 3]
    assert list(select(np.array([0.0, -0.0, 0.0]), 2)) == [0, 1]


def test_select_top_m_pins():
    pin_select_top_m(O.select_top_m)


def test_select_pins_catch_planted_mistakes():
    def ties_high(s, M):
        s = np.asarray(s, np.float64)
        order = np.lexsort((-np.arange(len(s)), -s))
        return np.sort(order[:M]).astype(np.int32)

    def unsorted(s, M):
        s = np.asarray(s, np.float64)
        return np.lexsort((np.arange(len(s)), -s))[:M].astype(np.int32)

    def bottom_m(s, M):
        s = np.asarray(s, np.float64)
        return np.sort(np.lexsort((np.arange(len(s)), s))[:M]).astype(np.int32)

    def signed_zero_order(s, M):
        # orders -0 below +0 (bit patterns instead of values)
        s = np.asarray(s, np.float64)
        key = s + np.where(np.signbit(s) & (s == 0), -1e-300, 0.0)
        return np.sort(np.lexsort((np.arange(len(s)), -key))[:M]).astype(np.int32)

    for bad in (ties_high, unsorted, bottom_m, signed_zero_order):
        with pytest.raises(AssertionError):
            pin_select_top_m(bad)
