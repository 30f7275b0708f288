"""Parity of the HIP path (through the C ABI) with the fp64 oracle on the same
seeded inputs.  Sizes span several key tiles, several splits and ragged tails.

Bars: bit-exact for codes, scales/zeros, dequantised values, token ids, accept
lengths and copied bytes; relative L2 <= 1e-3 and max-abs <= 5e-3 * max|ref| for
attention outputs.
"""
import numpy as np
import pytest

import oracle.vc_oracle as O
from oracle import round as R
from synth import configs as C
from synth import inputs as I

pytestmark = pytest.mark.gpu

REL_L2 = 1e-3
MAX_ABS = 5e-3


def _vc():
    import compressed_kv_draft_amd as vc
    return vc


def assert_close(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), what
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
    mx = np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-300)
    print(f"[parity] {what}: rel_l2={rel:.3e} max_abs/max|ref|={mx:.3e}", flush=True)
    assert rel <= REL_L2 and mx <= MAX_ABS, (what, rel, mx)


DRAFT_CASES = [
    C.TINY,
    C.TINY.with_(name="int2_d128_g4", B=2, Hq=8, Hkv=2, D=128, L=1056, k=5, bits=2, residual=32, seed=21),
    C.TINY.with_(name="int4_d128_g8", B=1, Hq=16, Hkv=2, D=128, L=800, k=3, bits=4, residual=32, seed=22),
    C.TINY.with_(name="int2_d64_g8_long", B=1, Hq=8, Hkv=1, D=64, L=4128, k=2, bits=2, residual=32, seed=23),
    C.TINY.with_(name="identity_d128_g8", B=2, Hq=16, Hkv=2, D=128, L=777, k=3, kind="identity", seed=24),
    C.TINY.with_(name="drop_d128_g8", B=2, Hq=16, Hkv=2, D=128, L=1000, k=4, kind="token_drop",
                 keep_frac=0.1, seed=25),
    C.TINY.with_(name="drop_d64_g4", B=1, Hq=4, Hkv=1, D=64, L=3000, k=2, kind="token_drop",
                 keep_frac=0.3, seed=26),
    C.TINY.with_(name="int4_d128_g2_longtail", B=2, Hq=4, Hkv=2, D=128, L=1636, k=4, bits=4, residual=100,
                 seed=27),
    C.TINY.with_(name="int2_d128_g1", B=1, Hq=2, Hkv=2, D=128, L=2080, k=3, bits=2, residual=32, seed=28),
    C.TINY.with_(name="int4_d64_allresidual", B=1, Hq=8, Hkv=2, D=64, L=96, k=3, bits=4, residual=96, seed=29),
    C.TINY.with_(name="int2_d128_g4_splits", B=1, Hq=4, Hkv=1, D=128, L=16512, k=2, bits=2, residual=128,
                 seed=30),
    # (batch x kv-head) units a multiple of 8: the XCD-affine grid and combine row mapping
    C.TINY.with_(name="xcd_int2_d128_g4_u8", B=2, Hq=16, Hkv=4, D=128, L=2080, k=3, bits=2, residual=64, seed=32),
    C.TINY.with_(name="xcd_int4_d64_g2_u16", B=4, Hq=8, Hkv=4, D=64, L=1100, k=2, bits=4, residual=44, seed=33),
    C.TINY.with_(name="xcd_drop_d128_g8_u8", B=1, Hq=64, Hkv=8, D=128, L=3000, k=2, kind="token_drop",
                 keep_frac=0.2, seed=34),
    C.TINY.with_(name="xcd_identity_d128_g1_u8", B=8, Hq=8, Hkv=8, D=128, L=500, k=2, kind="identity", seed=35),
    C.TINY.with_(name="xcd_int2_d128_g4_u8_ragged", B=2, Hq=16, Hkv=4, D=128, L=70, k=2, bits=2, residual=38,
                 seed=36),
]


@pytest.mark.parametrize("w", DRAFT_CASES, ids=lambda w: w.name)
def test_draft_parity(w):
    print(f"[case] draft {w.name}", flush=True)
    from compressed_kv_draft_amd.workload import DeviceWorkload
    dw = DeviceWorkload(w, with_vocab=False)
    for j in range(w.k):
        dw.draft_step(j)
    got = dw.draft_out.cpu().numpy()       # [k, B, Hq, D]
    g = w.g
    for b in range(w.B):
        for h in range(w.Hkv):
            keep = dw.keep_np[b, h] if w.kind == "token_drop" else None
            ref = R.unit_draft(w, dw.np["K"][b, h], dw.np["V"][b, h], dw.np["Kn"][b, h], dw.np["Vn"][b, h],
                               dw.np["Q"][b, h * g:(h + 1) * g], keep=keep)          # [g, k, D]
            assert_close(got[:, b, h * g:(h + 1) * g].transpose(1, 0, 2), ref, f"{w.name} b{b} h{h}")


QUANT_CASES = [(64, 4), (64, 2), (128, 4), (128, 2)]


@pytest.mark.parametrize("D,bits", QUANT_CASES)
def test_quantize_bit_exact(D, bits):
    import torch
    vc = _vc()
    print(f"[case] quantize D={D} bits={bits}", flush=True)
    w = C.TINY.with_(B=2, Hkv=2, Hq=4, D=D, L=320, seed=31 + D + bits)
    K = I.context_kv(w, "k")
    V = I.context_kv(w, "v")
    # edge groups: a constant K group, a constant V group, a tiny-range group, a huge-range group
    K[0, 0, 32:64, 3] = K[0, 0, 32, 3]
    V[1, 1, 7, 0:32] = V[1, 1, 7, 0]
    K[1, 0, 64:96, 5] = np.uint16(0x3F80) + np.arange(32, dtype=np.uint16) % 2   # 1.0 and 1.0078125
    V[0, 1, 9, 32:64] = np.where(np.arange(32) % 2, np.uint16(0x4700), np.uint16(0xC700))  # +-32768
    K[0, 1, 0:32, 0] = np.uint16(0x3A83) + np.arange(32, dtype=np.uint16) % 4   # scale is an f16 subnormal
    nq = 288
    from compressed_kv_draft_amd.workload import bf16_dev
    kd, vd = bf16_dev(K, "cuda"), bf16_dev(V, "cuda")
    comp = vc.quantize_kv(kd, vd, bits, nq)
    kc, vcd, km, vm = (t.cpu().numpy() for t in vc.unpack_quant(comp, w.B, w.Hkv, D))
    for b in range(w.B):
        for h in range(w.Hkv):
            kf = O.bf16_to_f64(K[b, h, :nq]).astype(np.float32)
            vf = O.bf16_to_f64(V[b, h, :nq]).astype(np.float32)
            _check_canonical_unit(kc[b, h], km[b, h], vcd[b, h], vm[b, h], kf, vf, bits, (b, h))
            c, s, z = O.quantize_k(kf, bits)
            dq = vc.debug_dequant(comp, w.B, w.Hkv, D, b, h, 0).cpu().numpy()
            assert np.array_equal(dq.astype(np.float64), O.dequant_k(c, s, z)), (b, h, "k dequant")
            c, s, z = O.quantize_v(vf, bits)
            dq = vc.debug_dequant(comp, w.B, w.Hkv, D, b, h, 1).cpu().numpy()
            assert np.array_equal(dq.astype(np.float64), O.dequant_v(c, s, z)), (b, h, "v dequant")


def _canonical(kf, vf, bits):
    """The oracle's quantisation of one unit in the canonical form of the C header:
    packed K and V code rows, K pairs [n/32, D, 2] and V pairs [n, D/32, 2] as f16 bits."""
    c, s, z = O.quantize_k(kf, bits)
    cv, sv, zv = O.quantize_v(vf, bits)
    pair = lambda a, b: np.stack([a.view(np.uint16), b.view(np.uint16)], axis=-1)
    return O.pack_codes(c, bits), pair(s, z), O.pack_codes(cv, bits), pair(sv, zv)


def _check_canonical_unit(kc, km, vcd, vm, kf, vf, bits, where):
    ck, ckm, cv, cvm = _canonical(kf, vf, bits)
    assert np.array_equal(kc, ck), (where, "k codes")
    assert np.array_equal(km.view(np.uint16), ckm), (where, "k meta")
    assert np.array_equal(vcd, cv), (where, "v codes")
    assert np.array_equal(vm.view(np.uint16), cvm), (where, "v meta")


@pytest.mark.parametrize("D,bits", QUANT_CASES)
def test_pack_canonical_feeds_draft(D, bits):
    """A compressor outside the library hands over the canonical form (here the
    oracle's own quantisation): vc_pack_quant turns it into the cache
    vc_draft_attn reads.  The packed cache equals vc_quantize_kv's byte for
    byte, unpacks to the same canonical arrays, and drafts like the oracle."""
    import torch
    vc = _vc()
    from compressed_kv_draft_amd.workload import bf16_dev
    print(f"[case] pack canonical D={D} bits={bits}", flush=True)
    w = C.TINY.with_(B=2, Hkv=2, Hq=8, D=D, L=384, seed=71 + D + bits)
    K = I.context_kv(w, "k")
    V = I.context_kv(w, "v")
    n, R = 320, 40
    canon = [np.zeros((w.B, w.Hkv) + shape, np.uint16 if i % 2 else np.uint8) for i, shape in
             enumerate([(n, D * bits // 8), (n // 32, D, 2), (n, D * bits // 8), (n, D // 32, 2)])]
    for b in range(w.B):
        for h in range(w.Hkv):
            kf = O.bf16_to_f64(K[b, h, :n]).astype(np.float32)
            vf = O.bf16_to_f64(V[b, h, :n]).astype(np.float32)
            for arr, part in zip(canon, _canonical(kf, vf, bits)):
                arr[b, h] = part
    dev = [torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda() for a in canon]
    kc_d, km_d, vc_d, vm_d = dev[0], dev[1].view(torch.float16), dev[2], dev[3].view(torch.float16)
    comp = vc.empty_quant(w.B, w.Hkv, D, bits, n + 64, "cuda")
    # two appends (blocks 0..5, then 6..9) to exercise dst_block
    vc.pack_quant(kc_d[:, :, :192].contiguous(), vc_d[:, :, :192].contiguous(), km_d[:, :, :6].contiguous(),
                  vm_d[:, :, :192].contiguous(), comp)
    vc.pack_quant(kc_d[:, :, 192:].contiguous(), vc_d[:, :, 192:].contiguous(), km_d[:, :, 6:].contiguous(),
                  vm_d[:, :, 192:].contiguous(), comp)
    assert comp.desc.n_quant == n
    ref = vc.quantize_kv(bf16_dev(K, "cuda"), bf16_dev(V, "cuda"), bits, n, capacity=n + 64)
    torch.cuda.synchronize()
    for f in ("k_codes", "v_codes", "k_meta", "v_meta"):
        a = comp.t[f].view(torch.uint8).reshape(w.B, w.Hkv, -1)
        r = ref.t[f].view(torch.uint8).reshape(w.B, w.Hkv, -1)
        live = a.shape[2] * n // (n + 64)
        assert torch.equal(a[:, :, :live], r[:, :, :live]), f
    kc, vcd, km, vm = (t.cpu().numpy() for t in vc.unpack_quant(comp, w.B, w.Hkv, D))
    for b in range(w.B):
        for h in range(w.Hkv):
            assert np.array_equal(kc[b, h], canon[0][b, h]) and np.array_equal(vcd[b, h], canon[2][b, h])
            assert np.array_equal(km[b, h].view(np.uint16), canon[1][b, h])
            assert np.array_equal(vm[b, h].view(np.uint16), canon[3][b, h])
    tk = bf16_dev(np.ascontiguousarray(K[:, :, n:n + R]), "cuda")
    tv = bf16_dev(np.ascontiguousarray(V[:, :, n:n + R]), "cuda")
    tail = vc.Tail(tk, tv, torch.full((w.B,), R, dtype=torch.int32, device="cuda"))
    Q = I.queries(w)[:, :, 0]
    scale = O.scale_for(D)
    got = vc.draft_attn(comp, tail, bf16_dev(np.ascontiguousarray(Q), "cuda"), scale).cpu().numpy()
    g = w.Hq // w.Hkv
    for b in range(w.B):
        for h in range(w.Hkv):
            kf = O.bf16_to_f64(K[b, h, :n]).astype(np.float32)
            vf = O.bf16_to_f64(V[b, h, :n]).astype(np.float32)
            keys, vals = O.draft_kv_rows("quant", k_deq=O.dequant_k(*O.quantize_k(kf, bits)),
                                         v_deq=O.dequant_v(*O.quantize_v(vf, bits)),
                                         tail_k=O.bf16_to_f64(K[b, h, n:n + R]),
                                         tail_v=O.bf16_to_f64(V[b, h, n:n + R]))
            want = O.draft_attention_unit(O.bf16_to_f64(Q[b, h * g:(h + 1) * g]), keys, vals, scale)
            assert_close(got[b, h * g:(h + 1) * g], want, f"packed draft D{D} int{bits} b{b} h{h}")


ROLLOVER_CASES = [(64, 4), (128, 2), (128, 4)]


@pytest.mark.parametrize("D,bits", ROLLOVER_CASES)
def test_quantize_rollover_blocks(D, bits):
    """A QUANT cache grown block by block (rows leaving the exact window are
    quantised into the next blocks of a larger-capacity cache) holds the bytes
    the oracle's one-shot quantisation of the whole prefix gives, leaves the
    rows past n_quant untouched, and drafts over the capacity stride correctly."""
    import torch
    vc = _vc()
    from compressed_kv_draft_amd.workload import bf16_dev
    print(f"[case] rollover D={D} bits={bits}", flush=True)
    w = C.TINY.with_(B=2, Hkv=2, Hq=8, D=D, L=448, seed=61 + D + bits)
    K = I.context_kv(w, "k")
    V = I.context_kv(w, "v")
    n0, cap, R = 96, 384, 40
    comp = vc.quantize_kv(bf16_dev(K, "cuda"), bf16_dev(V, "cuda"), bits, n0, capacity=cap)
    for f in ("k_codes", "v_codes", "k_meta", "v_meta"):  # sentinel past the live rows
        t = comp.t[f].view(torch.uint8).view(w.B, w.Hkv, -1)
        t[:, :, t.shape[2] * n0 // cap:] = 0xA5
    # the exact window lives in its own buffer: rows [off, off + m) of it are
    # context rows [n, n + m); appends read it at a row offset
    off = 8
    win_k = np.zeros((w.B, w.Hkv, off + w.L - n0, D), dtype=np.uint16)
    win_v = np.zeros_like(win_k)
    win_k[:, :, off:] = K[:, :, n0:]
    win_v[:, :, off:] = V[:, :, n0:]
    wk, wv = bf16_dev(win_k, "cuda"), bf16_dev(win_v, "cuda")
    n = n0
    for nb in (3, 1, 4):
        vc.quantize_blocks(wk, wv, comp, off + n - n0, nb)
        n += 32 * nb
    assert n == comp.t["n_quant"] == comp.desc.n_quant == 352
    torch.cuda.synchronize()
    raw = {f: comp.t[f].view(torch.uint8).reshape(w.B, w.Hkv, -1).cpu().numpy()
           for f in ("k_codes", "v_codes", "k_meta", "v_meta")}
    kc, vcd, km, vm = (t.cpu().numpy() for t in vc.unpack_quant(comp, w.B, w.Hkv, D))
    for b in range(w.B):
        for h in range(w.Hkv):
            kf = O.bf16_to_f64(K[b, h, :n]).astype(np.float32)
            vf = O.bf16_to_f64(V[b, h, :n]).astype(np.float32)
            _check_canonical_unit(kc[b, h], km[b, h], vcd[b, h], vm[b, h], kf, vf, bits, (b, h))
            c, s, z = O.quantize_k(kf, bits)
            dq = vc.debug_dequant(comp, w.B, w.Hkv, D, b, h, 0).cpu().numpy()
            assert np.array_equal(dq.astype(np.float64), O.dequant_k(c, s, z)), (b, h, "k dequant")
            for f, arr in raw.items():
                live = arr.shape[2] * n // cap
                assert (arr[b, h, live:] == 0xA5).all(), (b, h, f, "past n_quant")
    # draft over the grown cache: quantised [0, n), then exact rows [n, n + R)
    tk = bf16_dev(np.ascontiguousarray(K[:, :, n:n + R]), "cuda")
    tv = bf16_dev(np.ascontiguousarray(V[:, :, n:n + R]), "cuda")
    tail = vc.Tail(tk, tv, torch.full((w.B,), R, dtype=torch.int32, device="cuda"))
    Q = I.queries(w)[:, :, 0]
    scale = O.scale_for(D)
    got = vc.draft_attn(comp, tail, bf16_dev(np.ascontiguousarray(Q), "cuda"), scale).cpu().numpy()
    g = w.Hq // w.Hkv
    for b in range(w.B):
        for h in range(w.Hkv):
            kf = O.bf16_to_f64(K[b, h, :n]).astype(np.float32)
            vf = O.bf16_to_f64(V[b, h, :n]).astype(np.float32)
            keys, vals = O.draft_kv_rows("quant", k_deq=O.dequant_k(*O.quantize_k(kf, bits)),
                                         v_deq=O.dequant_v(*O.quantize_v(vf, bits)),
                                         tail_k=O.bf16_to_f64(K[b, h, n:n + R]),
                                         tail_v=O.bf16_to_f64(V[b, h, n:n + R]))
            ref = O.draft_attention_unit(O.bf16_to_f64(Q[b, h * g:(h + 1) * g]), keys, vals, scale)
            assert_close(got[b, h * g:(h + 1) * g], ref, f"rollover draft D{D} int{bits} b{b} h{h}")


VERIFY_CASES = [
    C.TINY,
    C.TINY.with_(name="v_d128_g4_k32", B=2, Hq=8, Hkv=2, D=128, L=1000, k=32, seed=41),
    C.TINY.with_(name="v_d128_g8_k32", B=1, Hq=16, Hkv=2, D=128, L=2085, k=32, seed=42),
    C.TINY.with_(name="v_d64_g4_k3", B=3, Hq=8, Hkv=2, D=64, L=97, k=3, seed=43),
    C.TINY.with_(name="v_paged_d128_g8", B=2, Hq=16, Hkv=2, D=128, L=1024, k=32, paged=True,
                 page_tokens=16, seed=44),
    C.TINY.with_(name="v_paged_d64_pt32", B=2, Hq=4, Hkv=1, D=64, L=320, k=7, paged=True,
                 page_tokens=32, seed=45),
]


@pytest.mark.parametrize("w", VERIFY_CASES, ids=lambda w: w.name)
def test_verify_parity(w):
    from compressed_kv_draft_amd.workload import DeviceWorkload
    print(f"[case] verify {w.name}", flush=True)
    w = w.with_(kind="identity")
    dw = DeviceWorkload(w, with_vocab=False)
    got = dw.verify().cpu().numpy()      # [B, Hq, n_q, D]
    g = w.g
    for b in range(w.B):
        for h in range(w.Hkv):
            ref = R.unit_verify(w, dw.np["K"][b, h], dw.np["V"][b, h], dw.np["Kn"][b, h], dw.np["Vn"][b, h],
                                dw.np["Q"][b, h * g:(h + 1) * g])
            assert_close(got[b, h * g:(h + 1) * g], ref, f"{w.name} b{b} h{h}")


def test_verify_paged_unreadable_slots_read_as_zeros():
    """A page-table slot outside [0, n_slots) reads as zero rows (include/vc.h,
    vc_kv_full): the oracle sees those pages' K and V rows as zeros."""
    from compressed_kv_draft_amd.workload import DeviceWorkload
    print("[case] verify paged, unreadable slots", flush=True)
    w = C.TINY.with_(name="v_paged_bad", B=2, Hq=8, Hkv=2, D=128, L=320, k=7, paged=True, page_tokens=16,
                     seed=46, kind="identity")
    dw = DeviceWorkload(w, with_vocab=False)
    n_slots = int(dw.full.desc.n_slots)
    bad = {(0, 1): -1, (1, 3): n_slots + 5, (1, 0): -7, (0, 20): n_slots}  # page 20 holds the drafted rows
    for (b, p), v in bad.items():
        dw.page_table[b, p] = v
    got = dw.verify().cpu().numpy()
    pt, g = w.page_tokens, w.g
    for b in range(w.B):
        for h in range(w.Hkv):
            K, V = dw.np["K"][b, h][:w.L].copy(), dw.np["V"][b, h][:w.L].copy()
            Kn, Vn = dw.np["Kn"][b, h].copy(), dw.np["Vn"][b, h].copy()
            for (bb, p) in bad:
                if bb != b:
                    continue
                for r in range(p * pt, (p + 1) * pt):
                    if r < w.L:
                        K[r] = 0
                        V[r] = 0
                    elif r < w.L + w.n_q:
                        Kn[r - w.L] = 0
                        Vn[r - w.L] = 0
            ref = R.unit_verify(w, K, V, Kn, Vn, dw.np["Q"][b, h * g:(h + 1) * g])
            assert_close(got[b, h * g:(h + 1) * g], ref, f"paged bad slots b{b} h{h}")


def test_verify_prefill_causal():
    """ctx_len = 0 and many positions: plain causal self-attention (prefill)."""
    import torch
    vc = _vc()
    from compressed_kv_draft_amd.workload import bf16_dev
    print("[case] verify prefill", flush=True)
    rng = np.random.default_rng(7)
    B, Hq, Hkv, D, n = 1, 8, 2, 64, 300
    q = (rng.standard_normal((B, Hq, n, D)) ).astype(np.float32)
    k = rng.standard_normal((B, Hkv, n, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, n, D)).astype(np.float32)
    from synth.gen import f32_to_bf16_bits
    qb, kb, vb = (f32_to_bf16_bits(x) for x in (q, k, v))
    kd, vd = bf16_dev(kb, "cuda"), bf16_dev(vb, "cuda")
    full = vc.FullKV(kd, vd, L_cap=n)
    ctx = torch.zeros(B, dtype=torch.int32, device="cuda")
    scale = O.scale_for(D)
    got = vc.verify_attn(bf16_dev(qb, "cuda"), full, ctx, 0, Hkv, scale).cpu().numpy()
    g = Hq // Hkv
    for h in range(Hkv):
        ref = O.verify_attention_unit(O.bf16_to_f64(qb[0, h * g:(h + 1) * g]), O.bf16_to_f64(kb[0, h]),
                                      O.bf16_to_f64(vb[0, h]), 0, scale)
        assert_close(got[0, h * g:(h + 1) * g], ref, f"prefill h{h}")


@pytest.mark.parametrize("ctx,D,g", [([600, 523, 17], 128, 4), ([0, 611, 1], 128, 8), ([0, 0, 40], 64, 2)],
                         ids=["ragged", "empty_and_one_g8", "empty_d64"])
def test_verify_ragged_context_lengths(ctx, D, g):
    """Each sequence of the batch has its own context length (0 included: only
    the new rows, causally); the cache rows after a sequence's ctx_len + n_q
    hold large values that must not leak into it."""
    import torch
    vc = _vc()
    from compressed_kv_draft_amd.workload import bf16_dev
    from synth.gen import f32_to_bf16_bits
    print(f"[case] verify ragged ctx_len {ctx} D={D} g={g}", flush=True)
    rng = np.random.default_rng(11 + D + g)
    B, Hkv, n_q, L_cap = 3, 2, 9, 700
    Hq = g * Hkv
    k = rng.standard_normal((B, Hkv, L_cap, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, L_cap, D)).astype(np.float32)
    for b in range(B):
        k[b, :, ctx[b] + n_q:] = 40.0      # would dominate every score if read
        v[b, :, ctx[b] + n_q:] = 1000.0
    q = rng.standard_normal((B, Hq, n_q, D)).astype(np.float32)
    kb, vb, qb = (f32_to_bf16_bits(x) for x in (k, v, q))
    full = vc.FullKV(bf16_dev(kb, "cuda"), bf16_dev(vb, "cuda"), L_cap=L_cap)
    ctx_t = torch.tensor(ctx, dtype=torch.int32, device="cuda")
    scale = O.scale_for(D)
    got = vc.verify_attn(bf16_dev(qb, "cuda"), full, ctx_t, max(ctx), Hkv, scale).cpu().numpy()
    for b in range(B):
        n = ctx[b] + n_q
        for h in range(Hkv):
            ref = O.verify_attention_unit(O.bf16_to_f64(qb[b, h * g:(h + 1) * g]), O.bf16_to_f64(kb[b, h, :n]),
                                          O.bf16_to_f64(vb[b, h, :n]), ctx[b], scale)
            assert_close(got[b, h * g:(h + 1) * g], ref, f"ragged ctx b{b} h{h}")


CHUNK_CASES = [
    (C.TINY.with_(name="chunk_d128_g8_k32", B=2, Hq=16, Hkv=2, D=128, L=2085, k=32, seed=44), [517, 1500]),
    (C.TINY.with_(name="chunk_paged_d128_g8", B=2, Hq=16, Hkv=2, D=128, L=1200, k=32, paged=True, page_tokens=16,
                  seed=45), [256, 512, 768, 1024]),
    (C.TINY.with_(name="chunk_d64_g4_k3", B=3, Hq=8, Hkv=2, D=64, L=97, k=3, seed=46), [40]),
    # paged ranges that start inside a page, at rows that are not multiples of
    # 8: a load instruction must not read rows of the next page from this one
    (C.TINY.with_(name="chunk_paged_d64_unaligned", B=2, Hq=8, Hkv=2, D=64, L=1204, k=7, paged=True,
                  page_tokens=16, seed=47), [203, 700]),
    (C.TINY.with_(name="chunk_paged_d128_g8_unaligned", B=2, Hq=16, Hkv=2, D=128, L=1203, k=32, paged=True,
                  page_tokens=8, seed=48), [5, 299, 1195]),
]


@pytest.mark.parametrize("w,cuts", CHUNK_CASES, ids=[c[0].name for c in CHUNK_CASES])
def test_verify_chunked_ranges_merge(w, cuts):
    """Verify taken one key range at a time (as chunks of a full cache arrive)
    and merged equals the causal verify of the oracle; the ranges end at the
    context and the new rows form a range of their own."""
    import torch
    vc = _vc()
    from compressed_kv_draft_amd.workload import DeviceWorkload
    print(f"[case] chunked verify {w.name} cuts={cuts}", flush=True)
    w = w.with_(kind="identity")
    dw = DeviceWorkload(w, with_vocab=False)
    edges = [0] + list(cuts) + [w.L, w.L + w.n_q]
    B, Hq, n_q, D = dw.q_verify.shape
    slots = [vc.verify_range_parts(B, Hq, w.Hkv, D, n_q, a, b) for a, b in zip(edges[:-1], edges[1:])]
    rows = B * Hq * n_q * (D + 2)
    parts = torch.full((sum(slots) * rows,), float("nan"), dtype=torch.float32, device="cuda")
    off = 0
    for (a, b), n in zip(zip(edges[:-1], edges[1:]), slots):
        got_n = vc.verify_attn_range(dw.q_verify, dw.full, dw.ctx_len, w.L, w.Hkv, dw.scale, a, b,
                                     parts[off * rows:])
        assert got_n == n
        off += n
    got = vc.verify_merge(parts, sum(slots), B, Hq, n_q, D).cpu().numpy()
    g = w.g
    for b in range(w.B):
        for h in range(w.Hkv):
            ref = R.unit_verify(w, dw.np["K"][b, h], dw.np["V"][b, h], dw.np["Kn"][b, h], dw.np["Vn"][b, h],
                                dw.np["Q"][b, h * g:(h + 1) * g])
            assert_close(got[b, h * g:(h + 1) * g], ref, f"{w.name} b{b} h{h}")


def test_verify_chunked_ragged_context():
    """Ranges past a sequence's ctx_len + n_q leave it untouched (empty partials),
    and cache rows after that limit never leak in."""
    import torch
    vc = _vc()
    from compressed_kv_draft_amd.workload import bf16_dev
    from synth.gen import f32_to_bf16_bits
    print("[case] chunked verify ragged ctx_len", flush=True)
    rng = np.random.default_rng(12)
    B, Hq, Hkv, D, n_q, L_cap = 3, 16, 2, 128, 33, 900
    ctx = [800, 331, 5]
    k = rng.standard_normal((B, Hkv, L_cap, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, L_cap, D)).astype(np.float32)
    for b in range(B):
        k[b, :, ctx[b] + n_q:] = 40.0
        v[b, :, ctx[b] + n_q:] = 1000.0
    q = rng.standard_normal((B, Hq, n_q, D)).astype(np.float32)
    kb, vb, qb = (f32_to_bf16_bits(x) for x in (k, v, q))
    full = vc.FullKV(bf16_dev(kb, "cuda"), bf16_dev(vb, "cuda"), L_cap=L_cap)
    ctx_t = torch.tensor(ctx, dtype=torch.int32, device="cuda")
    scale = O.scale_for(D)
    qd = bf16_dev(qb, "cuda")
    edges = [0, 300, 600, max(ctx) + n_q]
    slots = [vc.verify_range_parts(B, Hq, Hkv, D, n_q, a, b) for a, b in zip(edges[:-1], edges[1:])]
    rows = B * Hq * n_q * (D + 2)
    parts = torch.empty((sum(slots) * rows,), dtype=torch.float32, device="cuda")
    off = 0
    for (a, b), n in zip(zip(edges[:-1], edges[1:]), slots):
        vc.verify_attn_range(qd, full, ctx_t, max(ctx), Hkv, scale, a, b, parts[off * rows:])
        off += n
    got = vc.verify_merge(parts, sum(slots), B, Hq, n_q, D).cpu().numpy()
    g = Hq // Hkv
    for b in range(B):
        n = ctx[b] + n_q
        for h in range(Hkv):
            ref = O.verify_attention_unit(O.bf16_to_f64(qb[b, h * g:(h + 1) * g]), O.bf16_to_f64(kb[b, h, :n]),
                                          O.bf16_to_f64(vb[b, h, :n]), ctx[b], scale)
            assert_close(got[b, h * g:(h + 1) * g], ref, f"chunked ragged b{b} h{h}")


def _select_cases():
    rng = np.random.default_rng(51)
    pool = np.array([-np.inf, -2.5, -0.0, 0.0, 0.75, 3.0, np.inf], dtype=np.float32)
    cases = [("qwen_32b_rows_u01", rng.random((32, 131072), dtype=np.float32), 13107)]
    cases.append(("ties_signed_zero_inf", pool[rng.integers(0, len(pool), (6, 5000))], 1234))
    for L, M in ((1, 1), (37, 1), (37, 36), (1023, 500), (1025, 1024), (3000, 2999), (2048, 1)):
        cases.append((f"L{L}_M{M}", rng.standard_normal((3, L)).astype(np.float32).round(1), M))
    cases.append(("all_equal", np.full((2, 4100), 0.5, np.float32), 4000))
    cases.append(("M_eq_L", rng.random((2, 777), dtype=np.float32), 777))
    return cases


@pytest.mark.parametrize("name,scores,M", _select_cases(), ids=[c[0] for c in _select_cases()])
def test_select_top_m_bit_exact(name, scores, M):
    """The GPU top-M selector returns exactly the oracle's kept-index lists."""
    import time
    import torch
    vc = _vc()
    print(f"[case] select {name} rows={scores.shape[0]} L={scores.shape[1]} M={M}", flush=True)
    sd = torch.from_numpy(np.ascontiguousarray(scores)).to("cuda")
    got = vc.select_top_m(sd, M)
    torch.cuda.synchronize()
    if name.startswith("qwen"):
        t0 = time.perf_counter()
        for _ in range(5):
            vc.select_top_m(sd, M, keep_idx=got)
        torch.cuda.synchronize()
        print(f"[time] select {name}: {(time.perf_counter() - t0) / 5 * 1e6:.1f} us per call", flush=True)
    got = got.cpu().numpy()
    for r in range(scores.shape[0]):
        ref = O.select_top_m(scores[r], M)
        assert np.array_equal(got[r], ref), (name, r, np.flatnonzero(got[r] != ref)[:5])


@pytest.mark.parametrize("bits", [2, 4])
def test_draft_ragged_tail_lengths(bits):
    """Each sequence has its own exact-tail length (0 included): the rows past a
    sequence's len hold large values that must not be read."""
    import torch
    vc = _vc()
    from compressed_kv_draft_amd.workload import bf16_dev
    from synth.gen import f32_to_bf16_bits
    print(f"[case] draft ragged tail int{bits}", flush=True)
    rng = np.random.default_rng(12 + bits)
    B, Hq, Hkv, D, nq, T_cap = 3, 8, 2, 128, 256, 40
    lens = [0, 5, 33]
    k = rng.standard_normal((B, Hkv, nq, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, nq, D)).astype(np.float32)
    tk = rng.standard_normal((B, Hkv, T_cap, D)).astype(np.float32)
    tv = rng.standard_normal((B, Hkv, T_cap, D)).astype(np.float32)
    for b in range(B):
        tk[b, :, lens[b]:] = 40.0
        tv[b, :, lens[b]:] = 1000.0
    q = rng.standard_normal((B, Hq, D)).astype(np.float32)
    kb, vb, tkb, tvb, qb = (f32_to_bf16_bits(x) for x in (k, v, tk, tv, q))
    comp = vc.quantize_kv(bf16_dev(kb, "cuda"), bf16_dev(vb, "cuda"), bits, nq)
    lens_t = torch.tensor(lens, dtype=torch.int32, device="cuda")
    tail = vc.Tail(bf16_dev(tkb, "cuda"), bf16_dev(tvb, "cuda"), lens_t)
    scale = O.scale_for(D)
    got = vc.draft_attn(comp, tail, bf16_dev(qb, "cuda"), scale).cpu().numpy()
    g = Hq // Hkv
    for b in range(B):
        for h in range(Hkv):
            kf = O.bf16_to_f64(kb[b, h]).astype(np.float32)
            vf = O.bf16_to_f64(vb[b, h]).astype(np.float32)
            kd = O.dequant_k(*O.quantize_k(kf, bits))
            vd = O.dequant_v(*O.quantize_v(vf, bits))
            keys, vals = O.draft_kv_rows("quant", k_deq=kd, v_deq=vd,
                                         tail_k=O.bf16_to_f64(tkb[b, h, :lens[b]]),
                                         tail_v=O.bf16_to_f64(tvb[b, h, :lens[b]]))
            ref = O.draft_attention_unit(O.bf16_to_f64(qb[b, h * g:(h + 1) * g]), keys, vals, scale)
            assert_close(got[b, h * g:(h + 1) * g], ref, f"ragged tail int{bits} b{b} h{h}")


def _assert_lse(got, ref, what):
    """lse to the attention bar: finite rows within rel L2 1e-3 and max-abs
    5e-3 x max|ref| of the oracle's; rows with no key exactly -inf."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    empty = np.isneginf(ref)
    assert (np.isneginf(got) == empty).all(), (what, got, ref)
    if (~empty).any():
        assert_close(got[~empty], ref[~empty], what + " lse")


@pytest.mark.parametrize("kind", ["quant_splits", "quant_direct", "token_drop_none_kept", "identity_empty"])
def test_draft_lse_and_empty_key_sets(kind):
    """The optional lse output, on a call merged by the combine kernel
    (many splits) and on a single-split call written directly; and compressed
    parts that hold no row (no kept token, an empty identity cache) with tail
    lengths 0, 5 and 33: the tail-only sequences match the oracle, the sequence
    without any key gets o = 0 and lse = -inf."""
    import torch
    vc = _vc()
    from compressed_kv_draft_amd.workload import bf16_dev
    from synth.gen import f32_to_bf16_bits
    print(f"[case] draft lse / empty key sets: {kind}", flush=True)
    rng = np.random.default_rng({"quant_splits": 61, "quant_direct": 62}.get(kind, 63))
    B, Hq, Hkv, D, T_cap = 3, 8, 2, 128, 40
    g = Hq // Hkv
    nq = 16384 if kind == "quant_splits" else (64 if kind == "quant_direct" else 96)
    # quant_direct: two blocks and no tail, so one workgroup per (batch, kv-head) writes the output itself
    lens = {"quant_splits": [7, 0, 40], "quant_direct": [0, 0, 0]}.get(kind, [0, 5, 33])
    k = rng.standard_normal((B, Hkv, nq, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, nq, D)).astype(np.float32)
    tk = rng.standard_normal((B, Hkv, T_cap, D)).astype(np.float32)
    tv = rng.standard_normal((B, Hkv, T_cap, D)).astype(np.float32)
    q = rng.standard_normal((B, Hq, D)).astype(np.float32)
    kb, vb, tkb, tvb, qb = (f32_to_bf16_bits(x) for x in (k, v, tk, tv, q))
    kd_, vd_ = bf16_dev(kb, "cuda"), bf16_dev(vb, "cuda")
    if kind.startswith("quant"):
        comp = vc.quantize_kv(kd_, vd_, 4, nq)
    elif kind == "token_drop_none_kept":
        comp = vc.token_drop_cache(kd_, vd_, torch.empty((B, Hkv, 0), dtype=torch.int32, device="cuda"))
    else:
        comp = vc.identity_cache(kd_, vd_, 0)
    tail = vc.Tail() if kind == "quant_direct" else vc.Tail(
        bf16_dev(tkb, "cuda"), bf16_dev(tvb, "cuda"), torch.tensor(lens, dtype=torch.int32, device="cuda"))
    scale = O.scale_for(D)
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    got = vc.draft_attn(comp, tail, bf16_dev(qb, "cuda"), scale, lse=lse).cpu().numpy()
    got_lse = lse.cpu().numpy()
    for b in range(B):
        for h in range(Hkv):
            qh = O.bf16_to_f64(qb[b, h * g:(h + 1) * g])
            tail_k, tail_v = O.bf16_to_f64(tkb[b, h, :lens[b]]), O.bf16_to_f64(tvb[b, h, :lens[b]])
            if kind.startswith("quant"):
                kf = O.bf16_to_f64(kb[b, h]).astype(np.float32)
                vf = O.bf16_to_f64(vb[b, h]).astype(np.float32)
                keys, vals = O.draft_kv_rows("quant", k_deq=O.dequant_k(*O.quantize_k(kf, 4)),
                                             v_deq=O.dequant_v(*O.quantize_v(vf, 4)), tail_k=tail_k, tail_v=tail_v)
            elif kind == "token_drop_none_kept":
                keys, vals = O.draft_kv_rows("token_drop", k_full=O.bf16_to_f64(kb[b, h]),
                                             v_full=O.bf16_to_f64(vb[b, h]), keep_idx=np.zeros(0, np.int64),
                                             tail_k=tail_k, tail_v=tail_v)
            else:
                keys, vals = O.draft_kv_rows("identity", k_full=O.bf16_to_f64(kb[b, h]),
                                             v_full=O.bf16_to_f64(vb[b, h]), L=0, tail_k=tail_k, tail_v=tail_v)
            what = f"{kind} b{b} h{h} ({len(keys)} keys)"
            _assert_lse(got_lse[b, h * g:(h + 1) * g], O.draft_lse_unit(qh, keys, scale), what)
            if len(keys):
                assert_close(got[b, h * g:(h + 1) * g], O.draft_attention_unit(qh, keys, vals, scale), what)
            else:
                assert (got[b, h * g:(h + 1) * g] == 0).all(), what


def test_verify_future_rows_do_not_leak():
    """Perturbing rows after L + j leaves verify position j bitwise unchanged."""
    from compressed_kv_draft_amd.workload import DeviceWorkload
    w = C.TINY.with_(name="leak", B=1, Hq=8, Hkv=2, D=128, L=500, k=6, kind="identity", seed=51)
    dw = DeviceWorkload(w, with_vocab=False)
    base = dw.verify().clone()
    j = 2
    dw.full_k[:, :, w.L + j + 1:] += 3.0
    dw.full_v[:, :, w.L + j + 1:] -= 2.0
    pert = dw.verify()
    assert bool((pert[:, :, :j + 1] == base[:, :, :j + 1]).all())
    assert not bool((pert[:, :, j + 1:] == base[:, :, j + 1:]).all())


def test_accept_and_argmax():
    import torch
    vc = _vc()
    print("[case] accept", flush=True)
    rng = np.random.default_rng(9)
    for (B, k, V) in [(4, 8, 1000), (3, 32, 32000), (2, 0, 77), (5, 5, 13)]:
        logits = rng.standard_normal((B, k + 1, V)).astype(np.float32)
        y = np.array([[O.argmax_first(logits[b, j]) for j in range(k + 1)] for b in range(B)])
        d = y[:, :k].copy()
        for b in range(B):
            if k and b % 2 == 1:
                i = int(rng.integers(0, k))
                d[b, i] = (d[b, i] + 1) % V
        lt = torch.from_numpy(logits).cuda()
        dt = torch.from_numpy(d.astype(np.int32)).cuda()
        out, n = vc.accept(dt, lt)
        out, n = out.cpu().numpy(), n.cpu().numpy()
        for b in range(B):
            ro, rn = O.accept(d[b], y[b])
            assert n[b] == rn and list(out[b]) == list(ro), (B, k, V, b)
    # ties -> lowest index, V not a multiple of 4
    x = np.zeros((3, 10), np.float32)
    x[0, [3, 7]] = 5.0
    x[1, :] = -1.0
    x[2, 9] = 1.0
    ids = vc.argmax(torch.from_numpy(x).cuda()).cpu().numpy()
    assert list(ids) == [3, 0, 9]


def test_round_tiny_tokens_bit_exact():
    """Single-layer round at the tiny workload: query vectors are resampled until
    every top-1 margin exceeds the bound, then draft tokens, verify tokens,
    emitted ids and the accept length must equal the oracle's."""
    import torch
    vc = _vc()
    from compressed_kv_draft_amd.workload import DeviceWorkload
    for w in (C.TINY, C.TINY.with_(kind="identity", name="tiny_identity")):
        print(f"[case] round {w.name}", flush=True)
        K, V = I.context_kv(w, "k"), I.context_kv(w, "v")
        Kn, Vn = I.new_rows(w, "k"), I.new_rows(w, "v")
        W = I.vocab_matrix(w)
        attempts, Qb, r = R.plant_margins(w, 0, K[0], V[0], Kn[0], Vn[0], W)
        dw = DeviceWorkload(w, Q=Qb[None])
        for j in range(w.k):
            dw.draft_step(j)
        d_ids = vc.argmax(dw.draft_logits().contiguous()).reshape(w.B, w.k)
        dw.verify()
        out, n = vc.accept(d_ids, dw.verify_logits())
        torch.cuda.synchronize()
        assert list(d_ids.cpu().numpy()[0]) == list(r["draft_ids"])
        assert int(n.cpu().numpy()[0]) == r["n_accept"]
        assert list(out.cpu().numpy()[0]) == list(r["out_ids"])
        if w.kind == "identity":
            assert r["n_accept"] == w.k


def test_prefetch_pages_bit_exact():
    import torch
    vc = _vc()
    print("[case] prefetch", flush=True)
    page_bytes, slots, nseq, pps, pt = 4096, 64, 4, 16, 16
    rng = np.random.default_rng(3)
    table = rng.permutation(slots).astype(np.int32).reshape(nseq, pps)
    host = torch.from_numpy(rng.integers(0, 256, slots * page_bytes, dtype=np.uint8))
    staging = torch.empty(slots * page_bytes, dtype=torch.uint8, pin_memory=True)
    dev = torch.full((slots * page_bytes,), 7, dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    done = torch.cuda.Event()
    for (seqs, t0, t1) in [([1, 3], 40, 200), ([2], 0, 256), ([0, 1, 2, 3], 17, 18)]:
        vc.prefetch_full_kv(host, page_bytes, table, seqs, t0, t1, pt, staging, dev, stream=s, done_event=done)
        s.synchronize()
        want = O.prefetch_expected(host.numpy().reshape(slots, page_bytes), table, seqs, t0, t1, pt)
        got = dev.cpu().numpy()[:want.size].reshape(want.shape)
        assert np.array_equal(got, want), (seqs, t0, t1)
    # an unpinned staging buffer is rejected before any work
    with pytest.raises(vc.VcError):
        vc.prefetch_full_kv(host, page_bytes, table, [0], 0, 16, pt, torch.empty(page_bytes, dtype=torch.uint8),
                            dev, stream=s)


def test_prefetched_pages_feed_paged_verify():
    """Full-KV chunks of a shuffled host pool, prefetched chunk by chunk, then read
    through a device page table by the paged verify kernel: equals the oracle."""
    import torch
    vc = _vc()
    from compressed_kv_draft_amd.workload import bf16_dev, paged_pool
    print("[case] prefetch -> paged verify", flush=True)
    w = C.TINY.with_(name="pv", B=2, Hq=8, Hkv=2, D=64, L=512, k=7, kind="identity", paged=True, page_tokens=16,
                     chunk_tokens=128, seed=61)
    K, V = I.context_kv(w, "k"), I.context_kv(w, "v")
    Kn, Vn = I.new_rows(w, "k"), I.new_rows(w, "v")
    Q = I.queries(w)
    table, n_slots = I.page_table(w)
    pool = paged_pool(w, np.concatenate([K, Kn], 2), np.concatenate([V, Vn], 2), table, n_slots)
    page_bytes = pool[0].nbytes
    host = torch.from_numpy(pool.reshape(-1).view(np.uint8).copy())
    ctx_pages = w.L // w.page_tokens
    pps = table.shape[1]
    # device region: chunk c of all sequences, then the pages of the new rows
    per_chunk = w.chunk_tokens // w.page_tokens
    dev = torch.empty((w.B * pps + 1) * page_bytes, dtype=torch.uint8, device="cuda")
    dev_table = np.zeros_like(table)
    staging = [torch.empty(w.B * per_chunk * page_bytes, dtype=torch.uint8, pin_memory=True) for _ in range(2)]
    done = [torch.cuda.Event(), torch.cuda.Event()]
    s = torch.cuda.Stream()
    base = 0
    for c, t0 in enumerate(range(0, w.L, w.chunk_tokens)):
        seqs = list(range(w.B))
        vc.prefetch_full_kv(host, page_bytes, table, seqs, t0, t0 + w.chunk_tokens, w.page_tokens, staging[c % 2],
                            dev[base * page_bytes:], stream=s, done_event=done[c % 2],
                            staging_free=done[c % 2] if c >= 2 else None)
        for i, b in enumerate(seqs):
            dev_table[b, t0 // w.page_tokens:(t0 + w.chunk_tokens) // w.page_tokens] = \
                base + i * per_chunk + np.arange(per_chunk)
        base += w.B * per_chunk
    # the pages holding the drafted rows live only on the device
    for b in range(w.B):
        for p in range(ctx_pages, pps):
            dev[base * page_bytes:(base + 1) * page_bytes].copy_(
                torch.from_numpy(pool[table[b, p]].reshape(-1).view(np.uint8).copy()))
            dev_table[b, p] = base
            base += 1
    s.synchronize()
    torch.cuda.synchronize()
    pool_dev = dev.view(torch.bfloat16)
    tab_dev = torch.from_numpy(dev_table).cuda()
    full = vc.FullKV(pool_dev, None, 0, tab_dev, w.page_tokens, pps, base)
    ctx = torch.full((w.B,), w.L, dtype=torch.int32, device="cuda")
    got = vc.verify_attn(bf16_dev(Q, "cuda"), full, ctx, w.L, w.Hkv, O.scale_for(w.D)).cpu().numpy()
    g = w.g
    for b in range(w.B):
        for h in range(w.Hkv):
            ref = R.unit_verify(w, K[b, h], V[b, h], Kn[b, h], Vn[b, h], Q[b, h * g:(h + 1) * g])
            assert_close(got[b, h * g:(h + 1) * g], ref, f"prefetched paged verify b{b} h{h}")


def test_round_graph_replays_match_eager():
    """The round as the benchmark launches it, each phase (the k draft calls,
    verify, accept) recorded once as a HIP graph, gives bit-identical outputs
    to the eager calls on every replay, with eager work, scrambled outputs and
    synchronisation between the replays (nothing recorded may depend on state
    that only the first replay sees)."""
    import torch
    vc = _vc()
    from compressed_kv_draft_amd.workload import DeviceWorkload
    w = C.TINY.with_(name="graph_int2_d128_g4", B=2, Hq=8, Hkv=2, D=128, L=1056, k=5, bits=2, residual=32,
                     seed=71)
    print(f"[case] graph replay {w.name}", flush=True)
    dw = DeviceWorkload(w)
    for j in range(w.k):
        dw.draft_step(j)
    d_ids = vc.argmax(dw.draft_logits().contiguous()).reshape(w.B, w.k)
    dw.verify()
    vlog = dw.verify_logits()
    out_ids = torch.empty((w.B, w.n_q), dtype=torch.int32, device="cuda")
    n_acc = torch.empty(w.B, dtype=torch.int32, device="cuda")

    def drafts():
        for j in range(w.k):
            dw.draft_step(j)

    def accept():
        vc.accept(d_ids, vlog, out_ids=out_ids, n_accept=n_acc)

    phases = [drafts, dw.verify, accept]
    for ph in phases:
        ph()
    torch.cuda.synchronize()
    outs = [dw.draft_out, dw.verify_out, out_ids, n_acc]
    ref = [t.clone() for t in outs]
    graphs = []
    for ph in phases:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            ph()
        graphs.append(g)
    bits = lambda t: t.view(torch.int32) if t.dtype == torch.float32 else t  # noqa: E731
    for r in range(4):
        dw.draft_out.fill_(float("nan"))
        dw.verify_out.fill_(-1.0)
        out_ids.fill_(-7)
        n_acc.fill_(-7)
        dw.draft_step(1)          # eager work between replays
        torch.cuda.synchronize()
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("draft", "verify", "ids", "n_accept"), outs, ref):
            assert torch.equal(bits(got), bits(want)), (r, name)


def _random_cases(n=14, seed=2026):
    """Seeded draws over the parameters the kernels branch on: cache kind and
    bits, head dim, GQA group, unit count (so both grid mappings), context
    length (ragged against 32-token blocks and tiles), draft length and
    exact-window length."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        kind = ["quant2", "quant4", "token_drop", "identity"][i % 4]
        D = int(rng.choice([64, 128]))
        g = int(rng.choice([1, 2, 4, 8]))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        B = int(rng.integers(1, 5))
        L = int(rng.integers(40, 2600))
        k = int(rng.integers(1, 7))
        kw = dict(name=f"rand{i}_{kind}_d{D}_g{g}_b{B}x{Hkv}_l{L}_k{k}", B=B, Hq=g * Hkv, Hkv=Hkv, D=D, L=L, k=k,
                  seed=100 + i)
        if kind.startswith("quant"):
            R = L % 32 + 32 * int(rng.integers(0, 4))
            R = min(R, L)
            kw.update(kind="quant", bits=int(kind[-1]), residual=R)
        elif kind == "token_drop":
            kw.update(kind="token_drop", keep_frac=float(rng.uniform(0.05, 0.6)))
        else:
            kw.update(kind="identity")
        out.append(C.TINY.with_(**kw))
    return out


def _odd_group_cases():
    """GQA groups that are not powers of two (3, 5, 6, 7): the draft's replica
    count 8 // g leaves idle column slots, and at D = 128 with g >= 5 every
    lane carries two V channel groups."""
    out = []
    specs = [("quant2", 64, 3), ("quant4", 128, 3), ("token_drop", 128, 3), ("identity", 64, 5),
             ("quant2", 128, 5), ("quant4", 64, 6), ("quant2", 128, 6), ("token_drop", 64, 6),
             ("quant4", 128, 7), ("identity", 128, 7)]
    for i, (kind, D, g) in enumerate(specs):
        Hkv = 1 + i % 3
        L = 300 + 173 * i
        kw = dict(name=f"oddg{i}_{kind}_d{D}_g{g}_kv{Hkv}_l{L}", B=1 + i % 2, Hq=g * Hkv, Hkv=Hkv, D=D, L=L,
                  k=3, seed=300 + i)
        if kind.startswith("quant"):
            kw.update(kind="quant", bits=int(kind[-1]), residual=L % 32 + 32)
        elif kind == "token_drop":
            kw.update(kind="token_drop", keep_frac=0.25)
        else:
            kw.update(kind="identity")
        out.append(C.TINY.with_(**kw))
    return out


@pytest.mark.parametrize("w", _random_cases() + _odd_group_cases(), ids=lambda w: w.name)
def test_random_shapes_draft_and_verify(w):
    from compressed_kv_draft_amd.workload import DeviceWorkload
    print(f"[case] random {w.name}", flush=True)
    dw = DeviceWorkload(w, with_vocab=False)
    for j in range(w.k):
        dw.draft_step(j)
    got_d = dw.draft_out.cpu().numpy()
    got_v = dw.verify().cpu().numpy()
    g = w.g
    for b in range(w.B):
        for h in range(w.Hkv):
            keep = dw.keep_np[b, h] if w.kind == "token_drop" else None
            args = (dw.np["K"][b, h], dw.np["V"][b, h], dw.np["Kn"][b, h], dw.np["Vn"][b, h],
                    dw.np["Q"][b, h * g:(h + 1) * g])
            ref_d = R.unit_draft(w, *args, keep=keep)
            assert_close(got_d[:, b, h * g:(h + 1) * g].transpose(1, 0, 2), ref_d, f"{w.name} draft b{b} h{h}")
            ref_v = R.unit_verify(w, *args)
            assert_close(got_v[b, h * g:(h + 1) * g], ref_v, f"{w.name} verify b{b} h{h}")


def test_select_then_token_drop_draft():
    """The token-dropping compressor end to end on the GPU: importance scores
    -> vc_select_top_m -> a VC_KV_TOKEN_DROP cache -> vc_draft_attn, against
    the oracle's selection and its attention over the kept rows plus the tail.
    Ragged L and M, and scores with ties at the selection boundary."""
    import torch
    vc = _vc()
    from compressed_kv_draft_amd.workload import bf16_dev
    from synth.gen import f32_to_bf16_bits
    print("[case] select -> token-drop draft", flush=True)
    rng = np.random.default_rng(77)
    B, Hq, Hkv, D, L, M, T = 2, 16, 4, 128, 1517, 301, 9
    k = f32_to_bf16_bits(rng.standard_normal((B, Hkv, L, D)).astype(np.float32))
    v = f32_to_bf16_bits(rng.standard_normal((B, Hkv, L, D)).astype(np.float32))
    tk = f32_to_bf16_bits(rng.standard_normal((B, Hkv, T, D)).astype(np.float32))
    tv = f32_to_bf16_bits(rng.standard_normal((B, Hkv, T, D)).astype(np.float32))
    q = f32_to_bf16_bits(rng.standard_normal((B, Hq, D)).astype(np.float32))
    scores = rng.integers(0, 40, size=(B, Hkv, L)).astype(np.float32) / 8.0   # many ties
    keep = vc.select_top_m(torch.from_numpy(scores).cuda(), M)
    comp = vc.token_drop_cache(bf16_dev(k, "cuda"), bf16_dev(v, "cuda"), keep)
    tail = vc.Tail(bf16_dev(tk, "cuda"), bf16_dev(tv, "cuda"), torch.full((B,), T, dtype=torch.int32, device="cuda"))
    scale = O.scale_for(D)
    got = vc.draft_attn(comp, tail, bf16_dev(q, "cuda"), scale).cpu().numpy()
    keep_np = keep.cpu().numpy()
    g = Hq // Hkv
    for b in range(B):
        for h in range(Hkv):
            want_idx = O.select_top_m(scores[b, h], M)
            assert np.array_equal(keep_np[b, h], want_idx), (b, h)
            keys, vals = O.draft_kv_rows("token_drop", k_full=O.bf16_to_f64(k[b, h]), v_full=O.bf16_to_f64(v[b, h]),
                                         keep_idx=want_idx, tail_k=O.bf16_to_f64(tk[b, h]),
                                         tail_v=O.bf16_to_f64(tv[b, h]))
            ref = O.draft_attention_unit(O.bf16_to_f64(q[b, h * g:(h + 1) * g]), keys, vals, scale)
            assert_close(got[b, h * g:(h + 1) * g], ref, f"select+drop b{b} h{h}")


def _grid_values(rng, n, s, z, bits):
    """n x 32 values z + c s on a quantisation grid (each group of 32 holds codes 0
    and 2^bits - 1, so the group's scale and zero are exactly s and z)."""
    qmax = (1 << bits) - 1
    c = rng.integers(0, qmax + 1, (n, 32))
    c[:, 0], c[:, 1] = 0, qmax
    return (z + c * s).astype(np.float32)


@pytest.mark.parametrize("bits", [2, 4])
def test_draft_at_the_documented_range_limits(bits):
    """The draft carries q * s_K and p * s_V as f16 products; the header bounds them
    by |q| s_K < 4096 and s_V * 256 < 65504.  Inputs just inside both bounds:
    channel 5 of K is an exact grid of scale 240 and head 1's query holds 16 there
    (|q| s_K = 3840); channel group 0 of V is an exact grid of scale 240 and zero
    -1792 (s_V * 256 = 61440).  Every grid value is exact in bf16 and the scales
    and zeros in f16, so the quantiser reproduces them.  The result still
    matches the oracle."""
    import torch
    vc = _vc()
    from compressed_kv_draft_amd.workload import bf16_dev
    from synth.gen import f32_to_bf16_bits
    print(f"[case] draft at the range limits, int{bits}", flush=True)
    rng = np.random.default_rng(500 + bits)
    B, Hq, Hkv, D, n, T = 1, 4, 1, 128, 256, 8
    k = rng.standard_normal((B, Hkv, n + T, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, n + T, D)).astype(np.float32)
    k[0, 0, :n, 5] = _grid_values(rng, n // 32, 240.0, 0.0, bits).reshape(-1)   # K groups: 32 tokens of a channel
    v[0, 0, :n, :32] = _grid_values(rng, n, 240.0, -1792.0, bits)               # V groups: 32 channels of a token
    q = rng.standard_normal((B, Hq, D)).astype(np.float32) * 2.0
    q[0, 1, 5] = 16.0
    kb, vb, qb = (f32_to_bf16_bits(x) for x in (k, v, q))
    comp = vc.quantize_kv(bf16_dev(kb, "cuda"), bf16_dev(vb, "cuda"), bits, n)
    # the grid survived quantisation: the scales are exactly 250
    km = vc.unpack_quant(comp, B, Hkv, D)[2].cpu().numpy()
    vm = vc.unpack_quant(comp, B, Hkv, D)[3].cpu().numpy()
    assert (km[0, 0, :, 5, 0] == 240.0).all() and (vm[0, 0, :, 0, 0] == 240.0).all()
    tail = vc.Tail(bf16_dev(np.ascontiguousarray(kb[:, :, n:]), "cuda"), bf16_dev(np.ascontiguousarray(vb[:, :, n:]), "cuda"),
                   torch.full((B,), T, dtype=torch.int32, device="cuda"))
    scale = O.scale_for(D)
    got = vc.draft_attn(comp, tail, bf16_dev(qb, "cuda"), scale).cpu().numpy()
    kf = O.bf16_to_f64(kb[0, 0, :n]).astype(np.float32)
    vf = O.bf16_to_f64(vb[0, 0, :n]).astype(np.float32)
    keys, vals = O.draft_kv_rows("quant", k_deq=O.dequant_k(*O.quantize_k(kf, bits)),
                                 v_deq=O.dequant_v(*O.quantize_v(vf, bits)),
                                 tail_k=O.bf16_to_f64(kb[0, 0, n:]), tail_v=O.bf16_to_f64(vb[0, 0, n:]))
    want = O.draft_attention_unit(O.bf16_to_f64(qb[0]), keys, vals, scale)
    assert_close(got[0], want, f"range limits int{bits}")


def test_verify_at_the_value_range_limit():
    """Verify converts V from bf16 to f16 for the P.V product; the header bounds
    |v| < 65504.  Rows of +-59904 (the bf16 value nearest 60000 below it) among
    N(0,1) rows still match the oracle."""
    import torch
    vc = _vc()
    from compressed_kv_draft_amd.workload import bf16_dev
    from synth.gen import f32_to_bf16_bits
    print("[case] verify at the value range limit", flush=True)
    rng = np.random.default_rng(510)
    B, Hq, Hkv, D, L, n_q = 2, 8, 2, 128, 300, 5
    k = rng.standard_normal((B, Hkv, L + n_q, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, L + n_q, D)).astype(np.float32)
    v[:, :, ::7, ::3] = 59904.0 * np.sign(rng.standard_normal((B, Hkv, (L + n_q + 6) // 7, (D + 2) // 3)))
    q = rng.standard_normal((B, Hq, n_q, D)).astype(np.float32)
    kb, vb, qb = (f32_to_bf16_bits(x) for x in (k, v, q))
    assert (O.bf16_to_f64(vb).max() == 59904.0)
    full = vc.FullKV(bf16_dev(kb, "cuda"), bf16_dev(vb, "cuda"), L_cap=L + n_q)
    ctx = torch.full((B,), L, dtype=torch.int32, device="cuda")
    scale = O.scale_for(D)
    got = vc.verify_attn(bf16_dev(qb, "cuda"), full, ctx, L, Hkv, scale).cpu().numpy()
    g = Hq // Hkv
    for b in range(B):
        for h in range(Hkv):
            want = O.verify_attention_unit(O.bf16_to_f64(qb[b, h * g:(h + 1) * g]), O.bf16_to_f64(kb[b, h]),
                                           O.bf16_to_f64(vb[b, h]), L, scale)
            assert_close(got[b, h * g:(h + 1) * g], want, f"verify |v| limit b{b} h{h}")
