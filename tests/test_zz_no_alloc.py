"""vc_draft_attn_noalloc (the draft for callers that cannot allocate) against
vc_draft_attn through the C ABI: identical outputs on two calls in a row, the
second with a smaller input, both within the oracle's tolerance; and a call
whose split partials would not fit the scratch array is refused before
anything is enqueued."""
import ctypes

import numpy as np
import pytest

import oracle.vc_oracle as O
from oracle import round as R
from synth import configs as C

pytestmark = pytest.mark.gpu

REL_L2 = 1e-3
MAX_ABS = 5e-3

CASES = [
    # several splits per (batch, kv-head), XCD-affine grid (units % 8 == 0), exact tail
    C.TINY.with_(name="noalloc_int2_d128_g4_u8", B=2, Hq=16, Hkv=4, D=128, L=4128, k=2, bits=2, residual=64,
                 seed=91),
    # then a smaller one: fewer units, other head dim and bits
    C.TINY.with_(name="noalloc_int4_d64_g2_u2", B=1, Hq=4, Hkv=2, D=64, L=600, k=2, bits=4, residual=24, seed=92),
]


def _close(got, ref, what):
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    mx = np.abs(got - ref).max() / np.abs(ref).max()
    print(f"[parity] {what}: rel_l2={rel:.3e} max_abs/max|ref|={mx:.3e}", flush=True)
    assert rel <= REL_L2 and mx <= MAX_ABS, (what, rel, mx)


def test_noalloc_draft_matches_workspace_draft_twice():
    import torch
    import compressed_kv_draft_amd as vc
    from compressed_kv_draft_amd.workload import DeviceWorkload
    for w in CASES:
        print(f"[case] no-alloc draft {w.name}", flush=True)
        dw = DeviceWorkload(w, with_vocab=False)
        g = w.g
        for j in range(w.k):
            want = dw.draft_step(j).clone()
            out = torch.full_like(want, float("nan"))
            vc.draft_attn_noalloc(dw.comp, dw.tails[j], dw.q_steps[j], dw.scale, out, Hkv=w.Hkv)
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int32), want.view(torch.int32)), (w.name, j, "differs from vc_draft_attn")
            got = out.cpu().numpy()
            for b in range(w.B):
                for h in range(w.Hkv):
                    ref = R.unit_draft(w, dw.np["K"][b, h], dw.np["V"][b, h], dw.np["Kn"][b, h], dw.np["Vn"][b, h],
                                       dw.np["Q"][b, h * g:(h + 1) * g])      # [g, k, D]
                    _close(got[b, h * g:(h + 1) * g].astype(np.float64), ref[:, j], f"{w.name} step {j} b{b} h{h}")


def test_noalloc_draft_refuses_partials_beyond_scratch():
    """A 32k-row exact tail over 4 x 64 query heads asks for more split partials
    (256 splits x 256 rows x 130 floats) than the scratch array holds: the
    call fails with VC_ERR_UNSUPPORTED and leaves the output alone.  Every
    buffer is real and in bounds, so even a launch would be harmless."""
    import torch
    import compressed_kv_draft_amd as vc
    B, Hq, Hkv, D, T = 4, 64, 8, 128, 32768
    print(f"[case] no-alloc draft over the scratch limit: T={T}", flush=True)
    dev = "cuda"
    tk = torch.zeros((B, Hkv, T, D), dtype=torch.bfloat16, device=dev)
    tv = torch.zeros_like(tk)
    tail = vc.Tail(tk, tv, torch.full((B,), T, dtype=torch.int32, device=dev))
    ident = vc.identity_cache(tk, tv, 0)
    q = torch.zeros((B, Hq, D), dtype=torch.bfloat16, device=dev)
    need = vc.draft_ws_bytes(B, Hq, Hkv, D, T)
    assert need > 16 << 20, need
    out = torch.full((B, Hq, D), 7.0, dtype=torch.float32, device=dev)
    rc = vc.LIB.vc_draft_attn_noalloc(ctypes.byref(ident.desc), ctypes.byref(tail.desc), vc._lib._ptr(q),
                                      vc._lib._ptr(out), None, B, Hq, Hkv, D, ctypes.c_float(O.scale_for(D)),
                                      vc._lib._stream())
    torch.cuda.synchronize()
    msg = vc.LIB.vc_last_error().decode()
    print(f"[result] rc={rc} msg={msg}", flush=True)
    assert rc == -2 and "scratch" in msg, (rc, msg)
    assert bool((out == 7.0).all())
