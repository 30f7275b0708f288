"""One draft-then-verify round of a single-layer workload, in fp64 (test infrastructure only).

[VC Core Algorithm] draft k tokens with KV_comp, verify them in one pass with
KV_full, accept the matching prefix plus one verifier token.  In a single-layer
workload every draft position j has its own synthetic query vectors; position j
of the draft attends to the compressed context plus the exact tail (recent
window + new rows 0..j), and verify position j attends to the full context plus
new rows 0..j.  Logits are concat(head outputs) @ W; tokens are greedy.
"""
from __future__ import annotations

import numpy as np

from synth import inputs as I
from synth.configs import Workload

from . import vc_oracle as O


def unit_compressed(w: Workload, k_bits: np.ndarray, v_bits: np.ndarray):
    """Dequantised K'/V' rows [n_quant, D] of one unit (quant kind) plus the raw
    codes and meta, in the canonical (unpacked) layout."""
    nq = w.n_quant
    kf = O.bf16_to_f64(k_bits[:nq]).astype(np.float32)
    vf = O.bf16_to_f64(v_bits[:nq]).astype(np.float32)
    kc, ks, kz = O.quantize_k(kf, w.bits)
    vc, vs, vz = O.quantize_v(vf, w.bits)
    return dict(k_codes=kc, k_s=ks, k_z=kz, v_codes=vc, v_s=vs, v_z=vz,
                k_deq=O.dequant_k(kc, ks, kz), v_deq=O.dequant_v(vc, vs, vz))


def unit_draft(w: Workload, k_bits, v_bits, knew_bits, vnew_bits, q_bits, keep=None, comp=None,
               positions=None):
    """Draft outputs [g, k, D] of one (batch, kv-head); q_bits [g, n_q, D]."""
    scale = O.scale_for(w.D)
    kf = O.bf16_to_f64(k_bits)
    vf = O.bf16_to_f64(v_bits)
    kn = O.bf16_to_f64(knew_bits)
    vn = O.bf16_to_f64(vnew_bits)
    q = O.bf16_to_f64(q_bits)
    if w.kind == "quant" and comp is None:
        comp = unit_compressed(w, k_bits, v_bits)
    pos = range(w.k) if positions is None else positions
    out = np.zeros((q.shape[0], w.k, w.D))
    for j in pos:
        if w.kind == "quant":
            tail_k = np.concatenate([kf[w.n_quant:w.L], kn[:j + 1]])
            tail_v = np.concatenate([vf[w.n_quant:w.L], vn[:j + 1]])
            kc, vc = O.draft_kv_rows("quant", k_deq=comp["k_deq"], v_deq=comp["v_deq"],
                                     tail_k=tail_k, tail_v=tail_v)
        elif w.kind == "token_drop":
            kc, vc = O.draft_kv_rows("token_drop", k_full=kf, v_full=vf, keep_idx=keep,
                                     tail_k=kn[:j + 1], tail_v=vn[:j + 1])
        else:
            kc, vc = O.draft_kv_rows("identity", k_full=kf, v_full=vf, L=w.L,
                                     tail_k=kn[:j + 1], tail_v=vn[:j + 1])
        out[:, j, :] = O.draft_attention_unit(q[:, j, :], kc, vc, scale)
    return out


def unit_verify(w: Workload, k_bits, v_bits, knew_bits, vnew_bits, q_bits):
    """Verify outputs [g, n_q, D] of one (batch, kv-head)."""
    scale = O.scale_for(w.D)
    k_all = np.concatenate([O.bf16_to_f64(k_bits[:w.L]), O.bf16_to_f64(knew_bits)])
    v_all = np.concatenate([O.bf16_to_f64(v_bits[:w.L]), O.bf16_to_f64(vnew_bits)])
    return O.verify_attention_unit(O.bf16_to_f64(q_bits), k_all, v_all, w.L, scale)


def sequence_round(w: Workload, b: int, K, V, Knew, Vnew, Q, W, keep=None, comps=None):
    """Oracle round for sequence b.  K/V: [Hkv, L, D] bits of that sequence (or a
    callable h -> [L, D]); Q [Hq, n_q, D] bits.  Returns a dict with draft and
    verify outputs [Hq, *, D], logits, tokens, margins and the accept result."""
    g = w.g
    od = np.zeros((w.Hq, w.k, w.D))
    ov = np.zeros((w.Hq, w.n_q, w.D))
    for h in range(w.Hkv):
        kb = K(h) if callable(K) else K[h]
        vb = V(h) if callable(V) else V[h]
        qh = Q[h * g:(h + 1) * g]
        comp = None if comps is None else comps[h]
        od[h * g:(h + 1) * g] = unit_draft(w, kb, vb, Knew[h], Vnew[h], qh,
                                           keep=None if keep is None else keep[h], comp=comp)
        ov[h * g:(h + 1) * g] = unit_verify(w, kb, vb, Knew[h], Vnew[h], qh)
    dl = np.stack([O.logits(od[:, j], W) for j in range(w.k)])
    vl = np.stack([O.logits(ov[:, j], W) for j in range(w.n_q)])
    d_ids = np.array([O.argmax_first(x) for x in dl], dtype=np.int64)
    y_ids = np.array([O.argmax_first(x) for x in vl], dtype=np.int64)
    out, n = O.accept(d_ids, y_ids)
    return dict(draft_out=od, verify_out=ov, draft_logits=dl, verify_logits=vl,
                draft_ids=d_ids, verify_ids=y_ids, out_ids=out, n_accept=n)


def margin_bound(o_flat: np.ndarray, logit_row: np.ndarray, wcol_max: float, eps: float) -> float:
    """Smallest top-1 margin that an output error of relative size eps cannot flip:
    2 * eps * |o| * max_v |W[:, v]| (Cauchy-Schwarz) plus slack for the GEMM."""
    return 2.0 * eps * float(np.linalg.norm(o_flat)) * wcol_max + 1e-6 * float(np.abs(logit_row).max())


def plant_margins(w: Workload, b: int, K, V, Knew, Vnew, W, eps: float = 1e-3, max_attempts: int = 64,
                  keep=None, comps=None):
    """Resample the query vectors of every position of sequence b whose draft or
    verify top-1 margin is below the bound, from the next substream attempt.
    Returns (attempts [n_q] int, final Q bits [Hq, n_q, D], round dict)."""
    wcol = float(np.sqrt((W.astype(np.float64) ** 2).sum(axis=0)).max())
    attempts = np.zeros(w.n_q, dtype=np.int64)
    Q = np.stack([I.query_position(w, b, j, 0) for j in range(w.n_q)], axis=1)
    for _ in range(max_attempts):
        r = sequence_round(w, b, K, V, Knew, Vnew, Q, W, keep=keep, comps=comps)
        bad = []
        for j in range(w.n_q):
            ok = True
            if j < w.k:
                dl = r["draft_logits"][j]
                ok &= O.top2_margin(dl) > margin_bound(r["draft_out"][:, j].ravel(), dl, wcol, eps)
            vl = r["verify_logits"][j]
            ok &= O.top2_margin(vl) > margin_bound(r["verify_out"][:, j].ravel(), vl, wcol, eps)
            if not ok:
                bad.append(j)
        if not bad:
            return attempts, Q, r
        for j in bad:
            attempts[j] += 1
            Q[:, j, :] = I.query_position(w, b, j, int(attempts[j]))
    raise RuntimeError(f"margins not reached for sequence {b} after {max_attempts} attempts")
