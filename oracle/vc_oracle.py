"""fp64 reference of the draft-then-verify attention hot path (test infrastructure only).

Notation: B batch, Hq query heads, Hkv KV heads, g = Hq / Hkv, D head dim,
L context length, k draft length, n_q = k + 1 verify positions.

Format of the lossy cache (the KIVI-style compressor the VeriCache page names
under "Architecture Support"; the pages give no formula, so the reading is the
plain asymmetric min/max group quantiser written out in ``quantize_groups``):
  * K: groups of 32 consecutive tokens per channel; V: groups of 32 consecutive
    channels per token;
  * per group an fp16 scale s and fp16 zero z; codes are unsigned b-bit ints.
"""
from __future__ import annotations

import math

import numpy as np

GROUP = 32

# ----------------------------------------------------------------------------
# number formats (exact conversions; no rounding happens here)
# ----------------------------------------------------------------------------


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (exact: a bf16 is the top half of an fp32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f16_to_f64(h: np.ndarray) -> np.ndarray:
    return np.asarray(h, dtype=np.float16).astype(np.float64)


def f64_to_f32_rn(x: np.ndarray) -> np.ndarray:
    """Round float64 to the nearest float32 (ties to even), returned as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# quantisation  [VC Problem Statement: "quantization" as a lossy KV compressor;
#                VC Architecture Support: KIVI named behind the uniform interface]
# ----------------------------------------------------------------------------


def quantize_groups(x_f32: np.ndarray, bits: int):
    """Asymmetric min/max quantisation of groups laid along the last axis.

    Reading (the pages name quantisation but give no formula), in IEEE fp32 with
    round-to-nearest-even at every step:
      mn, mx = min, max of the group (exact)
      s32 = (mx - mn) / (2^bits - 1)          fp32 subtract, fp32 divide
      s = fp16(s32), z = fp16(mn)              round to nearest even
      code = 0                                  if s == 0
      code = clamp(rint((x - z) / s), 0, 2^bits - 1)  otherwise (fp32 ops,
                                                 rint = half-to-even)
    The clamp is needed because rounding s and z to fp16 can move a value just
    outside [z, z + (2^bits - 1) s].
    Returns (codes uint8 [..., G], s float16 [...], z float16 [...]).
    """
    x = np.asarray(x_f32, dtype=np.float32)
    qmax = np.float32((1 << bits) - 1)
    mn = x.min(axis=-1)
    mx = x.max(axis=-1)
    s32 = (mx - mn) / qmax                       # float32 ops
    s = s32.astype(np.float16)
    z = mn.astype(np.float16)
    s_b = s.astype(np.float32)[..., None]
    z_b = z.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (x - z_b) / s_b                      # float32 ops
    q = np.rint(t)
    q = np.where(s_b == 0, np.float32(0), q)
    q = np.clip(q, 0, qmax)
    return q.astype(np.uint8), s, z


def quantize_k(k_f32: np.ndarray, bits: int):
    """K [n, D] (n % 32 == 0): groups of 32 tokens per channel.
    Returns codes [n, D] uint8, s [n/32, D] fp16, z [n/32, D] fp16."""
    n, D = k_f32.shape
    assert n % GROUP == 0
    grp = k_f32.reshape(n // GROUP, GROUP, D).transpose(0, 2, 1)   # [n/32, D, 32]
    codes, s, z = quantize_groups(grp, bits)
    return codes.transpose(0, 2, 1).reshape(n, D), s, z


def quantize_v(v_f32: np.ndarray, bits: int):
    """V [n, D] (D % 32 == 0): groups of 32 channels per token.
    Returns codes [n, D] uint8, s [n, D/32] fp16, z [n, D/32] fp16."""
    n, D = v_f32.shape
    grp = v_f32.reshape(n, D // GROUP, GROUP)
    codes, s, z = quantize_groups(grp, bits)
    return codes.reshape(n, D), s, z


def dequant_k(codes: np.ndarray, s: np.ndarray, z: np.ndarray) -> np.ndarray:
    """x' = fp32(code * s + z): the product and sum are exact in fp64 (a <=4-bit
    integer times an fp16, plus an fp16), then rounded once to fp32."""
    n, D = codes.shape
    sf = np.repeat(f16_to_f64(s), GROUP, axis=0)
    zf = np.repeat(f16_to_f64(z), GROUP, axis=0)
    return f64_to_f32_rn(codes.astype(np.float64) * sf + zf)


def dequant_v(codes: np.ndarray, s: np.ndarray, z: np.ndarray) -> np.ndarray:
    """x' = fp32(code * s + z) with s, z the fp16 pair of the value's group: 32
    consecutive channels of its own token (codes [n, D], s and z [n, D/32]).
    Exact in fp64, rounded once to fp32, as for K."""
    n, D = codes.shape
    sf = np.repeat(f16_to_f64(s), GROUP, axis=1)
    zf = np.repeat(f16_to_f64(z), GROUP, axis=1)
    return f64_to_f32_rn(codes.astype(np.float64) * sf + zf)


def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Pack codes [n, D] along D into bytes [n, D*bits/8]: 4-bit codes put element
    2i in the low nibble of byte i and 2i+1 in the high nibble; 2-bit codes put
    element i at bit 2*(i mod 4) of byte i // 4."""
    n, D = codes.shape
    per = 8 // bits
    c = codes.astype(np.uint16).reshape(n, D // per, per)
    out = np.zeros((n, D // per), dtype=np.uint16)
    for i in range(per):
        out |= c[:, :, i] << np.uint16(bits * i)
    return out.astype(np.uint8)


# ----------------------------------------------------------------------------
# attention  [VC Core Algorithm: drafting with KV_comp, verification with KV_full]
# ----------------------------------------------------------------------------


def softmax_attention(q: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float) -> np.ndarray:
    """Scaled dot-product softmax attention of query rows q [m, D] over keys/values
    [n, D] (reading: the plain definition; the pages name attention only)."""
    s = (q @ keys.T) * scale                     # [m, n]
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ values


def draft_kv_rows(kind: str, *, k_full=None, v_full=None, L=None, keep_idx=None,
                  k_deq=None, v_deq=None, tail_k=None, tail_v=None):
    """Key/value rows one draft step of one (batch, kv-head) attends to.

    [VC Core Algorithm] the draft reads the compressed cache KV_comp; [VC
    Architecture Support] the uniform compressor interface admits token
    dropping and quantisation.  Reading: the draft step also attends to the
    exact (bf16) tail rows it holds: the recent-window rows kept uncompressed
    and the rows of this round's already drafted positions including its own.
      'identity'   : all L context rows of the full cache
      'token_drop' : context rows keep_idx (sorted, unique) of the full cache
      'quant'      : the dequantised rows (k_deq / v_deq)
    then the tail rows, in order."""
    if kind == "identity":
        kc, vc = k_full[:L], v_full[:L]
    elif kind == "token_drop":
        kc, vc = k_full[keep_idx], v_full[keep_idx]
    elif kind == "quant":
        kc, vc = k_deq, v_deq
    else:
        raise ValueError(kind)
    if tail_k is not None and len(tail_k):
        kc = np.concatenate([kc, tail_k], axis=0)
        vc = np.concatenate([vc, tail_v], axis=0)
    return kc, vc


def draft_attention_unit(q_heads: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float):
    """One decode step for the g query heads [g, D] sharing one KV head."""
    return softmax_attention(q_heads, keys, values, scale)


def draft_lse_unit(q_heads: np.ndarray, keys: np.ndarray, scale: float) -> np.ndarray:
    """Natural log of the softmax denominator of each query head [g, D] over keys
    [n, D]: ln sum_t exp(scale q . k_t) (the normaliser of the attention above,
    written out; -inf when there is no key).  Shifted by the row maximum before
    the exponentials, which leaves the value unchanged."""
    g = q_heads.shape[0]
    if keys.shape[0] == 0:
        return np.full(g, -np.inf)
    s = (q_heads @ keys.T) * scale              # [g, n]
    m = s.max(axis=1)
    return m + np.log(np.exp(s - m[:, None]).sum(axis=1))


def gqa_kv_head(h: int, Hq: int, Hkv: int) -> int:
    """Reading: query head h reads KV head floor(h * Hkv / Hq) (contiguous groups)."""
    return (h * Hkv) // Hq


def verify_attention_unit(q: np.ndarray, k_all: np.ndarray, v_all: np.ndarray, L: int, scale: float):
    """Causal verify attention for one (batch, kv-head).

    [VC Core Algorithm] verification is a single forward pass over KV_full that
    checks all drafted positions in parallel.  q [g, n_q, D]; k_all/v_all hold
    the L context rows followed by the n_q new rows.  Position j sees keys
    [0, L + j] (its own row and the rows of the earlier drafted positions).
    Written as one masked batch, a different code path from the decode step."""
    g, nq, D = q.shape
    n = L + nq
    s = np.matmul(q, k_all[:n].T) * scale                         # [g, n_q, n]
    tok = np.arange(n)[None, None, :]
    lim = (L + np.arange(nq))[None, :, None]
    s = np.where(tok <= lim, s, -np.inf)
    s = s - s.max(axis=2, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=2, keepdims=True)
    return np.matmul(p, v_all[:n])


# ----------------------------------------------------------------------------
# logits, argmax, acceptance  [VC Core Algorithm: acceptance up to the first
# mismatch, plus a bonus token when every draft matches; repeat from the last
# accepted token.  VC Experimental Results: output identical under greedy
# decoding]
# ----------------------------------------------------------------------------


def logits(o_heads: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Vocab logits of one position: the head outputs o [Hq, D] laid end to end
    head by head (head 0's D channels, then head 1's, ...), times W [Hq*D, V].
    Reading: the workloads define the logits as the concatenated head outputs
    times a vocabulary matrix; the pages give no formula."""
    return o_heads.reshape(-1) @ w


def argmax_first(x: np.ndarray) -> int:
    """Greedy token: index of the largest logit; ties go to the lowest index."""
    return int(np.argmax(x))


def top2_margin(x: np.ndarray) -> float:
    """Gap between the largest and second-largest logit."""
    part = np.partition(x, -2)
    return float(part[-1] - part[-2])


def accept(draft_ids: np.ndarray, verify_tokens: np.ndarray):
    """Greedy prefix acceptance for one sequence.

    draft_ids d_0..d_{k-1}; verify_tokens y_0..y_k (y_j = greedy token the full
    cache predicts after the pending token and drafts d_0..d_{j-1}).
    n = first j < k with d_j != y_j, else k.  Emitted: d_0..d_{n-1} then y_n
    (the bonus token when n == k; at a mismatch y_n replaces the rejected draft,
    which is the reading that lets the next round start from an exact token).
    Returns (emitted ids padded with -1 to length k+1, n)."""
    k = len(draft_ids)
    n = k
    for j in range(k):
        if int(draft_ids[j]) != int(verify_tokens[j]):
            n = j
            break
    out = np.full(k + 1, -1, dtype=np.int64)
    out[:n] = draft_ids[:n]
    out[n] = verify_tokens[n]
    return out, n


# ----------------------------------------------------------------------------
# token selection  [VC Problem Statement: token dropping keeps part of the
# context's tokens; VC Architecture Support: token-dropping compressors behind
# the uniform interface.  The pages describe no selection rule; the reading
# here keeps the M tokens of highest importance score per (batch, kv-head)]
# ----------------------------------------------------------------------------


def select_top_m(scores: np.ndarray, M: int) -> np.ndarray:
    """Indices of the M largest scores of one (batch, kv-head) row, ties broken
    toward the lower index, returned in ascending index order (the kept-row list
    the token-dropped draft gathers).  Scores compare as real numbers (-0 == +0);
    NaN is not allowed.  0 <= M <= len(scores)."""
    s = np.asarray(scores, dtype=np.float64)
    assert 0 <= M <= len(s) and not np.isnan(s).any()
    order = np.lexsort((np.arange(len(s)), -s))   # score descending, then index ascending
    return np.sort(order[:M]).astype(np.int32)


# ----------------------------------------------------------------------------
# full-KV prefetch  [VC Architecture Support, long-context decoding: compressed
# KV in HBM, full KV in CPU memory loaded over PCIe for verification; VC Key
# System Innovations P1: the load overlaps other requests' drafting]
# ----------------------------------------------------------------------------


def prefetch_expected(host_pool: np.ndarray, page_table: np.ndarray, seq_ids, tok_begin: int, tok_end: int,
                      page_tokens: int) -> np.ndarray:
    """Bytes the device receives for one prefetch: for every listed sequence in
    order, the pages holding tokens [tok_begin, tok_end), each taken from slot
    page_table[b, p] of the host pool [slots, page_bytes].  Returns
    [n_seq * n_pages, page_bytes]."""
    if tok_end <= tok_begin:
        return np.zeros((0, host_pool.shape[1]), dtype=host_pool.dtype)
    p0 = tok_begin // page_tokens
    p1 = (tok_end + page_tokens - 1) // page_tokens
    rows = [host_pool[int(page_table[b, p])] for b in seq_ids for p in range(p0, p1)]
    return np.stack(rows)


# ----------------------------------------------------------------------------
# whole-round reference for the single-layer workloads
# ----------------------------------------------------------------------------


def scale_for(D: int) -> float:
    """Attention scale 1/sqrt(D) as the fp32 value both sides receive."""
    return float(np.float32(1.0 / math.sqrt(D)))
