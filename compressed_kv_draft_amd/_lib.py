"""ctypes binding of libvc.so: argument marshalling only.

Every computation runs in the HIP kernels of the library; this module turns
torch tensors into device pointers and the current torch stream into a
hipStream_t.  If the library is missing the import fails loudly: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libvc.so")

VC_OK = 0
VC_KV_IDENTITY, VC_KV_QUANT, VC_KV_TOKEN_DROP = 0, 1, 2
KIND = {"identity": VC_KV_IDENTITY, "quant": VC_KV_QUANT, "token_drop": VC_KV_TOKEN_DROP}

c_int, c_float, c_size, c_void = ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p


class VcKvComp(ctypes.Structure):
    _fields_ = [("kind", c_int), ("bits", c_int), ("n_quant", c_int),
                ("k_codes", c_void), ("v_codes", c_void), ("k_meta", c_void), ("v_meta", c_void),
                ("k_full", c_void), ("v_full", c_void), ("L_full", c_int), ("L_cap", c_int),
                ("keep_idx", c_void), ("n_keep", c_int), ("q_cap", c_int)]


class VcTail(ctypes.Structure):
    _fields_ = [("k", c_void), ("v", c_void), ("len", c_void), ("T_cap", c_int)]


class VcKvFull(ctypes.Structure):
    _fields_ = [("k", c_void), ("v", c_void), ("L_cap", c_int), ("page_table", c_void),
                ("page_tokens", c_int), ("pages_per_seq", c_int), ("n_slots", c_int)]


EXPORTS = {
    # name: (restype, argtypes)
    "vc_version": (c_int, []),
    "vc_last_error": (ctypes.c_char_p, []),
    "vc_quantize_kv": (c_int, [c_void, c_void, c_int, c_int, c_int, c_int, ctypes.POINTER(VcKvComp), c_void]),
    "vc_quantize_blocks": (c_int, [c_void, c_void, c_int, c_int, c_int, c_int, c_int, c_int,
                                   ctypes.POINTER(VcKvComp), c_int, c_void]),
    "vc_pack_quant": (c_int, [c_void, c_void, c_void, c_void, c_int, c_int, c_int, c_int, ctypes.POINTER(VcKvComp),
                              c_int, c_void]),
    "vc_unpack_quant": (c_int, [ctypes.POINTER(VcKvComp), c_int, c_int, c_int, c_void, c_void, c_void, c_void,
                                c_void]),
    "vc_select_top_m": (c_int, [c_void, c_int, c_int, c_int, c_void, c_void]),
    "vc_sched_accept_rate": (ctypes.c_double, [ctypes.c_longlong, ctypes.c_longlong]),
    "vc_sched_expected_tokens": (ctypes.c_double, [ctypes.c_double, c_int]),
    "vc_sched_choose_k": (c_int, [ctypes.c_longlong, ctypes.c_longlong, ctypes.c_double, ctypes.c_double,
                                  ctypes.c_double, c_int, c_int]),
    "vc_debug_dequant": (c_int, [ctypes.POINTER(VcKvComp), c_int, c_int, c_int, c_int, c_int, c_int, c_void, c_void]),
    "vc_draft_ws_bytes": (c_size, [c_int, c_int, c_int, c_int, c_int]),
    "vc_draft_attn": (c_int, [ctypes.POINTER(VcKvComp), ctypes.POINTER(VcTail), c_void, c_void, c_void,
                              c_int, c_int, c_int, c_int, c_float, c_void, c_size, c_void]),
    "vc_draft_attn_noalloc": (c_int, [ctypes.POINTER(VcKvComp), ctypes.POINTER(VcTail), c_void, c_void, c_void,
                                      c_int, c_int, c_int, c_int, c_float, c_void]),
    "vc_verify_ws_bytes": (c_size, [c_int, c_int, c_int, c_int, c_int, c_int]),
    "vc_verify_attn": (c_int, [c_void, ctypes.POINTER(VcKvFull), c_void, c_int, c_int, c_void,
                               c_int, c_int, c_int, c_int, c_float, c_void, c_size, c_void]),
    "vc_verify_range_parts": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int, c_int]),
    "vc_verify_attn_range": (c_int, [c_void, ctypes.POINTER(VcKvFull), c_void, c_int, c_int, c_int, c_int, c_void,
                                     c_int, c_int, c_int, c_int, c_float, c_void]),
    "vc_verify_merge": (c_int, [c_void, c_int, c_int, c_int, c_int, c_int, c_void, c_void]),
    "vc_argmax": (c_int, [c_void, c_int, c_int, c_void, c_void]),
    "vc_accept": (c_int, [c_void, c_void, c_int, c_int, c_int, c_void, c_void, c_void]),
    "vc_prefetch_full_kv": (c_int, [c_void, c_size, c_int, c_void, c_int, c_int, c_void, c_int,
                                    c_int, c_int, c_int, c_void, c_size, c_void, c_void, c_void, c_void]),
}


class VcError(RuntimeError):
    pass


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libvc.so not built at {LIB_PATH}; run `python -m compressed_kv_draft_amd.build` "
                          "(no CPU fallback exists)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in EXPORTS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


LIB = _load()


def _check(rc: int, what: str):
    if rc != VC_OK:
        msg = LIB.vc_last_error().decode(errors="replace")
        raise VcError(f"{what} failed ({rc}): {msg}")


def _ptr(t):
    return None if t is None else c_void(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return c_void(s.cuda_stream)


def version() -> int:
    return LIB.vc_version()


# ------------------------------------------------------------------ compressor

class Compressed:
    """Device tensors of one compressed cache plus the C descriptor that points at them."""

    def __init__(self, kind: str, **t):
        self.kind = kind
        self.t = t
        d = VcKvComp()
        d.kind = KIND[kind]
        d.bits = int(t.get("bits", 0))
        d.n_quant = int(t.get("n_quant", 0))
        for f in ("k_codes", "v_codes", "k_meta", "v_meta", "k_full", "v_full", "keep_idx"):
            setattr(d, f, _ptr(t.get(f)).value if t.get(f) is not None else None)
        d.L_full = int(t.get("L_full", 0))
        d.L_cap = int(t.get("L_cap", 0))
        d.n_keep = int(t.get("n_keep", 0))
        d.q_cap = int(t.get("q_cap", 0))
        self.desc = d

    def set_n_quant(self, n: int):
        """Live quantised rows of a QUANT cache (after blocks were appended)."""
        cap = self.desc.q_cap or self.desc.n_quant
        if n % 32 or not 0 <= n <= cap:
            raise VcError(f"n_quant={n} must be a multiple of 32 in [0, {cap}]")
        self.t["n_quant"] = n
        self.desc.n_quant = n


def quantize_kv(k_src: torch.Tensor, v_src: torch.Tensor, bits: int, n_quant: int, stream=None,
                capacity: int | None = None) -> Compressed:
    """k_src/v_src: bf16 [B, Hkv, L_cap, D] on the device.  Returns the QUANT cache of
    rows [0, n_quant), in arrays that hold `capacity` rows (default n_quant) so that
    quantize_blocks can grow it."""
    B, Hkv, L_cap, D = k_src.shape
    dev = k_src.device
    rb = D * bits // 8
    cap = n_quant if capacity is None else int(capacity)
    if cap % 32 or cap < n_quant:
        raise VcError(f"capacity={cap} must be a multiple of 32 and >= n_quant={n_quant}")
    t = dict(bits=bits, n_quant=n_quant, q_cap=cap,
             k_codes=torch.empty((B, Hkv, cap, rb), dtype=torch.uint8, device=dev),
             v_codes=torch.empty((B, Hkv, cap, rb), dtype=torch.uint8, device=dev),
             k_meta=torch.empty((B, Hkv, cap // 32, 2, D), dtype=torch.float16, device=dev),
             v_meta=torch.empty((B, Hkv, cap // 32, D // 32, 32, 2), dtype=torch.float16, device=dev))
    comp = Compressed("quant", **t)
    rc = LIB.vc_quantize_kv(_ptr(k_src), _ptr(v_src), B, Hkv, L_cap, D, ctypes.byref(comp.desc), _stream(stream))
    _check(rc, "vc_quantize_kv")
    comp.t["src_keepalive"] = (k_src, v_src)
    return comp


def quantize_blocks(k_src: torch.Tensor, v_src: torch.Tensor, comp: Compressed, src_row0: int, n_blocks: int,
                    dst_block: int | None = None, stream=None) -> Compressed:
    """Quantise rows [src_row0, src_row0 + 32 n_blocks) of k_src/v_src (bf16 [B, Hkv, rows, D])
    into blocks [dst_block, dst_block + n_blocks) of comp.  dst_block None appends after
    the live rows and raises comp's n_quant by 32 n_blocks."""
    B, Hkv, rows, D = k_src.shape
    append = dst_block is None
    if append:
        dst_block = comp.desc.n_quant // 32
    rc = LIB.vc_quantize_blocks(_ptr(k_src), _ptr(v_src), B, Hkv, rows, D, int(src_row0), int(n_blocks),
                                ctypes.byref(comp.desc), int(dst_block), _stream(stream))
    _check(rc, "vc_quantize_blocks")
    if append:
        comp.set_n_quant(comp.desc.n_quant + 32 * n_blocks)
    return comp


def empty_quant(B: int, Hkv: int, D: int, bits: int, capacity: int, device) -> Compressed:
    """A QUANT cache (internal form) with room for `capacity` rows per (batch, kv-head)
    and no live rows yet; fill it with pack_quant, quantize_blocks or set_n_quant."""
    if capacity % 32 or capacity < 0:
        raise VcError(f"capacity={capacity} must be a non-negative multiple of 32")
    rb = D * bits // 8
    t = dict(bits=bits, n_quant=0, q_cap=capacity,
             k_codes=torch.empty((B, Hkv, capacity, rb), dtype=torch.uint8, device=device),
             v_codes=torch.empty((B, Hkv, capacity, rb), dtype=torch.uint8, device=device),
             k_meta=torch.empty((B, Hkv, capacity // 32, 2, D), dtype=torch.float16, device=device),
             v_meta=torch.empty((B, Hkv, capacity // 32, D // 32, 32, 2), dtype=torch.float16, device=device))
    return Compressed("quant", **t)


def pack_quant(k_codes: torch.Tensor, v_codes: torch.Tensor, k_meta: torch.Tensor, v_meta: torch.Tensor,
               comp: Compressed, dst_block: int | None = None, stream=None) -> Compressed:
    """Canonical QUANT arrays (device): k_codes/v_codes u8 [B, Hkv, n, D*bits/8],
    k_meta f16 [B, Hkv, n/32, D, 2] and v_meta f16 [B, Hkv, n, D/32, 2] ({scale, zero}
    pairs) into blocks [dst_block, dst_block + n/32) of comp.  dst_block None appends
    after the live rows and raises comp's n_quant by n."""
    B, Hkv, n, rb = k_codes.shape
    D = k_meta.shape[3]
    for t, dt in ((k_codes, torch.uint8), (v_codes, torch.uint8), (k_meta, torch.float16), (v_meta, torch.float16)):
        if t.dtype != dt or not t.is_contiguous():
            raise VcError("vc_pack_quant: canonical arrays must be contiguous u8 codes and f16 metadata")
    append = dst_block is None
    if append:
        dst_block = comp.desc.n_quant // 32
    rc = LIB.vc_pack_quant(_ptr(k_codes), _ptr(v_codes), _ptr(k_meta), _ptr(v_meta), B, Hkv, n, D,
                           ctypes.byref(comp.desc), int(dst_block), _stream(stream))
    _check(rc, "vc_pack_quant")
    if append:
        comp.set_n_quant(comp.desc.n_quant + n)
    return comp


def unpack_quant(comp: Compressed, B: int, Hkv: int, D: int, stream=None):
    """Live rows of a QUANT cache in canonical form: (k_codes, v_codes, k_meta, v_meta)
    with the shapes pack_quant takes."""
    n, bits = comp.desc.n_quant, comp.desc.bits
    dev = comp.t["k_codes"].device
    kc = torch.empty((B, Hkv, n, D * bits // 8), dtype=torch.uint8, device=dev)
    vcd = torch.empty_like(kc)
    km = torch.empty((B, Hkv, n // 32, D, 2), dtype=torch.float16, device=dev)
    vm = torch.empty((B, Hkv, n, D // 32, 2), dtype=torch.float16, device=dev)
    rc = LIB.vc_unpack_quant(ctypes.byref(comp.desc), B, Hkv, D, _ptr(kc), _ptr(vcd), _ptr(km), _ptr(vm),
                             _stream(stream))
    _check(rc, "vc_unpack_quant")
    return kc, vcd, km, vm


def identity_cache(k_full: torch.Tensor, v_full: torch.Tensor, L_full: int) -> Compressed:
    return Compressed("identity", k_full=k_full, v_full=v_full, L_full=L_full, L_cap=k_full.shape[2])


def token_drop_cache(k_full: torch.Tensor, v_full: torch.Tensor, keep_idx: torch.Tensor) -> Compressed:
    return Compressed("token_drop", k_full=k_full, v_full=v_full, keep_idx=keep_idx,
                      n_keep=keep_idx.shape[-1], L_full=k_full.shape[2], L_cap=k_full.shape[2])


def debug_dequant(comp: Compressed, B: int, Hkv: int, D: int, b: int, h: int, which: int, stream=None):
    n = comp.t["n_quant"]
    out = torch.empty((n, D), dtype=torch.float32, device=comp.t["k_codes"].device)
    rc = LIB.vc_debug_dequant(ctypes.byref(comp.desc), B, Hkv, D, b, h, which, _ptr(out), _stream(stream))
    _check(rc, "vc_debug_dequant")
    return out


# ------------------------------------------------------------------ attention

class Tail:
    def __init__(self, k=None, v=None, lens=None):
        self.k, self.v, self.lens = k, v, lens
        d = VcTail()
        if k is not None:
            d.k, d.v, d.len = k.data_ptr(), v.data_ptr(), lens.data_ptr()
            d.T_cap = k.shape[2]
        else:
            d.T_cap = 0
        self.desc = d


def select_top_m(scores: torch.Tensor, M: int, keep_idx=None, stream=None) -> torch.Tensor:
    """scores: fp32 [..., L] (one row per (batch, kv-head)).  Returns int32 [..., M]:
    the indices of the M largest scores of each row, ties to the lower index, ascending."""
    L = scores.shape[-1]
    rows = scores.numel() // L if L else 0
    if scores.dtype != torch.float32 or not scores.is_contiguous():
        raise VcError("vc_select_top_m: scores must be contiguous fp32")
    if keep_idx is None:
        keep_idx = torch.empty((*scores.shape[:-1], M), dtype=torch.int32, device=scores.device)
    _check(LIB.vc_select_top_m(_ptr(scores), rows, L, int(M), _ptr(keep_idx), _stream(stream)), "vc_select_top_m")
    return keep_idx


def sched_accept_rate(accepted: int, rejections: int) -> float:
    return float(LIB.vc_sched_accept_rate(int(accepted), int(rejections)))


def sched_expected_tokens(a: float, k: int) -> float:
    return float(LIB.vc_sched_expected_tokens(float(a), int(k)))


def sched_choose_k(accepted: int, rejections: int, t_draft: float, t_overlap: float, t_rest: float, k_min: int,
                   k_max: int) -> int:
    """Draft length of a group's next round (host policy; see include/vc.h)."""
    k = LIB.vc_sched_choose_k(int(accepted), int(rejections), float(t_draft), float(t_overlap), float(t_rest),
                              int(k_min), int(k_max))
    _check(k if k < 0 else 0, "vc_sched_choose_k")
    return int(k)


def draft_ws_bytes(B, Hq, Hkv, D, max_keys) -> int:
    return int(LIB.vc_draft_ws_bytes(B, Hq, Hkv, D, max_keys))


def draft_attn(comp: Compressed, tail: Tail, q: torch.Tensor, scale: float, out=None, lse=None, ws=None,
               Hkv: int | None = None, stream=None):
    """q: bf16 [B, Hq, D].  Returns fp32 [B, Hq, D]."""
    B, Hq, D = q.shape
    if Hkv is None:
        ref = comp.t.get("k_codes") if comp.kind == "quant" else comp.t.get("k_full")
        Hkv = ref.shape[1]
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if ws is None:
        n_main = comp.t.get("n_quant", 0) if comp.kind == "quant" else (
            comp.t.get("n_keep", 0) if comp.kind == "token_drop" else comp.t.get("L_full", 0))
        need = draft_ws_bytes(B, Hq, Hkv, D, n_main + tail.desc.T_cap)
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)  # every partial read is written by the call
    rc = LIB.vc_draft_attn(ctypes.byref(comp.desc), ctypes.byref(tail.desc), _ptr(q), _ptr(out), _ptr(lse),
                           B, Hq, Hkv, D, float(scale), _ptr(ws), ws.numel(), _stream(stream))
    _check(rc, "vc_draft_attn")
    return out


def draft_attn_noalloc(comp: Compressed, tail: Tail, q: torch.Tensor, scale: float, out: torch.Tensor,
                       lse=None, Hkv: int | None = None, stream=None):
    """vc_draft_attn_noalloc: like draft_attn, but the caller passes `out` and the split
    partials live in the library's per-GPU scratch array (nothing is allocated)."""
    B, Hq, D = q.shape
    if Hkv is None:
        ref = comp.t.get("k_codes") if comp.kind == "quant" else comp.t.get("k_full")
        Hkv = ref.shape[1]
    rc = LIB.vc_draft_attn_noalloc(ctypes.byref(comp.desc), ctypes.byref(tail.desc), _ptr(q), _ptr(out), _ptr(lse),
                                   B, Hq, Hkv, D, float(scale), _stream(stream))
    _check(rc, "vc_draft_attn_noalloc")
    return out


class FullKV:
    def __init__(self, k, v=None, L_cap=0, page_table=None, page_tokens=0, pages_per_seq=0, n_slots=0):
        self.k, self.v, self.page_table = k, v, page_table
        d = VcKvFull()
        d.k = k.data_ptr()
        d.v = v.data_ptr() if v is not None else None
        d.L_cap = int(L_cap)
        d.page_table = page_table.data_ptr() if page_table is not None else None
        d.page_tokens = int(page_tokens)
        d.pages_per_seq = int(pages_per_seq)
        d.n_slots = int(n_slots)
        self.desc = d


def verify_ws_bytes(B, Hq, Hkv, D, n_q, max_ctx) -> int:
    return int(LIB.vc_verify_ws_bytes(B, Hq, Hkv, D, n_q, max_ctx))


def verify_attn(q: torch.Tensor, kv: FullKV, ctx_len: torch.Tensor, max_ctx: int, Hkv: int, scale: float,
                out=None, ws=None, stream=None):
    """q: bf16 [B, Hq, n_q, D].  Returns fp32 [B, Hq, n_q, D]."""
    B, Hq, n_q, D = q.shape
    if out is None:
        out = torch.empty((B, Hq, n_q, D), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = torch.empty(verify_ws_bytes(B, Hq, Hkv, D, n_q, max_ctx), dtype=torch.uint8, device=q.device)
    rc = LIB.vc_verify_attn(_ptr(q), ctypes.byref(kv.desc), _ptr(ctx_len), int(max_ctx), n_q, _ptr(out),
                            B, Hq, Hkv, D, float(scale), _ptr(ws), ws.numel(), _stream(stream))
    _check(rc, "vc_verify_attn")
    return out


def verify_range_parts(B, Hq, Hkv, D, n_q, key_begin, key_end) -> int:
    """Partial slots one vc_verify_attn_range call over [key_begin, key_end) writes."""
    return int(LIB.vc_verify_range_parts(B, Hq, Hkv, D, n_q, key_begin, key_end))


def verify_attn_range(q: torch.Tensor, kv: FullKV, ctx_len: torch.Tensor, max_ctx: int, Hkv: int, scale: float,
                      key_begin: int, key_end: int, parts: torch.Tensor, stream=None) -> int:
    """Verify partials over keys [key_begin, key_end) into `parts` (fp32, at least
    verify_range_parts(...) * B*Hq*n_q*(D+2) elements, slots back to back).
    Returns the number of slots written."""
    B, Hq, n_q, D = q.shape
    n = verify_range_parts(B, Hq, Hkv, D, n_q, key_begin, key_end)
    if n <= 0 or parts.numel() < n * B * Hq * n_q * (D + 2) or parts.dtype != torch.float32:
        raise VcError(f"vc_verify_attn_range: parts too small or not fp32 ({parts.numel()} < {n} slots)")
    rc = LIB.vc_verify_attn_range(_ptr(q), ctypes.byref(kv.desc), _ptr(ctx_len), int(max_ctx), n_q, int(key_begin),
                                  int(key_end), _ptr(parts), B, Hq, Hkv, D, float(scale), _stream(stream))
    _check(rc, "vc_verify_attn_range")
    return n


def verify_merge(parts: torch.Tensor, n_parts: int, B: int, Hq: int, n_q: int, D: int, out=None, stream=None):
    """Merge n_parts consecutive verify partial slots into fp32 [B, Hq, n_q, D]."""
    if out is None:
        out = torch.empty((B, Hq, n_q, D), dtype=torch.float32, device=parts.device)
    if parts.numel() < n_parts * B * Hq * n_q * (D + 2):
        raise VcError("vc_verify_merge: parts holds fewer slots than n_parts")
    rc = LIB.vc_verify_merge(_ptr(parts), int(n_parts), B, Hq, n_q, D, _ptr(out), _stream(stream))
    _check(rc, "vc_verify_merge")
    return out


# ------------------------------------------------------------------ tokens

def argmax(logits: torch.Tensor, ids=None, stream=None):
    rows, V = logits.reshape(-1, logits.shape[-1]).shape
    if ids is None:
        ids = torch.empty(rows, dtype=torch.int32, device=logits.device)
    _check(LIB.vc_argmax(_ptr(logits), rows, V, _ptr(ids), _stream(stream)), "vc_argmax")
    return ids


def accept(draft_ids: torch.Tensor, verify_logits: torch.Tensor, out_ids=None, n_accept=None, stream=None):
    """draft_ids int32 [B, k]; verify_logits fp32 [B, k+1, V]."""
    B, k1, V = verify_logits.shape
    k = k1 - 1
    if out_ids is None:
        out_ids = torch.empty((B, k1), dtype=torch.int32, device=verify_logits.device)
    if n_accept is None:
        n_accept = torch.empty(B, dtype=torch.int32, device=verify_logits.device)
    rc = LIB.vc_accept(_ptr(draft_ids), _ptr(verify_logits), B, k, V, _ptr(out_ids), _ptr(n_accept),
                       _stream(stream))
    _check(rc, "vc_accept")
    return out_ids, n_accept


# ------------------------------------------------------------------ prefetch

def prefetch_full_kv(host_pool: torch.Tensor, page_bytes: int, page_table_host, seq_ids, tok_begin: int,
                     tok_end: int, page_tokens: int, staging: torch.Tensor, dev_dst: torch.Tensor, stream=None,
                     done_event=None, staging_free=None):
    """host_pool: CPU uint8 [slots * page_bytes]; page_table_host: int32 numpy [n_seq, pages];
    staging: pinned CPU uint8; dev_dst: device uint8.  Pages land in dev_dst in
    (sequence, page) order."""
    import numpy as np
    tab = np.ascontiguousarray(page_table_host, dtype=np.int32)
    seqs = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int32))
    n_slots = host_pool.numel() // page_bytes
    p0 = tok_begin // page_tokens
    p1 = (tok_end + page_tokens - 1) // page_tokens
    need = len(seqs) * (p1 - p0) * page_bytes
    if dev_dst.numel() < need:
        raise VcError(f"dev_dst holds {dev_dst.numel()} bytes < {need}")
    s = torch.cuda.current_stream() if stream is None else stream
    # torch creates an event's HIP handle at its first record; record `done_event`
    # on the copy stream first so that it has one for the library to record after
    # the copy (an unrecorded `staging_free` has nothing to wait for: NULL)
    if done_event is not None and not done_event.cuda_event:
        done_event.record(s)
    ev = c_void(done_event.cuda_event) if done_event is not None else None
    fr = c_void(staging_free.cuda_event) if staging_free is not None and staging_free.cuda_event else None
    rc = LIB.vc_prefetch_full_kv(c_void(host_pool.data_ptr()), page_bytes, n_slots, tab.ctypes.data_as(c_void),
                                 tab.shape[0], tab.shape[1], seqs.ctypes.data_as(c_void), len(seqs), tok_begin,
                                 tok_end, page_tokens, c_void(staging.data_ptr()), staging.numel(),
                                 _ptr(dev_dst), fr, c_void(s.cuda_stream), ev)
    _check(rc, "vc_prefetch_full_kv")
