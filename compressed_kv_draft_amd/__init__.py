"""MI355X (gfx950) hot path of compressed-KV drafting with lossless verification.

Importing the package loads libvc.so (built in place by ``build.py``) and fails
loudly if it is missing: every step of the path runs in its HIP kernels.
"""
from ._lib import (  # noqa: F401
    LIB, VcError, Compressed, Tail, FullKV, version, quantize_kv, quantize_blocks, empty_quant, pack_quant, unpack_quant,
    identity_cache, token_drop_cache,
    select_top_m,
    debug_dequant, draft_ws_bytes, draft_attn, draft_attn_noalloc, verify_ws_bytes, verify_attn, verify_range_parts,
    verify_attn_range, verify_merge, argmax, accept,
    prefetch_full_kv, sched_accept_rate, sched_expected_tokens, sched_choose_k,
)
