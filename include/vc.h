/*
 * vc.h — C ABI of libvc.so, the gfx950 (MI355X) hot path of compressed-KV
 * drafting with lossless verification.
 *
 * Source of the method: "VeriCache: Turning Lossy KV Cache into Lossless LLM
 * Inference" (gist.science explainer of the paper, English and Korean pages).
 * Each entry point below names the section of that page that defines the
 * operation.  The pages describe the method in prose only; every layout,
 * precision and error rule here is this library's own.
 *
 * Conventions shared by all entry points
 *  - Return value: VC_OK (0) or a negative VC_ERR_* code.  vc_last_error()
 *    returns a thread-local message for the last failure on this thread.
 *  - Every argument is validated on the host before anything is enqueued; a
 *    rejected call enqueues nothing.  Device-side faults surface as
 *    VC_ERR_HIP from a later call or from the caller's own synchronisation.
 *  - Pointers marked "device" must be device memory on the current HIP device;
 *    "host" pointers are read during the call only.  The caller owns every
 *    buffer; the library never allocates, frees or retains device memory.
 *  - Calls are asynchronous on the given stream: they enqueue work and return
 *    without waiting for the device.  The one exception is
 *    vc_prefetch_full_kv, whose host-side gather blocks the calling thread and
 *    may wait on the host for a staging event (see there).  Calls are
 *    reentrant; two calls that share a workspace must be stream-ordered.
 *  - bf16 = IEEE bfloat16 bit patterns; f16 = IEEE binary16; all tensors are
 *    dense row-major with the shapes given.
 *  - Heads: query head h reads KV head h / (Hq / Hkv) (contiguous GQA groups).
 */
#ifndef VC_H_
#define VC_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VC_OK 0
#define VC_ERR_INVALID -1     /* bad shape, null or misaligned pointer, bad enum */
#define VC_ERR_UNSUPPORTED -2 /* valid but not built (e.g. head_dim not in {64, 128}) */
#define VC_ERR_HIP -3         /* a HIP runtime call failed */
#define VC_ERR_WORKSPACE -4   /* workspace smaller than the matching *_ws_bytes() */

/* ------------------------------------------------------------------------ */
/* Uniform compressor interface                                              */
/* [VC Architecture Support: one compressor interface for token-dropping and */
/*  quantisation methods; VC Core Algorithm: drafting reads KV_comp]         */
/* ------------------------------------------------------------------------ */

#define VC_KV_IDENTITY 0   /* no compression: all L_full context rows      */
#define VC_KV_QUANT 1      /* asymmetric b-bit groups of 32 (KIVI-style)   */
#define VC_KV_TOKEN_DROP 2 /* a kept subset of context rows, by index      */

/*
 * QUANT caches exist in two forms.
 *
 * Canonical form (what a compressor produces; vc_pack_quant reads it and
 * vc_unpack_quant writes it), per (b, kv-head) unit of n rows, units
 * consecutive, dense:
 *   K codes  u8 [B][Hkv][n][D*bits/8]  token rows packed along D: 4-bit:
 *            channel 2i in the low nibble of byte i, 2i+1 in the high nibble;
 *            2-bit: channel i at bit 2*(i%4) of byte i/4
 *   V codes  u8 [B][Hkv][n][D*bits/8]  the same packing
 *   K meta   f16x2 {scale, zero} [B][Hkv][n/32][D]  one pair per group of 32
 *            tokens of one channel
 *   V meta   f16x2 {scale, zero} [B][Hkv][n][D/32]  one pair per group of 32
 *            channels of one token
 *   value = fp32(code * scale + zero), a single rounding.
 *
 * Internal form (what vc_draft_attn reads; written by vc_quantize_kv,
 * vc_quantize_blocks and vc_pack_quant).  Per (b, kv-head) slices are
 * consecutive; each holds Q = q_cap rows, q_cap = n_quant when the field is
 * 0, of which [0, n_quant) are live:
 *   k_codes  u8 [B][Hkv][Q][D*bits/8]  codes of token t packed along D:
 *            4-bit: channel 2i in the low nibble of byte i, 2i+1 in the high
 *            nibble; 2-bit: channel i at bit 2*(i%4) of byte i/4.
 *   v_codes  u8 [B][Hkv][Q/32][32*D*bits/8]  tiled: the codes of each
 *            block of 32 tokens are laid out as the operands of the draft
 *            kernel's matrix product.  Token tau (0..31) of a block, channel c:
 *              q = (tau % 16) / 4, e = tau % 4 + 4 * (tau / 16),
 *              lane = 16 q + c % 16, i = e / 2, hf = e % 2, ct = c / 16,
 *              pi = i * (D/16) + ct, dword = pi / (16/bits), j = pi % (16/bits),
 *              bit = bits * j + 16 * hf,
 *              byte = lane * (D*bits/16) + 4 * dword + bit / 8,
 *            code at bit (bit % 8) of that byte.
 *   k_meta   f16 [B][Hkv][Q/32][2][D]  per 32-token block, a plane of
 *            the scales and then a plane of the zeros of the groups formed by
 *            the block's 32 tokens of one channel, each plane in pair order:
 *            channel c (quad = c / (D/4), r = c % (D/4), cpd = 32/bits,
 *            ppd = cpd/2, d = r / cpd, h = (r % cpd) / ppd, j = r % ppd,
 *            pi = d * ppd + j) sits at
 *              2 * ((quad * (D/32) + pi / 4) * 4 + pi % 4) + h,
 *            so that each dword pairs the two channels one K code dword holds
 *            at bits b and b + 16.
 *   v_meta   f16x2 [B][Hkv][Q/32][D/32][32]  {scale, zero} of the group
 *            formed by 32 consecutive channels of one token; token tau of a
 *            block sits in slot 8 * ((tau % 16) / 4) + tau % 4 + 4 * (tau / 16).
 *   All four arrays must be 16-byte aligned for vc_draft_attn.
 *   Dequantised value = fp32(code * scale + zero), a single rounding.
 *   Inputs must keep |q| * K scale < 4096 and |V| scale * 256 < 65504 (the
 *   draft kernel carries these products in f16).  Nothing checks them at run
 *   time (the values are device data); beyond them the f16 products overflow
 *   and the results are undefined (in practice inf or NaN).
 * IDENTITY / TOKEN_DROP read k_full / v_full  bf16 [B][Hkv][L_cap][D]; rows
 *   [0, L_full) are context.  keep_idx int32 [B][Hkv][n_keep], sorted,
 *   each in [0, L_full); out-of-range entries are skipped, not dereferenced.
 * All pointers are device pointers; unused ones may be NULL.
 */
typedef struct vc_kv_comp {
  int kind;          /* VC_KV_*                                    */
  int bits;          /* QUANT: 2 or 4                              */
  int n_quant;       /* QUANT: quantised context rows, % 32 == 0   */
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const void* k_meta;
  const void* v_meta;
  const void* k_full;
  const void* v_full;
  int L_full;        /* IDENTITY: context rows                     */
  int L_cap;         /* IDENTITY/TOKEN_DROP: row capacity of k_full */
  const int32_t* keep_idx;
  int n_keep;        /* TOKEN_DROP: kept rows per (b, kv-head)      */
  int q_cap;         /* QUANT: rows each (b, kv-head) slice of the code
                        and meta arrays holds, % 32 == 0, >= n_quant;
                        0 means n_quant (a cache that never grows)  */
} vc_kv_comp;

/*
 * Exact rows every draft step also attends to, after the compressed part:
 * the uncompressed recent window followed by the rows of this round's drafted
 * positions up to and including the current one.
 *   k, v  device bf16 [B][Hkv][T_cap][D];  len device int32 [B], each clamped
 *   to [0, T_cap].  T_cap may be 0 (then k, v, len may be NULL).
 */
typedef struct vc_tail {
  const void* k;
  const void* v;
  const int32_t* len;
  int T_cap;
} vc_tail;

/*
 * Full (exact) cache for verification.
 *  Contiguous (page_table == NULL): k, v device bf16 [B][Hkv][L_cap][D].
 *  Paged: k = device pool base; v unused.  A page holds page_tokens tokens of
 *   every KV head as bf16 [Hkv][2 (K then V)][page_tokens][D]; logical page p
 *   of sequence b sits in slot page_table[b * pages_per_seq + p] (device
 *   int32).  page_tokens is a power of two >= 8; the pool holds n_slots
 *   pages, and a slot outside [0, n_slots) reads as zeros, never out of
 *   bounds.
 */
typedef struct vc_kv_full {
  const void* k;
  const void* v;
  int L_cap;
  const int32_t* page_table;
  int page_tokens;
  int pages_per_seq;
  int n_slots;
} vc_kv_full;

/* ------------------------------------------------------------------------ */

int vc_version(void);
const char* vc_last_error(void);

/*
 * vc_quantize_kv — build the QUANT cache from bf16 rows [0, n_quant) of
 * k_src / v_src (device bf16 [B][Hkv][L_cap][D]).  [VC Problem Statement:
 * quantisation as a lossy KV compressor; VC Architecture Support: KIVI]
 * Per group: mn/mx exact; s = f16((mx - mn) / (2^bits - 1)) and z = f16(mn)
 * (fp32 subtract and divide, round-to-nearest-even); code = 0 if s == 0, else
 * clamp(rint((x - z) / s), 0, 2^bits - 1) in fp32.  Writes the QUANT layout
 * above (out->k_codes etc. are written through; kind/bits/n_quant/q_cap are
 * read).  D in {64, 128}; bits in {2, 4}; n_quant % 32 == 0, n_quant <= L_cap,
 * n_quant <= q_cap.
 */
int vc_quantize_kv(const void* k_src, const void* v_src, int B, int Hkv, int L_cap, int D,
                   const vc_kv_comp* out, hipStream_t stream);

/*
 * vc_quantize_blocks — grow a QUANT cache by whole 32-token blocks: the rows
 * that leave the exact recent window are quantised into the next blocks of
 * the cache.  [VC Architecture Support: KIVI is one of the quantisers the
 * uniform compressor interface names]  The pages do not say how a quantised
 * cache grows during decoding; moving whole 32-token blocks out of an exact
 * recent window is this library's rule.
 * Source rows [src_row0, src_row0 + 32 * n_blocks) of every (b, kv-head) of
 * k_src / v_src (device bf16 [B][Hkv][src_rows][D]) become cache blocks
 * [dst_block, dst_block + n_blocks) of out, with the same per-group
 * arithmetic as vc_quantize_kv, so that quantising a context in pieces gives
 * the same bytes as quantising it at once.  Needs
 * 32 * (dst_block + n_blocks) <= q_cap (out->q_cap must be set, or n_quant
 * large enough).  out->n_quant is neither read nor changed: the caller
 * raises it (in its own descriptor) once the blocks are written, by
 * 32 * n_blocks when they are appended.  n_blocks == 0 is a no-op.
 * Errors: VC_ERR_INVALID for a range outside the source or the cache, a bad
 * kind/bits or a null pointer; VC_ERR_UNSUPPORTED for D not in {64, 128}.
 * Launches on `stream`; nothing is allocated.
 */
int vc_quantize_blocks(const void* k_src, const void* v_src, int B, int Hkv, int src_rows, int D, int src_row0,
                       int n_blocks, const vc_kv_comp* out, int dst_block, hipStream_t stream);

/*
 * vc_pack_quant — the compressor-facing side of the uniform interface: turn a
 * QUANT cache in canonical form (k_codes, v_codes, k_meta, v_meta: device, n
 * rows per unit, layouts above) into blocks [dst_block, dst_block + n/32) of
 * the internal form that `out` describes (its kind, bits and q_cap are read;
 * its arrays are written).  [VC Architecture Support: a uniform compressor
 * interface admits existing quantisation methods without changes to the
 * scheduling or verification logic]  A compressor that produces the
 * canonical form can feed vc_draft_attn through this call; quantising with
 * vc_quantize_kv gives the same bytes as packing the canonical form of the
 * same quantisation.  n % 32 == 0 and 32 * dst_block + n <= q_cap (or
 * n_quant when q_cap is 0); n == 0 is a no-op.  out->n_quant is not changed.
 * Canonical K codes and the internal K codes must be 16-byte aligned, all
 * metadata 4-byte aligned.  Errors: VC_ERR_INVALID (bad kind/bits, range,
 * NULL or misaligned pointer), VC_ERR_UNSUPPORTED (D not in {64, 128}).
 * One launch on `stream`; nothing is allocated.
 *
 * vc_unpack_quant — the inverse: rows [0, in->n_quant) of the internal form
 * into canonical arrays of n_quant rows per unit.  Same rules.
 */
int vc_pack_quant(const uint8_t* k_codes, const uint8_t* v_codes, const void* k_meta, const void* v_meta,
                  int B, int Hkv, int n, int D, const vc_kv_comp* out, int dst_block, hipStream_t stream);
int vc_unpack_quant(const vc_kv_comp* in, int B, int Hkv, int D, uint8_t* k_codes, uint8_t* v_codes,
                    void* k_meta, void* v_meta, hipStream_t stream);

/*
 * vc_select_top_m — the token-dropping compressor's selection: for each of
 * `rows` rows (one per (batch, kv-head)) of importance scores (device fp32
 * [rows][L]), keep_idx[r] (device int32 [rows][M]) receives the indices of
 * the M largest scores, ties to the lower index, in ascending order: the
 * kept-row list of a VC_KV_TOKEN_DROP cache.  Scores compare as numbers (-0
 * equals +0); NaN scores give an unspecified (but valid, sorted, unique) set.
 * 0 <= M <= L.  [VC Problem Statement: token dropping; VC Architecture
 * Support: token-dropping compressors behind the uniform interface]
 * Errors: VC_ERR_INVALID for rows < 0, L < 0, M outside [0, L], or a NULL
 * scores / keep_idx when there is work; rows == 0 or M == 0 is a no-op.
 * One workgroup per row on `stream`; nothing is allocated.
 */
int vc_select_top_m(const float* scores, int rows, int L, int M, int32_t* keep_idx, hipStream_t stream);

/*
 * vc_debug_dequant — dequantised K (which = 0) or V (which = 1) of the live
 * rows [0, n_quant) of one (b, kv-head) as fp32 [n_quant][D] into out
 * (device).  For bit-exact checks.
 */
int vc_debug_dequant(const vc_kv_comp* comp, int B, int Hkv, int D, int b, int h, int which,
                     float* out, hipStream_t stream);

/*
 * vc_draft_attn — one draft decode step.  [VC Core Algorithm: drafting
 * generates candidate tokens with the compressed cache KV_comp; VC Key System
 * Innovations P1: drafting is HBM-bandwidth bound]
 * For every (b, h): o = softmax(scale * q K^T) V over the compressed context
 * rows of KV head h/(Hq/Hkv) followed by the tail rows [0, tail.len[b]).
 *   q    device bf16 [B][Hq][D]
 *   out  device fp32 [B][Hq][D]
 *   lse  device fp32 [B][Hq] or NULL: natural log of sum_t exp(scale q.k_t)
 *   ws   device workspace of at least vc_draft_ws_bytes(B, Hq, Hkv, D,
 *        n_main + T_cap) bytes, 16-byte aligned (n_main = n_quant, L_full or
 *        n_keep).  QUANT codes must be 16-byte aligned, V meta 8-byte.
 * A sequence with no key at all (an empty compressed part and a zero tail
 * length) gets o = 0 and lse = -inf.
 * D in {64, 128}; Hq % Hkv == 0; Hq / Hkv <= 8.
 */
size_t vc_draft_ws_bytes(int B, int Hq, int Hkv, int D, int max_keys);
int vc_draft_attn(const vc_kv_comp* comp, const vc_tail* tail, const void* q, float* out,
                  float* lse, int B, int Hq, int Hkv, int D, float scale, void* ws,
                  size_t ws_bytes, hipStream_t stream);

/*
 * vc_draft_attn_noalloc — vc_draft_attn for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments without the workspace.  The split partials
 * go to a scratch array of VC_DRAFT_SCRATCH_BYTES that the library holds on
 * each GPU it runs on until the process ends; the call itself allocates
 * nothing.  Every call on one GPU shares that GPU's array, so calls that
 * overlap in time on one GPU (different streams, or several threads) race
 * and must be ordered by the caller.  A call whose partials would not fit
 * (vc_draft_ws_bytes gives an upper bound) returns VC_ERR_UNSUPPORTED before
 * enqueueing anything.  Results are identical to vc_draft_attn's.
 */
#define VC_DRAFT_SCRATCH_BYTES (16u << 20)
int vc_draft_attn_noalloc(const vc_kv_comp* comp, const vc_tail* tail, const void* q, float* out, float* lse,
                          int B, int Hq, int Hkv, int D, float scale, hipStream_t stream);

/*
 * vc_verify_attn — causal verification of n_q positions in one pass.
 * [VC Core Algorithm: a single forward pass with KV_full verifies all drafted
 * tokens in parallel; VC Key System Innovations P1: verification is
 * interconnect- and compute-bound]
 * Position j of sequence b (query q[b][h][j]) attends to keys [0,
 * ctx_len[b] + j] of the full cache: the context and the new rows of the
 * positions up to and including j, which the caller wrote at rows
 * ctx_len[b] .. ctx_len[b] + n_q - 1 beforehand.  Also serves as prefill
 * (ctx_len = 0, large n_q).
 *   q        device bf16 [B][Hq][n_q][D]
 *   ctx_len  device int32 [B]; each must be <= max_ctx (host int) and
 *            ctx_len + n_q must fit the cache (L_cap or pages_per_seq pages).
 *   out      device fp32 [B][Hq][n_q][D]
 *   ws       device workspace of at least vc_verify_ws_bytes(...) bytes.
 * Precision: q.k products on bf16 matrix cores with fp32 accumulation; the
 * softmax in fp32; probabilities rounded to f16 (nearest even) and values
 * converted bf16 -> f16 for the P.V product (fp32 accumulation).  Values must
 * lie in the f16 range (|v| < 65504); larger ones become f16 infinities (not
 * checked at run time).
 * D in {64, 128}; Hq % Hkv == 0.
 */
size_t vc_verify_ws_bytes(int B, int Hq, int Hkv, int D, int n_q, int max_ctx);
int vc_verify_attn(const void* q, const vc_kv_full* kv, const int32_t* ctx_len, int max_ctx,
                   int n_q, float* out, int B, int Hq, int Hkv, int D, float scale, void* ws,
                   size_t ws_bytes, hipStream_t stream);

/*
 * Chunked verify: the same attention as vc_verify_attn, taken one key range
 * at a time, so that a caller can verify each chunk of a full cache as it
 * arrives from host memory and merge at the end.  [VC Key System Innovations
 * P1: the full KV is loaded over the interconnect while compute proceeds;
 * VC Architecture Support: long-context decoding keeps the full KV in CPU
 * memory]
 *
 * vc_verify_attn_range — keys [key_begin, key_end) of every sequence, clipped
 * to the causal limit ctx_len[b] + j of query position j.  Arguments as in
 * vc_verify_attn.  Reads start at the multiple of 8 at or below key_begin
 * (the rows before key_begin are masked out); that row lies in key_begin's
 * page, so only the pages holding rows of the range are read and the rest of
 * a paged cache may still be in flight.  key_begin need not be aligned.  Writes
 * vc_verify_range_parts(B, Hq, Hkv, D, n_q, key_begin, key_end) partial
 * slots to parts (device fp32, 16-byte aligned), each [B*Hq*n_q][D + 2]:
 * per query row the unnormalised sum o[0..D) of 2^(s - m) v over its keys,
 * the score maximum m (log2 units of scale * q.k) and the sum l of 2^(s - m);
 * m = -inf and l = 0 for a row that saw no key.  No output, no workspace.
 * 0 <= key_begin < key_end <= max_ctx + n_q.
 *
 * vc_verify_merge — out[r] = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p
 * with M = max_p m_p over n_parts (1..256) consecutive partial slots; rows
 * = B*Hq*n_q, out device fp32 [rows][D].  A row no part saw gets 0.  Merging
 * the parts of ranges that tile [0, max_ctx + n_q) gives vc_verify_attn's
 * result up to rounding order.
 */
int vc_verify_range_parts(int B, int Hq, int Hkv, int D, int n_q, int key_begin, int key_end);
int vc_verify_attn_range(const void* q, const vc_kv_full* kv, const int32_t* ctx_len, int max_ctx,
                         int n_q, int key_begin, int key_end, float* parts, int B, int Hq, int Hkv, int D,
                         float scale, hipStream_t stream);
int vc_verify_merge(const float* parts, int n_parts, int B, int Hq, int n_q, int D, float* out,
                    hipStream_t stream);

/*
 * vc_argmax — greedy token of each row: ids[r] = index of the largest of
 * logits[r][0..V) (device fp32 [rows][V]); ties go to the lowest index.
 * Rows containing NaN give an unspecified index in [0, V).
 */
int vc_argmax(const float* logits, int rows, int V, int32_t* ids, hipStream_t stream);

/*
 * vc_accept — greedy acceptance.  [VC Core Algorithm: acceptance]  Each
 * sequence keeps its drafts up to the first one the verifier disagrees with,
 * then the verifier's own token; with no disagreement that token is the
 * bonus.
 *   draft_ids      device int32 [B][k]      d_0 .. d_{k-1}
 *   verify_logits  device fp32 [B][k+1][V]  logits of verify positions 0..k
 *   out_ids        device int32 [B][k+1]    d_0..d_{n-1}, y_n, then -1
 *   n_accept       device int32 [B]         n = first j < k with d_j != y_j,
 *                                           else k;  y_j = argmax (lowest
 *                                           index on ties) of position j
 * The emitted count is n + 1: at a mismatch the verifier's token replaces the
 * rejected draft.  k >= 0 (k = 0 emits the single verifier token).
 */
int vc_accept(const int32_t* draft_ids, const float* verify_logits, int B, int k, int V,
              int32_t* out_ids, int32_t* n_accept, hipStream_t stream);

/*
 * vc_prefetch_full_kv — move the full-KV pages of tokens [tok_begin, tok_end)
 * of the listed sequences from the host pool to device memory with one
 * host-to-device DMA copy on copy_stream, then record `done` (if not NULL) on
 * copy_stream.  [VC Architecture Support: long-context decoding keeps the full
 * KV in CPU memory and loads it over PCIe for verification; VC Key System
 * Innovations P1: the load overlaps other requests' drafting]
 *   host_pool    host memory of n_slots pages of page_bytes; logical page p of
 *                sequence b sits in slot page_table[b * pages_per_seq + p]
 *   page_table   host int32 [n_seq_total][pages_per_seq], slots < n_slots
 *   seq_ids      host int32 [n_seq]
 *   staging      pinned host memory (hipHostMalloc) of at least
 *                n_seq * n_pages * page_bytes, n_pages = ceil(tok_end /
 *                page_tokens) - tok_begin / page_tokens
 *   staging_free host waits on this event (if not NULL) before writing staging:
 *                pass the `done` of the previous copy out of the same buffer
 *   dev_dst      device memory of the same size
 * Host threads gather the pages into staging in order (sequence i of seq_ids,
 * then page p): output page k = i * n_pages + (p - tok_begin / page_tokens)
 * lands at dev_dst + k * page_bytes, the device layout a page table for
 * vc_verify_attn then points at.  The call returns once the gather is done and
 * the copy is enqueued.  No kernel runs.  An unpinned staging buffer is rejected
 * with VC_ERR_INVALID before any work.
 */
int vc_prefetch_full_kv(const void* host_pool, size_t page_bytes, int n_slots, const int32_t* page_table,
                        int n_seq_total, int pages_per_seq, const int32_t* seq_ids, int n_seq,
                        int tok_begin, int tok_end, int page_tokens, void* staging, size_t staging_bytes,
                        void* dev_dst, hipEvent_t staging_free, hipStream_t copy_stream, hipEvent_t done);

/* ------------------------------------------------------------------------ */
/* Staggering scheduler policy (host only: no device work, no GPU needed)    */
/* [VC Key System Innovations P2: long drafts amortise verification when     */
/*  acceptance is high; P1: one group drafts while another loads its full KV */
/*  and verifies]  The pages state the principle; the rule below is this     */
/* library's.                                                                */
/* ------------------------------------------------------------------------ */

/*
 * vc_sched_accept_rate — per-draft match probability estimated from a
 * group's history: `accepted` = drafts accepted over its rounds (the sum of
 * n_accept), `rejections` = rounds that stopped at a mismatch (n_accept < k).
 * Returns (accepted + 1) / (accepted + rejections + 2) (the estimate with one
 * prior match and one prior mismatch, so it lies in (0, 1)); NaN for negative
 * counts.
 */
double vc_sched_accept_rate(long long accepted, long long rejections);

/*
 * vc_sched_expected_tokens — tokens a round with draft length k emits on
 * average when each draft matches with probability a until the first
 * mismatch: the accepted drafts plus the verifier's token,
 * 1 + a + a^2 + ... + a^k, summed in that order in fp64.  NaN for a outside
 * [0, 1] or k < 0.
 */
double vc_sched_expected_tokens(double a, int k);

/*
 * vc_sched_choose_k — draft length of a group's next round: the k in
 * [k_min, k_max] that maximises
 *   vc_sched_expected_tokens(a, k) / (max(k * t_draft, t_overlap) + t_rest),
 * a = vc_sched_accept_rate(accepted, rejections), ties to the smaller k.
 *   t_draft    time of one draft step of this group
 *   t_overlap  work of the other group that this group's drafting runs
 *              beside (its full-KV transfer and verification); 0 unstaggered
 *   t_rest     the rest of the cycle, independent of k (this group's own
 *              verification and accept, or the other group's drafting when
 *              that is longer)
 * Any time unit, the same for all three.  Returns k >= 1, or VC_ERR_INVALID
 * for negative counts, 1 <= k_min <= k_max <= 64 violated, t_draft <= 0, or a
 * negative or non-finite time.
 */
int vc_sched_choose_k(long long accepted, long long rejections, double t_draft, double t_overlap, double t_rest,
                      int k_min, int k_max);

#ifdef __cplusplus
}
#endif
#endif /* VC_H_ */
