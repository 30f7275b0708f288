// Draft decode attention over the lossy cache (one query position per call).
//
// [VC Core Algorithm: drafting generates candidate tokens with KV_comp;
//  VC Key System Innovations P1: drafting is GPU-HBM-bandwidth bound]
//
// The g query heads of a GQA group read the same compressed K/V, so q.K^T and
// P.V are thin matrix products (g rows).  With int2/int4 codes they carry 20-26
// multiply-adds per HBM byte, more than fp32 vector ALUs sustain at HBM speed,
// so both products run on the f16 matrix cores, exactly:
//  * a code c placed at bit p of the mantissa of an f16 bit pattern is the
//    subnormal c * 2^(p - 24) -- a shift and an AND turn two packed codes into
//    two exact f16 operands (always at p >= 4, see code_target);
//  * K is grouped per channel, so its scale goes into the query: q_h * s is
//    computed in f16 as hi + lo (a rounded product and its exact residual, one
//    fma), giving 22 significand bits; hi and lo are adjacent MFMA columns;
//  * V is grouped per token and channel group G, so its scale goes into the
//    probabilities: p * s_{t,G} is split into f16 hi and lo and applied in two
//    products; the zero points enter as sum_t p_t z_{t,G} (fp32) and, for K,
//    as one more small product z . q per 32-token group.
// Exact bf16 rows (the uncompressed recent window and this round's drafted
// rows, or the identity / token-dropped caches) use bf16 products: q.k exactly,
// P.V with P split into bf16 hi + lo, V transposed through LDS with the gfx950
// transpose read.
//
// Work split: a workgroup (4 wavefronts) owns one (batch, kv-head) and a range
// of 32-token blocks; wavefronts take every 4th block and keep their own
// online-softmax state, merged in LDS at the end.  The last workgroups of each
// (batch, kv-head) first take a range of the exact tail rows as a partial of
// their own.  draft_combine_kernel merges the partials.
#include <map>
#include <mutex>

#include "lds_dma.h"
#include "mfma.h"
#include "vc_common.h"

namespace vc {
namespace {

struct DraftArgs {
  int n_main;     // rows of the compressed part (quant: n_quant; identity: L_full; drop: n_keep)
  int q_cap;      // quant: rows per unit the code/meta arrays hold (their stride)
  int L_cap;      // identity / drop: rows per unit of k_full / v_full (their stride)
  int row_bound;  // valid physical rows of k_full/v_full (identity / drop)
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const uint32_t* k_meta;  // f16x2 {scale, zero}
  const uint32_t* v_meta;
  const uint16_t* k_full;
  const uint16_t* v_full;
  const int32_t* keep_idx;
  const uint16_t* tail_k;
  const uint16_t* tail_v;
  const int32_t* tail_len;
  int T_cap;
  const uint16_t* q;
  float* out;
  float* lse;
  int B, Hq, Hkv, g;
  float scale_log2;
  int main_splits;            // workgroups of one (batch, kv-head)
  int main_bpw, main_bpw_t;   // compressed blocks per workgroup: before / from tail_first
  int tail_first, tail_bpw;   // workgroups >= tail_first first take tail_bpw exact tail blocks
  int splits;                 // partials per (batch, kv-head): main_splits + tail workgroups
  int direct;                 // 1: a single partial, written as the output
  int xcd_affine;             // 1: 1-D grid, every split of unit u on XCD u % 8 (units % 8 == 0)
  float* ws;                  // split partials [splits][B][Hq][D + 2]
};

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kTau = 8.0f;  // lazy rescale: the running max moves only when exceeded by 2^8
constexpr int kQExp = 4;      // q is scaled by 2^kQExp before it multiplies the K scales

constexpr int cmax(int x, int y) { return x > y ? x : y; }
constexpr int cmin(int x, int y) { return x < y ? x : y; }
constexpr int kLdsPerCu = 160 * 1024;

template <int D, int BITS>
struct Cfg {
  static constexpr int NKS = D / 32;   // k-steps of q.k
  static constexpr int NCT = D / 16;   // 16-channel column tiles of P.V
  static constexpr int NG = D / 32;    // V channel groups
  static constexpr int B_ = BITS > 0 ? BITS : 2;
  static constexpr int CPD = 32 / B_;  // K channels per code dword
  static constexpr int PPD = CPD / 2;  // code pairs per dword
  // V channel tile ct always takes pair ct % PPD when the tiles cover a whole dword
  static constexpr bool VWIDE = NCT >= PPD;
  static constexpr int PER = 8 / B_;   // codes per byte
  static constexpr uint32_t MASK = B_ == 2 ? 0x00030003u : 0x000F000Fu;
  static constexpr int KDW = D * B_ / 128;  // K code dwords per lane per 16-token tile
  static constexpr int VDW = D * B_ / 64;   // V code dwords per lane per block
  static constexpr int VMD = NG / 2;        // V meta dwords staged per lane per block
  static constexpr int VPITCH = D + 16;     // LDS row pitch (elements) of staged bf16 V
  static constexpr int ROWS_WAVE = 32 * VPITCH * 2;  // per-wavefront LDS of the exact-row path
  // one 32-token block of the compressed streams (all multiples of 16 bytes)
  static constexpr int ROW_BYTES = D * B_ / 8;  // K codes of one token
  static constexpr int KC_BYTES = 32 * ROW_BYTES;
  static constexpr int VC_BYTES = 32 * ROW_BYTES;
  static constexpr int KM_BYTES = 4 * D;  // scale plane + zero plane, f16, pair order
  static constexpr int VM_BYTES = 4 * D;  // [NG][32 tokens] {scale, zero}
  static constexpr int VC_OFF = KC_BYTES, KM_OFF = VC_OFF + VC_BYTES, VM_OFF = KM_OFF + KM_BYTES;
  static constexpr int SLOT = VM_OFF + VM_BYTES;
  static constexpr int NDMA = lds_dma_count(KC_BYTES) + lds_dma_count(VC_BYTES) + lds_dma_count(KM_BYTES) +
                              lds_dma_count(VM_BYTES);  // load instructions per block
  // shared by the workgroup's wavefronts: zeros, and (int2) the query as f16
  static constexpr int ZERO_BYTES = 64 * NKS;
  static constexpr int QZ_BYTES = BITS == 2 ? 8 * 4 * NKS * 16 : 0;  // [ks][quad][head] u32x4
  static constexpr int SHARED_BYTES = BITS == 0 ? 0 : ZERO_BYTES + QZ_BYTES;
  // ring slots per wavefront: up to 4; as many as leave room for 4 workgroups
  // per CU if that gives at least 2, else for 3
  static constexpr int D4 = (kLdsPerCu / 4 - SHARED_BYTES) / kWaves / SLOT;
  static constexpr int D3 = (kLdsPerCu / 3 - SHARED_BYTES) / kWaves / SLOT;
  static constexpr int DEPTH = BITS == 0 ? 0 : cmin(4, D4 >= 2 ? D4 : D3);
  static constexpr int RING_WAVE = DEPTH * SLOT;
  static constexpr int ZERO_OFF = kWaves * RING_WAVE, QZ_OFF = ZERO_OFF + ZERO_BYTES;
  static constexpr int EPI_BYTES = kWaves * (8 * D + 8 + 8 + 8 * 4) * 4;
  static constexpr int SMEM = cmax(cmax(kWaves * RING_WAVE + SHARED_BYTES, kWaves * ROWS_WAVE), EPI_BYTES);
  // wavefronts per SIMD the register allocation aims at: as many as LDS allows, up to 4
  static constexpr int WAVES = cmin(4, kLdsPerCu / SMEM);
};

// Bit position (in units of `bits`, inside its 16-bit half) at which code pair j
// of a dword is handed to the matrix cores.  The f16 products sum with a
// truncating internal alignment when their magnitudes differ widely; keeping
// every code operand at least 2^(4-24) avoids the systematic bias the lowest
// subnormals (2^-24) showed on the device.  int4: bits 4..7 (jt 1).  int2,
// WIDE: bits 4..9 (jt 2, 3, 4), reached with two shift amounts per dword (<< 4
// for pairs 0-1, none for 2-4, >> 6 for 5-7); otherwise bits 4..7 by parity of
// j (three shift amounts), for operands whose channel takes pairs j and j + 4.
template <int BITS, bool WIDE>
__host__ __device__ constexpr int code_target(int j) {
  if constexpr (BITS == 4) {
    return 1;
  } else if constexpr (WIDE) {
    constexpr int t[8] = {2, 3, 2, 3, 4, 2, 3, 4};
    return t[j % 8];
  } else {
    return 2 + ((j % 4) & 1);
  }
}

// Two packed codes (bits b and b+16 of w, pair position j of the dword) as an
// f16 pair: code * 2^(bits * code_target(j) - 24) each, exactly.
template <int BITS, bool WIDE>
__device__ __forceinline__ uint32_t code_pair(uint32_t w, int j) {
  constexpr int PER = 8 / BITS;
  constexpr uint32_t MASK = BITS == 2 ? 0x00030003u : 0x000F000Fu;
  const int jt = code_target<BITS, WIDE>(j);
  const int sh = 8 * (j / PER) + BITS * (j % PER) - BITS * jt;
  const uint32_t ws = sh >= 0 ? (w >> sh) : (w << -sh);
  return ws & (MASK << (BITS * jt));
}

// N consecutive dwords from an address aligned to min(16, 4N) bytes.
template <int N>
__device__ __forceinline__ void load_dwords(const void* p, uint32_t* out) {
  if constexpr (N == 1) {
    out[0] = *reinterpret_cast<const uint32_t*>(p);
  } else if constexpr (N == 2) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    out[0] = w.x;
    out[1] = w.y;
  } else {
    static_assert(N % 4 == 0, "");
#pragma unroll
    for (int k = 0; k < N / 4; ++k) {
      const u32x4 w = reinterpret_cast<const u32x4*>(p)[k];
      out[4 * k] = w[0];
      out[4 * k + 1] = w[1];
      out[4 * k + 2] = w[2];
      out[4 * k + 3] = w[3];
    }
  }
}

// Value of the neighbouring lane (lane ^ 1) through DPP quad_perm [1, 0, 3, 2].
__device__ __forceinline__ float swap_adjacent(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}

// Per-lane softmax state: running max m (log2 units) of this lane's head, the
// offset mu the scores are taken relative to (m, or 0 while m is -inf), the
// amount thr a block max must exceed to move m (-inf while m is -inf, else
// kTau), the partial sum l over this lane's tokens, zero-point sums, output
// accumulators.
template <int NCT, int NV>
struct State {
  float m, mu, thr, l;
  float zacc[NV];
  f32x4 O[NCT];
  __device__ __forceinline__ void clear() {
    m = kNegInf;
    mu = 0.0f;
    thr = kNegInf;
    l = 0.0f;
#pragma unroll
    for (int v = 0; v < NV; ++v) zacc[v] = 0.0f;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) O[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
};

// Online softmax over the 8 scores a lane holds for one block (its head, tokens
// 4q..4q+3 and 16+4q..16+4q+3).  Scores arrive relative to st.mu.  The running
// max only moves when some score exceeds it by kTau, so in the common case no
// cross-lane reduction and no rescale happen; P <= 2^kTau.
template <int NCT, int NV>
__device__ __forceinline__ void softmax_block(float (&x)[8], State<NCT, NV>& st, float (&P)[8], int quad) {
  float tl = x[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) tl = fmaxf(tl, x[e]);
  if (__any(tl > st.thr)) {
    float tr = fmaxf(tl, shfl_xor(tl, 16));
    tr = fmaxf(tr, shfl_xor(tr, 32));  // max over the head's tokens of this block
    const float mu = st.mu;
    const float mn = fmaxf(st.m, mu + tr);
    const float alpha = mn == kNegInf ? 1.0f : fast_exp2(st.m - mn);
    st.l *= alpha;
#pragma unroll
    for (int v = 0; v < NV; ++v) st.zacc[v] *= alpha;
    // output row 4q+i belongs to the head of column 4q+i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float ar = __shfl(alpha, 4 * quad + i, 64);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) st.O[ct][i] *= ar;
    }
    const float delta = mn == kNegInf ? 0.0f : mn - mu;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] -= delta;
    st.m = mn;
    st.mu = mn == kNegInf ? 0.0f : mn;
    st.thr = mn == kNegInf ? kNegInf : kTau;
  }
  float ps = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    P[e] = fast_exp2(x[e]);
    ps += P[e];
  }
  st.l += ps;
}

// Source of exact bf16 rows: the tail, the identity cache or the kept rows.
struct RowSrc {
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* idx;  // logical -> physical row (token drop) or nullptr
  size_t unit_row0;    // first row of this (batch, kv-head)
  int n_valid;         // logical rows
  int bound;           // physical rows in [0, bound) are readable
};

// The kept-row index (or the row itself) of logical row blk * 32 + (lane & 31),
// unchecked; -1 past the valid rows.  Loaded a block ahead of its use, so that
// a block's row loads wait for one memory latency, not for two in sequence.
__device__ __forceinline__ int block_row_index(const RowSrc& src, int blk, int lane) {
  const int t = blk * 32 + (lane & 31);
  if (t >= src.n_valid) return -1;
  return src.idx != nullptr ? src.idx[t] : t;
}

// One block of 32 exact rows: q.k on bf16 matrix cores, P.V with P = hi + lo in
// bf16 and V staged in LDS, read transposed.  row_idx: block_row_index of this
// block for this lane.
template <int D, int NV>
__device__ __forceinline__ void rows_block(const RowSrc& src, int row_idx, const bf16x8 (&qb)[D / 32],
                                           float scale_log2, uint16_t* vst, State<D / 16, NV>& st, int lane,
                                           int col, int quad, int hilo) {
  constexpr int NKS = D / 32, NCT = D / 16, VPITCH = D + 16;
  // physical row of this lane's logical row (lane & 31) of the block, or -1 (past
  // the valid rows, or an index outside [0, bound): skipped, never dereferenced)
  const int myrow = (row_idx >= 0 && row_idx < src.bound) ? row_idx : -1;
  // K rows of tokens col and 16 + col; k-step ks takes channels 32 ks + 8 quad
  // .. + 7, so the four quads of a row read 64 contiguous bytes per load
  u32x4 kr[2][NKS];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int pr = __shfl(myrow, 16 * tt + col, 64);
    const uint16_t* p = src.k + (src.unit_row0 + (size_t)(pr < 0 ? 0 : pr)) * D + 8 * quad;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      kr[tt][ks] = pr >= 0 ? *reinterpret_cast<const u32x4*>(p + 32 * ks) : u32x4{0u, 0u, 0u, 0u};
  }
  // V rows into LDS (row-major, padded pitch)
#pragma unroll
  for (int u = 0; u < D / 16; ++u) {
    const int c = lane + 64 * u;
    const int row = c / (D / 8), off = (c % (D / 8)) * 8;
    const int pr = __shfl(myrow, row, 64);
    const u32x4 val = pr >= 0 ? *reinterpret_cast<const u32x4*>(src.v + (src.unit_row0 + (size_t)pr) * D + off)
                              : u32x4{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(vst + row * VPITCH + off) = val;
  }
  // scores (log2 units, relative to the running max), invalid rows masked
  const float mu = st.mu;
  float x[8];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) acc = mfma_bf16(__builtin_bit_cast(bf16x8, kr[tt][ks]), qb[ks], acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * tt + 4 * quad + i;
      const int pr = __shfl(myrow, r, 64);
      x[4 * tt + i] = pr >= 0 ? fmaf(acc[i], scale_log2, -mu) : kNegInf;
    }
  }
  float P[8];
  softmax_block<NCT, NV>(x, st, P, quad);
  // A operand: bf16 hi part (even columns) or lo residual (odd columns) of P
  u32x4 ap;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float p = P[2 * k + h];
      const uint32_t hb = __float_as_uint(p) & 0xFFFF0000u;
      const float lo = p - __uint_as_float(hb);
      w[h] = (hilo ? __float_as_uint(lo) : hb) >> 16;
    }
    ap[k] = w[0] | (w[1] << 16);
  }
  const bf16x8 A = __builtin_bit_cast(bf16x8, ap);
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const uint16_t* base = vst + 16 * ct + 4 * (col & 3);
    const s16x4 lo4 = lds_read_tr16(base + (4 * quad + (col >> 2)) * VPITCH);
    const s16x4 hi4 = lds_read_tr16(base + (16 + 4 * quad + (col >> 2)) * VPITCH);
    const s16x8 bv8 = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
    st.O[ct] = mfma_bf16(A, __builtin_bit_cast(bf16x8, bv8), st.O[ct]);
  }
}

// This wavefront's exact-row blocks first, first + kWaves, ... below end, each
// block's row indices loaded while the previous block is computed.
template <int D, int NV>
__device__ __forceinline__ void rows_loop(const RowSrc& src, int first, int end, const bf16x8 (&qb)[D / 32],
                                          float scale_log2, uint16_t* vst, State<D / 16, NV>& st, int lane,
                                          int col, int quad, int hilo) {
  int idx_next = first < end ? block_row_index(src, first, lane) : -1;
  for (int blk = first; blk < end; blk += kWaves) {
    const int idx = idx_next;
    if (blk + kWaves < end) idx_next = block_row_index(src, blk + kWaves, lane);
    rows_block<D, NV>(src, idx, qb, scale_log2, vst, st, lane, col, quad, hilo);
  }
}

template <int D, int BITS, int NV>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(Cfg<D, BITS>::WAVES))) void draft_mfma_kernel(
    DraftArgs a) {
  using C = Cfg<D, BITS>;
  constexpr int NKS = C::NKS, NCT = C::NCT, NG = C::NG;
  __shared__ __attribute__((aligned(16))) unsigned char smem[C::SMEM];

  // Workgroups are dispatched to the 8 XCDs round-robin by id.  With an
  // XCD-affine grid, the splits of one (batch, kv-head) unit all run on one
  // XCD, so the partials they write stay in that XCD's L2 for the combine.
  int unit, split;
  if (a.xcd_affine) {
    const int id = blockIdx.x, x8 = id % 8, y = id / 8;
    unit = (y / a.main_splits) * 8 + x8;
    split = y % a.main_splits;
  } else {
    unit = blockIdx.y;
    split = blockIdx.x;
  }
  const int b = unit / a.Hkv, hk = unit % a.Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, quad = lane >> 4;
  const int g = a.g;
  // column / row r of the 16-wide tiles <-> (head, hi-or-lo, replica)
  const int hp = col >> 1, hilo = col & 1;
  const int head = hp % g, rep = hp / g;
  const int R8 = 8 / g, SP = 2 * R8;  // replicas of the head set; V-group slots per head
  const int slot = 2 * rep + hilo;
  const bool slot_ok = rep < R8;

  uint16_t* vst = reinterpret_cast<uint16_t*>(smem + wave * C::ROWS_WAVE);  // exact-row path

  // this lane's query head: q for the exact rows' products (k-step ks takes
  // channels 32 ks + 8 quad .. + 7), loaded where it is used
  const uint16_t* qhead = a.q + ((size_t)b * a.Hq + hk * g + head) * D;
  auto load_qb = [&](bf16x8 (&qb)[NKS]) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qb[ks] = *reinterpret_cast<const bf16x8*>(qhead + 8 * quad + 32 * ks);
  };

  State<NCT, NV> st;
  st.clear();

  const size_t unit_rows = (size_t)unit;

  // Merge the wavefronts' states through LDS and write partial `part` (or the
  // output).  quant: the state holds the compressed part's code-scaled,
  // slot-grouped P.V (else exact-row P.V with hi/lo rows).
  auto finish = [&](int part, bool quant) __attribute__((always_inline)) {
    float lt = st.l;
    lt += shfl_xor(lt, 16);
    lt += shfl_xor(lt, 32);
    float zt[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      zt[v] = st.zacc[v];
      zt[v] += shfl_xor(zt[v], 16);
      zt[v] += shfl_xor(zt[v], 32);
    }
    __syncthreads();  // every wavefront is done with its staging region
    float* s_o = reinterpret_cast<float*>(smem);  // [kWaves][8][D]
    float* s_m = s_o + kWaves * 8 * D;            // [kWaves][8]
    float* s_l = s_m + kWaves * 8;                // [kWaves][8]
    float* s_z = s_l + kWaves * 8;                // [kWaves][8][4]
    const bool quant_wg = BITS > 0 && quant;
    if (quad == 0 && rep == 0 && hilo == 0) {
      s_m[wave * 8 + head] = st.m;
      s_l[wave * 8 + head] = lt;
      if (!quant_wg) {
#pragma unroll
        for (int G = 0; G < NG; ++G) s_z[(wave * 8 + head) * 4 + G] = 0.0f;
      }
    }
    if (quant_wg && quad == 0 && slot_ok) {
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int G = slot + v * SP;
        if (G < NG) s_z[(wave * 8 + head) * 4 + G] = zt[v];
      }
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      if (quant_wg) {
        constexpr int B2 = BITS > 0 ? BITS : 2;
        const float osc = __builtin_ldexpf(1.0f, 24 - B2 * code_target<B2, Cfg<D, B2>::VWIDE>(ct % Cfg<D, B2>::PPD));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * quad + i;
          const int hp_ = r >> 1, rep_ = hp_ / g;
          const int slot_ = 2 * rep_ + (r & 1);
          if (rep_ < R8 && (ct / 2) % SP == slot_) s_o[(wave * 8 + hp_ % g) * D + 16 * ct + col] = st.O[ct][i] * osc;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const int hp_ = 2 * quad + i / 2;
          if (hp_ < g) s_o[(wave * 8 + hp_) * D + 16 * ct + col] = st.O[ct][i] + st.O[ct][i + 1];
        }
      }
    }
    __syncthreads();
    for (int t = threadIdx.x; t < g * D; t += kThreads) {
      const int h = t / D, d = t % D;
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w * 8 + h]);
      float L = 0.0f, O = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = s_m[w * 8 + h];
        const float f = mw == kNegInf ? 0.0f : fast_exp2(mw - M);
        L += s_l[w * 8 + h] * f;
        O += (s_o[(w * 8 + h) * D + d] + s_z[(w * 8 + h) * 4 + d / 32]) * f;
      }
      const int hq = hk * g + h;
      if (a.direct) {
        a.out[((size_t)b * a.Hq + hq) * D + d] = L > 0.0f ? O / L : 0.0f;
        if (a.lse != nullptr && d == 0) a.lse[(size_t)b * a.Hq + hq] = L > 0.0f ? (M + __log2f(L)) * kLn2 : kNegInf;
      } else {
        float* p = a.ws + (((size_t)part * a.B + b) * a.Hq + hq) * (D + 2);
        p[d] = O;
        if (d == 0) {
          p[D] = M;
          p[D + 1] = L;
        }
      }
    }
  };

  // ---------------------------------------------------------- exact tail
  // (the last workgroups first take a range of the exact rows, as a partial
  // of their own, then a correspondingly smaller range of the compressed part)
  if (split >= a.tail_first && a.T_cap > 0) {
    int tl = a.tail_len[b];
    tl = tl < 0 ? 0 : (tl > a.T_cap ? a.T_cap : tl);
    RowSrc src;
    src.k = a.tail_k;
    src.v = a.tail_v;
    src.idx = nullptr;
    src.unit_row0 = unit_rows * a.T_cap;
    src.n_valid = tl;
    src.bound = a.T_cap;
    const int nb = (tl + 31) / 32;
    const int blo = (split - a.tail_first) * a.tail_bpw;
    const int bhi = min(blo + a.tail_bpw, nb);
    bf16x8 qb[NKS];
    load_qb(qb);
    rows_loop<D, NV>(src, blo + wave, bhi, qb, a.scale_log2, vst, st, lane, col, quad, hilo);
    finish(a.main_splits + split - a.tail_first, false);
    st.clear();
    __syncthreads();  // the epilogue's LDS is reused below
  }

  {
    // ------------------------------------------------ the compressed part
    const int nb = (a.n_main + 31) / 32;
    const int before = min(split, a.tail_first);
    const int blo = before * a.main_bpw + (split - before) * a.main_bpw_t;
    const int bhi = min(blo + (split < a.tail_first ? a.main_bpw : a.main_bpw_t), nb);
    if constexpr (BITS > 0) {
      // ---------------------------------------------------------------- quant
      // q scaled per k slot (f16, exact): qF = q 2^(kQExp - bits*jj).  The zero-
      // point product needs q itself: for int4 that is qF (jj is 1), for int2
      // it comes from a workgroup table in LDS.
      // q in the codes' channel order: k-step ks, channels quad * D/4 + 8 ks .. + 7
      u32x4 qraw[NKS];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        qraw[ks] = *reinterpret_cast<const u32x4*>(qhead + quad * (D / 4) + 8 * ks);
      uint32_t qF[NKS][4];
      uint32_t* zero = reinterpret_cast<uint32_t*>(smem + C::ZERO_OFF);
      // [ks][quad][head][4]: a quad's heads in consecutive 16-byte chunks
      uint32_t* qzt = reinterpret_cast<uint32_t*>(smem + C::QZ_OFF);
      {
        const uint16_t* qh = reinterpret_cast<const uint16_t*>(qraw);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          u32x4 z4;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int pi = 4 * ks + i, d = pi / C::PPD, j = pi % C::PPD;
            const int ca = C::CPD * d + j, cb = ca + C::CPD / 2;
            const float xa = bf16_to_f32(qh[ca]), xb = bf16_to_f32(qh[cb]);
            const float f = __builtin_ldexpf(1.0f, kQExp - BITS * code_target<BITS, true>(j));
            const f16x2 pf = {(_Float16)(xa * f), (_Float16)(xb * f)};
            const f16x2 pz = {(_Float16)xa, (_Float16)xb};
            qF[ks][i] = __builtin_bit_cast(uint32_t, pf);
            z4[i] = __builtin_bit_cast(uint32_t, pz);
          }
          if (BITS == 2 && wave == 0 && rep == 0 && hilo == 0)
            *reinterpret_cast<u32x4*>(qzt + ((ks * 4 + quad) * 8 + head) * 4) = z4;
        }
      }
      for (int i = threadIdx.x; i < C::ZERO_BYTES / 4; i += kThreads) zero[i] = 0u;
      __syncthreads();

      // This wavefront's blocks stream through a ring of DEPTH LDS slots filled
      // by direct global->LDS loads, DEPTH-1 blocks ahead of the block in use:
      // no registers hold data in flight, and the metadata arrive already in
      // the order the matrix-core operands read them.  All addressing of the
      // loads is wave-uniform (scalar registers) plus the lane's 16-byte offset.
      const int nq32 = a.q_cap / 32;
      const int wave_u = __builtin_amdgcn_readfirstlane(wave);
      const unsigned char* kcodes = a.k_codes + unit_rows * nq32 * C::KC_BYTES;
      const unsigned char* vcodes = a.v_codes + unit_rows * nq32 * C::VC_BYTES;
      const unsigned char* kmeta = reinterpret_cast<const unsigned char*>(a.k_meta) + unit_rows * nq32 * C::KM_BYTES;
      const unsigned char* vmeta = reinterpret_cast<const unsigned char*>(a.v_meta) + unit_rows * nq32 * C::VM_BYTES;
      const unsigned char* ring = smem + wave * C::RING_WAVE;
      const uint32_t ring_lds = lds_address(smem) + wave_u * C::RING_WAVE;
      const uint32_t voff = 16 * lane;
      const int first = blo + wave_u;
      const int nw = first < bhi ? (bhi - first + kWaves - 1) / kWaves : 0;  // blocks of this wavefront
      auto issue = [&](int k) {
        const size_t blk = (size_t)(first + kWaves * k);
        const uint32_t sl = ring_lds + (k % C::DEPTH) * C::SLOT;
        lds_dma<C::KC_BYTES>(kcodes + blk * C::KC_BYTES, voff, sl, lane);
        lds_dma<C::VC_BYTES>(vcodes + blk * C::VC_BYTES, voff, sl + C::VC_OFF, lane);
        lds_dma<C::KM_BYTES>(kmeta + blk * C::KM_BYTES, voff, sl + C::KM_OFF, lane);
        lds_dma<C::VM_BYTES>(vmeta + blk * C::VM_BYTES, voff, sl + C::VM_OFF, lane);
      };
#pragma unroll
      for (int k = 0; k < C::DEPTH - 1; ++k)
        if (k < nw) issue(k);
      // operand of the rounded product q~hi = qF s: the block's scales in the lo
      // columns, zeros in the hi columns (whose q~ is then RN(qF s) itself)
      const int tsel = hilo ? 1 : 0;

      for (int k = 0; k < nw; ++k) {
        if (k + C::DEPTH - 1 < nw) {
          wait_lds_reads();  // the slot being refilled was last read in the previous iteration
          issue(k + C::DEPTH - 1);
        }
        // block k has landed once at most the loads of the blocks after it are outstanding
        const int ahead = min(nw - 1 - k, C::DEPTH - 1);
        if (ahead >= 3) wait_vmem<3 * C::NDMA>();
        else if (ahead == 2) wait_vmem<2 * C::NDMA>();
        else if (ahead == 1) wait_vmem<C::NDMA>();
        else wait_vmem<0>();
        const unsigned char* sl = ring + (k % C::DEPTH) * C::SLOT;
        const uint32_t* sp = reinterpret_cast<const uint32_t*>(sl + C::KM_OFF);  // [4 quads][NKS][4] scale pairs
        const uint32_t* zp = sp + 16 * NKS;                                     // [4][NKS][4] zero pairs
        const uint32_t* vm = reinterpret_cast<const uint32_t*>(sl + C::VM_OFF);  // [NG][4 quads][8] {scale, zero}
        const uint32_t* tp = tsel ? sp : zero;

        // q~ = hi or lo part of qF * s_K, and the K zero-point product z . q
        f32x4 accZ = {0.f, 0.f, 0.f, 0.f};
        f16x8 qt[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const int o = (quad * NKS + ks) * 4;
          const u32x4 z4 = *reinterpret_cast<const u32x4*>(zp + o);
          u32x4 qz4;
          if constexpr (BITS == 4) {
            qz4 = u32x4{qF[ks][0], qF[ks][1], qF[ks][2], qF[ks][3]};
          } else {
            qz4 = *reinterpret_cast<const u32x4*>(qzt + ((ks * 4 + quad) * 8 + head) * 4);
          }
          accZ = mfma_f16(__builtin_bit_cast(f16x8, z4), __builtin_bit_cast(f16x8, qz4), accZ);
          const u32x4 s4 = *reinterpret_cast<const u32x4*>(sp + o);
          const u32x4 t4 = *reinterpret_cast<const u32x4*>(tp + o);
          u32x4 r4;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            // (bit-casting the subscript s4[i] directly reads element 0: copy it out first)
            const uint32_t sw = s4[i], tw = t4[i];
            const f16x2 sv = __builtin_bit_cast(f16x2, sw);
            const f16x2 qf = __builtin_bit_cast(f16x2, qF[ks][i]);
            const f16x2 t = qf * __builtin_bit_cast(f16x2, tw);  // RN(qF s) or 0
            r4[i] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(qf, sv, -t));  // hi or lo
          }
          qt[ks] = __builtin_bit_cast(f16x8, r4);
        }
        // code part of q.k for tokens col and 16 + col; hi + lo columns summed
        const float code_scale = 0x1p20f * a.scale_log2;  // undoes 2^-24 (codes) * 2^kQExp (q)
        const float zpart = fmaf(accZ[0], a.scale_log2, -st.mu);  // rows of accZ all hold z . q
        float x[8];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          uint32_t kw[C::KDW];
          load_dwords<C::KDW>(sl + (16 * tt + col) * C::ROW_BYTES + quad * (C::ROW_BYTES / 4), kw);
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            u32x4 a4;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int pi = 4 * ks + i;
              a4[i] = code_pair<BITS, true>(kw[pi / C::PPD], pi % C::PPD);
            }
            acc = mfma_f16(__builtin_bit_cast(f16x8, a4), qt[ks], acc);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float v = acc[i] + swap_adjacent(acc[i]);
            x[4 * tt + i] = fmaf(v, code_scale, zpart);
          }
        }
        float P[8];
        softmax_block<NCT, NV>(x, st, P, quad);
        // A operands: hi and lo of P * s_V for this lane's channel group(s);
        // hi = RN_f16(P s), lo = RN_f16(P s - hi), each one mixed-precision fma
        f16x8 Ahi[NV], Alo[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          const int G = slot + v * SP;
          const bool gok = slot_ok && G < NG;
          const uint32_t* vmg = gok ? vm + (G * 4 + quad) * 8 : zero;
          const u32x4 m0 = *reinterpret_cast<const u32x4*>(vmg);
          const u32x4 m1 = *reinterpret_cast<const u32x4*>(vmg + 4);
          const uint32_t mm[8] = {m0[0], m0[1], m0[2], m0[3], m1[0], m1[1], m1[2], m1[3]};
          // hi = RN_f16 of the fp32 product P s (two per packed conversion); lo =
          // RN_f16 of the residual P s - hi, taken in one fma against the rounded
          // hi, so that hi + lo carries P s to about 22 significant bits.
          float zs = 0.0f;
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const f16x2 s0 = __builtin_bit_cast(f16x2, mm[e]), s1 = __builtin_bit_cast(f16x2, mm[e + 1]);
            const f32x2 h32 = {fmaf(P[e], (float)s0[0], -0.0f), fmaf(P[e + 1], (float)s1[0], -0.0f)};
            const f16x2 h = __builtin_convertvector(h32, f16x2);
            const f32x2 l32 = {fmaf(P[e], (float)s0[0], -(float)h[0]), fmaf(P[e + 1], (float)s1[0], -(float)h[1])};
            const f16x2 lo = __builtin_convertvector(l32, f16x2);
            Ahi[v][e] = h[0];
            Ahi[v][e + 1] = h[1];
            Alo[v][e] = lo[0];
            Alo[v][e + 1] = lo[1];
            zs = fmaf(P[e], (float)s0[1], zs);
            zs = fmaf(P[e + 1], (float)s1[1], zs);
          }
          st.zacc[v] += zs;
        }
        // P.V code part
        uint32_t vw[C::VDW];
        load_dwords<C::VDW>(sl + C::VC_OFF + lane * (C::VDW * 4), vw);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const int v = NV == 1 ? 0 : ct / 4;
          u32x4 b4;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int pi = i * NCT + ct;
            b4[i] = code_pair<BITS, C::VWIDE>(vw[pi / C::PPD], pi % C::PPD);
          }
          st.O[ct] = mfma_f16(Ahi[v], __builtin_bit_cast(f16x8, b4), st.O[ct]);
          st.O[ct] = mfma_f16(Alo[v], __builtin_bit_cast(f16x8, b4), st.O[ct]);
        }
      }
    } else {
      // ---------------------------------------------------- exact rows (main)
      RowSrc src;
      src.k = a.k_full;
      src.v = a.v_full;
      src.idx = a.keep_idx != nullptr ? a.keep_idx + unit_rows * a.n_main : nullptr;
      src.unit_row0 = unit_rows * a.L_cap;
      src.n_valid = a.n_main;
      src.bound = a.row_bound;
      bf16x8 qb[NKS];
      load_qb(qb);
      rows_loop<D, NV>(src, blo + wave, bhi, qb, a.scale_log2, vst, st, lane, col, quad, hilo);
    }
  }
  finish(split, true);
}

// Merge the split partials (o unnormalised, m in log2 units, l) of one (b, h)
// row per workgroup, one thread per channel.  The channel values of the first
// kCombineChunk splits are loaded while the splits' maxima and sums go to LDS,
// so that up to kCombineChunk splits cost one memory latency and one barrier.
constexpr int kCombineChunk = 16;
constexpr int kMaxCombineSplits = 256;
// g_affine > 0: the rows of unit u (g_affine query heads each) are merged on
// XCD u % 8, where the draft kernel's XCD-affine grid wrote their partials.
__global__ __launch_bounds__(128) void draft_combine_kernel(const float* __restrict__ ws, int splits, int rows,
                                                            int D, float* __restrict__ out,
                                                            float* __restrict__ lse, int g_affine) {
  __shared__ float s_m[kMaxCombineSplits], s_l[kMaxCombineSplits];
  int row = blockIdx.x;
  if (g_affine > 0) {
    const int x8 = row % 8, y = row / 8;
    row = ((y / g_affine) * 8 + x8) * g_affine + y % g_affine;
  }
  const int d = threadIdx.x;
  float o[kCombineChunk];
#pragma unroll
  for (int j = 0; j < kCombineChunk; ++j)
    o[j] = j < splits ? ws[((size_t)j * rows + row) * (D + 2) + d] : 0.0f;
  for (int sp = d; sp < splits; sp += blockDim.x) {
    const float* p = ws + ((size_t)sp * rows + row) * (D + 2);
    s_m[sp] = p[D];
    s_l[sp] = p[D + 1];
  }
  __syncthreads();
  float M = kNegInf;
  for (int sp = 0; sp < splits; ++sp) M = fmaxf(M, s_m[sp]);
  float L = 0.0f, O = 0.0f;
  if (M != kNegInf) {
#pragma unroll
    for (int j = 0; j < kCombineChunk; ++j) {
      if (j < splits) {
        const float w = s_m[j] == kNegInf ? 0.0f : fast_exp2(s_m[j] - M);
        L = fmaf(s_l[j], w, L);
        O = fmaf(o[j], w, O);
      }
    }
    for (int sp = kCombineChunk; sp < splits; ++sp) {
      const float w = s_m[sp] == kNegInf ? 0.0f : fast_exp2(s_m[sp] - M);
      L = fmaf(s_l[sp], w, L);
      O = fmaf(ws[((size_t)sp * rows + row) * (D + 2) + d], w, O);
    }
  }
  out[(size_t)row * D + d] = L > 0.0f ? O / L : 0.0f;
  if (lse != nullptr && d == 0) lse[row] = L > 0.0f ? (M + __log2f(L)) * kLn2 : kNegInf;
}

// Workspace: the split partials.
size_t draft_ws_need(int B, int Hq, int Hkv, int D, int splits) {
  (void)Hkv;
  const size_t need = (size_t)splits * B * Hq * (D + 2) * sizeof(float);
  return need < 256 ? 256 : need;
}

struct DraftPlan {
  int main_splits, main_bpw, main_bpw_t, tail_first, tail_bpw, splits;
};

constexpr int kTailBpw = 2 * kWaves;  // exact tail blocks per workgroup: up to 2 per wavefront

// Time of one exact-row block (bf16, loaded straight to registers, latency-
// bound when taken alone) per wavefront, in quarters of one block of the
// compressed part (measured on MI355X: about 3.25 int2 blocks, 2.5 int4 blocks;
// an exact-row main part costs the same per block).
inline int tail_block_cost_q4(int bits) { return bits == 2 ? 13 : bits == 4 ? 10 : 4; }

// wgs_per_cu: resident workgroups per CU of the kernel that will run.  Every
// resident slot runs compressed blocks.  The exact tail goes to the last
// workgroups of each (batch, kv-head), which take it first, as a partial of its
// own, and then correspondingly fewer compressed blocks, so that all
// workgroups finish together.
DraftPlan plan_draft(int units, int main_blocks, int tail_blocks, int wgs_per_cu, int bits) {
  DraftPlan p{};
  int s = wgs_per_cu * num_cus() / units;
  const int cap = (main_blocks + 2 * kWaves - 1) / (2 * kWaves);  // >= 2 blocks per wavefront
  if (s > cap) s = cap;
  if (s < 1) s = 1;
  int t = tail_blocks > 0 ? (tail_blocks + kTailBpw - 1) / kTailBpw : 0;
  if (t > s) s = t;
  p.main_splits = s;
  p.tail_first = s - t;
  p.tail_bpw = t > 0 ? (tail_blocks + t - 1) / t : 0;
  // compressed blocks a tail workgroup gives up: the tail's rounds (one block
  // per wavefront each) times the cost of a round in compressed blocks
  const int cut = (tail_block_cost_q4(bits) * kWaves * ((p.tail_bpw + kWaves - 1) / kWaves) + 3) / 4;
  p.main_bpw = (main_blocks + t * cut + s - 1) / s;
  p.main_bpw_t = p.main_bpw > cut ? p.main_bpw - cut : 0;
  if (t == 0) p.main_bpw_t = p.main_bpw;
  // the tail workgroups may have taken less than their share: the others cover the rest
  while ((long long)p.tail_first * p.main_bpw + (long long)t * p.main_bpw_t < main_blocks) ++p.main_bpw;
  p.splits = s + t;
  return p;
}

typedef void (*DraftKernel)(DraftArgs);

template <int D, int NV>
DraftKernel pick_kernel(int bits) {
  if (bits == 4) return draft_mfma_kernel<D, 4, NV>;
  if (bits == 2) return draft_mfma_kernel<D, 2, NV>;
  return draft_mfma_kernel<D, 0, 1>;
}

// Resident workgroups per CU of kernel k (cached per kernel and device).
int wgs_per_cu(DraftKernel k) {
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, int> cache;
  int dev = 0;
  (void)hipGetDevice(&dev);
  std::lock_guard<std::mutex> lk(mu);
  auto key = std::make_pair(reinterpret_cast<const void*>(k), dev);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k, kThreads, 0) != hipSuccess || n < 1) n = 2;
  cache[key] = n;
  return n;
}

}  // namespace
}  // namespace vc

using namespace vc;

extern "C" size_t vc_draft_ws_bytes(int B, int Hq, int Hkv, int D, int max_keys) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || max_keys < 0) return 0;
  // upper bound over every split of max_keys between the compressed part and the tail
  const int nb = (max_keys + 31) / 32;
  // (one more tail workgroup than the worst split of max_keys could need)
  const DraftPlan p = plan_draft(B * Hkv, nb, 0, 8, 0);  // 8 resident workgroups per CU bound any kernel
  const int s = p.main_splits + 2 * ((nb + kTailBpw - 1) / kTailBpw) + 1;
  return draft_ws_need(B, Hq, Hkv, D, s);
}

// Validates, plans and launches one draft step.  ws/ws_bytes: the split
// partials' buffer (caller's workspace, or the file-scope scratch array for
// the allocation-free entry point, which reports its own limit).
static int draft_launch(const char* fn, bool scratch_ws, const vc_kv_comp* comp, const vc_tail* tail,
                        const void* q, float* out, float* lse, int B, int Hq, int Hkv, int D, float scale,
                        void* ws, size_t ws_bytes, hipStream_t stream) {
  VC_CHECK(comp != nullptr && q != nullptr && out != nullptr, "%s: null comp/q/out", fn);
  VC_CHECK(B > 0 && Hq > 0 && Hkv > 0 && Hq % Hkv == 0, "%s: bad B/Hq/Hkv (%d,%d,%d)", fn, B, Hq, Hkv);
  if (D != 64 && D != 128) return fail(VC_ERR_UNSUPPORTED, "%s: D=%d not in {64,128}", fn, D);
  const int g = Hq / Hkv;
  if (g > 8) return fail(VC_ERR_UNSUPPORTED, "%s: GQA group %d > 8", fn, g);
  VC_CHECK(aligned(q, 16) && aligned(out, 16), "%s: q/out must be 16-byte aligned", fn);
  DraftArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.out = out;
  a.lse = lse;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.g = g;
  a.scale_log2 = scale * kLog2e;
  int bits = 0;
  switch (comp->kind) {
    case VC_KV_QUANT:
      VC_CHECK(comp->bits == 2 || comp->bits == 4, "%s: bits must be 2 or 4 (got %d)", fn, comp->bits);
      VC_CHECK(comp->n_quant >= 0 && comp->n_quant % 32 == 0, "%s: n_quant=%d not a multiple of 32", fn,
               comp->n_quant);
      VC_CHECK(comp->n_quant == 0 || (comp->k_codes && comp->v_codes && comp->k_meta && comp->v_meta),
               "%s: null codes/meta", fn);
      VC_CHECK(aligned(comp->k_codes, 16) && aligned(comp->v_codes, 16) && aligned(comp->k_meta, 16) &&
                   aligned(comp->v_meta, 16),
               "%s: codes and meta must be 16-byte aligned", fn);
      VC_CHECK(quant_cap(comp) >= comp->n_quant && quant_cap(comp) % 32 == 0,
               "%s: q_cap=%d below n_quant=%d or not a multiple of 32", fn, comp->q_cap, comp->n_quant);
      bits = comp->bits;
      a.q_cap = quant_cap(comp);
      a.n_main = comp->n_quant;
      a.k_codes = comp->k_codes;
      a.v_codes = comp->v_codes;
      a.k_meta = static_cast<const uint32_t*>(comp->k_meta);
      a.v_meta = static_cast<const uint32_t*>(comp->v_meta);
      break;
    case VC_KV_IDENTITY:
    case VC_KV_TOKEN_DROP:
      VC_CHECK(comp->L_cap >= 0, "%s: bad L_cap", fn);
      VC_CHECK(comp->L_full >= 0 && comp->L_full <= comp->L_cap, "%s: L_full=%d outside [0, L_cap=%d]", fn,
               comp->L_full, comp->L_cap);
      if (comp->kind == VC_KV_IDENTITY) {
        a.n_main = comp->L_full;
        a.keep_idx = nullptr;
      } else {
        VC_CHECK(comp->n_keep >= 0, "%s: bad n_keep", fn);
        VC_CHECK(comp->n_keep == 0 || comp->keep_idx != nullptr, "%s: null keep_idx", fn);
        a.n_main = comp->n_keep;
        a.keep_idx = comp->keep_idx;
      }
      VC_CHECK(a.n_main == 0 || (comp->k_full && comp->v_full), "%s: null k_full/v_full", fn);
      VC_CHECK(aligned(comp->k_full, 16) && aligned(comp->v_full, 16), "%s: k_full/v_full misaligned", fn);
      a.k_full = static_cast<const uint16_t*>(comp->k_full);
      a.v_full = static_cast<const uint16_t*>(comp->v_full);
      a.L_cap = comp->L_cap;
      a.row_bound = comp->L_full;
      break;
    default:
      return fail(VC_ERR_INVALID, "%s: unknown compressor kind %d", fn, comp->kind);
  }
  if (tail != nullptr && tail->T_cap > 0) {
    VC_CHECK(tail->k && tail->v && tail->len, "%s: null tail pointers", fn);
    VC_CHECK(aligned(tail->k, 16) && aligned(tail->v, 16), "%s: tail misaligned", fn);
    a.tail_k = static_cast<const uint16_t*>(tail->k);
    a.tail_v = static_cast<const uint16_t*>(tail->v);
    a.tail_len = tail->len;
    a.T_cap = tail->T_cap;
  } else {
    VC_CHECK(tail == nullptr || tail->T_cap == 0, "%s: negative T_cap", fn);
    a.T_cap = 0;
  }
  const int units = B * Hkv;
  const int main_blocks = (a.n_main + 31) / 32;
  const int tail_blocks = (a.T_cap + 31) / 32;
  // two V-group variants per lane are needed when fewer than NG slots exist per head
  const int NG = D / 32, SP = 2 * (8 / g);
  const int nv = bits > 0 && SP < NG ? 2 : 1;
  const DraftKernel kern = D == 128 ? (nv == 2 ? pick_kernel<128, 2>(bits) : pick_kernel<128, 1>(bits))
                                    : pick_kernel<64, 1>(bits);
  const DraftPlan p = plan_draft(units, main_blocks, tail_blocks, wgs_per_cu(kern), bits);
  VC_CHECK(p.splits <= kMaxCombineSplits, "%s: %d splits exceed %d", fn, p.splits, kMaxCombineSplits);
  const size_t need = draft_ws_need(B, Hq, Hkv, D, p.splits);
  if (p.splits > 1) {
    if (scratch_ws && need > ws_bytes)
      return fail(VC_ERR_UNSUPPORTED, "%s: this call needs %zu bytes of split partials, above the %zu-byte "
                  "scratch array (use vc_draft_attn with a workspace)", fn, need, ws_bytes);
    if (ws == nullptr || ws_bytes < need)
      return fail(VC_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
    VC_CHECK(aligned(ws, 16), "%s: workspace misaligned", fn);
    a.ws = static_cast<float*>(ws);
  }
  a.main_splits = p.main_splits;
  a.main_bpw = p.main_bpw;
  a.main_bpw_t = p.main_bpw_t;
  a.tail_first = p.tail_first;
  a.tail_bpw = p.tail_bpw;
  a.splits = p.splits;
  a.direct = p.splits == 1;
  a.xcd_affine = units % 8 == 0 ? 1 : 0;
  if (a.xcd_affine) {
    VC_CHECK((long long)p.main_splits * units < (1LL << 31), "%s: grid too large", fn);
    kern<<<dim3(p.main_splits * units), kThreads, 0, stream>>>(a);
  } else {
    kern<<<dim3(p.main_splits, units), kThreads, 0, stream>>>(a);
  }
  VC_HIP(hipGetLastError());
  if (p.splits > 1) {
    draft_combine_kernel<<<B * Hq, D, 0, stream>>>(a.ws, p.splits, B * Hq, D, out, lse, a.xcd_affine ? g : 0);
    VC_HIP(hipGetLastError());
  }
  return VC_OK;
}

extern "C" int vc_draft_attn(const vc_kv_comp* comp, const vc_tail* tail, const void* q, float* out,
                             float* lse, int B, int Hq, int Hkv, int D, float scale, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  return draft_launch("vc_draft_attn", false, comp, tail, q, out, lse, B, Hq, Hkv, D, scale, ws, ws_bytes, stream);
}

// ------------------------------------------------------------------------
// Allocation-free draft: the split partials live in a file-scope device array
// (one copy per GPU, held until the process ends).  In host code `scratch`
// names a host-side stand-in, never the device copy: its device address is
// taken once per device with hipGetSymbolAddress and only that address is
// handed to kernels.  The partials need no clearing: every slot a combine
// reads is written by the same call first.
constexpr size_t kScratchBytes = VC_DRAFT_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

static int scratch_ptr(void** out) {
  static std::mutex mu;
  static std::map<int, void*> ptrs;
  int dev = 0;
  VC_HIP(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lk(mu);
  auto it = ptrs.find(dev);
  if (it == ptrs.end()) {
    void* p = nullptr;
    VC_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    VC_CHECK(p != nullptr && aligned(p, 256), "vc_draft_attn_noalloc: scratch array has no usable device address");
    it = ptrs.emplace(dev, p).first;
  }
  *out = it->second;
  return VC_OK;
}

extern "C" int vc_draft_attn_noalloc(const vc_kv_comp* comp, const vc_tail* tail, const void* q, float* out,
                                     float* lse, int B, int Hq, int Hkv, int D, float scale, hipStream_t stream) {
  void* ws = nullptr;
  const int rc = scratch_ptr(&ws);
  if (rc != VC_OK) return rc;
  return draft_launch("vc_draft_attn_noalloc", true, comp, tail, q, out, lse, B, Hq, Hkv, D, scale, ws,
                      kScratchBytes, stream);
}
