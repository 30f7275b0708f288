// Causal verify attention over the full bf16 cache on gfx950 matrix cores.
//
// [VC Core Algorithm: one forward pass with KV_full verifies all drafted
//  tokens in parallel; VC Key System Innovations P1: verification is
//  interconnect-bound and compute-bound]
//
// The g query heads of a GQA group times the n_q positions form R = g * n_q
// query rows that share one KV head, so q.K^T and P.V are real contractions.
// Per 32-key tile a workgroup (4 or 8 wavefronts) stages K (bf16) and V
// (converted to f16) in LDS once, rows XOR-swizzled; every wavefront owns up to
// MT 16-row query tiles and computes, for each,
//   S[32 keys x 16 rows] = K . Q^T   (bf16 MFMA: keys are the A rows, so each
//                                     lane ends up with 8 keys of one row)
//   online softmax per row in fp32 (lazy rescale, running max moves by >= 2^8)
//   O[16 rows x D]     += P . V      (f16 MFMA; P rounded to nearest even; V
//                                     read transposed with ds_read_b64_tr_b16)
// The K and V operands of a tile are read from LDS once per wavefront and
// shared by its query tiles.  The tiles stream through a ring of kDepth LDS
// slots by direct global->LDS loads issued kDepth - 1 tiles ahead, with one
// barrier per tile, so the next tiles' loads are in flight during this tile's
// math.
// A workgroup has 8 wavefronts when 4 cannot hold every query tile (a GQA group
// of 8 at k = 32 has 17), so that the cache is read from HBM once.  Query rows
// beyond 3 tiles per wavefront go to further row groups, laid out so that the
// row groups of one key range run on the same XCD.
#include <map>
#include <mutex>
#include <type_traits>

#include "lds_dma.h"
#include "mfma.h"
#include "vc_common.h"

namespace vc {
namespace {

constexpr int kWaves = 4;     // wavefronts per workgroup, or 2 * kWaves for many query tiles
constexpr int kKT = 32;       // keys per tile
constexpr int kMaxMT = 3;     // query tiles per wavefront
constexpr int kDepth = 4;     // K/V tiles in the LDS ring
constexpr float kTau = 8.0f;  // lazy rescale threshold (log2 units)

struct VerifyArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  int L_cap;
  const int32_t* page_table;
  int page_log2;
  int pages_per_seq;
  int n_slots;
  const int32_t* ctx_len;
  int max_ctx;
  float* out;
  float* ws;
  int B, Hq, Hkv, g, n_q, R, NT;
  int rowgroups, tiles_per_group;  // query tiles per workgroup <= NW * MT
  int splits, keys_per_split;
  int key_begin, key_limit;        // keys [key_begin, key_limit) of every sequence, clipped to ctx_len + n_q
  int key_lo;                      // keys below key_lo are masked (key_begin rounded down for paged loads)
  int write_partials;              // 1: always write split partials to ws (range calls), never the output
  int n_su;                        // splits * units
  float scale_log2;
};

// 8 bf16 (one 16-byte chunk) -> 8 f16, round to nearest even.
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 w) {
  u32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const f16x2 h = {(_Float16)bf16_lo(w[e]), (_Float16)bf16_hi(w[e])};
    r[e] = __builtin_bit_cast(uint32_t, h);
  }
  return r;
}

// The XOR key of key row `row` in the LDS tile layout: 16-byte chunk c of the
// row sits at chunk position c ^ swz(row).  Chosen so that both operand reads
// hit distinct banks: a K read (16 consecutive rows, one chunk each) needs
// distinct keys per 256-byte bank window, a transposed V read (8 consecutive
// rows, an aligned chunk pair each) distinct keys >> 1.  With 256-byte rows
// (D = 128) rotating the row's low 4 bits left by one does both (row % 16
// alone maps rows r and r ^ 1 onto the same chunk pair); with 128-byte rows
// (D = 64, two rows per window) rows of one parity must differ.
template <int CPR>
__device__ __forceinline__ int swz(int row) {
  if constexpr (CPR == 16) return ((row << 1) | ((row >> 3) & 1)) & 15;
  else return ((row >> 1) & 3) << 1 | ((row >> 3) & 1);
}

template <int D, int MT, bool PAGED, int NW>
__global__ __launch_bounds__(64 * NW) void verify_mfma_kernel(VerifyArgs a) {
  constexpr int NKS = D / 32, NCT = D / 16;
  constexpr int CPR = D / 8;                      // 16-byte chunks per key row
  constexpr int TILE = kKT * D * 2;               // bytes of one K or V tile
  // wavefronts that stage tiles (one 1 KiB load instruction each per round)
  constexpr int LW = TILE / 1024 < NW ? TILE / 1024 : NW;
  constexpr int ROUNDS = TILE / (1024 * LW);      // direct loads per staging thread per tile and tensor
  static_assert(TILE % (1024 * LW) == 0, "a tile is whole rounds of 16-byte loads");
  constexpr int NDMA = 2 * ROUNDS;                // load instructions per staging thread per tile
  // ring of kDepth K tiles, then kDepth V tiles (bf16 as loaded, f16 once converted)
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * kDepth * TILE];

  // workgroup -> (row group, split, unit): the row groups of one (split, unit)
  // are 8 workgroups apart, i.e. on the same XCD under round-robin dispatch
  const int id = blockIdx.x;
  const int x8 = id % 8, y = id / 8;
  const int rg = y % a.rowgroups;
  const int su = (y / a.rowgroups) * 8 + x8;
  if (su >= a.n_su) return;
  const int split = su % a.splits, unit = su / a.splits;
  const int b = unit / a.Hkv, hk = unit % a.Hkv;
  const int lane = threadIdx.x & 63;
  // wave-uniform (scalar) so that the tile guards below are scalar branches
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, quad = lane >> 4;

  int ctx = a.ctx_len[b];
  ctx = ctx < 0 ? 0 : (ctx > a.max_ctx ? a.max_ctx : ctx);
  const int key_end = min(ctx + a.n_q, a.key_limit);
  const int kb = a.key_begin + split * a.keys_per_split;
  const int ke = min(kb + a.keys_per_split, key_end);

  // this wavefront's query tiles: tile0 + wave + NW * i
  const int tile0 = rg * a.tiles_per_group;
  const int tile_end = min(tile0 + a.tiles_per_group, a.NT);
  bf16x8 qb[MT][NKS];
  f32x4 O[MT][NCT];
  // m: running max (log2 units, -inf until a key is seen); mu: the offset the
  // scores are taken relative to (m, or 0 while m is -inf); thr: the amount a
  // block max must exceed to move m (-inf while m is -inf, else kTau)
  float m[MT], l[MT], mu[MT], thr[MT];
  int rlim[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int tile = tile0 + wave + NW * i;
    const int r = tile * 16 + col;
    rlim[i] = -1;
    if (tile < tile_end && r < a.R) {
      const int hl = r / a.n_q, j = r % a.n_q;
      rlim[i] = ctx + j;
      const uint16_t* qp = a.q + ((size_t)(b * a.Hq + hk * a.g + hl) * a.n_q + j) * D + quad * (D / 4);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) qb[i][ks] = *reinterpret_cast<const bf16x8*>(qp + 8 * ks);
    } else {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) qb[i][ks] = bf16x8{};
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) O[i][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[i] = kNegInf;
    mu[i] = 0.0f;
    thr[i] = kNegInf;
    l[i] = 0.0f;
  }
  settle_compiler_loads();  // q is in registers before the key loop starts
  int n_live = 0;  // live query tiles of this wavefront (MT or MT - 1 by the plan)
#pragma unroll
  for (int i = 0; i < MT; ++i) n_live += tile0 + wave + NW * i < tile_end ? 1 : 0;

  // Staging: tile t's K and V go to ring slot t % kDepth by direct 16-byte
  // global->LDS loads issued kDepth - 1 tiles ahead; no registers hold them in flight.
  // In round r a thread of staging wavefront wave < LW fills LDS chunk
  // s = (r * LW + wave) * 64 + lane
  // of the tile, which holds 16-byte chunk (s % CPR) ^ swz(key) of key row
  // key = s / CPR: the XOR swizzle makes the operand reads below conflict-free.
  // One load instruction covers 64 / CPR consecutive rows (4 or 8) starting at
  // a multiple of that count: tiles start at key_begin + 32 n and a paged
  // call's key_begin is a multiple of 8, so those rows lie in one page (pages
  // hold a power-of-two count >= 8 of rows) and one scalar page lookup serves
  // the whole instruction.
  const uint32_t lds0 = lds_address(smem);
  const unsigned char* kv8 = reinterpret_cast<const unsigned char*>(a.k);
  const unsigned char* vv8 = reinterpret_cast<const unsigned char*>(a.v);
  const size_t unit_row0 = (size_t)(b * a.Hkv + hk) * a.L_cap;
  const int page_rows = 1 << a.page_log2;
  const size_t page_bytes = (size_t)a.Hkv * 2 * page_rows * D * 2;
  using cptr = const __attribute__((address_space(4))) int32_t*;  // scalar reads: uniform indices
  const cptr ptab = (cptr)(a.page_table);
  uint32_t zfill = 0;  // bit (slot * ROUNDS + r): that round of that ring slot reads as zeros
  auto issue = [&](int t) __attribute__((always_inline)) {
    if (LW < NW && wave >= LW) return;
    const int t0 = kb + t * kKT;
    const int sl = t % kDepth;
    const uint32_t kl = lds0 + sl * TILE, vl = lds0 + (kDepth + sl) * TILE;
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
      const int s = (r * LW + wave) * 64 + lane;
      const int row = s / CPR, cc = (s % CPR) ^ swz<CPR>(row);
      // rows past the split's range are clamped to its last row (masked later)
      const int key = min(t0 + row, ke - 1);
      const unsigned char *kp, *vp;
      if constexpr (PAGED) {
        const int key0 = min(t0 + (r * LW + wave) * (64 / CPR), ke - 1);  // wave-uniform
        int pslot = ptab[(size_t)b * a.pages_per_seq + (key0 >> a.page_log2)];
        const bool bad = pslot < 0 || pslot >= a.n_slots;
        const uint32_t bit = 1u << (sl * ROUNDS + r);
        zfill = bad ? (zfill | bit) : (zfill & ~bit);
        if (bad) pslot = 0;  // a readable page; the chunk is zero-filled before use
        kp = kv8 + (size_t)pslot * page_bytes +
             ((size_t)(hk * 2) * page_rows + (key & (page_rows - 1))) * D * 2 + cc * 16;
        vp = kp + (size_t)page_rows * D * 2;
      } else {
        kp = kv8 + ((unit_row0 + key) * D) * 2 + cc * 16;
        vp = vv8 + ((unit_row0 + key) * D) * 2 + cc * 16;
      }
      lds_dma16(kp, kl + (r * LW + wave) * 1024);
      lds_dma16(vp, vl + (r * LW + wave) * 1024);
    }
  };
  // once tile u has landed: each lane converts the V chunks it loaded to f16 in
  // place (or zero-fills both chunks of an unreadable page).  Split in a read,
  // issued before the current tile's math, and a write after it, so the LDS
  // read latency hides behind the math.
  auto vread = [&](int u, u32x4 (&vr)[ROUNDS]) __attribute__((always_inline)) {
    if (LW < NW && wave >= LW) return;
    const int sl = u % kDepth;
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r)
      vr[r] = *reinterpret_cast<const u32x4*>(smem + (kDepth + sl) * TILE + ((r * LW + wave) * 64 + lane) * 16);
  };
  auto vwrite = [&](int u, const u32x4 (&vr)[ROUNDS]) __attribute__((always_inline)) {
    if (LW < NW && wave >= LW) return;
    const int sl = u % kDepth;
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
      const int s = (r * LW + wave) * 64 + lane;
      u32x4* vc = reinterpret_cast<u32x4*>(smem + (kDepth + sl) * TILE + s * 16);
      if (PAGED && (zfill >> (sl * ROUNDS + r)) & 1u) {
        *vc = u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(smem + sl * TILE + s * 16) = u32x4{0u, 0u, 0u, 0u};
      } else {
        *vc = bf16x8_to_f16x8(vr[r]);
      }
    }
  };
  // wait until tile u's loads have landed, given the last tile issued so far
  auto wait_tile = [&](int u, int last_issued) __attribute__((always_inline)) {
    const int after = last_issued - u;  // tiles issued after u
    if (after >= 2) wait_vmem<2 * NDMA>();
    else if (after == 1) wait_vmem<NDMA>();
    else wait_vmem<0>();
  };

  const int ntiles = ke > kb ? (ke - kb + kKT - 1) / kKT : 0;
  static_assert(kDepth == 4, "wait_tile covers up to 2 tiles in flight behind the one awaited");
  if (ntiles > 0) {
#pragma unroll
    for (int u = 0; u < kDepth - 1; ++u)
      if (u < ntiles) issue(u);
    wait_tile(0, min(ntiles - 1, kDepth - 2));
    u32x4 vr[ROUNDS];
    vread(0, vr);
    vwrite(0, vr);
  }
  __syncthreads();
  // The key loop, compiled for the number of live query tiles of this
  // wavefront (MT or MT - 1; 0 only when MT is 1): a wavefront computes only
  // its live tiles, and the choice is made once, outside the loop.
  auto key_loop = [&](auto live_c) __attribute__((always_inline)) {
  constexpr int LIVE = decltype(live_c)::value;
  for (int t = 0; t < ntiles; ++t) {
    const int t0 = kb + t * kKT;
    // ring slot (t + 3) % 4 was last read in step t - 1, which ended with a barrier
    if (t + kDepth - 1 < ntiles) {
      wait_lds_reads();
      issue(t + kDepth - 1);
    }
    // tile t + 1: its loads (issued two steps ago) must have landed; read its V
    // chunks now, convert and write them after this tile's math
    u32x4 vnext[ROUNDS];
    const bool has_next = t + 1 < ntiles;
    if (has_next) {
      wait_tile(t + 1, min(ntiles - 1, t + kDepth - 1));
      vread(t + 1, vnext);
    }
    const unsigned char* kt = smem + (t % kDepth) * TILE;
    const unsigned char* vt = smem + (kDepth + t % kDepth) * TILE;
    // the tile's math for this wavefront's LIVE query tiles: no guards
    // inside, so each phase is one straight block the compiler can
    // software-pipeline
    auto compute = [&]() __attribute__((always_inline)) {
      // scores for every query tile; K operands read once, shared by the tiles,
      // each read issued one step ahead of its use
      auto kread = [&](int idx) __attribute__((always_inline)) {
        const int row = 16 * (idx / NKS) + col, c = quad * (CPR / 4) + idx % NKS;
        return *reinterpret_cast<const bf16x8*>(kt + (row * CPR + (c ^ swz<CPR>(row))) * 16);
      };
      f32x4 s[LIVE > 0 ? LIVE : 1][2];
#pragma unroll
      for (int i = 0; i < LIVE; ++i) s[i][0] = s[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      bf16x8 kcur = kread(0);
#pragma unroll
      for (int idx = 0; idx < 2 * NKS; ++idx) {
        bf16x8 knext = kcur;
        if (idx + 1 < 2 * NKS) knext = kread(idx + 1);
        const int h = idx / NKS, ks = idx % NKS;
#pragma unroll
        for (int i = 0; i < LIVE; ++i) s[i][h] = mfma_bf16(kcur, qb[i][ks], s[i][h]);
        kcur = knext;
      }
      // mask only tiles that reach the drafted rows, the end of the range, or
      // start below its first key
      const bool need_mask = t0 + kKT > ctx || t0 + kKT > ke || t0 < a.key_lo;
      f16x8 A[LIVE > 0 ? LIVE : 1];
#pragma unroll
      for (int i = 0; i < LIVE; ++i) {
        float xv[8];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e) xv[4 * h + e] = fmaf(s[i][h][e], a.scale_log2, -mu[i]);
        if (__builtin_expect(need_mask, 0)) {
          // key t0 + 16h + 4q + e is visible iff lo <= 16h + e <= lim
          const int lim = min(rlim[i], ke - 1) - t0 - 4 * quad;
          const int lo = a.key_lo - t0 - 4 * quad;
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (16 * h + e > lim || 16 * h + e < lo) xv[4 * h + e] = kNegInf;
        }
        float tl = xv[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) tl = fmaxf(tl, xv[e]);
        const bool need = tl > thr[i];
        if (__any(need)) {
          float tr = fmaxf(tl, shfl_xor(tl, 16));
          tr = fmaxf(tr, shfl_xor(tr, 32));
          const float mn = fmaxf(m[i], mu[i] + tr);
          const float alpha = mn == kNegInf ? 1.0f : fast_exp2(m[i] - mn);
          l[i] *= alpha;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float ar = __shfl(alpha, 4 * quad + e, 64);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) O[i][ct][e] *= ar;
          }
          const float delta = mn == kNegInf ? 0.0f : mn - mu[i];
#pragma unroll
          for (int e = 0; e < 8; ++e) xv[e] -= delta;
          m[i] = mn;
          mu[i] = mn == kNegInf ? 0.0f : mn;
          thr[i] = mn == kNegInf ? kNegInf : kTau;
        }
        float ps = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = fast_exp2(xv[e]);
          ps += p;
          A[i][e] = (_Float16)p;  // round to nearest even
        }
        l[i] += ps;
      }
      // P . V: V operands read once per column tile (transposed), shared by the
      // query tiles, each read issued one column tile ahead of its use
      auto vload = [&](int ct) __attribute__((always_inline)) {
        const int c = 2 * ct + ((col & 3) >> 1);
        const int r0 = 4 * quad + (col >> 2), r1 = r0 + 16;
        const uint16_t* p0 =
            reinterpret_cast<const uint16_t*>(vt + (r0 * CPR + (c ^ swz<CPR>(r0))) * 16 + 8 * (col & 1));
        const uint16_t* p1 =
            reinterpret_cast<const uint16_t*>(vt + (r1 * CPR + (c ^ swz<CPR>(r1))) * 16 + 8 * (col & 1));
        const s16x4 lo4 = lds_read_tr16(p0);
        const s16x4 hi4 = lds_read_tr16(p1);
        return __builtin_bit_cast(f16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      f16x8 bcur = vload(0);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        f16x8 bnext = bcur;
        if (ct + 1 < NCT) bnext = vload(ct + 1);
#pragma unroll
        for (int i = 0; i < LIVE; ++i) O[i][ct] = mfma_f16(A[i], bcur, O[i][ct]);
        bcur = bnext;
      }
    };
    if constexpr (LIVE > 0) compute();
    if (has_next) vwrite(t + 1, vnext);
    __syncthreads();
  }
  };
  if (n_live == MT) {
    key_loop(std::integral_constant<int, MT>{});
  } else {
    key_loop(std::integral_constant<int, MT - 1>{});
  }

  // finalise: the row sum over the 4 lanes of a column, then write o (or the
  // split partial).  Output row 4q+e of O belongs to query row (tile*16 + 4q+e),
  // whose max and sum live in the lanes with col == 4q+e.
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int tile = tile0 + wave + NW * i;
    if (tile >= tile_end) continue;  // wave-uniform
    float lt = l[i];
    lt += shfl_xor(lt, 16);
    lt += shfl_xor(lt, 32);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int rr = 4 * quad + e;
      const float le = __shfl(lt, rr, 64);
      const float me = __shfl(m[i], rr, 64);
      const int r = tile * 16 + rr;
      if (r >= a.R) continue;
      const int hl = r / a.n_q, j = r % a.n_q;
      const size_t row = (size_t)(b * a.Hq + hk * a.g + hl) * a.n_q + j;
      if (a.splits == 1 && !a.write_partials) {
        const float inv = le > 0.0f ? 1.0f / le : 0.0f;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) a.out[row * D + 16 * ct + col] = O[i][ct][e] * inv;
      } else {
        const size_t rows = (size_t)a.B * a.Hq * a.n_q;
        float* pp = a.ws + ((size_t)split * rows + row) * (D + 2);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) pp[16 * ct + col] = O[i][ct][e];
        if (col == 0) {
          pp[D] = me;
          pp[D + 1] = le;
        }
      }
    }
  }
}

// Merge split partials of one query row per workgroup (see draft_combine_kernel).
constexpr int kMaxCombineSplits = 256;
__global__ __launch_bounds__(128) void verify_combine_kernel(const float* __restrict__ ws, int splits, int rows,
                                                             int D, float* __restrict__ out) {
  __shared__ float s_f[kMaxCombineSplits], s_l[kMaxCombineSplits];
  __shared__ float s_L;
  const int row = blockIdx.x;
  for (int s = threadIdx.x; s < splits; s += blockDim.x) {
    const float* p = ws + ((size_t)s * rows + row) * (D + 2);
    s_f[s] = p[D];
    s_l[s] = p[D + 1];
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    float M = kNegInf;
    for (int s = threadIdx.x; s < splits; s += 64) M = fmaxf(M, s_f[s]);
#pragma unroll
    for (int mm = 32; mm >= 1; mm >>= 1) M = fmaxf(M, __shfl_xor(M, mm, 64));
    float L = 0.0f;
    for (int s = threadIdx.x; s < splits; s += 64) {
      const float f = s_f[s] == kNegInf ? 0.0f : fast_exp2(s_f[s] - M);
      s_f[s] = f;
      L += s_l[s] * f;
    }
#pragma unroll
    for (int mm = 32; mm >= 1; mm >>= 1) L += __shfl_xor(L, mm, 64);
    if (threadIdx.x == 0) s_L = L;
  }
  __syncthreads();
  const float L = s_L;
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float O = 0.0f;
#pragma unroll 8
    for (int s = 0; s < splits; ++s) O += ws[((size_t)s * rows + row) * (D + 2) + d] * s_f[s];
    out[(size_t)row * D + d] = L > 0.0f ? O / L : 0.0f;
  }
}

typedef void (*VerifyKernel)(VerifyArgs);

template <int D, bool PAGED, int NW>
VerifyKernel pick_mt(int mt) {
  if (mt == 1) return verify_mfma_kernel<D, 1, PAGED, NW>;
  if (mt == 2) return verify_mfma_kernel<D, 2, PAGED, NW>;
  return verify_mfma_kernel<D, 3, PAGED, NW>;
}

template <int D, bool PAGED>
VerifyKernel pick(int mt, int nw) {
  return nw == 8 ? pick_mt<D, PAGED, 8>(mt) : pick_mt<D, PAGED, 4>(mt);
}

int wgs_per_cu(VerifyKernel k, int threads) {
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, int> cache;
  int dev = 0;
  (void)hipGetDevice(&dev);
  std::lock_guard<std::mutex> lk(mu);
  auto key = std::make_pair(reinterpret_cast<const void*>(k), dev);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k, threads, 0) != hipSuccess || n < 1) n = 1;
  cache[key] = n;
  return n;
}

struct Plan {
  int nw, mt, tiles_per_group, rowgroups, splits, kps;
};

// wpc: resident workgroups per CU of the kernel (8 bounds every variant).
// keys: length of the key range the call covers (max_ctx + n_q for a whole verify).
Plan plan_verify(int B, int Hq, int Hkv, int n_q, int keys, int wpc) {
  Plan p{};
  const int g = Hq / Hkv;
  const int R = g * n_q;
  const int NT = (R + 15) / 16;
  // 8 wavefronts when 4 cannot hold every tile at kMaxMT each; then as few row
  // groups as hold the tiles, the tiles spread evenly over them
  p.nw = NT > kWaves * kMaxMT ? 2 * kWaves : kWaves;
  p.rowgroups = (NT + p.nw * kMaxMT - 1) / (p.nw * kMaxMT);
  const int per_group = (NT + p.rowgroups - 1) / p.rowgroups;
  p.mt = (per_group + p.nw - 1) / p.nw;
  p.tiles_per_group = per_group;
  const int units = B * Hkv * p.rowgroups;
  const int target = wpc * num_cus();
  int s = target / units;
  const int cap = (keys + 4 * kKT - 1) / (4 * kKT);  // >= 4 tiles per split
  if (s > cap) s = cap;
  if (s < 1) s = 1;
  int kps = (keys + s - 1) / s;
  kps = ((kps + kKT - 1) / kKT) * kKT;
  s = (keys + kps - 1) / kps;
  p.splits = s;
  p.kps = kps;
  return p;
}

size_t verify_ws_need(int B, int Hq, int n_q, int D, int splits) {
  const size_t need = splits > 1 ? (size_t)splits * B * Hq * n_q * (D + 2) * sizeof(float) : 0;
  return need < 256 ? 256 : need;
}

// First row a call over keys [key_begin, ...) reads: rounded down to a multiple of 8.
inline int range_base(int key_begin) { return key_begin & ~7; }

// Resident workgroups per CU the partial layout of a range call is planned
// for: a fixed number per kernel shape (2 wavefronts per SIMD), so that
// vc_verify_range_parts needs no device and always agrees with the call.
int range_wpc(const Plan& p) { return p.nw == 2 * kWaves ? 1 : 2; }

// Validates the arguments, plans and launches verify_mfma_kernel over keys
// [key_begin, key_limit) of every sequence (clipped to ctx_len[b] + n_q).
// parts != nullptr (a range call): the kernel writes its split partials there
// and nothing else runs.  Otherwise the output goes to out, through the split
// partials in ws and verify_combine_kernel when the keys are split.
int verify_launch(const char* fn, const void* q, const vc_kv_full* kv, const int32_t* ctx_len, int max_ctx,
                  int n_q, int key_begin, int key_limit, float* out, float* parts, int B, int Hq, int Hkv, int D,
                  float scale, void* ws, size_t ws_bytes, hipStream_t stream) {
  VC_CHECK(q && kv && ctx_len && (out || parts), "%s: null q/kv/ctx_len/out", fn);
  VC_CHECK(B > 0 && Hq > 0 && Hkv > 0 && Hq % Hkv == 0, "%s: bad B/Hq/Hkv (%d,%d,%d)", fn, B, Hq, Hkv);
  if (D != 64 && D != 128) return fail(VC_ERR_UNSUPPORTED, "%s: D=%d not in {64,128}", fn, D);
  VC_CHECK(n_q >= 1 && max_ctx >= 0, "%s: n_q=%d max_ctx=%d", fn, n_q, max_ctx);
  VC_CHECK(aligned(q, 16) && (out == nullptr || aligned(out, 16)) && (parts == nullptr || aligned(parts, 16)),
           "%s: q/out/parts must be 16-byte aligned", fn);
  VerifyArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(kv->k);
  a.v = static_cast<const uint16_t*>(kv->v);
  VC_CHECK(kv->k != nullptr, "%s: null kv->k", fn);
  VC_CHECK(aligned(kv->k, 16), "%s: kv->k misaligned", fn);
  if (kv->page_table == nullptr) {
    VC_CHECK(kv->v != nullptr && aligned(kv->v, 16), "%s: null or misaligned kv->v", fn);
    VC_CHECK((long long)max_ctx + n_q <= kv->L_cap, "%s: max_ctx + n_q = %d exceeds L_cap = %d", fn,
             max_ctx + n_q, kv->L_cap);
    a.L_cap = kv->L_cap;
  } else {
    const int pt = kv->page_tokens;
    VC_CHECK(pt >= 8 && (pt & (pt - 1)) == 0, "%s: page_tokens=%d must be a power of two >= 8", fn, pt);
    VC_CHECK((long long)kv->pages_per_seq * pt >= (long long)max_ctx + n_q,
             "%s: %d pages of %d tokens cannot hold max_ctx + n_q = %d", fn, kv->pages_per_seq, pt, max_ctx + n_q);
    VC_CHECK(kv->n_slots > 0, "%s: n_slots must be > 0", fn);
    a.page_table = kv->page_table;
    a.page_log2 = __builtin_ctz(pt);
    a.pages_per_seq = kv->pages_per_seq;
    a.n_slots = kv->n_slots;
  }
  a.ctx_len = ctx_len;
  a.max_ctx = max_ctx;
  a.out = out;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.g = Hq / Hkv;
  a.n_q = n_q;
  a.R = a.g * n_q;
  a.NT = (a.R + 15) / 16;
  a.scale_log2 = scale * kLog2e;
  // the cache is read from the 8-aligned row at or below key_begin (the rows
  // in between are masked), so that no load instruction of a paged cache
  // spans two pages; contiguous caches take the same plan, so that
  // vc_verify_range_parts needs no cache description
  a.key_lo = key_begin;
  a.key_begin = range_base(key_begin);
  a.key_limit = key_limit;
  a.write_partials = parts != nullptr ? 1 : 0;
  const int keys = key_limit - a.key_begin;
  Plan p = plan_verify(B, Hq, Hkv, n_q, keys, 8);
  const bool paged = kv->page_table != nullptr;
  const VerifyKernel kern = D == 128 ? (paged ? pick<128, true>(p.mt, p.nw) : pick<128, false>(p.mt, p.nw))
                                     : (paged ? pick<64, true>(p.mt, p.nw) : pick<64, false>(p.mt, p.nw));
  p = plan_verify(B, Hq, Hkv, n_q, keys, parts != nullptr ? range_wpc(p) : wgs_per_cu(kern, 64 * p.nw));
  a.rowgroups = p.rowgroups;
  a.tiles_per_group = p.tiles_per_group;
  a.splits = p.splits;
  a.keys_per_split = p.kps;
  a.n_su = p.splits * B * Hkv;
  if (parts != nullptr) {
    a.ws = parts;
  } else if (p.splits > 1) {
    const size_t need = verify_ws_need(B, Hq, n_q, D, p.splits);
    if (ws == nullptr || ws_bytes < need)
      return fail(VC_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
    VC_CHECK(aligned(ws, 16), "%s: workspace misaligned", fn);
    VC_CHECK(p.splits <= kMaxCombineSplits, "%s: %d splits exceed %d", fn, p.splits, kMaxCombineSplits);
    a.ws = static_cast<float*>(ws);
  }
  // 1-D grid: 8 consecutive (split, unit) pairs per group of 8 * rowgroups workgroups
  const int n_wg = ((a.n_su + 7) / 8) * 8 * p.rowgroups;
  kern<<<n_wg, 64 * p.nw, 0, stream>>>(a);
  VC_HIP(hipGetLastError());
  if (parts == nullptr && p.splits > 1) {
    const int rows = B * Hq * n_q;
    verify_combine_kernel<<<rows, 128, 0, stream>>>(a.ws, p.splits, rows, D, out);
    VC_HIP(hipGetLastError());
  }
  return VC_OK;
}

}  // namespace
}  // namespace vc

using namespace vc;

extern "C" size_t vc_verify_ws_bytes(int B, int Hq, int Hkv, int D, int n_q, int max_ctx) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || D <= 0 || n_q <= 0 || max_ctx < 0) return 0;
  const Plan p = plan_verify(B, Hq, Hkv, n_q, max_ctx + n_q, 8);
  return verify_ws_need(B, Hq, n_q, D, p.splits);
}

extern "C" int vc_verify_attn(const void* q, const vc_kv_full* kv, const int32_t* ctx_len, int max_ctx, int n_q,
                              float* out, int B, int Hq, int Hkv, int D, float scale, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  VC_CHECK(out != nullptr, "vc_verify_attn: null out");
  return verify_launch("vc_verify_attn", q, kv, ctx_len, max_ctx, n_q, 0, max_ctx + n_q, out, nullptr, B, Hq, Hkv,
                       D, scale, ws, ws_bytes, stream);
}

extern "C" int vc_verify_range_parts(int B, int Hq, int Hkv, int D, int n_q, int key_begin, int key_end) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || (D != 64 && D != 128) || n_q <= 0 || key_begin < 0 ||
      key_end <= key_begin)
    return 0;
  const int keys = key_end - range_base(key_begin);
  const Plan p = plan_verify(B, Hq, Hkv, n_q, keys, 8);
  return plan_verify(B, Hq, Hkv, n_q, keys, range_wpc(p)).splits;
}

extern "C" int vc_verify_attn_range(const void* q, const vc_kv_full* kv, const int32_t* ctx_len, int max_ctx,
                                    int n_q, int key_begin, int key_end, float* parts, int B, int Hq, int Hkv, int D,
                                    float scale, hipStream_t stream) {
  VC_CHECK(parts != nullptr, "vc_verify_attn_range: null parts");
  VC_CHECK(key_begin >= 0 && key_end > key_begin && key_end <= max_ctx + n_q,
           "vc_verify_attn_range: key range [%d, %d) outside [0, max_ctx + n_q = %d)", key_begin, key_end,
           max_ctx + n_q);
  return verify_launch("vc_verify_attn_range", q, kv, ctx_len, max_ctx, n_q, key_begin, key_end, nullptr, parts, B,
                       Hq, Hkv, D, scale, nullptr, 0, stream);
}

extern "C" int vc_verify_merge(const float* parts, int n_parts, int B, int Hq, int n_q, int D, float* out,
                               hipStream_t stream) {
  VC_CHECK(parts != nullptr && out != nullptr, "vc_verify_merge: null parts/out");
  VC_CHECK(B > 0 && Hq > 0 && n_q > 0 && (D == 64 || D == 128), "vc_verify_merge: bad B/Hq/n_q/D (%d,%d,%d,%d)", B,
           Hq, n_q, D);
  VC_CHECK(n_parts >= 1 && n_parts <= kMaxCombineSplits, "vc_verify_merge: n_parts=%d outside [1, %d]", n_parts,
           kMaxCombineSplits);
  VC_CHECK(aligned(parts, 16) && aligned(out, 16), "vc_verify_merge: parts/out must be 16-byte aligned");
  const int rows = B * Hq * n_q;
  verify_combine_kernel<<<rows, 128, 0, stream>>>(parts, n_parts, rows, D, out);
  VC_HIP(hipGetLastError());
  return VC_OK;
}
