// Causal verify attention over the full bf16 cache on gfx950 matrix cores.
//
// [VC Core Algorithm: one forward pass with KV_full verifies all drafted
//  tokens in parallel; VC Key System Innovations P1: verification is
//  interconnect-bound and compute-bound]
//
// The g query heads of a GQA group times the n_q positions form R = g * n_q
// query rows that share one KV head, so q.K^T and P.V are real contractions.
// A workgroup (4 wavefronts) owns one (batch, kv-head), one group of row tiles
// and one split of the keys.  Per 32-key tile the workgroup stages K (bf16,
// row-major) and V^T (converted to f16, keys permuted to the MFMA operand
// order) in LDS once; each wavefront then runs, for each of its 16-row tiles,
//   S^T[32 keys x 16 rows] = K . Q^T    (bf16 MFMA, fp32 accumulate)
//   online softmax per row (all of a row's state lives in one lane column)
//   O^T[D x 16 rows]     += V^T . P^T  (f16 MFMA, fp32 accumulate)
// Computing the transposed products keeps a row's scores, softmax state and
// output accumulators in the same lanes, so no data moves between lanes except
// the 2-step max reduction over the 4 lanes of a column.
#include "mfma.h"
#include "vc_common.h"

namespace vc {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 32;

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
  int B, Hq, Hkv, g, n_q, R, NT, tiles_per_group;
  int splits, keys_per_split;
  float scale_log2;
};

// Address of row `key` (K if kv == 0, V if kv == 1) of (b, hk), or nullptr.
template <int D>
__device__ __forceinline__ const uint16_t* row_ptr(const VerifyArgs& a, int b, int hk, int key, int kv) {
  if (a.page_table == nullptr) {
    const uint16_t* base = kv == 0 ? a.k : a.v;
    return base + ((size_t)(b * a.Hkv + hk) * a.L_cap + key) * D;
  }
  const int pt = 1 << a.page_log2;
  const int slot = a.page_table[(size_t)b * a.pages_per_seq + (key >> a.page_log2)];
  if (slot < 0 || slot >= a.n_slots) return nullptr;
  const size_t page_elems = (size_t)a.Hkv * 2 * pt * D;
  return a.k + (size_t)slot * page_elems + ((size_t)(hk * 2 + kv) * pt + (key & (pt - 1))) * D;
}

// Position of key kk (0..31 in the tile) in the permuted P^T / V^T operand order:
// lane group jj = (kk % 16) / 4 holds keys {4jj + i, 16 + 4jj + i}, i < 4.
__device__ __forceinline__ int perm_slot(int kk) {
  const int mt = kk >> 4, w = kk & 15;
  return (w >> 2) * 8 + mt * 4 + (w & 3);
}

template <int D, int MAXT>
__global__ __launch_bounds__(kThreads) void verify_mfma_kernel(VerifyArgs a) {
  constexpr int KS = D / 32;   // k-steps of the q.k contraction
  constexpr int DT = D / 16;   // 16-row tiles of O^T
  constexpr int KPAD = D + 8;  // LDS row pitch (elements) of K
  constexpr int VPAD = kTile + 8;
  constexpr int CH = kTile * D / 8;            // 16-byte chunks per tile
  constexpr int CPT = (CH + kThreads - 1) / kThreads;  // chunks per thread

  __shared__ __attribute__((aligned(16))) uint16_t Ks[kTile * KPAD];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VPAD];

  const int unit = blockIdx.y;
  const int b = unit / a.Hkv;
  const int hk = unit % a.Hkv;
  const int split = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int quad = lane >> 4;

  int ctx = a.ctx_len[b];
  ctx = ctx < 0 ? 0 : (ctx > a.max_ctx ? a.max_ctx : ctx);

  // rows of this workgroup and the last key any of them may see
  const int tile0 = blockIdx.z * a.tiles_per_group;
  const int r_lo = tile0 * 16;
  int r_hi = (tile0 + a.tiles_per_group) * 16;
  r_hi = r_hi < a.R ? r_hi : a.R;
  int jmax = a.n_q - 1;
  if (r_hi - r_lo <= a.n_q && r_lo / a.n_q == (r_hi - 1) / a.n_q) jmax = (r_hi - 1) % a.n_q;
  const int key_end = ctx + jmax + 1;
  const int kb = split * a.keys_per_split;
  int ke = kb + a.keys_per_split;
  ke = ke < key_end ? ke : key_end;

  // per-wavefront row tiles: tile0 + wave + 4 * i, below tile_end
  const int tile_end = min(tile0 + a.tiles_per_group, a.NT);
  bf16x8 qb[MAXT][KS];
  f32x4 acc[MAXT][DT];
  float mrow[MAXT], lrow[MAXT];
  int rlim[MAXT];  // last visible key of this lane's row, -1 if the row is padding
#pragma unroll
  for (int i = 0; i < MAXT; ++i) {
    const int tile = tile0 + wave + kWaves * i;
    const int r = tile * 16 + col;
    const bool live = tile < tile_end && r < a.R;
    rlim[i] = -1;
    if (live) {
      const int hl = r / a.n_q, j = r % a.n_q;
      rlim[i] = ctx + j;
      const uint16_t* qp = a.q + ((size_t)(b * a.Hq + hk * a.g + hl) * a.n_q + j) * D + quad * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qb[i][ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 32);
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qb[i][ks] = bf16x8{};
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[i][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    mrow[i] = kNegInf;
    lrow[i] = 0.0f;
  }

  // register staging of one tile: chunk c -> key c / (D/8), 8 channels at (c % (D/8)) * 8
  u32x4 kreg[CPT], vreg[CPT];
  auto load_tile = [&](int t0) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = threadIdx.x + u * kThreads;
      kreg[u] = u32x4{0, 0, 0, 0};
      vreg[u] = u32x4{0, 0, 0, 0};
      if (c < CH) {
        const int kk = c / (D / 8), c8 = c % (D / 8);
        const int key = t0 + kk;
        if (key < ke) {
          const uint16_t* kp = row_ptr<D>(a, b, hk, key, 0);
          const uint16_t* vp = row_ptr<D>(a, b, hk, key, 1);
          if (kp != nullptr) {
            kreg[u] = *reinterpret_cast<const u32x4*>(kp + c8 * 8);
            vreg[u] = *reinterpret_cast<const u32x4*>(vp + c8 * 8);
          }
        }
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = threadIdx.x + u * kThreads;
      if (c < CH) {
        const int kk = c / (D / 8), c8 = c % (D / 8);
        *reinterpret_cast<u32x4*>(&Ks[kk * KPAD + c8 * 8]) = kreg[u];
        const int slot = perm_slot(kk);
        const u32x4 w = vreg[u];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t x = w[e];
          const _Float16 lo = (_Float16)__uint_as_float(x << 16);
          const _Float16 hi = (_Float16)__uint_as_float(x & 0xFFFF0000u);
          Vt[(c8 * 8 + 2 * e) * VPAD + slot] = __builtin_bit_cast(uint16_t, lo);
          Vt[(c8 * 8 + 2 * e + 1) * VPAD + slot] = __builtin_bit_cast(uint16_t, hi);
        }
      }
    }
  };

  if (kb < ke) load_tile(kb);
  for (int t0 = kb; t0 < ke; t0 += kTile) {
    __syncthreads();  // previous tile fully consumed
    store_tile();
    __syncthreads();
    if (t0 + kTile < ke) load_tile(t0 + kTile);

#pragma unroll
    for (int i = 0; i < MAXT; ++i) {
      if (tile0 + wave + kWaves * i >= tile_end) continue;  // wave-uniform
      // S^T for the two 16-key halves of the tile
      f32x4 s[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        f32x4 c4 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 av = *reinterpret_cast<const bf16x8*>(&Ks[(mt * 16 + col) * KPAD + ks * 32 + quad * 8]);
          c4 = mfma_bf16(av, qb[i][ks], c4);
        }
        s[mt] = c4;
      }
      // mask, scale, online softmax (row = this lane's column)
      float tmax = kNegInf;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = t0 + mt * 16 + quad * 4 + e;
          const bool ok = key <= rlim[i] && key < ke;
          const float x = ok ? s[mt][e] * a.scale_log2 : kNegInf;
          s[mt][e] = x;
          tmax = fmaxf(tmax, x);
        }
      }
      tmax = fmaxf(tmax, shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, shfl_xor(tmax, 32));
      const float mnew = fmaxf(mrow[i], tmax);
      const float muse = mnew == kNegInf ? 0.0f : mnew;
      const float alpha = fast_exp2(mrow[i] - muse);
      mrow[i] = mnew;
      f16x8 pb;
      float psum = 0.0f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = fast_exp2(s[mt][e] - muse);
          const _Float16 ph = (_Float16)p;  // round to nearest even
          psum += (float)ph;                // sum the rounded weights actually applied
          pb[mt * 4 + e] = ph;
        }
      }
      lrow[i] = lrow[i] * alpha + psum;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        acc[i][dt] *= alpha;
        const f16x8 av = *reinterpret_cast<const f16x8*>(&Vt[(dt * 16 + col) * VPAD + quad * 8]);
        acc[i][dt] = mfma_f16(av, pb, acc[i][dt]);
      }
    }
  }

  // finalise: total row sum over the 4 lanes of the column, then write
#pragma unroll
  for (int i = 0; i < MAXT; ++i) {
    float lt = lrow[i];
    lt += shfl_xor(lt, 16);
    lt += shfl_xor(lt, 32);
    if (rlim[i] < 0) continue;
    const int r = (tile0 + wave + kWaves * i) * 16 + col;
    const int hl = r / a.n_q, j = r % a.n_q;
    const size_t row = (size_t)(b * a.Hq + hk * a.g + hl) * a.n_q + j;
    if (a.splits == 1) {
      const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
      float* op = a.out + row * D + quad * 4;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        f32x4 v = acc[i][dt] * inv;
        *reinterpret_cast<f32x4*>(op + dt * 16) = v;
      }
    } else {
      const size_t rows = (size_t)a.B * a.Hq * a.n_q;
      float* pp = a.ws + ((size_t)split * rows + row) * (D + 2);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        float* dst = pp + dt * 16 + quad * 4;
        dst[0] = acc[i][dt][0];
        dst[1] = acc[i][dt][1];
        dst[2] = acc[i][dt][2];
        dst[3] = acc[i][dt][3];
      }
      if (quad == 0) {
        pp[D] = mrow[i];
        pp[D + 1] = lt;
      }
    }
  }
}

__global__ void verify_combine_kernel(const float* __restrict__ ws, int splits, int rows, int D,
                                      float* __restrict__ out) {
  const int row = blockIdx.x;
  const int d = threadIdx.x;
  float M = kNegInf;
  for (int s = 0; s < splits; ++s) M = fmaxf(M, ws[((size_t)s * rows + row) * (D + 2) + D]);
  float L = 0.0f, O = 0.0f;
  for (int s = 0; s < splits; ++s) {
    const float* p = ws + ((size_t)s * rows + row) * (D + 2);
    const float ms = p[D];
    const float f = ms == kNegInf ? 0.0f : fast_exp2(ms - M);
    L += p[D + 1] * f;
    O += p[d] * f;
  }
  out[(size_t)row * D + d] = L > 0.0f ? O / L : 0.0f;
}

struct Plan {
  int maxt, tiles_per_group, groups, splits, kps;
};

Plan plan_verify(int B, int Hq, int Hkv, int n_q, int max_ctx) {
  Plan p{};
  const int g = Hq / Hkv;
  const int R = g * n_q;
  const int NT = (R + 15) / 16;
  int maxt = (NT + kWaves - 1) / kWaves;
  if (maxt > 4 && NT > 5 * kWaves) maxt = 4;
  if (maxt > 5) maxt = 5;
  p.maxt = maxt;
  p.tiles_per_group = maxt * kWaves;
  p.groups = (NT + p.tiles_per_group - 1) / p.tiles_per_group;
  const int units = B * Hkv * p.groups;
  const int keys = max_ctx + n_q;
  const int target = 2 * num_cus();
  int s = (target + units - 1) / units;
  const int cap = (keys + 255) / 256;
  if (s > cap) s = cap;
  if (s < 1) s = 1;
  int kps = (keys + s - 1) / s;
  kps = ((kps + kTile - 1) / kTile) * kTile;
  s = (keys + kps - 1) / kps;
  p.splits = s;
  p.kps = kps;
  return p;
}

template <int D>
void launch_verify(const VerifyArgs& a, int maxt, dim3 grid, hipStream_t st) {
  switch (maxt) {
    case 1: verify_mfma_kernel<D, 1><<<grid, kThreads, 0, st>>>(a); break;
    case 2: verify_mfma_kernel<D, 2><<<grid, kThreads, 0, st>>>(a); break;
    case 3: verify_mfma_kernel<D, 3><<<grid, kThreads, 0, st>>>(a); break;
    case 4: verify_mfma_kernel<D, 4><<<grid, kThreads, 0, st>>>(a); break;
    default: verify_mfma_kernel<D, 5><<<grid, kThreads, 0, st>>>(a); break;
  }
}

}  // namespace
}  // namespace vc

using namespace vc;

extern "C" size_t vc_verify_ws_bytes(int B, int Hq, int Hkv, int D, int n_q, int max_ctx) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || D <= 0 || n_q <= 0 || max_ctx < 0) return 0;
  const Plan p = plan_verify(B, Hq, Hkv, n_q, max_ctx);
  const size_t need = p.splits > 1 ? (size_t)p.splits * B * Hq * n_q * (D + 2) * sizeof(float) : 0;
  return need < 256 ? 256 : need;
}

extern "C" int vc_verify_attn(const void* q, const vc_kv_full* kv, const int32_t* ctx_len, int max_ctx, int n_q,
                              float* out, int B, int Hq, int Hkv, int D, float scale, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  VC_CHECK(q && kv && ctx_len && out, "vc_verify_attn: null q/kv/ctx_len/out");
  VC_CHECK(B > 0 && Hq > 0 && Hkv > 0 && Hq % Hkv == 0, "vc_verify_attn: bad B/Hq/Hkv (%d,%d,%d)", B, Hq, Hkv);
  if (D != 64 && D != 128) return fail(VC_ERR_UNSUPPORTED, "vc_verify_attn: D=%d not in {64,128}", D);
  VC_CHECK(n_q >= 1 && max_ctx >= 0, "vc_verify_attn: n_q=%d max_ctx=%d", n_q, max_ctx);
  VC_CHECK(aligned(q, 16) && aligned(out, 16), "vc_verify_attn: q/out must be 16-byte aligned");
  VerifyArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(kv->k);
  a.v = static_cast<const uint16_t*>(kv->v);
  VC_CHECK(kv->k != nullptr, "vc_verify_attn: null kv->k");
  VC_CHECK(aligned(kv->k, 16), "vc_verify_attn: kv->k misaligned");
  if (kv->page_table == nullptr) {
    VC_CHECK(kv->v != nullptr && aligned(kv->v, 16), "vc_verify_attn: null or misaligned kv->v");
    VC_CHECK((long long)max_ctx + n_q <= kv->L_cap, "vc_verify_attn: max_ctx + n_q = %d exceeds L_cap = %d",
             max_ctx + n_q, kv->L_cap);
    a.L_cap = kv->L_cap;
  } else {
    const int pt = kv->page_tokens;
    VC_CHECK(pt >= 8 && (pt & (pt - 1)) == 0, "vc_verify_attn: page_tokens=%d must be a power of two >= 8", pt);
    VC_CHECK((long long)kv->pages_per_seq * pt >= (long long)max_ctx + n_q,
             "vc_verify_attn: %d pages of %d tokens cannot hold max_ctx + n_q = %d", kv->pages_per_seq, pt,
             max_ctx + n_q);
    VC_CHECK(kv->n_slots > 0, "vc_verify_attn: n_slots must be > 0");
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
  const Plan p = plan_verify(B, Hq, Hkv, n_q, max_ctx);
  a.tiles_per_group = p.tiles_per_group;
  a.splits = p.splits;
  a.keys_per_split = p.kps;
  if (p.splits > 1) {
    const size_t need = vc_verify_ws_bytes(B, Hq, Hkv, D, n_q, max_ctx);
    if (ws == nullptr || ws_bytes < need)
      return fail(VC_ERR_WORKSPACE, "vc_verify_attn: workspace %zu < %zu bytes", ws_bytes, need);
    VC_CHECK(aligned(ws, 16), "vc_verify_attn: workspace misaligned");
    a.ws = static_cast<float*>(ws);
  }
  dim3 grid(p.splits, B * Hkv, p.groups);
  if (D == 128)
    launch_verify<128>(a, p.maxt, grid, stream);
  else
    launch_verify<64>(a, p.maxt, grid, stream);
  VC_HIP(hipGetLastError());
  if (p.splits > 1) {
    const int rows = B * Hq * n_q;
    verify_combine_kernel<<<rows, D, 0, stream>>>(a.ws, p.splits, rows, D, out);
    VC_HIP(hipGetLastError());
  }
  return VC_OK;
}
