// Draft decode attention over the lossy cache (one query position per call).
//
// [VC Core Algorithm: drafting generates candidate tokens with KV_comp;
//  VC Key System Innovations P1: drafting is GPU-HBM-bandwidth bound]
//
// Vector-ALU kernel.  A workgroup (4 wavefronts) owns one (batch, kv-head)
// and one split of its keys.  Inside a wavefront, 8 lanes share a key: each
// holds D/8 channels, dequantises them in registers (fp32, a single fma per
// value), forms partial q.k dot products for the g query heads of the GQA
// group and reduces them with 3 lane shuffles.  Every 8-lane slot keeps its own
// online-softmax state (running max in log2 units, sum, unnormalised output for
// its channels); slots are merged with lane shuffles and the 4 wavefronts in
// LDS at the end.  Splits are merged by draft_combine_kernel.
#include "vc_common.h"

namespace vc {
namespace {

struct alignas(4) H2 {
  _Float16 s, z;
};

struct DraftArgs {
  int kind, bits, n_quant, L_full, L_cap, n_keep;
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const H2* k_meta;
  const H2* v_meta;
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
  int n_main;
  int keys_per_split;
  int splits;
  float* ws;
};

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

// Load CPL consecutive bf16 values as fp32.
template <int CPL>
__device__ __forceinline__ void load_bf16_row(const uint16_t* p, float* x) {
  static_assert(CPL % 8 == 0, "");
#pragma unroll
  for (int c = 0; c < CPL; c += 8) {
    const uint4 w = *reinterpret_cast<const uint4*>(p + c);
    x[c + 0] = bf16_lo(w.x);
    x[c + 1] = bf16_hi(w.x);
    x[c + 2] = bf16_lo(w.y);
    x[c + 3] = bf16_hi(w.y);
    x[c + 4] = bf16_lo(w.z);
    x[c + 5] = bf16_hi(w.z);
    x[c + 6] = bf16_lo(w.w);
    x[c + 7] = bf16_hi(w.w);
  }
}

// Unpack CPL codes (canonical packing) starting at channel c0 of a code row.
template <int CPL, int BITS>
__device__ __forceinline__ void load_codes(const uint8_t* row, int c0, uint32_t* code) {
  constexpr int BYTES = CPL * BITS / 8;
  const uint8_t* p = row + c0 * BITS / 8;
  uint64_t w;
  if constexpr (BYTES == 8) {
    w = *reinterpret_cast<const uint64_t*>(p);
  } else if constexpr (BYTES == 4) {
    w = *reinterpret_cast<const uint32_t*>(p);
  } else {
    w = *reinterpret_cast<const uint16_t*>(p);
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) code[c] = (uint32_t)(w >> (BITS * c)) & ((1u << BITS) - 1u);
}

// Fetch the CPL channels [c0, c0 + CPL) of key `key` of unit `unit` as fp32.
template <int D, int CPL, int BITS>
__device__ __forceinline__ void fetch_key_row(const DraftArgs& a, int unit, int b, int key, int c0,
                                              bool is_k, float* x) {
  if (key < a.n_main) {
    if (BITS > 0) {  // QUANT
      constexpr int RB = D * BITS / 8;
      const uint8_t* codes = (is_k ? a.k_codes : a.v_codes) + ((size_t)unit * a.n_quant + key) * RB;
      uint32_t code[CPL];
      load_codes<CPL, BITS>(codes, c0, code);
      if (is_k) {
        const H2* m = a.k_meta + ((size_t)unit * (a.n_quant / 32) + key / 32) * D + c0;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const H2 sz = m[c];
          x[c] = fmaf((float)code[c], (float)sz.s, (float)sz.z);
        }
      } else {
        const H2 sz = a.v_meta[((size_t)unit * a.n_quant + key) * (D / 32) + c0 / 32];
        const float s = (float)sz.s, z = (float)sz.z;
#pragma unroll
        for (int c = 0; c < CPL; ++c) x[c] = fmaf((float)code[c], s, z);
      }
    } else {
      int row = key;
      if (a.kind == VC_KV_TOKEN_DROP) row = a.keep_idx[(size_t)unit * a.n_keep + key];
      const uint16_t* src = is_k ? a.k_full : a.v_full;
      if (row < 0 || row >= a.L_cap) {  // invalid index: contributes nothing
#pragma unroll
        for (int c = 0; c < CPL; ++c) x[c] = 0.0f;
        return;
      }
      load_bf16_row<CPL>(src + ((size_t)unit * a.L_cap + row) * D + c0, x);
    }
  } else {
    const uint16_t* src = is_k ? a.tail_k : a.tail_v;
    load_bf16_row<CPL>(src + ((size_t)unit * a.T_cap + (key - a.n_main)) * D + c0, x);
  }
}

template <int D, int GM, int BITS>
__global__ __launch_bounds__(kThreads) void draft_valu_kernel(DraftArgs a) {
  constexpr int CPL = D / 8;
  const int unit = blockIdx.y;
  const int b = unit / a.Hkv;
  const int hk = unit % a.Hkv;
  const int split = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int slot = lane >> 3;
  const int c0 = (lane & 7) * CPL;
  const int g = a.g;

  int tl = a.T_cap > 0 ? a.tail_len[b] : 0;
  tl = tl < 0 ? 0 : (tl > a.T_cap ? a.T_cap : tl);
  const int n_keys = a.n_main + tl;
  const int k0 = split * a.keys_per_split;
  int k1 = k0 + a.keys_per_split;
  k1 = k1 < n_keys ? k1 : n_keys;

  float qf[GM][CPL];
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    if (h < g) {
      load_bf16_row<CPL>(a.q + ((size_t)b * a.Hq + hk * g + h) * D + c0, qf[h]);
    } else {
#pragma unroll
      for (int c = 0; c < CPL; ++c) qf[h][c] = 0.0f;
    }
  }
  float m[GM], l[GM], o[GM][CPL];
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    m[h] = kNegInf;
    l[h] = 0.0f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) o[h][c] = 0.0f;
  }

  const int span = k1 > k0 ? k1 - k0 : 0;
  const int iters = (span + 8 * kWaves - 1) / (8 * kWaves);
  for (int it = 0; it < iters; ++it) {
    const int key = k0 + (it * kWaves + wave) * 8 + slot;
    const bool valid = key < k1;
    float kx[CPL];
    if (valid) {
      fetch_key_row<D, CPL, BITS>(a, unit, b, key, c0, true, kx);
    } else {
#pragma unroll
      for (int c = 0; c < CPL; ++c) kx[c] = 0.0f;
    }
    float s[GM];
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      float acc = 0.0f;
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc = fmaf(qf[h][c], kx[c], acc);
      acc += shfl_xor(acc, 1);
      acc += shfl_xor(acc, 2);
      acc += shfl_xor(acc, 4);
      s[h] = acc * a.scale_log2;
    }
    if (valid) {
      float vx[CPL];
      fetch_key_row<D, CPL, BITS>(a, unit, b, key, c0, false, vx);
#pragma unroll
      for (int h = 0; h < GM; ++h) {
        if (h < g) {
          const float mn = fmaxf(m[h], s[h]);
          const float alpha = fast_exp2(m[h] - mn);  // 0 when m was -inf
          const float p = fast_exp2(s[h] - mn);
          l[h] = fmaf(l[h], alpha, p);
#pragma unroll
          for (int c = 0; c < CPL; ++c) o[h][c] = fmaf(o[h][c], alpha, p * vx[c]);
          m[h] = mn;
        }
      }
    }
  }

  // merge the 8 slots of the wavefront (lanes with equal channel chunk)
#pragma unroll
  for (int mask = 8; mask < 64; mask <<= 1) {
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      const float mo = shfl_xor(m[h], mask);
      const float lo = shfl_xor(l[h], mask);
      const float mn = fmaxf(m[h], mo);
      const float wa = m[h] == kNegInf ? 0.0f : fast_exp2(m[h] - mn);
      const float wb = mo == kNegInf ? 0.0f : fast_exp2(mo - mn);
      l[h] = l[h] * wa + lo * wb;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const float oo = shfl_xor(o[h][c], mask);
        o[h][c] = o[h][c] * wa + oo * wb;
      }
      m[h] = mn;
    }
  }

  // merge the wavefronts in LDS
  __shared__ float s_o[kWaves][GM][D];
  __shared__ float s_ml[kWaves][GM][2];
  if (slot == 0) {
#pragma unroll
    for (int h = 0; h < GM; ++h) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) s_o[wave][h][c0 + c] = o[h][c];
      if (c0 == 0) {
        s_ml[wave][h][0] = m[h];
        s_ml[wave][h][1] = l[h];
      }
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < g * D; t += kThreads) {
    const int h = t / D, d = t % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_ml[w][h][0]);
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = s_ml[w][h][0];
      const float f = mw == kNegInf ? 0.0f : fast_exp2(mw - M);
      L += s_ml[w][h][1] * f;
      O += s_o[w][h][d] * f;
    }
    const int hq = hk * g + h;
    if (a.splits == 1) {
      a.out[((size_t)b * a.Hq + hq) * D + d] = L > 0.0f ? O / L : 0.0f;
      if (a.lse != nullptr && d == 0) a.lse[(size_t)b * a.Hq + hq] = L > 0.0f ? (M + __log2f(L)) * kLn2 : kNegInf;
    } else {
      float* p = a.ws + (((size_t)split * a.B + b) * a.Hq + hq) * (D + 2);
      p[d] = O;
      if (d == 0) {
        p[D] = M;
        p[D + 1] = L;
      }
    }
  }
}

// Merge split partials (o unnormalised, m in log2 units, l) of every (b, h) row.
__global__ void draft_combine_kernel(const float* __restrict__ ws, int splits, int rows, int D,
                                     float* __restrict__ out, float* __restrict__ lse) {
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
  if (lse != nullptr && d == 0) lse[row] = L > 0.0f ? (M + __log2f(L)) * kLn2 : kNegInf;
}

int plan_draft_splits(int units, int max_keys) {
  const int target = 4 * num_cus();
  int s = (target + units - 1) / units;
  const int cap = (max_keys + 255) / 256;
  if (s > cap) s = cap;
  if (s < 1) s = 1;
  return s;
}

template <int D, int GM>
void launch_draft(const DraftArgs& a, dim3 grid, hipStream_t st) {
  if (a.kind == VC_KV_QUANT) {
    if (a.bits == 4)
      draft_valu_kernel<D, GM, 4><<<grid, kThreads, 0, st>>>(a);
    else
      draft_valu_kernel<D, GM, 2><<<grid, kThreads, 0, st>>>(a);
  } else {
    draft_valu_kernel<D, GM, 0><<<grid, kThreads, 0, st>>>(a);
  }
}

}  // namespace
}  // namespace vc

using namespace vc;

extern "C" size_t vc_draft_ws_bytes(int B, int Hq, int Hkv, int D, int max_keys) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || max_keys < 0) return 0;
  const int s = plan_draft_splits(B * Hkv, max_keys);
  const size_t need = s > 1 ? (size_t)s * B * Hq * (D + 2) * sizeof(float) : 0;
  return need < 256 ? 256 : need;
}

extern "C" int vc_draft_attn(const vc_kv_comp* comp, const vc_tail* tail, const void* q, float* out,
                             float* lse, int B, int Hq, int Hkv, int D, float scale, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  VC_CHECK(comp != nullptr && q != nullptr && out != nullptr, "vc_draft_attn: null comp/q/out");
  VC_CHECK(B > 0 && Hq > 0 && Hkv > 0 && Hq % Hkv == 0, "vc_draft_attn: bad B/Hq/Hkv (%d,%d,%d)", B, Hq, Hkv);
  if (D != 64 && D != 128) return fail(VC_ERR_UNSUPPORTED, "vc_draft_attn: D=%d not in {64,128}", D);
  const int g = Hq / Hkv;
  if (g > 8) return fail(VC_ERR_UNSUPPORTED, "vc_draft_attn: GQA group %d > 8", g);
  VC_CHECK(aligned(q, 16) && aligned(out, 16), "vc_draft_attn: q/out must be 16-byte aligned");
  DraftArgs a{};
  a.kind = comp->kind;
  a.q = static_cast<const uint16_t*>(q);
  a.out = out;
  a.lse = lse;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.g = g;
  a.scale_log2 = scale * kLog2e;
  switch (comp->kind) {
    case VC_KV_QUANT:
      VC_CHECK(comp->bits == 2 || comp->bits == 4, "vc_draft_attn: bits must be 2 or 4 (got %d)", comp->bits);
      VC_CHECK(comp->n_quant >= 0 && comp->n_quant % 32 == 0, "vc_draft_attn: n_quant=%d not a multiple of 32",
               comp->n_quant);
      VC_CHECK(comp->n_quant == 0 || (comp->k_codes && comp->v_codes && comp->k_meta && comp->v_meta),
               "vc_draft_attn: null codes/meta");
      VC_CHECK(aligned(comp->k_codes, 8) && aligned(comp->v_codes, 8) && aligned(comp->k_meta, 4) &&
                   aligned(comp->v_meta, 4),
               "vc_draft_attn: codes must be 8-byte and meta 4-byte aligned");
      a.bits = comp->bits;
      a.n_quant = comp->n_quant;
      a.n_main = comp->n_quant;
      a.k_codes = comp->k_codes;
      a.v_codes = comp->v_codes;
      a.k_meta = static_cast<const H2*>(comp->k_meta);
      a.v_meta = static_cast<const H2*>(comp->v_meta);
      break;
    case VC_KV_IDENTITY:
    case VC_KV_TOKEN_DROP:
      VC_CHECK(comp->L_cap >= 0, "vc_draft_attn: bad L_cap");
      if (comp->kind == VC_KV_IDENTITY) {
        VC_CHECK(comp->L_full >= 0 && comp->L_full <= comp->L_cap, "vc_draft_attn: L_full=%d outside [0, L_cap=%d]",
                 comp->L_full, comp->L_cap);
        a.n_main = comp->L_full;
      } else {
        VC_CHECK(comp->n_keep >= 0, "vc_draft_attn: bad n_keep");
        VC_CHECK(comp->n_keep == 0 || comp->keep_idx != nullptr, "vc_draft_attn: null keep_idx");
        a.n_main = comp->n_keep;
      }
      VC_CHECK(a.n_main == 0 || (comp->k_full && comp->v_full), "vc_draft_attn: null k_full/v_full");
      VC_CHECK(aligned(comp->k_full, 16) && aligned(comp->v_full, 16), "vc_draft_attn: k_full/v_full misaligned");
      a.k_full = static_cast<const uint16_t*>(comp->k_full);
      a.v_full = static_cast<const uint16_t*>(comp->v_full);
      a.L_full = comp->L_full;
      a.L_cap = comp->L_cap;
      a.keep_idx = comp->keep_idx;
      a.n_keep = comp->n_keep;
      break;
    default:
      return fail(VC_ERR_INVALID, "vc_draft_attn: unknown compressor kind %d", comp->kind);
  }
  if (tail != nullptr && tail->T_cap > 0) {
    VC_CHECK(tail->k && tail->v && tail->len, "vc_draft_attn: null tail pointers");
    VC_CHECK(aligned(tail->k, 16) && aligned(tail->v, 16), "vc_draft_attn: tail misaligned");
    a.tail_k = static_cast<const uint16_t*>(tail->k);
    a.tail_v = static_cast<const uint16_t*>(tail->v);
    a.tail_len = tail->len;
    a.T_cap = tail->T_cap;
  } else {
    VC_CHECK(tail == nullptr || tail->T_cap == 0, "vc_draft_attn: negative T_cap");
    a.T_cap = 0;
  }
  const int units = B * Hkv;
  const int max_keys = a.n_main + a.T_cap;
  const int splits = plan_draft_splits(units, max_keys);
  const size_t need = vc_draft_ws_bytes(B, Hq, Hkv, D, max_keys);
  if (splits > 1) {
    if (ws == nullptr || ws_bytes < need)
      return fail(VC_ERR_WORKSPACE, "vc_draft_attn: workspace %zu < %zu bytes", ws_bytes, need);
    VC_CHECK(aligned(ws, 16), "vc_draft_attn: workspace misaligned");
  }
  int kps = (max_keys + splits - 1) / splits;
  kps = ((kps + 31) / 32) * 32;
  if (kps == 0) kps = 32;
  a.keys_per_split = kps;
  a.splits = splits;
  a.ws = static_cast<float*>(ws);
  dim3 grid(splits, units);
  if (D == 128) {
    if (g <= 4)
      launch_draft<128, 4>(a, grid, stream);
    else
      launch_draft<128, 8>(a, grid, stream);
  } else {
    if (g <= 4)
      launch_draft<64, 4>(a, grid, stream);
    else
      launch_draft<64, 8>(a, grid, stream);
  }
  VC_HIP(hipGetLastError());
  if (splits > 1) {
    draft_combine_kernel<<<B * Hq, D, 0, stream>>>(a.ws, splits, B * Hq, D, out, lse);
    VC_HIP(hipGetLastError());
  }
  return VC_OK;
}
