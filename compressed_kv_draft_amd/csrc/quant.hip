// KIVI-style asymmetric group quantiser for the lossy draft cache, and a
// dequantising read-back used to check it bit for bit.
//
// [VC Problem Statement: token dropping and quantisation are the lossy KV
//  compressors; VC Architecture Support: KIVI behind the uniform interface]
// The page gives no formula; the quantiser is the plain min/max one, every
// step an IEEE fp32 operation with round-to-nearest-even (no contraction).
#include "mfma.h"
#include "vc_common.h"

namespace vc {
namespace {

struct alignas(4) H2 {
  _Float16 s, z;
};

// One group's scale/zero: s = f16((mx - mn) / qmax), z = f16(mn).
__device__ __forceinline__ void group_params(float mn, float mx, int qmax, _Float16& sh, _Float16& zh) {
#pragma clang fp contract(off)
  float s32 = (mx - mn) / (float)qmax;  // correctly rounded division (no fast-math)
  sh = (_Float16)s32;
  zh = (_Float16)mn;
}

__device__ __forceinline__ uint32_t code_of(float x, float s, float z, int qmax) {
#pragma clang fp contract(off)
  if (s == 0.0f) return 0u;
  float t = (x - z) / s;
  float r = rintf(t);
  r = fminf(fmaxf(r, 0.0f), (float)qmax);
  return (uint32_t)r;
}

// Every kernel below quantises source rows [32 i, 32 i + 32) of each (batch,
// kv-head), i < n_blocks (src already points at the first row; rows are
// src_cap apart per unit), into cache block blk0 + i of arrays that hold cap32
// blocks per unit.
//
// K: groups of 32 tokens of one channel.  One thread per (32-token block, byte
// column): it owns the 8/bits channels packed into that byte.
template <int BITS>
__global__ void quant_k_kernel(const uint16_t* __restrict__ src, int L_cap, int D, int blk0, int cap32,
                               uint8_t* __restrict__ codes, H2* __restrict__ meta) {
  constexpr int PER = 8 / BITS;
  constexpr int QMAX = (1 << BITS) - 1;
  const int unit = blockIdx.y;
  const int blk = blockIdx.x;
  const int col = threadIdx.x;  // byte column
  const int row_bytes = D * BITS / 8;
  if (col >= row_bytes) return;
  const uint16_t* base = src + ((size_t)unit * L_cap + (size_t)blk * 32) * D;
  uint32_t packed[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) packed[i] = 0;
  for (int e = 0; e < PER; ++e) {
    const int d = col * PER + e;
    float x[32];
    float mn, mx;
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = bf16_to_f32(base[(size_t)i * D + d]);
    mn = x[0];
    mx = x[0];
#pragma unroll
    for (int i = 1; i < 32; ++i) {
      mn = fminf(mn, x[i]);
      mx = fmaxf(mx, x[i]);
    }
    _Float16 sh, zh;
    group_params(mn, mx, QMAX, sh, zh);
    const float s = (float)sh, z = (float)zh;
#pragma unroll
    for (int i = 0; i < 32; ++i) packed[i] |= code_of(x[i], s, z, QMAX) << (BITS * e);
    _Float16* plane = reinterpret_cast<_Float16*>(meta + ((size_t)unit * cap32 + blk0 + blk) * D);
    const int pos = kmeta_pos(D, BITS, d);
    plane[pos] = sh;
    plane[D + pos] = zh;
  }
  uint8_t* out = codes + ((size_t)unit * cap32 + blk0 + blk) * 32 * row_bytes + col;
#pragma unroll
  for (int i = 0; i < 32; ++i) out[(size_t)i * row_bytes] = (uint8_t)packed[i];
}

// V: groups of 32 channels of one token.  Pass 1, one thread per (token, group):
// the group's scale and zero.
template <int BITS>
__global__ void quant_v_meta_kernel(const uint16_t* __restrict__ src, int L_cap, int D, int n_blocks, int blk0,
                                    int cap32, H2* __restrict__ meta) {
  constexpr int QMAX = (1 << BITS) - 1;
  const int unit = blockIdx.y;
  const int G = D / 32;
  const int gid = blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= n_blocks * 32 * G) return;
  const int t = gid / G, grp = gid % G;
  const uint16_t* row = src + ((size_t)unit * L_cap + t) * D + grp * 32;
  float mn = bf16_to_f32(row[0]), mx = mn;
#pragma unroll
  for (int i = 1; i < 32; ++i) {
    const float x = bf16_to_f32(row[i]);
    mn = fminf(mn, x);
    mx = fmaxf(mx, x);
  }
  H2 m;
  group_params(mn, mx, QMAX, m.s, m.z);
  meta[(((size_t)unit * cap32 + blk0 + t / 32) * G + grp) * 32 + vmeta_slot(t % 32)] = m;
}

// V pass 2, one thread per code byte of the tiled layout (vc_vcode_locate in
// vc_common.h): the byte's codes all belong to one token.
template <int BITS>
__global__ void quant_v_pack_kernel(const uint16_t* __restrict__ src, int L_cap, int D, int n_blocks, int blk0,
                                    int cap32, const H2* __restrict__ meta, uint8_t* __restrict__ codes) {
  constexpr int QMAX = (1 << BITS) - 1;
  const int unit = blockIdx.y;
  const int block_bytes = 4 * D * BITS;  // 32 tokens x D codes
  const int gid = blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= n_blocks * block_bytes) return;
  const int blk = gid / block_bytes, byte = gid % block_bytes;
  uint32_t v = 0;
#pragma unroll
  for (int k = 0; k < 8 / BITS; ++k) {
    int tau, c;
    vcode_inverse(D, BITS, byte, k, tau, c);
    const int t = blk * 32 + tau;
    const float x = bf16_to_f32(src[((size_t)unit * L_cap + t) * D + c]);
    const H2 m = meta[(((size_t)unit * cap32 + blk0 + blk) * (D / 32) + c / 32) * 32 + vmeta_slot(tau)];
    v |= code_of(x, (float)m.s, (float)m.z, QMAX) << (BITS * k);
  }
  codes[((size_t)unit * cap32 + blk0) * block_bytes + gid] = (uint8_t)v;
}

__device__ __forceinline__ uint32_t unpack_code(const uint8_t* row, int d, int bits) {
  if (bits == 4) return (row[d >> 1] >> ((d & 1) * 4)) & 15u;
  return (row[d >> 2] >> ((d & 3) * 2)) & 3u;
}

__global__ void dequant_kernel(const uint8_t* __restrict__ codes, const H2* __restrict__ meta, int bits,
                               int n_quant, int D, int which, float* __restrict__ out) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n_quant * D) return;
  const int t = idx / D, d = idx % D;
  uint32_t c;
  if (which == 0) {
    c = unpack_code(codes + (size_t)t * (D * bits / 8), d, bits);
  } else {
    int byte, shift;
    vcode_locate(D, bits, t % 32, d, byte, shift);
    c = (codes[(size_t)(t / 32) * 4 * D * bits + byte] >> shift) & ((1u << bits) - 1u);
  }
  float s, z;
  if (which == 0) {
    const _Float16* plane = reinterpret_cast<const _Float16*>(meta + (size_t)(t / 32) * D);
    const int pos = kmeta_pos(D, bits, d);
    s = (float)plane[pos];
    z = (float)plane[D + pos];
  } else {
    const H2 m = meta[((size_t)(t / 32) * (D / 32) + d / 32) * 32 + vmeta_slot(t % 32)];
    s = (float)m.s;
    z = (float)m.z;
  }
  out[idx] = fmaf((float)c, s, z);
}

// Conversions between the canonical (dense) QUANT format and the internal
// one.  Canonical, per (batch, kv-head) unit of n rows:
//   K and V codes  u8 [n][D*bits/8], token rows packed along D (4-bit: channel
//                  2i low nibble of byte i; 2-bit: channel i at bit 2 (i % 4))
//   K meta         f16x2 {scale, zero} [n/32][D]   (a pair per 32 tokens of a channel)
//   V meta         f16x2 {scale, zero} [n][D/32]   (a pair per 32 channels of a token)
// Internal: K codes as canonical; V codes tiled (vcode_locate); K meta in pair
// order (kmeta_pos); V meta in score-tile token order (vmeta_slot).  One thread
// per output item; part = blockIdx.z selects K codes (16-byte chunks), V
// codes (bytes), K meta, V meta (pairs).
struct PackArgs {
  int D, bits, n32, cap32, blk0;  // canonical blocks n32; internal blocks per unit cap32; first block blk0
  uint8_t* ck;                    // canonical side (read when packing, written when unpacking)
  uint8_t* cv;
  H2* ckm;
  H2* cvm;
  uint8_t* ik;                    // internal side (written when packing, read when unpacking)
  uint8_t* iv;
  H2* ikm;
  H2* ivm;
};

// pack = true: canonical -> internal (writes the internal arrays, blocks
// blk0 .. blk0 + n32 - 1); false: internal blocks blk0 .. -> canonical.
template <bool PACK>
__global__ void convert_quant_kernel(PackArgs a) {
  const int unit = blockIdx.y, part = blockIdx.z;
  const int D = a.D, bits = a.bits, G = D / 32;
  const int row_bytes = D * bits / 8, blk_bytes = 32 * row_bytes;
  const size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t cblk0 = (size_t)unit * a.n32;                // first canonical block of the unit
  const size_t iblk0 = (size_t)unit * a.cap32 + a.blk0;     // first internal block of the unit
  if (part == 0) {  // K codes: the same bytes, 16 at a time
    const size_t n16 = (size_t)a.n32 * blk_bytes / 16;
    if (gid >= n16) return;
    const u32x4* src = reinterpret_cast<const u32x4*>(PACK ? a.ck + cblk0 * blk_bytes : a.ik + iblk0 * blk_bytes);
    u32x4* dst = reinterpret_cast<u32x4*>(PACK ? a.ik + iblk0 * blk_bytes : a.ck + cblk0 * blk_bytes);
    dst[gid] = src[gid];
  } else if (part == 1) {  // V codes: one internal byte (pack) or canonical byte (unpack)
    if (gid >= (size_t)a.n32 * blk_bytes) return;
    const int blk = (int)(gid / blk_bytes), byte = (int)(gid % blk_bytes);
    const int per = 8 / bits;
    const uint32_t mask = (1u << bits) - 1u;
    uint32_t v = 0;
    if (PACK) {
      const uint8_t* rows = a.cv + (cblk0 + blk) * blk_bytes;
      for (int k = 0; k < per; ++k) {
        int tau, c;
        vcode_inverse(D, bits, byte, k, tau, c);
        const uint32_t code = (rows[tau * row_bytes + c / per] >> (bits * (c % per))) & mask;
        v |= code << (bits * k);
      }
      a.iv[(iblk0 + blk) * blk_bytes + byte] = (uint8_t)v;
    } else {
      const uint8_t* tiled = a.iv + (iblk0 + blk) * blk_bytes;
      const int tau = byte / row_bytes, c0 = (byte % row_bytes) * per;
      for (int k = 0; k < per; ++k) {
        int tb, sh;
        vcode_locate(D, bits, tau, c0 + k, tb, sh);
        v |= ((tiled[tb] >> sh) & mask) << (bits * k);
      }
      a.cv[(cblk0 + blk) * blk_bytes + byte] = (uint8_t)v;
    }
  } else if (part == 2) {  // K meta: one (block, channel) pair
    if (gid >= (size_t)a.n32 * D) return;
    const int blk = (int)(gid / D), c = (int)(gid % D);
    _Float16* plane = reinterpret_cast<_Float16*>(a.ikm + (iblk0 + blk) * D);
    const int pos = kmeta_pos(D, bits, c);
    H2& canon = a.ckm[(cblk0 + blk) * D + c];
    if (PACK) {
      plane[pos] = canon.s;
      plane[D + pos] = canon.z;
    } else {
      canon.s = plane[pos];
      canon.z = plane[D + pos];
    }
  } else {  // V meta: one (token, channel group) pair
    if (gid >= (size_t)a.n32 * 32 * G) return;
    const int t = (int)(gid / G), grp = (int)(gid % G);
    const size_t ci = (cblk0 * 32 + t) * G + grp;
    const size_t ii = ((iblk0 + t / 32) * G + grp) * 32 + vmeta_slot(t % 32);
    if (PACK) a.ivm[ii] = a.cvm[ci];
    else a.cvm[ci] = a.ivm[ii];
  }
}

}  // namespace
}  // namespace vc

using namespace vc;

// Quantise source rows [src_row0, src_row0 + 32 n_blocks) of every unit into
// cache blocks [dst_block, dst_block + n_blocks) of out.
static int quantize_blocks(const char* fn, const void* k_src, const void* v_src, int B, int Hkv, int src_cap, int D,
                           int src_row0, int n_blocks, const vc_kv_comp* out, int dst_block, hipStream_t stream) {
  VC_CHECK(out != nullptr, "%s: out descriptor is NULL", fn);
  VC_CHECK(out->kind == VC_KV_QUANT, "%s: out->kind must be VC_KV_QUANT", fn);
  VC_CHECK(out->bits == 2 || out->bits == 4, "%s: bits must be 2 or 4 (got %d)", fn, out->bits);
  VC_CHECK(B > 0 && Hkv > 0 && src_cap > 0, "%s: bad B/Hkv/src rows (%d,%d,%d)", fn, B, Hkv, src_cap);
  if (D != 64 && D != 128) return fail(VC_ERR_UNSUPPORTED, "%s: D=%d not in {64,128}", fn, D);
  const int cap = quant_cap(out);
  VC_CHECK(cap >= 0 && cap % 32 == 0, "%s: q_cap=%d must be a multiple of 32", fn, cap);
  VC_CHECK(n_blocks >= 0 && src_row0 >= 0 && (long long)src_row0 + 32LL * n_blocks <= src_cap,
           "%s: source rows [%d, %d) outside [0, %d)", fn, src_row0, src_row0 + 32 * n_blocks, src_cap);
  VC_CHECK(dst_block >= 0 && 32LL * (dst_block + n_blocks) <= cap, "%s: blocks [%d, %d) outside the %d-row cache",
           fn, dst_block, dst_block + n_blocks, cap);
  if (n_blocks == 0) return VC_OK;
  VC_CHECK(k_src && v_src && out->k_codes && out->v_codes && out->k_meta && out->v_meta, "%s: null pointer", fn);
  VC_CHECK(aligned(k_src, 2) && aligned(v_src, 2) && aligned(out->k_meta, 4) && aligned(out->v_meta, 4),
           "%s: misaligned pointer", fn);
  const int units = B * Hkv;
  uint8_t* kc = const_cast<uint8_t*>(out->k_codes);
  uint8_t* vcodes = const_cast<uint8_t*>(out->v_codes);
  H2* km = reinterpret_cast<H2*>(const_cast<void*>(out->k_meta));
  H2* vm = reinterpret_cast<H2*>(const_cast<void*>(out->v_meta));
  const uint16_t* ks = static_cast<const uint16_t*>(k_src) + (size_t)src_row0 * D;
  const uint16_t* vs = static_cast<const uint16_t*>(v_src) + (size_t)src_row0 * D;
  const int cap32 = cap / 32;
  dim3 gk(n_blocks, units);
  const int cols = D * out->bits / 8;
  const int G = D / 32;
  dim3 gv((n_blocks * 32 * G + 255) / 256, units);
  dim3 gp((n_blocks * 4 * D * out->bits + 255) / 256, units);
  if (out->bits == 4) {
    quant_k_kernel<4><<<gk, cols, 0, stream>>>(ks, src_cap, D, dst_block, cap32, kc, km);
    quant_v_meta_kernel<4><<<gv, 256, 0, stream>>>(vs, src_cap, D, n_blocks, dst_block, cap32, vm);
    quant_v_pack_kernel<4><<<gp, 256, 0, stream>>>(vs, src_cap, D, n_blocks, dst_block, cap32, vm, vcodes);
  } else {
    quant_k_kernel<2><<<gk, cols, 0, stream>>>(ks, src_cap, D, dst_block, cap32, kc, km);
    quant_v_meta_kernel<2><<<gv, 256, 0, stream>>>(vs, src_cap, D, n_blocks, dst_block, cap32, vm);
    quant_v_pack_kernel<2><<<gp, 256, 0, stream>>>(vs, src_cap, D, n_blocks, dst_block, cap32, vm, vcodes);
  }
  VC_HIP(hipGetLastError());
  return VC_OK;
}

extern "C" int vc_quantize_kv(const void* k_src, const void* v_src, int B, int Hkv, int L_cap, int D,
                              const vc_kv_comp* out, hipStream_t stream) {
  VC_CHECK(out != nullptr, "vc_quantize_kv: out descriptor is NULL");
  const int nq = out->n_quant;
  VC_CHECK(nq >= 0 && nq % 32 == 0 && nq <= L_cap, "vc_quantize_kv: n_quant=%d must be a multiple of 32 <= L_cap",
           nq);
  return quantize_blocks("vc_quantize_kv", k_src, v_src, B, Hkv, L_cap, D, 0, nq / 32, out, 0, stream);
}

extern "C" int vc_quantize_blocks(const void* k_src, const void* v_src, int B, int Hkv, int src_cap, int D,
                                  int src_row0, int n_blocks, const vc_kv_comp* out, int dst_block,
                                  hipStream_t stream) {
  return quantize_blocks("vc_quantize_blocks", k_src, v_src, B, Hkv, src_cap, D, src_row0, n_blocks, out,
                         dst_block, stream);
}

extern "C" int vc_debug_dequant(const vc_kv_comp* comp, int B, int Hkv, int D, int b, int h, int which,
                                float* out, hipStream_t stream) {
  VC_CHECK(comp && out, "vc_debug_dequant: null pointer");
  VC_CHECK(comp->kind == VC_KV_QUANT, "vc_debug_dequant: kind must be VC_KV_QUANT");
  VC_CHECK(comp->bits == 2 || comp->bits == 4, "vc_debug_dequant: bits must be 2 or 4");
  if (D != 64 && D != 128) return fail(VC_ERR_UNSUPPORTED, "vc_debug_dequant: D=%d not in {64,128}", D);
  VC_CHECK(b >= 0 && b < B && h >= 0 && h < Hkv && (which == 0 || which == 1), "vc_debug_dequant: bad index");
  const int nq = comp->n_quant;
  VC_CHECK(nq >= 0 && nq % 32 == 0, "vc_debug_dequant: bad n_quant");
  if (nq == 0) return VC_OK;
  const int cap = quant_cap(comp);
  VC_CHECK(cap >= nq && cap % 32 == 0, "vc_debug_dequant: q_cap=%d below n_quant=%d or not a multiple of 32", cap, nq);
  const size_t unit = (size_t)b * Hkv + h;
  const int row_bytes = D * comp->bits / 8;
  const uint8_t* codes = (which == 0 ? comp->k_codes : comp->v_codes) + unit * cap * row_bytes;
  const H2* meta = reinterpret_cast<const H2*>(which == 0 ? comp->k_meta : comp->v_meta);
  meta += unit * (cap / 32) * D;  // both: D dwords per 32-token block
  VC_CHECK(codes && meta, "vc_debug_dequant: null codes/meta");
  const int n = nq * D;
  dequant_kernel<<<(n + 255) / 256, 256, 0, stream>>>(codes, meta, comp->bits, nq, D, which, out);
  VC_HIP(hipGetLastError());
  return VC_OK;
}

// Shared validation and launch of the canonical <-> internal conversion.
static int convert_quant(const char* fn, bool pack, const uint8_t* k_codes, const uint8_t* v_codes,
                         const void* k_meta, const void* v_meta, int B, int Hkv, int n, int D,
                         const vc_kv_comp* comp, int blk0, hipStream_t stream) {
  VC_CHECK(comp != nullptr, "%s: descriptor is NULL", fn);
  VC_CHECK(comp->kind == VC_KV_QUANT, "%s: kind must be VC_KV_QUANT", fn);
  VC_CHECK(comp->bits == 2 || comp->bits == 4, "%s: bits must be 2 or 4 (got %d)", fn, comp->bits);
  VC_CHECK(B > 0 && Hkv > 0, "%s: bad B/Hkv (%d,%d)", fn, B, Hkv);
  if (D != 64 && D != 128) return fail(VC_ERR_UNSUPPORTED, "%s: D=%d not in {64,128}", fn, D);
  const int cap = quant_cap(comp);
  VC_CHECK(cap >= 0 && cap % 32 == 0, "%s: q_cap=%d must be a multiple of 32", fn, cap);
  VC_CHECK(n >= 0 && n % 32 == 0, "%s: rows n=%d must be a multiple of 32", fn, n);
  VC_CHECK(blk0 >= 0 && 32LL * blk0 + n <= cap, "%s: blocks [%d, %d) outside the %d-row cache", fn, blk0,
           blk0 + n / 32, cap);
  if (n == 0) return VC_OK;
  VC_CHECK(k_codes && v_codes && k_meta && v_meta, "%s: null canonical array", fn);
  VC_CHECK(comp->k_codes && comp->v_codes && comp->k_meta && comp->v_meta, "%s: null cache array", fn);
  VC_CHECK(aligned(k_codes, 16) && aligned(comp->k_codes, 16) && aligned(k_meta, 4) && aligned(v_meta, 4) &&
               aligned(comp->k_meta, 4) && aligned(comp->v_meta, 4),
           "%s: K codes must be 16-byte aligned and metadata 4-byte aligned", fn);
  PackArgs a{};
  a.D = D;
  a.bits = comp->bits;
  a.n32 = n / 32;
  a.cap32 = cap / 32;
  a.blk0 = blk0;
  a.ck = const_cast<uint8_t*>(k_codes);
  a.cv = const_cast<uint8_t*>(v_codes);
  a.ckm = static_cast<H2*>(const_cast<void*>(k_meta));
  a.cvm = static_cast<H2*>(const_cast<void*>(v_meta));
  a.ik = const_cast<uint8_t*>(comp->k_codes);
  a.iv = const_cast<uint8_t*>(comp->v_codes);
  a.ikm = reinterpret_cast<H2*>(const_cast<void*>(comp->k_meta));
  a.ivm = reinterpret_cast<H2*>(const_cast<void*>(comp->v_meta));
  // the largest part: V code bytes (n * D * bits / 8) >= pairs and 16-byte chunks
  const size_t items = (size_t)n * D * comp->bits / 8;
  VC_CHECK((items + 255) / 256 < (1u << 31), "%s: too many rows", fn);
  const dim3 grid((unsigned)((items + 255) / 256), B * Hkv, 4);
  if (pack) convert_quant_kernel<true><<<grid, 256, 0, stream>>>(a);
  else convert_quant_kernel<false><<<grid, 256, 0, stream>>>(a);
  VC_HIP(hipGetLastError());
  return VC_OK;
}

extern "C" int vc_pack_quant(const uint8_t* k_codes, const uint8_t* v_codes, const void* k_meta,
                             const void* v_meta, int B, int Hkv, int n, int D, const vc_kv_comp* out,
                             int dst_block, hipStream_t stream) {
  return convert_quant("vc_pack_quant", true, k_codes, v_codes, k_meta, v_meta, B, Hkv, n, D, out, dst_block,
                       stream);
}

extern "C" int vc_unpack_quant(const vc_kv_comp* in, int B, int Hkv, int D, uint8_t* k_codes, uint8_t* v_codes,
                               void* k_meta, void* v_meta, hipStream_t stream) {
  VC_CHECK(in != nullptr, "vc_unpack_quant: descriptor is NULL");
  return convert_quant("vc_unpack_quant", false, k_codes, v_codes, k_meta, v_meta, B, Hkv, in->n_quant, D, in, 0,
                       stream);
}
