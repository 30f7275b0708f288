// Internal helpers shared by the libvc translation units (host + device).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include <string>

#include "../../include/vc.h"

namespace vc {

// ---------------------------------------------------------------- errors ---
void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int hip_fail(hipError_t e, const char* what);
int num_cus();  // compute units of the current device (cached per device)

#define VC_CHECK(cond, ...)                          \
  do {                                               \
    if (!(cond)) return ::vc::fail(VC_ERR_INVALID, __VA_ARGS__); \
  } while (0)

#define VC_HIP(call)                                 \
  do {                                               \
    hipError_t e_ = (call);                          \
    if (e_ != hipSuccess) return ::vc::hip_fail(e_, #call); \
  } while (0)

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Rows per (batch, kv-head) the code and metadata arrays of a QUANT cache hold.
inline int quant_cap(const vc_kv_comp* c) { return c->q_cap > 0 ? c->q_cap : c->n_quant; }

// ---------------------------------------------------------- device utils ---
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Lane shuffles inside a 64-wide wavefront.
__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }

// ------------------------------------------------ tiled V code layout ---
// V codes of 32 consecutive tokens (a "block") are stored as the B operands of
// the draft kernel's P.V matrix product, so that one wavefront reads a block
// with one coalesced load of D*bits/16 bytes per lane and unpacks it with bit
// masks only.  Token tau (0..31) of a block and channel c (0..D-1) map to
//   lane  = 16 * q + (c % 16)       with q = (tau % 16) / 4
//   slot  e = tau % 4 + 4 * (tau / 16)   (k index of the 16x16x32 product)
//   pair  i = e / 2, half hf = e % 2, column tile ct = c / 16
//   pi    = i * (D / 16) + ct,   pairs per dword PPD = 16 / bits
//   dword = pi / PPD, position j = pi % PPD
//   bit   = bits * j + 16 * hf   inside that dword of the lane's chunk
// A lane's chunk holds D*bits/16 bytes; chunks follow each other by lane, and
// blocks by block index.  The two codes of a pair sit at bit b and b + 16 of
// one dword, so masking the dword gives both as f16 bit patterns at once.
__host__ __device__ inline void vcode_locate(int D, int bits, int tau, int c, int& byte, int& shift) {
  const int q = (tau % 16) / 4, e = tau % 4 + 4 * (tau / 16);
  const int lane = 16 * q + c % 16, i = e / 2, hf = e % 2, ct = c / 16;
  const int pi = i * (D / 16) + ct, ppd = 16 / bits;
  const int dword = pi / ppd, j = pi % ppd;
  const int bit = bits * j + 16 * hf;
  byte = lane * (D * bits / 16) + dword * 4 + bit / 8;
  shift = bit % 8;
}

// Inverse of vcode_locate for the k-th code (k < 8 / bits) of block byte `byte`.
__host__ __device__ inline void vcode_inverse(int D, int bits, int byte, int k, int& tau, int& c) {
  const int lb = D * bits / 16;
  const int lane = byte / lb, rem = byte % lb;
  const int dword = rem / 4, bpos = rem % 4;
  const int hf = bpos / 2;
  const int bit = 8 * (bpos % 2) + bits * k;  // bit inside the 16-bit half
  const int j = bit / bits;
  const int pi = dword * (16 / bits) + j;
  const int i = pi / (D / 16), ct = pi % (D / 16);
  const int e = 2 * i + hf, q = lane / 16;
  tau = e < 4 ? 4 * q + e : 16 + 4 * q + (e - 4);
  c = 16 * ct + lane % 16;
}

// K metadata of one 32-token block: a plane of D f16 scales, then a plane of D
// f16 zeros, both in "pair order": channel c sits at f16 index kmeta_pos(c), so
// that dword w of a plane holds the two channels whose codes one code dword
// carries at bits b and b + 16 (the matrix-core operand pairs).
__host__ __device__ inline int kmeta_pos(int D, int bits, int c) {
  const int cpd = 32 / bits, ppd = cpd / 2, nks = D / 32;
  const int quad = c / (D / 4), r = c % (D / 4);
  const int d = r / cpd, rem = r % cpd;
  const int h = rem / ppd, j = rem % ppd;
  const int pi = d * ppd + j;
  return 2 * ((quad * nks + pi / 4) * 4 + pi % 4) + h;
}

// V metadata of one 32-token block: [D/32 groups][32 slots] {scale, zero}; token
// tau of the block sits in slot 8 ((tau % 16) / 4) + tau % 4 + 4 (tau / 16), the
// token order of the score tiles.
__host__ __device__ inline int vmeta_slot(int tau) { return 8 * ((tau % 16) / 4) + tau % 4 + 4 * (tau / 16); }

struct Partial {  // split-K partial of one (row): unnormalised o, running max (log2 units), sum
  float m, l;
};

}  // namespace vc
