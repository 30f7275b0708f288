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

struct Partial {  // split-K partial of one (row): unnormalised o, running max (log2 units), sum
  float m, l;
};

}  // namespace vc
