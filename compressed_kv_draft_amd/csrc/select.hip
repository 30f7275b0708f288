// Top-M token selection for the token-dropping compressor on gfx950.
//
// [VC Problem Statement: token dropping keeps part of the context's tokens;
//  VC Architecture Support: token-dropping compressors behind the uniform
//  interface]  The pages give no selection rule; the library keeps the M tokens
// of highest importance score per (batch, kv-head), ties to the lower index,
// as the sorted index list the token-dropped draft gathers.
//
// One workgroup per row.  Scores map to 32-bit keys whose unsigned order is
// the scores' numeric order (-0 taken as +0).  The M-th largest key T is found
// by bisection on its bits, MSB first, each step one pass that counts the keys
// >= a candidate (per-thread counters and a workgroup reduction: no atomics,
// whatever the distribution of the scores).  A last pass walks the row in
// index order, one contiguous stretch per thread, and writes every index with
// key > T, and the first need = M - #(key > T) indices with key == T, at the
// position given by two workgroup exclusive scans.
#include "vc_common.h"

namespace vc {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

__device__ __forceinline__ uint32_t score_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;  // -0 orders as +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Workgroup sum of v (all threads get it).  scratch: kSelWaves words.
__device__ __forceinline__ uint32_t block_sum(uint32_t v, uint32_t* scratch) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();  // scratch free (a previous call may still be reading it)
  if (lane == 0) scratch[wave] = v;
  __syncthreads();
  uint32_t t = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) t += scratch[w];
  return t;
}

// Workgroup exclusive prefix sum of v in thread order.  scratch: kSelWaves words.
__device__ __forceinline__ uint32_t block_exclusive(uint32_t v, uint32_t* scratch) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint32_t inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(inc, o, 64);
    if (lane >= o) inc += y;
  }
  __syncthreads();
  if (lane == 63) scratch[wave] = inc;
  __syncthreads();
  uint32_t before = 0;
  for (int w = 0; w < wave; ++w) before += scratch[w];
  return before + inc - v;
}

__global__ __launch_bounds__(kSelThreads) void select_top_m_kernel(const float* __restrict__ scores, int L, int M,
                                                                   int32_t* __restrict__ keep) {
  __shared__ uint32_t scratch[2][kSelWaves];
  const float* s = scores + (size_t)blockIdx.x * L;
  int32_t* out = keep + (size_t)blockIdx.x * M;
  const int tid = threadIdx.x;
  if (M == L) {  // every index
    for (int i = tid; i < L; i += kSelThreads) out[i] = i;
    return;
  }
  // T = max { t : #(key >= t) >= M }, bit by bit from the top.  Each count
  // pass reads the row as 16-byte vectors (4 in flight per thread) when it is
  // 16-byte aligned, else element by element.
  const bool vec = (reinterpret_cast<uintptr_t>(s) & 15) == 0;
  const int L4 = vec ? L / 4 : 0;
  const float4* s4 = reinterpret_cast<const float4*>(s);
  auto count_ge = [&](uint32_t cand) __attribute__((always_inline)) {
    uint32_t c = 0;
    int i = tid;
    for (; i + 3 * kSelThreads < L4; i += 4 * kSelThreads) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = s4[i + u * kSelThreads];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        c += (score_key(v[u].x) >= cand) + (score_key(v[u].y) >= cand) + (score_key(v[u].z) >= cand) +
             (score_key(v[u].w) >= cand);
    }
    for (; i < L4; i += kSelThreads) {
      const float4 v = s4[i];
      c += (score_key(v.x) >= cand) + (score_key(v.y) >= cand) + (score_key(v.z) >= cand) + (score_key(v.w) >= cand);
    }
    for (int j = 4 * L4 + tid; j < L; j += kSelThreads) c += score_key(s[j]) >= cand ? 1u : 0u;
    return c;
  };
  uint32_t T = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = T | (1u << bit);
    if (block_sum(count_ge(cand), scratch[bit & 1]) >= (uint32_t)M) T = cand;
  }
  // this thread's stretch [i0, i1) of the row, in index order
  const int per = (L + kSelThreads - 1) / kSelThreads;
  const int i0 = min(tid * per, L), i1 = min(i0 + per, L);
  uint32_t cg = 0, ce = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t k = score_key(s[i]);
    cg += k > T ? 1u : 0u;
    ce += k == T ? 1u : 0u;
  }
  uint32_t g = block_exclusive(cg, scratch[0]);
  uint32_t e = block_exclusive(ce, scratch[1]);
  const uint32_t gt_total = block_sum(cg, scratch[0]);
  const uint32_t need = (uint32_t)M - gt_total;  // keys == T kept, 1 <= need <= #(key == T)
  for (int i = i0; i < i1; ++i) {
    const uint32_t k = score_key(s[i]);
    if (k > T) {
      out[g + min(e, need)] = i;
      ++g;
    } else if (k == T) {
      if (e < need) out[g + e] = i;
      ++e;
    }
  }
}

}  // namespace
}  // namespace vc

using namespace vc;

extern "C" int vc_select_top_m(const float* scores, int rows, int L, int M, int32_t* keep_idx, hipStream_t stream) {
  VC_CHECK(rows >= 0 && L >= 0, "vc_select_top_m: rows=%d L=%d", rows, L);
  VC_CHECK(M >= 0 && M <= L, "vc_select_top_m: M=%d outside [0, L=%d]", M, L);
  if (rows == 0 || M == 0) return VC_OK;
  VC_CHECK(scores != nullptr && keep_idx != nullptr, "vc_select_top_m: null scores/keep_idx");
  select_top_m_kernel<<<rows, kSelThreads, 0, stream>>>(scores, L, M, keep_idx);
  VC_HIP(hipGetLastError());
  return VC_OK;
}
