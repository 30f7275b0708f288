// Greedy token selection and prefix acceptance.
//
// [VC Core Algorithm: acceptance; VC Experimental Results: identical output
//  under greedy decoding]  The rule: n is the position of the first draft that
//  differs from the verifier's greedy token at that position (k when none
//  does); the drafts before it are kept and the verifier's token at n follows
//  them, so every round emits n + 1 tokens and the next round starts there.
#include "vc_common.h"

namespace vc {
namespace {

constexpr int kArgThreads = 1024;
constexpr int kArgLoads = 8;  // 16-byte loads in flight per thread

// (value, index) max with ties to the lower index; NaN never wins a compare.
__device__ __forceinline__ void better(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

// One workgroup per row: strided scan, then wavefront and LDS reductions.
__global__ __launch_bounds__(kArgThreads) void argmax_kernel(const float* __restrict__ x, int V, int32_t* __restrict__ ids) {
  const int row = blockIdx.x;
  const float* p = x + (size_t)row * V;
  float bv = kNegInf;
  int bi = 0x7fffffff;
  if ((V & 3) == 0 && (reinterpret_cast<uintptr_t>(p) & 15) == 0) {
    // 16-byte loads, kArgLoads of them in flight per thread before any compare
    // (the running best is order-independent: ties go to the lowest index)
    const float4* p4 = reinterpret_cast<const float4*>(p);
    const int n4 = V / 4;
    for (int i = threadIdx.x; i < n4; i += kArgLoads * kArgThreads) {
      float4 w[kArgLoads];
#pragma unroll
      for (int u = 0; u < kArgLoads; ++u) {
        const int j = i + u * kArgThreads;
        w[u] = j < n4 ? p4[j] : make_float4(kNegInf, kNegInf, kNegInf, kNegInf);
      }
#pragma unroll
      for (int u = 0; u < kArgLoads; ++u) {
        const int j = 4 * (i + u * kArgThreads);
        better(bv, bi, w[u].x, j);
        better(bv, bi, w[u].y, j + 1);
        better(bv, bi, w[u].z, j + 2);
        better(bv, bi, w[u].w, j + 3);
      }
    }
  } else {
    for (int i = threadIdx.x; i < V; i += kArgThreads) better(bv, bi, p[i], i);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float ov = __shfl_xor(bv, m, 64);
    const int oi = __shfl_xor(bi, m, 64);
    better(bv, bi, ov, oi);
  }
  __shared__ float sv[kArgThreads / 64];
  __shared__ int si[kArgThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    sv[wave] = bv;
    si[wave] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kArgThreads / 64; ++w) better(bv, bi, sv[w], si[w]);
    // all-NaN (or empty) rows fall back to index 0
    ids[row] = (bi >= 0 && bi < V) ? bi : 0;
  }
}

// out_ids holds y_0..y_k of every sequence; keep d_0..d_{n-1} (== y_0..y_{n-1}),
// y_n, and pad the rest with -1.
__global__ void accept_kernel(const int32_t* __restrict__ draft, int B, int k, int32_t* __restrict__ out,
                              int32_t* __restrict__ n_accept) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int32_t* d = draft + (size_t)b * k;
  int32_t* y = out + (size_t)b * (k + 1);
  int n = k;
  for (int j = 0; j < k; ++j) {
    if (d[j] != y[j]) {
      n = j;
      break;
    }
  }
  for (int j = n + 1; j <= k; ++j) y[j] = -1;
  n_accept[b] = n;
}

}  // namespace
}  // namespace vc

using namespace vc;

extern "C" int vc_argmax(const float* logits, int rows, int V, int32_t* ids, hipStream_t stream) {
  VC_CHECK(logits && ids, "vc_argmax: null pointer");
  VC_CHECK(rows >= 0 && V > 0, "vc_argmax: rows=%d V=%d", rows, V);
  VC_CHECK(aligned(logits, 16), "vc_argmax: logits must be 16-byte aligned");
  if (rows == 0) return VC_OK;
  argmax_kernel<<<rows, kArgThreads, 0, stream>>>(logits, V, ids);
  VC_HIP(hipGetLastError());
  return VC_OK;
}

extern "C" int vc_accept(const int32_t* draft_ids, const float* verify_logits, int B, int k, int V,
                         int32_t* out_ids, int32_t* n_accept, hipStream_t stream) {
  VC_CHECK(verify_logits && out_ids && n_accept, "vc_accept: null pointer");
  VC_CHECK(B > 0 && k >= 0 && V > 0, "vc_accept: B=%d k=%d V=%d", B, k, V);
  VC_CHECK(k == 0 || draft_ids != nullptr, "vc_accept: null draft_ids");
  VC_CHECK(aligned(verify_logits, 16), "vc_accept: logits must be 16-byte aligned");
  const int rows = B * (k + 1);
  argmax_kernel<<<rows, kArgThreads, 0, stream>>>(verify_logits, V, out_ids);
  VC_HIP(hipGetLastError());
  accept_kernel<<<(B + 255) / 256, 256, 0, stream>>>(draft_ids, B, k, out_ids, n_accept);
  VC_HIP(hipGetLastError());
  return VC_OK;
}
