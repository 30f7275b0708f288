// Full-KV page prefetch from a pinned host pool into the device pool.
//
// [VC Architecture Support: in long-context decoding the compressed KV stays in
//  GPU HBM while the full KV lives in CPU memory and is loaded over PCIe for
//  verification.  VC Key System Innovations P1: the load runs while other
//  requests draft, so the interconnect and HBM are busy at the same time.]
//
// Host-side only: builds the list of page slots (the same slot in both pools),
// sorts it, merges runs of consecutive slots and issues one host-to-device DMA
// copy per run on the caller's copy stream.  No kernel runs.
#include <algorithm>
#include <vector>

#include "vc_common.h"

using namespace vc;

extern "C" int vc_prefetch_full_kv(const void* host_pool, void* dev_pool, size_t page_bytes, int n_slots,
                                   const int32_t* page_table, int n_seq_total, int pages_per_seq,
                                   const int32_t* seq_ids, int n_seq, int tok_begin, int tok_end,
                                   int page_tokens, hipStream_t copy_stream, hipEvent_t done) {
  VC_CHECK(host_pool && dev_pool && page_table, "vc_prefetch_full_kv: null pool or page table");
  VC_CHECK(page_bytes > 0 && n_slots > 0 && n_seq_total > 0 && pages_per_seq > 0 && page_tokens > 0,
           "vc_prefetch_full_kv: bad sizes");
  VC_CHECK(n_seq >= 0 && (n_seq == 0 || seq_ids), "vc_prefetch_full_kv: bad seq list");
  VC_CHECK(tok_begin >= 0 && tok_end >= tok_begin, "vc_prefetch_full_kv: bad token range [%d, %d)", tok_begin,
           tok_end);
  const long long p0 = tok_begin / page_tokens;
  const long long p1 = ((long long)tok_end + page_tokens - 1) / page_tokens;
  VC_CHECK(p1 <= pages_per_seq, "vc_prefetch_full_kv: token range needs %lld pages > pages_per_seq=%d", p1,
           pages_per_seq);

  // the host pool must be page-locked memory the DMA engines can read
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, host_pool);
  if (e != hipSuccess || attr.type != hipMemoryTypeHost) {
    (void)hipGetLastError();
    return fail(VC_ERR_INVALID, "vc_prefetch_full_kv: host_pool is not pinned host memory");
  }

  std::vector<int32_t> slots;
  slots.reserve((size_t)n_seq * (size_t)(p1 - p0));
  for (int i = 0; i < n_seq; ++i) {
    const int b = seq_ids[i];
    VC_CHECK(b >= 0 && b < n_seq_total, "vc_prefetch_full_kv: seq id %d out of range", b);
    for (long long p = p0; p < p1; ++p) {
      const int32_t s = page_table[(size_t)b * pages_per_seq + p];
      VC_CHECK(s >= 0 && s < n_slots, "vc_prefetch_full_kv: slot %d of seq %d page %lld out of range", s, b, p);
      slots.push_back(s);
    }
  }
  if (!slots.empty()) {
    std::sort(slots.begin(), slots.end());
    slots.erase(std::unique(slots.begin(), slots.end()), slots.end());
    std::vector<void*> dsts, srcs;
    std::vector<size_t> sizes;
    size_t i = 0;
    while (i < slots.size()) {
      size_t j = i + 1;
      while (j < slots.size() && slots[j] == slots[j - 1] + 1) ++j;
      const size_t off = (size_t)slots[i] * page_bytes;
      dsts.push_back(static_cast<char*>(dev_pool) + off);
      srcs.push_back(const_cast<char*>(static_cast<const char*>(host_pool)) + off);
      sizes.push_back((j - i) * page_bytes);
      i = j;
    }
    for (size_t r = 0; r < dsts.size(); ++r)
      VC_HIP(hipMemcpyAsync(dsts[r], srcs[r], sizes[r], hipMemcpyHostToDevice, copy_stream));
  }
  if (done != nullptr) VC_HIP(hipEventRecord(done, copy_stream));
  return VC_OK;
}
