// Full-KV chunk prefetch from the host pool to device memory.
//
// [VC Architecture Support: in long-context decoding the compressed KV stays in
//  GPU HBM while the full KV lives in CPU memory and is loaded over PCIe for
//  verification.  VC Key System Innovations P1: the load runs while other
//  requests draft, so the interconnect and HBM are busy at the same time.]
//
// The host pool is paged with a shuffled page table, so a 4096-token chunk is
// thousands of scattered 64 KiB pages.  One DMA command per page is bound by
// the per-command cost (~10 us each), far below the link rate.  So host threads
// gather the chunk's pages into a pinned staging buffer, in (sequence, page)
// order, and a single host-to-device DMA moves the whole chunk on the caller's
// copy stream.  No kernel runs: the copy engines carry the transfer and every
// compute unit stays with the other group's drafting.
#include <algorithm>
#include <atomic>
#include <cstring>
#include <thread>
#include <vector>

#include "vc_common.h"

using namespace vc;

namespace {

bool is_pinned(const void* p) {
  hipPointerAttribute_t attr;
  const hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return attr.type == hipMemoryTypeHost;
}

constexpr size_t kGatherThreads = 4;

// Copy `n` pages (src slot list -> consecutive staging pages) with up to
// kGatherThreads host threads.
void gather_pages(const char* pool, const std::vector<int32_t>& slots, size_t page_bytes, char* staging) {
  const size_t n = slots.size();
  // Four threads keep up with the host-to-device DMA; more of them compete
  // with it for host memory bandwidth.  Measured on MI355X with the Llama-70B-
  // shaped cycle (two 2 GiB group transfers per cycle): 2 threads 105 ms per
  // cycle, 3: 80, 4: 78, 6: 82, 8: 85, 12 and 16: 90.
  unsigned hw = std::thread::hardware_concurrency();
  size_t threads = std::min<size_t>(hw == 0 ? 4 : hw, kGatherThreads);
  threads = std::min(threads, (n + 63) / 64);  // at least 64 pages per thread
  if (threads <= 1) {
    for (size_t k = 0; k < n; ++k) std::memcpy(staging + k * page_bytes, pool + (size_t)slots[k] * page_bytes, page_bytes);
    return;
  }
  std::atomic<size_t> next{0};
  auto work = [&]() {
    constexpr size_t kBatch = 32;
    for (;;) {
      const size_t k0 = next.fetch_add(kBatch);
      if (k0 >= n) return;
      const size_t k1 = std::min(n, k0 + kBatch);
      for (size_t k = k0; k < k1; ++k)
        std::memcpy(staging + k * page_bytes, pool + (size_t)slots[k] * page_bytes, page_bytes);
    }
  };
  std::vector<std::thread> pool_threads;
  pool_threads.reserve(threads - 1);
  for (size_t t = 1; t < threads; ++t) pool_threads.emplace_back(work);
  work();
  for (auto& th : pool_threads) th.join();
}

}  // namespace

extern "C" int vc_prefetch_full_kv(const void* host_pool, size_t page_bytes, int n_slots, const int32_t* page_table,
                                   int n_seq_total, int pages_per_seq, const int32_t* seq_ids, int n_seq,
                                   int tok_begin, int tok_end, int page_tokens, void* staging, size_t staging_bytes,
                                   void* dev_dst, hipEvent_t staging_free, hipStream_t copy_stream, hipEvent_t done) {
  VC_CHECK(host_pool && page_table, "vc_prefetch_full_kv: null pool or page table");
  VC_CHECK(page_bytes > 0 && n_slots > 0 && n_seq_total > 0 && pages_per_seq > 0 && page_tokens > 0,
           "vc_prefetch_full_kv: bad sizes");
  VC_CHECK(n_seq >= 0 && (n_seq == 0 || seq_ids), "vc_prefetch_full_kv: bad seq list");
  VC_CHECK(tok_begin >= 0 && tok_end >= tok_begin, "vc_prefetch_full_kv: bad token range [%d, %d)", tok_begin,
           tok_end);
  const long long p0 = tok_begin / page_tokens;
  const long long p1 = ((long long)tok_end + page_tokens - 1) / page_tokens;
  VC_CHECK(p1 <= pages_per_seq, "vc_prefetch_full_kv: token range needs %lld pages > pages_per_seq=%d", p1,
           pages_per_seq);
  const size_t n_pages = (size_t)n_seq * (size_t)(p1 - p0);
  const size_t bytes = n_pages * page_bytes;
  if (bytes > 0) {
    VC_CHECK(staging && dev_dst, "vc_prefetch_full_kv: null staging or destination");
    VC_CHECK(staging_bytes >= bytes, "vc_prefetch_full_kv: staging holds %zu bytes < %zu", staging_bytes, bytes);
    // the staging buffer must be page-locked memory the DMA engines can read
    VC_CHECK(is_pinned(staging), "vc_prefetch_full_kv: staging is not pinned host memory");
  }
  std::vector<int32_t> slots;
  slots.reserve(n_pages);
  for (int i = 0; i < n_seq; ++i) {
    const int b = seq_ids[i];
    VC_CHECK(b >= 0 && b < n_seq_total, "vc_prefetch_full_kv: seq id %d out of range", b);
    for (long long p = p0; p < p1; ++p) {
      const int32_t s = page_table[(size_t)b * pages_per_seq + p];
      VC_CHECK(s >= 0 && s < n_slots, "vc_prefetch_full_kv: slot %d of seq %d page %lld out of range", s, b, p);
      slots.push_back(s);
    }
  }
  if (bytes > 0) {
    if (staging_free != nullptr) VC_HIP(hipEventSynchronize(staging_free));
    gather_pages(static_cast<const char*>(host_pool), slots, page_bytes, static_cast<char*>(staging));
    VC_HIP(hipMemcpyAsync(dev_dst, staging, bytes, hipMemcpyHostToDevice, copy_stream));
  }
  if (done != nullptr) VC_HIP(hipEventRecord(done, copy_stream));
  return VC_OK;
}
