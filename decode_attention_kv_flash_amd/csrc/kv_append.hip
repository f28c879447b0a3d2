// Append of the new token's cache entries, the step right before attention.
//
// Decoding writes the current token into the cache and then attends over it
// ("Attention Optimizations", "DSA: DeepSeek Sparse Attention", "Computation
// Path": update_cache of the 576-value latent row [c_KV | k_pe] and of the
// 128-value indexer key; for GQA, one K and one V row per KV head).  The
// cache is paged: the entry goes to slot pos % page_size of the physical page
// the sequence's block table names for logical page pos / page_size ("All
// the attentions", section 8, PagedAttention).
//
// Rolling buffer ("All the attentions", section 4: with a sliding window the
// cache becomes a rolling buffer of fixed size, new entries replacing the
// oldest): with ring_pages > 0, a write into logical page j >= fixed_pages +
// ring_pages first points table entry j at the physical page of entry
// j - ring_pages, which has left the window.  The first fixed_pages entries
// (the attention-sink tokens' pages) are never recycled.  The attention
// kernels need nothing else: they never read outside the window and sinks.
//
// One workgroup per sequence: thread 0 resolves (and if needed recycles) the
// page, then the workgroup copies the sequence's rows in 16-byte pieces.
#include "common.hpp"
#include "internal.hpp"

namespace dattn {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void kv_append_kernel(const KvAppendArgs a) {
  const int b = blockIdx.x;
  const int pos = a.positions[b];
  __shared__ int s_phys;
  if (threadIdx.x == 0) {
    int phys = -1;
    if (pos >= 0) {
      if (a.page_table) {
        int32_t* row = a.page_table + (size_t)b * a.max_pages;
        const int j = pos >> a.log2_page;
        if (j < a.max_pages) {
          if (a.ring_pages > 0 && j >= a.fixed_pages + a.ring_pages) row[j] = row[j - a.ring_pages];
          phys = row[j];
        }
      } else if (pos < a.page_size) {
        phys = b;  // contiguous cache: one page of S_max = page_size slots per sequence
      }
    }
    s_phys = phys;
  }
  __syncthreads();
  const int phys = s_phys;
  if (phys < 0) return;  // no append for this sequence, or a position past the cache
  const size_t slot = a.page_table ? (size_t)(pos & (a.page_size - 1)) : (size_t)pos;
  const int pieces = a.row_bytes / 16;            // per head row
  const int per_cache = a.heads * pieces;
  const int total = (a.cache1 ? 2 : 1) * per_cache;
  for (int i = threadIdx.x; i < total; i += kThreads) {
    const int which = i / per_cache;               // 0: first cache (K / rows), 1: second (V)
    const int hp = i - which * per_cache;
    const int h = hp / pieces, p = hp - h * pieces;
    const char* src = (const char*)(which ? a.new1 : a.new0) +
                      (((size_t)b * a.heads + h) * a.row_bytes + (size_t)p * 16);
    char* dst = (char*)(which ? a.cache1 : a.cache0) +
                ((((size_t)phys * a.heads + h) * a.page_size + slot) * a.row_bytes + (size_t)p * 16);
    *(uint4*)dst = *(const uint4*)src;
  }
}

}  // namespace

hipError_t launch_kv_append(const KvAppendArgs& a, hipStream_t s) {
  launch_kernel(kv_append_kernel, a.B, kThreads, s, a);
  return hipGetLastError();
}

}  // namespace dattn
