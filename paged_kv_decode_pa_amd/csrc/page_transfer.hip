// Page export / import: the on-GPU half of moving a sequence's KV cache
// between engines (prefill instance -> decode instance, llm-d blog post,
// disaggregated prefill/decode section).  Export gathers whole pages, in the
// order of a page-id list (a block-table row, say), into one contiguous
// buffer; import scatters such a buffer into pages of a pool.  Both are bit
// copies of each page's block, which holds every kv head in the pool's own
// layout:
//     buffer[0][i] = k_cache[page_ids[i]]   ([num_kv_heads][16][head_dim])
//     buffer[1][i] = v_cache[page_ids[i]]   ([num_kv_heads][head_dim][16])
// so a receiving pool of the same shape needs no re-layout.
//
// One workgroup per (page, pool) block; each thread moves 16-byte vectors,
// four in flight, with the nontemporal hint on both sides (every byte is
// touched once).  A block is Hkv * 16 * D * esz bytes, a multiple of 2 KB.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kUnroll = 4;

template <bool Export>
__global__ __launch_bounds__(kThreads) void page_copy_kernel(char* __restrict__ buf,
                                                             char* __restrict__ k_cache,
                                                             char* __restrict__ v_cache,
                                                             const int32_t* __restrict__ page_ids,
                                                             int64_t num_ids, int64_t num_pages,
                                                             int64_t block_bytes) {
  const int64_t i = blockIdx.x >> 1;  // position in the id list
  const int which = blockIdx.x & 1;   // 0 = K block, 1 = V block
  if (i >= num_ids) return;
  const int64_t page = page_ids[i];
  if (page < 0 || page >= num_pages) return;  // skipped: nothing read or written
  char* pool = (which ? v_cache : k_cache) + page * block_bytes;
  char* side = buf + (which * num_ids + i) * block_bytes;
  const char* src = Export ? pool : side;
  char* dst = Export ? side : pool;
  const int64_t n = block_bytes / 16;
  int64_t v = threadIdx.x;
  for (; v + (kUnroll - 1) * kThreads < n; v += kUnroll * kThreads) {
    u32x4 x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      x[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + v + u * kThreads);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      __builtin_nontemporal_store(x[u], reinterpret_cast<u32x4*>(dst) + v + u * kThreads);
  }
  for (; v < n; v += kThreads)
    __builtin_nontemporal_store(__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + v),
                                reinterpret_cast<u32x4*>(dst) + v);
}

}  // namespace

hipError_t launch_page_copy(bool export_dir, void* buf, void* k_cache, void* v_cache,
                            const int32_t* page_ids, int64_t num_ids, int64_t num_pages,
                            int64_t block_bytes, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(2 * num_ids));
  if (export_dir)
    page_copy_kernel<true><<<grid, kThreads, 0, stream>>>(
        static_cast<char*>(buf), static_cast<char*>(k_cache), static_cast<char*>(v_cache),
        page_ids, num_ids, num_pages, block_bytes);
  else
    page_copy_kernel<false><<<grid, kThreads, 0, stream>>>(
        static_cast<char*>(buf), static_cast<char*>(k_cache), static_cast<char*>(v_cache),
        page_ids, num_ids, num_pages, block_bytes);
  return hipGetLastError();
}

}  // namespace pa
