// Slot-mapped cache write: token t's K row goes to k_cache[page][h][slot][:]
// as whole 16-byte vectors; its V row is scattered down the dim-major V page
// (v_cache[page][h][d][slot]), one element per dim.  A bit copy, no arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kPage = 16;
constexpr int kThreads = 128;

template <typename T>
__global__ __launch_bounds__(kThreads) void reshape_and_cache_kernel(
    const T* __restrict__ key, const T* __restrict__ value, T* __restrict__ k_cache,
    T* __restrict__ v_cache, const int64_t* __restrict__ slots, int num_kv_heads, int head_dim,
    int64_t num_pages) {
  const int64_t tok = blockIdx.x;
  const int64_t slot = slots[tok];
  if (slot < 0 || slot >= num_pages * kPage) return;  // padding, or out of the pool
  const int64_t page = slot / kPage;
  const int off = int(slot % kPage);
  const int row = num_kv_heads * head_dim;
  constexpr int kVec = 16 / sizeof(T);
  const T* ksrc = key + tok * row;
  for (int i = threadIdx.x; i < row / kVec; i += kThreads) {
    const int h = (i * kVec) / head_dim;
    const int d = (i * kVec) % head_dim;
    const u32x4 x = *reinterpret_cast<const u32x4*>(ksrc + i * kVec);
    *reinterpret_cast<u32x4*>(k_cache + ((page * num_kv_heads + h) * kPage + off) * head_dim + d) = x;
  }
  const T* vsrc = value + tok * row;
  for (int i = threadIdx.x; i < row; i += kThreads) {
    const int h = i / head_dim;
    const int d = i % head_dim;
    v_cache[((page * num_kv_heads + h) * head_dim + d) * kPage + off] = vsrc[i];
  }
}

}  // namespace

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* k_cache,
                                    void* v_cache, const int64_t* slots, int64_t num_tokens,
                                    int num_kv_heads, int head_dim, int64_t num_pages, bool bf16,
                                    hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(num_tokens));
  if (bf16)
    reshape_and_cache_kernel<uint16_t><<<grid, kThreads, 0, stream>>>(
        static_cast<const uint16_t*>(key), static_cast<const uint16_t*>(value),
        static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache), slots, num_kv_heads,
        head_dim, num_pages);
  else
    reshape_and_cache_kernel<float><<<grid, kThreads, 0, stream>>>(
        static_cast<const float*>(key), static_cast<const float*>(value),
        static_cast<float*>(k_cache), static_cast<float*>(v_cache), slots, num_kv_heads, head_dim,
        num_pages);
  return hipGetLastError();
}

}  // namespace pa
