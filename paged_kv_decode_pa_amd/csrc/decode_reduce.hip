// Log-sum-exp merge of split-KV partials: one workgroup per (sequence, query
// head), one thread per output dim, partitions summed in increasing order.
#include "pa_device.hpp"

namespace pa {
namespace {

template <typename OutT>
__global__ void decode_reduce_kernel(void* out, const float* __restrict__ part_out,
                                     const float* __restrict__ part_max,
                                     const float* __restrict__ part_sum,
                                     const int32_t* __restrict__ context_lens, int num_q_heads,
                                     int head_dim, int partition_size, int max_parts) {
  const int row = blockIdx.x;  // seq * num_q_heads + head
  const int seq = row / num_q_heads;
  const int L = context_lens[seq];
  int n = L > 0 ? (L + partition_size - 1) / partition_size : 0;
  if (n > max_parts) n = max_parts;
  const float* m = part_max + size_t(row) * max_parts;
  const float* s = part_sum + size_t(row) * max_parts;
  const float* o = part_out + size_t(row) * max_parts * head_dim;
  float M = -INFINITY;
  for (int k = 0; k < n; ++k) M = fmaxf(M, m[k]);
  for (int d = threadIdx.x; d < head_dim; d += blockDim.x) {
    float wsum = 0.f, num = 0.f;
    for (int k = 0; k < n; ++k) {
      const float wk = s[k] * expf(m[k] - M);
      wsum += wk;
      num += wk * o[size_t(k) * head_dim + d];
    }
    Elem<OutT>::store(out, size_t(row) * head_dim + d, n > 0 ? num / wsum : 0.f);
  }
}

}  // namespace

hipError_t launch_decode_reduce(void* out, const float* part_out, const float* part_max,
                                const float* part_sum, const int32_t* context_lens, int num_seqs,
                                int num_q_heads, int head_dim, int partition_size, int max_parts,
                                bool bf16, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(num_seqs) * num_q_heads);
  if (bf16)
    decode_reduce_kernel<uint16_t><<<grid, head_dim, 0, stream>>>(
        out, part_out, part_max, part_sum, context_lens, num_q_heads, head_dim, partition_size,
        max_parts);
  else
    decode_reduce_kernel<float><<<grid, head_dim, 0, stream>>>(
        out, part_out, part_max, part_sum, context_lens, num_q_heads, head_dim, partition_size,
        max_parts);
  return hipGetLastError();
}

}  // namespace pa
