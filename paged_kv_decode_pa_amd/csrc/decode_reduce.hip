// Log-sum-exp merge of split-KV partials.  One wave per (sequence, query
// head): lane k holds partition k's reference score and sum (64 partitions
// per pass), a wave max gives M, lane k's weight is l_k * exp(m_k - M), and
// each lane then accumulates D/64 output dims over the partitions in
// increasing order with the weights broadcast from their lanes.
#include "pa_device.hpp"

namespace pa {
namespace {

constexpr int kReduceWaves = 4;  // (sequence, head) rows per workgroup
constexpr int kUnroll = 8;       // partitions whose loads are in flight together

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int x = 1; x < 64; x <<= 1) v = fmaxf(v, __shfl_xor(v, x));
  return v;
}

template <typename OutT, int D>
__global__ __launch_bounds__(64 * kReduceWaves) void decode_reduce_kernel(
    void* out, const float* __restrict__ part_out, const float* __restrict__ part_max,
    const float* __restrict__ part_sum, const int32_t* __restrict__ context_lens, int num_rows,
    int num_q_heads, int partition_size, int max_parts) {
  constexpr int VD = D / 64;  // output dims per lane
  const int row = blockIdx.x * kReduceWaves + (threadIdx.x >> 6);  // seq * num_q_heads + head
  if (row >= num_rows) return;
  const int lane = threadIdx.x & 63;
  const int L = context_lens[row / num_q_heads];
  int n = L > 0 ? (L + partition_size - 1) / partition_size : 0;
  if (n > max_parts) n = max_parts;
  const float* m = part_max + size_t(row) * max_parts;
  const float* s = part_sum + size_t(row) * max_parts;
  const float* o = part_out + size_t(row) * max_parts * D;

  // M over all partitions, 64 per pass.
  float M = -INFINITY;
  for (int base = 0; base < n; base += 64)
    M = fmaxf(M, base + lane < n ? m[base + lane] : -INFINITY);
  M = wave_max(M);

  float acc[VD];
#pragma unroll
  for (int i = 0; i < VD; ++i) acc[i] = 0.f;
  float wsum = 0.f;
  for (int base = 0; base < n; base += 64) {
    const int k = base + lane;
    const float w = k < n ? s[k] * expf(m[k] - M) : 0.f;
    wsum += w;
    const int cnt = min(64, n - base);
    // Eight partitions per step, all loads issued before the first use, so a
    // long context costs n/8 memory round trips instead of n.
    for (int t0 = 0; t0 < cnt; t0 += kUnroll) {
      float v[kUnroll][VD];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const float* ok = o + size_t(base + min(t0 + u, cnt - 1)) * D;
#pragma unroll
        for (int i = 0; i < VD; ++i) v[u][i] = ok[lane + 64 * i];
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (t0 + u < cnt) {
          const float wt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), t0 + u));
#pragma unroll
          for (int i = 0; i < VD; ++i) acc[i] = fmaf(wt, v[u][i], acc[i]);
        }
      }
    }
  }
  // Denominator: lanes hold disjoint partitions; a butterfly sum in a fixed
  // order gives every lane the same total.
#pragma unroll
  for (int x = 1; x < 64; x <<= 1) wsum += __shfl_xor(wsum, x);
#pragma unroll
  for (int i = 0; i < VD; ++i)
    Elem<OutT>::store(out, size_t(row) * D + lane + 64 * i, n > 0 ? acc[i] / wsum : 0.f);
}

template <typename OutT>
hipError_t launch_t(void* out, const float* part_out, const float* part_max, const float* part_sum,
                    const int32_t* context_lens, int num_seqs, int num_q_heads, int head_dim,
                    int partition_size, int max_parts, hipStream_t stream) {
  const int rows = num_seqs * num_q_heads;
  const dim3 grid((rows + kReduceWaves - 1) / kReduceWaves);
  if (head_dim == 128)
    decode_reduce_kernel<OutT, 128><<<grid, 64 * kReduceWaves, 0, stream>>>(
        out, part_out, part_max, part_sum, context_lens, rows, num_q_heads, partition_size, max_parts);
  else
    decode_reduce_kernel<OutT, 64><<<grid, 64 * kReduceWaves, 0, stream>>>(
        out, part_out, part_max, part_sum, context_lens, rows, num_q_heads, partition_size, max_parts);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_reduce(void* out, const float* part_out, const float* part_max,
                                const float* part_sum, const int32_t* context_lens, int num_seqs,
                                int num_q_heads, int head_dim, int partition_size, int max_parts,
                                bool bf16, hipStream_t stream) {
  return bf16 ? launch_t<uint16_t>(out, part_out, part_max, part_sum, context_lens, num_seqs,
                                   num_q_heads, head_dim, partition_size, max_parts, stream)
              : launch_t<float>(out, part_out, part_max, part_sum, context_lens, num_seqs,
                                num_q_heads, head_dim, partition_size, max_parts, stream);
}

}  // namespace pa
