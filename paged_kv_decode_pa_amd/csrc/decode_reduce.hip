// Log-sum-exp merge of split-KV partials.  One wave per (sequence, query
// head): lane k holds partition k's reference score and sum (64 partitions
// per chunk), a wave max gives M, lane k's weight is l_k * exp(m_k - M), and
// each lane accumulates D/64 output dims over the partitions in increasing
// order with the weights broadcast from their lanes.
//
// The pass is latency bound (a few loads per row, in dependent steps), so
// the output rows are read 16 partitions at a time in two register sets in
// ping-pong, and the first set is requested together with the scores and
// sums: a row of up to 16 partitions costs one memory round trip, 48
// partitions three.
#include <limits.h>

#include "pa_device.hpp"

namespace pa {
namespace {

constexpr int kReduceWaves = 4;  // (sequence, head) rows per workgroup
constexpr int kGroup = 16;       // partitions per register set (a chunk holds 64 / kGroup sets)

// Wavefront max and sum from the device library (cross-lane moves within the
// vector unit, in a fixed order): the max is exact in any order, and the sum's
// fixed order keeps the merge deterministic.
extern "C" __device__ __attribute__((const)) float __ockl_wfred_max_f32(float);
extern "C" __device__ __attribute__((const)) float __ockl_wfred_add_f32(float);

__device__ inline float wave_max(float v) { return __ockl_wfred_max_f32(v); }

template <int D>
struct RowSet {
  float v[kGroup][D / 64];
  // Output rows of partitions g*16 .. g*16+15 (clamped to the last one).
  __device__ void load(const float* o, int g, int n, int lane) {
#pragma unroll
    for (int u = 0; u < kGroup; ++u) {
      const float* r = o + size_t(min(g * kGroup + u, n - 1)) * D;
#pragma unroll
      for (int i = 0; i < D / 64; ++i) v[u][i] = r[lane + 64 * i];
    }
  }
  // acc += w_t * o_t for the set's partitions below n, in increasing t; the
  // weight of partition t sits in lane t % 64 of `w`.
  __device__ void use(float (&acc)[D / 64], float w, int g, int n) const {
#pragma unroll
    for (int u = 0; u < kGroup; ++u) {
      const int t = g * kGroup + u;
      if (t < n) {
        const float wt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), t & 63));
#pragma unroll
        for (int i = 0; i < D / 64; ++i) acc[i] = fmaf(wt, v[u][i], acc[i]);
      }
    }
  }
};

// Rows of the multi-token split form: grid row (b * max_query_len + i) *
// num_q_heads + h is token i of sequence b, head h; its partials and output
// sit at token row query_start[b] + i, and its partitions are those of the
// sequence's context.  Decode rows have no token table (query_start NULL).
// The multi-token kernels clamp a context to the block table's width
// (max_context tokens) and compute partitions of the clamped context only.
struct TokenRows {
  const int32_t* query_start;  // [num_seqs + 1] or NULL
  int max_query_len;
  int num_query_tokens;
  int max_context;             // INT_MAX for decode rows
};

template <typename OutT, int D>
__global__ __launch_bounds__(64 * kReduceWaves) void decode_reduce_kernel(
    void* out, const float* __restrict__ part_out, const float* __restrict__ part_max,
    const float* __restrict__ part_sum, const int32_t* __restrict__ context_lens, int num_rows,
    int num_q_heads, int partition_size, int max_parts, TokenRows tok) {
  constexpr int VD = D / 64;  // output dims per lane
  int row = blockIdx.x * kReduceWaves + (threadIdx.x >> 6);  // seq * num_q_heads + head
  if (row >= num_rows) return;
  const int lane = threadIdx.x & 63;
  int seq = row / num_q_heads;
  if (tok.query_start) {
    const int h = row % num_q_heads;
    const int i = seq % tok.max_query_len;
    seq /= tok.max_query_len;
    const int q0 = tok.query_start[seq];
    const int q_len = tok.query_start[seq + 1] - q0;
    if (i >= q_len || q0 < 0 || q0 + q_len > tok.num_query_tokens) return;
    row = (q0 + i) * num_q_heads + h;
  }
  const int L = min(context_lens[seq], tok.max_context);
  int n = L > 0 ? int((int64_t(L) + partition_size - 1) / partition_size) : 0;
  if (n > max_parts) n = max_parts;
  float acc[VD];
#pragma unroll
  for (int i = 0; i < VD; ++i) acc[i] = 0.f;
  float wsum = 0.f;
  if (n > 0) {
    const float* m = part_max + size_t(row) * max_parts;
    const float* s = part_sum + size_t(row) * max_parts;
    const float* o = part_out + size_t(row) * max_parts * D;

    // Requested together: chunk 0's scores and sums, and the first set of rows.
    RowSet<D> a, b;
    const float m0 = lane < n ? m[lane] : -INFINITY;
    const float s0 = lane < n ? s[lane] : 0.f;
    a.load(o, 0, n, lane);
    float M = m0;
    for (int base = 64; base < n; base += 64)
      M = fmaxf(M, base + lane < n ? m[base + lane] : -INFINITY);
    M = wave_max(M);

    const int sets = (n + kGroup - 1) / kGroup;
    float w = 0.f;
    for (int g = 0; g < sets; g += 2) {
      if ((g * kGroup) % 64 == 0) {  // first set of a chunk: its weights
        const int k = g * kGroup + lane;
        w = k == lane ? (lane < n ? s0 * expf(m0 - M) : 0.f)
                      : (k < n ? s[k] * expf(m[k] - M) : 0.f);
        wsum += w;
      }
      b.load(o, g + 1, n, lane);
      a.use(acc, w, g, n);
      if (g + 1 >= sets) break;
      if (g + 2 < sets) a.load(o, g + 2, n, lane);
      b.use(acc, w, g + 1, n);
    }
  }
  // Denominator: lanes hold disjoint partitions; the wavefront sum (a fixed
  // order) gives every lane the same total.
  wsum = __ockl_wfred_add_f32(wsum);
#pragma unroll
  for (int i = 0; i < VD; ++i)
    Elem<OutT>::store(out, size_t(row) * D + lane + 64 * i, n > 0 ? acc[i] / wsum : 0.f);
}

template <typename OutT>
hipError_t launch_t(void* out, const float* part_out, const float* part_max, const float* part_sum,
                    const int32_t* context_lens, int rows, int num_q_heads, int head_dim,
                    int partition_size, int max_parts, TokenRows tok, hipStream_t stream) {
  const dim3 grid((rows + kReduceWaves - 1) / kReduceWaves);
  if (head_dim == 128)
    decode_reduce_kernel<OutT, 128><<<grid, 64 * kReduceWaves, 0, stream>>>(
        out, part_out, part_max, part_sum, context_lens, rows, num_q_heads, partition_size,
        max_parts, tok);
  else
    decode_reduce_kernel<OutT, 64><<<grid, 64 * kReduceWaves, 0, stream>>>(
        out, part_out, part_max, part_sum, context_lens, rows, num_q_heads, partition_size,
        max_parts, tok);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_reduce(void* out, const float* part_out, const float* part_max,
                                const float* part_sum, const int32_t* context_lens, int num_seqs,
                                int num_q_heads, int head_dim, int partition_size, int max_parts,
                                bool bf16, hipStream_t stream) {
  const TokenRows none{nullptr, 1, 0, INT_MAX};
  const int rows = num_seqs * num_q_heads;
  return bf16 ? launch_t<uint16_t>(out, part_out, part_max, part_sum, context_lens, rows,
                                   num_q_heads, head_dim, partition_size, max_parts, none, stream)
              : launch_t<float>(out, part_out, part_max, part_sum, context_lens, rows,
                                num_q_heads, head_dim, partition_size, max_parts, none, stream);
}

hipError_t launch_chunk_reduce(void* out, const float* part_out, const float* part_max,
                               const float* part_sum, const int32_t* context_lens,
                               const int32_t* query_start, int num_seqs, int max_query_len,
                               int num_query_tokens, int num_q_heads, int head_dim,
                               int partition_size, int max_parts, int max_pages_per_seq,
                               hipStream_t stream) {
  const TokenRows tok{query_start, max_query_len, num_query_tokens,
                      max_pages_per_seq > INT_MAX / kPage ? INT_MAX : max_pages_per_seq * kPage};
  const int rows = num_seqs * max_query_len * num_q_heads;
  return launch_t<uint16_t>(out, part_out, part_max, part_sum, context_lens, rows, num_q_heads,
                            head_dim, partition_size, max_parts, tok, stream);
}

}  // namespace pa
