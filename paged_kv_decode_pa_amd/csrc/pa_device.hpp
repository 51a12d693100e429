// Device-side pieces shared by the decode kernels: launch parameters, the
// work-unit schedule and the cross-wave log-sum-exp merge.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kPage = 16;          // tokens per KV page
constexpr int kWaves = 4;          // waves per workgroup; each owns every 4th page
constexpr int kBlock = 64 * kWaves;
constexpr int kMaxGroup = 16;      // query heads per kv head the kernels accept
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct DecodeParams {
  void* out;
  const void* query;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* partial_out;
  float* partial_max;
  float* partial_sum;
  int num_seqs;
  int num_q_heads;
  int num_kv_heads;
  int group;                // num_q_heads / num_kv_heads
  int max_pages_per_seq;
  int64_t num_pages;
  float scale_log2;         // scale * log2(e): scores are kept in base-2 units
  int pages_per_partition;  // 0: the whole context is one unit
  int num_partitions;       // partition slots per (sequence, head) row of the partials
  int grid_partitions;      // partitions per (sequence, kv head) in the unit grid
  int num_units;            // num_seqs * grid_partitions * num_kv_heads
  // The step's appended token per sequence, written by the decode launch
  // itself (NULL new_key: the caller wrote it with pa_reshape_and_cache).
  const void* new_key;      // [num_seqs][num_kv_heads][head_dim]
  const void* new_value;    // [num_seqs][num_kv_heads][head_dim]
  const int64_t* new_slots; // [num_seqs]; < 0 writes nothing
  // Partitions below first_partition[b] of sequence b are computed elsewhere
  // (a shared prefix, once per group); NULL: every partition here.  With
  // four-wave units the grid's partition index counts from first_partition[b]
  // (grid_partitions bounds every sequence's remaining partitions), so no
  // workgroup is spent on a partition computed elsewhere.
  const int32_t* first_partition;
  // Split-KV with four waves per (sequence, partition, kv head) unit instead
  // of one: for batches with few units for the machine.
  bool four_wave_units;
  // Single pass: sequences per round of units over the compute units (see
  // snake_rank); 0 keeps the batch order.
  int snake_period;
};

// Split-KV partials of the pages a group of sequences shares from position 0:
// each shared partition is read once per (group, kv head), its tiles serving
// every member's query heads as the columns of the matrix tiles, and every
// member's partial for that partition is written as the decode's split
// kernel would (o normalised, m in natural-log units, l).
struct PrefixParams {
  const void* query;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  float* partial_out;
  float* partial_max;
  float* partial_sum;
  const int32_t* group_start;       // [num_groups + 1]: members are group_seqs[start[g] ..]
  const int32_t* group_seqs;        // batch indices
  const int32_t* group_partitions;  // [num_groups]: shared partitions from position 0
  int num_groups;
  int num_seqs;                     // members outside [0, num_seqs) are skipped
  int num_q_heads;
  int num_kv_heads;
  int group;                        // query heads per kv head
  int max_pages_per_seq;
  int64_t num_pages;
  float scale_log2;
  int pages_per_partition;
  int num_partitions;               // partition slots per row of the partial arrays
  int max_group_partitions;         // grid bound
  int blocks_per_wave;              // 16-column blocks a wave carries (1 or 2)
  int column_groups;                // ceil(max members * group / (16 * blocks_per_wave))
  int num_units;
};

// Multi-token causal attention over the same cache: sequence b's new query
// tokens are rows query_start[b] .. query_start[b + 1] - 1 of `query`, at
// positions L_b - q_len_b + i.  A work unit is (sequence, kv head, group of
// up to four column blocks): a block's 16 matrix columns are (query token,
// head of the group) pairs, column c = i * group + h.
struct ChunkParams {
  void* out;
  const void* query;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start;
  int num_seqs;
  int num_q_heads;
  int num_kv_heads;
  int group;
  int max_pages_per_seq;
  int64_t num_pages;
  float scale_log2;
  int num_query_tokens;
  int blocks_per_wave;  // column blocks a wave carries: min(4, ceil(max_query_len * group / 16))
  int groups_per_seq;   // ceil(ceil(max_query_len * group / 16) / blocks_per_wave)
  int num_units;        // num_seqs * num_kv_heads * groups_per_seq (* num_partitions if split)
  // Split-KV (pages_per_partition > 0): one wave per (sequence, partition, kv
  // head, column group) writes each of its tokens' partials, rows indexed
  // like `out`: partial_out[(t * num_q_heads + head) * num_partitions + part][D].
  int pages_per_partition;
  int num_partitions;
  float* partial_out;
  float* partial_max;
  float* partial_sum;
  const int32_t* first_partition;  // always NULL here (the unit plan's field)
  int snake_period;                 // single pass: compute units per round of units (0: none)
};

// Number of workgroups: one per work unit.
__host__ __device__ inline int decode_grid(int num_units) { return num_units; }

// Work unit u enumerates (sequence, partition, kv head) with the kv head
// fastest.  Workgroups are dispatched round-robin over the 8 XCDs (block b
// runs on XCD b % 8), so with 8 kv heads (or a multiple) each XCD owns whole
// kv heads: every XCD gets the same share of every sequence, and all the
// sequences that share a prefix page read it through one XCD's L2.  With
// first_partition the partition index counts from the sequence's first.
// A unit whose partition index reaches num_partitions (a sequence's first
// partition plus a grid bound can exceed it) has no partial row: false.
__host__ __device__ inline bool unit_of(const DecodeParams& p, int u, int& seq, int& kvh,
                                        int& part) {
  if (u >= p.num_units) return false;
  kvh = u % p.num_kv_heads;
  const int rest = u / p.num_kv_heads;
  part = rest % p.grid_partitions;
  seq = rest / p.grid_partitions;
  if (p.first_partition) {  // partitions below it are computed elsewhere
    const int f = p.first_partition[seq];
    part += f < 0 ? 0 : f > p.num_partitions ? p.num_partitions : f;
  }
  return part < p.num_partitions;
}

// Page range [lo, hi) of a unit; false when the unit has no tokens.
__host__ __device__ inline bool unit_pages(const DecodeParams& p, int seq, int part, int L,
                                           int& lo, int& hi) {
  int n = (L + kPage - 1) / kPage;
  if (n > p.max_pages_per_seq) n = p.max_pages_per_seq;
  if (p.pages_per_partition > 0) {
    lo = part * p.pages_per_partition;
    hi = lo + p.pages_per_partition < n ? lo + p.pages_per_partition : n;
  } else {
    lo = 0;
    hi = n;
  }
  return lo < hi;
}

__device__ inline float bf16_to_f32(uint16_t x) { return __uint_as_float(uint32_t(x) << 16); }

__device__ inline uint16_t f32_to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));  // round to nearest even
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ static void store(void* base, size_t i, float v) { static_cast<float*>(base)[i] = v; }
};
template <> struct Elem<uint16_t> {
  __device__ static void store(void* base, size_t i, float v) {
    static_cast<uint16_t*>(base)[i] = f32_to_bf16(v);
  }
};

// Rows of accumulators merged through LDS are head_dim + kAccPad floats
// apart.  A matrix-core lane holds four consecutive dims of one column and
// writes them as one 16-byte store; with unpadded rows the 16 columns' lanes
// of a store would all hit the same banks (a 16-way conflict), with the pad
// they cover all 64 banks.
constexpr int kAccPad = 4;

// LDS used by the merge: per wave a reference max and a sum per head, and
// the un-normalised accumulator [wave][head][dim] for the group's heads.
__host__ __device__ inline size_t merge_lds_bytes(int group, int head_dim) {
  return sizeof(float) *
         (2 * kWaves * kMaxGroup + size_t(kWaves) * group * (head_dim + kAccPad));
}

struct MergeLds {
  float* m;    // [kWaves][kMaxGroup]  base-2 reference score
  float* l;    // [kWaves][kMaxGroup]  sum of 2^(s - m)
  float* acc;  // [kWaves][group][D + kAccPad]
  __device__ MergeLds(float* smem) : m(smem), l(smem + kWaves * kMaxGroup),
                                     acc(smem + 2 * kWaves * kMaxGroup) {}
};

// Combine the four waves' online-softmax states of one unit (fixed wave
// order, so the result is deterministic) and store either the final output
// or the unit's split-KV partial.  Every thread of the block must call it.
template <typename OutT, int D>
__device__ inline void merge_and_store(const DecodeParams& p, const MergeLds& s, int seq, int kvh,
                                       int part) {
  __syncthreads();
  const int G = p.group;
  for (int idx = threadIdx.x; idx < G * D; idx += kBlock) {
    const int h = idx / D;
    const int d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s.m[w * kMaxGroup + h]);
    float wsum = 0.f, num = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = s.m[w * kMaxGroup + h];
      const float f = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      wsum += s.l[w * kMaxGroup + h] * f;
      num += s.acc[(w * G + h) * (D + kAccPad) + d] * f;
    }
    const float o = wsum > 0.f ? num / wsum : 0.f;
    const int qh = kvh * G + h;
    if (p.pages_per_partition == 0) {
      Elem<OutT>::store(p.out, (size_t(seq) * p.num_q_heads + qh) * D + d, o);
    } else {
      const size_t row = (size_t(seq) * p.num_q_heads + qh) * p.num_partitions + part;
      p.partial_out[row * D + d] = o;
      if (d == 0) {
        p.partial_max[row] = M * kLn2;  // natural-log units of scale * q.k
        p.partial_sum[row] = wsum;
      }
    }
  }
}

// Split-KV partitions that the merge counts for a context of L tokens:
// ceil(L / partition size), at most num_partitions.  It counts from the raw
// length, while the kernels clamp a length to the block table's width, so
// partitions past the clamped context get empty partials (empty_partials).
__host__ __device__ inline int merged_partitions(const DecodeParams& p, int L) {
  if (L <= 0 || p.pages_per_partition <= 0) return 0;
  const int64_t ps = int64_t(p.pages_per_partition) * kPage;
  const int64_t n = (int64_t(L) + ps - 1) / ps;
  return n < p.num_partitions ? int(n) : p.num_partitions;
}

// Empty partials (o = 0, m = -inf, l = 0; the merge weighs them by 0) for
// partitions [from, to) of one (sequence, kv head): thread tid of nthreads.
template <int D>
__device__ inline void empty_partials(const DecodeParams& p, int seq, int kvh, int from, int to,
                                      int tid, int nthreads) {
  const int G = p.group;
  const int n = to > from ? (to - from) * G * D : 0;
  for (int idx = tid; idx < n; idx += nthreads) {
    const int d = idx % D;
    const int h = (idx / D) % G;
    const int part = from + idx / (D * G);
    const size_t row = (size_t(seq) * p.num_q_heads + kvh * G + h) * p.num_partitions + part;
    p.partial_out[row * D + d] = 0.f;
    if (d == 0) {
      p.partial_max[row] = -INFINITY;
      p.partial_sum[row] = 0.f;
    }
  }
}

// Zero output rows of a unit with an empty context (single pass only).
template <typename OutT, int D>
__device__ inline void store_zeros(const DecodeParams& p, int seq, int kvh) {
  const int G = p.group;
  for (int idx = threadIdx.x; idx < G * D; idx += kBlock) {
    const int qh = kvh * G + idx / D;
    Elem<OutT>::store(p.out, (size_t(seq) * p.num_q_heads + qh) * D + idx % D, 0.f);
  }
}

}  // namespace pa
