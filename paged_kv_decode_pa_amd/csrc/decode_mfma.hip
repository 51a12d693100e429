// bf16 paged decode on the matrix cores (gfx950): the per-page step
// (wave_attn.hpp) in two kernels,
//   decode_split_kernel  split-KV: one wave per (sequence, partition, kv
//                        head), streaming the partition's pages and writing
//                        its partial straight from registers;
//   decode_whole_kernel  four waves per (sequence, kv head), each taking
//                        every fourth page, merged through LDS (single pass,
//                        or four-wave split-KV units).
#include "split_plan.hpp"
#include "wave_attn.hpp"

namespace pa {
namespace {

// ---------------------------------------------------------------- split-KV
// Unit = one wave.  Block b runs on XCD b % 8 and the kv head is the fastest
// index, so with 8 kv heads each XCD owns one kv head and sequences sharing
// prefix pages read them through one L2.
template <int D, int NC>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeParams p) {
  const int u = blockIdx.x;
  if (u >= p.num_units) return;
  // The prologue (the unit plan and the first loads) runs at raised priority:
  // a wave's SIMD otherwise issues for its older, streaming waves first, and a
  // younger wave's page ids then arrive only when those have finished.
  __builtin_amdgcn_s_setprio(3);
  const int kvh = u % p.num_kv_heads;
  const int useq = u / p.num_kv_heads;
  const int lane = threadIdx.x;
  const int r = lane & 15, j = lane >> 4;
  const int G = p.group;

  // The sharing test's loads (column 0 of every block-table row) depend on
  // nothing: they go out with the plan's length loads.
  SharingTest<NC> sharing;
  sharing.request(p, lane);
  int seq, part, seq_pages = 0;
  if constexpr (NC > 0) {
    if (!split_unit<NC>(p, useq, lane, seq, part, seq_pages)) return;
  } else {
    seq = useq % p.num_seqs;  // plain grid: partitions past a context exit below
    part = useq / p.num_seqs;
    if (p.first_partition && part < p.first_partition[seq]) return;  // computed elsewhere
  }
  seq = __builtin_amdgcn_readfirstlane(seq);
  part = __builtin_amdgcn_readfirstlane(part);

  // Issued together before any of them returns: the new token (when this
  // partition holds the sequence's last page and the launch appends), length,
  // page ids, query.
  const bool appends = p.new_key != nullptr;
  bool writes = false;
  NewToken<D> nt;
  if constexpr (NC > 0) {
    writes = appends && (part + 1) * p.pages_per_partition >= seq_pages;
    if (writes) nt.request(p, seq, kvh, lane);
  }
  const int lo = part * p.pages_per_partition;
  const int row_end = min(lo + p.pages_per_partition, p.max_pages_per_seq);
  PageStream<D> ps = make_stream<D>(p, seq, kvh, lo, 1, row_end, lane);
  const int L = p.context_lens[seq];
  WaveAttn<D> wa;
  wa.init(static_cast<const uint16_t*>(p.query) + (size_t(seq) * p.num_q_heads + kvh * G + r) * D,
          r < G, r, j, p.scale_log2);

  int n = (L + kPage - 1) / kPage;
  if (n > p.max_pages_per_seq) n = p.max_pages_per_seq;
  const int hi = min(lo + p.pages_per_partition, n);
  if (lo >= hi) {
    // A partition past the context writes nothing, except one that the merge
    // counts (past a length clamped to the table's width): an empty partial.
    if constexpr (NC == 0)
      if (part < merged_partitions(p, L)) empty_partials<D>(p, seq, kvh, part, part + 1, lane, 64);
    return;
  }
  if constexpr (NC == 0) {  // the plain grid learns the length only now
    writes = appends && hi == n;
    if (writes) nt.request(p, seq, kvh, lane);
  }
  writes = writes && nt.valid(p);
  ps.count = hi - lo;
  __builtin_amdgcn_s_setprio(0);
  wa.run(ps, lo, L, lane, sharing.shared(p, seq, lane), writes, nt);
  if (writes) nt.store(p, kvh, lane);

  // Partial of this partition: o = acc / l, m in natural-log units, l.
  const float l = __shfl(wa.acc[D / 16][0], r);  // row 0 of the denominator block
  if (r < G) {
    const size_t row = (size_t(seq) * p.num_q_heads + kvh * G + r) * p.num_partitions + part;
    float* dst = p.partial_out + row * D;
    const float inv = 1.0f / l;
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
      *reinterpret_cast<f32x4*>(dst + 16 * db + 4 * j) = wa.acc[db] * inv;
    if (j == 0) {
      p.partial_max[row] = wa.m_run * kLn2;
      p.partial_sum[row] = l;
    }
  }
  // The plan has no units past a length clamped to the block table's width;
  // the unit of the last partition with tokens gives the partitions after it
  // that the merge counts empty partials.
  if constexpr (NC > 0)
    if (hi == n) empty_partials<D>(p, seq, kvh, part + 1, merged_partitions(p, L), lane, 64);
}

// ---------------------------------------------------------------- single pass
// Unit = (sequence, kv head), four waves; wave w takes pages w, w+4, ...
// In batches of up to 1024 sequences, unit slot i (kv head fastest) takes the
// sequence of rank snake_rank(i) by length, longest first, so each compute
// unit's units add up to about the same number of pages, and a sequence that
// shares no first page with another streams with the nontemporal hint
// (larger batches: batch order, cached loads).  A batch in which neighbours
// share their first page keeps batch order: a prefix group's units then run
// together and read the shared pages through one L2 while they stay there.
// With partitions (the four-wave split-KV units, chosen when the batch has
// few units for the machine, as a shared-prefix step's suffixes do), unit =
// (sequence, partition, kv head) over the partition's pages, and the merged
// state is written as that partition's partial.
template <int D, int NC>
__global__ __launch_bounds__(kBlock) void decode_whole_kernel(DecodeParams p) {
  extern __shared__ float smem[];
  int seq, kvh, part;
  if (!unit_of(p, blockIdx.x, seq, kvh, part)) return;
  __builtin_amdgcn_s_setprio(3);  // lowered before the page stream starts
  bool shared = true;
  if constexpr (NC > 0)
    if (p.pages_per_partition == 0) seq = snake_unit_seq<NC>(p, seq, threadIdx.x & 63, shared);
  whole_unit<D>(p, seq, kvh, part, smem, shared);
}

template <int D>
hipError_t launch_d(const DecodeParams& p, hipStream_t stream) {
  if (p.pages_per_partition > 0 && !p.four_wave_units) {
    switch (plan_chunks_for(p.num_seqs)) {
      case 1: decode_split_kernel<D, 1><<<dim3(p.num_units), 64, 0, stream>>>(p); break;
      case 4: decode_split_kernel<D, 4><<<dim3(p.num_units), 64, 0, stream>>>(p); break;
      case kPlanChunks:
        decode_split_kernel<D, kPlanChunks><<<dim3(p.num_units), 64, 0, stream>>>(p);
        break;
      default: decode_split_kernel<D, 0><<<dim3(p.num_units), 64, 0, stream>>>(p); break;
    }
  } else {
    const size_t lds = merge_lds_bytes(p.group, D);
    const dim3 grid(decode_grid(p.num_units));
    switch (p.pages_per_partition == 0 ? plan_chunks_for(p.num_seqs) : 0) {
      case 1: decode_whole_kernel<D, 1><<<grid, kBlock, lds, stream>>>(p); break;
      case 4: decode_whole_kernel<D, 4><<<grid, kBlock, lds, stream>>>(p); break;
      case kPlanChunks: decode_whole_kernel<D, kPlanChunks><<<grid, kBlock, lds, stream>>>(p); break;
      default: decode_whole_kernel<D, 0><<<grid, kBlock, lds, stream>>>(p); break;
    }
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeParams& p, int head_dim, hipStream_t stream) {
  return head_dim == 128 ? launch_d<128>(p, stream) : launch_d<64>(p, stream);
}

}  // namespace pa
