// bf16 paged decode on the matrix cores (gfx950): the per-page step
// (wave_attn.hpp) in two kernels,
//   decode_split_kernel  split-KV: one wave per (sequence, partition, kv
//                        head), streaming the partition's pages and writing
//                        its partial straight from registers;
//   decode_whole_kernel  four waves per (sequence, kv head), each taking
//                        every fourth page, merged through LDS (single pass,
//                        or four-wave split-KV units).
#include "wave_attn.hpp"

namespace pa {
namespace {

// ---------------------------------------------------------------- split-KV
constexpr int kPlanChunks = 16;  // batches up to 1024 sequences use the unit plan

__device__ inline int wave_sum(int v) {
#pragma unroll
  for (int x = 1; x < 64; x <<= 1) v += __shfl_xor(v, x);
  return v;
}

// Index (within its 64-lane chunk) of the k-th set bit of a wave ballot.
__device__ inline int kth_set_lane(uint64_t mask, int k, int lane) {
  const bool set = (mask >> lane) & 1;
  const int rank = __builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32),
                                             __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0));
  const uint64_t hit = __ballot(set && rank == k);
  return hit ? __builtin_ctzll(hit) : -1;
}

// True when sequence `seq` (its first page id is lane seq % 64 of
// first[seq / 64]; -1 for a sequence with no pages) starts with the same
// physical page as another sequence of the batch.  Prefix reuse always shares
// a sequence's first page, so a sequence that passes this test reads no page
// that another sequence reads.
template <int NC>
__device__ inline bool first_page_shared(const int (&first)[NC], int seq) {
  int f = -1;
#pragma unroll
  for (int c = 0; c < NC; ++c)
    if (c == (seq >> 6)) f = __builtin_amdgcn_readlane(first[c], seq & 63);
  if (f < 0) return false;
  int count = 0;
#pragma unroll
  for (int c = 0; c < NC; ++c) count += __popcll(__ballot(first[c] == f));
  return count > 1;
}

// Context length in pages of sequence 64c + lane for c < NC, where NC * 64
// >= the batch (0 past the batch).  The loads are unconditional (a lane past
// the batch re-reads the last sequence), so they are all in flight together
// and the batch costs one memory round trip.
template <int NC>
__device__ inline void load_pages(const DecodeParams& p, int lane, int (&pages)[NC]) {
  int len[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) len[c] = p.context_lens[min(64 * c + lane, p.num_seqs - 1)];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const bool in = 64 * c + lane < p.num_seqs;
    pages[c] = in ? min((max(len[c], 0) + kPage - 1) / kPage, p.max_pages_per_seq) : 0;
  }
}

// First page id of sequence 64c + lane (-1 past the batch or for an empty
// context), requested for every chunk at once.
template <int NC>
struct FirstPages {
  int len[NC], fid[NC];
  __device__ void request(const DecodeParams& p, int lane) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int b = min(64 * c + lane, p.num_seqs - 1);
      len[c] = p.context_lens[b];
      fid[c] = p.block_tables[size_t(b) * p.max_pages_per_seq];  // column 0 always exists
    }
  }
  __device__ bool shared(const DecodeParams& p, int seq, int lane) const {
    int first[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c)
      first[c] = (64 * c + lane < p.num_seqs && len[c] > 0) ? fid[c] : -1;
    return first_page_shared<NC>(first, seq);
  }
};

// The split-KV units that hold tokens, enumerated without scratch memory:
// every wave reads all context lengths and derives the same list.  Per kv
// head, the full partitions come first in partition-major order (partition 0
// of every sequence, then partition 1, ...) and each sequence's partly filled
// last partition comes after all of them, so the longest units are dispatched
// first and no wave is spent on a partition past a context's end.  Returns
// false for an index past the last unit.  NC * 64 >= batch.
template <int NC>
__device__ bool split_unit(const DecodeParams& p, int useq, int lane, int& seq, int& part,
                           int& seq_pages) {
  const int PP = p.pages_per_partition;
  int pages[NC], nfull[NC], hasp[NC], first[NC];
  load_pages<NC>(p, lane, pages);
#pragma unroll
  for (int c = 0; c < NC; ++c)  // partitions computed elsewhere (a shared prefix)
    first[c] = p.first_partition ? max(p.first_partition[min(64 * c + lane, p.num_seqs - 1)], 0)
                                 : 0;
  int full_total = 0, part_total = 0;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int nparts = min((pages[c] + PP - 1) / PP, p.num_partitions);
    const int full = min(pages[c] / PP, p.num_partitions);
    first[c] = min(first[c], full);  // only whole partitions are skipped
    nfull[c] = full - first[c];      // counted from the first partition computed here
    hasp[c] = nparts > full ? 1 : 0;
    full_total += nfull[c];
    part_total += hasp[c];
  }
  full_total = wave_sum(full_total);
  part_total = wave_sum(part_total);
  seq = -1;
  part = 0;
  if (useq < full_total) {
    // Smallest p with sum_b min(nfull_b, p + 1) > useq.
    int lo = 0, hi = p.num_partitions;  // O(lo) <= useq < O(hi)
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      int o = 0;
#pragma unroll
      for (int c = 0; c < NC; ++c) o += min(nfull[c], mid);
      if (wave_sum(o) <= useq) lo = mid; else hi = mid;
    }
    int o = 0;
#pragma unroll
    for (int c = 0; c < NC; ++c) o += min(nfull[c], lo);
    int k = useq - wave_sum(o);  // rank among the sequences with a full partition lo
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint64_t m = __ballot(nfull[c] > lo);
      const int n = __popcll(m);
      if (seq < 0 && k < n && k >= 0) {
        seq = 64 * c + kth_set_lane(m, k, lane);
        part = lo + __builtin_amdgcn_readlane(first[c], seq - 64 * c);
      }
      k -= n;
    }
  } else {
    int k = useq - full_total;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint64_t m = __ballot(hasp[c] != 0);
      const int n = __popcll(m);
      if (seq < 0 && k < n && k >= 0) {
        seq = 64 * c + kth_set_lane(m, k, lane);
        part = __builtin_amdgcn_readlane(nfull[c] + first[c], seq - 64 * c);
      }
      k -= n;
    }
  }
  seq = __builtin_amdgcn_readfirstlane(seq);
  seq_pages = 0;
#pragma unroll
  for (int c = 0; c < NC; ++c)
    if (c == (seq >> 6)) seq_pages = __builtin_amdgcn_readlane(pages[c], seq & 63);
  return seq >= 0;
}

// Batch-size buckets of the device-side plan and the sharing test: their
// arrays are sized for NC * 64 sequences, NC in {1, 4, 16}, picked by the
// host.  NC = 0 (batches above 1024 sequences) does without both: a plain
// unit grid, and cached loads throughout.
constexpr int kPlanMaxSeqs = 64 * kPlanChunks;

__host__ __device__ constexpr int plan_chunks_for(int num_seqs) {
  return num_seqs <= 64 ? 1 : num_seqs <= 256 ? 4 : num_seqs <= kPlanMaxSeqs ? kPlanChunks : 0;
}

// The sharing test of sequence `seq`: its loads are issued by request(), the
// answer is read by shared() after other loads have been issued.
template <int NC>
struct SharingTest {
  FirstPages<NC> fp;
  __device__ void request(const DecodeParams& p, int lane) { fp.request(p, lane); }
  __device__ bool shared(const DecodeParams& p, int seq, int lane) const {
    return fp.shared(p, seq, lane);
  }
};
template <>
struct SharingTest<0> {
  __device__ void request(const DecodeParams&, int) {}
  __device__ bool shared(const DecodeParams&, int, int) const { return true; }
};

// Unit = one wave.  Block b runs on XCD b % 8 and the kv head is the fastest
// index, so with 8 kv heads each XCD owns one kv head and sequences sharing
// prefix pages read them through one L2.
template <int D, int NC>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeParams p) {
  const int u = blockIdx.x;
  if (u >= p.num_units) return;
  const int kvh = u % p.num_kv_heads;
  const int useq = u / p.num_kv_heads;
  const int lane = threadIdx.x;
  const int r = lane & 15, j = lane >> 4;
  const int G = p.group;

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
  // partition holds the sequence's last page and the launch appends), the
  // sharing test, length, page ids, query.
  const bool appends = p.new_key != nullptr;
  bool writes = false;
  NewToken<D> nt;
  if constexpr (NC > 0) {
    writes = appends && (part + 1) * p.pages_per_partition >= seq_pages;
    if (writes) nt.request(p, seq, kvh, lane);
  }
  SharingTest<NC> sharing;
  sharing.request(p, lane);
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
  if (lo >= hi) return;  // partition past the context: nothing to write
  if constexpr (NC == 0) {  // the plain grid learns the length only now
    writes = appends && hi == n;
    if (writes) nt.request(p, seq, kvh, lane);
  }
  writes = writes && nt.valid(p);
  ps.count = hi - lo;
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
}

// ---------------------------------------------------------------- single pass
// Unit = (sequence, kv head), four waves; wave w takes pages w, w+4, ...
// With partitions (the four-wave split-KV units, chosen when the batch has
// few units for the machine, as a shared-prefix step's suffixes do), unit =
// (sequence, partition, kv head) over the partition's pages, and the merged
// state is written as that partition's partial.
template <int D>
__global__ __launch_bounds__(kBlock) void decode_whole_kernel(DecodeParams p) {
  extern __shared__ float smem[];
  int seq, kvh, part;
  if (!unit_of(p, blockIdx.x, seq, kvh, part)) return;
  whole_unit<D>(p, seq, kvh, part, smem);
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
    decode_whole_kernel<D><<<dim3(decode_grid(p.num_units)), kBlock, lds, stream>>>(p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeParams& p, int head_dim, hipStream_t stream) {
  return head_dim == 128 ? launch_d<128>(p, stream) : launch_d<64>(p, stream);
}

}  // namespace pa
