// The device-side plan of split-KV work units and the page-sharing test,
// shared by the split decode and the split multi-token kernels (any params
// struct with context_lens, block_tables, num_seqs, max_pages_per_seq,
// pages_per_partition, num_partitions and first_partition).
#pragma once

#include "pa_device.hpp"

namespace pa {

constexpr int kPlanChunks = 16;  // batches up to 1024 sequences use the unit plan

// Whole-wave sums and maxima through the device library's wavefront
// reductions (cross-lane moves within the vector unit), not six LDS-routed
// shuffles: the unit plan chains several of them before a wave's first load.
extern "C" __device__ __attribute__((const)) int __ockl_wfred_add_i32(int);
extern "C" __device__ __attribute__((const)) int __ockl_wfred_max_i32(int);

__device__ inline int wave_sum(int v) { return __ockl_wfred_add_i32(v); }
__device__ inline int wave_max_i32(int v) { return __ockl_wfred_max_i32(v); }

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
template <int NC, class Params>
__device__ inline void load_pages(const Params& p, int lane, int (&pages)[NC]) {
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
  template <class Params>
  __device__ void request(const Params& p, int lane) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int b = min(64 * c + lane, p.num_seqs - 1);
      len[c] = p.context_lens[b];
      fid[c] = p.block_tables[size_t(b) * p.max_pages_per_seq];  // column 0 always exists
    }
  }
  template <class Params>
  __device__ bool shared(const Params& p, int seq, int lane) const {
    int first[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c)
      first[c] = (64 * c + lane < p.num_seqs && len[c] > 0) ? fid[c] : -1;
    return first_page_shared<NC>(first, seq);
  }
  // Whether two sequences next to each other in the batch share their first
  // page (a prefix group laid out contiguously, as a scheduler batches the
  // requests of one prompt): then batch order keeps a group's units together
  // in time, and the second reader of a page finds it in L2.
  template <class Params>
  __device__ bool adjacent_shared(const Params& p, int lane) const {
    uint64_t hits = 0;
    int last = -1;  // first page of sequence 64c - 1
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int f = (64 * c + lane < p.num_seqs && len[c] > 0) ? fid[c] : -1;
      int prev = __shfl_up(f, 1);
      if (lane == 0) prev = last;
      hits |= __ballot(f >= 0 && f == prev);
      last = __builtin_amdgcn_readlane(f, 63);
    }
    return hits != 0;
  }
};

// The split-KV units that hold tokens, enumerated without scratch memory:
// every wave reads all context lengths and derives the same list.  Per kv
// head, the full partitions come first in partition-major order (partition 0
// of every sequence, then partition 1, ...) and each sequence's partly filled
// last partition comes after all of them, largest first, so the longest
// units are dispatched first and no wave is spent on a partition past a
// context's end.  Returns
// false for an index past the last unit.  NC * 64 >= batch.
template <int NC, class Params>
__device__ bool split_unit(const Params& p, int useq, int lane, int& seq, int& part,
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
    // Partly filled partitions, largest first (ties in batch order).  Blocks
    // are placed on CUs by index (block b on XCD b % 8, then the XCD's CUs
    // in turn), so after the full partitions the first of these land on the
    // CUs that got one full partition fewer: the largest go there.
    int k = useq - full_total;
    int psize[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) psize[c] = hasp[c] ? pages[c] - (pages[c] / PP) * PP : 0;
    auto count_ge = [&](int t) {  // partly filled partitions of at least t pages
      int n = 0;
#pragma unroll
      for (int c = 0; c < NC; ++c) n += __popcll(__ballot(psize[c] >= t));
      return n;
    };
    if (k < part_total) {
      // Unit k's size: the sz in [1, PP) with count_ge(sz + 1) <= k < count_ge(sz),
      // by bisection (a scan over the sizes costs PP rounds of ballots).
      int lo = 1, hi = PP;  // count_ge(lo) = part_total > k >= 0 = count_ge(hi)
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (count_ge(mid) > k) lo = mid; else hi = mid;
      }
      k -= count_ge(lo + 1);  // rank among the partitions of lo pages, in batch order
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const uint64_t m = __ballot(psize[c] == lo);
        const int n = __popcll(m);
        if (seq < 0 && k < n && k >= 0) {
          seq = 64 * c + kth_set_lane(m, k, lane);
          part = __builtin_amdgcn_readlane(nfull[c] + first[c], seq - 64 * c);
        }
        k -= n;
      }
    }
  }
  seq = __builtin_amdgcn_readfirstlane(seq);
  seq_pages = 0;
#pragma unroll
  for (int c = 0; c < NC; ++c)
    if (c == (seq >> 6)) seq_pages = __builtin_amdgcn_readlane(pages[c], seq & 63);
  return seq >= 0;
}

// The sequence of rank `rank` when the batch is ordered by context length,
// longest first, ties in batch order.  len[c] is the length of sequence
// 64c + lane (-1 past the batch) for the first nc chunks.  The rank's length
// comes from a binary search on the count of lengths at or above a threshold
// (wave ballots), then the tie by its batch order.  -1 for a rank past the
// batch.
template <int NC>
__device__ inline int seq_of_rank(const int (&len)[NC], int nc, int rank, int lane) {
  int top = 0;
#pragma unroll
  for (int c = 0; c < NC; ++c) top = max(top, len[c]);
  top = wave_max_i32(top);
  auto count_ge = [&](int t) {
    int n = 0;
#pragma unroll
    for (int c = 0; c < NC; ++c)
      if (c < nc) n += __popcll(__ballot(len[c] >= t));
    return n;
  };
  int lo = 0, hi = top + 1;  // count_ge(lo) > rank >= count_ge(hi)
  while (hi - lo > 1) {
    const int mid = lo + ((hi - lo) >> 1);
    if (count_ge(mid) > rank) lo = mid; else hi = mid;
  }
  int k = rank - count_ge(lo + 1);  // rank among the sequences of length lo
  int seq = -1;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (c < nc) {
      const uint64_t m = __ballot(len[c] == lo);
      const int n = __popcll(m);
      if (seq < 0 && k >= 0 && k < n) seq = 64 * c + kth_set_lane(m, k, lane);
      k -= n;
    }
  }
  return __builtin_amdgcn_readfirstlane(seq);
}

// Single-pass units go to the compute units in grid order, one each per
// round of `period` sequences (the machine's compute units divided by the kv
// heads, which vary fastest), and a unit shares its compute unit with the
// units one, two, ... rounds later.  Ranks run forward in even rounds and
// backward in odd ones, so a compute unit that takes a long sequence in one
// round takes a short one in the next and the totals even out.  period 0:
// rank = slot.
__host__ __device__ inline int snake_rank(int slot, int period, int num_seqs) {
  if (period <= 0) return slot;
  const int k = slot / period, j = slot % period;
  const int m = min(period, num_seqs - k * period);  // sequences in this round
  return k * period + ((k & 1) ? m - 1 - j : j);
}

// Batch-size buckets of the device-side plan and the sharing test: their
// arrays are sized for NC * 64 sequences, NC in {1, 4, 16}, picked by the
// host.  NC = 0 (batches above 1024 sequences) does without both: a plain
// unit grid, and cached loads throughout.
constexpr int kPlanMaxSeqs = 64 * kPlanChunks;

__host__ __device__ constexpr int plan_chunks_for(int num_seqs) {
  return num_seqs <= 64 ? 1 : num_seqs <= 256 ? 4 : num_seqs <= kPlanMaxSeqs ? kPlanChunks : 0;
}

// The sequence of rank `rank` when the batch is ordered by context length
// (clamped to the table), longest first, ties in batch order; a batch above
// kPlanMaxSeqs keeps its order.  Units are dispatched in grid order, so the
// long sequences' units start first and the short ones fill in behind them,
// instead of a long sequence's units starting late and setting the end.
// The rank's length is found by a binary search on the count of lengths at
// or above a threshold (wave ballots), then the tie by its batch order.
// NC: chunks of 64 sequences loaded (NC * 64 >= the batch; the default
// covers any batch the order applies to).
template <int NC = kPlanChunks, class Params>
__device__ inline int longest_first(const Params& p, int rank, int lane) {
  if (p.num_seqs > 64 * NC) return rank;
  const int nc = (p.num_seqs + 63) >> 6;
  const int cap = min(p.max_pages_per_seq, (1 << 30) / kPage - 1) * kPage;
  // The loads go out together, unconditionally (a lane past the batch
  // re-reads the last sequence): under a branch, the compiler waits for each
  // load before the next.
  int len[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c)
    len[c] = p.context_lens[min(64 * c + lane, p.num_seqs - 1)];
#pragma unroll
  for (int c = 0; c < NC; ++c)
    len[c] = 64 * c + lane < p.num_seqs ? min(max(len[c], 0), cap) : -1;  // -1: past the batch
  const int seq = seq_of_rank<NC>(len, nc, rank, lane);
  return seq >= 0 ? seq : rank;
}

// longest_first with as many chunks as the batch needs: every wave of a
// launch runs it, and the chunks past the batch would each re-read one
// length, the same address from every wave.
template <class Params>
__device__ inline int longest_first_of_batch(const Params& p, int rank, int lane) {
  const int nc = plan_chunks_for(p.num_seqs);
  if (nc == 1) return longest_first<1>(p, rank, lane);
  if (nc == 4) return longest_first<4>(p, rank, lane);
  return longest_first<kPlanChunks>(p, rank, lane);  // batch order past kPlanMaxSeqs
}

// The sequence of a single-pass unit in slot `slot` when all the launch's
// units are resident at once, as the single-pass decode picks it: the
// sequence of rank snake_rank(slot) by length, longest first (batch order
// when neighbours share their first page), so that each compute unit's
// units add up to about the same work.  `shared` says whether its first page
// is another sequence's too (else it may stream with the nontemporal hint).
// Past the batch sizes the plan covers: batch order, shared.
template <int NC, class Params>
__device__ inline int snake_unit_seq(const Params& p, int slot, int lane, bool& shared) {
  FirstPages<NC> fp;
  fp.request(p, lane);
  const int cap = min(p.max_pages_per_seq, (1 << 30) / kPage - 1) * kPage;
  int len[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c)
    len[c] = 64 * c + lane < p.num_seqs ? min(max(fp.len[c], 0), cap) : -1;
  int seq = slot;
  if (!fp.adjacent_shared(p, lane)) {
    const int s = seq_of_rank<NC>(len, NC, snake_rank(slot, p.snake_period, p.num_seqs), lane);
    seq = s >= 0 ? s : slot;
  }
  shared = fp.shared(p, seq, lane);
  return seq;
}

template <class Params>
__device__ inline int snake_unit_seq_of_batch(const Params& p, int slot, int lane, bool& shared) {
  int seq = slot;
  shared = true;
  switch (plan_chunks_for(p.num_seqs)) {
    case 1: seq = snake_unit_seq<1>(p, slot, lane, shared); break;
    case 4: seq = snake_unit_seq<4>(p, slot, lane, shared); break;
    case kPlanChunks: seq = snake_unit_seq<kPlanChunks>(p, slot, lane, shared); break;
    default: break;
  }
  shared = __builtin_amdgcn_readfirstlane(int(shared)) != 0;
  return __builtin_amdgcn_readfirstlane(seq);
}

// The sharing test of sequence `seq`: its loads are issued by request(), the
// answer is read by shared() after other loads have been issued.
template <int NC>
struct SharingTest {
  FirstPages<NC> fp;
  template <class Params>
  __device__ void request(const Params& p, int lane) { fp.request(p, lane); }
  template <class Params>
  __device__ bool shared(const Params& p, int seq, int lane) const {
    return fp.shared(p, seq, lane);
  }
};
template <>
struct SharingTest<0> {
  template <class Params>
  __device__ void request(const Params&, int) {}
  template <class Params>
  __device__ bool shared(const Params&, int, int) const { return true; }
};

}  // namespace pa
