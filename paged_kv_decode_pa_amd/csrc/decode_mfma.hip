// bf16 paged decode on the matrix cores (gfx950).
//
// Per 16-token page and kv head, with the grouped query heads as the 16
// columns of a matrix tile (groups below 16 are zero-padded):
//   S^T[16 tok][16 heads]  = K[16 tok][D] . Q^T[D][16 heads]
//                            D/32 x v_mfma_f32_16x16x32_bf16; A = the K page
//                            tile straight from HBM (each lane a 16-byte row
//                            chunk), B = the query group, loaded once.
//   online softmax on the S^T accumulator (lane = head r, tokens 4j..4j+3)
//   O^T[D][16 heads]      += V^T[D][16 tok] . P^T[16 tok][16 heads]
//                            D/16 x v_mfma_f32_16x16x16_bf16; A = the V page
//                            tile (stored dim-major, each lane an 8-byte
//                            chunk of 4 tokens), B = P^T, which is exactly
//                            the S^T accumulator's lane layout in bf16.
//   plus one 16x16x16 product of a row of ones with P^T: the softmax
//   denominator, summed from the same rounded P as the numerator.
// A page thus costs 3*D/32 + 1 matrix instructions and ~25 vector ones;
// the loads dominate.
//
// Two kernels share that per-page step:
//   decode_split_kernel  split-KV: one wave per (sequence, partition, kv
//                        head), streaming the partition's pages and writing
//                        its partial straight from registers;
//   decode_whole_kernel  single pass: four waves per (sequence, kv head),
//                        each taking every fourth page, merged through LDS.
#include "page_stream.hpp"

namespace pa {
namespace {

constexpr float kRescaleSlack = 8.0f;   // base 2: P may reach 2^8 before a rescale

// The step's new token of sequence `seq` (bf16): its K row and V column for
// kv head `kvh`, requested with the unit's first loads.  The wave that reads
// the sequence's last page puts the token into that page's tile registers
// (patch), so the tile need not wait for the pool, and stores it into the pool
// slot after its stream (store).  Lane l < D/8 holds the K row's 16-byte chunk
// l; every lane holds V dims l and l + 64.
template <int D>
struct NewToken {
  u32x4 k;
  uint16_t v[D / 64];
  int64_t slot;
  __device__ void request(const DecodeParams& p, int seq, int kvh, int lane) {
    slot = p.new_slots[seq];
    const size_t row = (size_t(seq) * p.num_kv_heads + kvh) * D;
    const uint16_t* kr = static_cast<const uint16_t*>(p.new_key) + row;
    const uint16_t* vr = static_cast<const uint16_t*>(p.new_value) + row;
    k = u32x4{0u, 0u, 0u, 0u};
    if (lane < D / 8) k = *reinterpret_cast<const u32x4*>(kr + 8 * lane);
#pragma unroll
    for (int i = 0; i < D / 64; ++i) v[i] = vr[lane + 64 * i];
  }
  __device__ bool valid(const DecodeParams& p) const {
    return slot >= 0 && slot < p.num_pages * kPage;
  }
  // Overwrite in-page slot s of a page tile with this token (tile layouts as
  // in PageTile: lane (r, j) holds K row r's chunks 4kb + j and V^T rows
  // 16db + r at tokens 4j .. 4j + 3).
  __device__ void patch(PageTile<D>& t, int s, int lane) const {
    const int r = lane & 15, j = lane >> 4;
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb) {
      u32x4 x;
#pragma unroll
      for (int c = 0; c < 4; ++c) x[c] = __shfl(k[c], 4 * kb + j);
      if (r == s) t.k[kb] = __builtin_bit_cast(bf16x8, x);
    }
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const int x = __shfl(int(v[db / 4]), 16 * (db % 4) + r);
      if (j == s / 4) t.v[db][s % 4] = short(x);
    }
  }
  __device__ void store(const DecodeParams& p, int kvh, int lane) const {
    const int64_t page = slot / kPage;
    const int off = int(slot % kPage);
    const size_t tile = (size_t(page) * p.num_kv_heads + kvh) * kPage * D;
    uint16_t* kt = static_cast<uint16_t*>(const_cast<void*>(p.k_cache)) + tile + size_t(off) * D;
    uint16_t* vt = static_cast<uint16_t*>(const_cast<void*>(p.v_cache)) + tile;
    if (lane < D / 8) *reinterpret_cast<u32x4*>(kt + 8 * lane) = k;
#pragma unroll
    for (int i = 0; i < D / 64; ++i) vt[(lane + 64 * i) * kPage + off] = v[i];
  }
};

// One wave's online-softmax attention state for one kv head's query group.
template <int D>
struct WaveAttn {
  bf16x8 qop[D / 32];    // B operand: column r = query head r of the group
  s16x4 ones;            // A operand of the denominator block
  f32x4 acc[D / 16 + 1]; // O^T blocks (lane: dims 16db+4j.., head r), then the denominator
  float m_run;           // base-2 reference score of head r, equal in all 4 lane groups
  float scale_log2;
  int j;

  __device__ void init(const uint16_t* qrow, bool real_head, int r, int j_, float sl2) {
    j = j_;
    scale_log2 = sl2;
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (real_head) v = *reinterpret_cast<const u32x4*>(qrow + 32 * kb + 8 * j);
      qop[kb] = __builtin_bit_cast(bf16x8, v);
    }
    ones = s16x4{0, 0, 0, 0};
    if (r == 0) ones = s16x4{0x3F80, 0x3F80, 0x3F80, 0x3F80};
    m_run = -INFINITY;
#pragma unroll
    for (int db = 0; db <= D / 16; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // One page with `valid` tokens of the context (< 16 only on the last page).
  // m_run is raised only when a score exceeds it by more than kRescaleSlack,
  // so P stays <= 2^kRescaleSlack and the accumulator rescale (with its
  // cross-lane max) runs on few pages.
  __device__ void page(PageTile<D>& t, int valid) {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(t.k[kb], qop[kb], s, 0, 0, 0);
    float s2[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) s2[e] = s[e] * scale_log2;
    if (valid < kPage) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * j + e >= valid) s2[e] = -INFINITY;
#pragma unroll
      for (int db = 0; db < D / 16; ++db)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * j + e >= valid) t.v[db][e] = 0;  // unwritten slots may hold NaN
    }
    const float lm = fmaxf(fmaxf(s2[0], s2[1]), fmaxf(s2[2], s2[3]));
    if (__ballot(lm > m_run + kRescaleSlack) != 0) {
      float pm = fmaxf(lm, __shfl_xor(lm, 16));
      pm = fmaxf(pm, __shfl_xor(pm, 32));
      const float m_new = fmaxf(m_run, pm);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
#pragma unroll
      for (int db = 0; db <= D / 16; ++db) acc[db] *= alpha;
    }
    s16x4 pb;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      pb[e] = static_cast<short>(f32_to_bf16(__builtin_amdgcn_exp2f(s2[e] - m_run)));
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(t.v[db], pb, acc[db], 0, 0, 0);
    acc[D / 16] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ones, pb, acc[D / 16], 0, 0, 0);
  }

  // Walk the stream with two tiles in ping-pong: the next page's loads are in
  // flight while the current page is computed, and no register copy forces
  // an early wait.  `page0` is the logical index of ordinal 0, `L` the length.
  // The steady-state loop runs only while all four tiles it touches exist,
  // so its loads are unconditional and no tile is requested twice (a repeat
  // would go back to HBM under the nontemporal hint); the last one to three
  // pages are finished after it.  Only a one-page stream requests a tile
  // twice (its clamped second request).
  // With `append`, the stream's last page is the sequence's last page and
  // the step's new token `nt` goes into its tile (in-page slot (L-1) % 16)
  // before it is computed.
  template <bool Stream>
  __device__ void walk(PageStream<D>& ps, int page0, int L, int lane, bool append,
                       const NewToken<D>& nt) {
    const int n = ps.count;
    auto valid = [&](int k) { return L - (page0 + ps.step * k) * kPage; };
    const int s = (L - 1) % kPage;
    PageTile<D> ta, tb;
    bool ok_a = ps.template issue<Stream>(ta, 0, lane);
    bool ok_b = ps.template issue<Stream>(tb, 1, lane);  // a one-page stream repeats tile 0
    int k = 0;
    for (; k + 3 < n; k += 2) {
      if (ok_a) page(ta, valid(k));
      ok_a = ps.template issue<Stream>(ta, k + 2, lane);
      if (ok_b) page(tb, valid(k + 1));
      ok_b = ps.template issue<Stream>(tb, k + 3, lane);
    }
    const int rem = n - k;  // 1 (only when n == 1), 2 or 3 pages left
    if (append && rem == 1) nt.patch(ta, s, lane);
    if (ok_a) page(ta, valid(k));
    if (rem >= 2) {
      const bool ok_c = rem == 3 && ps.template issue<Stream>(ta, k + 2, lane);
      if (append && rem == 2) nt.patch(tb, s, lane);
      if (ok_b) page(tb, valid(k + 1));
      if (append && rem == 3) nt.patch(ta, s, lane);
      if (ok_c) page(ta, valid(k + 2));
    }
  }
  // `shared`: some page of this sequence may also be read by another
  // sequence (cached loads); otherwise the pages stream with the nontemporal
  // hint.  Its loads were issued with the page ids, which the first tile
  // needs anyway, so deciding first costs no extra round trip.
  __device__ void run(PageStream<D>& ps, int page0, int L, int lane, bool shared,
                      bool append, const NewToken<D>& nt) {
    if (ps.count <= 0) return;
    if (shared)
      walk<false>(ps, page0, L, lane, append, nt);
    else
      walk<true>(ps, page0, L, lane, append, nt);
  }
};

template <int D>
__device__ inline PageStream<D> make_stream(const DecodeParams& p, int seq, int kvh, int first,
                                            int step, int row_end, int lane) {
  PageStream<D> ps;
  ps.table = p.block_tables + size_t(seq) * p.max_pages_per_seq;
  ps.first = first;
  ps.step = step;
  ps.row_end = row_end;
  ps.count = 0;
  ps.kpool = static_cast<const char*>(p.k_cache);
  ps.vpool = static_cast<const char*>(p.v_cache);
  ps.num_pages = p.num_pages;
  ps.num_kv_heads = p.num_kv_heads;
  ps.kvh = kvh;
  const int r = lane & 15, j = lane >> 4;
  ps.koff = uint32_t(r * D + 8 * j) * 2u;        // K row r, dims 8j .. (+32kb per load)
  ps.voff = uint32_t(r * kPage + 4 * j) * 2u;    // V^T row r, tokens 4j .. (+16 rows per load)
  ps.start(lane);
  return ps;
}

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
  if (!unit_of_block(p, seq, kvh, part)) return;
  if (p.first_partition)  // partitions below it are computed elsewhere
    part += min(max(p.first_partition[seq], 0), p.num_partitions);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, j = lane >> 4;
  const int G = p.group;
  const int PP = p.pages_per_partition;
  const int lo0 = part * PP;  // 0 for the single pass

  // Every wave requests the new token with its first loads (the length, which
  // says which wave reads the last page, is not known yet).
  const bool appends = p.new_key != nullptr;
  NewToken<D> nt;
  if (appends) nt.request(p, seq, kvh, lane);
  PageStream<D> ps = make_stream<D>(p, seq, kvh, lo0 + w, kWaves,
                                    PP > 0 ? min(lo0 + PP, p.max_pages_per_seq)
                                           : p.max_pages_per_seq,
                                    lane);
  const int L = p.context_lens[seq];
  WaveAttn<D> wa;
  wa.init(static_cast<const uint16_t*>(p.query) + (size_t(seq) * p.num_q_heads + kvh * G + r) * D,
          r < G, r, j, p.scale_log2);

  int lo, hi;
  if (!unit_pages(p, seq, part, L, lo, hi)) {
    if (PP == 0) store_zeros<uint16_t, D>(p, seq, kvh);
    return;  // a partition past the context writes nothing
  }
  const int n = min((L + kPage - 1) / kPage, p.max_pages_per_seq);
  const bool writes = appends && hi == n && (hi - 1 - lo) % kWaves == w && nt.valid(p);
  ps.count = w < hi - lo ? (hi - lo - w + kWaves - 1) / kWaves : 0;
  // Cached loads throughout: with four waves per unit this kernel runs far
  // fewer waves than the split one, and the nontemporal hint measured up to
  // 25% slower here (long contexts of the 256-sequence batch).
  wa.run(ps, lo + w, L, lane, /*shared=*/true, writes, nt);
  if (writes) nt.store(p, kvh, lane);

  MergeLds lds(smem);
  if (r < G) {
    if (j == 0) {
      lds.m[w * kMaxGroup + r] = wa.m_run;
      lds.l[w * kMaxGroup + r] = wa.acc[D / 16][0];
    }
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
      *reinterpret_cast<f32x4*>(lds.acc + (w * G + r) * (D + kAccPad) + 16 * db + 4 * j) =
          wa.acc[db];
  }
  merge_and_store<uint16_t, D>(p, lds, seq, kvh, part);
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
