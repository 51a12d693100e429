// The matrix-core page step of bf16 decode (gfx950) and the four-wave decode
// unit built on it, shared by the decode kernels and the shared-prefix
// launch.
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
#pragma once

#include "page_stream.hpp"

namespace pa {

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

// Four-wave unit (sequence, partition, kv head) -- or (sequence, kv head)
// over the whole context when pages_per_partition is 0; wave w takes pages
// w, w+4, ... of the unit, and the four states merge through LDS into the
// output row or the partition's partial.  `shared`: some page the unit reads
// may also be read by another sequence (cached loads); otherwise its pages
// stream with the nontemporal hint.  Every thread of the 256-thread block
// must call it.
template <int D>
__device__ inline void whole_unit(const DecodeParams& p, int seq, int kvh, int part, float* smem,
                                  bool shared) {
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
    if (PP == 0)
      store_zeros<uint16_t, D>(p, seq, kvh);
    else if (part < merged_partitions(p, L))  // past a length clamped to the table
      empty_partials<D>(p, seq, kvh, part, part + 1, threadIdx.x, kBlock);
    return;  // any other partition past the context writes nothing
  }
  const int n = min((L + kPage - 1) / kPage, p.max_pages_per_seq);
  const bool writes = appends && hi == n && (hi - 1 - lo) % kWaves == w && nt.valid(p);
  ps.count = w < hi - lo ? (hi - lo - w + kWaves - 1) / kWaves : 0;
  __builtin_amdgcn_s_setprio(0);  // the prologue ran at raised priority
  wa.run(ps, lo + w, L, lane, shared, writes, nt);
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

}  // namespace pa
