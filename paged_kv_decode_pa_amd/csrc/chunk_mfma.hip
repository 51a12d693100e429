// Multi-token causal attention over the paged cache on the matrix cores
// (bf16, gfx950): the step that serves chunked prefill and the verification
// of drafted tokens.  Sequence b's q_len new tokens are its last q_len
// positions (their K/V already in the cache) and the token at position p
// attends to positions 0..p.
//
// The per-page step is the decode kernel's, with the 16 columns of the
// matrix tile generalised from "the group's query heads" to (query token,
// head) pairs: column c = i * group + h of a block is token i, head h.  So a
// group of 4 puts four consecutive tokens of one kv head's four query heads
// in one tile, and every K/V page loaded serves all of them.  Scores past a
// column's own position are masked to -inf by select, per lane.
//
// Unit = (sequence, kv head, column block), four waves; wave w takes pages
// w, w+4, ... up to the block's last position, and the four online-softmax
// states merge through LDS in a fixed order.  Pages are read with cached
// loads: the column blocks of one (sequence, kv head) reread the same pages,
// and the kv-head-fastest unit order puts them on one XCD's L2.
#include "page_stream.hpp"

namespace pa {
namespace {

constexpr float kSlack = 8.0f;  // base 2: P may reach 2^8 before a rescale

// One wave's online-softmax state for one block of 16 (token, head) columns.
template <int D>
struct ColumnAttn {
  bf16x8 qop[D / 32];    // B operand: column r = (token, head) pair r of the block
  s16x4 ones;            // A operand of the denominator block
  f32x4 acc[D / 16 + 1]; // O^T blocks (lane: dims 16db+4j.., column r), then the denominator
  float m_run;           // base-2 reference score of column r (equal in its 4 lane groups)
  float scale_log2;
  int j;
  int pos;               // position of column r's token; tokens after it are masked

  __device__ void init(const uint16_t* qrow, bool real, int r, int j_, int pos_, float sl2) {
    j = j_;
    pos = pos_;
    scale_log2 = sl2;
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (real) v = *reinterpret_cast<const u32x4*>(qrow + 32 * kb + 8 * j);
      qop[kb] = __builtin_bit_cast(bf16x8, v);
    }
    ones = s16x4{0, 0, 0, 0};
    if (r == 0) ones = s16x4{0x3F80, 0x3F80, 0x3F80, 0x3F80};
    m_run = -INFINITY;
#pragma unroll
    for (int db = 0; db <= D / 16; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Page starting at token `base`, with `valid` tokens of the context in it.
  // A column may have no unmasked token on a page (its position precedes the
  // page): its P is then 0, and while its reference is still -inf nothing is
  // rescaled, so no 0 * inf or inf - inf arises.
  //
  // Between the score products and the first vector instruction that reads
  // them there is no branch: with a data-dependent branch in between (the
  // zeroing of a partial page's V, which used to sit there), the compiler let
  // a taken branch reach the reads fewer wait states after the matrix
  // instruction than its result needs, and the scores of whole pages came out
  // wrong and varied from run to run.  Only the sequence's last page can hold
  // unwritten slots, and a wave meets it only after the steady-state loop
  // (`Tail`); there the V zeroing is done by select, with no branch at all.
  template <bool Tail>
  __device__ void page(PageTile<D>& t, int base, int valid) {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(t.k[kb], qop[kb], s, 0, 0, 0);
    float s2[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)  // causal, which also masks past the context
      s2[e] = base + 4 * j + e > pos ? -INFINITY : s[e] * scale_log2;
    if constexpr (Tail) {
#pragma unroll
      for (int db = 0; db < D / 16; ++db)
#pragma unroll
        for (int e = 0; e < 4; ++e)  // unwritten slots may hold NaN
          t.v[db][e] = 4 * j + e < valid ? t.v[db][e] : short(0);
    }
    const float lm = fmaxf(fmaxf(s2[0], s2[1]), fmaxf(s2[2], s2[3]));
    if (__ballot(lm > m_run + kSlack) != 0) {
      float pm = fmaxf(lm, __shfl_xor(lm, 16));
      pm = fmaxf(pm, __shfl_xor(pm, 32));
      const float m_new = fmaxf(m_run, pm);
      const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
#pragma unroll
      for (int db = 0; db <= D / 16; ++db) acc[db] *= alpha;
    }
    s16x4 pb;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      pb[e] = s2[e] == -INFINITY
                  ? short(0)
                  : static_cast<short>(f32_to_bf16(__builtin_amdgcn_exp2f(s2[e] - m_run)));
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(t.v[db], pb, acc[db], 0, 0, 0);
    acc[D / 16] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ones, pb, acc[D / 16], 0, 0, 0);
  }

  // Two tiles in ping-pong, as in the decode kernel; ordinal k is page
  // page0 + step * k.  The loop stops three ordinals before the end, so the
  // pages it computes are all full; the last one to three go through the
  // tail step.
  __device__ void run(PageStream<D>& ps, int page0, int L, int lane) {
    const int n = ps.count;
    if (n <= 0) return;
    auto base = [&](int k) { return (page0 + ps.step * k) * kPage; };
    PageTile<D> ta, tb;
    bool ok_a = ps.template issue<false>(ta, 0, lane);
    bool ok_b = ps.template issue<false>(tb, 1, lane);
    int k = 0;
    for (; k + 3 < n; k += 2) {
      if (ok_a) page<false>(ta, base(k), kPage);
      ok_a = ps.template issue<false>(ta, k + 2, lane);
      if (ok_b) page<false>(tb, base(k + 1), kPage);
      ok_b = ps.template issue<false>(tb, k + 3, lane);
    }
    const int rem = n - k;
    if (ok_a) page<true>(ta, base(k), L - base(k));
    if (rem >= 2) {
      const bool ok_c = rem == 3 && ps.template issue<false>(ta, k + 2, lane);
      if (ok_b) page<true>(tb, base(k + 1), L - base(k + 1));
      if (ok_c) page<true>(ta, base(k + 2), L - base(k + 2));
    }
  }
};

// LDS of the four-wave merge: per wave a reference and a sum per column and
// the un-normalised accumulator [wave][column][D].
__host__ __device__ inline size_t chunk_lds_bytes(int head_dim) {
  return sizeof(float) * (2 * kWaves * 16 + size_t(kWaves) * 16 * head_dim);
}

template <int D>
__global__ __launch_bounds__(kBlock) void chunk_attention_kernel(ChunkParams p) {
  extern __shared__ float smem[];
  const int u = blockIdx.x;
  if (u >= p.num_units) return;
  const int kvh = u % p.num_kv_heads;
  const int rest = u / p.num_kv_heads;
  const int cb = rest % p.blocks_per_seq;
  const int seq = rest / p.blocks_per_seq;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, j = lane >> 4;
  const int G = p.group;

  const int q0 = p.query_start[seq];
  const int q_len = p.query_start[seq + 1] - q0;
  const int cols = q_len * G;                  // (token, head) columns of this kv head
  const int c_lo = cb * 16;
  // The whole workgroup leaves together; malformed offsets write nothing.
  if (q_len <= 0 || c_lo >= cols || q0 < 0 || q0 + q_len > p.num_query_tokens) return;
  const int L = min(p.context_lens[seq], p.max_pages_per_seq * kPage);

  const int c = c_lo + r;
  const bool real = c < cols;
  const int i = real ? c / G : 0;
  const int h = real ? c % G : 0;
  const int pos = L - q_len + i;               // < 0 only if q_len exceeds the context
  const int last_pos = L - q_len + (min(c_lo + 15, cols - 1) / G);
  const int n_pages = last_pos >= 0 ? last_pos / kPage + 1 : 0;

  PageStream<D> ps;
  ps.table = p.block_tables + size_t(seq) * p.max_pages_per_seq;
  ps.first = w;
  ps.step = kWaves;
  ps.row_end = p.max_pages_per_seq;
  ps.kpool = static_cast<const char*>(p.k_cache);
  ps.vpool = static_cast<const char*>(p.v_cache);
  ps.num_pages = p.num_pages;
  ps.num_kv_heads = p.num_kv_heads;
  ps.kvh = kvh;
  ps.koff = uint32_t(r * D + 8 * j) * 2u;
  ps.voff = uint32_t(r * kPage + 4 * j) * 2u;
  ps.start(lane);
  ps.count = w < n_pages ? (n_pages - w + kWaves - 1) / kWaves : 0;

  ColumnAttn<D> wa;
  const uint16_t* qrow =
      static_cast<const uint16_t*>(p.query) + (size_t(q0 + i) * p.num_q_heads + kvh * G + h) * D;
  wa.init(qrow, real, r, j, real ? pos : -1, p.scale_log2);
  wa.run(ps, w, L, lane);

  // Merge the four waves per column (fixed wave order) and store the rows.
  float* lm = smem;                       // [kWaves][16]
  float* ll = smem + kWaves * 16;         // [kWaves][16]
  float* la = smem + 2 * kWaves * 16;     // [kWaves][16][D]
  if (j == 0) {
    lm[w * 16 + r] = wa.m_run;
    ll[w * 16 + r] = wa.acc[D / 16][0];
  }
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
#pragma unroll
    for (int e = 0; e < 4; ++e) la[(w * 16 + r) * D + 16 * db + 4 * j + e] = wa.acc[db][e];
  __syncthreads();
  for (int idx = threadIdx.x; idx < 16 * D; idx += kBlock) {
    const int col = idx / D;
    const int d = idx % D;
    const int cc = c_lo + col;
    if (cc >= cols) continue;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) M = fmaxf(M, lm[v * 16 + col]);
    float wsum = 0.f, num = 0.f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
      const float mv = lm[v * 16 + col];
      const float f = mv == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mv - M);
      wsum += ll[v * 16 + col] * f;
      num += la[(v * 16 + col) * D + d] * f;
    }
    const int row = q0 + cc / G;
    const int head = kvh * G + cc % G;
    Elem<uint16_t>::store(p.out, (size_t(row) * p.num_q_heads + head) * D + d,
                          wsum > 0.f ? num / wsum : 0.f);
  }
}

}  // namespace

hipError_t launch_chunk_attention(const ChunkParams& p, int head_dim, hipStream_t stream) {
  const size_t lds = chunk_lds_bytes(head_dim);
  if (head_dim == 128)
    chunk_attention_kernel<128><<<dim3(p.num_units), kBlock, lds, stream>>>(p);
  else
    chunk_attention_kernel<64><<<dim3(p.num_units), kBlock, lds, stream>>>(p);
  return hipGetLastError();
}

}  // namespace pa
