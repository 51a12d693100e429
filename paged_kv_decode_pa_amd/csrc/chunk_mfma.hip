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
// in one tile.  Scores past a column's own position are masked to -inf by
// select, per lane.
//
// A wave carries NB <= 4 consecutive column blocks, so every K/V tile it
// loads serves up to 64 columns (16 new tokens at a group of 4) from one
// read.  Unit = (sequence, kv head, group of NB blocks), four waves; wave w
// takes pages w, w+4, ... up to the group's last position, and the four
// online-softmax states of each block merge through LDS in a fixed order.
// With three or four blocks the query operands sit in LDS (each wave writes
// one block's), which keeps a wave within 256 registers, two per SIMD.
// Units take their sequences as the single-pass decode does: by length,
// longest first, snaked over the compute units (batch order when neighbours
// share their first page), and a sequence that shares no page with another
// streams with the nontemporal hint.  A chunk long enough for several
// column groups rereads its pages, with cached loads, through one XCD's L2
// (the kv-head-fastest unit order puts the groups there).
//
// The same column machinery serves three more kernels here:
//   chunk_split_kernel  the split-KV form of the above (one wave per
//                       sequence, partition, kv head and column group, with
//                       the decode's unit plan), merged by the reduce kernel;
//   prefix_unit         a shared prefix's partition read once per group, the
//                       members' query heads as the columns;
//   cascade_kernel      prefix units and the decode's four-wave units of each
//                       sequence's own partitions in one grid.
#include <limits.h>

#include "split_plan.hpp"
#include "wave_attn.hpp"

namespace pa {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kSlack = 8.0f;  // base 2: P may reach 2^8 before a rescale
constexpr int kChunkRing = 2;   // page tiles per wave in flight or in use (multi-token)
constexpr int kPrefixRing = 2;  // the same for the shared-prefix units

// One wave's online-softmax state for one block of 16 (token, head) columns.
// The query operands live in registers, or (QL) in LDS shared by the
// workgroup's waves, read again for every page: that frees D / 8 registers
// per block, which lets four-block waves run two to a SIMD.
template <int D, bool QL = false>
struct ColumnAttn {
  bf16x8 qop[QL ? 1 : D / 32];  // B operand: column r = (token, head) pair r of the block
  const bf16x8* qlds;    // QL: this lane's operand of k-step kb at qlds[64 * kb]
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
    init_state(r);
  }

  // QL: `slot` is this lane's LDS operand slot of the block; a writer wave
  // fills it from the query row (zero for a padding column).  The caller
  // synchronises the workgroup before the first page.
  __device__ void init_lds(bf16x8* slot, bool writer, const uint16_t* qrow, bool real, int r,
                           int j_, int pos_, float sl2) {
    j = j_;
    pos = pos_;
    scale_log2 = sl2;
    qlds = slot;
    if (writer) {
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (real) v = *reinterpret_cast<const u32x4*>(qrow + 32 * kb + 8 * j);
        slot[64 * kb] = __builtin_bit_cast(bf16x8, v);
      }
    }
    init_state(r);
  }

  __device__ void init_state(int r) {
    ones = s16x4{0, 0, 0, 0};
    if (r == 0) ones = s16x4{0x3F80, 0x3F80, 0x3F80, 0x3F80};
    m_run = -INFINITY;
#pragma unroll
    for (int db = 0; db <= D / 16; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  __device__ bf16x8 q(int kb) const {
    if constexpr (QL) return qlds[64 * kb];
    else return qop[kb];
  }

  // Scores of the page starting at token `base`, base 2.  Masked: with the
  // causal mask (which also masks positions past the context); otherwise
  // every token of the page precedes every real column's position.
  template <bool Masked>
  __device__ void scores(const PageTile<D>& t, int base, float (&s2)[4]) const {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(t.k[kb], q(kb), s, 0, 0, 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (Masked)
        s2[e] = base + 4 * j + e > pos ? -INFINITY : s[e] * scale_log2;
      else
        s2[e] = s[e] * scale_log2;
    }
  }

  // Online-softmax update with the page's scores, given whether any lane's
  // score exceeds its reference by more than kSlack (`raise`, a wave ballot).
  // A column may have no unmasked token on a page (its position precedes the
  // page): its P is then 0, and while its reference is still -inf the
  // rescale factor is 0, so no 0 * inf or inf - inf arises.
  // Unmasked, every column has 16 finite scores, so after the rescale its
  // reference is finite and no select is needed.
  template <bool Masked>
  __device__ void accumulate(const PageTile<D>& t, const float (&s2)[4], float lm, bool raise) {
    if (raise) {
      float pm = fmaxf(lm, __shfl_xor(lm, 16));
      pm = fmaxf(pm, __shfl_xor(pm, 32));
      const float m_new = fmaxf(m_run, pm);
      const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
#pragma unroll
      for (int db = 0; db <= D / 16; ++db) acc[db] *= alpha;
    }
    // P to bf16 (round to nearest even) two at a time; a masked score gives 0.
    float pf[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p = __builtin_amdgcn_exp2f(s2[e] - m_run);
      if constexpr (Masked)
        pf[e] = s2[e] == -INFINITY ? 0.f : p;
      else
        pf[e] = p;
    }
    const bf16x2 lo2 = __builtin_convertvector((f32x2){pf[0], pf[1]}, bf16x2);
    const bf16x2 hi2 = __builtin_convertvector((f32x2){pf[2], pf[3]}, bf16x2);
    const s16x4 pb = __builtin_bit_cast(
        s16x4, (u32x2){__builtin_bit_cast(uint32_t, lo2), __builtin_bit_cast(uint32_t, hi2)});
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(t.v[db], pb, acc[db], 0, 0, 0);
    acc[D / 16] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ones, pb, acc[D / 16], 0, 0, 0);
  }
};

// Slots at or past `valid` of a partial page may hold NaN; 0 * NaN would
// reach the accumulator, so their V elements are zeroed (by select).
template <int D>
__device__ inline void zero_past(PageTile<D>& t, int valid, int j) {
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
#pragma unroll
    for (int e = 0; e < 4; ++e) t.v[db][e] = 4 * j + e < valid ? t.v[db][e] : short(0);
}

// One page for the wave's NB column blocks.  All blocks' score products and
// their first vector reads come before the first branch (the ballots'
// rescales): with a data-dependent branch between a matrix instruction and
// the reads of its result, the compiler was seen to let a taken branch reach
// the reads fewer wait states after the instruction than the result needs
// (wrong, run-to-run varying scores).
template <int D, int NB, bool Masked, bool QL>
__device__ inline void page_blocks(ColumnAttn<D, QL> (&wa)[NB], const PageTile<D>& t, int base) {
  float s2[NB][4];
  float lm[NB];
  bool raise[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) wa[nb].template scores<Masked>(t, base, s2[nb]);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    lm[nb] = fmaxf(fmaxf(s2[nb][0], s2[nb][1]), fmaxf(s2[nb][2], s2[nb][3]));
    raise[nb] = __ballot(lm[nb] > wa[nb].m_run + kSlack) != 0;
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) wa[nb].template accumulate<Masked>(t, s2[nb], lm[nb], raise[nb]);
}

// A ring of R tiles per wave; ordinal k is page page0 + step * k.  Pages
// k .. k+R-1 are computed in turn, each slot refilled with the page R
// ordinals ahead as soon as it has been used, so R - 1 loads are in flight
// while a page is computed.  (Three or four tiles measured no faster than
// two at 4 to 64 new tokens, and slower for the shared-prefix units: the
// page step's own vector and matrix work, not the load latency, sets the
// pace at one wave per SIMD.)  The first loop runs while all R pages of a
// step lie wholly before `visible_end` (every real column of the wave sees
// all their tokens): far from the diagonal, which is most pages of a long
// context, the step skips the causal mask and its selects.  One loop per
// variant keeps a single copy of the page step in each loop body.  The
// loops stop while every refill still exists (k + 2R <= n), so the pages
// they compute are all full (only the sequence's last page can be partial);
// the tail computes the ring's pages, refills what remains, and computes
// those, each zeroed past the context first.
template <int D, int NB, int R, bool Stream = false, bool QL = false>
__device__ inline void run_blocks(ColumnAttn<D, QL> (&wa)[NB], PageStream<D>& ps, int page0, int L,
                                  int visible_end, int lane) {
  const int n = ps.count;
  if (n <= 0) return;
  const int j = lane >> 4;
  auto base = [&](int k) { return (page0 + ps.step * k) * kPage; };
  // Ordinals below n_clear hold pages wholly before visible_end.
  const int last_clear = visible_end / kPage - 1;  // last page index wholly visible
  const int n_clear = last_clear < page0 ? 0 : (last_clear - page0) / ps.step + 1;
  PageTile<D> t[R];
  bool ok[R];
#pragma unroll
  for (int i = 0; i < R; ++i) ok[i] = ps.template issue<Stream>(t[i], i, lane);
  int k = 0;
  for (; k + 2 * R <= n && k + R <= n_clear; k += R) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      if (ok[i]) page_blocks<D, NB, false, QL>(wa, t[i], base(k + i));
      ok[i] = ps.template issue<Stream>(t[i], k + i + R, lane);
    }
  }
  for (; k + 2 * R <= n; k += R) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      if (ok[i]) page_blocks<D, NB, true, QL>(wa, t[i], base(k + i));
      ok[i] = ps.template issue<Stream>(t[i], k + i + R, lane);
    }
  }
#pragma unroll
  for (int i = 0; i < R; ++i) {
    if (k + i < n) {
      if (ok[i]) {
        zero_past(t[i], L - base(k + i), j);
        page_blocks<D, NB, true, QL>(wa, t[i], base(k + i));
      }
      ok[i] = k + i + R < n && ps.template issue<Stream>(t[i], k + i + R, lane);
    }
  }
#pragma unroll
  for (int i = 0; i < R; ++i) {
    if (k + R + i < n && ok[i]) {
      zero_past(t[i], L - base(k + R + i), j);
      page_blocks<D, NB, true, QL>(wa, t[i], base(k + R + i));
    }
  }
}

// Every page of the stream is seen whole by every column (a shared prefix):
// the mask-free step throughout, and no page is partial.  Ring as above.
template <int D, int NB, int R>
__device__ inline void run_clear(ColumnAttn<D> (&wa)[NB], PageStream<D>& ps, int page0, int lane) {
  const int n = ps.count;
  if (n <= 0) return;
  auto base = [&](int k) { return (page0 + ps.step * k) * kPage; };
  PageTile<D> t[R];
  bool ok[R];
#pragma unroll
  for (int i = 0; i < R; ++i) ok[i] = ps.template issue<false>(t[i], i, lane);
  int k = 0;
  for (; k + 2 * R <= n; k += R) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      if (ok[i]) page_blocks<D, NB, false, false>(wa, t[i], base(k + i));
      ok[i] = ps.template issue<false>(t[i], k + i + R, lane);
    }
  }
#pragma unroll
  for (int i = 0; i < R; ++i) {
    if (k + i < n) {
      if (ok[i]) page_blocks<D, NB, false, false>(wa, t[i], base(k + i));
      ok[i] = k + i + R < n && ps.template issue<false>(t[i], k + i + R, lane);
    }
  }
#pragma unroll
  for (int i = 0; i < R; ++i)
    if (k + R + i < n && ok[i]) page_blocks<D, NB, false, false>(wa, t[i], base(k + R + i));
}

// LDS of the four-wave merge: per wave a reference and a sum per column and
// the un-normalised accumulator [wave][column][D].
__host__ __device__ inline size_t chunk_lds_bytes(int head_dim) {
  return sizeof(float) * (2 * kWaves * 16 + size_t(kWaves) * 16 * (head_dim + kAccPad));
}

// Waves of three or four column blocks keep the query operands in LDS, after
// the merge's area: 16 bytes per lane and k-step of each block.
constexpr bool chunk_query_in_lds(int nb) { return nb >= 3; }
__host__ __device__ inline size_t chunk_query_lds_bytes(int head_dim, int nb) {
  return chunk_query_in_lds(nb) ? size_t(nb) * (head_dim / 32) * 64 * 16 : 0;
}

template <int D, int NB>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(NB >= 3 ? 2 : 1)))
void chunk_attention_kernel(ChunkParams p) {
  extern __shared__ float smem[];
  const int u = blockIdx.x;
  if (u >= p.num_units) return;
  const int lane = threadIdx.x & 63;
  const int kvh = u % p.num_kv_heads;
  const int rest = u / p.num_kv_heads;
  const int grp = rest % p.groups_per_seq;
  const int slot = rest / p.groups_per_seq;
  bool shared;
  const int seq = snake_unit_seq_of_batch(p, slot, lane, shared);
  shared = shared || p.groups_per_seq > 1;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, j = lane >> 4;
  const int G = p.group;

  const int q0 = p.query_start[seq];
  const int q_len = p.query_start[seq + 1] - q0;
  const int cols = q_len * G;                  // (token, head) columns of this kv head
  const int c0 = grp * NB * 16;                // first column of the group's first block
  // The whole workgroup leaves together; malformed offsets write nothing.
  if (q_len <= 0 || c0 >= cols || q0 < 0 || q0 + q_len > p.num_query_tokens) return;
  const int L = min(p.context_lens[seq], p.max_pages_per_seq * kPage);
  const int last_pos = L - q_len + (min(c0 + NB * 16 - 1, cols - 1) / G);
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

  constexpr bool QL = chunk_query_in_lds(NB);
  bf16x8* qslots = reinterpret_cast<bf16x8*>(smem + chunk_lds_bytes(D) / sizeof(float));
  ColumnAttn<D, QL> wa[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int c = c0 + 16 * nb + r;
    const bool real = c < cols;
    const int i = real ? c / G : 0;
    const int h = real ? c % G : 0;
    const uint16_t* qrow = static_cast<const uint16_t*>(p.query) +
                           (size_t(q0 + i) * p.num_q_heads + kvh * G + h) * D;
    // position of the column's token (< 0 only if q_len exceeds the context)
    const int pos = real ? L - q_len + i : -1;
    if constexpr (QL)  // wave nb writes block nb's operands
      wa[nb].init_lds(qslots + (nb * (D / 32)) * 64 + lane, w == nb, qrow, real, r, j, pos,
                      p.scale_log2);
    else
      wa[nb].init(qrow, real, r, j, pos, p.scale_log2);
  }
  if constexpr (QL) __syncthreads();
  // Tokens below visible_end are seen by every real column of the group (the
  // first column's token sits at the smallest position).
  const int visible_end = L - q_len + c0 / G + 1;
  if (shared)
    run_blocks<D, NB, kChunkRing, false, QL>(wa, ps, w, L, visible_end, lane);
  else
    run_blocks<D, NB, kChunkRing, true, QL>(wa, ps, w, L, visible_end, lane);

  // Merge the four waves per column (fixed wave order) and store the rows,
  // one block at a time through the same LDS.
  float* lm = smem;                       // [kWaves][16]
  float* ll = smem + kWaves * 16;         // [kWaves][16]
  float* la = smem + 2 * kWaves * 16;     // [kWaves][16][D + kAccPad]
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int c_lo = c0 + 16 * nb;
    if (c_lo >= cols) break;  // uniform: the group's remaining blocks are empty
    if (nb > 0) __syncthreads();  // the previous block's reads are done
    if (j == 0) {
      lm[w * 16 + r] = wa[nb].m_run;
      ll[w * 16 + r] = wa[nb].acc[D / 16][0];
    }
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
      *reinterpret_cast<f32x4*>(la + (w * 16 + r) * (D + kAccPad) + 16 * db + 4 * j) =
          wa[nb].acc[db];
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
        num += la[(v * 16 + col) * (D + kAccPad) + d] * f;
      }
      const int row = q0 + cc / G;
      const int head = kvh * G + cc % G;
      Elem<uint16_t>::store(p.out, (size_t(row) * p.num_q_heads + head) * D + d,
                            wsum > 0.f ? num / wsum : 0.f);
    }
  }
}

// Split-KV form for a few new tokens per sequence (draft verification): the
// single-pass units above take as long as their longest sequence's four
// waves, so here one wave per (sequence, partition, kv head, column group)
// streams the partition's pages and writes each of its (token, head)
// columns' partial straight from registers, as the split decode does, with
// the decode's device-side unit plan (full partitions first, no unit past a
// context) and its load policy (the nontemporal hint for pages that only
// this unit reads).  A column whose position precedes the whole partition
// sees none of its keys: its partial is empty (o = 0, m = -inf, l = 0),
// which the merge weighs by 0.
template <int D, int NB, int NC>
__global__ __launch_bounds__(64) void chunk_split_kernel(ChunkParams p) {
  const int u = blockIdx.x;
  if (u >= p.num_units) return;
  const int kvh = u % p.num_kv_heads;
  const int rest = u / p.num_kv_heads;
  const int grp = rest % p.groups_per_seq;
  const int useq = rest / p.groups_per_seq;
  const int lane = threadIdx.x;
  const int r = lane & 15, j = lane >> 4;
  const int G = p.group;

  // The sharing test's loads depend on nothing: they go out with the plan's.
  SharingTest<NC> sharing;
  sharing.request(p, lane);
  int seq, part, seq_pages = 0;
  if constexpr (NC > 0) {
    if (!split_unit<NC>(p, useq, lane, seq, part, seq_pages)) return;
  } else {
    seq = useq % p.num_seqs;  // plain grid: partitions past a context exit below
    part = useq / p.num_seqs;
  }
  seq = __builtin_amdgcn_readfirstlane(seq);
  part = __builtin_amdgcn_readfirstlane(part);

  // Issued together before any of them returns: the token offsets, the
  // length and the partition's page ids.
  const int qa = p.query_start[seq];
  const int qb = p.query_start[seq + 1];
  const int L_raw = p.context_lens[seq];
  const int PP = p.pages_per_partition;
  const int lo = part * PP;
  PageStream<D> ps;
  ps.table = p.block_tables + size_t(seq) * p.max_pages_per_seq;
  ps.first = lo;
  ps.step = 1;
  ps.row_end = min(lo + PP, p.max_pages_per_seq);
  ps.kpool = static_cast<const char*>(p.k_cache);
  ps.vpool = static_cast<const char*>(p.v_cache);
  ps.num_pages = p.num_pages;
  ps.num_kv_heads = p.num_kv_heads;
  ps.kvh = kvh;
  ps.koff = uint32_t(r * D + 8 * j) * 2u;
  ps.voff = uint32_t(r * kPage + 4 * j) * 2u;
  ps.start(lane);

  const int q0 = qa;
  const int q_len = qb - qa;
  const int cols = q_len * G;
  const int c0 = grp * NB * 16;
  if (q_len <= 0 || c0 >= cols || q0 < 0 || q0 + q_len > p.num_query_tokens) return;
  const int L = min(L_raw, p.max_pages_per_seq * kPage);
  const int n = (L + kPage - 1) / kPage;
  if (lo >= n) return;  // partition past the context: the merge does not read it
  // Pages this group's last column can see (its token is the group's latest).
  const int last_pos = L - q_len + (min(c0 + NB * 16 - 1, cols - 1) / G);
  const int hi = max(lo, min(min(lo + PP, n), last_pos >= 0 ? last_pos / kPage + 1 : 0));
  ps.count = hi - lo;

  ColumnAttn<D> wa[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int c = c0 + 16 * nb + r;
    const bool real = c < cols;
    const int i = real ? c / G : 0;
    const int h = real ? c % G : 0;
    const uint16_t* qrow = static_cast<const uint16_t*>(p.query) +
                           (size_t(q0 + i) * p.num_q_heads + kvh * G + h) * D;
    wa[nb].init(qrow, real, r, j, real ? L - q_len + i : -1, p.scale_log2);
  }
  const int visible_end = L - q_len + c0 / G + 1;
  // One reader per page: a single column group and a sequence whose pages
  // no other sequence holds.
  if (p.groups_per_seq == 1 && !sharing.shared(p, seq, lane))
    run_blocks<D, NB, kChunkRing, true>(wa, ps, lo, L, visible_end, lane);
  else
    run_blocks<D, NB, kChunkRing, false>(wa, ps, lo, L, visible_end, lane);

  // Partials of this partition: o = acc / l, m in natural-log units, l.
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int c = c0 + 16 * nb + r;
    const float l = __shfl(wa[nb].acc[D / 16][0], r);  // row 0 of the denominator block
    if (c < cols) {
      const size_t row =
          (size_t(q0 + c / G) * p.num_q_heads + kvh * G + c % G) * p.num_partitions + part;
      float* dst = p.partial_out + row * D;
      const float inv = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
      for (int db = 0; db < D / 16; ++db)
        *reinterpret_cast<f32x4*>(dst + 16 * db + 4 * j) = wa[nb].acc[db] * inv;
      if (j == 0) {
        p.partial_max[row] = l > 0.f ? wa[nb].m_run * kLn2 : -INFINITY;
        p.partial_sum[row] = l;
      }
    }
  }
}

// Shared-prefix partials.  Unit = (group, shared partition, column group,
// kv head), four waves; wave w takes the partition's pages w, w+4, ... from
// the first member's block-table row (the members hold the same page ids
// there).  Column c of the unit's blocks is member c / group, query head
// c % group of the kv head.  (Eight waves per unit, each walking half the
// pages, measured slower.)
template <int D, int NB>
__device__ inline void prefix_unit(const PrefixParams& p, int u, float* smem) {
  const int kvh = u % p.num_kv_heads;
  int rest = u / p.num_kv_heads;
  const int cg = rest % p.column_groups;
  rest /= p.column_groups;
  const int part = rest % p.max_group_partitions;
  const int g = rest / p.max_group_partitions;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, j = lane >> 4;
  const int G = p.group;

  const int gs = p.group_start[g];
  const int members = p.group_start[g + 1] - gs;
  const int cols = members * G;
  const int c0 = cg * NB * 16;
  if (members <= 0 || part >= p.group_partitions[g] || c0 >= cols) return;  // uniform
  const int PP = p.pages_per_partition;
  const int lo = part * PP;
  const int hi = min(lo + PP, p.max_pages_per_seq);
  const int first_seq = p.group_seqs[gs];
  if (first_seq < 0 || first_seq >= p.num_seqs) return;  // uniform

  PageStream<D> ps;
  ps.table = p.block_tables + size_t(first_seq) * p.max_pages_per_seq;
  ps.first = lo + w;
  ps.step = kWaves;
  ps.row_end = hi;
  ps.kpool = static_cast<const char*>(p.k_cache);
  ps.vpool = static_cast<const char*>(p.v_cache);
  ps.num_pages = p.num_pages;
  ps.num_kv_heads = p.num_kv_heads;
  ps.kvh = kvh;
  ps.koff = uint32_t(r * D + 8 * j) * 2u;
  ps.voff = uint32_t(r * kPage + 4 * j) * 2u;
  ps.start(lane);
  ps.count = lo + w < hi ? (hi - lo - w + kWaves - 1) / kWaves : 0;

  ColumnAttn<D> wa[NB];
  int col_seq[NB];  // batch index of column r's member, -1 for no member
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int c = c0 + 16 * nb + r;
    int seq = c < cols ? p.group_seqs[gs + c / G] : -1;
    const bool real = seq >= 0 && seq < p.num_seqs;
    col_seq[nb] = real ? seq : -1;
    if (!real) seq = 0;
    const int h = real ? c % G : 0;
    const uint16_t* qrow = static_cast<const uint16_t*>(p.query) +
                           (size_t(seq) * p.num_q_heads + kvh * G + h) * D;
    wa[nb].init(qrow, real, r, j, INT_MAX, p.scale_log2);
  }
  run_clear<D, NB, kPrefixRing>(wa, ps, lo + w, lane);

  // Merge the four waves per column and write each member's partial for this
  // partition, one block at a time through the same LDS.  The columns'
  // members go to LDS once, so the stores wait on no global load.
  float* lm = smem;                 // [kWaves][16]
  float* ll = smem + kWaves * 16;        // [kWaves][16]
  float* la = smem + 2 * kWaves * 16;    // [kWaves][16][D + kAccPad]
  int* lseq = reinterpret_cast<int*>(la + kWaves * 16 * (D + kAccPad));  // [NB][16]
  if (w == 0 && j == 0) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) lseq[nb * 16 + r] = col_seq[nb];
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int c_lo = c0 + 16 * nb;
    if (c_lo >= cols) break;  // uniform
    if (nb > 0) __syncthreads();
    if (j == 0) {
      lm[w * 16 + r] = wa[nb].m_run;
      ll[w * 16 + r] = wa[nb].acc[D / 16][0];
    }
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
      *reinterpret_cast<f32x4*>(la + (w * 16 + r) * (D + kAccPad) + 16 * db + 4 * j) =
          wa[nb].acc[db];
    __syncthreads();
    // Thread: one column's four consecutive dims per step.
    for (int idx = threadIdx.x; idx < 16 * (D / 4); idx += kBlock) {
      const int col = idx / (D / 4);
      const int d = 4 * (idx % (D / 4));
      const int cc = c_lo + col;
      const int seq = lseq[nb * 16 + col];
      if (cc >= cols || seq < 0) continue;
      float M = -INFINITY;
#pragma unroll
      for (int v = 0; v < kWaves; ++v) M = fmaxf(M, lm[v * 16 + col]);
      float wsum = 0.f;
      f32x4 num = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int v = 0; v < kWaves; ++v) {
        const float mv = lm[v * 16 + col];
        const float f = mv == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mv - M);
        wsum += ll[v * 16 + col] * f;
        num += *reinterpret_cast<const f32x4*>(la + (v * 16 + col) * (D + kAccPad) + d) * f;
      }
      const size_t row =
          (size_t(seq) * p.num_q_heads + kvh * G + cc % G) * p.num_partitions + part;
      f32x4 o = {0.f, 0.f, 0.f, 0.f};
      if (wsum > 0.f) {
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = num[e] / wsum;
      }
      *reinterpret_cast<f32x4*>(p.partial_out + row * D + d) = o;
      if (d == 0) {
        p.partial_max[row] = M * kLn2;
        p.partial_sum[row] = wsum;
      }
    }
  }
}

// The shared-prefix step in one launch: blocks below q.num_units are the
// prefix units (the longest, dispatched first), the rest the four-wave
// split-KV units of every sequence's own partitions.  The two sets write
// disjoint partials and touch disjoint pages (a page that receives the
// step's token is never shared), so they need no ordering; in one grid the
// suffix units fill the machine while the prefix units stream, and each
// set's setup and merge phases overlap the other's page loads.
template <int D, int NB>
__global__ __launch_bounds__(kBlock) void cascade_kernel(PrefixParams q, DecodeParams p) {
  extern __shared__ float smem[];
  const int b = blockIdx.x;
  if (b < q.num_units) {
    prefix_unit<D, NB>(q, b, smem);
    return;
  }
  int seq, kvh, part;
  if (!unit_of(p, b - q.num_units, seq, kvh, part)) return;
  __builtin_amdgcn_s_setprio(3);  // lowered before the page stream starts
  if (p.grid_partitions == 1 && p.first_partition != nullptr) {
    // One suffix unit per (sequence, kv head): the longest sequences first,
    // so the second round of units ends with the short ones.
    const int slot = (b - q.num_units) / p.num_kv_heads;
    seq = longest_first_of_batch(p, slot, threadIdx.x & 63);
    const int f = p.first_partition[seq];
    part = f < 0 ? 0 : f > p.num_partitions ? p.num_partitions : f;
    if (part >= p.num_partitions) return;
  }
  // Cached loads: the nontemporal hint on these units (a sequence's own
  // partitions, past its group's shared prefix) measured 5% slower.
  whole_unit<D>(p, seq, kvh, part, smem, /*shared=*/true);
}

template <int D>
void launch_d(const ChunkParams& p, hipStream_t stream) {
  const dim3 grid(p.num_units);
  const size_t lds = chunk_lds_bytes(D);
#define PA_CHUNK(NBB) \
  chunk_attention_kernel<D, NBB><<<grid, kBlock, lds + chunk_query_lds_bytes(D, NBB), stream>>>(p)
  switch (p.blocks_per_wave) {
    case 1: PA_CHUNK(1); break;
    case 2: PA_CHUNK(2); break;
    case 3: PA_CHUNK(3); break;
    default: PA_CHUNK(4); break;
  }
#undef PA_CHUNK
}

}  // namespace

hipError_t launch_cascade(const PrefixParams& q, const DecodeParams& p, int head_dim,
                          hipStream_t stream) {
  const size_t prefix_lds = sizeof(float) * (2 * kWaves * 16 + size_t(kWaves) * 16 *
                                             (head_dim + kAccPad)) + sizeof(int) * 2 * 16;
  const size_t suffix_lds = merge_lds_bytes(p.group, head_dim);
  const size_t lds = prefix_lds > suffix_lds ? prefix_lds : suffix_lds;
  const dim3 grid(q.num_units + p.num_units);
#define PA_CASCADE(DD, NBB) cascade_kernel<DD, NBB><<<grid, kBlock, lds, stream>>>(q, p)
  if (head_dim == 128) {
    if (q.blocks_per_wave == 1) PA_CASCADE(128, 1); else PA_CASCADE(128, 2);
  } else {
    if (q.blocks_per_wave == 1) PA_CASCADE(64, 1); else PA_CASCADE(64, 2);
  }
#undef PA_CASCADE
  return hipGetLastError();
}

hipError_t launch_chunk_attention(const ChunkParams& p, int head_dim, hipStream_t stream) {
  if (p.pages_per_partition > 0) {
    const dim3 grid(p.num_units);
#define PA_CHUNK_SPLIT(DD, NBB)                                                          \
  switch (plan_chunks_for(p.num_seqs)) {                                                 \
    case 1: chunk_split_kernel<DD, NBB, 1><<<grid, 64, 0, stream>>>(p); break;           \
    case 4: chunk_split_kernel<DD, NBB, 4><<<grid, 64, 0, stream>>>(p); break;           \
    case kPlanChunks: chunk_split_kernel<DD, NBB, kPlanChunks><<<grid, 64, 0, stream>>>(p); break; \
    default: chunk_split_kernel<DD, NBB, 0><<<grid, 64, 0, stream>>>(p); break;          \
  }
#define PA_CHUNK_SPLIT_D(DD)                                   \
  switch (p.blocks_per_wave) {                                 \
    case 1: PA_CHUNK_SPLIT(DD, 1); break;                      \
    case 2: PA_CHUNK_SPLIT(DD, 2); break;                      \
    case 3: PA_CHUNK_SPLIT(DD, 3); break;                      \
    default: PA_CHUNK_SPLIT(DD, 4); break;                     \
  }
    if (head_dim == 128) {
      PA_CHUNK_SPLIT_D(128)
    } else {
      PA_CHUNK_SPLIT_D(64)
    }
#undef PA_CHUNK_SPLIT_D
#undef PA_CHUNK_SPLIT
    return hipGetLastError();
  }
  if (head_dim == 128)
    launch_d<128>(p, stream);
  else
    launch_d<64>(p, stream);
  return hipGetLastError();
}

}  // namespace pa
