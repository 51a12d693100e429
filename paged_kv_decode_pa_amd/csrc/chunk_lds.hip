// Multi-token causal attention for many new tokens per sequence (chunked
// prefill, long drafts) on the matrix cores, bf16 (gfx950).
//
// Where chunk_attention_kernel splits a sequence's pages over four waves and
// has every wave carry up to 64 columns, this kernel splits the columns:
// unit = (sequence, kv head, group of 32 W columns), W = 4 waves (up to 128
// columns per kv head) or 8 (more), wave w owns 32 columns (column c = token
// * group + head, as there) and walks every key position its columns can
// see.  The K and V of each 32-key step (two pages) are read from HBM once
// per unit by all its threads, staged in LDS (double buffered, further steps
// of loads in flight in registers) and read by the W waves from there.
//
// Per step and wave, with v_mfma_f32_32x32x16_bf16:
//   S^T[32 keys][32 cols]  = K[32][D] . Q^T[D][32]    D/16 products; A = K
//                            rows from LDS, B = the wave's query columns
//                            (registers, loaded once);
//   online softmax on S^T  (a lane holds 16 keys of one column, its partner
//                            lane 32 apart the other 16);
//   O^T[D][32 cols]       += V^T[D][32 keys] . P^T     D/32 x 2 products;
//                            A = V rows (dim-major) from LDS, B = P^T;
//   den[32 cols]          += the same bf16 P summed per lane (vector ALU).
// The K rows are read in a permuted order (key row r holds key sigma(r),
// sigma swapping bits 2 and 3 of r) so that the score accumulator's lane
// layout is exactly the P.V product's B operand: P needs no cross-lane move.
// A step costs D/16 + D/16 = 16 (D = 128) matrix instructions per wave
// against about 90 vector instructions for its 1024 scores.
#include "split_plan.hpp"
#include "page_stream.hpp"

namespace pa {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int kTile = 32;            // columns per wave, keys per step
constexpr float kLdsSlack = 8.0f;    // base 2: P may reach 2^8 before a rescale

// LDS rows are padded by 16 bytes so that a matrix operand read (16 bytes
// per lane, 16 lanes on 16 different rows) touches every bank once.
template <int D> struct LdsTile {
  static constexpr int kRow = 2 * D + 16;      // bytes per key row of K
  static constexpr int kVRow = 2 * kTile + 16;  // bytes per dim row of V (32 keys)
  static constexpr int kK = kTile * kRow;
  static constexpr int kV = D * kVRow;
  static constexpr int kBuf = kK + kV;
  static constexpr int kStepChunks = 4 * D;    // 16-byte chunks of K (and of V) per step
};

// Threads, register-staged chunks per thread and steps in flight of a unit
// of W waves: a step's 8 KB of K and 8 KB of V (D = 128) spread over the
// unit's threads, and as many steps in flight as fit in 32 registers.
template <int D, int W> struct UnitShape {
  static constexpr int kThreads = 64 * W;
  static constexpr int kChunks = (LdsTile<D>::kStepChunks + kThreads - 1) / kThreads;
  static constexpr int kRing = 4 / kChunks < 2 ? 2 : 4 / kChunks;
};

__host__ __device__ constexpr size_t chunk_lds_kernel_bytes(int head_dim) {
  return head_dim == 128 ? 2 * LdsTile<128>::kBuf : 2 * LdsTile<64>::kBuf;
}

// Key row r of a step's K operand holds key sigma(r): bits 2 and 3 swapped.
__device__ __host__ constexpr int sigma(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Page ids of a sequence's block-table row.  A step's two ids are the same
// for every lane: they are read with scalar loads, whose completion count is
// separate from the vector loads', so waiting for them never waits for the
// page data in flight.
struct RowIds {
  const int32_t* row;
  int row_end;
  __device__ int page(int k) const {
    typedef const __attribute__((address_space(4))) int32_t* ConstPtr;
    const int i = min(k, row_end - 1);
    return ((ConstPtr)row)[i];
  }
};

// One step's K and V in registers, on their way to LDS: thread t carries
// 16-byte chunks t and t + 256 (D = 128) of the two pages' K tiles and of
// their V tiles.
template <int D, int W>
struct StepRegs {
  u32x4 k[UnitShape<D, W>::kChunks];
  u32x4 v[UnitShape<D, W>::kChunks];
  bool ok0, ok1;  // the step's two page ids are in range
};

// NT: the nontemporal hint (pages that no other unit reads).
template <int D, int W, bool NT>
__device__ inline void load_step(StepRegs<D, W>& r, const ChunkParams& p, RowIds& ids, int step,
                                 int n_pages, int kvh, int tid, int lane) {
  constexpr int CPP = 2 * D;  // 16-byte chunks per page tile (K or V)
  const int pg0 = 2 * step;
  const int id0 = ids.page(min(pg0, n_pages - 1));
  const int id1 = ids.page(min(pg0 + 1, n_pages - 1));
  r.ok0 = id0 >= 0 && id0 < p.num_pages;
  r.ok1 = pg0 + 1 < n_pages && id1 >= 0 && id1 < p.num_pages;
  const size_t tile = size_t(kPage) * D * 2;
  const char* kp = static_cast<const char*>(p.k_cache);
  const char* vp = static_cast<const char*>(p.v_cache);
  const size_t b0 = (size_t(r.ok0 ? id0 : 0) * p.num_kv_heads + kvh) * tile;
  const size_t b1 = (size_t(r.ok1 ? id1 : 0) * p.num_kv_heads + kvh) * tile;
#pragma unroll
  for (int i = 0; i < UnitShape<D, W>::kChunks; ++i) {
    const int q = min(tid + UnitShape<D, W>::kThreads * i, 2 * CPP - 1);  // chunk (page q / CPP)
    const size_t base = q < CPP ? b0 : b1;
    const uint32_t off = uint32_t(q % CPP) * 16u;
    const u32x4* ka = reinterpret_cast<const u32x4*>(kp + base + off);
    const u32x4* va = reinterpret_cast<const u32x4*>(vp + base + off);
    if constexpr (NT) {
      r.k[i] = __builtin_nontemporal_load(ka);
      r.v[i] = __builtin_nontemporal_load(va);
    } else {
      r.k[i] = *ka;
      r.v[i] = *va;
    }
  }
}

// Registers -> LDS buffer.  K chunk q: page q / CPP, key (q % CPP) / (D / 8),
// 16-byte dim chunk q % (D / 8).  V chunk q: page q / CPP, dim (q % CPP) / 2,
// keys 8 * (q % 2) .. + 7 of the page; keys at or past `limit` (the end of the
// context, or the whole page when its id is out of range) are written as
// zeros, since unwritten slots may hold NaN and 0 * NaN would reach the sums.
template <int D, int W>
__device__ inline void store_step(const StepRegs<D, W>& r, char* buf, int t0, int limit, int tid) {
  constexpr int CPP = 2 * D;
  char* kb = buf;
  char* vb = buf + LdsTile<D>::kK;
#pragma unroll
  for (int i = 0; i < UnitShape<D, W>::kChunks; ++i) {
    const int q = tid + UnitShape<D, W>::kThreads * i;
    if (q >= 2 * CPP) break;  // (W = 8, D = 64: half the threads carry a chunk)
    const int pg = q / CPP, rq = q % CPP;
    const int key = 16 * pg + rq / (D / 8);
    *reinterpret_cast<u32x4*>(kb + key * LdsTile<D>::kRow + (rq % (D / 8)) * 16) = r.k[i];
    const int dim = rq / 2;
    const int k0 = 16 * pg + 8 * (rq % 2);
    u32x4 v = r.v[i];
    if (t0 + kTile > limit || !r.ok0 || !r.ok1) {  // uniform: the last step, or a bad page
      const bool page_ok = pg == 0 ? r.ok0 : r.ok1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {  // two keys per dword
        const int ka = t0 + k0 + 2 * e;
        const uint32_t lo = (page_ok && ka < limit) ? 0x0000ffffu : 0u;
        const uint32_t hi = (page_ok && ka + 1 < limit) ? 0xffff0000u : 0u;
        v[e] &= lo | hi;
      }
    }
    *reinterpret_cast<u32x4*>(vb + dim * LdsTile<D>::kVRow + k0 * 2) = v;
  }
}

// One wave's 32 columns: online-softmax state and the query operands.
template <int D>
struct WaveCols {
  bf16x8 q[D / 16];      // B operand of k-step kk: dims 16kk + 8g .. +7 of column l % 32
  f32x16 o[D / 32];      // O^T block db: dims 32db + 8(j/4) + 4g + j%4, column l % 32
  float den;             // sum of this lane's 16 keys' bf16 P (the column's: + lane l^32)
  float m_run;           // base-2 reference score of the column (equal in lanes l, l^32)
  int pos;               // position of the column's token; keys after it are masked
};

// One 32-key step from LDS buffer `buf` for the wave's columns.  `masked`
// (uniform): the causal mask, out-of-range pages and keys past the context
// apply; otherwise every key of the step is visible to every column.  Only
// the scores branch on it, and the rescale multiplies the accumulators in
// place, so the accumulators stay in the same registers on every path (with
// a branch around their products, the register allocator copies all of them
// on every step).
template <int D>
__device__ inline void wave_step(WaveCols<D>& wc, const char* buf, int t0, bool masked, bool ok0,
                                 bool ok1, float scale_log2, int lane) {
  const int g = lane >> 5;
  const int m = lane & 31;
  const char* kb = buf + sigma(m) * LdsTile<D>::kRow + 16 * g;
  f32x16 s = {};
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(kb + 32 * kk);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, wc.q[kk], s, 0, 0, 0);
  }
  // Accumulator j holds key t0 + (j & 7) + 16 * (j >> 3) + 8g of column m.
  if (masked) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int key = t0 + (j & 7) + 16 * (j >> 3) + 8 * g;
      const bool ok = (j >> 3) ? ok1 : ok0;
      s[j] = (key > wc.pos || !ok) ? -INFINITY : s[j];
    }
  }
  // The column's keys are split over lanes l and l ^ 32, whose reference is
  // the same: some lane's own maximum passes the slack exactly when some
  // column's does, so the two halves are combined only for a rescale.
  float mx = s[0];
#pragma unroll
  for (int j = 1; j < 16; ++j) mx = fmaxf(mx, s[j]);
  const float lc = mx * scale_log2;  // -inf stays -inf (scale > 0)
  if (__ballot(lc > wc.m_run + kLdsSlack) != 0) {
    const float mc = fmaxf(lc, __shfl_xor(lc, 32));
    const float m_new = fmaxf(wc.m_run, mc);
    const float alpha = wc.m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(wc.m_run - m_new);
    wc.m_run = m_new;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j) asm("v_mul_f32 %0, %1, %0" : "+v"(wc.o[db][j]) : "v"(alpha));
    asm("v_mul_f32 %0, %1, %0" : "+v"(wc.den) : "v"(alpha));
  }
  // A column that has seen no key yet keeps reference -inf; its scores are
  // all -inf, and against reference 0 their P is exactly 0 (no inf - inf).
  const float m_ref = wc.m_run == -INFINITY ? 0.f : wc.m_run;
  // P to bf16 (nearest even) two at a time; the denominator sums the same
  // rounded values exactly (a dot product with (1, 1)), so the output stays a
  // convex combination of V rows.
  bf16x8 pb[2];
  const bf16x2_t one2 = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
  float dsum = wc.den;
#pragma unroll
  for (int kc = 0; kc < 2; ++kc)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * kc + 2 * e], scale_log2, -m_ref));
      const float p1 =
          __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * kc + 2 * e + 1], scale_log2, -m_ref));
      const bf16x2_t two = __builtin_convertvector((f32x2_t){p0, p1}, bf16x2_t);
      pb[kc][2 * e] = two[0];
      pb[kc][2 * e + 1] = two[1];
      dsum = __builtin_amdgcn_fdot2_f32_bf16(two, one2, dsum, false);
    }
  wc.den = dsum;
  const char* vb = buf + LdsTile<D>::kK + m * LdsTile<D>::kVRow + 16 * g;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(vb + 32 * db * LdsTile<D>::kVRow + 32 * kc);
      wc.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kc], wc.o[db], 0, 0, 0);
    }
}

// A unit's steps.  Step t is computed from LDS buffer t % 2 while step t + 1
// goes from registers to the other buffer and steps up to t + R - 1 are
// loading into the other register sets (set t % R takes step t + R).
template <int D, int W, bool NT>
__device__ inline void unit_steps(WaveCols<D>& wc, const ChunkParams& p, RowIds& ids, char* lds,
                                  int n_steps, int n_pages, int kvh, int L, int pos_lo, int tid,
                                  int lane) {
  constexpr int R = UnitShape<D, W>::kRing;
  char* bufs[2] = {lds, lds + LdsTile<D>::kBuf};
  // Loads are unconditional (step indices clamped to the last step): with a
  // load under a branch the compiler cannot count the loads in flight and
  // waits for all of them before the next use of any loaded register.
  StepRegs<D, W> r[R];
#pragma unroll
  for (int i = 0; i < R; ++i)
    load_step<D, W, NT>(r[i], p, ids, min(i, n_steps - 1), n_pages, kvh, tid, lane);
  store_step<D, W>(r[0], bufs[0], 0, L, tid);
  __syncthreads();
  for (int s = 0; s < n_steps; s += R) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int t = s + i;
      if (t < n_steps) {  // uniform
        const bool ok0 = r[i].ok0, ok1 = r[i].ok1;
        load_step<D, W, NT>(r[i], p, ids, min(t + R, n_steps - 1), n_pages, kvh, tid, lane);
        const int t0 = kTile * t;
        const char* buf = (i & 1) ? bufs[1] : bufs[0];
        // (A wave whose columns see none of the step computes it anyway:
        // every P is 0, and a skip would again copy the accumulators.)
        wave_step<D>(wc, buf, t0, !(t0 + kTile - 1 <= pos_lo && ok0 && ok1), ok0, ok1,
                     p.scale_log2, lane);
        if (t + 1 < n_steps)
          store_step<D, W>(r[(i + 1) % R], (i & 1) ? bufs[0] : bufs[1], t0 + kTile, L, tid);
        __syncthreads();
      }
    }
  }
}

template <int D, int W>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(2)))
void chunk_lds_kernel(ChunkParams p) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int u = blockIdx.x;
  if (u >= p.num_units) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kvh = u % p.num_kv_heads;
  const int rest = u / p.num_kv_heads;
  const int grp = rest % p.groups_per_seq;
  // Four-wave units run two per compute unit, all resident at once: the
  // single-pass decode's snake order by length balances each compute unit's
  // pair.  Eight-wave units run one per compute unit in rounds, where
  // longest first lets the dispatcher even them out.
  bool shared = true;
  const int seq = W == 4 && p.snake_period > 0
                      ? snake_unit_seq_of_batch(p, rest / p.groups_per_seq, lane, shared)
                      : longest_first_of_batch(p, rest / p.groups_per_seq, lane);
  const int G = p.group;

  const int q0 = p.query_start[seq];
  const int q_len = p.query_start[seq + 1] - q0;
  const int cols = q_len * G;
  const int c_unit = grp * W * kTile;  // first column of the unit
  // The whole workgroup leaves together; malformed offsets write nothing.
  if (q_len <= 0 || c_unit >= cols || q0 < 0 || q0 + q_len > p.num_query_tokens) return;
  const int L = min(p.context_lens[seq], p.max_pages_per_seq * kPage);
  const int unit_last = min(c_unit + W * kTile, cols) - 1;
  const int visible = max(L - q_len + unit_last / G + 1, 0);  // keys any column of the unit sees
  const int n_pages = (visible + kPage - 1) / kPage;
  const int n_steps = (visible + kTile - 1) / kTile;

  RowIds ids;
  ids.row = p.block_tables + size_t(seq) * p.max_pages_per_seq;
  ids.row_end = p.max_pages_per_seq;

  // The wave's columns and their queries.
  WaveCols<D> wc;
  const int g = lane >> 5;
  const int c = c_unit + w * kTile + (lane & 31);
  const bool real = c < cols;
  const int ti = real ? c / G : 0;
  const int hh = real ? c % G : 0;
  wc.pos = real ? L - q_len + ti : -1;
  const uint16_t* qrow = static_cast<const uint16_t*>(p.query) +
                         (size_t(q0 + ti) * p.num_q_heads + kvh * G + hh) * D;
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (real) v = *reinterpret_cast<const u32x4*>(qrow + 16 * kk + 8 * g);
    wc.q[kk] = __builtin_bit_cast(bf16x8, v);
  }
#pragma unroll
  for (int db = 0; db < D / 32; ++db) wc.o[db] = f32x16{};
  wc.den = 0.f;
  wc.m_run = -INFINITY;
  // Last key the wave's first real column sees: steps wholly at or below it
  // need no mask.  A wave with no real column (the unit's last columns past
  // the sequence's) takes the unmasked step too, as far as the context's
  // keys go: its query is zero, its scores finite, and its output dropped;
  // masking every step would make it the slowest wave at each barrier.
  const int w_first = c_unit + w * kTile;
  const int pos_lo = w_first < cols ? L - q_len + w_first / G : L - 1;

  // A unit whose column group is its sequence's only one, and whose first
  // page no other sequence starts with, is the only reader of its pages: a
  // four-wave unit (two per compute unit) streams them with the nontemporal
  // hint.  (Eight-wave units measured no faster with it, and fetched 2.6%
  // more.)  Two instantiations of the step loop, so that no load sits under
  // a branch.
  const bool nt = W == 4 && p.groups_per_seq == 1 && !shared;
  if (n_steps > 0) {
    if (nt)
      unit_steps<D, W, true>(wc, p, ids, lds, n_steps, n_pages, kvh, L, pos_lo, tid, lane);
    else
      unit_steps<D, W, false>(wc, p, ids, lds, n_steps, n_pages, kvh, L, pos_lo, tid, lane);
  }

  // out = O / den for the wave's real columns.  Lane l holds column l % 32,
  // dims 32db + 8(j/4) + 4g + j%4 (four consecutive dims per j / 4).
  const float l_sum = wc.den + __shfl_xor(wc.den, 32);
  if (real) {
    const float inv = l_sum > 0.f ? 1.0f / l_sum : 0.f;
    uint16_t* orow = static_cast<uint16_t*>(p.out) +
                     (size_t(q0 + ti) * p.num_q_heads + kvh * G + hh) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        uint32_t pk[2];
#pragma unroll
        for (int e = 0; e < 2; ++e)
          pk[e] = uint32_t(f32_to_bf16(wc.o[db][4 * a + 2 * e] * inv)) |
                  (uint32_t(f32_to_bf16(wc.o[db][4 * a + 2 * e + 1] * inv)) << 16);
        *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * a + 4 * g) = (u32x2){pk[0], pk[1]};
      }
  }
}

}  // namespace

// Units of `waves` (4 or 8) waves of 32 columns each.
hipError_t launch_chunk_lds(const ChunkParams& p, int head_dim, int waves, hipStream_t stream) {
  const dim3 grid(p.num_units);
  const size_t lds = chunk_lds_kernel_bytes(head_dim);
  if (head_dim == 128) {
    if (waves == 8) chunk_lds_kernel<128, 8><<<grid, 512, lds, stream>>>(p);
    else chunk_lds_kernel<128, 4><<<grid, 256, lds, stream>>>(p);
  } else {
    if (waves == 8) chunk_lds_kernel<64, 8><<<grid, 512, lds, stream>>>(p);
    else chunk_lds_kernel<64, 4><<<grid, 256, lds, stream>>>(p);
  }
  return hipGetLastError();
}

}  // namespace pa
