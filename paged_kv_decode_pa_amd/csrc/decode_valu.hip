// Paged decode on the vector ALU: fp32 and bf16, head_dim 64/128, groups up
// to 16.  Same work units and merge as the matrix-core kernel (four waves per
// unit, wave w taking every fourth page); each wave keeps two pages in flight.
//
// Per page and kv head, lane (t, c) = (lane / 4, lane % 4) holds token t's
// key slice [c*D/4, (c+1)*D/4) and forms partial dots against the query
// group (kept in LDS: fp32, or the bf16 pairs as stored, which bf16 keys
// take two at a time with v_dot2); a quad butterfly (DPP) finishes each
// score.
// The page maximum per head comes from DPP mirrors and gfx950's lane-swap
// instructions, without an LDS round trip.  For P.V, lane d owns output dims
// d and d+64 and reads those dims' 16 value slots (the V page is stored
// dim-major, so that is one contiguous row per dim); each token's weight is
// broadcast from its owner lane with readlane.  For bf16 pools P is rounded
// to bf16 and two tokens go into one v_dot2 with their value words as loaded
// (the denominator sums the same rounded P); fp32 pools keep fp32 P.
#include "split_plan.hpp"

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// One page's K slice and V rows of a lane, as loaded (bf16 or fp32 bits).
template <typename T, int D>
struct RawPage {
  static constexpr int KQ = D / 4 * sizeof(T) / 16;      // 16-byte loads of the key slice
  static constexpr int VQ = kPage * sizeof(T) / 16;      // 16-byte loads per value row
  u32x4 k[KQ];
  u32x4 v[D / 64][VQ];
};

// n fp32 values from their loaded words.
template <int n>
__device__ inline void words_to_f32(const u32x4* src, float* dst) {
#pragma unroll
  for (int i = 0; i < n / 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[4 * i + e] = __uint_as_float(src[i][e]);
}

// The sum over a lane quad (a token's four key slices), in the order of two
// xor-butterflies: lanes 1,0,3,2 then 2,3,0,1 of each quad (DPP).
__device__ inline float quad_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
  return x;
}

// The maximum over the wave's 16 tokens of a value that is equal within each
// quad: mirrors inside 8 and 16 lanes (DPP), then the row and half swaps of
// gfx950 (v_permlane16_swap, v_permlane32_swap).  No LDS round trip.
__device__ inline float token_max(float m) {
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x141, 0xF, 0xF,
                                                          false)));  // row_half_mirror
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x140, 0xF, 0xF,
                                                          false)));  // row_mirror
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false,
                                                  false);
  m = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false,
                                                  false);
  return fmaxf(__uint_as_float(h[0]), __uint_as_float(h[1]));
}

// GB: a bound on the group (1, 2, 4, 8 or 16), so that the per-head state
// is indexed by unrolled constants only.
// NC > 0 (split-KV, batches the unit plan covers): unit b is the b-th
// entry of the split decode's unit list (longest units first, none past a
// context's end); otherwise the plain grid of (sequence, partition, kv head).
template <typename T, int D, int GB, int NC>
__global__ __launch_bounds__(kBlock) void decode_valu_kernel(DecodeParams p) {
  extern __shared__ float smem[];
  constexpr int QD = D / 4;    // key dims per lane
  constexpr int VD = D / 64;   // value dims per lane
  typedef RawPage<T, D> Raw;
  int seq, kvh, part;
  if constexpr (NC > 0) {
    const int u = blockIdx.x;
    if (u >= p.num_units) return;
    kvh = u % p.num_kv_heads;
    int seq_pages = 0;
    if (!split_unit<NC>(p, u / p.num_kv_heads, threadIdx.x & 63, seq, part, seq_pages)) return;
    seq = __builtin_amdgcn_readfirstlane(seq);
    part = __builtin_amdgcn_readfirstlane(part);
  } else {
    if (!unit_of(p, blockIdx.x, seq, kvh, part)) return;
  }
  // Single pass: the snake order by length of the matrix-core single pass
  // (when the host asks for it).  Loads stay cached: a lane reads 16-byte
  // pieces of several rows, so one 128-byte line serves several of a wave's
  // loads (the nontemporal hint measured 14% slower here).
  bool shared = true;
  if (NC == 0 && p.pages_per_partition == 0 && p.snake_period > 0)
    seq = snake_unit_seq_of_batch(p, seq, threadIdx.x & 63, shared);
  const int L = p.context_lens[seq];
  int lo, hi;
  if (!unit_pages(p, seq, part, L, lo, hi)) {
    if (p.pages_per_partition == 0)
      store_zeros<T, D>(p, seq, kvh);
    else if (part < merged_partitions(p, L))  // past a length clamped to the table
      empty_partials<D>(p, seq, kvh, part, part + 1, threadIdx.x, kBlock);
    return;
  }
  const int G = p.group;
  MergeLds lds(smem);
  float* qs = smem + merge_lds_bytes(G, D) / sizeof(float);  // [G][D] fp32 (bf16: pairs)

  if constexpr (sizeof(T) == 4) {
    for (int idx = threadIdx.x; idx < G * D; idx += kBlock)
      qs[idx] = static_cast<const float*>(p.query)[(size_t(seq) * p.num_q_heads + kvh * G) * D + idx];
  } else {  // bf16 pairs, as stored
    const uint32_t* qg = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p.query) +
                                                         (size_t(seq) * p.num_q_heads + kvh * G) * D);
    for (int idx = threadIdx.x; idx < G * D / 2; idx += kBlock)
      reinterpret_cast<uint32_t*>(qs)[idx] = qg[idx];
  }
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t = lane >> 2;
  const int c = lane & 3;
  const int32_t* table = p.block_tables + size_t(seq) * p.max_pages_per_seq;
  const size_t tile_elems = size_t(kPage) * D;
  const int n_my = w < hi - lo ? (hi - lo - w + kWaves - 1) / kWaves : 0;  // this wave's pages

  float m_run[GB], l_run[GB], acc[GB][VD];
#pragma unroll
  for (int h = 0; h < GB; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
#pragma unroll
    for (int i = 0; i < VD; ++i) acc[h][i] = 0.f;
  }

  // The wave's k-th page (clamped to its last): loads issued unconditionally,
  // so that the compiler counts the loads in flight exactly; an out-of-range
  // id loads page 0 and the page is skipped.
  auto issue = [&](Raw& r, int k, int& ord, bool& ok) {
    const int kk = min(k, n_my - 1);
    ord = lo + w + kk * kWaves;
    const int page = table[ord];
    ok = k < n_my && page >= 0 && page < p.num_pages;
    const size_t base = (size_t(ok ? page : 0) * p.num_kv_heads + kvh) * tile_elems;
    const u32x4* ks = reinterpret_cast<const u32x4*>(static_cast<const T*>(p.k_cache) + base +
                                                     t * D + c * QD);
#pragma unroll
    for (int i = 0; i < Raw::KQ; ++i) r.k[i] = ks[i];
#pragma unroll
    for (int vi = 0; vi < VD; ++vi) {
      const u32x4* vs = reinterpret_cast<const u32x4*>(static_cast<const T*>(p.v_cache) + base +
                                                       (lane + 64 * vi) * kPage);
#pragma unroll
      for (int i = 0; i < Raw::VQ; ++i) r.v[vi][i] = vs[i];
    }
  };

  auto compute = [&](const Raw& r, int ord) {
    const int valid = L - ord * kPage;
    float kv[sizeof(T) == 4 ? QD : 1];
    if constexpr (sizeof(T) == 4) words_to_f32<QD>(r.k, kv);
    // fp32: the value rows widened; bf16: kept as words of two tokens.
    float vv[VD][sizeof(T) == 4 ? kPage : 1];
    uint32_t vw[VD][sizeof(T) == 4 ? 1 : kPage / 2];
#pragma unroll
    for (int vi = 0; vi < VD; ++vi) {
      if constexpr (sizeof(T) == 4) {
        words_to_f32<kPage>(r.v[vi], vv[vi]);
        if (valid < kPage) {
#pragma unroll
          for (int tt = 0; tt < kPage; ++tt)
            if (tt >= valid) vv[vi][tt] = 0.f;  // unwritten slots may hold NaN
        }
      } else {
#pragma unroll
        for (int w2 = 0; w2 < kPage / 2; ++w2) {
          const uint32_t x = r.v[vi][w2 / 4][w2 % 4];
          vw[vi][w2] = x;
        }
        if (valid < kPage) {
#pragma unroll
          for (int w2 = 0; w2 < kPage / 2; ++w2)
            vw[vi][w2] &= (2 * w2 < valid ? 0x0000ffffu : 0u) | (2 * w2 + 1 < valid ? 0xffff0000u : 0u);
        }
      }
    }
#pragma unroll
    for (int h = 0; h < GB; ++h) {
      if (h < G) {  // uniform
        float part_dot = 0.f;
        if constexpr (sizeof(T) == 4) {
          const float* qh = qs + h * D + c * QD;
#pragma unroll
          for (int e = 0; e < QD; ++e) part_dot = fmaf(qh[e], kv[e], part_dot);
        } else {
          // bf16 keys and query: two products per instruction (v_dot2), no
          // widening.  The words go through plain variables: a bit_cast of
          // the vector element itself compiled to element 0 for every f.
          const uint32_t* qh = reinterpret_cast<const uint32_t*>(qs) + h * (D / 2) + c * (QD / 2);
#pragma unroll
          for (int e = 0; e < QD / 8; ++e)
#pragma unroll
            for (int f = 0; f < 4; ++f)
            {
              const uint32_t kw = r.k[e][f];
              const uint32_t qw = qh[4 * e + f];
              part_dot = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, kw),
                                                         __builtin_bit_cast(bf16x2_t, qw), part_dot,
                                                         false);
            }
        }
        const float s2 = (t < valid) ? quad_sum(part_dot) * p.scale_log2 : -INFINITY;
        const float m_new = fmaxf(m_run[h], token_max(s2));
        const float alpha = __builtin_amdgcn_exp2f(m_run[h] - m_new);
        m_run[h] = m_new;
        const float pe = __builtin_amdgcn_exp2f(s2 - m_new);
#pragma unroll
        for (int vi = 0; vi < VD; ++vi) acc[h][vi] *= alpha;
        if constexpr (sizeof(T) == 4) {
          l_run[h] = l_run[h] * alpha + (c == 0 ? pe : 0.f);
#pragma unroll
          for (int tt = 0; tt < kPage; ++tt) {
            const float wt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pe), 4 * tt));
#pragma unroll
            for (int vi = 0; vi < VD; ++vi) acc[h][vi] = fmaf(wt, vv[vi][tt], acc[h][vi]);
          }
        } else {
          // bf16 V: P rounded to bf16 (nearest even), two tokens per v_dot2;
          // the denominator sums the same rounded P.
          const uint32_t pb = f32_to_bf16(pe);
          l_run[h] = l_run[h] * alpha + (c == 0 ? __uint_as_float(pb << 16) : 0.f);
#pragma unroll
          for (int w2 = 0; w2 < kPage / 2; ++w2) {
            const uint32_t lo = uint32_t(__builtin_amdgcn_readlane(int(pb), 8 * w2));
            const uint32_t hi = uint32_t(__builtin_amdgcn_readlane(int(pb), 8 * w2 + 4));
            const uint32_t pw = lo | (hi << 16);
#pragma unroll
            for (int vi = 0; vi < VD; ++vi) {
              const uint32_t x = vw[vi][w2];
              acc[h][vi] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x),
                                                           __builtin_bit_cast(bf16x2_t, pw),
                                                           acc[h][vi], false);
            }
          }
        }
      }
    }
  };

  // Two pages in flight: page k + 1 loads while page k is computed.
  if (n_my > 0) {
    Raw r0, r1;
    int o0, o1;
    bool ok0, ok1;
    issue(r0, 0, o0, ok0);
    for (int k = 0; k < n_my; k += 2) {
      issue(r1, k + 1, o1, ok1);
      if (ok0) compute(r0, o0);
      issue(r0, k + 2, o0, ok0);
      if (ok1) compute(r1, o1);
    }
  }

#pragma unroll
  for (int h = 0; h < GB; ++h) {
    if (h < G) {
      float l = l_run[h];
#pragma unroll
      for (int x = 1; x < 64; x <<= 1) l += __shfl_xor(l, x);
      if (lane == 0) {
        lds.m[w * kMaxGroup + h] = m_run[h];
        lds.l[w * kMaxGroup + h] = l;
      }
#pragma unroll
      for (int vi = 0; vi < VD; ++vi)
        lds.acc[(w * G + h) * (D + kAccPad) + lane + 64 * vi] = acc[h][vi];
    }
  }
  merge_and_store<T, D>(p, lds, seq, kvh, part);
  // The plan has no units past a length clamped to the block table's width:
  // the unit of the last partition with tokens writes the empty partials of
  // the partitions after it that the merge counts.
  if constexpr (NC > 0) {
    const int n = min((L + kPage - 1) / kPage, p.max_pages_per_seq);
    if (hi == n) empty_partials<D>(p, seq, kvh, part + 1, merged_partitions(p, L), threadIdx.x, kBlock);
  }
}

template <typename T, int D, int NC>
void launch_g(const DecodeParams& p, const dim3& grid, size_t lds, hipStream_t stream) {
  if (p.group <= 1)
    decode_valu_kernel<T, D, 1, NC><<<grid, kBlock, lds, stream>>>(p);
  else if (p.group <= 2)
    decode_valu_kernel<T, D, 2, NC><<<grid, kBlock, lds, stream>>>(p);
  else if (p.group <= 4)
    decode_valu_kernel<T, D, 4, NC><<<grid, kBlock, lds, stream>>>(p);
  else if (p.group <= 8)
    decode_valu_kernel<T, D, 8, NC><<<grid, kBlock, lds, stream>>>(p);
  else
    decode_valu_kernel<T, D, 16, NC><<<grid, kBlock, lds, stream>>>(p);
}

template <typename T>
hipError_t launch_t(const DecodeParams& p, int head_dim, hipStream_t stream) {
  const dim3 grid(decode_grid(p.num_units));
  const size_t lds = merge_lds_bytes(p.group, head_dim) + sizeof(float) * p.group * head_dim;
  // The split decode's unit list, when it covers the batch and no other
  // launch computes some partitions (a shared prefix's).
  const bool plan = p.pages_per_partition > 0 && p.first_partition == nullptr &&
                    plan_chunks_for(p.num_seqs) > 0;
  if (head_dim == 128) {
    if (plan) launch_g<T, 128, kPlanChunks>(p, grid, lds, stream);
    else launch_g<T, 128, 0>(p, grid, lds, stream);
  } else {
    if (plan) launch_g<T, 64, kPlanChunks>(p, grid, lds, stream);
    else launch_g<T, 64, 0>(p, grid, lds, stream);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_valu(const DecodeParams& p, int head_dim, bool bf16, hipStream_t stream) {
  return bf16 ? launch_t<uint16_t>(p, head_dim, stream) : launch_t<float>(p, head_dim, stream);
}

}  // namespace pa
