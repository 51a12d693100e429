// Paged decode on the vector ALU: fp32 and bf16, head_dim 64/128, groups up
// to 16.  Same work units, page walk and merge as the matrix-core kernel;
// only the per-page arithmetic differs.
//
// Per page and kv head, lane (t, c) = (lane / 4, lane % 4) holds token t's
// key slice [c*D/4, (c+1)*D/4) and forms partial dots against the query
// group (kept in LDS as fp32); two xor-shuffles finish each score.  The page
// maximum per head is a four-step xor-shuffle over the tokens.  For P.V, lane
// d owns output dims d and d+64 and reads those dims' 16 value slots (the V
// page is stored dim-major, so that is one contiguous row per dim); each
// token's weight is broadcast from its owner lane with readlane.
#include "pa_device.hpp"

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T> struct Load;
template <> struct Load<float> {
  // n floats (n % 4 == 0) from 16-byte aligned global memory
  template <int n> __device__ static void run(const void* src, float* dst) {
    const u32x4* s = static_cast<const u32x4*>(src);
#pragma unroll
    for (int i = 0; i < n / 4; ++i) {
      const u32x4 v = s[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[4 * i + e] = __uint_as_float(v[e]);
    }
  }
};
template <> struct Load<uint16_t> {
  // n bf16 values (n % 8 == 0), widened exactly
  template <int n> __device__ static void run(const void* src, float* dst) {
    const u32x4* s = static_cast<const u32x4*>(src);
#pragma unroll
    for (int i = 0; i < n / 8; ++i) {
      const u32x4 v = s[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dst[8 * i + 2 * e] = __uint_as_float(v[e] << 16);
        dst[8 * i + 2 * e + 1] = __uint_as_float(v[e] & 0xffff0000u);
      }
    }
  }
};

template <typename T>
__device__ inline float load_one(const void* base, size_t i) {
  if constexpr (sizeof(T) == 4) return static_cast<const float*>(base)[i];
  else return bf16_to_f32(static_cast<const uint16_t*>(base)[i]);
}

template <typename T, int D>
__global__ __launch_bounds__(kBlock) void decode_valu_kernel(DecodeParams p) {
  extern __shared__ float smem[];
  constexpr int QD = D / 4;    // key dims per lane
  constexpr int VD = D / 64;   // value dims per lane
  int seq, kvh, part;
  if (!unit_of(p, blockIdx.x, seq, kvh, part)) return;
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
  float* qs = smem + merge_lds_bytes(G, D) / sizeof(float);  // [G][D] fp32

  for (int idx = threadIdx.x; idx < G * D; idx += kBlock)
    qs[idx] = load_one<T>(p.query, (size_t(seq) * p.num_q_heads + kvh * G) * D + idx);
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t = lane >> 2;
  const int c = lane & 3;
  const int32_t* table = p.block_tables + size_t(seq) * p.max_pages_per_seq;
  const size_t tile_elems = size_t(kPage) * D;

  float m_run[kMaxGroup], l_run[kMaxGroup], acc[kMaxGroup][VD];
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
#pragma unroll
    for (int i = 0; i < VD; ++i) acc[h][i] = 0.f;
  }

  for (int i = lo + w; i < hi; i += kWaves) {
    const int page = table[i];
    if (page < 0 || page >= p.num_pages) continue;
    const size_t base = (size_t(page) * p.num_kv_heads + kvh) * tile_elems;
    const int valid = L - i * kPage;
    float kv[QD];
    Load<T>::template run<QD>(static_cast<const T*>(p.k_cache) + base + t * D + c * QD, kv);
    float vv[VD][kPage];
#pragma unroll
    for (int vi = 0; vi < VD; ++vi) {
      Load<T>::template run<kPage>(static_cast<const T*>(p.v_cache) + base + (lane + 64 * vi) * kPage,
                                   vv[vi]);
      if (valid < kPage) {
#pragma unroll
        for (int tt = 0; tt < kPage; ++tt)
          if (tt >= valid) vv[vi][tt] = 0.f;  // unwritten slots may hold NaN
      }
    }
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) {
      if (h >= G) break;
      const float* qh = qs + h * D + c * QD;
      float part_dot = 0.f;
#pragma unroll
      for (int e = 0; e < QD; ++e) part_dot = fmaf(qh[e], kv[e], part_dot);
      part_dot += __shfl_xor(part_dot, 1);
      part_dot += __shfl_xor(part_dot, 2);
      const float s2 = (t < valid) ? part_dot * p.scale_log2 : -INFINITY;
      float pm = s2;
      pm = fmaxf(pm, __shfl_xor(pm, 4));
      pm = fmaxf(pm, __shfl_xor(pm, 8));
      pm = fmaxf(pm, __shfl_xor(pm, 16));
      pm = fmaxf(pm, __shfl_xor(pm, 32));
      const float m_new = fmaxf(m_run[h], pm);
      const float alpha = __builtin_amdgcn_exp2f(m_run[h] - m_new);
      m_run[h] = m_new;
      const float pe = __builtin_amdgcn_exp2f(s2 - m_new);
      l_run[h] = l_run[h] * alpha + (c == 0 ? pe : 0.f);
#pragma unroll
      for (int vi = 0; vi < VD; ++vi) acc[h][vi] *= alpha;
#pragma unroll
      for (int tt = 0; tt < kPage; ++tt) {
        const float wt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pe), 4 * tt));
#pragma unroll
        for (int vi = 0; vi < VD; ++vi) acc[h][vi] = fmaf(wt, vv[vi][tt], acc[h][vi]);
      }
    }
  }

#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) {
    if (h >= G) break;
    float l = l_run[h];
#pragma unroll
    for (int x = 1; x < 64; x <<= 1) l += __shfl_xor(l, x);
    if (lane == 0) {
      lds.m[w * kMaxGroup + h] = m_run[h];
      lds.l[w * kMaxGroup + h] = l;
    }
#pragma unroll
    for (int vi = 0; vi < VD; ++vi) lds.acc[(w * G + h) * (D + kAccPad) + lane + 64 * vi] = acc[h][vi];
  }
  merge_and_store<T, D>(p, lds, seq, kvh, part);
}

template <typename T>
hipError_t launch_t(const DecodeParams& p, int head_dim, hipStream_t stream) {
  const dim3 grid(decode_grid(p.num_units));
  const size_t lds = merge_lds_bytes(p.group, head_dim) + sizeof(float) * p.group * head_dim;
  if (head_dim == 128)
    decode_valu_kernel<T, 128><<<grid, kBlock, lds, stream>>>(p);
  else
    decode_valu_kernel<T, 64><<<grid, kBlock, lds, stream>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_valu(const DecodeParams& p, int head_dim, bool bf16, hipStream_t stream) {
  return bf16 ? launch_t<uint16_t>(p, head_dim, stream) : launch_t<float>(p, head_dim, stream);
}

}  // namespace pa
