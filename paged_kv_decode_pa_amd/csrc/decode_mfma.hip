// bf16 paged decode on the matrix cores (gfx950).
//
// Work unit: one (sequence, kv head, partition).  A workgroup of four waves
// takes one unit; wave w walks pages lo+w, lo+w+4, ... with its own online
// softmax, and the four states are merged through LDS at the end.
//
// Per 16-token page and kv head, with the grouped query heads as the 16
// columns of a matrix tile (groups of 4 or 8 are zero-padded to 16):
//   S^T[16 tok][16 heads]  = K[16 tok][D] . Q^T[D][16 heads]
//                            D/32 x v_mfma_f32_16x16x32_bf16; A = the K page
//                            tile straight from HBM (each lane a 16-byte
//                            row chunk), B = the query group, loaded once.
//   online softmax on the S^T accumulator (lane = head r, tokens 4j..4j+3)
//   O^T[D][16 heads]      += V^T[D][16 tok] . P^T[16 tok][16 heads]
//                            D/16 x v_mfma_f32_16x16x16_bf16; A = the V page
//                            tile (stored dim-major, each lane an 8-byte
//                            chunk of 4 tokens), B = P^T, which is exactly
//                            the S^T accumulator's lane layout rounded to bf16.
// The matrix cores turn a page's 2*G*D*16 multiply-adds into 3*D/32 issue
// slots, so the vector ALU only runs the softmax and the loads dominate.
#include "pa_device.hpp"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int D>
struct PageTile {
  bf16x8 k[D / 32];  // K[token r][32kb + 8j .. +8]
  s16x4 v[D / 16];   // V^T[16db + r][4j .. 4j+3]
};

template <int D>
__device__ inline void load_tile(PageTile<D>& t, const uint16_t* kt, const uint16_t* vt, int r,
                                 int j) {
#pragma unroll
  for (int kb = 0; kb < D / 32; ++kb)
    t.k[kb] = __builtin_bit_cast(bf16x8,
                                 *reinterpret_cast<const u32x4*>(kt + r * D + 32 * kb + 8 * j));
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
    t.v[db] = __builtin_bit_cast(s16x4,
                                 *reinterpret_cast<const u32x2*>(vt + (16 * db + r) * kPage + 4 * j));
}

template <int D>
__global__ __launch_bounds__(kBlock) void decode_mfma_kernel(DecodeParams p) {
  extern __shared__ float smem[];
  int seq, kvh, part;
  if (!unit_of_block(p, seq, kvh, part)) return;
  const int L = p.context_lens[seq];
  int lo, hi;
  if (!unit_pages(p, seq, part, L, lo, hi)) {
    if (p.pages_per_partition == 0) store_zeros<uint16_t, D>(p, seq, kvh);
    return;
  }

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15;
  const int j = lane >> 4;
  const int G = p.group;

  // Query group as the B operand: column r = query head kvh*G + r.
  bf16x8 qop[D / 32];
  {
    const uint16_t* qrow =
        static_cast<const uint16_t*>(p.query) + (size_t(seq) * p.num_q_heads + kvh * G + r) * D;
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (r < G) v = *reinterpret_cast<const u32x4*>(qrow + 32 * kb + 8 * j);
      qop[kb] = __builtin_bit_cast(bf16x8, v);
    }
  }

  const uint16_t* kpool = static_cast<const uint16_t*>(p.k_cache);
  const uint16_t* vpool = static_cast<const uint16_t*>(p.v_cache);
  const int32_t* table = p.block_tables + size_t(seq) * p.max_pages_per_seq;
  const size_t tile_elems = size_t(kPage) * D;

  float m_run = -INFINITY;  // base-2 running max for head r
  float l_run = 0.f;        // this lane's share of the softmax denominator
  f32x4 acc[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Page ids of this wave's pages, 64 at a time: lane k holds page lo+w+4k.
  int ids = -1;
  auto fetch_ids = [&](int first) {
    const int i = first + 4 * lane;
    ids = (i < hi) ? table[i] : -1;
  };
  auto page_at = [&](int k) { return __builtin_amdgcn_readlane(ids, k & 63); };
  auto tile_ptrs = [&](int page, const uint16_t*& kt, const uint16_t*& vt) {
    const bool ok = page >= 0 && page < p.num_pages;
    const size_t base = (size_t(ok ? page : 0) * p.num_kv_heads + kvh) * tile_elems;
    kt = kpool + base;
    vt = vpool + base;
    return ok;
  };

  const int first = lo + w;
  const int count = first < hi ? (hi - first + 3) / 4 : 0;
  PageTile<D> cur;
  bool cur_ok = false;
  if (count > 0) {
    fetch_ids(first);
    const uint16_t *kt, *vt;
    cur_ok = tile_ptrs(page_at(0), kt, vt);
    load_tile<D>(cur, kt, vt, r, j);
  }
  for (int k = 0; k < count; ++k) {
    // Issue the next page's loads before working on this one.
    PageTile<D> nxt;
    bool nxt_ok = false;
    if (k + 1 < count) {
      if (((k + 1) & 63) == 0) fetch_ids(first + 4 * (k + 1));
      const uint16_t *kt, *vt;
      nxt_ok = tile_ptrs(page_at(k + 1), kt, vt);
      load_tile<D>(nxt, kt, vt, r, j);
    }
    if (cur_ok) {
      const int i = first + 4 * k;        // logical page index
      const int valid = L - i * kPage;    // tokens of this page inside the context
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb)
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.k[kb], qop[kb], s, 0, 0, 0);
      float s2[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) s2[e] = s[e] * p.scale_log2;
      if (valid < kPage) {  // the context's last, partly filled page
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * j + e >= valid) s2[e] = -INFINITY;
#pragma unroll
        for (int db = 0; db < D / 16; ++db)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (4 * j + e >= valid) cur.v[db][e] = 0;  // unwritten slots may hold NaN
      }
      float pm = fmaxf(fmaxf(s2[0], s2[1]), fmaxf(s2[2], s2[3]));
      pm = fmaxf(pm, __shfl_xor(pm, 16));
      pm = fmaxf(pm, __shfl_xor(pm, 32));
      const float m_new = fmaxf(m_run, pm);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      s16x4 pb;
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint16_t b16 = f32_to_bf16(__builtin_amdgcn_exp2f(s2[e] - m_new));
        pb[e] = static_cast<short>(b16);
        psum += bf16_to_f32(b16);
      }
      l_run = l_run * alpha + psum;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        acc[db] *= alpha;
        acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(cur.v[db], pb, acc[db], 0, 0, 0);
      }
    }
    cur = nxt;
    cur_ok = nxt_ok;
  }

  // Per-head denominator: sum the four lane groups' shares.
  float l_head = l_run + __shfl_xor(l_run, 16);
  l_head = l_head + __shfl_xor(l_head, 32);

  MergeLds lds(smem);
  if (r < G) {
    if (j == 0) {
      lds.m[w * kMaxGroup + r] = m_run;
      lds.l[w * kMaxGroup + r] = l_head;
    }
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e) lds.acc[(w * G + r) * D + 16 * db + 4 * j + e] = acc[db][e];
  }
  merge_and_store<uint16_t, D>(p, lds, seq, kvh, part);
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeParams& p, int head_dim, hipStream_t stream) {
  const dim3 grid(decode_grid(p.num_units));
  const size_t lds = merge_lds_bytes(p.group, head_dim);
  if (head_dim == 128)
    decode_mfma_kernel<128><<<grid, kBlock, lds, stream>>>(p);
  else
    decode_mfma_kernel<64><<<grid, kBlock, lds, stream>>>(p);
  return hipGetLastError();
}

}  // namespace pa
