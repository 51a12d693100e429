// Streaming of paged K/V tiles into matrix-core operand registers, shared by
// the decode and multi-token kernels.  A (page, kv head) tile of 16 tokens is
// read straight from HBM into the MFMA A-operand layouts:
//   K[16 tok][D]  token r's 16-byte row chunks, lane (r, j) holding dims
//                 32kb + 8j .. +8 for kb < D/32 (v_mfma_f32_16x16x32_bf16);
//   V^T[D][16 tok] from the dim-major V page, lane (r, j) holding tokens
//                 4j .. 4j+3 of dims 16db + r for db < D/16
//                 (v_mfma_f32_16x16x16_bf16).
#pragma once

#include "pa_device.hpp"

namespace pa {

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

// Page tiles are read with global loads from a wave-uniform tile base plus
// a fixed 32-bit per-lane offset.  (Buffer-descriptor loads were measured 6-7%
// slower on the long-context and prefix-reuse workloads.)  With Stream set the
// loads carry the nontemporal hint: a page that no other sequence reads is
// used once, and keeping it out of the caches' normal replacement measured
// 8-9% faster on unshared batches.  Pages that several sequences read are
// loaded normally so that the other readers hit in L2.
template <bool Stream, typename V>
__device__ inline V load_vec(const char* ptr) {
  if constexpr (Stream)
    return __builtin_nontemporal_load(reinterpret_cast<const V*>(ptr));
  else
    return *reinterpret_cast<const V*>(ptr);
}

template <int D, bool Stream>
__device__ inline void load_tile(PageTile<D>& t, const char* kt, const char* vt, uint32_t koff,
                                 uint32_t voff) {
#pragma unroll
  for (int kb = 0; kb < D / 32; ++kb)
    t.k[kb] = __builtin_bit_cast(bf16x8, load_vec<Stream, u32x4>(kt + koff + 64 * kb));
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
    t.v[db] = __builtin_bit_cast(s16x4, load_vec<Stream, u32x2>(vt + voff + 32 * kPage * db));
}

// The pages one wave walks: logical pages first, first+step, ... (count of
// them).  Their ids are fetched 64 at a time into a vector register (lane i
// = the wave's i-th page) 64 to 128 pages ahead of use.  A tile load never
// depends on the data: the ordinal is clamped to the stream, and an invalid
// page id loads page 0's tile (which always exists) and reports the tile as
// not to be used.
template <int D>
struct PageStream {
  const int32_t* table;
  int first, step, row_end, count;
  int ids_cur, ids_nxt, chunk;
  const char* kpool;
  const char* vpool;
  int64_t num_pages;
  int num_kv_heads, kvh;
  uint32_t koff, voff;

  __device__ int fetch(int c, int lane) const {
    const int i = first + step * (64 * c + lane);
    return i < row_end ? table[i] : -1;
  }
  // Request the first 128 page ids (before the context length is known).
  __device__ void start(int lane) {
    ids_cur = fetch(0, lane);
    ids_nxt = fetch(1, lane);
    chunk = 0;
  }
  template <bool Stream>
  __device__ bool issue(PageTile<D>& t, int k, int lane) {
    const int kk = min(k, count - 1);
    if ((kk >> 6) != chunk) {
      chunk = kk >> 6;
      ids_cur = ids_nxt;
      ids_nxt = fetch(chunk + 1, lane);
    }
    const int page = __builtin_amdgcn_readlane(ids_cur, kk & 63);
    const bool ok = page >= 0 && page < num_pages;
    constexpr size_t tile_bytes = size_t(kPage) * D * 2;
    const size_t base = (size_t(ok ? page : 0) * num_kv_heads + kvh) * tile_bytes;
    // The per-lane offsets pass through an empty asm in place, so each load
    // is formed as the scalar tile base plus a 32-bit vector offset.
    // (Otherwise the offsets are folded into 64-bit vector addresses whose
    // temporaries reuse registers of loads still in flight and force full
    // memory waits.)
    asm volatile("" : "+v"(koff), "+v"(voff));
    load_tile<D, Stream>(t, kpool + base, vpool + base, koff, voff);
    return ok && k < count;
  }
};

}  // namespace pa
