// The C ABI of libpa.so: host-side argument checks, then kernel launches on
// the caller's stream.  Every check runs before the first HIP call, so a
// rejected call touches no device state.
#include <limits.h>
#include <math.h>

#include <atomic>
#include <mutex>

#include "pa.h"
#include "pa_device.hpp"

namespace pa {
hipError_t launch_decode_mfma(const DecodeParams& p, int head_dim, hipStream_t stream);
hipError_t launch_decode_valu(const DecodeParams& p, int head_dim, bool bf16, hipStream_t stream);
hipError_t launch_reshape_and_cache(const void* key, const void* value, void* k_cache,
                                    void* v_cache, const int64_t* slots, int64_t num_tokens,
                                    int num_kv_heads, int head_dim, int64_t num_pages, bool bf16,
                                    hipStream_t stream);
hipError_t launch_chunk_attention(const ChunkParams& p, int head_dim, hipStream_t stream);
hipError_t launch_chunk_lds(const ChunkParams& p, int head_dim, int waves, hipStream_t stream);
hipError_t launch_cascade(const PrefixParams& q, const DecodeParams& p, int head_dim,
                          hipStream_t stream);
hipError_t launch_page_copy(bool export_dir, void* buf, void* k_cache, void* v_cache,
                            const int32_t* page_ids, int64_t num_ids, int64_t num_pages,
                            int64_t block_bytes, hipStream_t stream);
hipError_t launch_decode_reduce(void* out, const float* part_out, const float* part_max,
                                const float* part_sum, const int32_t* context_lens, int num_seqs,
                                int num_q_heads, int head_dim, int partition_size, int max_parts,
                                bool bf16, hipStream_t stream);
hipError_t launch_chunk_reduce(void* out, const float* part_out, const float* part_max,
                               const float* part_sum, const int32_t* context_lens,
                               const int32_t* query_start, int num_seqs, int max_query_len,
                               int num_query_tokens, int num_q_heads, int head_dim,
                               int partition_size, int max_parts, int max_pages_per_seq,
                               hipStream_t stream);
}  // namespace pa

namespace {

constexpr int kVersion = 10000;  // 1.0.0

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_common(int head_dim, int page_size, int dtype) {
  if (dtype != PA_DTYPE_F32 && dtype != PA_DTYPE_BF16) return PA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (page_size != PA_PAGE_SIZE) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

enum class DecodeKernel { kAuto, kValu };

// Multi-token single pass: the LDS-staged kernel (units of four or eight
// 32-column waves) takes batches with more than 64 (new token, head)
// columns per kv head, units of eight waves past 128 columns; at 64 columns
// and below the 16-column-block kernel is faster (measured on the
// Llama-3-8B-shaped batch: 16 new tokens 142 against 167 us, 32 tokens 171
// against 156, 64 tokens 282 against 199).
constexpr int64_t kLdsMinColumns = 65;
constexpr int64_t kLdsEightWaveFrom = 1;  // units of 8 waves past 128 * this columns

// Compute units of the current device, looked up once per device (0 when
// unknown): the single-pass decode's unit order pairs sequences per compute
// unit.
constexpr int kMaxDevicesCached = 64;
std::atomic<int> g_device_cus[kMaxDevicesCached];

int device_compute_units() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevicesCached) return 0;
  int n = g_device_cus[dev].load(std::memory_order_relaxed);
  if (n == 0 &&
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      n > 0)
    g_device_cus[dev].store(n, std::memory_order_relaxed);
  return n > 0 ? n : 0;
}

// Checks a decode call's host arguments and fills its launch parameters;
// *empty when there is nothing to launch.  new_key == NULL: decode only.
// Otherwise the launch first writes each sequence's new token (new_key /
// new_value rows, slot new_slots[b]): inside the matrix-core kernels (*fused),
// or as a separate cache-write launch for the others.
int decode_setup(DecodeKernel which, void* out, const void* query, const void* k_cache,
                 const void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                 int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                 int max_pages_per_seq, int64_t num_pages, float scale, int partition_size,
                 int max_num_partitions, float* partial_out, float* partial_max,
                 float* partial_sum, int dtype, const void* new_key, const void* new_value,
                 const int64_t* new_slots, const int32_t* first_partition, bool four_wave_units,
                 int grid_partitions, pa::DecodeParams& p, bool& mfma, bool& empty) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_pages_per_seq <= 0 ||
      num_pages <= 0 || partition_size < 0)
    return PA_ERR_INVALID_ARGUMENT;
  if (int s = check_common(head_dim, page_size, dtype)) return s;
  if (num_q_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARGUMENT;
  const int group = num_q_heads / num_kv_heads;
  if (group > PA_MAX_GQA_GROUP) return PA_ERR_UNSUPPORTED;
  if (!query || !k_cache || !v_cache || !block_tables || !context_lens)
    return PA_ERR_INVALID_ARGUMENT;
  if (!aligned16(query) || !aligned16(k_cache) || !aligned16(v_cache))
    return PA_ERR_INVALID_ARGUMENT;
  if (!isfinite(scale)) return PA_ERR_INVALID_ARGUMENT;
  if (new_key && (!new_value || !new_slots || !aligned16(new_key))) return PA_ERR_INVALID_ARGUMENT;
  const bool split = partition_size > 0;
  if (split) {
    if (partition_size % PA_PAGE_SIZE != 0 || max_num_partitions < 1) return PA_ERR_INVALID_ARGUMENT;
    if (!partial_out || !partial_max || !partial_sum || !aligned16(partial_out))
      return PA_ERR_INVALID_ARGUMENT;
  } else if (!out) {
    return PA_ERR_INVALID_ARGUMENT;
  }
  const int64_t parts = split ? max_num_partitions : 1;
  // Partitions per (sequence, kv head) in the unit grid: all of them, or for
  // the shared-prefix step's four-wave units a bound on those from each
  // sequence's first_partition on.
  const int64_t grid_parts =
      split && four_wave_units && first_partition && grid_partitions > 0
          ? (grid_partitions < parts ? grid_partitions : parts)
          : parts;
  const int64_t units = int64_t(num_seqs) * num_kv_heads * grid_parts;
  if (units > INT_MAX / 2) return PA_ERR_UNSUPPORTED;
  empty = num_seqs == 0;

  p.out = out;
  p.query = query;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.partial_out = partial_out;
  p.partial_max = partial_max;
  p.partial_sum = partial_sum;
  p.num_seqs = num_seqs;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = group;
  p.max_pages_per_seq = max_pages_per_seq;
  p.num_pages = num_pages;
  p.scale_log2 = scale * pa::kLog2e;
  p.pages_per_partition = split ? partition_size / PA_PAGE_SIZE : 0;
  p.num_partitions = int(parts);
  p.grid_partitions = int(grid_parts);
  p.num_units = int(units);
  p.first_partition = first_partition;
  p.four_wave_units = four_wave_units && split;
  p.snake_period = 0;
  mfma = dtype == PA_DTYPE_BF16 && which == DecodeKernel::kAuto;
  p.new_key = mfma ? new_key : nullptr;
  p.new_value = mfma ? new_value : nullptr;
  p.new_slots = mfma ? new_slots : nullptr;
  return PA_OK;
}

int decode_impl(DecodeKernel which, void* out, const void* query, const void* k_cache,
                const void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                int max_pages_per_seq, int64_t num_pages, float scale, int partition_size,
                int max_num_partitions, float* partial_out, float* partial_max,
                float* partial_sum, int dtype, void* stream, const void* new_key = nullptr,
                const void* new_value = nullptr, const int64_t* new_slots = nullptr) {
  pa::DecodeParams p;
  bool mfma = false, empty = false;
  if (int st = decode_setup(which, out, query, k_cache, v_cache, block_tables, context_lens,
                            num_seqs, num_q_heads, num_kv_heads, head_dim, page_size,
                            max_pages_per_seq, num_pages, scale, partition_size,
                            max_num_partitions, partial_out, partial_max, partial_sum, dtype,
                            new_key, new_value, new_slots, nullptr, false, 0, p, mfma, empty))
    return st;
  if (empty) return PA_OK;
  if (partition_size == 0) {
    // The single pass takes its units in the snake order by length.  The
    // vector kernel does so only when its units outnumber the compute units:
    // below that the order changes nothing and its length loads cost a round
    // trip (tiny fp32 batch: 17.4 -> 19.9 us).
    const int cus = device_compute_units();
    if (mfma || int64_t(num_seqs) * num_kv_heads > cus)
      p.snake_period = cus > 0 ? (cus / num_kv_heads > 0 ? cus / num_kv_heads : 1) : 0;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf16 = dtype == PA_DTYPE_BF16;
  if (new_key && !mfma) {
    const hipError_t e = pa::launch_reshape_and_cache(new_key, new_value, const_cast<void*>(k_cache),
                                                      const_cast<void*>(v_cache), new_slots,
                                                      num_seqs, num_kv_heads, head_dim, num_pages,
                                                      bf16, s);
    if (e != hipSuccess) return PA_ERR_LAUNCH;
  }
  const hipError_t err = mfma ? pa::launch_decode_mfma(p, head_dim, s)
                              : pa::launch_decode_valu(p, head_dim, bf16, s);
  return err == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int page_copy_impl(bool export_dir, void* buffer, int64_t buffer_bytes, void* k_cache,
                   void* v_cache, const int32_t* page_ids, int64_t num_ids, int num_kv_heads,
                   int head_dim, int page_size, int64_t num_pages, int dtype, void* stream) {
  if (num_ids < 0 || buffer_bytes < 0 || num_kv_heads <= 0 || num_pages <= 0)
    return PA_ERR_INVALID_ARGUMENT;
  if (int s = check_common(head_dim, page_size, dtype)) return s;
  if (num_ids > INT_MAX / 2) return PA_ERR_UNSUPPORTED;  // two workgroups per page
  const int64_t esz = dtype == PA_DTYPE_BF16 ? 2 : 4;
  const int64_t block_bytes = int64_t(num_kv_heads) * page_size * head_dim * esz;
  if (num_ids > 0 && buffer_bytes / 2 / num_ids < block_bytes) return PA_ERR_INVALID_ARGUMENT;
  if (num_ids == 0) return PA_OK;  // an empty list examines no pointer
  if (!buffer || !k_cache || !v_cache || !page_ids) return PA_ERR_INVALID_ARGUMENT;
  if (!aligned16(buffer) || !aligned16(k_cache) || !aligned16(v_cache))
    return PA_ERR_INVALID_ARGUMENT;
  const hipError_t err = pa::launch_page_copy(export_dir, buffer, k_cache, v_cache, page_ids,
                                              num_ids, num_pages, block_bytes,
                                              static_cast<hipStream_t>(stream));
  return err == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

// ------------------------------------------------------------------ scratch
// Split partials of pa_chunk_attention_split_noalloc: one fixed array per
// GPU, held until the process ends, so that call allocates nothing.  In host
// code `scratch` names a host-side stand-in; its device address comes from
// hipGetSymbolAddress, taken once per device (with that device current) and
// kept per device.
constexpr int64_t kScratchBytes = int64_t(PA_SCRATCH_BYTES);
static __device__ __align__(256) unsigned char scratch[PA_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];

int scratch_of_current_device(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PA_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return PA_ERR_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return PA_OK;
}

// Multi-token attention, single pass (partition_size 0) or split-KV with the
// merge in the same call; with use_scratch the split partials live in this
// device's scratch array instead of the caller's buffers.
int chunk_impl(void* out, const void* query, const void* k_cache, const void* v_cache,
               const int32_t* block_tables, const int32_t* context_lens,
               const int32_t* query_start, int num_seqs, int num_query_tokens, int max_query_len,
               int num_q_heads, int num_kv_heads, int head_dim, int page_size,
               int max_pages_per_seq, int64_t num_pages, float scale, int partition_size,
               int max_num_partitions, float* partial_out, float* partial_max,
               float* partial_sum, int dtype, void* stream, bool use_scratch = false) {
  if (num_seqs < 0 || num_query_tokens < 0 || max_query_len < 0 || num_q_heads <= 0 ||
      num_kv_heads <= 0 || max_pages_per_seq <= 0 || num_pages <= 0)
    return PA_ERR_INVALID_ARGUMENT;
  if (int s = check_common(head_dim, page_size, dtype)) return s;
  if (dtype != PA_DTYPE_BF16) return PA_ERR_UNSUPPORTED;  // matrix-core kernel only
  if (num_q_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARGUMENT;
  const int group = num_q_heads / num_kv_heads;
  if (group > PA_MAX_GQA_GROUP) return PA_ERR_UNSUPPORTED;
  if (!out || !query || !k_cache || !v_cache || !block_tables || !context_lens || !query_start)
    return PA_ERR_INVALID_ARGUMENT;
  if (!aligned16(query) || !aligned16(k_cache) || !aligned16(v_cache))
    return PA_ERR_INVALID_ARGUMENT;
  if (!isfinite(scale)) return PA_ERR_INVALID_ARGUMENT;
  if (max_query_len > num_query_tokens) return PA_ERR_INVALID_ARGUMENT;
  const bool split = partition_size > 0;
  if (split) {
    if (partition_size % PA_PAGE_SIZE != 0 || max_num_partitions < 1) return PA_ERR_INVALID_ARGUMENT;
    if (!use_scratch && (!partial_out || !partial_max || !partial_sum || !aligned16(partial_out)))
      return PA_ERR_INVALID_ARGUMENT;
  }
  // Scratch layout: partial_out [T][Hq][P][D], then partial_max and
  // partial_sum [T][Hq][P] (every part a multiple of 16 bytes from the start).
  const int64_t scratch_rows = int64_t(num_query_tokens) * num_q_heads * max_num_partitions;
  if (use_scratch && scratch_rows * (head_dim + 2) * int64_t(sizeof(float)) > kScratchBytes)
    return PA_ERR_SCRATCH_LIMIT;
  const int64_t blocks = (int64_t(max_query_len) * group + 15) / 16;
  const int64_t per_wave = blocks < 4 ? (blocks > 0 ? blocks : 1) : 4;
  // Single pass with at least kLdsMinColumns (new token, head) columns per
  // kv head: the LDS-staged kernel, units of 128 columns; otherwise units of
  // per_wave 16-column blocks.
  const int64_t max_cols = int64_t(max_query_len) * group;
  const bool lds = !split && max_cols >= kLdsMinColumns;
  const int lds_waves = max_cols > 4 * 32 * kLdsEightWaveFrom ? 8 : 4;
  const int64_t groups = lds ? (max_cols + 32 * lds_waves - 1) / (32 * lds_waves)
                             : (blocks + per_wave - 1) / per_wave;
  const int64_t units =
      int64_t(num_seqs) * num_kv_heads * groups * (split ? max_num_partitions : 1);
  if (units > INT_MAX / 2) return PA_ERR_UNSUPPORTED;
  if (int64_t(num_query_tokens) * num_q_heads * (split ? max_num_partitions : 1) > INT_MAX ||
      int64_t(num_seqs) * max_query_len * num_q_heads > INT_MAX)
    return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0 || num_query_tokens == 0 || max_query_len == 0) return PA_OK;
  if (use_scratch) {
    void* base = nullptr;
    if (int st = scratch_of_current_device(&base)) return st;
    partial_out = static_cast<float*>(base);
    partial_max = partial_out + scratch_rows * head_dim;
    partial_sum = partial_max + scratch_rows;
  }

  pa::ChunkParams p;
  p.out = out;
  p.query = query;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.query_start = query_start;
  p.num_seqs = num_seqs;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = group;
  p.max_pages_per_seq = max_pages_per_seq;
  p.num_pages = num_pages;
  p.scale_log2 = scale * pa::kLog2e;
  p.num_query_tokens = num_query_tokens;
  p.blocks_per_wave = int(per_wave);
  p.groups_per_seq = int(groups);
  p.num_units = int(units);
  p.pages_per_partition = split ? partition_size / PA_PAGE_SIZE : 0;
  p.num_partitions = split ? max_num_partitions : 1;
  p.partial_out = partial_out;
  p.partial_max = partial_max;
  p.partial_sum = partial_sum;
  p.first_partition = nullptr;
  // Single pass: units per round over the compute units, for the snake
  // order (the register kernel and four-wave LDS units).
  p.snake_period = 0;
  if (!split && (!lds || lds_waves == 4)) {
    const int cus = device_compute_units();
    const int64_t per_round = int64_t(num_kv_heads) * groups;
    p.snake_period = cus > 0 ? int(cus / per_round > 0 ? cus / per_round : 1) : 0;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  if ((lds ? pa::launch_chunk_lds(p, head_dim, lds_waves, st)
           : pa::launch_chunk_attention(p, head_dim, st)) !=
      hipSuccess)
    return PA_ERR_LAUNCH;
  if (split && pa::launch_chunk_reduce(out, partial_out, partial_max, partial_sum, context_lens,
                                       query_start, num_seqs, max_query_len, num_query_tokens,
                                       num_q_heads, head_dim, partition_size, max_num_partitions,
                                       max_pages_per_seq, st) != hipSuccess)
    return PA_ERR_LAUNCH;
  return PA_OK;
}

}  // namespace

extern "C" {

int pa_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                         const int64_t* slot_mapping, int64_t num_tokens, int num_kv_heads,
                         int head_dim, int page_size, int64_t num_pages, int dtype,
                         void* stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || num_pages <= 0) return PA_ERR_INVALID_ARGUMENT;
  if (int s = check_common(head_dim, page_size, dtype)) return s;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping) return PA_ERR_INVALID_ARGUMENT;
  if (!aligned16(key) || !aligned16(k_cache)) return PA_ERR_INVALID_ARGUMENT;
  if (num_tokens > INT_MAX) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  const hipError_t err = pa::launch_reshape_and_cache(
      key, value, k_cache, v_cache, slot_mapping, num_tokens, num_kv_heads, head_dim, num_pages,
      dtype == PA_DTYPE_BF16, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int pa_decode(void* out, const void* query, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
              int num_q_heads, int num_kv_heads, int head_dim, int page_size,
              int max_pages_per_seq, int64_t num_pages, float scale, int partition_size,
              int max_num_partitions, float* partial_out, float* partial_max,
              float* partial_sum, int dtype, void* stream) {
  return decode_impl(DecodeKernel::kAuto, out, query, k_cache, v_cache, block_tables,
                     context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, page_size,
                     max_pages_per_seq, num_pages, scale, partition_size, max_num_partitions,
                     partial_out, partial_max, partial_sum, dtype, stream);
}

int pa_decode_append(void* out, const void* query, const void* key, const void* value,
                     const int64_t* slot_mapping, void* k_cache, void* v_cache,
                     const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                     int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                     int max_pages_per_seq, int64_t num_pages, float scale, int partition_size,
                     int max_num_partitions, float* partial_out, float* partial_max,
                     float* partial_sum, int dtype, void* stream) {
  if (!key) return PA_ERR_INVALID_ARGUMENT;
  return decode_impl(DecodeKernel::kAuto, out, query, k_cache, v_cache, block_tables,
                     context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, page_size,
                     max_pages_per_seq, num_pages, scale, partition_size, max_num_partitions,
                     partial_out, partial_max, partial_sum, dtype, stream, key, value,
                     slot_mapping);
}

int pa_decode_cascade(const void* query, const void* key, const void* value,
                      const int64_t* slot_mapping, void* k_cache, void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                      int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                      int max_pages_per_seq, int64_t num_pages, float scale, int partition_size,
                      int max_num_partitions, float* partial_out, float* partial_max,
                      float* partial_sum, int num_groups, int max_group_size,
                      int max_group_partitions, int max_suffix_partitions,
                      const int32_t* group_start,
                      const int32_t* group_seqs, const int32_t* group_partitions,
                      const int32_t* seq_first_partition, int dtype, void* stream) {
  if (partition_size <= 0 || num_groups < 0 || max_group_size < 0 || max_group_partitions < 0 ||
      max_suffix_partitions < 0)
    return PA_ERR_INVALID_ARGUMENT;
  if (dtype != PA_DTYPE_BF16) return PA_ERR_UNSUPPORTED;  // matrix-core kernels only
  if (num_groups > 0 && (!group_start || !group_seqs || !group_partitions ||
                         !seq_first_partition || max_group_partitions > max_num_partitions))
    return PA_ERR_INVALID_ARGUMENT;
  if ((key != nullptr) != (value != nullptr) || (key != nullptr) != (slot_mapping != nullptr))
    return PA_ERR_INVALID_ARGUMENT;
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return PA_ERR_INVALID_ARGUMENT;
  pa::DecodeParams p;
  bool mfma = false, empty = false;
  if (int st = decode_setup(DecodeKernel::kAuto, nullptr, query, k_cache, v_cache, block_tables,
                            context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                            page_size, max_pages_per_seq, num_pages, scale, partition_size,
                            max_num_partitions, partial_out, partial_max, partial_sum, dtype, key,
                            value, slot_mapping, num_groups > 0 ? seq_first_partition : nullptr,
                            /*four_wave_units=*/num_groups > 0, max_suffix_partitions, p, mfma,
                            empty))
    return st;
  const int group = num_q_heads / num_kv_heads;
  // At most two 16-column blocks per wave (202 VGPRs, two waves per SIMD):
  // measured faster here than four blocks at one wave per SIMD, and than
  // one block (146 VGPRs, three waves per SIMD).
  const int64_t blocks = (int64_t(max_group_size) * group + 15) / 16;
  const int64_t per_wave = blocks < 2 ? (blocks > 0 ? blocks : 1) : 2;
  const int64_t col_groups = (blocks + per_wave - 1) / per_wave;
  const int64_t prefix_units =
      int64_t(num_groups) * max_group_partitions * col_groups * num_kv_heads;
  if (prefix_units > INT_MAX / 2 || prefix_units + p.num_units > INT_MAX / 2)
    return PA_ERR_UNSUPPORTED;
  if (empty) return PA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (prefix_units == 0)
    return pa::launch_decode_mfma(p, head_dim, s) == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
  pa::PrefixParams q;
  q.query = query;
  q.k_cache = k_cache;
  q.v_cache = v_cache;
  q.block_tables = block_tables;
  q.partial_out = partial_out;
  q.partial_max = partial_max;
  q.partial_sum = partial_sum;
  q.group_start = group_start;
  q.group_seqs = group_seqs;
  q.group_partitions = group_partitions;
  q.num_groups = num_groups;
  q.num_seqs = num_seqs;
  q.num_q_heads = num_q_heads;
  q.num_kv_heads = num_kv_heads;
  q.group = group;
  q.max_pages_per_seq = max_pages_per_seq;
  q.num_pages = num_pages;
  q.scale_log2 = scale * pa::kLog2e;
  q.pages_per_partition = partition_size / PA_PAGE_SIZE;
  q.num_partitions = max_num_partitions;
  q.max_group_partitions = max_group_partitions;
  q.blocks_per_wave = int(per_wave);
  q.column_groups = int(col_groups);
  q.num_units = int(prefix_units);
  return pa::launch_cascade(q, p, head_dim, s) == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int pa_chunk_attention(void* out, const void* query, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, const int32_t* context_lens,
                       const int32_t* query_start, int num_seqs, int num_query_tokens,
                       int max_query_len, int num_q_heads, int num_kv_heads, int head_dim,
                       int page_size, int max_pages_per_seq, int64_t num_pages, float scale,
                       int dtype, void* stream) {
  return chunk_impl(out, query, k_cache, v_cache, block_tables, context_lens, query_start,
                    num_seqs, num_query_tokens, max_query_len, num_q_heads, num_kv_heads,
                    head_dim, page_size, max_pages_per_seq, num_pages, scale, 0, 0, nullptr,
                    nullptr, nullptr, dtype, stream);
}

int pa_chunk_attention_split(void* out, const void* query, const void* k_cache,
                             const void* v_cache, const int32_t* block_tables,
                             const int32_t* context_lens, const int32_t* query_start,
                             int num_seqs, int num_query_tokens, int max_query_len,
                             int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                             int max_pages_per_seq, int64_t num_pages, float scale,
                             int partition_size, int max_num_partitions, float* partial_out,
                             float* partial_max, float* partial_sum, int dtype, void* stream) {
  if (partition_size <= 0) return PA_ERR_INVALID_ARGUMENT;
  return chunk_impl(out, query, k_cache, v_cache, block_tables, context_lens, query_start,
                    num_seqs, num_query_tokens, max_query_len, num_q_heads, num_kv_heads,
                    head_dim, page_size, max_pages_per_seq, num_pages, scale, partition_size,
                    max_num_partitions, partial_out, partial_max, partial_sum, dtype, stream);
}

int pa_chunk_attention_split_noalloc(void* out, const void* query, const void* k_cache,
                                     const void* v_cache, const int32_t* block_tables,
                                     const int32_t* context_lens, const int32_t* query_start,
                                     int num_seqs, int num_query_tokens, int max_query_len,
                                     int num_q_heads, int num_kv_heads, int head_dim,
                                     int page_size, int max_pages_per_seq, int64_t num_pages,
                                     float scale, int partition_size, int max_num_partitions,
                                     int dtype, void* stream) {
  if (partition_size <= 0) return PA_ERR_INVALID_ARGUMENT;
  return chunk_impl(out, query, k_cache, v_cache, block_tables, context_lens, query_start,
                    num_seqs, num_query_tokens, max_query_len, num_q_heads, num_kv_heads,
                    head_dim, page_size, max_pages_per_seq, num_pages, scale, partition_size,
                    max_num_partitions, nullptr, nullptr, nullptr, dtype, stream,
                    /*use_scratch=*/true);
}

int pa_export_pages(void* buffer, int64_t buffer_bytes, const void* k_cache, const void* v_cache,
                    const int32_t* page_ids, int64_t num_ids, int num_kv_heads, int head_dim,
                    int page_size, int64_t num_pages, int dtype, void* stream) {
  return page_copy_impl(true, buffer, buffer_bytes, const_cast<void*>(k_cache),
                        const_cast<void*>(v_cache), page_ids, num_ids, num_kv_heads, head_dim,
                        page_size, num_pages, dtype, stream);
}

int pa_import_pages(const void* buffer, int64_t buffer_bytes, void* k_cache, void* v_cache,
                    const int32_t* page_ids, int64_t num_ids, int num_kv_heads, int head_dim,
                    int page_size, int64_t num_pages, int dtype, void* stream) {
  return page_copy_impl(false, const_cast<void*>(buffer), buffer_bytes, k_cache, v_cache,
                        page_ids, num_ids, num_kv_heads, head_dim, page_size, num_pages, dtype,
                        stream);
}

int pa_decode_valu(void* out, const void* query, const void* k_cache, const void* v_cache,
                   const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                   int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                   int max_pages_per_seq, int64_t num_pages, float scale, int partition_size,
                   int max_num_partitions, float* partial_out, float* partial_max,
                   float* partial_sum, int dtype, void* stream) {
  return decode_impl(DecodeKernel::kValu, out, query, k_cache, v_cache, block_tables,
                     context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, page_size,
                     max_pages_per_seq, num_pages, scale, partition_size, max_num_partitions,
                     partial_out, partial_max, partial_sum, dtype, stream);
}

int pa_decode_reduce(void* out, const float* partial_out, const float* partial_max,
                     const float* partial_sum, const int32_t* context_lens, int num_seqs,
                     int num_q_heads, int head_dim, int partition_size, int max_num_partitions,
                     int dtype, void* stream) {
  if (num_seqs < 0 || num_q_heads <= 0 || partition_size <= 0 || max_num_partitions < 1)
    return PA_ERR_INVALID_ARGUMENT;
  if (int s = check_common(head_dim, PA_PAGE_SIZE, dtype)) return s;
  if (partition_size % PA_PAGE_SIZE != 0) return PA_ERR_INVALID_ARGUMENT;
  if (!out || !partial_out || !partial_max || !partial_sum || !context_lens)
    return PA_ERR_INVALID_ARGUMENT;
  if (int64_t(num_seqs) * num_q_heads > INT_MAX) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PA_OK;
  const hipError_t err = pa::launch_decode_reduce(
      out, partial_out, partial_max, partial_sum, context_lens, num_seqs, num_q_heads, head_dim,
      partition_size, max_num_partitions, dtype == PA_DTYPE_BF16,
      static_cast<hipStream_t>(stream));
  return err == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID_ARGUMENT: return "PA_ERR_INVALID_ARGUMENT";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
    case PA_ERR_LAUNCH: return "PA_ERR_LAUNCH";
    case PA_ERR_SCRATCH_LIMIT: return "PA_ERR_SCRATCH_LIMIT";
    default: return "PA_ERR_UNKNOWN";
  }
}

int pa_version(void) { return kVersion; }

}  // extern "C"
