// C ABI of the paged-KV library: host-side argument validation, kernel
// choice and launch on the caller's stream. Every check runs before any HIP
// call, so invalid calls enqueue nothing and are testable without a GPU.
#include <hip/hip_runtime.h>

#include "../../include/pagedkv.h"
#include "launch.h"

namespace {

int elem_bytes(int dtype) {
  switch (dtype) {
    case PKV_F32: return 4;
    case PKV_F16: return 2;
    case PKV_BF16: return 2;
    default: return 0;
  }
}

constexpr int kMaxGridYZ = 65535;

int launch_status(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// Checks shared by the whole-block moves; 0 when the geometry is valid.
int move_checks(void* const* k_caches, void* const* v_caches, int num_layers, int64_t n,
                int64_t num_blocks, int num_kv_heads, int block_size, int head_size,
                int dtype, int64_t* slab_bytes) {
  const int eb = elem_bytes(dtype);
  if (eb == 0) return PKV_ERR_DTYPE;
  if (num_layers < 0 || n < 0 || num_blocks < 1 || num_kv_heads < 1 || block_size < 1 ||
      head_size < 1)
    return PKV_ERR_SHAPE;
  if (num_layers == 0 || n == 0) return PKV_OK;
  if (!k_caches || !v_caches) return PKV_ERR_NULL;
  for (int l = 0; l < num_layers; ++l)
    if (!k_caches[l] || !v_caches[l]) return PKV_ERR_NULL;
  // one 256-lane workgroup per slab: the grid's x extent in lanes stays
  // below 2^32
  if (n >= (int64_t{1} << 24)) return PKV_ERR_UNSUPPORTED;
  *slab_bytes = static_cast<int64_t>(num_kv_heads) * block_size * head_size * eb;
  return PKV_OK;
}

// The device-visible address of a pinned host buffer, or nullptr. Pinned
// host memory on this platform is reached at its host address; anything
// else (pageable memory, device memory, another mapping) is refused.
void* pinned_device_address(const void* host) {
  hipPointerAttribute_t attr{};
  if (hipPointerGetAttributes(&attr, host) != hipSuccess) {
    (void)hipGetLastError();  // a failed query must not surface as a launch error
    return nullptr;
  }
  if (attr.type != hipMemoryTypeHost) return nullptr;
  if (attr.devicePointer != host && attr.devicePointer != attr.hostPointer) return nullptr;
  return const_cast<void*>(host);
}

int swap_common(void* host, int64_t host_bytes, void* const* k_caches, void* const* v_caches,
                int num_layers, const int64_t* block_ids, int64_t num_ids, int64_t num_blocks,
                int num_kv_heads, int block_size, int head_size, int dtype, bool out,
                void* stream) {
  int64_t slab = 0;
  const int rc = move_checks(k_caches, v_caches, num_layers, num_ids, num_blocks, num_kv_heads,
                             block_size, head_size, dtype, &slab);
  if (rc != PKV_OK || num_layers == 0 || num_ids == 0) return rc;
  if (!host || !block_ids) return PKV_ERR_NULL;
  if (host_bytes / slab / 2 / num_layers < num_ids) return PKV_ERR_HOST;  // too small
  void* dev = pinned_device_address(host);
  if (!dev) return PKV_ERR_HOST;
  pkv::MoveArgs m{k_caches, v_caches, num_layers, dev, block_ids, num_ids, num_blocks, slab};
  return launch_status(pkv::launch_swap(m, out, as_stream(stream)));
}

// paged_varlen_attention's argument checks (all before any HIP call); fills
// `a` except the workspace. Returns kLaunch when there is work to launch,
// else the status to return (PKV_OK for an empty call).
constexpr int kLaunch = 1;

// paged_decode_attention's argument checks (all before any HIP call); fills
// `a`. Returns kLaunch when there is work to launch, else the status.
int decode_args(pkv::DecodeArgs& a, float* out, const void* query, const void* k_cache,
                const void* v_cache, const int32_t* block_table, const int32_t* context_lens,
                int num_seqs, int num_heads, int num_kv_heads, int head_size, int block_size,
                int64_t num_blocks, int max_blocks_per_seq, float scale, int partition_size,
                int max_partitions, float* max_logits, float* exp_sums, float* tmp_out,
                int dtype) {
  if (elem_bytes(dtype) == 0) return PKV_ERR_DTYPE;
  if (num_seqs < 0 || num_heads < 1 || num_kv_heads < 1 || head_size < 1 || block_size < 1 ||
      num_blocks < 1 || max_blocks_per_seq < 1 || partition_size < 0)
    return PKV_ERR_SHAPE;
  if (num_heads % num_kv_heads != 0) return PKV_ERR_SHAPE;
  const bool split = partition_size > 0;
  if (split && (partition_size % block_size != 0 || max_partitions < 1)) return PKV_ERR_SHAPE;
  if (static_cast<int64_t>(max_blocks_per_seq) * block_size > 0x7fffffff) return PKV_ERR_SHAPE;
  if (head_size > 256) return PKV_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PKV_OK;
  if (!query || !k_cache || !v_cache || !block_table || !context_lens) return PKV_ERR_NULL;
  if (!split && !out) return PKV_ERR_NULL;
  if (split && (!max_logits || !exp_sums || !tmp_out)) return PKV_ERR_WORKSPACE;
  a.out = out;
  a.query = query;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_table = block_table;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_size = head_size;
  a.block_size = block_size;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.scale = scale;
  a.partition_size = partition_size;
  a.max_partitions = split ? max_partitions : 1;
  a.max_logits = max_logits;
  a.exp_sums = exp_sums;
  a.tmp_out = tmp_out;
  a.dtype = dtype;
  return kLaunch;
}

int varlen_args(pkv::DecodeArgs& a, float* out, const void* query, const void* k_cache,
                const void* v_cache, const int32_t* block_table,
                const int32_t* query_start_loc, const int32_t* context_lens, int num_seqs,
                int num_tokens, int num_heads, int num_kv_heads, int head_size, int block_size,
                int64_t num_blocks, int max_blocks_per_seq, float scale, int max_partitions,
                int dtype) {
  if (elem_bytes(dtype) == 0) return PKV_ERR_DTYPE;
  if (num_seqs < 0 || num_tokens < 0 || num_heads < 1 || num_kv_heads < 1 || head_size < 1 ||
      block_size < 1 || num_blocks < 1 || max_blocks_per_seq < 1 || max_partitions < 1)
    return PKV_ERR_SHAPE;
  if (num_heads % num_kv_heads != 0) return PKV_ERR_SHAPE;
  if (static_cast<int64_t>(max_blocks_per_seq) * block_size > 0x7fffffff) return PKV_ERR_SHAPE;
  if (head_size > 256) return PKV_ERR_UNSUPPORTED;
  if (num_seqs == 0 || num_tokens == 0) return PKV_OK;
  if (!out || !query || !k_cache || !v_cache || !block_table || !query_start_loc ||
      !context_lens)
    return PKV_ERR_NULL;
  // one 64-lane wave per (row, head) on the plain path and in the merge
  const int64_t rows = static_cast<int64_t>(num_tokens) * num_heads;
  if (rows * 64 > 0xffffffffLL) return PKV_ERR_UNSUPPORTED;
  a.out = out;
  a.query = query;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_table = block_table;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_size = head_size;
  a.block_size = block_size;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.scale = scale;
  a.partition_size = 0;
  a.max_partitions = max_partitions;
  a.dtype = dtype;
  a.query_start_loc = query_start_loc;
  a.num_tokens = num_tokens;
  return kLaunch;
}

int varlen_launch(const pkv::DecodeArgs& a, hipStream_t stream) {
  if (!pkv::fast_varlen_supported(a)) return launch_status(pkv::launch_varlen_generic(a, stream));
  // sequences with short query sets, then those with long chunks (each
  // kernel takes its own kind), then the merge of all query rows
  hipError_t e = pkv::launch_varlen_fast(a, stream);
  if (e == hipSuccess) e = pkv::launch_prefill_fast(a, stream);
  if (e != hipSuccess) return PKV_ERR_LAUNCH;
  return launch_status(pkv::launch_reduce(a.out, a.max_logits, a.exp_sums, a.tmp_out, nullptr,
                                          a.num_tokens, a.num_heads, a.head_size, 1,
                                          a.max_partitions, stream));
}

// Bytes of one part of the static scratch, rounded up to 256 (each part
// starts 256-byte aligned).
size_t scratch_part(size_t floats) { return (floats * sizeof(float) + 255) & ~size_t(255); }

}  // namespace

extern "C" {

int paged_slot_mapping(int64_t* slot_mapping, const int32_t* block_table,
                       const int32_t* positions, int num_seqs, int max_blocks_per_seq,
                       int block_size, void* stream) {
  if (num_seqs < 0 || max_blocks_per_seq < 1 || block_size < 1) return PKV_ERR_SHAPE;
  if (num_seqs == 0) return PKV_OK;
  if (!slot_mapping || !block_table || !positions) return PKV_ERR_NULL;
  return launch_status(pkv::launch_slot_mapping(slot_mapping, block_table, positions, num_seqs,
                                                max_blocks_per_seq, block_size,
                                                as_stream(stream)));
}

int paged_kv_write(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                   const int64_t* slot_mapping, int64_t num_tokens, int64_t num_blocks,
                   int num_kv_heads, int block_size, int head_size, int dtype, void* stream) {
  const int eb = elem_bytes(dtype);
  if (eb == 0) return PKV_ERR_DTYPE;
  if (num_tokens < 0 || num_blocks < 1 || num_kv_heads < 1 || block_size < 1 || head_size < 1)
    return PKV_ERR_SHAPE;
  if (num_tokens == 0) return PKV_OK;
  if (!k_cache || !v_cache || !k_new || !v_new || !slot_mapping) return PKV_ERR_NULL;
  // the grid is one thread per 2-byte chunk at worst
  const int64_t chunks = num_tokens * num_kv_heads * (static_cast<int64_t>(head_size) * eb / 2);
  if (chunks / 256 >= 0x7fffffff) return PKV_ERR_UNSUPPORTED;
  return launch_status(pkv::launch_kv_write(k_cache, v_cache, k_new, v_new, slot_mapping,
                                            num_tokens, num_blocks, num_kv_heads, block_size,
                                            head_size, eb, as_stream(stream)));
}

int paged_decode_attention(float* out, const void* query, const void* k_cache,
                           const void* v_cache, const int32_t* block_table,
                           const int32_t* context_lens, int num_seqs, int num_heads,
                           int num_kv_heads, int head_size, int block_size, int64_t num_blocks,
                           int max_blocks_per_seq, float scale, int partition_size,
                           int max_partitions, float* max_logits, float* exp_sums,
                           float* tmp_out, int dtype, void* stream) {
  pkv::DecodeArgs a{};
  const int rc = decode_args(a, out, query, k_cache, v_cache, block_table, context_lens,
                             num_seqs, num_heads, num_kv_heads, head_size, block_size,
                             num_blocks, max_blocks_per_seq, scale, partition_size,
                             max_partitions, max_logits, exp_sums, tmp_out, dtype);
  if (rc != kLaunch) return rc;
  if (pkv::fast_decode_supported(a))
    return launch_status(pkv::launch_decode_fast(a, as_stream(stream)));
  if (num_seqs > kMaxGridYZ || num_heads > kMaxGridYZ) return PKV_ERR_UNSUPPORTED;
  return launch_status(pkv::launch_decode_generic(a, as_stream(stream)));
}

int paged_decode_attention_merged(float* out, const void* query, const void* k_cache,
                                  const void* v_cache, const int32_t* block_table,
                                  const int32_t* context_lens, int num_seqs, int num_heads,
                                  int num_kv_heads, int head_size, int block_size,
                                  int64_t num_blocks, int max_blocks_per_seq, float scale,
                                  int partition_size, int max_partitions, float* max_logits,
                                  float* exp_sums, float* tmp_out, int32_t* counters, int dtype,
                                  void* stream) {
  if (partition_size < 1) return PKV_ERR_SHAPE;
  pkv::DecodeArgs a{};
  const int rc = decode_args(a, out, query, k_cache, v_cache, block_table, context_lens,
                             num_seqs, num_heads, num_kv_heads, head_size, block_size,
                             num_blocks, max_blocks_per_seq, scale, partition_size,
                             max_partitions, max_logits, exp_sums, tmp_out, dtype);
  if (rc != kLaunch) return rc;
  if (!out) return PKV_ERR_NULL;
  if (!counters) return PKV_ERR_WORKSPACE;
  if (pkv::fast_decode_supported(a)) {
    a.counters = counters;
    return launch_status(pkv::launch_decode_fast(a, as_stream(stream)));
  }
  // the plain kernel writes partials; the merge follows as a second launch
  if (num_seqs > kMaxGridYZ || num_heads > kMaxGridYZ) return PKV_ERR_UNSUPPORTED;
  a.out = nullptr;
  hipError_t e = pkv::launch_decode_generic(a, as_stream(stream));
  if (e != hipSuccess) return PKV_ERR_LAUNCH;
  return launch_status(pkv::launch_reduce(out, max_logits, exp_sums, tmp_out, context_lens,
                                          num_seqs, num_heads, head_size, partition_size,
                                          max_partitions, as_stream(stream)));
}

int paged_decode_attention_append(float* out, const void* query, void* k_cache, void* v_cache,
                                  const void* k_new, const void* v_new,
                                  const int32_t* block_table, const int32_t* context_lens,
                                  int num_seqs, int num_heads, int num_kv_heads, int head_size,
                                  int block_size, int64_t num_blocks, int max_blocks_per_seq,
                                  float scale, int partition_size, int max_partitions,
                                  float* max_logits, float* exp_sums, float* tmp_out,
                                  int32_t* counters, int dtype, void* stream) {
  if (partition_size < 1) return PKV_ERR_SHAPE;
  pkv::DecodeArgs a{};
  const int rc = decode_args(a, out, query, k_cache, v_cache, block_table, context_lens,
                             num_seqs, num_heads, num_kv_heads, head_size, block_size,
                             num_blocks, max_blocks_per_seq, scale, partition_size,
                             max_partitions, max_logits, exp_sums, tmp_out, dtype);
  if (rc != kLaunch) return rc;
  if (!out || !k_new || !v_new) return PKV_ERR_NULL;
  if (!counters) return PKV_ERR_WORKSPACE;
  // the write's grid is one thread per 2-byte chunk at worst
  const int64_t chunks = static_cast<int64_t>(num_seqs) * num_kv_heads *
                         (static_cast<int64_t>(head_size) * elem_bytes(dtype) / 2);
  if (chunks / 256 >= 0x7fffffff) return PKV_ERR_UNSUPPORTED;
  if (pkv::fast_decode_supported(a)) {
    a.counters = counters;
    a.k_new = k_new;
    a.v_new = v_new;
    return launch_status(pkv::launch_decode_fast(a, as_stream(stream)));
  }
  // elsewhere: the write (each sequence's last position), the plain split
  // kernel, the merge
  if (num_seqs > kMaxGridYZ || num_heads > kMaxGridYZ) return PKV_ERR_UNSUPPORTED;
  hipError_t e = pkv::launch_kv_write(k_cache, v_cache, k_new, v_new, nullptr, num_seqs,
                                      num_blocks, num_kv_heads, block_size, head_size,
                                      elem_bytes(dtype), as_stream(stream), block_table,
                                      context_lens, max_blocks_per_seq);
  if (e != hipSuccess) return PKV_ERR_LAUNCH;
  a.out = nullptr;
  e = pkv::launch_decode_generic(a, as_stream(stream));
  if (e != hipSuccess) return PKV_ERR_LAUNCH;
  return launch_status(pkv::launch_reduce(out, max_logits, exp_sums, tmp_out, context_lens,
                                          num_seqs, num_heads, head_size, partition_size,
                                          max_partitions, as_stream(stream)));
}

int paged_attention_reduce(float* out, const float* max_logits, const float* exp_sums,
                           const float* tmp_out, const int32_t* context_lens, int num_seqs,
                           int num_heads, int head_size, int partition_size, int max_partitions,
                           void* stream) {
  if (num_seqs < 0 || num_heads < 1 || head_size < 1 || partition_size < 1 ||
      max_partitions < 1)
    return PKV_ERR_SHAPE;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !max_logits || !exp_sums || !tmp_out || !context_lens) return PKV_ERR_NULL;
  // one wave per (sequence, head), four per workgroup
  if (static_cast<int64_t>(num_seqs) * num_heads / 4 >= 0x7fffffff) return PKV_ERR_UNSUPPORTED;
  return launch_status(pkv::launch_reduce(out, max_logits, exp_sums, tmp_out, context_lens,
                                          num_seqs, num_heads, head_size, partition_size,
                                          max_partitions, as_stream(stream)));
}

int paged_varlen_attention(float* out, const void* query, const void* k_cache,
                           const void* v_cache, const int32_t* block_table,
                           const int32_t* query_start_loc, const int32_t* context_lens,
                           int num_seqs, int num_tokens, int num_heads, int num_kv_heads,
                           int head_size, int block_size, int64_t num_blocks,
                           int max_blocks_per_seq, float scale, int max_partitions,
                           float* max_logits, float* exp_sums, float* tmp_out, int dtype,
                           void* stream) {
  pkv::DecodeArgs a{};
  const int rc = varlen_args(a, out, query, k_cache, v_cache, block_table, query_start_loc,
                             context_lens, num_seqs, num_tokens, num_heads, num_kv_heads,
                             head_size, block_size, num_blocks, max_blocks_per_seq, scale,
                             max_partitions, dtype);
  if (rc != kLaunch) return rc;
  if (!max_logits || !exp_sums || !tmp_out) return PKV_ERR_WORKSPACE;
  a.max_logits = max_logits;
  a.exp_sums = exp_sums;
  a.tmp_out = tmp_out;
  return varlen_launch(a, as_stream(stream));
}

int paged_varlen_attention_noalloc(float* out, const void* query, const void* k_cache,
                                   const void* v_cache, const int32_t* block_table,
                                   const int32_t* query_start_loc, const int32_t* context_lens,
                                   int num_seqs, int num_tokens, int num_heads, int num_kv_heads,
                                   int head_size, int block_size, int64_t num_blocks,
                                   int max_blocks_per_seq, float scale, int max_partitions,
                                   int dtype, void* stream) {
  pkv::DecodeArgs a{};
  const int rc = varlen_args(a, out, query, k_cache, v_cache, block_table, query_start_loc,
                             context_lens, num_seqs, num_tokens, num_heads, num_kv_heads,
                             head_size, block_size, num_blocks, max_blocks_per_seq, scale,
                             max_partitions, dtype);
  if (rc != kLaunch) return rc;
  const size_t bytes = paged_varlen_attention_noalloc_bytes(num_tokens, num_heads, head_size,
                                                            max_partitions);
  if (bytes == 0 || bytes > pkv::kNoAllocScratchBytes) return PKV_ERR_SCRATCH;
  // the first HIP call: the static buffer's address on the current device
  void* base = nullptr;
  if (pkv::noalloc_scratch(&base) != hipSuccess) return PKV_ERR_LAUNCH;
  const size_t ml = scratch_part(static_cast<size_t>(num_tokens) * num_heads * max_partitions);
  char* p = static_cast<char*>(base);
  a.max_logits = reinterpret_cast<float*>(p);
  a.exp_sums = reinterpret_cast<float*>(p + ml);
  a.tmp_out = reinterpret_cast<float*>(p + 2 * ml);
  return varlen_launch(a, as_stream(stream));
}

size_t paged_varlen_attention_noalloc_bytes(int num_tokens, int num_heads, int head_size,
                                            int max_partitions) {
  if (num_tokens <= 0 || num_heads <= 0 || head_size <= 0 || max_partitions <= 0) return 0;
  const size_t slots = static_cast<size_t>(num_tokens) * num_heads * max_partitions;
  return 2 * scratch_part(slots) + scratch_part(slots * head_size);
}

size_t paged_varlen_attention_noalloc_limit(void) { return pkv::kNoAllocScratchBytes; }

int paged_kv_copy_blocks(void* const* k_caches, void* const* v_caches, int num_layers,
                         const int64_t* block_mapping, int64_t num_pairs, int64_t num_blocks,
                         int num_kv_heads, int block_size, int head_size, int dtype,
                         void* stream) {
  int64_t slab = 0;
  const int rc = move_checks(k_caches, v_caches, num_layers, num_pairs, num_blocks,
                             num_kv_heads, block_size, head_size, dtype, &slab);
  if (rc != PKV_OK || num_layers == 0 || num_pairs == 0) return rc;
  if (!block_mapping) return PKV_ERR_NULL;
  pkv::MoveArgs m{k_caches, v_caches, num_layers, nullptr, block_mapping, num_pairs,
                  num_blocks, slab};
  return launch_status(pkv::launch_copy_blocks(m, as_stream(stream)));
}

int paged_kv_swap_out(void* host_dst, int64_t host_bytes, void* const* k_caches,
                      void* const* v_caches, int num_layers, const int64_t* block_ids,
                      int64_t num_ids, int64_t num_blocks, int num_kv_heads, int block_size,
                      int head_size, int dtype, void* stream) {
  return swap_common(host_dst, host_bytes, k_caches, v_caches, num_layers, block_ids, num_ids,
                     num_blocks, num_kv_heads, block_size, head_size, dtype, true, stream);
}

int paged_kv_swap_in(const void* host_src, int64_t host_bytes, void* const* k_caches,
                     void* const* v_caches, int num_layers, const int64_t* block_ids,
                     int64_t num_ids, int64_t num_blocks, int num_kv_heads, int block_size,
                     int head_size, int dtype, void* stream) {
  return swap_common(const_cast<void*>(host_src), host_bytes, k_caches, v_caches, num_layers,
                     block_ids, num_ids, num_blocks, num_kv_heads, block_size, head_size, dtype,
                     false, stream);
}

size_t paged_attention_workspace_bytes(int num_seqs, int num_heads, int head_size,
                                       int max_partitions) {
  if (num_seqs <= 0 || num_heads <= 0 || head_size <= 0 || max_partitions <= 0) return 0;
  return static_cast<size_t>(num_seqs) * num_heads * max_partitions * (head_size + 2) *
         sizeof(float);
}

int paged_kv_gather(void* k_out, void* v_out, const void* k_cache, const void* v_cache,
                    const int32_t* block_table, const int32_t* context_lens, int num_seqs,
                    int num_kv_heads, int head_size, int block_size, int64_t num_blocks,
                    int max_blocks_per_seq, int max_ctx, int dtype, void* stream) {
  const int eb = elem_bytes(dtype);
  if (eb == 0) return PKV_ERR_DTYPE;
  if (num_seqs < 0 || num_kv_heads < 1 || head_size < 1 || block_size < 1 || num_blocks < 1 ||
      max_blocks_per_seq < 1 || max_ctx < 0)
    return PKV_ERR_SHAPE;
  if (num_seqs == 0 || max_ctx == 0) return PKV_OK;
  if (!k_out || !v_out || !k_cache || !v_cache || !block_table || !context_lens)
    return PKV_ERR_NULL;
  const int64_t chunks = static_cast<int64_t>(num_seqs) * num_kv_heads * max_ctx *
                         (static_cast<int64_t>(head_size) * eb / 2);
  if (chunks / 256 >= 0x7fffffff) return PKV_ERR_UNSUPPORTED;
  return launch_status(pkv::launch_kv_gather(k_out, v_out, k_cache, v_cache, block_table,
                                             context_lens, num_seqs, num_kv_heads, head_size,
                                             block_size, num_blocks, max_blocks_per_seq, max_ctx,
                                             eb, as_stream(stream)));
}

const char* pkv_strerror(int code) {
  switch (code) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "a required pointer is NULL";
    case PKV_ERR_SHAPE: return "a size is out of range or inconsistent";
    case PKV_ERR_DTYPE: return "unknown dtype code";
    case PKV_ERR_UNSUPPORTED: return "no kernel handles this shape";
    case PKV_ERR_WORKSPACE: return "split mode needs max_logits, exp_sums and tmp_out";
    case PKV_ERR_LAUNCH: return "the HIP runtime refused a kernel launch";
    case PKV_ERR_HOST: return "the host buffer is too small or not pinned memory the GPU reaches";
    case PKV_ERR_STATE: return "not valid in the block pool's current state";
    case PKV_ERR_CAPACITY: return "not enough free blocks (nothing was taken)";
    case PKV_ERR_SCRATCH:
      return "the call's partials exceed the library's static scratch buffer";
    default: return "unknown pkv status code";
  }
}

}  // extern "C"
