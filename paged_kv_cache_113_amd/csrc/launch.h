// Host-side launchers of the gfx950 kernels. Arguments are already
// validated by the C ABI layer (api.cpp); each launcher returns the HIP error
// of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

hipError_t launch_slot_mapping(int64_t* slot_mapping, const int32_t* block_table,
                               const int32_t* positions, int num_seqs, int max_blocks,
                               int block_size, hipStream_t stream);

// slot_mapping NULL: token i is sequence i's last position (ctx_i - 1),
// stored where that position translates through block_table.
hipError_t launch_kv_write(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                           const int64_t* slot_mapping, int64_t num_tokens, int64_t num_blocks,
                           int num_kv_heads, int block_size, int head_size, int elem_bytes,
                           hipStream_t stream, const int32_t* block_table = nullptr,
                           const int32_t* context_lens = nullptr, int max_blocks = 0);

hipError_t launch_kv_gather(void* k_out, void* v_out, const void* k_cache, const void* v_cache,
                            const int32_t* block_table, const int32_t* context_lens,
                            int num_seqs, int num_kv_heads, int head_size, int block_size,
                            int64_t num_blocks, int max_blocks, int max_ctx, int elem_bytes,
                            hipStream_t stream);

struct DecodeArgs {
  float* out;
  const void* query;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  const int32_t* context_lens;
  int num_seqs, num_heads, num_kv_heads, head_size, block_size;
  int64_t num_blocks;
  int max_blocks;
  float scale;
  int partition_size;  // 0: unsplit
  int max_partitions;  // >= 1
  float* max_logits;
  float* exp_sums;
  float* tmp_out;
  int dtype;           // pkv_dtype
  // multi-token queries: [num_seqs + 1] query row starts, NULL for decode
  const int32_t* query_start_loc;
  int num_tokens;      // query rows (multi-token queries)
  // split decode merged in the same launch: [num_seqs * num_kv_heads]
  // arrival counters, zero on entry and left zero; NULL otherwise
  int32_t* counters;
  // decode step: the new tokens' K/V [num_seqs, Hkv, D]; the split kernel
  // stores each at its sequence's last position before reading it; NULL
  // otherwise
  const void* k_new;
  const void* v_new;
};

// Matrix-core path: f16/bf16, head_size 128, block_size % 16 == 0, G <= 16.
bool fast_decode_supported(const DecodeArgs& a);
hipError_t launch_decode_fast(const DecodeArgs& a, hipStream_t stream);
// Plain path: every supported shape.
hipError_t launch_decode_generic(const DecodeArgs& a, hipStream_t stream);

// Multi-token queries (query_start_loc set). Matrix-core path: the balanced
// split kernel over (sequence, column group) units, writing partials for the
// merge; same shapes as the decode fast path.
bool fast_varlen_supported(const DecodeArgs& a);
hipError_t launch_varlen_fast(const DecodeArgs& a, hipStream_t stream);
// Long chunks (at least 128 (token, head) columns per KV head): workgroups
// share each K/V tile in LDS among 128 columns; partials for the merge.
hipError_t launch_prefill_fast(const DecodeArgs& a, hipStream_t stream);
// Plain path: one wave per (query row, head), output written directly.
hipError_t launch_varlen_generic(const DecodeArgs& a, hipStream_t stream);

// Static scratch of paged_varlen_attention_noalloc: its size, and its device
// address on the current device (looked up on the first call per device).
constexpr size_t kNoAllocScratchBytes = size_t{128} << 20;
hipError_t noalloc_scratch(void** out);

// context_lens NULL: every row takes part (multi-token queries).
hipError_t launch_reduce(float* out, const float* max_logits, const float* exp_sums,
                         const float* tmp_out, const int32_t* context_lens, int num_seqs,
                         int num_heads, int head_size, int partition_size, int max_partitions,
                         hipStream_t stream);

// Whole-block moves (copy-on-write copies, swap out / in), one workgroup per
// (slab, layer, K or V); up to kMaxLayersPerLaunch layers' pool pointers ride
// in the kernel arguments, more layers take more launches.
constexpr int kMaxLayersPerLaunch = 64;
struct LayerPtrs {
  char* k[kMaxLayersPerLaunch];
  char* v[kMaxLayersPerLaunch];
};
struct MoveArgs {
  void* const* k_caches;  // host array [num_layers] of device pool pointers
  void* const* v_caches;
  int num_layers;
  void* host;             // swap: device-visible address of the pinned buffer
  const int64_t* ids;     // device: (src, dst) pairs [n][2] (copy) or block ids [n]
  int64_t n;
  int64_t num_blocks;
  int64_t slab_bytes;     // Hkv * B * D * element bytes
};
hipError_t launch_copy_blocks(const MoveArgs& m, hipStream_t stream);
hipError_t launch_swap(const MoveArgs& m, bool out, hipStream_t stream);

}  // namespace pkv
