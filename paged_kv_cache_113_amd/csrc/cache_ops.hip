// Slot mapping, new-token K/V write and the checking gather, for gfx950.
//
// All three are integer/bit-copy work: no floating point touches the data,
// so their results are bit-exact by construction.
#include "device.h"
#include "launch.h"

namespace pkv {

// slot = table[p / B] * B + p % B ("vLLM PagedAttention: from fragmentation
// to slot mapping", section 3), -1 when p < 0 or the table does not cover p.
__global__ void slot_mapping_kernel(int64_t* __restrict__ slot_mapping,
                                    const int32_t* __restrict__ block_table,
                                    const int32_t* __restrict__ positions, int num_seqs,
                                    int max_blocks, int block_size) {
  int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= num_seqs) return;
  int p = positions[s];
  int64_t slot = -1;
  if (p >= 0) {
    int lb = p / block_size;
    if (lb < max_blocks) {
      int64_t b = block_table[static_cast<int64_t>(s) * max_blocks + lb];
      if (b >= 0) slot = b * block_size + p % block_size;
    }
  }
  slot_mapping[s] = slot;
}

hipError_t launch_slot_mapping(int64_t* slot_mapping, const int32_t* block_table,
                               const int32_t* positions, int num_seqs, int max_blocks,
                               int block_size, hipStream_t stream) {
  const int threads = 256;
  int blocks = (num_seqs + threads - 1) / threads;
  slot_mapping_kernel<<<blocks, threads, 0, stream>>>(slot_mapping, block_table, positions,
                                                      num_seqs, max_blocks, block_size);
  return hipGetLastError();
}

// Copy unit of W bytes (W = 16, 8, 4 or 2).
template <int W> struct Chunk;
template <> struct Chunk<16> { using type = uint4; };
template <> struct Chunk<8> { using type = uint2; };
template <> struct Chunk<4> { using type = uint32_t; };
template <> struct Chunk<2> { using type = uint16_t; };

// One thread per W-byte chunk of one (token, kv head) row, for K and V.
// The backend writes new K/V to the slots the slot mapping names ("vLLM
// PagedAttention ...", section 6); slot s is block s / B, offset s % B.
// Without a slot mapping (slot_mapping == NULL) token i is the last
// position ctx_i - 1 of sequence i, stored where that position translates
// through the sequence's table row.
template <int W>
__global__ void kv_write_kernel(char* __restrict__ k_cache, char* __restrict__ v_cache,
                                const char* __restrict__ k_new, const char* __restrict__ v_new,
                                const int64_t* __restrict__ slot_mapping, int64_t num_tokens,
                                int64_t num_slots, int num_kv_heads, int block_size,
                                int row_bytes, const int32_t* __restrict__ block_table,
                                const int32_t* __restrict__ context_lens, int max_blocks) {
  using T = typename Chunk<W>::type;
  const int cpr = row_bytes / W;  // chunks per (token, head) row
  int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  int64_t total = num_tokens * num_kv_heads * cpr;
  if (g >= total) return;
  int c = static_cast<int>(g % cpr);
  int64_t r = g / cpr;
  int h = static_cast<int>(r % num_kv_heads);
  int64_t i = r / num_kv_heads;
  int64_t slot = -1;
  if (slot_mapping != nullptr) {
    slot = slot_mapping[i];
  } else {
    const int p = context_lens[i] - 1;
    const int64_t b = physical_block(block_table + i * max_blocks, p, block_size, max_blocks,
                                     num_slots / block_size);
    slot = b >= 0 ? b * block_size + p % block_size : -1;
  }
  if (slot < 0 || slot >= num_slots) return;
  int64_t blk = slot / block_size;
  int off = static_cast<int>(slot % block_size);
  int64_t dst = ((blk * num_kv_heads + h) * block_size + off) * row_bytes + c * W;
  int64_t src = (i * num_kv_heads + h) * row_bytes + c * W;
  *reinterpret_cast<T*>(k_cache + dst) = *reinterpret_cast<const T*>(k_new + src);
  *reinterpret_cast<T*>(v_cache + dst) = *reinterpret_cast<const T*>(v_new + src);
}

static int chunk_width(int row_bytes, const void* const* ptrs, int n) {
  uintptr_t acc = 0;
  for (int i = 0; i < n; ++i) acc |= reinterpret_cast<uintptr_t>(ptrs[i]);
  for (int w : {16, 8, 4}) {
    if (row_bytes % w == 0 && acc % w == 0) return w;
  }
  return 2;
}

hipError_t launch_kv_write(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                           const int64_t* slot_mapping, int64_t num_tokens, int64_t num_blocks,
                           int num_kv_heads, int block_size, int head_size, int elem_bytes,
                           hipStream_t stream, const int32_t* block_table,
                           const int32_t* context_lens, int max_blocks) {
  int row_bytes = head_size * elem_bytes;
  const void* ptrs[4] = {k_cache, v_cache, k_new, v_new};
  int w = chunk_width(row_bytes, ptrs, 4);
  int64_t total = num_tokens * num_kv_heads * (row_bytes / w);
  const int threads = 256;
  unsigned blocks = static_cast<unsigned>((total + threads - 1) / threads);
  int64_t num_slots = num_blocks * block_size;
  auto* kc = static_cast<char*>(k_cache);
  auto* vc = static_cast<char*>(v_cache);
  auto* kn = static_cast<const char*>(k_new);
  auto* vn = static_cast<const char*>(v_new);
  switch (w) {
    case 16:
      kv_write_kernel<16><<<blocks, threads, 0, stream>>>(kc, vc, kn, vn, slot_mapping,
                                                          num_tokens, num_slots, num_kv_heads,
                                                          block_size, row_bytes, block_table,
                                                          context_lens, max_blocks);
      break;
    case 8:
      kv_write_kernel<8><<<blocks, threads, 0, stream>>>(kc, vc, kn, vn, slot_mapping,
                                                         num_tokens, num_slots, num_kv_heads,
                                                         block_size, row_bytes, block_table,
                                                         context_lens, max_blocks);
      break;
    case 4:
      kv_write_kernel<4><<<blocks, threads, 0, stream>>>(kc, vc, kn, vn, slot_mapping,
                                                         num_tokens, num_slots, num_kv_heads,
                                                         block_size, row_bytes, block_table,
                                                         context_lens, max_blocks);
      break;
    default:
      kv_write_kernel<2><<<blocks, threads, 0, stream>>>(kc, vc, kn, vn, slot_mapping,
                                                         num_tokens, num_slots, num_kv_heads,
                                                         block_size, row_bytes, block_table,
                                                         context_lens, max_blocks);
  }
  return hipGetLastError();
}

// Paged -> contiguous copy through the same translation helper the attention
// kernels use (the glossary page's gather_paged). One thread per W-byte chunk
// of one (seq, head, position) row.
template <int W>
__global__ void kv_gather_kernel(char* __restrict__ k_out, char* __restrict__ v_out,
                                 const char* __restrict__ k_cache,
                                 const char* __restrict__ v_cache,
                                 const int32_t* __restrict__ block_table,
                                 const int32_t* __restrict__ context_lens, int num_seqs,
                                 int num_kv_heads, int block_size, int64_t num_blocks,
                                 int max_blocks, int max_ctx, int row_bytes, int elem_bytes) {
  using T = typename Chunk<W>::type;
  const int cpr = row_bytes / W;
  int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  int64_t total = static_cast<int64_t>(num_seqs) * num_kv_heads * max_ctx * cpr;
  if (g >= total) return;
  int c = static_cast<int>(g % cpr);
  int64_t r = g / cpr;
  int t = static_cast<int>(r % max_ctx);
  r /= max_ctx;
  int h = static_cast<int>(r % num_kv_heads);
  int s = static_cast<int>(r / num_kv_heads);
  if (t >= context_lens[s]) return;
  int64_t blk = physical_block(block_table + static_cast<int64_t>(s) * max_blocks, t,
                               block_size, max_blocks, num_blocks);
  if (blk < 0) return;
  int head_size = row_bytes / elem_bytes;
  int64_t src = pool_row(blk, h, t % block_size, num_kv_heads, block_size, head_size) *
                    elem_bytes + c * W;
  int64_t dst = ((static_cast<int64_t>(s) * num_kv_heads + h) * max_ctx + t) * row_bytes + c * W;
  *reinterpret_cast<T*>(k_out + dst) = *reinterpret_cast<const T*>(k_cache + src);
  *reinterpret_cast<T*>(v_out + dst) = *reinterpret_cast<const T*>(v_cache + src);
}

hipError_t launch_kv_gather(void* k_out, void* v_out, const void* k_cache, const void* v_cache,
                            const int32_t* block_table, const int32_t* context_lens,
                            int num_seqs, int num_kv_heads, int head_size, int block_size,
                            int64_t num_blocks, int max_blocks, int max_ctx, int elem_bytes,
                            hipStream_t stream) {
  int row_bytes = head_size * elem_bytes;
  const void* ptrs[4] = {k_out, v_out, k_cache, v_cache};
  int w = chunk_width(row_bytes, ptrs, 4);
  int64_t total = static_cast<int64_t>(num_seqs) * num_kv_heads * max_ctx * (row_bytes / w);
  const int threads = 256;
  unsigned blocks = static_cast<unsigned>((total + threads - 1) / threads);
  auto* ko = static_cast<char*>(k_out);
  auto* vo = static_cast<char*>(v_out);
  auto* kc = static_cast<const char*>(k_cache);
  auto* vc = static_cast<const char*>(v_cache);
#define PKV_GATHER(W_)                                                                    \
  kv_gather_kernel<W_><<<blocks, threads, 0, stream>>>(ko, vo, kc, vc, block_table,        \
                                                       context_lens, num_seqs, num_kv_heads, \
                                                       block_size, num_blocks, max_blocks,   \
                                                       max_ctx, row_bytes, elem_bytes)
  switch (w) {
    case 16: PKV_GATHER(16); break;
    case 8: PKV_GATHER(8); break;
    case 4: PKV_GATHER(4); break;
    default: PKV_GATHER(2);
  }
#undef PKV_GATHER
  return hipGetLastError();
}

}  // namespace pkv
