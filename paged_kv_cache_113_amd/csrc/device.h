// Device helpers shared by the gfx950 kernels of the paged-KV library.
//
// Block-table translation follows "vLLM PagedAttention: from fragmentation to
// slot mapping", section 3: position p of a sequence lives in physical block
// table[p / B] at offset p % B. Pools are [num_blocks, Hkv, B, D].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// Storage types. Conversions to float are exact.
struct bf16_t { uint16_t bits; };
struct f16_t { uint16_t bits; };

__device__ __forceinline__ float to_float(float x) { return x; }
__device__ __forceinline__ float to_float(bf16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x.bits) << 16);
}
__device__ __forceinline__ float to_float(f16_t x) {
  _Float16 h;
  __builtin_memcpy(&h, &x.bits, 2);
  return static_cast<float>(h);
}

// The two halves of a 32-bit word holding two 16-bit values, widened.
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float lo_f16(uint32_t w) {
  _Float16 h;
  uint16_t b = static_cast<uint16_t>(w);
  __builtin_memcpy(&h, &b, 2);
  return static_cast<float>(h);
}
__device__ __forceinline__ float hi_f16(uint32_t w) {
  _Float16 h;
  uint16_t b = static_cast<uint16_t>(w >> 16);
  __builtin_memcpy(&h, &b, 2);
  return static_cast<float>(h);
}

// Loads of data the kernels only read (block tables, lengths) go through the
// constant address space: with a uniform address they become scalar loads,
// which do not wait behind the vector loads of K/V tiles in flight.
template <typename T>
__device__ __forceinline__ T read_only(const T* p) {
  return *reinterpret_cast<const __attribute__((address_space(4))) T*>(
      reinterpret_cast<uintptr_t>(p));
}

// 16-byte load of data read once per call (K/V tiles), with the non-temporal
// hint: the lines are not kept in the caches at the expense of other data.
// On MI355X a stream of such loads sustains ~6.6 TB/s against ~6.0 TB/s for
// plain loads of the same addresses.
__device__ __forceinline__ uint4 stream_load(const void* p) {
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t x = __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
  return make_uint4(x[0], x[1], x[2], x[3]);
}

// Stores of partial results from inside a streaming loop. On this GPU
// family loads and stores share one outstanding-operation counter, and
// loads complete in issue order while stores may not. Once the compiler
// sees a store that may still be pending beside loads, it stops counting
// and waits for every outstanding operation before each tile, so no tile
// load stays in flight across a tile. These stores are emitted as
// instructions the compiler does not track, which keeps its load waits
// exact. Those waits remain correct: waiting until at most N operations are
// outstanding, N the loads issued after the one needed, cannot finish before
// that load, whatever stores sit in between. Nothing in the issuing kernel
// reads what these stores write; the kernel's end makes it visible. The
// two wait states after each store are the ones the compiler puts between a
// store and the next write of its data registers (it does not see inside
// the asm statement, so it cannot add them itself).
__device__ __forceinline__ void store_untracked(float* p, float4 v) {
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  const f32x4_t x = {v.x, v.y, v.z, v.w};
  asm volatile("global_store_dwordx4 %0, %1, off\n\ts_nop 1" : : "v"(p), "v"(x));
}
__device__ __forceinline__ void store_untracked(float* p, float v) {
  asm volatile("global_store_dword %0, %1, off\n\ts_nop 1" : : "v"(p), "v"(v));
}
// A 16-byte store of raw data, untracked like the stores above.
__device__ __forceinline__ void store_untracked(void* p, uint4 v) {
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t x = {v.x, v.y, v.z, v.w};
  asm volatile("global_store_dwordx4 %0, %1, off\n\ts_nop 1" : : "v"(p), "v"(x));
}
// The same stores at device scope (sc1): written through to the memory side,
// where waves of the other XCDs read them with device-scope loads, once the
// issuing wave has waited for them (s_waitcnt vmcnt(0)).
__device__ __forceinline__ void store_untracked_device(float* p, float4 v) {
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  const f32x4_t x = {v.x, v.y, v.z, v.w};
  asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 1" : : "v"(p), "v"(x));
}
__device__ __forceinline__ void store_untracked_device(float* p, float v) {
  asm volatile("global_store_dword %0, %1, off sc1\n\ts_nop 1" : : "v"(p), "v"(v));
}
// A device-scope load (reads the value at the memory side, past any copy the
// XCD's own cache may hold).
__device__ __forceinline__ float load_device(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Physical block of logical position `pos`, or -1 when the table row does not
// cover it or holds an id outside [0, num_blocks). Callers skip such
// positions, so a bad table never turns into an out-of-bounds access.
__device__ __forceinline__ int64_t physical_block(const int32_t* table_row, int pos,
                                                  int block_size, int max_blocks,
                                                  int64_t num_blocks) {
  int lb = pos / block_size;
  if (pos < 0 || lb >= max_blocks) return -1;
  int64_t b = read_only(table_row + lb);
  return (b >= 0 && b < num_blocks) ? b : -1;
}

// Element offset of pool[block][kv][off][0] in a [num_blocks, Hkv, B, D] pool.
__device__ __forceinline__ int64_t pool_row(int64_t block, int kv, int off, int num_kv_heads,
                                            int block_size, int head_size) {
  return ((block * num_kv_heads + kv) * block_size + off) * static_cast<int64_t>(head_size);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

// 2^x on the hardware exponential unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace pkv
