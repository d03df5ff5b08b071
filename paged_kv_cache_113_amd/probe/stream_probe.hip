// Read-stream probe (bench-only library libpkvprobe.so, not part of the
// attention library): the read bandwidth that a read-once stream with the
// split decode kernel's access pattern reaches on the current device,
// without the kernel's arithmetic. The bench sets it beside the datasheet
// peak as the practical bound of that pattern.
//
// The pattern: K and V pools of blocks whose `heads` KV-head slabs lie side
// by side (a [blocks, heads, rows, dims] pool), each slab `tiles_per_head`
// 4 KiB tiles long. Blocks are visited in a caller-given order (a shuffled
// pool). Wave (range r, head h) reads slab h of every block in range r of
// that order, K and V at the same place, tile by tile with two tiles in
// flight; the waves of one range and all heads run side by side, numbered
// XCD by XCD (workgroup i runs on XCD i % 8), so the slabs of one block,
// contiguous in memory, are read by neighbouring waves at about the same
// time. 16-byte loads with the non-temporal hint; `wg_per_cu` 4-wave
// workgroups per CU. This is the decode kernel's launch shape, load width,
// loads in flight, cache policy and address order.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kDepth = 2;                 // tiles in flight per wave
constexpr int64_t kTileBytes = 4096;
constexpr int kXcds = 8;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct Tile {
  u32x4 k[4];
  u32x4 v[4];
};

template <typename T>
__device__ __forceinline__ T scalar_read(const T* p) {
  return *reinterpret_cast<const __attribute__((address_space(4))) T*>(
      reinterpret_cast<uintptr_t>(p));
}

__global__ __launch_bounds__(kThreads) void read_probe_kernel(
    const char* __restrict__ kbuf, const char* __restrict__ vbuf,
    const int32_t* __restrict__ order, int64_t n_blocks, int64_t buf_blocks, int heads,
    int tiles_per_head, u32x4* sink) {
  const int lane = threadIdx.x & 63;
  const int n_wg = gridDim.x;
  const int xcd_rank = (blockIdx.x % kXcds) * (n_wg / kXcds) + blockIdx.x / kXcds;
  const int wg_rank = n_wg % kXcds == 0 ? xcd_rank : static_cast<int>(blockIdx.x);
  const int64_t gw = static_cast<int64_t>(wg_rank) * kWaves +
                     __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t ranges = static_cast<int64_t>(n_wg) * kWaves / heads;
  const int h = static_cast<int>(gw % heads);
  const int64_t r = gw / heads;
  if (r >= ranges) return;
  // the wave's tiles: tiles_per_head per block of its range
  const int64_t t0 = r * n_blocks / ranges * tiles_per_head;
  const int64_t t1 = (r + 1) * n_blocks / ranges * tiles_per_head;
  if (t0 >= t1) return;
  const int64_t slab = static_cast<int64_t>(tiles_per_head) * kTileBytes;
  const int64_t block_bytes = slab * heads;
  u32x4 acc[kDepth];
#pragma unroll
  for (int d = 0; d < kDepth; ++d) acc[d] = u32x4{0u, 0u, 0u, 0u};
  // tile j of the wave: block order[j / tiles_per_head] (an index outside
  // the pools reads block 0), tile j % tiles_per_head of slab h
  auto load = [&](int64_t j, Tile& t) {
    int64_t blk = scalar_read(order + j / tiles_per_head);
    blk = (blk >= 0 && blk < buf_blocks) ? blk : 0;
    const int64_t base = blk * block_bytes + h * slab + (j % tiles_per_head) * kTileBytes +
                         lane * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      t.k[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbuf + base + i * 1024));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      t.v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vbuf + base + i * 1024));
  };
  auto eat = [&](const Tile& t, u32x4& x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x ^= t.k[i] ^ t.v[i];
  };
  Tile buf[kDepth];
  // (a wave with fewer tiles than slots reads its last tile again)
#pragma unroll
  for (int d = 0; d < kDepth; ++d) load(t0 + d < t1 ? t0 + d : t1 - 1, buf[d]);
  int64_t i = t0;
  // steady state: every next tile exists, so the loads are unconditional and
  // each use waits only for its own tile's loads
  for (; i + 2 * kDepth <= t1; i += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      eat(buf[d], acc[d]);
      load(i + d + kDepth, buf[d]);
      // keep the next tile's loads issued before the following use waits
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  for (; i < t1; i += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      if (i + d < t1) {
        eat(buf[d], acc[d]);
        if (i + d + kDepth < t1) load(i + d + kDepth, buf[d]);
      }
    }
  }
  // the loads' results decide a store that (for any real data) never
  // happens, so the loads cannot be dropped
#pragma unroll
  for (int d = 1; d < kDepth; ++d) acc[0] ^= acc[d];
  if (acc[0].x == 0x9e3779b9u && acc[0].y == 0x7f4a7c15u && acc[0].z == 0x85ebca6bu &&
      acc[0].w == 0xc2b2ae35u)
    sink[0] = acc[0];
}

}  // namespace

extern "C" {

// Reads slabs 0..heads-1 (tiles_per_head 4 KiB tiles each) of K and V block
// block_order[i] for every i < num_blocks: 2 * heads * tiles_per_head * 4096
// bytes per listed block. k, v: device buffers of buffer_bytes each, a whole
// number of blocks; block_order: device int32 [num_blocks] (an entry outside
// the buffers reads block 0); sink: 16 bytes of device memory, written only on
// a data-dependent condition that keeps the loads (its contents mean
// nothing); wg_per_cu: 1 or 2. The caller owns every buffer and times the
// call on its stream. Returns 0, or -2 for inconsistent sizes, -1 for a NULL
// pointer, -6 when the HIP runtime refuses the launch. num_blocks == 0 is a
// no-op.
int pkvprobe_read_stream(const void* k, const void* v, int64_t buffer_bytes,
                         const int32_t* block_order, int64_t num_blocks, int heads,
                         int tiles_per_head, int wg_per_cu, void* sink, void* stream) {
  if (heads < 1 || tiles_per_head < 1 || wg_per_cu < 1 || wg_per_cu > 2 || num_blocks < 0)
    return -2;
  const int64_t block_bytes = kTileBytes * heads * tiles_per_head;
  if (buffer_bytes < block_bytes || buffer_bytes % block_bytes != 0) return -2;
  if (num_blocks == 0) return 0;
  if (!k || !v || !block_order || !sink) return -1;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return -6;
  // whole groups of `heads` waves, as the decode kernel launches
  const int64_t waves = static_cast<int64_t>(cus) * wg_per_cu * kWaves;
  const int64_t per_head = waves / heads > 0 ? waves / heads : 1;
  const int64_t wgs = (per_head * heads + kWaves - 1) / kWaves;
  read_probe_kernel<<<dim3(static_cast<unsigned>(wgs)), dim3(kThreads), 0,
                      static_cast<hipStream_t>(stream)>>>(
      static_cast<const char*>(k), static_cast<const char*>(v), block_order, num_blocks,
      buffer_bytes / block_bytes, heads, tiles_per_head, static_cast<u32x4*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"
