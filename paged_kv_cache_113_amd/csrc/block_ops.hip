// Whole-block moves for gfx950: copy-on-write block copies inside each
// layer's pools, and swapping blocks out to / back in from pinned host
// memory.
//
// Copy-on-write: when a sequence must write into a partly filled block that
// other sequences still reference, the block's KV data is first copied into
// a fresh block (nxmr.cn article, section 4.2); only that block is copied,
// never the whole cache (paper-notes page, beam search and parallel
// sampling). The copy covers every layer, both K and V.
//
// Swapping: a preempted request's KV blocks are copied from GPU to CPU
// memory and back once the GPU has room again (paper-notes page, preemption
// by swapping); on the way back they land in newly allocated blocks and the
// table is rewritten (nxmr.cn article, section 6.2).
//
// All of it is a bit copy of whole [Hkv, B, D] slabs. One workgroup moves one
// (block, layer, K or V) slab: 256 lanes x 16 B x 8 loads in flight = 32 KiB,
// the slab of Hkv = 8, B = 16, D = 128 at 16 bits, in one pass with every
// load issued before the first store.
#include "device.h"
#include "launch.h"

namespace pkv {
namespace {

constexpr int kMoveThreads = 256;
constexpr int kUnroll = 8;

// Copy units are clang vector types: an array of them stays in registers
// (an array of HIP's struct vectors would be staged through scratch memory).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <int W> struct Unit;
template <> struct Unit<16> { using type = u32x4; };
template <> struct Unit<8> { using type = u32x2; };
template <> struct Unit<4> { using type = uint32_t; };
template <> struct Unit<2> { using type = uint16_t; };

// Mode: what moves where. The slab index i of a launch names
//   kCopy:    mapping[2i] -> mapping[2i+1] inside the layer's pool;
//   kSwapOut: pool block ids[i] -> host slab [layer][K/V][i];
//   kSwapIn:  host slab [layer][K/V][i] -> pool block ids[i].
enum Mode { kCopy = 0, kSwapOut = 1, kSwapIn = 2 };

template <int W, int M>
__global__ __launch_bounds__(kMoveThreads) void move_blocks_kernel(
    LayerPtrs p, int layer0, char* __restrict__ host,
    const int64_t* __restrict__ ids, int64_t n, int64_t num_blocks, int64_t slab_bytes) {
  using T = typename Unit<W>::type;
  const int64_t i = blockIdx.x;
  const int ly = blockIdx.y;
  const int kv = blockIdx.z;
  char* pool = kv ? p.v[ly] : p.k[ly];
  const char* src;
  char* dst;
  if constexpr (M == kCopy) {
    const int64_t a = read_only(ids + 2 * i);
    const int64_t b = read_only(ids + 2 * i + 1);
    if (a < 0 || a >= num_blocks || b < 0 || b >= num_blocks || a == b) return;
    src = pool + a * slab_bytes;
    dst = pool + b * slab_bytes;
  } else {
    const int64_t blk = read_only(ids + i);
    if (blk < 0 || blk >= num_blocks) return;  // skipped: nothing moves
    char* h = host + ((static_cast<int64_t>(layer0 + ly) * 2 + kv) * n + i) * slab_bytes;
    if constexpr (M == kSwapOut) {
      src = pool + blk * slab_bytes;
      dst = h;
    } else {
      src = h;
      dst = pool + blk * slab_bytes;
    }
  }
  const int64_t units = slab_bytes / W;
  const T* __restrict__ s = reinterpret_cast<const T*>(src);
  T* __restrict__ d = reinterpret_cast<T*>(dst);
  // whole batches of kUnroll chunks per lane: no per-chunk guard, so all the
  // loads of a batch are issued before the first one is waited for
  constexpr int kBatch = kMoveThreads * kUnroll;
  const int64_t whole = units / kBatch * kBatch;
  for (int64_t u0 = threadIdx.x; u0 < whole; u0 += kBatch) {
    T r[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) r[k] = s[u0 + k * kMoveThreads];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) d[u0 + k * kMoveThreads] = r[k];
  }
  for (int64_t u = whole + threadIdx.x; u < units; u += kMoveThreads) d[u] = s[u];
}

int unit_width(int64_t slab_bytes, uintptr_t addr_bits) {
  for (int w : {16, 8, 4}) {
    if (slab_bytes % w == 0 && addr_bits % w == 0) return w;
  }
  return 2;
}

template <int M>
hipError_t launch_moves(const MoveArgs& m, hipStream_t stream) {
  uintptr_t bits = reinterpret_cast<uintptr_t>(m.host);
  for (int l = 0; l < m.num_layers; ++l)
    bits |= reinterpret_cast<uintptr_t>(m.k_caches[l]) | reinterpret_cast<uintptr_t>(m.v_caches[l]);
  const int w = unit_width(m.slab_bytes, bits);
  for (int l0 = 0; l0 < m.num_layers; l0 += kMaxLayersPerLaunch) {
    const int nl = m.num_layers - l0 < kMaxLayersPerLaunch ? m.num_layers - l0
                                                           : kMaxLayersPerLaunch;
    LayerPtrs p{};
    for (int l = 0; l < nl; ++l) {
      p.k[l] = static_cast<char*>(m.k_caches[l0 + l]);
      p.v[l] = static_cast<char*>(m.v_caches[l0 + l]);
    }
    const dim3 grid(static_cast<unsigned>(m.n), static_cast<unsigned>(nl), 2);
    char* host = static_cast<char*>(m.host);
#define PKV_MOVE(W_)                                                                      \
  move_blocks_kernel<W_, M><<<grid, kMoveThreads, 0, stream>>>(p, l0, host, m.ids, m.n,     \
                                                               m.num_blocks, m.slab_bytes)
    switch (w) {
      case 16: PKV_MOVE(16); break;
      case 8: PKV_MOVE(8); break;
      case 4: PKV_MOVE(4); break;
      default: PKV_MOVE(2);
    }
#undef PKV_MOVE
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_copy_blocks(const MoveArgs& m, hipStream_t stream) {
  return launch_moves<kCopy>(m, stream);
}

hipError_t launch_swap(const MoveArgs& m, bool out, hipStream_t stream) {
  return out ? launch_moves<kSwapOut>(m, stream) : launch_moves<kSwapIn>(m, stream);
}

}  // namespace pkv
