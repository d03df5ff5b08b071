// Paged decode attention, plain path: any dtype (f32/f16/bf16), head size up
// to 256, any block size and head grouping. One wave per (sequence, query
// head, partition); positions are visited one at a time through the block
// table (block = p / B, offset = p % B: "vLLM PagedAttention: from
// fragmentation to slot mapping", section 3) with an online softmax. It is
// the path for the small and unusual shapes; the matrix-core kernel covers
// the 128-wide heads that carry the bandwidth.
//
// Also the split-partial merge: out = sum_p l_p e^{m_p - M} o_p /
// sum_p l_p e^{m_p - M} (the merge of the source-walkthrough page's V2
// partitions, section 1.8; the pages do not print its formula).
#include "device.h"
#include "launch.h"

namespace pkv {
namespace {

constexpr int kMaxPerLane = 4;  // head_size <= 256

template <typename T>
__global__ __launch_bounds__(64) void decode_generic_kernel(DecodeArgs a) {
  const int lane = threadIdx.x;
  const int part = blockIdx.x;
  const int h = blockIdx.y;
  const int seq = blockIdx.z;
  const int G = a.num_heads / a.num_kv_heads;
  const int kvh = h / G;
  const int D = a.head_size;
  const int B = a.block_size;

  int ctx = a.context_lens[seq];
  const int cap = a.max_blocks * B;
  ctx = ctx < cap ? ctx : cap;
  int lo = 0, hi = ctx;
  if (a.partition_size > 0) {
    lo = part * a.partition_size;
    if (lo >= ctx) {  // no positions here: mark the slot unused for the merge
      if (lane == 0) {
        const int64_t pidx = (static_cast<int64_t>(seq) * a.num_heads + h) * a.max_partitions + part;
        a.max_logits[pidx] = -INFINITY;
        a.exp_sums[pidx] = 0.f;
      }
      return;
    }
    hi = lo + a.partition_size < ctx ? lo + a.partition_size : ctx;
  }
  const T* __restrict__ q = static_cast<const T*>(a.query) +
                            (static_cast<int64_t>(seq) * a.num_heads + h) * D;
  const T* __restrict__ kc = static_cast<const T*>(a.k_cache);
  const T* __restrict__ vc = static_cast<const T*>(a.v_cache);
  const int32_t* __restrict__ row = a.block_table + static_cast<int64_t>(seq) * a.max_blocks;

  float qv[kMaxPerLane], acc[kMaxPerLane];
#pragma unroll
  for (int k = 0; k < kMaxPerLane; ++k) {
    const int d = lane + 64 * k;
    qv[k] = d < D ? to_float(q[d]) : 0.f;
    acc[k] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int t = lo; t < hi; ++t) {
    const int64_t blk = physical_block(row, t, B, a.max_blocks, a.num_blocks);
    if (blk < 0) continue;  // a table entry outside the pool: skipped
    const int64_t base = pool_row(blk, kvh, t % B, a.num_kv_heads, B, D);
    float dot = 0.f;
#pragma unroll
    for (int k = 0; k < kMaxPerLane; ++k) {
      const int d = lane + 64 * k;
      if (d < D) dot = fmaf(qv[k], to_float(kc[base + d]), dot);
    }
    const float z = wave_sum(dot) * a.scale;
    const float m_new = fmaxf(m, z);
    const float alpha = expf(m - m_new);  // 0 on the first position
    const float p = expf(z - m_new);
    l = l * alpha + p;
#pragma unroll
    for (int k = 0; k < kMaxPerLane; ++k) {
      const int d = lane + 64 * k;
      const float v = d < D ? to_float(vc[base + d]) : 0.f;
      acc[k] = fmaf(p, v, acc[k] * alpha);
    }
    m = m_new;
  }
  const int64_t orow = static_cast<int64_t>(seq) * a.num_heads + h;
  if (a.partition_size > 0) {
    const int64_t pidx = orow * a.max_partitions + part;
#pragma unroll
    for (int k = 0; k < kMaxPerLane; ++k) {
      const int d = lane + 64 * k;
      if (d < D) a.tmp_out[pidx * D + d] = l > 0.f ? acc[k] / l : 0.f;
    }
    if (lane == 0) {
      a.max_logits[pidx] = m;
      a.exp_sums[pidx] = l;
    }
  } else {
#pragma unroll
    for (int k = 0; k < kMaxPerLane; ++k) {
      const int d = lane + 64 * k;
      if (d < D) a.out[orow * D + d] = l > 0.f ? acc[k] / l : 0.f;
    }
  }
}

// Merge of split partials: one 256-thread workgroup per (sequence, head).
// Every slot with l_p > 0 takes part (a real partial has l_p >= 1: its
// largest score contributes e^0); unused slots carry l_p = 0. The weights
// w_p = l_p e^{m_p - M} are computed once per slot (all threads in parallel)
// and staged in LDS in chunks; each wave then accumulates every 4th used slot
// over all dims (lane owns dims lane + 64k, coalesced 4-byte rows), and the
// four waves' sums meet in LDS.
constexpr int kRedThreads = 256;
constexpr int kRedChunk = 2048;

__global__ __launch_bounds__(kRedThreads) void reduce_kernel(
    float* __restrict__ out, const float* __restrict__ max_logits,
    const float* __restrict__ exp_sums, const float* __restrict__ tmp_out,
    const int32_t* __restrict__ context_lens, int num_heads, int head_size,
    int max_partitions) {
  __shared__ float s_w[kRedChunk];
  __shared__ float s_red[kRedThreads / 64];
  __shared__ float s_acc[kRedThreads / 64][kMaxPerLane * 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int h = blockIdx.x;
  const int seq = blockIdx.y;
  const int D = head_size;
  const int64_t orow = static_cast<int64_t>(seq) * num_heads + h;
  const int n = context_lens[seq] > 0 ? max_partitions : 0;
  const float* __restrict__ m = max_logits + orow * max_partitions;
  const float* __restrict__ l = exp_sums + orow * max_partitions;
  const float* __restrict__ o = tmp_out + orow * max_partitions * D;

  float mx = -INFINITY;
  for (int p = tid; p < n; p += kRedThreads)
    if (l[p] > 0.f) mx = fmaxf(mx, m[p]);
  mx = wave_max(mx);
  if (lane == 0) s_red[w] = mx;
  __syncthreads();
  float M = s_red[0];
#pragma unroll
  for (int i = 1; i < kRedThreads / 64; ++i) M = fmaxf(M, s_red[i]);

  float acc[kMaxPerLane] = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  for (int c0 = 0; c0 < n; c0 += kRedChunk) {
    const int cn = n - c0 < kRedChunk ? n - c0 : kRedChunk;
    __syncthreads();  // previous chunk's weights are no longer read
    for (int p = tid; p < cn; p += kRedThreads) {
      const float lp = l[c0 + p];
      const float wp = lp > 0.f ? lp * expf(m[c0 + p] - M) : 0.f;
      s_w[p] = wp;
      den += wp;
    }
    __syncthreads();
#pragma unroll 4
    for (int p = w; p < cn; p += kRedThreads / 64) {
      const float wp = s_w[p];
      if (wp == 0.f) continue;  // unused slot: its row is never read
      const float* __restrict__ row = o + static_cast<int64_t>(c0 + p) * D;
#pragma unroll
      for (int k = 0; k < kMaxPerLane; ++k) {
        const int d = lane + 64 * k;
        if (d < D) acc[k] = fmaf(wp, row[d], acc[k]);
      }
    }
  }
  den = wave_sum(den);
  __syncthreads();
  if (lane == 0) s_red[w] = den;
#pragma unroll
  for (int k = 0; k < kMaxPerLane; ++k) s_acc[w][lane + 64 * k] = acc[k];
  __syncthreads();
  float total = 0.f;
#pragma unroll
  for (int i = 0; i < kRedThreads / 64; ++i) total += s_red[i];
  for (int d = tid; d < D; d += kRedThreads) {
    float num = 0.f;
#pragma unroll
    for (int i = 0; i < kRedThreads / 64; ++i) num += s_acc[i][d];
    out[orow * D + d] = (n > 0 && total > 0.f) ? num / total : 0.f;
  }
}

}  // namespace

hipError_t launch_decode_generic(const DecodeArgs& a, hipStream_t stream) {
  dim3 grid(a.partition_size > 0 ? a.max_partitions : 1, a.num_heads, a.num_seqs);
  dim3 block(64);
  switch (a.dtype) {
    case 0: decode_generic_kernel<float><<<grid, block, 0, stream>>>(a); break;
    case 1: decode_generic_kernel<f16_t><<<grid, block, 0, stream>>>(a); break;
    default: decode_generic_kernel<bf16_t><<<grid, block, 0, stream>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_reduce(float* out, const float* max_logits, const float* exp_sums,
                         const float* tmp_out, const int32_t* context_lens, int num_seqs,
                         int num_heads, int head_size, int partition_size, int max_partitions,
                         hipStream_t stream) {
  dim3 grid(num_heads, num_seqs);
  (void)partition_size;
  reduce_kernel<<<grid, kRedThreads, 0, stream>>>(out, max_logits, exp_sums, tmp_out, context_lens,
                                                  num_heads, head_size, max_partitions);
  return hipGetLastError();
}

}  // namespace pkv
