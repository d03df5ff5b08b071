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

// Online softmax over positions [lo, hi) of one sequence for one query
// (q, D values, lane d = lane + 64k), reading KV head kvh. Table entries
// outside the pool are skipped.
template <typename T>
struct Positions {
  float m = -INFINITY, l = 0.f;
  float acc[kMaxPerLane] = {0.f, 0.f, 0.f, 0.f};

  __device__ void run(const DecodeArgs& a, const T* __restrict__ q, const int32_t* row,
                      int kvh, int lo, int hi, int lane) {
    const int D = a.head_size;
    const int B = a.block_size;
    const T* __restrict__ kc = static_cast<const T*>(a.k_cache);
    const T* __restrict__ vc = static_cast<const T*>(a.v_cache);
    float qv[kMaxPerLane];
#pragma unroll
    for (int k = 0; k < kMaxPerLane; ++k) {
      const int d = lane + 64 * k;
      qv[k] = d < D ? to_float(q[d]) : 0.f;
    }
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
  }

  // normalised output (0 when nothing was attended) into dst[0..D)
  __device__ void store(float* dst, int D, int lane) const {
#pragma unroll
    for (int k = 0; k < kMaxPerLane; ++k) {
      const int d = lane + 64 * k;
      if (d < D) dst[d] = l > 0.f ? acc[k] / l : 0.f;
    }
  }
};

template <typename T>
__global__ __launch_bounds__(64) void decode_generic_kernel(DecodeArgs a) {
  const int lane = threadIdx.x;
  const int part = blockIdx.x;
  const int h = blockIdx.y;
  const int seq = blockIdx.z;
  const int G = a.num_heads / a.num_kv_heads;
  const int kvh = h / G;
  const int D = a.head_size;

  int ctx = a.context_lens[seq];
  const int cap = a.max_blocks * a.block_size;
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
  const int32_t* __restrict__ row = a.block_table + static_cast<int64_t>(seq) * a.max_blocks;
  Positions<T> st;
  st.run(a, q, row, kvh, lo, hi, lane);
  const int64_t orow = static_cast<int64_t>(seq) * a.num_heads + h;
  if (a.partition_size > 0) {
    const int64_t pidx = orow * a.max_partitions + part;
    st.store(a.tmp_out + pidx * D, D, lane);
    if (lane == 0) {
      a.max_logits[pidx] = st.m;
      a.exp_sums[pidx] = st.l;
    }
  } else {
    st.store(a.out + orow * D, D, lane);
  }
}

// Multi-token queries, plain path: one wave per (query row, head). Row r
// belongs to the sequence s with query_start_loc[s] <= r < query_start_loc[s+1];
// as token i of that sequence it sits at position ctx - q_s + i and attends
// positions 0 .. ctx - q_s + i. A row no sequence claims gets 0.
template <typename T>
__global__ __launch_bounds__(64) void varlen_generic_kernel(DecodeArgs a) {
  const int lane = threadIdx.x;
  const int64_t unit = blockIdx.x;
  const int r = static_cast<int>(unit / a.num_heads);
  const int h = static_cast<int>(unit % a.num_heads);
  const int G = a.num_heads / a.num_kv_heads;
  const int D = a.head_size;
  const int32_t* qsl = a.query_start_loc;
  // largest s with qsl[s] <= r
  int lo = 0, hi = a.num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (read_only(qsl + mid) <= r) lo = mid; else hi = mid - 1;
  }
  const int s = lo;
  const int q0 = read_only(qsl + s);
  const int q1 = read_only(qsl + s + 1);
  int vis = 0;
  if (q0 <= r && r < q1) {
    int ctx = read_only(a.context_lens + s);
    const int cap = a.max_blocks * a.block_size;
    ctx = ctx < cap ? ctx : cap;
    vis = ctx - (q1 - q0) + (r - q0) + 1;
    vis = vis < 0 ? 0 : (vis > ctx ? ctx : vis);
  }
  const T* __restrict__ q = static_cast<const T*>(a.query) +
                            (static_cast<int64_t>(r) * a.num_heads + h) * D;
  const int32_t* __restrict__ row = a.block_table + static_cast<int64_t>(s) * a.max_blocks;
  Positions<T> st;
  st.run(a, q, row, h / G, 0, vis, lane);
  st.store(a.out + unit * D, D, lane);
}

// Merge of split partials: 16 lanes per (row, head) unit, four units per
// wave, four waves per workgroup, no LDS and no barrier. Every slot with
// l_p > 0 takes part (a real partial has l_p > 0); unused slots carry l_p = 0
// and their output rows are never read. A unit's lanes read its slots'
// (m, l) 16 at a time; a ballot gives the used ones, whose weights
// w_p = l_p e^{m_p - M} are broadcast inside the unit while its lanes
// accumulate their dims of o_p, four slots in flight per round. kVec: the
// head size is a multiple of 64 and each lane moves 16 B per 64 dims (dims
// 4j .. 4j + 3 + 64k); otherwise one float per 16 dims (dims j + 16k).
constexpr int kRedWaves = 4;
constexpr int kRedUnits = 4;    // units per wave
constexpr int kRedLanes = 16;   // lanes per unit
constexpr int kRedSlots = 4;    // slots in flight per round

__device__ __forceinline__ float unit_max(float v) {
#pragma unroll
  for (int off = kRedLanes / 2; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kRedLanes));
  return v;
}
__device__ __forceinline__ float unit_sum(float v) {
#pragma unroll
  for (int off = kRedLanes / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, kRedLanes);
  return v;
}

template <bool kVec>
__global__ __launch_bounds__(kRedWaves * 64) void reduce_kernel(
    float* __restrict__ out, const float* __restrict__ max_logits,
    const float* __restrict__ exp_sums, const float* __restrict__ tmp_out,
    const int32_t* __restrict__ context_lens, int num_seqs, int num_heads, int head_size,
    int max_partitions) {
  // per lane: kVec 4 float4 (D <= 256), else 16 floats (D <= 256)
  constexpr int kPer = 16;
  const int lane = threadIdx.x & 63;
  const int sub = lane >> 4;
  const int j = lane & (kRedLanes - 1);
  const int64_t total = static_cast<int64_t>(num_seqs) * num_heads;
  const int64_t first = (static_cast<int64_t>(blockIdx.x) * kRedWaves +
                         __builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) * kRedUnits;
  if (first >= total) return;  // the whole wave
  const int64_t unit = first + sub;
  const bool active = unit < total;
  const int64_t orow = active ? unit : first;  // = seq * num_heads + h
  const int seq = static_cast<int>(orow / num_heads);
  const int D = head_size;
  const int mp = max_partitions;
  const float* __restrict__ m = max_logits + orow * mp;
  const float* __restrict__ l = exp_sums + orow * mp;
  // without lengths every row takes part (multi-token queries: every query
  // row's pieces are written, unused ones with l = 0), except a row whose
  // work was a single piece: that piece wrote the output itself and marked
  // its first slot with l = -1
  const bool done = active && context_lens == nullptr && l[0] < 0.f;
  const int n = !active || done ? 0
                : (context_lens == nullptr || read_only(context_lens + seq) > 0) ? mp : 0;
  const float* __restrict__ o = tmp_out + orow * mp * D;

  float mx = -INFINITY;
  for (int p = j; p < n; p += kRedLanes)
    if (l[p] > 0.f) mx = fmaxf(mx, m[p]);
  const float M = unit_max(mx);

  float acc[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) acc[k] = 0.f;
  float den = 0.f;
  for (int c0 = 0; c0 < mp; c0 += kRedLanes) {  // uniform over the wave
    const int p = c0 + j;
    float wp = 0.f;
    if (p < n) {
      const float lp = l[p];
      wp = lp > 0.f ? lp * expf(m[p] - M) : 0.f;
    }
    den += wp;
    uint32_t used = static_cast<uint32_t>(__ballot(wp != 0.f) >> (kRedLanes * sub)) & 0xffffu;
    while (__any(used != 0u)) {
      int b[kRedSlots];
      float wb[kRedSlots];
#pragma unroll
      for (int u = 0; u < kRedSlots; ++u) {
        b[u] = used ? __builtin_ctz(used) : -1;
        used &= used ? used - 1u : 0u;
        wb[u] = __shfl(wp, kRedLanes * sub + (b[u] < 0 ? 0 : b[u]), 64);
      }
#pragma unroll
      for (int u = 0; u < kRedSlots; ++u) {
        const float* __restrict__ row = o + static_cast<int64_t>(c0 + (b[u] < 0 ? 0 : b[u])) * D;
        if constexpr (kVec) {
#pragma unroll
          for (int k = 0; k < kPer / 4; ++k) {
            const int d = 4 * j + 64 * k;
            if (b[u] >= 0 && d < D) {
              const float4 v = *reinterpret_cast<const float4*>(row + d);
              acc[4 * k + 0] = fmaf(wb[u], v.x, acc[4 * k + 0]);
              acc[4 * k + 1] = fmaf(wb[u], v.y, acc[4 * k + 1]);
              acc[4 * k + 2] = fmaf(wb[u], v.z, acc[4 * k + 2]);
              acc[4 * k + 3] = fmaf(wb[u], v.w, acc[4 * k + 3]);
            }
          }
        } else {
#pragma unroll
          for (int k = 0; k < kPer; ++k) {
            const int d = j + kRedLanes * k;
            if (b[u] >= 0 && d < D) acc[k] = fmaf(wb[u], row[d], acc[k]);
          }
        }
      }
    }
  }
  den = unit_sum(den);
  if (!active || done) return;
  const bool any = n > 0 && den > 0.f;
  float* __restrict__ dst = out + orow * D;
  if constexpr (kVec) {
#pragma unroll
    for (int k = 0; k < kPer / 4; ++k) {
      const int d = 4 * j + 64 * k;
      if (d < D)
        *reinterpret_cast<float4*>(dst + d) =
            any ? make_float4(acc[4 * k] / den, acc[4 * k + 1] / den, acc[4 * k + 2] / den,
                              acc[4 * k + 3] / den)
                : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  } else {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int d = j + kRedLanes * k;
      if (d < D) dst[d] = any ? acc[k] / den : 0.f;
    }
  }
}

// Merge with many slots per row: one wave per (row, head), so that the
// pieces of a long context (tens of them per row) are read with many loads
// in flight instead of a few per 16-lane unit. The wave reads 64 slots'
// (m, l) at a time; each output row o_p is read by D/4 lanes, 16 bytes each,
// so one load instruction covers 256/D slots, and eight of them are in
// flight per round. Sums are fp32 as in reduce_kernel (only their order
// differs).
template <int D>
__global__ __launch_bounds__(kRedWaves * 64) void reduce_row_kernel(
    float* __restrict__ out, const float* __restrict__ max_logits,
    const float* __restrict__ exp_sums, const float* __restrict__ tmp_out,
    const int32_t* __restrict__ context_lens, int num_seqs, int num_heads,
    int max_partitions) {
  constexpr int kLps = D / 4;      // lanes per slot row
  constexpr int kSps = 64 / kLps;  // slots per load instruction
  constexpr int kBatch = 8;        // load instructions in flight per round
  constexpr int kPick = kBatch * kSps;
  const int lane = threadIdx.x & 63;
  const int64_t total = static_cast<int64_t>(num_seqs) * num_heads;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kRedWaves +
                      __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (row >= total) return;  // the whole wave
  const int seq = static_cast<int>(row / num_heads);
  const int mp = max_partitions;
  const int n = (context_lens == nullptr || read_only(context_lens + seq) > 0) ? mp : 0;
  const float* __restrict__ m = max_logits + row * mp;
  const float* __restrict__ l = exp_sums + row * mp;
  // multi-token queries: a row done in a single piece (l = -1 in its first
  // slot) already holds its output (the whole wave)
  if (context_lens == nullptr && l[0] < 0.f) return;
  const float* __restrict__ o = tmp_out + row * mp * D;

  float mx = -INFINITY;
  for (int p = lane; p < n; p += 64)
    if (l[p] > 0.f) mx = fmaxf(mx, m[p]);
  const float M = wave_max(mx);

  const int my_s = lane / kLps;      // which of the instruction's slots
  const int my_d = 4 * (lane % kLps);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float den = 0.f;
  for (int c0 = 0; c0 < n; c0 += 64) {  // uniform over the wave
    const int p = c0 + lane;
    float wp = 0.f;
    if (p < n) {
      const float lp = l[p];
      wp = lp > 0.f ? lp * expf(m[p] - M) : 0.f;
    }
    den += wp;
    uint64_t used = __ballot(wp != 0.f);
    while (used) {
      // the next kPick used slots of the chunk, in order (-1: none)
      int pick[kPick];
#pragma unroll
      for (int i = 0; i < kPick; ++i) {
        pick[i] = used ? static_cast<int>(__builtin_ctzll(used)) : -1;
        used &= used ? used - 1 : 0;
      }
      int b[kBatch];
      float wb[kBatch];
      float4 v[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        int x = pick[k * kSps];
#pragma unroll
        for (int t = 1; t < kSps; ++t) x = my_s == t ? pick[k * kSps + t] : x;
        b[k] = x;
        wb[k] = __shfl(wp, x < 0 ? 0 : x, 64);
      }
#pragma unroll
      for (int k = 0; k < kBatch; ++k)
        v[k] = b[k] >= 0 ? *reinterpret_cast<const float4*>(o + static_cast<int64_t>(c0 + b[k]) * D + my_d)
                         : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const float w = b[k] >= 0 ? wb[k] : 0.f;
        acc.x = fmaf(w, v[k].x, acc.x);
        acc.y = fmaf(w, v[k].y, acc.y);
        acc.z = fmaf(w, v[k].z, acc.z);
        acc.w = fmaf(w, v[k].w, acc.w);
      }
    }
  }
  // lanes holding the same dims (one per slot of an instruction) add up
#pragma unroll
  for (int off = kLps; off < 64; off <<= 1) {
    acc.x += __shfl_xor(acc.x, off, 64);
    acc.y += __shfl_xor(acc.y, off, 64);
    acc.z += __shfl_xor(acc.z, off, 64);
    acc.w += __shfl_xor(acc.w, off, 64);
  }
  den = wave_sum(den);
  if (my_s != 0) return;
  const bool any = n > 0 && den > 0.f;
  *reinterpret_cast<float4*>(out + row * D + my_d) =
      any ? make_float4(acc.x / den, acc.y / den, acc.z / den, acc.w / den)
          : make_float4(0.f, 0.f, 0.f, 0.f);
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

hipError_t launch_varlen_generic(const DecodeArgs& a, hipStream_t stream) {
  const unsigned grid = static_cast<unsigned>(static_cast<int64_t>(a.num_tokens) * a.num_heads);
  switch (a.dtype) {
    case 0: varlen_generic_kernel<float><<<grid, 64, 0, stream>>>(a); break;
    case 1: varlen_generic_kernel<f16_t><<<grid, 64, 0, stream>>>(a); break;
    default: varlen_generic_kernel<bf16_t><<<grid, 64, 0, stream>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_reduce(float* out, const float* max_logits, const float* exp_sums,
                         const float* tmp_out, const int32_t* context_lens, int num_seqs,
                         int num_heads, int head_size, int partition_size, int max_partitions,
                         hipStream_t stream) {
  (void)partition_size;
  const int64_t units = static_cast<int64_t>(num_seqs) * num_heads;
  constexpr int per_block = kRedWaves * kRedUnits;
  const unsigned blocks = static_cast<unsigned>((units + per_block - 1) / per_block);
  // the float4 path needs 16-byte aligned rows
  const bool vec = head_size % 64 == 0 &&
                   ((reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(tmp_out)) & 15) == 0;
  // more slots than one 16-lane round covers: a wave per row
  if (vec && max_partitions > kRedLanes && (head_size == 64 || head_size == 128 ||
                                            head_size == 256)) {
    const unsigned rb = static_cast<unsigned>((units + kRedWaves - 1) / kRedWaves);
#define PKV_ROW(DD)                                                                          \
  reduce_row_kernel<DD><<<rb, kRedWaves * 64, 0, stream>>>(out, max_logits, exp_sums, tmp_out, \
                                                          context_lens, num_seqs, num_heads,  \
                                                          max_partitions)
    if (head_size == 64) PKV_ROW(64);
    else if (head_size == 128) PKV_ROW(128);
    else PKV_ROW(256);
#undef PKV_ROW
    return hipGetLastError();
  }
  if (vec)
    reduce_kernel<true><<<blocks, kRedWaves * 64, 0, stream>>>(
        out, max_logits, exp_sums, tmp_out, context_lens, num_seqs, num_heads, head_size,
        max_partitions);
  else
    reduce_kernel<false><<<blocks, kRedWaves * 64, 0, stream>>>(
        out, max_logits, exp_sums, tmp_out, context_lens, num_seqs, num_heads, head_size,
        max_partitions);
  return hipGetLastError();
}

}  // namespace pkv
