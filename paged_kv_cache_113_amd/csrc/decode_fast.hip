// Paged decode attention, matrix-core path for gfx950 (CDNA4).
//
// What it computes: for each sequence s and query head h, softmax(scale *
// q K^T) V over the sequence's positions, where position t's K/V row sits in
// physical block table[t / B] at offset t % B ("vLLM PagedAttention: from
// fragmentation to slot mapping", sections 3 and 7). The paper-notes page
// shows that computing scores block by block and normalising once over all
// of them equals standard attention; here the normalisation is an online
// (running max / running sum) softmax, as FlashAttention-style tiling does
// (paper-notes page, FlashAttention vs PagedAttention).
//
// Work decomposition: one workgroup of NW waves per (sequence, KV head,
// partition). A partition is `partition_size` positions (split mode, the
// source-walkthrough page's V2 grid) or the whole context. Positions are
// processed in tiles of 16 consecutive positions = B/16 tiles per physical
// block; wave w takes tiles w, w+NW, ... and keeps its own running (m, l,
// acc); the waves merge through LDS at the end.
//
// Per tile (16 positions x 128 dims of one KV head, 4 KiB for 16-bit data):
//  * K: lane (row r = lane%16, group j = lane/16) loads 16 B of row r at dim
//    chunk 4*kk + j for kk = 0..3; each load instruction covers 16 rows x
//    64 contiguous bytes. Those registers are the A operand of four
//    v_mfma_f32_16x16x32 (bf16/f16): S = K_tile . Q^T, where Q^T (the B
//    operand, lane (col n = lane%16, group j) holding q[n] at the same dim
//    chunk) stays in registers for the whole workgroup. Column n is query head
//    kv*G + n; columns n >= G hold zeros. The dot-product order over dims is a
//    fixed permutation shared by both operands, so any k-ordering the matrix
//    core uses gives the same sum.
//  * S lands as lane (col n, group j), register i -> position 4j + i. The
//    tile max per column needs one in-lane max over i and two cross-group
//    swaps; exp2 of pre-scaled scores runs on v_exp_f32.
//  * V: lane (dim chunk c = lane%16, group j) loads 16 B of rows 4j + i
//    (i = 0..3), each load covering 4 rows x 256 contiguous bytes. The
//    probability of row 4j+i for head n lives in lane 16j + n of the same
//    16-lane DPP row, so `row_newbcast:n` broadcasts it and P.V accumulates in
//    fp32 on the VALU (P is never rounded to 16 bits).
#include <type_traits>

#include "device.h"
#include "launch.h"

namespace pkv {
namespace {

constexpr int kD = 128;     // head size of this path
constexpr int kTile = 16;   // positions per tile
constexpr int kWavesUnsplit = 4;  // waves per (sequence, KV head) without a split

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Broadcast lane N of each 16-lane row to the whole row (DPP row_newbcast).
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + N, 0xf, 0xf, false));
}

// max / sum of x over the lane pairs (l, l ^ 16) and (l, l ^ 32), returned in
// every lane. v_permlane{16,32}_swap exchange rows between two registers on
// the VALU; with both operands = x, the two results hold x of both rows.
__device__ __forceinline__ float max_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <typename T>
__device__ __forceinline__ f32x4 mfma_k32(uint4 a, uint4 b, f32x4 c) {
  if constexpr (std::is_same<T, bf16_t>::value) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

template <typename T>
__device__ __forceinline__ void widen8(uint4 w, float* f) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if constexpr (std::is_same<T, bf16_t>::value) {
      f[2 * k] = lo_bf16(u[k]);
      f[2 * k + 1] = hi_bf16(u[k]);
    } else {
      f[2 * k] = lo_f16(u[k]);
      f[2 * k + 1] = hi_f16(u[k]);
    }
  }
}

struct TileRegs {
  uint4 k[4];
  uint4 v[4];
};

__device__ __forceinline__ void load_tile(TileRegs& t, const char* __restrict__ kbase,
                                          const char* __restrict__ vbase, int k_off,
                                          int v_off) {
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    t.k[kk] = *reinterpret_cast<const uint4*>(kbase + k_off + kk * 64);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    t.v[i] = *reinterpret_cast<const uint4*>(vbase + v_off + i * 256);
}

// NW waves share one (sequence, KV head, partition) item and merge through
// LDS (NW = 4, used without a split), or each 64-lane workgroup is one item
// (NW = 1, used with a split: each wave owns a whole partition, so the
// serial start of an item -- length, table entry, first tile -- is paid once
// per partition, and no barrier is needed).
template <typename T, int GM, int NW>
__global__ __launch_bounds__(NW * 64) void decode_fast_kernel(DecodeArgs a) {
  const int lane = threadIdx.x & 63;
  // wave index, made visibly uniform so table reads become scalar loads
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15;  // K row / score column (head) / V dim chunk
  const int grp = lane >> 4;  // row group j

  // Item order: KV head fastest, then sequence, then partition. Workgroups
  // that run at the same time then read the KV heads of the same physical
  // blocks, which sit next to each other in the pool (Hkv * B * D contiguous
  // elements per block), and every sequence's first partitions go first.
  const int item = blockIdx.x;
  const int kvh = item % a.num_kv_heads;
  const int seq = (item / a.num_kv_heads) % a.num_seqs;
  const int part = item / (a.num_kv_heads * a.num_seqs);
  const int G = a.num_heads / a.num_kv_heads;
  const int B = a.block_size;

  int ctx = a.context_lens[seq];
  const int cap = a.max_blocks * B;
  ctx = ctx < cap ? ctx : cap;
  int lo = 0, hi = ctx;
  if (a.partition_size > 0) {
    lo = part * a.partition_size;
    if (lo >= ctx) return;  // this partition does not exist for this sequence
    hi = lo + a.partition_size < ctx ? lo + a.partition_size : ctx;
  }
  const int n_tiles = (hi - lo + kTile - 1) / kTile;
  const int my_n = n_tiles > w ? (n_tiles - w + NW - 1) / NW : 0;

  const int32_t* __restrict__ row = a.block_table + static_cast<int64_t>(seq) * a.max_blocks;
  const char* __restrict__ kc = static_cast<const char*>(a.k_cache);
  const char* __restrict__ vc = static_cast<const char*>(a.v_cache);
  const int64_t head_stride = static_cast<int64_t>(B) * kD * 2;        // bytes per (block, head)
  const int64_t block_stride = head_stride * a.num_kv_heads;           // bytes per block

  // Q^T operand: lane (col n, group j) holds q[n] dims of chunks 4*kk + j.
  uint4 qreg[4];
  {
    const char* qp = static_cast<const char*>(a.query) +
                     ((static_cast<int64_t>(seq) * a.num_heads + kvh * G + col) * kD) * 2;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      qreg[kk] = col < G ? *reinterpret_cast<const uint4*>(qp + (4 * kk + grp) * 16)
                         : make_uint4(0, 0, 0, 0);
    }
  }
  const float qk_scale = a.scale * kLog2e;  // scores kept in log2 units

  // lane offsets inside a 16-row tile (bytes)
  const int k_off = col * (kD * 2) + grp * 16;     // row col, chunk grp (+64 B per kk)
  const int v_off = (4 * grp) * (kD * 2) + col * 16;  // rows 4j.., chunk col (+256 B per i)

  float m_run = -INFINITY;  // running max of column `col` (log2 units)
  float l_part = 0.f;       // running sum over this lane's rows
  float acc[GM][8];
#pragma unroll
  for (int n = 0; n < GM; ++n)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[n][e] = 0.f;

  // Issue the loads of tile ti. Returns false when the table entry is outside
  // the pool: block 0 is loaded instead (in bounds) and the tile is masked.
  auto load = [&](TileRegs& t, int ti) -> bool {
    const int tok0 = lo + (w + NW * ti) * kTile;
    const int64_t blk = physical_block(row, tok0, B, a.max_blocks, a.num_blocks);
    const int64_t base = (blk < 0 ? 0 : blk) * block_stride + kvh * head_stride +
                         static_cast<int64_t>(tok0 % B) * kD * 2;
    load_tile(t, kc + base, vc + base, k_off, v_off);
    return blk >= 0;
  };

  auto process = [&](const TileRegs& t, int ti, bool good) {
    const int tok0 = lo + (w + NW * ti) * kTile;
    const int lim = good ? hi - tok0 : 0;  // rows >= lim are masked
    f32x4 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) S = mfma_k32<T>(t.k[kk], qreg[kk], S);
    float s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = (4 * grp + i < lim) ? S[i] * qk_scale : -INFINITY;
    float mt = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mt = max_xor32(max_xor16(mt));
    const float m_new = fmaxf(m_run, mt);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = fast_exp2(s[i] - m_use);
    l_part = l_part * alpha + ((p[0] + p[1]) + (p[2] + p[3]));

    // rescale, then accumulate P.V for this lane's dims
    static_for<0, GM>([&](auto nc) {
      constexpr int n = decltype(nc)::value;
      const float an = row_bcast<n>(alpha);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[n][e] *= an;
    });
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float vf[8];
      widen8<T>(t.v[i], vf);
      if (lim < kTile) {  // tail tile: masked rows may hold anything (NaN)
        const bool ok = 4 * grp + i < lim;
#pragma unroll
        for (int e = 0; e < 8; ++e) vf[e] = ok ? vf[e] : 0.f;
      }
      static_for<0, GM>([&](auto nc) {
        constexpr int n = decltype(nc)::value;
        const float pn = row_bcast<n>(p[i]);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[n][e] = fmaf(pn, vf[e], acc[n][e]);
      });
    }
  };

  // software pipeline: the next tile's loads are in flight while this one
  // is computed (two register sets, unrolled by two to avoid copies)
  // (every processed tile has either exactly one tile of loads issued after
  // it or none, on every path, so the wait before it is precise)
  TileRegs ta, tb;
  bool ga = true, gb = true;
  if (my_n > 0) ga = load(ta, 0);
  int ti = 0;
  for (; ti + 1 < my_n; ti += 2) {
    gb = load(tb, ti + 1);
    process(ta, ti, ga);
    if (ti + 2 < my_n) {
      ga = load(ta, ti + 2);
      process(tb, ti + 1, gb);
    } else {
      process(tb, ti + 1, gb);
    }
  }
  if (ti < my_n) process(ta, ti, ga);

  // merge the four row groups of this wave (same running max per column)
#pragma unroll
  for (int n = 0; n < GM; ++n)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[n][e] = sum_xor32(sum_xor16(acc[n][e]));
  l_part = sum_xor32(sum_xor16(l_part));

  const int64_t out_row0 = static_cast<int64_t>(seq) * a.num_heads + kvh * G;
  if constexpr (NW == 1) {
    // lane (0, n) holds column n's running max and sum; every lane holds
    // acc[n][dims 8*col..8*col+7] for all heads n
    static_for<0, GM>([&](auto nc) {
      constexpr int n = decltype(nc)::value;
      if (n < G) {
        const float ln = row_bcast<n>(l_part);
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = ln > 0.f ? acc[n][e] / ln : 0.f;
        float* dst = a.partition_size > 0
                         ? a.tmp_out + ((out_row0 + n) * a.max_partitions + part) * kD
                         : a.out + (out_row0 + n) * kD;
        if (grp == 0) {
          reinterpret_cast<float4*>(dst + col * 8)[0] = make_float4(o[0], o[1], o[2], o[3]);
          reinterpret_cast<float4*>(dst + col * 8)[1] = make_float4(o[4], o[5], o[6], o[7]);
        }
      }
    });
    if (a.partition_size > 0 && grp == 0 && col < G) {
      const int64_t pidx = (out_row0 + col) * a.max_partitions + part;
      a.max_logits[pidx] = m_run * kLn2;  // back to natural-log units
      a.exp_sums[pidx] = l_part;
    }
  } else {
    // merge the waves through LDS
    __shared__ float sm_m[NW][16];
    __shared__ float sm_l[NW][16];
    __shared__ float sm_acc[NW][GM][kD];
    if (grp == 0) {
      sm_m[w][col] = m_run;
      sm_l[w][col] = l_part;
#pragma unroll
      for (int n = 0; n < GM; ++n)
#pragma unroll
        for (int e = 0; e < 8; ++e) sm_acc[w][n][col * 8 + e] = acc[n][e];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * kD; idx += NW * 64) {
      const int n = idx / kD;
      const int d = idx % kD;
      float M = -INFINITY;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, sm_m[ww][n]);
      const float Mu = M == -INFINITY ? 0.f : M;
      float den = 0.f, num = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        const float f = fast_exp2(sm_m[ww][n] - Mu);
        den = fmaf(f, sm_l[ww][n], den);
        num = fmaf(f, sm_acc[ww][n][d], num);
      }
      const float o = den > 0.f ? num / den : 0.f;
      if (a.partition_size > 0) {
        const int64_t pidx = (out_row0 + n) * a.max_partitions + part;
        a.tmp_out[pidx * kD + d] = o;
        if (d == 0) {
          a.max_logits[pidx] = M * kLn2;  // back to natural-log units
          a.exp_sums[pidx] = den;
        }
      } else {
        a.out[(out_row0 + n) * kD + d] = o;
      }
    }
  }
}

template <typename T, int NW>
hipError_t launch_nw(const DecodeArgs& a, hipStream_t stream) {
  const int G = a.num_heads / a.num_kv_heads;
  const int parts = a.partition_size > 0 ? a.max_partitions : 1;
  const int64_t items = static_cast<int64_t>(a.num_seqs) * a.num_kv_heads * parts;
  dim3 grid(static_cast<unsigned>(items));
  dim3 block(NW * 64);
  if (G <= 1) decode_fast_kernel<T, 1, NW><<<grid, block, 0, stream>>>(a);
  else if (G <= 2) decode_fast_kernel<T, 2, NW><<<grid, block, 0, stream>>>(a);
  else if (G <= 4) decode_fast_kernel<T, 4, NW><<<grid, block, 0, stream>>>(a);
  else if (G <= 8) decode_fast_kernel<T, 8, NW><<<grid, block, 0, stream>>>(a);
  else decode_fast_kernel<T, 16, NW><<<grid, block, 0, stream>>>(a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  return a.partition_size > 0 ? launch_nw<T, 1>(a, stream) : launch_nw<T, kWavesUnsplit>(a, stream);
}

}  // namespace

bool fast_decode_supported(const DecodeArgs& a) {
  const int G = a.num_heads / a.num_kv_heads;
  const int64_t parts = a.partition_size > 0 ? a.max_partitions : 1;
  const int64_t items = static_cast<int64_t>(a.num_seqs) * a.num_kv_heads * parts;
  return (a.dtype == 1 || a.dtype == 2) && a.head_size == kD && a.block_size % kTile == 0 &&
         G >= 1 && G <= 16 && items <= 0x7fffffff;
}

hipError_t launch_decode_fast(const DecodeArgs& a, hipStream_t stream) {
  return a.dtype == 2 ? launch_t<bf16_t>(a, stream) : launch_t<f16_t>(a, stream);
}

}  // namespace pkv
