// Matrix-core tile math shared by the gfx950 attention kernels: scores of
// 16 positions x 16 query columns on v_mfma_f32_16x16x32, an online softmax
// in the MFMA output layout, and P.V on v_mfma_f32_16x16x16 with V^T read
// from LDS by ds_read_b64_tr_b16. Layouts and their derivation are described
// at the top of decode_fast.hip; the kernels differ only in where K and V
// come from (a wave's own registers, or a tile a workgroup shares in LDS).
#pragma once

#include <type_traits>

#include "device.h"

namespace pkv {
namespace {

constexpr int kD = 128;           // head size of this path
constexpr int kTile = 16;         // positions per tile
// One wave's V tile in LDS: 16 rows of 256 B, each padded to 288 B so that
// the 16 rows of a transpose read start 8 banks apart (a 2-way pattern, the
// minimum for 512 B) and every access is a lane base plus an immediate.
constexpr int kSlotRow = kD * 2 + 32;
constexpr int kSlotBytes = kTile * kSlotRow;

#define PKV_LDS __attribute__((address_space(3)))

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

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
__device__ __forceinline__ f32x4 mfma_k16(uint2 a, uint2 b, f32x4 c) {
  if constexpr (std::is_same<T, bf16_t>::value) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
  }
}

// p (four probabilities in [0, 1]) as a 16-bit high part and the 16-bit
// rounding of the remainder: hi + lo = p to about 2^-16 relative.
template <typename T>
__device__ __forceinline__ void split_p(const float* p, uint2& hi, uint2& lo) {
  uint16_t h[4], r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (std::is_same<T, bf16_t>::value) {
      const __bf16 a = static_cast<__bf16>(p[i]);
      const __bf16 b = static_cast<__bf16>(p[i] - static_cast<float>(a));
      h[i] = __builtin_bit_cast(uint16_t, a);
      r[i] = __builtin_bit_cast(uint16_t, b);
    } else {
      const _Float16 a = static_cast<_Float16>(p[i]);
      const _Float16 b = static_cast<_Float16>(p[i] - static_cast<float>(a));
      h[i] = __builtin_bit_cast(uint16_t, a);
      r[i] = __builtin_bit_cast(uint16_t, b);
    }
  }
  hi = make_uint2(h[0] | (uint32_t(h[1]) << 16), h[2] | (uint32_t(h[3]) << 16));
  lo = make_uint2(r[0] | (uint32_t(r[1]) << 16), r[2] | (uint32_t(r[3]) << 16));
}

struct TileRegs {
  uint4 k[4];
  uint4 v[4];
};

// Keeps the compiler from moving the next tile's loads below the wait for the
// current tile: the loads must be in flight while this tile is computed.
__device__ __forceinline__ void issue_fence() { __builtin_amdgcn_sched_barrier(0); }

// A column's reference max (log2 units) moves only when a score exceeds it
// by more than this: the probabilities then stay below 2^8, and the
// accumulators are rescaled only on such a move (a few tiles per piece)
// instead of on every tile. Sums and outputs are taken against the same
// reference, so the partial stays exact.
constexpr float kLazyRef = 8.f;

// Running softmax state of one wave: lane (col n, group j) keeps column n's
// reference max (m_run, see kLazyRef), its running max (m_max) and its
// partial sum over rows 4j..4j+3 against the reference, and acc[db][r] =
// O^T[16*db + 4j + r][n] (unnormalised, same reference), for 16 query
// columns.
template <typename T>
struct Attend {
  float m_run;
  float m_max;
  float l_part;
  f32x4 acc[8];

  __device__ __forceinline__ void reset() {
    m_run = -INFINITY;
    m_max = -INFINITY;
    l_part = 0.f;
#pragma unroll
    for (int db = 0; db < 8; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // The column's partial sum against its running max (the max itself):
  // l_ref 2^(m_run - m_max); 0 for a column with no position.
  __device__ __forceinline__ float sum_at_max(float l_ref) const {
    return m_max == -INFINITY ? 0.f : l_ref * fast_exp2(m_run - m_max);
  }

  // S^T tile = K_tile . Q^T: lane (col n, group j), register i -> position 4j + i.
  static __device__ __forceinline__ f32x4 scores(const uint4* k, const uint4* q) {
    f32x4 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) S = mfma_k32<T>(k[kk], q[kk], S);
    return S;
  }

  // Online softmax over one tile: rows >= slim get no weight in this lane's
  // column (slim may differ from column to column: a causal limit per query
  // token). Returns the tile's probabilities, the factor that rescales the
  // running sums, and (wave-uniform) whether any column's reference moved.
  __device__ __forceinline__ float softmax(const f32x4& S, int slim, float qk_scale, int grp,
                                           float* p, bool& moved) {
    float s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = (4 * grp + i < slim) ? S[i] * qk_scale : -INFINITY;
    float mt = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mt = max_xor32(max_xor16(mt));
    m_max = fmaxf(m_max, mt);
    // (from -inf any finite max moves the reference)
    const bool move = mt > m_run + kLazyRef;
    const float m_ref = move ? mt : m_run;
    const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
    const float alpha = move ? fast_exp2(m_run - m_use) : 1.f;
    m_run = m_ref;
    moved = __any(move);
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = fast_exp2(s[i] - m_use);
    l_part = l_part * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
    return alpha;
  }

  // V rows of a tile into a 16-row LDS slot; rows >= vlim become zeros (P is
  // 0 there, and 0 * NaN would still be NaN). Lane (chunk c, group j) holds
  // 16 B of rows 4j + i.
  static __device__ __forceinline__ void stage_v(const uint4* v, int vlim, int grp, int col,
                                                 PKV_LDS char* slot) {
    PKV_LDS char* wbase = slot + (4 * grp) * kSlotRow + col * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint4 x = v[i];
      if (vlim < kTile && 4 * grp + i >= vlim) x = make_uint4(0, 0, 0, 0);
      *(PKV_LDS u32x4*)(wbase + i * kSlotRow) = __builtin_bit_cast(u32x4, x);
    }
  }

  // acc = alpha * acc + V^T . P^T with V from an LDS slot (alpha is 1 in
  // every lane unless `moved`).
  __device__ __forceinline__ void pv(const float* p, float alpha, bool moved, int grp, int col,
                                     const PKV_LDS char* slot) {
    uint2 phi, plo;
    split_p<T>(p, phi, plo);
    if (moved) {
#pragma unroll
      for (int db = 0; db < 8; ++db) acc[db] *= alpha;
    }
    // lane (d = col, group j): positions 4j..4j+3 of dim 16*db + d, gathered by
    // the transpose read from row 4j + col/4, bytes 32*db + 8*(col%4)
    const PKV_LDS char* rbase = slot + (4 * grp + (col >> 2)) * kSlotRow + (col & 3) * 8;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const s16x4 vt = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (PKV_LDS s16x4*)(rbase + 32 * db));
      const uint2 a = __builtin_bit_cast(uint2, vt);
      acc[db] = mfma_k16<T>(a, phi, acc[db]);
      acc[db] = mfma_k16<T>(a, plo, acc[db]);
    }
  }

  // One tile of a wave's own stream: K and V in registers, V staged through
  // the wave's 4 KiB LDS slot. vlim is the wave-uniform limit over all
  // columns (>= every slim).
  __device__ __forceinline__ void tile(const TileRegs& t, const uint4* q, int slim, int vlim,
                                       float qk_scale, int grp, int col, PKV_LDS char* slot) {
    const f32x4 S = scores(t.k, q);
    float p[4];
    bool moved;
    const float alpha = softmax(S, slim, qk_scale, grp, p, moved);
    stage_v(t.v, vlim, grp, col, slot);
    pv(p, alpha, moved, grp, col, slot);
  }

  // Column sum of l over the four row groups, in every lane.
  __device__ __forceinline__ float column_sum() const {
    return sum_xor32(sum_xor16(l_part));
  }
};

}  // namespace
}  // namespace pkv
