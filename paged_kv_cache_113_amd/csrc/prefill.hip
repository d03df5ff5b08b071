// Multi-token queries over paged KV, long chunks (chunked prefill): the
// prefill kernel for gfx950.
//
// What it computes is the causal attention of paged_varlen_attention: token
// i of a sequence with ctx positions and q_s query tokens sits at position
// ctx - q_s + i and attends positions 0 .. ctx - q_s + i, softmax(scale q K^T)
// V over K/V rows found through the block table ("vLLM PagedAttention: from
// fragmentation to slot mapping", sections 3 and 7; a step mixing prefill
// chunks and decode tokens: "vLLM source walkthrough: PagedAttention and
// continuous batching", section 2.8).
//
// It takes the sequences whose query tokens fill at least kPrefillCols
// (token, head) columns per KV head. There q.K^T is a real dense contraction
// and the cost is in the matrix cores, the VALU softmax and re-reading K/V,
// so a workgroup of 4 waves loads each 64-position stage of K and V once into
// LDS and all 4 waves use it, each for 2 groups of 16 columns (128 columns
// per stage):
//  * unit = (sequence, 8 column groups of 16/G tokens x G heads); wave w owns
//    groups 2w and 2w + 1 of the unit;
//  * a stage arrives by in-LDS loads (global_load_lds_dwordx4, 1 KiB per
//    instruction) into one of two stage buffers while the other is computed;
//    rows are unpadded and swizzled against bank conflicts (K row r keeps
//    16-byte chunk c at c ^ (r % 16), V row r keeps 32-byte segment g at
//    g ^ (r % 8)); one barrier per stage;
//  * per stage and group: the scores of its 64 positions (four 16-row blocks
//    on v_mfma_f32_16x16x32; lane (col n, group j) gets positions
//    16b + 4j .. 16b + 4j + 3 of block b), one online-softmax step over the
//    lane's 16 positions, and P.V on v_mfma_f32_16x16x32 over the two
//    32-position halves with k running over exactly those positions: the
//    lane's own probabilities are the P^T operand (a 16-bit high part and the
//    rounding of the remainder), two transposed LDS reads give the V^T
//    operand, shared by both groups. The accumulators are rescaled only when
//    some column's running max moved by more than 2^8;
//  * work split: for each KV head the stream of all units' stages is cut into
//    equal ranges, one per workgroup (the decode kernel's balanced split at
//    workgroup granularity); a range ends a piece wherever a unit or the
//    range ends, and the reduce kernel merges the pieces (a unit done in one
//    piece writes its output rows itself).
#include <atomic>
#include <type_traits>

#include "device.h"
#include "launch.h"
#include "mfma_tile.h"
#include "varlen.h"

namespace pkv {
namespace {

constexpr int kPfThreads = 256;
constexpr int kPfWaves = kPfThreads / 64;
constexpr int kGroupsPerWave = 2;                          // 2 x 16 columns
constexpr int kGroupsPerUnit = kPfWaves * kGroupsPerWave;  // 128 columns
constexpr int kStage = 64;                                 // positions per stage
constexpr int kSub = kStage / kTile;                       // 16-row blocks per stage
constexpr int kStageBytes = kStage * kD * 2;               // K or V rows of a stage
constexpr int kPreInts = 4 * kStageBytes / 4;              // dynamic LDS ints before the prefix
constexpr int kMaxSeqsPrefill = 8192;                      // LDS prefix capacity
constexpr int kXcdCount = 8;                               // MI355X: 8 XCDs

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef float f32x2v __attribute__((ext_vector_type(2)));

// The running max a column's probabilities are taken against moves only when
// a score exceeds it by more than this (log2 units): probabilities then stay
// below 2^8, and the accumulators are rescaled only on such a move instead of
// whenever the max creeps up. The partial (max, sum, output) stays exact: the
// sum and the output are taken against the same reference.
constexpr float kLazyLog2 = 8.f;

// s_waitcnt vmcnt(0): every vector memory load issued so far has arrived.
__device__ __forceinline__ void wait_all_loads() {
  // gfx9 encoding: vmcnt [3:0] and [15:14] = 0, expcnt [6:4] and lgkmcnt
  // [11:8] at their maxima (not waited for)
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Two probabilities as their 16-bit roundings (high parts) and the 16-bit
// roundings of the remainders, each pair packed in one register: hi + lo is
// p to about 2^-16 relative (packed conversions, two values per instruction).
template <typename T>
__device__ __forceinline__ void split_pair(float a, float b, uint32_t& hi, uint32_t& lo) {
  const f32x2v x = {a, b};
  if constexpr (std::is_same<T, bf16_t>::value) {
    typedef __bf16 h2 __attribute__((ext_vector_type(2)));
    hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, h2));
    // a bf16 value is the top half of the float with the same bits
    const f32x2v hf = {__uint_as_float(hi << 16), __uint_as_float(hi & 0xffff0000u)};
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(x - hf, h2));
  } else {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 h = __builtin_convertvector(x, h2);
    hi = __builtin_bit_cast(uint32_t, h);
    lo = __builtin_bit_cast(uint32_t,
                            __builtin_convertvector(x - __builtin_convertvector(h, f32x2v), h2));
  }
}

// Maximum of two scores. The NaN-propagating form needs no quieting of its
// inputs (the IEEE-mode fmaxf does, one extra instruction per matrix-core
// result); no score that reaches it is NaN: positions a column must not see
// are replaced by -inf first.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float vmax_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float vmax_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// 8 probabilities in k order as a 16x16x32 operand pair (high parts, remainders).
template <typename T>
__device__ __forceinline__ void split_p8(const float* p, uint4& hi, uint4& lo) {
  split_pair<T>(p[0], p[1], hi.x, lo.x);
  split_pair<T>(p[2], p[3], hi.y, lo.y);
  split_pair<T>(p[4], p[5], hi.z, lo.z);
  split_pair<T>(p[6], p[7], hi.w, lo.w);
}

// A stage of the per-KV-head stream: stage t of the n stages of unit (s, u).
struct PfCursor {
  int s, u, nu, t, n, ctx, q0, qn;
};

// Stages a group of query tokens [u*per, min((u+1)*per, qn)) reads: what its
// last token sees, in 64-position stages, at least one.
__device__ __forceinline__ int unit_stages(int ctx, int qn, int u, int per) {
  const int e = (u + 1) * per < qn ? (u + 1) * per : qn;
  const int vis = ctx - qn + e;
  const int n = vis > 0 ? (vis + kStage - 1) / kStage : 0;
  return n > 0 ? n : 1;
}

template <typename T>
__global__ __launch_bounds__(kPfThreads) void prefill_split_kernel(DecodeArgs a, int wgs_per_kv) {
  // dynamic LDS: two stage buffers (K rows, then V rows, kStageBytes each),
  // then the prefix [S + 1]: stages of units before sequence s
  extern __shared__ __attribute__((aligned(16))) int s_dyn[];
  __shared__ int s_max[kPfWaves];
  __shared__ int s_wsum[kPfWaves];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int S = a.num_seqs;
  const int G = a.num_heads / a.num_kv_heads;
  const int mp = a.max_partitions;
  const int cap = a.max_blocks * a.block_size;
  const int tpg = kTile / G;                // query tokens per column group
  const int utok = kGroupsPerUnit * tpg;    // query tokens per unit

  auto seq_ctx = [&](int s) {
    int c = read_only(a.context_lens + s);
    return c < cap ? c : cap;
  };
  auto units_of = [&](int qn) { return prefill_sized(qn, G) ? (qn + utok - 1) / utok : 0; };
  auto seq_stages = [&](int s, int& last) {
    const int ctx = seq_ctx(s);
    int q0, qn;
    query_rows(a, s, q0, qn);
    const int nu = units_of(qn);
    int tot = 0;
    last = 0;
    for (int u = 0; u < nu; ++u) {
      last = unit_stages(ctx, qn, u, utok);
      tot += last;
    }
    return tot;
  };

  // 1. stages per sequence and their exclusive prefix (every workgroup
  //    builds the same table)
  const int per = (S + kPfThreads - 1) / kPfThreads;
  const int s_lo = tid * per;
  int local = 0, nmax = 0;
  for (int i = 0; i < per; ++i) {
    const int s = s_lo + i;
    if (s < S) {
      int last;
      local += seq_stages(s, last);
      nmax = last > nmax ? last : nmax;
    }
  }
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  const int wave_total = __shfl(incl, 63, 64);
  int wmax = nmax;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const int y = __shfl_xor(wmax, off, 64);
    wmax = y > wmax ? y : wmax;
  }
  if (lane == 0) {
    s_wsum[w] = wave_total;
    s_max[w] = wmax;
  }
  __syncthreads();
  int base = 0, T1 = 0, n_max = 0;
#pragma unroll
  for (int i = 0; i < kPfWaves; ++i) {
    base += i < w ? s_wsum[i] : 0;
    T1 += s_wsum[i];
    n_max = s_max[i] > n_max ? s_max[i] : n_max;
  }
  {
    int run = base + incl - local;
    for (int i = 0; i < per; ++i) {
      const int s = s_lo + i;
      if (s < S) {
        s_dyn[kPreInts + s] = run;
        int last;
        run += seq_stages(s, last);
      }
    }
    if (tid == 0) s_dyn[kPreInts + S] = T1;
  }
  __syncthreads();
  T1 = __builtin_amdgcn_readfirstlane(T1);
  if (T1 == 0) return;

  // 2. this workgroup's KV head and range (workgroups numbered XCD by XCD:
  //    one XCD streams a contiguous run of ranges over all KV heads)
  const int n_wg = gridDim.x;
  const int xcd_rank = (blockIdx.x % kXcdCount) * (n_wg / kXcdCount) + blockIdx.x / kXcdCount;
  const int wg_rank = n_wg % kXcdCount == 0 ? xcd_rank : static_cast<int>(blockIdx.x);
  const int kvh = wg_rank % a.num_kv_heads;
  const int k = wg_rank / a.num_kv_heads;
  int64_t Wk = wgs_per_kv;
  n_max = __builtin_amdgcn_readfirstlane(n_max);
  if (mp >= 2) {
    const int q_min = n_max > 1 ? (n_max - 1 + mp - 2) / (mp - 1) : 1;
    const int64_t lim = T1 / q_min;
    Wk = Wk < lim ? Wk : lim;
  } else {
    Wk = 1;
  }
  Wk = Wk < 1 ? 1 : Wk;
  if (k >= Wk) return;  // the whole workgroup: no barrier is left waiting
  const int b0 = static_cast<int>(static_cast<int64_t>(k) * T1 / Wk);
  const int b1 = static_cast<int>(static_cast<int64_t>(k + 1) * T1 / Wk);
  const int len = b1 - b0;
  auto range_of = [&](int x) {
    return static_cast<int>(((static_cast<int64_t>(x) + 1) * Wk - 1) / T1);
  };
  auto pre = [&](int s) { return __builtin_amdgcn_readfirstlane(s_dyn[kPreInts + s]); };
  int lo = 0, hi = S - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pre(mid) <= b0) lo = mid; else hi = mid - 1;
  }
  auto open_seq = [&](int s) {
    PfCursor c;
    c.s = s;
    c.u = 0;
    c.t = 0;
    c.ctx = seq_ctx(s);
    query_rows(a, s, c.q0, c.qn);
    c.nu = units_of(c.qn);
    c.n = unit_stages(c.ctx, c.qn, 0, utok);
    return c;
  };
  PfCursor cur = open_seq(lo);
  int ustart = pre(lo);
  {
    int x = b0 - ustart;
    while (x >= cur.n && cur.u + 1 < cur.nu) {
      x -= cur.n;
      ustart += cur.n;
      ++cur.u;
      cur.n = unit_stages(cur.ctx, cur.qn, cur.u, utok);
    }
    cur.t = x;
  }
  int piece = k - range_of(ustart);
  auto advance = [&](const PfCursor& c) {
    PfCursor r = c;
    if (c.t + 1 < c.n) {
      r.t = c.t + 1;
      return r;
    }
    if (c.u + 1 < c.nu) {
      r.u = c.u + 1;
      r.t = 0;
      r.n = unit_stages(c.ctx, c.qn, r.u, utok);
      return r;
    }
    int s = c.s + 1;
    while (s < S - 1 && pre(s + 1) == pre(s)) ++s;  // sequences with no units here
    return open_seq(s);
  };

  // this lane's two columns: group 2w + gi of the unit, token (within the
  // unit) (2w + gi) * tpg + col / G, head col % G
  const int my_head = col % G;
  const bool my_col = col < tpg * G;
  auto token_of = [&](const PfCursor& c, int gi) {
    return c.u * utok + (kGroupsPerWave * w + gi) * tpg + col / G;
  };
  auto live = [&](const PfCursor& c, int gi) { return my_col && token_of(c, gi) < c.qn; };
  // a group with no live column in the wave: its math is skipped (uniform)
  auto group_live = [&](const PfCursor& c, int gi) {
    return c.u * utok + (kGroupsPerWave * w + gi) * tpg < c.qn;
  };

  const char* __restrict__ kc = static_cast<const char*>(a.k_cache);
  const char* __restrict__ vc = static_cast<const char*>(a.v_cache);
  const int64_t head_stride = static_cast<int64_t>(a.block_size) * kD * 2;
  const int64_t block_stride = head_stride * a.num_kv_heads;
  auto row_of = [&](int s) { return a.block_table + static_cast<int64_t>(s) * a.max_blocks; };
  // Stage buffers. Rows are 256 B with no padding (in-LDS loads write whole
  // 1 KiB runs), so bank conflicts are avoided by swizzles instead: K row r
  // keeps its 16-byte chunk c at chunk c ^ (r % 16), which spreads the 16
  // rows of an A-operand read over all banks; V row r keeps its 32-byte
  // segment g at segment g ^ (r % 8), which does the same for the eight rows
  // of a transposed read.
  auto kbuf = [&](int par) { return (PKV_LDS char*)(s_dyn) + par * (2 * kStageBytes); };
  auto vbuf = [&](int par) { return (PKV_LDS char*)(s_dyn) + par * (2 * kStageBytes) + kStageBytes; };
  // The lane's byte offsets inside its 16-row block for the in-LDS loads:
  // instruction j, row r = 4 j + l / 16, the global chunk that the row's
  // swizzle keeps at LDS chunk l % 16.
  uint32_t kdo[4], vdo[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 4 * j + (lane >> 4);
    const int cs = lane & 15;
    kdo[j] = static_cast<uint32_t>(r * kD * 2 + ((cs ^ r) << 4));
    vdo[j] = static_cast<uint32_t>(r * kD * 2 + ((cs ^ ((r & 7) << 1)) << 4));
  }
  // The table entries of a stage. A power-of-two block size (the usual case)
  // turns the position -> entry division into a shift, and the at most four
  // consecutive entries the stage touches come in one scalar load (plus one
  // for the entry of this wave's 16-row block): this scalar work sits on
  // every stage's path. Entries are int32, so one unsigned compare against
  // min(num_blocks, 2^31 - 1) checks 0 <= entry < num_blocks.
  const int bsh = (a.block_size & (a.block_size - 1)) == 0 ? __builtin_ctz(a.block_size) : -1;
  const uint32_t nb32 = a.num_blocks < 0x7fffffff ? static_cast<uint32_t>(a.num_blocks)
                                                  : 0x7fffffffu;
  // Validity bits of the stage's four 16-row blocks (bit m: the block has a
  // table entry in the pool; if not, block 0 is read instead and its rows
  // are masked), the entry of block w and the offset of its first row inside
  // its block.
  auto stage_blocks = [&](const PfCursor& c, int& ok, int32_t& bw, int& in_block) {
    const int32_t* row = row_of(c.s);
    const int t0 = c.t * kStage;
    const int tw = t0 + w * kTile;
    if (bsh >= 0 && (t0 >> bsh) + 3 < a.max_blocks) {
      // t0 is a multiple of 64: of B too when B <= 64, and a larger block
      // holds the whole stage; so block m is entry (t0 >> log2 B) + (16 m >> log2 B)
      typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
      const i32x4 e = read_only(reinterpret_cast<const i32x4*>(row + (t0 >> bsh)));
      const int vb = (static_cast<uint32_t>(e.x) < nb32) | (static_cast<uint32_t>(e.y) < nb32) << 1 |
                     (static_cast<uint32_t>(e.z) < nb32) << 2 |
                     (static_cast<uint32_t>(e.w) < nb32) << 3;
      ok = 0;
#pragma unroll
      for (int m = 0; m < kSub; ++m) ok |= ((vb >> ((m * kTile) >> bsh)) & 1) << m;
      const int32_t ew = read_only(row + (tw >> bsh));
      bw = static_cast<uint32_t>(ew) < nb32 ? ew : -1;
      in_block = tw & (a.block_size - 1);
      return;
    }
    ok = 0;
    bw = -1;
#pragma unroll
    for (int m = 0; m < kSub; ++m) {
      const int64_t b = physical_block(row, t0 + m * kTile, a.block_size, a.max_blocks,
                                       a.num_blocks);
      ok |= (b >= 0) << m;
      if (m == w) bw = static_cast<int32_t>(b);  // a valid id is an int32 entry
    }
    in_block = tw % a.block_size;
  };
  // In-LDS loads of a stage into buffer par: wave w fills 16-row block w of
  // the stage (K and V, four 1 KiB load instructions each); lane l of
  // instruction j writes chunk l % 16 of block row 4j + l / 16, so it loads
  // the global chunk the row's swizzle puts there. Returns the blocks'
  // validity bits.
  auto dma_stage = [&](const PfCursor& c, PKV_LDS char* kd, PKV_LDS char* vd) {
    int ok, in_block;
    int32_t bw;
    stage_blocks(c, ok, bw, in_block);
    const int64_t mine = static_cast<int64_t>(bw < 0 ? 0 : bw) * block_stride +
                         kvh * head_stride + static_cast<int64_t>(in_block) * kD * 2;
    // a wave-uniform base plus the lane's fixed 32-bit offset: one add per
    // load, no per-lane offset arithmetic
    const char* kg = kc + mine;
    const char* vg = vc + mine;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int at = (kTile * w + 4 * j) * kD * 2;
      __builtin_amdgcn_global_load_lds(kg + kdo[j], (PKV_LDS void*)(kd + at), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(vg + vdo[j], (PKV_LDS void*)(vd + at), 16, 0, 0);
    }
    return ok;
  };
  // per-lane LDS offsets of the operand reads (rows of the first half of a
  // stage; the second half and the second 16-row block add 8 KiB and 4 KiB)
  int koff[4], voff[8];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) koff[kk] = col * (kD * 2) + (((grp + 4 * kk) ^ col) << 4);
  {
    const int vr = 4 * grp + (col >> 2);
#pragma unroll
    for (int db = 0; db < 8; ++db)
      voff[db] = vr * (kD * 2) + ((db ^ (vr & 7)) << 5) + (col & 3) * 8;
  }
  // wave-uniform V limit: positions the unit's last token sees, from the stage
  auto vlimit = [&](const PfCursor& c) {
    const int e = (c.u + 1) * utok < c.qn ? (c.u + 1) * utok : c.qn;
    return c.ctx - c.qn + e - c.t * kStage;
  };

  const float qk_scale = a.scale * kLog2e;
  uint4 q[kGroupsPerWave][4];
  auto load_q_unit = [&](const PfCursor& c) {
#pragma unroll
    for (int gi = 0; gi < kGroupsPerWave; ++gi) {
      const bool ok = live(c, gi);
      const char* qp = static_cast<const char*>(a.query) +
                       ((static_cast<int64_t>(c.q0 + token_of(c, gi)) * a.num_heads +
                         kvh * G + my_head) * kD) * 2;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        q[gi][kk] = ok ? *reinterpret_cast<const uint4*>(qp + (4 * kk + grp) * 16)
                       : make_uint4(0, 0, 0, 0);
    }
  };
  Attend<T> st[kGroupsPerWave];
#pragma unroll
  for (int gi = 0; gi < kGroupsPerWave; ++gi) st[gi].reset();

  // A unit done in a single piece writes its output rows itself and l = -1
  // into their first slot, which tells the merge to leave them alone.
  auto finish = [&](const PfCursor& c) {
    const bool single = piece == 0 && c.t == c.n - 1;
#pragma unroll
    for (int gi = 0; gi < kGroupsPerWave; ++gi) {
      const float l_col = st[gi].column_sum();
      if (live(c, gi)) {
        const int64_t prow = static_cast<int64_t>(c.q0 + token_of(c, gi)) * a.num_heads +
                             kvh * G + my_head;
        if (single) {
          const float inv = l_col > 0.f ? 1.f / l_col : 0.f;
          float* dst = a.out + prow * kD + 4 * grp;
#pragma unroll
          for (int db = 0; db < 8; ++db)
            *reinterpret_cast<float4*>(dst + 16 * db) =
                make_float4(st[gi].acc[db][0] * inv, st[gi].acc[db][1] * inv,
                            st[gi].acc[db][2] * inv, st[gi].acc[db][3] * inv);
          if (grp == 0) a.exp_sums[prow * mp] = -1.f;
        } else if (piece < mp) {
          const float inv = l_col > 0.f ? 1.f / l_col : 0.f;
          float* dst = a.tmp_out + (prow * mp + piece) * kD + 4 * grp;
#pragma unroll
          for (int db = 0; db < 8; ++db)
            *reinterpret_cast<float4*>(dst + 16 * db) =
                make_float4(st[gi].acc[db][0] * inv, st[gi].acc[db][1] * inv,
                            st[gi].acc[db][2] * inv, st[gi].acc[db][3] * inv);
          if (grp == 0) {
            a.max_logits[prow * mp + piece] = st[gi].m_run * kLn2;
            a.exp_sums[prow * mp + piece] = l_col;
          }
        }
        if (!single && c.t == c.n - 1 && grp == 0) {
          for (int p = piece + 1; p < mp; ++p) {
            a.max_logits[prow * mp + p] = -INFINITY;
            a.exp_sums[prow * mp + p] = 0.f;
          }
        }
      }
      st[gi].reset();
    }
    piece = 0;
  };

  // One stage of the staged buffers (kb_, vb_) for the first NG groups of
  // this wave (NG is 2, or 1 when the unit has no tokens for the second), in
  // three phases the compiler can overlap across groups: the scores of all
  // 64 positions (four 16-row blocks; lane (col n, group j) gets positions
  // 16b + 4j .. 16b + 4j + 3 of block b), one online-softmax step over the
  // lane's 16 positions, then P.V over the two 32-position halves. masked
  // (wave-uniform): the stage reaches past some column's causal limit or
  // misses a block; without it every position of the stage is visible to
  // every live column of the wave (dead columns, whose q is zero, compute
  // finite values that are never written).
  auto stage_math = [&](auto ng, bool masked, int ok, int stage0, const PKV_LDS char* kb_,
                        const PKV_LDS char* vb_) {
    constexpr int NG = decltype(ng)::value;
    // The matrix-core bursts run at raised wave priority: the other wave on
    // the SIMD then issues its softmax in their gaps (3.5 % faster on the
    // mixed step's chunks).
    __builtin_amdgcn_s_setprio(1);
    f32x4 S[NG][kSub];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // K operands of the half's two 16-row blocks: row 16 b + col, chunk 4 kk + grp
      uint4 ka[4], kb[4];
      const PKV_LDS char* kbase = kb_ + 32 * h * (kD * 2);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        ka[kk] = __builtin_bit_cast(uint4, *(const PKV_LDS u32x4v*)(kbase + koff[kk]));
        kb[kk] = __builtin_bit_cast(uint4, *(const PKV_LDS u32x4v*)(kbase + koff[kk] +
                                                                     16 * (kD * 2)));
      }
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        S[gi][2 * h] = Attend<T>::scores(ka, q[gi]);
        S[gi][2 * h + 1] = Attend<T>::scores(kb, q[gi]);
      }
    }
    uint4 p_hi[NG][2], p_lo[NG][2];
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      float s16[16];
      if (masked) {
        // this column sees positions < lim of the stage (relative to its start)
        const int lim = live(cur, gi) ? cur.ctx - cur.qn + token_of(cur, gi) + 1 - stage0 : 0;
#pragma unroll
        for (int b = 0; b < kSub; ++b) {
          const bool vb = (ok >> b) & 1;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            s16[4 * b + i] = (vb && kTile * b + 4 * grp + i < lim) ? S[gi][b][i] : -INFINITY;
        }
      } else {
#pragma unroll
        for (int b = 0; b < kSub; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i) s16[4 * b + i] = S[gi][b][i];
      }
      // the max is taken on the raw scores: scaling by qk_scale > 0 keeps it
      float m8[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) m8[i] = vmax(s16[i], s16[8 + i]);
      float mt = vmax(vmax(vmax(m8[0], m8[1]), vmax(m8[2], m8[3])),
                      vmax(vmax(m8[4], m8[5]), vmax(m8[6], m8[7])));
      mt = vmax_xor32(vmax_xor16(mt)) * qk_scale;
      const float m_old = st[gi].m_run;
      const bool move = mt > m_old + kLazyLog2;
      const float m_ref = move ? mt : m_old;
      st[gi].m_run = m_ref;
      // a column with no visible position yet keeps -inf
      const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
      const float alpha = move ? fast_exp2(m_old - m_use) : 1.f;
      float p[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) p[i] = fast_exp2(fmaf(s16[i], qk_scale, -m_use));
      float ps[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) ps[b] = (p[4 * b] + p[4 * b + 1]) + (p[4 * b + 2] + p[4 * b + 3]);
      st[gi].l_part = st[gi].l_part * alpha + ((ps[0] + ps[1]) + (ps[2] + ps[3]));
      // P of half h: blocks 2h and 2h + 1, the k order of the V^T operand
      split_p8<T>(p, p_hi[gi][0], p_lo[gi][0]);
      split_p8<T>(p + 8, p_hi[gi][1], p_lo[gi][1]);
      // a column with no max yet has nothing accumulated
      if (__any(move && m_old != -INFINITY)) {
#pragma unroll
        for (int db = 0; db < 8; ++db) st[gi].acc[db] *= alpha;
      }
    }
    // V^T operands of the 8 dim blocks: lane (d = col, group j) takes
    // positions 4j..4j+3 of each 16-row block (the same k order as P);
    // shared by the groups
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const PKV_LDS char* vbase = vb_ + 32 * h * (kD * 2);
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const s16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (PKV_LDS s16x4*)(vbase + voff[db]));
        const s16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (PKV_LDS s16x4*)(vbase + voff[db] + 16 * (kD * 2)));
        const uint2 u0 = __builtin_bit_cast(uint2, t0);
        const uint2 u1 = __builtin_bit_cast(uint2, t1);
        const uint4 vt = make_uint4(u0.x, u0.y, u1.x, u1.y);
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
          st[gi].acc[db] = mfma_k32<T>(vt, p_hi[gi][h], st[gi].acc[db]);
          st[gi].acc[db] = mfma_k32<T>(vt, p_lo[gi][h], st[gi].acc[db]);
        }
      }
    }
    // software pipeline: the transposed reads of the next dim block are in
    // flight while the matrix cores work on this one
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int k = 0; k < 15; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * NG, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * NG, 0);
    __builtin_amdgcn_s_setprio(0);
  };

  // 3. the range, one stage at a time, two LDS buffers: wait for this
  //    stage's in-LDS loads, barrier (every wave's loads of this stage have
  //    landed and every wave is done with the other buffer), the next
  //    stage's loads into the other buffer (in flight during this stage's
  //    math), then the math. V rows past what the unit sees, and rows of a
  //    block with no table entry, are zeroed first (one more barrier): P is 0
  //    there, and 0 * NaN would still be NaN.
  //    The next stage's loads and this stage's math go through restrict
  //    pointers of one function, so the compiler knows the in-LDS loads
  //    write the other buffer and does not make this stage's LDS reads wait
  //    for them.
  using Two = std::integral_constant<int, 2>;
  using One = std::integral_constant<int, 1>;
  auto stage_step = [&](PKV_LDS char* __restrict__ kd, PKV_LDS char* __restrict__ vd,
                        PKV_LDS char* __restrict__ ks, PKV_LDS char* __restrict__ vs,
                        const PfCursor& nx, bool more, int ok_now, int& okb) {
    if (more) okb = dma_stage(nx, kd, vd);
    const int vl = vlimit(cur);
    if (vl < kStage || ok_now != (1 << kSub) - 1) {
#pragma unroll
      for (int m = 0; m < kSub; ++m) {
        const int row = kTile * m + (tid >> 4);
        if (row >= vl || !((ok_now >> m) & 1))
          *(PKV_LDS u32x4v*)(vs + row * (kD * 2) + (tid & 15) * 16) = u32x4v{0u, 0u, 0u, 0u};
      }
      // the zeros are LDS writes: wait for those only (not for the next
      // stage's loads in flight), then meet the other waves
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      __builtin_amdgcn_s_barrier();
    }
    const int stage0 = cur.t * kStage;
    // the whole stage is visible to the wave's first token (the others see
    // more) and all its blocks are in the pool: no masking
    const int first_tok = cur.u * utok + kGroupsPerWave * w * tpg;
    const bool interior = ok_now == (1 << kSub) - 1 &&
                          stage0 + kStage <= cur.ctx - cur.qn + first_tok + 1;
    // groups are filled in order: the second has tokens only if the first does
    if (group_live(cur, 1)) {
      stage_math(Two(), !interior, ok_now, stage0, ks, vs);
    } else if (group_live(cur, 0)) {
      stage_math(One(), true, ok_now, stage0, ks, vs);
    }
  };
  load_q_unit(cur);
  int okb = dma_stage(cur, kbuf(0), vbuf(0));
  for (int i = 0; i < len; ++i) {
    const int par = i & 1;
    wait_all_loads();
    __syncthreads();
    const int ok_now = okb;
    const bool more = i + 1 < len;
    const PfCursor nx = more ? advance(cur) : cur;
    stage_step(kbuf(par ^ 1), vbuf(par ^ 1), kbuf(par), vbuf(par), nx, more, ok_now, okb);
    const bool unit_ends = cur.t + 1 >= cur.n;
    if (unit_ends || !more) finish(cur);
    if (more && unit_ends) {
      load_q_unit(nx);
      // once per unit: the q loads are waited for here, with the next
      // stage's (so no later wait has to count them)
      wait_all_loads();
    }
    cur = nx;
  }
}

// Resident workgroups per CU, per device and LDS size class, computed once.
constexpr int kPfMaxDevices = 64;
constexpr int kPfLdsClasses = 4;
inline int pf_lds_class(size_t dyn) {
  dyn -= 4 * static_cast<size_t>(kStageBytes);
  return dyn <= 2048 ? 0 : dyn <= 8192 ? 1 : dyn <= 16384 ? 2 : 3;
}
inline size_t pf_lds_class_bytes(int c) {
  const size_t b[kPfLdsClasses] = {2048, 8192, 16384, (kMaxSeqsPrefill + 1) * sizeof(int)};
  return 4 * static_cast<size_t>(kStageBytes) + b[c];
}

template <typename T>
hipError_t prefill_grid(int& cus, int& per_cu, size_t dyn) {
  static std::atomic<int> cache[kPfMaxDevices][kPfLdsClasses][2];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const int c = pf_lds_class(dyn);
  if (dev >= 0 && dev < kPfMaxDevices) {
    cus = cache[dev][c][0].load(std::memory_order_relaxed);
    per_cu = cache[dev][c][1].load(std::memory_order_relaxed);
    if (cus > 0 && per_cu > 0) return hipSuccess;
  }
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(prefill_split_kernel<T>),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(pf_lds_class_bytes(kPfLdsClasses - 1)));
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, prefill_split_kernel<T>,
                                                     kPfThreads, pf_lds_class_bytes(c));
  if (e != hipSuccess) return e;
  if (per_cu < 1) per_cu = 1;
  if (dev >= 0 && dev < kPfMaxDevices) {
    cache[dev][c][1].store(per_cu, std::memory_order_relaxed);
    cache[dev][c][0].store(cus, std::memory_order_relaxed);
  }
  return hipSuccess;
}

template <typename T>
hipError_t launch_prefill_t(const DecodeArgs& a, hipStream_t stream) {
  const size_t dyn = 4 * static_cast<size_t>(kStageBytes) +
                     static_cast<size_t>(a.num_seqs + 1) * sizeof(int);
  int cus = 0, per_cu = 0;
  hipError_t e = prefill_grid<T>(cus, per_cu, dyn);
  if (e != hipSuccess) return e;
  int64_t per_kv = static_cast<int64_t>(cus) * per_cu / a.num_kv_heads;
  if (per_kv < 1) per_kv = 1;
  const int64_t wgs = per_kv * a.num_kv_heads;
  prefill_split_kernel<T><<<dim3(static_cast<unsigned>(wgs)), dim3(kPfThreads), dyn, stream>>>(
      a, static_cast<int>(per_kv));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_fast(const DecodeArgs& a, hipStream_t stream) {
  return a.dtype == 2 ? launch_prefill_t<bf16_t>(a, stream) : launch_prefill_t<f16_t>(a, stream);
}

}  // namespace pkv
