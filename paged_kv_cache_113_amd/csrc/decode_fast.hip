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
// Positions are processed in tiles of 16 consecutive positions (B/16 tiles
// per physical block). Per tile (16 positions x 128 dims of one KV head,
// 4 KiB of K and 4 KiB of V for 16-bit data), both products run on the
// matrix cores:
//  * K: lane (row r = lane%16, group j = lane/16) loads 16 B of row r at dim
//    chunk 4*kk + j for kk = 0..3; each load instruction covers 16 rows x
//    64 contiguous bytes. Those registers are the A operand of four
//    v_mfma_f32_16x16x32 (bf16/f16): S = K_tile . Q^T, where Q^T (the B
//    operand, lane (col n = lane%16, group j) holding q[n] at the same dim
//    chunk) stays in registers. Column n is query head kv*G + n; columns
//    n >= G hold zeros. The dot-product order over dims is a fixed
//    permutation shared by both operands, so any k-ordering the matrix core
//    uses gives the same sum.
//  * S lands as lane (col n, group j), register i -> position 4j + i. The
//    tile max per column needs one in-lane max over i and two cross-row
//    swaps (v_permlane{16,32}_swap); exp2 of pre-scaled scores runs on
//    v_exp_f32. The probabilities of lane (n, j) are exactly the B operand
//    (P^T, positions 4j..4j+3 of column n) of v_mfma_f32_16x16x16, split
//    into a 16-bit high part and a 16-bit remainder so that P keeps ~16
//    significant bits.
//  * V: lane (dim chunk c = lane%16, group j) loads 16 B of rows 4j + i
//    (i = 0..3), 4 rows x 256 contiguous bytes per load, and stores them in
//    the wave's LDS slot (rows padded to 288 B against bank conflicts).
//    ds_read_b64_tr_b16 then hands lane (d, j) the four
//    positions 4j..4j+3 of dim 16*db + d: the A operand (V^T) of the P.V
//    product, eight blocks db per tile, accumulated in fp32 as O^T[d][n].
//
// Two ways to share the work:
//  * whole context (no split): one 4-wave workgroup per (sequence, KV head),
//    waves take every 4th tile and merge through LDS (the single-pass "V1"
//    grid of the source-walkthrough page, section 1.8, per KV head);
//  * split (the "V2" partitions of the same section, balanced): a persistent
//    grid of exactly the resident waves. For each KV head the stream of all
//    sequences' tiles is cut into equal ranges, one per wave; a wave streams
//    its range without stopping, ending a piece (one partial) wherever a
//    sequence or its range ends. Waves with the same range and different KV
//    heads run side by side, so the KV heads of a physical block (contiguous
//    in the pool) are read at about the same time.
#include <atomic>
#include <type_traits>

#include "device.h"
#include "launch.h"
#include "mfma_tile.h"
#include "varlen.h"

namespace pkv {
namespace {

constexpr int kWavesUnsplit = 4;  // waves per (sequence, KV head) without a split
constexpr int kSplitThreads = 256;
constexpr int kMaxSeqsBalanced = 8192;  // LDS prefix capacity of the split kernel
constexpr int kXcds = 8;                // MI355X: 8 XCDs of 32 CUs

// Pool geometry and the lane's byte offsets inside a 16-row tile.
struct Geo {
  const char* __restrict__ kc;
  const char* __restrict__ vc;
  int64_t head_stride;   // bytes per (block, KV head) slab
  int64_t block_stride;  // bytes per block
  int B;
  int max_blocks;
  int64_t num_blocks;
  int k_off;  // row `col`, chunk `grp` (+64 B per kk)
  int v_off;  // rows 4*grp.., chunk `col` (+256 B per i)

  __device__ Geo(const DecodeArgs& a, int col, int grp)
      : kc(static_cast<const char*>(a.k_cache)),
        vc(static_cast<const char*>(a.v_cache)),
        head_stride(static_cast<int64_t>(a.block_size) * kD * 2),
        block_stride(static_cast<int64_t>(a.block_size) * kD * 2 * a.num_kv_heads),
        B(a.block_size),
        max_blocks(a.max_blocks),
        num_blocks(a.num_blocks),
        k_off(col * (kD * 2) + grp * 16),
        v_off((4 * grp) * (kD * 2) + col * 16) {}

  // Issue the loads of the tile starting at position tok0 of the sequence
  // whose table row is `row`. Returns false when the table entry is outside
  // the pool: block 0 is loaded instead (in bounds) and the caller masks it.
  __device__ __forceinline__ bool load(TileRegs& t, const int32_t* __restrict__ row, int tok0,
                                       int kvh) const {
    const int64_t blk = physical_block(row, tok0, B, max_blocks, num_blocks);
    const int64_t base = (blk < 0 ? 0 : blk) * block_stride + kvh * head_stride +
                         static_cast<int64_t>(tok0 % B) * kD * 2;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) t.k[kk] = stream_load(kc + base + k_off + kk * 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) t.v[i] = stream_load(vc + base + v_off + i * 256);
    return blk >= 0;
  }

};

// Q^T operand of (sequence seq, KV head kvh): lane (col n, group j) holds
// q[kvh*G + n] at dim chunks 4*kk + j; zero for n >= G.
__device__ __forceinline__ void load_q(uint4* q, const DecodeArgs& a, int seq, int kvh, int G,
                                       int col, int grp) {
  const char* qp = static_cast<const char*>(a.query) +
                   ((static_cast<int64_t>(seq) * a.num_heads + kvh * G + col) * kD) * 2;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    q[kk] = col < G ? *reinterpret_cast<const uint4*>(qp + (4 * kk + grp) * 16)
                    : make_uint4(0, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// whole context: 4 waves per (sequence, KV head)
// ---------------------------------------------------------------------------

template <typename T>
__global__ __launch_bounds__(kWavesUnsplit * 64) void decode_whole_kernel(DecodeArgs a) {
  constexpr int NW = kWavesUnsplit;
  // V slots during the tile loop; the waves' partial outputs afterwards
  __shared__ __attribute__((aligned(16))) char smem[NW * 16 * kD * 4];
  __shared__ float sm_m[NW][16];
  __shared__ float sm_l[NW][16];
  const int lane = threadIdx.x & 63;
  // wave index, made visibly uniform so table reads become scalar loads
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15;
  const int grp = lane >> 4;
  // KV head fastest: workgroups running together read the KV heads of the
  // same physical blocks, which are contiguous in the pool
  const int kvh = blockIdx.x % a.num_kv_heads;
  const int seq = blockIdx.x / a.num_kv_heads;
  const int G = a.num_heads / a.num_kv_heads;

  int ctx = read_only(a.context_lens + seq);
  const int cap = a.max_blocks * a.block_size;
  ctx = ctx < cap ? ctx : cap;
  const int n_tiles = ctx > 0 ? (ctx + kTile - 1) / kTile : 0;
  const int my_n = n_tiles > w ? (n_tiles - w + NW - 1) / NW : 0;
  const int32_t* __restrict__ row = a.block_table + static_cast<int64_t>(seq) * a.max_blocks;
  const Geo geo(a, col, grp);
  uint4 q[4];
  load_q(q, a, seq, kvh, G, col, grp);
  const float qk_scale = a.scale * kLog2e;
  PKV_LDS char* slot = (PKV_LDS char*)(smem) + w * kSlotBytes;

  Attend<T> st;
  st.reset();
  auto tok = [&](int ti) { return (w + NW * ti) * kTile; };

  // The next tile's loads are issued before this one is computed (two
  // register sets, unrolled by two). The last pair loads nothing ahead, and
  // the compiler's wait analysis, which also walks that path, waits for all
  // loads at the top of each pair: one tile in flight per wave, which at
  // this kernel's occupancy (several workgroups per CU) keeps HBM busy.
  // Issuing loads on every path (the last one redundant) gives exact waits
  // but measured about 5 % slower on 64 x 32-head MHA: the redundant tile
  // costs more than the deeper pipeline gains.
  TileRegs ta, tb;
  bool ga = true, gb = true;
  if (my_n > 0) ga = geo.load(ta, row, tok(0), kvh);
  int ti = 0;
  for (; ti + 1 < my_n; ti += 2) {
    gb = geo.load(tb, row, tok(ti + 1), kvh);
    issue_fence();
    st.tile(ta, q, ga ? ctx - tok(ti) : 0, ga ? ctx - tok(ti) : 0, qk_scale, grp, col, slot);
    if (ti + 2 < my_n) {
      ga = geo.load(ta, row, tok(ti + 2), kvh);
      issue_fence();
      st.tile(tb, q, gb ? ctx - tok(ti + 1) : 0, gb ? ctx - tok(ti + 1) : 0, qk_scale, grp,
              col, slot);
    } else {
      st.tile(tb, q, gb ? ctx - tok(ti + 1) : 0, gb ? ctx - tok(ti + 1) : 0, qk_scale, grp,
              col, slot);
    }
  }
  if (ti < my_n) st.tile(ta, q, ga ? ctx - tok(ti) : 0, ga ? ctx - tok(ti) : 0, qk_scale, grp, col, slot);
  const float l_col = st.column_sum();

  __syncthreads();  // every wave is done with its V slot
  float* sm_acc = reinterpret_cast<float*>(smem);  // [NW][16][kD]
  if (grp == 0) {
    sm_m[w][col] = st.m_run;
    sm_l[w][col] = l_col;
  }
#pragma unroll
  for (int db = 0; db < 8; ++db)
    *reinterpret_cast<float4*>(sm_acc + (w * 16 + col) * kD + 16 * db + 4 * grp) =
        make_float4(st.acc[db][0], st.acc[db][1], st.acc[db][2], st.acc[db][3]);
  __syncthreads();
  const int64_t out_row0 = static_cast<int64_t>(seq) * a.num_heads + kvh * G;
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
      num = fmaf(f, sm_acc[(ww * 16 + n) * kD + d], num);
    }
    a.out[(out_row0 + n) * kD + d] = den > 0.f ? num / den : 0.f;
  }
}

// ---------------------------------------------------------------------------
// split: persistent, balanced over tiles
// ---------------------------------------------------------------------------

// Stream units. Decode: one unit per sequence, its single query token in
// columns 0..G-1. Multi-token queries (kVar): a sequence's q_s tokens are cut
// into column groups of tpg = 16 / G tokens; column n of group c is token
// c*tpg + n / G, query head kv*G + n % G. Token i of a sequence with ctx
// positions sits at position ctx - q_s + i and sees positions 0 .. ctx - q_s + i
// (causal); a group's tiles cover what its last token sees, and each group
// re-reads the sequence's K/V from position 0. Sequences with enough query
// tokens to fill kPrefillCols columns are left to the prefill kernel.
//
// A tile of the per-KV-head stream: tile t of the n tiles of unit (s, c).
struct Cursor {
  int s, t, n, ctx;
  int c, nu;   // column group and groups of s (kVar; 0 and 1 for decode)
  int q0, qn;  // first query row of s and its query tokens (kVar)
};

// The merge of one (sequence, KV head) from its n > 1 pieces in the
// workspace, by one wave: rows s*Hq + kvh*G + r for r < G, slots p < n. Two
// rows per pass (one per 32-lane half), four dims of the row per lane:
//   M = max_p m_p, w_p = l_p e^{m_p - M}, out = sum_p w_p o_p / sum_p w_p
// (the log-sum-exp merge of paged_attention_reduce, summed in slot order).
// The pieces are read with device-scope loads (they may come from other
// XCDs), whose latency is long: lane q of a half holds (m, l) of slot
// c0 + q, and each batch of eight slots' rows is loaded before any is used.
__device__ __forceinline__ float half_max(float v) {
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 32));
  return v;
}
__device__ __forceinline__ float half_sum(float v) {
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) v += __shfl_xor(v, off, 32);
  return v;
}

__device__ __forceinline__ void merge_pieces(const DecodeArgs& a, int s, int kvh, int G, int mp,
                                             int n) {
  constexpr int kBatch = 8;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;
  const int q = lane & 31;
  for (int r0 = 0; r0 < G; r0 += 2) {
    // with an odd G the second half repeats the last row and stores nothing
    const int r = r0 + half < G ? r0 + half : G - 1;
    const int64_t row = static_cast<int64_t>(s) * a.num_heads + kvh * G + r;
    const float* m = a.max_logits + row * mp;
    const float* l = a.exp_sums + row * mp;
    const float* o = a.tmp_out + row * mp * kD + 4 * q;
    if (n <= kBatch) {
      // the common case: every load of the row in flight at once
      const int pq = q < n ? q : n - 1;
      const float mq = load_device(m + pq);
      const float lq = load_device(l + pq);
      float4 v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const float* op = o + static_cast<int64_t>(u < n ? u : n - 1) * kD;
        v[u] = make_float4(load_device(op), load_device(op + 1), load_device(op + 2),
                           load_device(op + 3));
      }
      const bool ok = q < n && lq > 0.f;
      const float Mh = half_max(ok ? mq : -INFINITY);
      const float w = ok ? lq * expf(mq - Mh) : 0.f;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const float wu = __shfl(w, (half << 5) + u, 64);
        if (u < n && wu != 0.f) {
          acc.x = fmaf(wu, v[u].x, acc.x);
          acc.y = fmaf(wu, v[u].y, acc.y);
          acc.z = fmaf(wu, v[u].z, acc.z);
          acc.w = fmaf(wu, v[u].w, acc.w);
        }
      }
      const float den = half_sum(w);
      if (r0 + half < G)
        *reinterpret_cast<float4*>(a.out + row * kD + 4 * q) =
            den > 0.f ? make_float4(acc.x / den, acc.y / den, acc.z / den, acc.w / den)
                      : make_float4(0.f, 0.f, 0.f, 0.f);
      continue;
    }
    // (m, l) of slot c0 + q, chunk by chunk; the first chunk is kept
    float m0 = -INFINITY, l0 = 0.f;
    float M = -INFINITY;
    for (int c0 = 0; c0 < n; c0 += 32) {
      const int p = c0 + q < n ? c0 + q : n - 1;
      const float mq = load_device(m + p);
      const float lq = load_device(l + p);
      const bool ok = c0 + q < n && lq > 0.f;
      if (ok) M = fmaxf(M, mq);
      if (c0 == 0) {
        m0 = ok ? mq : -INFINITY;
        l0 = ok ? lq : 0.f;
      }
    }
    M = half_max(M);
    float den = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int c0 = 0; c0 < n; c0 += 32) {
      float mq = m0, lq = l0;
      if (c0 > 0) {
        const int p = c0 + q < n ? c0 + q : n - 1;
        mq = load_device(m + p);
        lq = load_device(l + p);
        if (!(c0 + q < n && lq > 0.f)) {
          mq = -INFINITY;
          lq = 0.f;
        }
      }
      const float w = lq > 0.f ? lq * expf(mq - M) : 0.f;
      den += w;
      const int cn = n - c0 < 32 ? n - c0 : 32;
      for (int b = 0; b < cn; b += kBatch) {
        float4 v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int p = c0 + b + u < n ? c0 + b + u : n - 1;
          const float* op = o + static_cast<int64_t>(p) * kD;
          v[u] = make_float4(load_device(op), load_device(op + 1), load_device(op + 2),
                             load_device(op + 3));
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const float wu = __shfl(w, (half << 5) + ((b + u) & 31), 64);
          if (b + u < cn && wu != 0.f) {
            acc.x = fmaf(wu, v[u].x, acc.x);
            acc.y = fmaf(wu, v[u].y, acc.y);
            acc.z = fmaf(wu, v[u].z, acc.z);
            acc.w = fmaf(wu, v[u].w, acc.w);
          }
        }
      }
    }
    den = half_sum(den);
    if (r0 + half < G)
      *reinterpret_cast<float4*>(a.out + row * kD + 4 * q) =
          den > 0.f ? make_float4(acc.x / den, acc.y / den, acc.z / den, acc.w / den)
                    : make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

// After a wave has written all its pieces: every sequence its range
// [b0, b1) of the stream touched got one piece from it. For each such
// sequence cut into n > 1 pieces, count the arrival; the wave whose arrival
// is the n-th merges the sequence's pieces for its KV head and sets the
// counter back to 0 for the next call. Pieces are stored at device scope
// (written through the XCD's cache) and the wave waits for its stores
// before it counts; the merging wave reads them with device-scope loads
// after its count, so it sees every piece whichever XCD wrote it. (A cache
// write-back and invalidate per wave instead cost more than the merge
// saves.)
template <typename PiecesOf>
__device__ __forceinline__ void merge_arrivals(const DecodeArgs& a, const int* s_pre, int S,
                                               int lo, int b0, int b1, int kvh, int G, int mp,
                                               PiecesOf pieces_of) {
  const int lane = threadIdx.x & 63;
  auto pre = [&](int s) { return __builtin_amdgcn_readfirstlane(s_pre[s]); };
  // the pieces' stores were issued as instructions the compiler does not
  // track: wait for all of them explicitly
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  // the range's sequences, 64 at a time: lane i counts the arrival for
  // sequence s0 + i (all counts in flight together), then the wave merges
  // the sequences whose count it completed
  for (int s0 = lo; s0 < S && pre(s0) < b1; s0 += 64) {
    const int s = s0 + lane;
    bool last = false;
    int n = 0;
    if (s < S) {
      const int t0 = s_pre[s], t1 = s_pre[s + 1];
      if (t0 < b1 && t1 > b0 && t1 > t0) {
        n = pieces_of(s, t0, t1);
        if (n > 1) {
          int32_t* ctr = a.counters + static_cast<int64_t>(s) * a.num_kv_heads + kvh;
          last = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                 n - 1;
          if (last) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    uint64_t mine = __ballot(last);
    while (mine) {
      const int i = static_cast<int>(__builtin_ctzll(mine));
      mine &= mine - 1;
      merge_pieces(a, s0 + i, kvh, G, mp, __shfl(n, i, 64));
    }
  }
}

// Blocks shared by several sequences (a common prompt prefix, the branches
// of a forked sequence: glossary page, shared prefix; nxmr.cn article,
// section 4) sit at the same logical index of each sharer's table. The
// split kernel finds them in its prologue by the sequences' first blocks (a
// hash in LDS): for each first block held by more than one sequence, the
// shared run is the leading blocks the lowest-numbered holder and another
// holder have in common. Before the stream starts, the workgroups of each
// XCD read every line of those runs once with plain loads, so that the lines
// sit in that XCD's cache when the sharers' non-temporal stream reaches them.
constexpr int kShareSlotBytes = 16;   // hash slot: key, lowest holder, count / run, highest
__device__ __forceinline__ uint32_t share_hash(int32_t b, int bits) {
  return (static_cast<uint32_t>(b) * 2654435761u) >> (32 - bits);
}

// Largest i in [0, n) with v[i] <= x, for v nondecreasing with v[0] <= x
// (a prefix table in LDS), found by the whole wave: each round every lane
// compares one of 64 evenly spaced entries, and the ballot (a prefix of the
// lanes, v being sorted) narrows the interval to one step. Two rounds for up
// to 4096 entries. The result is wave-uniform.
__device__ __forceinline__ int last_le(const int* v, int n, int64_t x) {
  const int lane = threadIdx.x & 63;
  int lo = 0, hi = n;  // the answer lies in [lo, hi)
  while (hi - lo > 1) {
    const int step = (hi - lo + 63) / 64;
    const int i = lo + lane * step;
    const bool le = i < hi && v[i] <= x;
    const int cnt = __popcll(__ballot(le));  // >= 1: v[lo] <= x
    lo += (cnt - 1) * step;
    hi = lo + step < hi ? lo + step : hi;
  }
  return lo;
}

template <typename T, bool kVar>
__global__ __launch_bounds__(kSplitThreads) void decode_split_kernel(DecodeArgs a,
                                                                     int waves_per_kv,
                                                                     int stage_bytes,
                                                                     int share_bits) {
  // dynamic LDS: the tile prefix [S + 1], then one staging area of
  // stage_bytes per wave for finished pieces
  extern __shared__ __attribute__((aligned(16))) int s_pre[];  // [S + 1]: tiles before sequence s
  __shared__ __attribute__((aligned(16))) char s_slots[(kSplitThreads / 64) * kSlotBytes];
  __shared__ int s_max[kSplitThreads / 64];
  __shared__ int s_wsum[kSplitThreads / 64];
  __shared__ int s_ngroups;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int S = a.num_seqs;
  const int G = a.num_heads / a.num_kv_heads;
  const int mp = a.max_partitions;
  const int cap = a.max_blocks * a.block_size;
  const int tpg = kVar ? kTile / G : 1;  // query tokens per column group
  // decode merged in this launch: pieces still go to the workspace, the wave
  // that delivers a sequence's last piece (per KV head) merges them into out
  const bool fused = !kVar && a.counters != nullptr;

  auto seq_ctx = [&](int s) {
    int c = read_only(a.context_lens + s);
    return c < cap ? c : cap;
  };
  // query rows of sequence s, clamped to [0, num_tokens]
  auto seq_rows = [&](int s, int& q0, int& qn) {
    if constexpr (kVar) {
      query_rows(a, s, q0, qn);
    } else {
      q0 = s;
      qn = 1;
    }
  };
  // column groups of a sequence; none for those the prefill kernel takes
  auto groups_of = [&](int qn) {
    if constexpr (kVar) return prefill_sized(qn, G) ? 0 : (qn + tpg - 1) / tpg;
    return 1;
  };
  auto unit_tiles = [&](int ctx, int qn, int c) {
    if constexpr (kVar) return group_tiles(ctx, qn, c, tpg);
    return ctx > 0 ? (ctx + kTile - 1) / kTile : 0;
  };
  // tiles of all units of sequence s, and of its largest (last) unit
  auto seq_tiles = [&](int s, int& last) {
    const int ctx = seq_ctx(s);
    int q0, qn;
    seq_rows(s, q0, qn);
    const int nu = groups_of(qn);
    int tot = 0;
    last = 0;
    for (int c = 0; c < nu; ++c) {
      last = unit_tiles(ctx, qn, c);
      tot += last;
    }
    return tot;
  };

  // 1. tiles per sequence and their exclusive prefix (every workgroup builds
  //    the same table; it is tiny next to the KV stream). Each sequence's
  //    tile count waits in its prefix entry until the scan is done; its first
  //    block (for the shared-block detection further down) is read in the
  //    same pass and kept in the staging areas, which are free until the
  //    stream starts.
  // (with shared-block detection a second prefix, of costs, follows the
  // first: see step 3)
  const int pre_ints = (S + 1 + 3) & ~3;
  int* s_cost = s_pre + pre_ints;
  char* stage_base = reinterpret_cast<char*>(s_pre + pre_ints * (share_bits > 0 ? 2 : 1));
  int* first_of = reinterpret_cast<int*>(stage_base);
  // first-block hash: slot = {first block, lowest holder, holders, highest
  // holder}, then the list of the slots held more than once
  const int H = 1 << share_bits;
  int4* slots = reinterpret_cast<int4*>(reinterpret_cast<char*>(first_of) +
                                        ((static_cast<int>(sizeof(int)) * S + 15) & ~15));
  int* groups = reinterpret_cast<int*>(slots + H);   // [n_groups]
  if (share_bits > 0) {
    for (int i = tid; i < H; i += kSplitThreads) slots[i] = make_int4(-1, 0x7fffffff, 0, -1);
    if (tid == 0) s_ngroups = 0;
  }
  const int per = (S + kSplitThreads - 1) / kSplitThreads;
  const int s_lo = tid * per;
  int local = 0, nmax = 0;
  for (int i = 0; i < per; ++i) {
    const int s = s_lo + i;
    if (s < S) {
      int last;
      const int n = seq_tiles(s, last);
      s_pre[s] = n;
      if (share_bits > 0)
        first_of[s] = read_only(a.block_table + static_cast<int64_t>(s) * a.max_blocks);
      local += n;
      nmax = last > nmax ? last : nmax;
    }
  }
  int incl = local;  // inclusive scan over the wave
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
  for (int i = 0; i < kSplitThreads / 64; ++i) {
    base += i < w ? s_wsum[i] : 0;
    T1 += s_wsum[i];
    n_max = s_max[i] > n_max ? s_max[i] : n_max;
  }
  {
    int run = base + incl - local;  // exclusive prefix of this thread's chunk
    for (int i = 0; i < per; ++i) {
      const int s = s_lo + i;
      if (s < S) {
        const int n = s_pre[s];
        s_pre[s] = run;
        run += n;
      }
    }
    if (tid == 0) s_pre[S] = T1;
  }
  if (fused && blockIdx.x == 0) {
    // sequences without positions get out = 0 (no piece will merge them)
    for (int i = 0; i < per; ++i) {
      const int s = s_lo + i;
      if (s < S && seq_ctx(s) <= 0) {
        float4* o = reinterpret_cast<float4*>(a.out + static_cast<int64_t>(s) * a.num_heads * kD);
        for (int x = 0; x < a.num_heads * kD / 4; ++x) o[x] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  }
  __syncthreads();
  if (T1 == 0) return;

  // 2. Shared runs (blocks several sequences hold at the same logical index,
  //    found by the sequences' first blocks: see share_hash): the groups are
  //    found in LDS, then each group's run is measured in the table.
  auto find_groups = [&]() -> int {
    if (share_bits == 0) return 0;
    for (int i = 0; i < per; ++i) {
      const int s = s_lo + i;
      if (s >= S) break;
      if (s_pre[s + 1] == s_pre[s]) continue;          // no positions
      const int32_t fb = first_of[s];
      if (fb < 0 || fb >= a.num_blocks) continue;
      int h = static_cast<int>(share_hash(fb, share_bits));
      while (true) {
        const int old = atomicCAS(&slots[h].x, -1, fb);
        if (old == -1 || old == fb) break;
        h = (h + 1) & (H - 1);
      }
      atomicMin(&slots[h].y, s);
      atomicMax(&slots[h].w, s);
      atomicAdd(&slots[h].z, 1);
    }
    __syncthreads();
    for (int h = tid; h < H; h += kSplitThreads)
      if (slots[h].z > 1) groups[atomicAdd(&s_ngroups, 1)] = h;
    __syncthreads();
    return s_ngroups;
  };
  const int n_wg = gridDim.x;
  const int n_groups = find_groups();
  const bool touched = n_groups > 0 && n_wg % kXcds == 0;
  if (touched) {
    // a group's run: the leading blocks its lowest and highest holders have
    // in common, within both contexts; one wave per group, 64 blocks
    // compared at a time (into .z, as -run - 1: the holder count is no
    // longer needed)
    for (int g = w; g < n_groups; g += kSplitThreads / 64) {
      const int h = groups[g];
      const int r0 = slots[h].y, r1 = slots[h].w;
      const int n0 = (seq_ctx(r0) + a.block_size - 1) / a.block_size;
      const int n1 = (seq_ctx(r1) + a.block_size - 1) / a.block_size;
      const int lim = n0 < n1 ? n0 : n1;
      const int32_t* row0 = a.block_table + static_cast<int64_t>(r0) * a.max_blocks;
      const int32_t* row1 = a.block_table + static_cast<int64_t>(r1) * a.max_blocks;
      int run = 0;
      for (int c0 = 0; c0 < lim; c0 += 64) {
        const int b = c0 + lane;
        bool same = false;
        if (b < lim) {
          const int32_t x0 = row0[b];
          same = x0 == row1[b] && x0 >= 0 && x0 < a.num_blocks;
        }
        const uint64_t diff = ~__ballot(same);
        if (diff != 0) {
          run = c0 + static_cast<int>(__builtin_ctzll(diff));
          break;
        }
        run = c0 + 64;
      }
      run = run < lim ? run : lim;
      if (lane == 0) slots[h].z = -run - 1;
    }
    __syncthreads();
  }
  // The shared runs' lines are touched now, well before this wave's first
  // tile loads go out, so that a wave whose range starts inside a shared run
  // finds them in its XCD's cache; the touches' own results are waited for
  // after the tile's loads are issued.
  constexpr int kTouch = 4;
  uint32_t sink = 0;
  uint32_t last_touch[kTouch] = {0u, 0u, 0u, 0u};
  auto touch_runs = [&](int n_groups) {
    if (n_groups > 0 && n_wg % kXcds == 0) {
      // every line of every run, spread over the workgroups of this XCD
      // (workgroup i runs on XCD i % 8)
      const int J = n_wg / kXcds;
      const int j = blockIdx.x / kXcds;
      const int lpb = a.block_size * kD * 2 / 128;           // lines per (block, head) slab
      const int64_t head_stride = static_cast<int64_t>(a.block_size) * kD * 2;
      const int64_t block_stride = head_stride * a.num_kv_heads;
      const int per_blk = a.num_kv_heads * 2 * lpb;          // lines per block, K and V
      // Four lines per thread per round: their table entries, then their
      // loads, all in flight together (plain loads, which keep the lines in
      // the XCD's cache). A round's values are summed in the next round, the
      // last round's after the first tile's loads are issued, so no wait
      // for them stands before those loads.
      for (int g = 0; g < n_groups; ++g) {
        const int h = groups[g];
        const int run = -slots[h].z - 1;
        const int32_t* row = a.block_table + static_cast<int64_t>(slots[h].y) * a.max_blocks;
        const int lines = run * per_blk;
        for (int e0 = j * kSplitThreads * kTouch + tid; e0 < lines;
             e0 += J * kSplitThreads * kTouch) {
          int32_t blk[kTouch];
#pragma unroll
          for (int u = 0; u < kTouch; ++u) {
            const int e = e0 + u * kSplitThreads;
            blk[u] = e < lines ? row[e / per_blk] : -1;
          }
#pragma unroll
          for (int u = 0; u < kTouch; ++u) {
            const int e = e0 + u * kSplitThreads;
            const int r = e % per_blk;
            const int hh = r / (2 * lpb);
            const int kv = (r / lpb) & 1;
            const bool ok = e < lines && blk[u] >= 0 && blk[u] < a.num_blocks;
            // (no branch around the load: the four stay in flight together;
            // a line out of range reads the pool's first line instead)
            const int64_t off = ok ? static_cast<int64_t>(blk[u]) * block_stride +
                                         hh * head_stride + static_cast<int64_t>(r % lpb) * 128
                                   : 0;
            sink += last_touch[u];
            last_touch[u] = *reinterpret_cast<const uint32_t*>(
                static_cast<const char*>(kv ? a.v_cache : a.k_cache) + off);
          }
        }
      }
    }
  };
  touch_runs(n_groups);

  // 3. The split balances work, not tiles. Without shared runs every tile
  //    is one unit. With them, a tile of a sharer's shared run costs 3 and
  //    any other tile 4: the runs are touched into each XCD's cache before
  //    the stream, and a wave reads such a tile in about three quarters of
  //    the time of a tile from HBM (0.84 against 1.12 us measured), so
  //    waves whose ranges hold shared tiles take more tiles. s_cost is the
  //    exclusive prefix of the costs per sequence (the shared tiles of a
  //    sequence lead it, so a sequence's cost and tile count give both).
  const bool weighted = touched && static_cast<int64_t>(T1) * 4 < 0x7fffffff;
  int64_t C = T1;
  if (weighted) {
    const int tiles_per_block = a.block_size / kTile;
    int lc = 0;
    for (int i = 0; i < per; ++i) {
      const int s = s_lo + i;
      if (s < S) {
        const int n = s_pre[s + 1] - s_pre[s];
        int sh = 0;
        const int32_t fb = first_of[s];
        if (n > 0 && fb >= 0 && fb < a.num_blocks) {
          int h = static_cast<int>(share_hash(fb, share_bits));
          while (slots[h].x != fb && slots[h].x != -1) h = (h + 1) & (H - 1);
          const int z = slots[h].x == fb ? slots[h].z : 1;
          sh = z < 0 ? (-z - 1) * tiles_per_block : 0;
          sh = sh < n ? sh : n;
        }
        s_cost[s] = 4 * n - sh;
        lc += 4 * n - sh;
      }
    }
    int ci = lc;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(ci, off, 64);
      if (lane >= off) ci += y;
    }
    if (lane == 63) s_wsum[w] = ci;
    __syncthreads();
    int cbase = 0, ctot = 0;
#pragma unroll
    for (int i = 0; i < kSplitThreads / 64; ++i) {
      cbase += i < w ? s_wsum[i] : 0;
      ctot += s_wsum[i];
    }
    int run = cbase + ci - lc;
    for (int i = 0; i < per; ++i) {
      const int s = s_lo + i;
      if (s < S) {
        const int c = s_cost[s];
        s_cost[s] = run;
        run += c;
      }
    }
    if (tid == 0) s_cost[S] = ctot;
    C = ctot;
    __syncthreads();
  }

  // 4. this wave's KV head and range of the stream. Workgroups are dealt to
  //    the 8 XCDs round-robin (workgroup i runs on XCD i % 8); numbering the
  //    waves XCD by XCD gives each XCD a contiguous run of ranges over all KV
  //    heads, so the heads of a block are read side by side on one XCD.
  //    Ranges hold at least q_min tiles so that no unit is cut into more
  //    than max_partitions pieces: a unit of n tiles meets at most
  //    ceil((n-1)/q_min) + 1 (weighted, a range of cost C/Wk >= 4 q_min
  //    holds at least q_min tiles: a tile costs at most 4).
  const int xcd_rank = (blockIdx.x % kXcds) * (n_wg / kXcds) + blockIdx.x / kXcds;
  const int wg_rank = n_wg % kXcds == 0 ? xcd_rank : static_cast<int>(blockIdx.x);
  const int gw = wg_rank * (kSplitThreads / 64) + w;
  const int kvh = gw % a.num_kv_heads;
  const int k = gw / a.num_kv_heads;
  int64_t Wk = waves_per_kv;
  if (mp >= 2) {
    const int q_min = n_max > 1 ? (n_max - 1 + mp - 2) / (mp - 1) : 1;
    const int64_t lim = weighted ? C / (4 * q_min) : T1 / q_min;
    Wk = Wk < lim ? Wk : lim;
  } else {
    Wk = 1;
  }
  Wk = Wk < 1 ? 1 : Wk;
  // waves past Wk have no range of their own: they take the last range's
  // bounds to stay well-formed, store nothing, and leave after the shared
  // runs' touches (whose barrier counts every wave of the workgroup)
  const bool active = k < Wk;
  const int kr = active ? k : static_cast<int>(Wk) - 1;

  // LDS reads come back in VGPRs; the prefix is the same for every lane, and
  // saying so keeps the cursor, table reads and tile addresses scalar
  auto pre = [&](int s) { return __builtin_amdgcn_readfirstlane(s_pre[s]); };
  auto cst = [&](int s) { return __builtin_amdgcn_readfirstlane(s_cost[s]); };
  // Range r covers the tiles whose cost starts in [floor(r C / Wk),
  // floor((r+1) C / Wk)); unweighted, a tile's cost start is its stream
  // index. The range holding cost c: the largest r with floor(r C/Wk) <= c.
  auto range_of_cost = [&](int64_t c) { return static_cast<int>(((c + 1) * Wk - 1) / C); };
  // cost start of tile t of a sequence (per lane: c0 = its cost prefix, n its
  // tiles, n_cost its cost; its shared tiles lead it)
  auto cost_in = [](int64_t c0, int n, int n_cost, int t) -> int64_t {
    const int sh = 4 * n - n_cost;
    return c0 + (t < sh ? 3 * t : 3 * sh + 4 * (t - sh));
  };
  // first stream tile whose cost starts at c or later (wave-uniform)
  auto tile_at = [&](int64_t c) -> int {
    if (!weighted) return static_cast<int>(c);
    if (c >= C) return T1;
    const int l = last_le(s_cost, S, c);  // a sequence with tiles
    const int n = pre(l + 1) - pre(l);
    const int sh = 4 * n - (cst(l + 1) - cst(l));
    const int r = static_cast<int>(c - cst(l));
    return pre(l) + (r <= 3 * sh ? (r + 2) / 3 : sh + (r - 3 * sh + 3) / 4);
  };
  const int b0 = tile_at(static_cast<int64_t>(kr) * C / Wk);
  const int b1 = tile_at(static_cast<int64_t>(kr + 1) * C / Wk);
  const int len = b1 - b0;  // >= 1: Wk <= T1, or C/Wk >= 4
  // sequence holding tile b0: largest s with s_pre[s] <= b0
  const int lo = last_le(s_pre, S, b0);
  auto open_seq = [&](int s) {
    Cursor c;
    c.s = s;
    c.t = 0;
    c.c = 0;
    c.ctx = seq_ctx(s);
    seq_rows(s, c.q0, c.qn);
    c.nu = groups_of(c.qn);
    c.n = unit_tiles(c.ctx, c.qn, 0);
    return c;
  };
  Cursor cur = open_seq(lo);
  int ustart = pre(lo);  // stream index of the first tile of cur's unit
  {
    int x = b0 - ustart;
    if constexpr (kVar) {
      while (x >= cur.n && cur.c + 1 < cur.nu) {
        x -= cur.n;
        ustart += cur.n;
        ++cur.c;
        cur.n = unit_tiles(cur.ctx, cur.qn, cur.c);
      }
    }
    cur.t = x;
  }
  // index of this wave's piece of the unit (weighted: decode, unit = sequence)
  int piece = kr - range_of_cost(weighted ? static_cast<int64_t>(cst(lo)) : ustart);

  auto advance = [&](const Cursor& c) {
    Cursor r = c;
    if (c.t + 1 < c.n) {
      r.t = c.t + 1;
      return r;
    }
    if (kVar && c.c + 1 < c.nu) {
      r.c = c.c + 1;
      r.t = 0;
      r.n = unit_tiles(c.ctx, c.qn, r.c);
      return r;
    }
    int s = c.s + 1;
    while (s < S - 1 && pre(s + 1) == pre(s)) ++s;  // sequences with no tiles
    return open_seq(s);
  };
  auto row_of = [&](int s) { return a.block_table + static_cast<int64_t>(s) * a.max_blocks; };

  // this lane's column: token offset within its group and head within the
  // KV head's group of query heads
  const int my_tok = kVar ? col / G : 0;
  const int my_g = kVar ? col % G : col;
  const bool my_col = kVar ? col < tpg * G : col < G;
  auto lane_token = [&](const Cursor& c) { return c.c * tpg + my_tok; };
  auto lane_live = [&](const Cursor& c) { return my_col && lane_token(c) < c.qn; };

  const Geo geo(a, col, grp);
  const float qk_scale = a.scale * kLog2e;
  PKV_LDS char* slot = (PKV_LDS char*)(s_slots) + w * kSlotBytes;

  // Q^T operand of a unit: lane (col n, group j) holds its column's query at
  // dim chunks 4*kk + j; zero for unused columns.
  auto load_q_unit = [&](uint4* qq, const Cursor& c) {
    if constexpr (kVar) {
      const bool ok = lane_live(c);
      const char* qp = static_cast<const char*>(a.query) +
                       ((static_cast<int64_t>(c.q0 + lane_token(c)) * a.num_heads + kvh * G +
                         my_g) * kD) * 2;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        qq[kk] = ok ? *reinterpret_cast<const uint4*>(qp + (4 * kk + grp) * 16)
                    : make_uint4(0, 0, 0, 0);
    } else {
      load_q(qq, a, c.s, kvh, G, col, grp);
    }
  };
  // score limit of this lane's column and the wave-uniform V limit, relative
  // to the first position of tile c.t
  auto limits = [&](const Cursor& c, bool g_ok, int& slim, int& vlim) {
    const int tok0 = c.t * kTile;
    if (!g_ok) {
      slim = vlim = 0;
      return;
    }
    if constexpr (kVar) {
      const int e = (c.c + 1) * tpg < c.qn ? (c.c + 1) * tpg : c.qn;
      vlim = c.ctx - c.qn + e - tok0;
      slim = lane_live(c) ? c.ctx - c.qn + lane_token(c) + 1 - tok0 : 0;
    } else {
      slim = vlim = c.ctx - tok0;
    }
  };

  uint4 q[4], qn[4];
  load_q_unit(q, cur);
  Attend<T> st;
  st.reset();

  // Finished pieces. A piece's partial (m, l and the normalised output of its
  // live columns) waits in this wave's LDS staging area and is written to the
  // workspace when the wave's range ends, or earlier when the area is full:
  // stores spread through the KV stream slow down the loads of the whole GPU
  // (a few MB of partials cost several percent of the stream's time), while
  // the same stores issued in one burst at the end of the range do not. A
  // unit's last piece also marks its remaining slots unused (l = 0) so the
  // merge skips them. Live columns are a prefix [0, nl) of the 16 columns.
  // With multi-token queries a unit done in a single piece writes its output
  // rows themselves, and l = -1 into their first slot, so the merge leaves
  // them alone (decode calls keep the output untouched, as their contract
  // says).
  //
  // Record: int4 header {sequence (decode) or first query row, column group,
  // slot, nl | mark << 16 | single << 17}, then nl rows of 128 floats, then
  // nl (m, l) pairs.
  PKV_LDS char* stage = (PKV_LDS char*)(stage_base) + w * stage_bytes;
  int st_used = 0, st_n = 0;  // bytes and records staged (wave-uniform)
  auto live_cols = [&](const Cursor& c) {
    if constexpr (kVar) {
      int k = c.qn - c.c * tpg;
      k = k < tpg ? k : tpg;
      return k > 0 ? k * G : 0;
    }
    return G;
  };
  // workspace row (query row x heads + head) of column n of a piece
  auto row_index = [&](int sq, int cg, int n) -> int64_t {
    if constexpr (kVar)
      return static_cast<int64_t>(sq + cg * tpg + n / G) * a.num_heads + kvh * G + n % G;
    return static_cast<int64_t>(sq) * a.num_heads + kvh * G + n;
  };
  auto rec_bytes = [](int nl) { return (16 + nl * (kD * 4 + 8) + 15) & ~15; };
  // A unit's last piece marks slots piece+1 .. mp-1 of its nl rows unused.
  auto mark_rest = [&](int sq, int cg, int pc, int nl) {
    const int rest = mp - pc - 1;
    for (int idx = lane; idx < nl * rest; idx += 64) {
      const int r = idx / rest;
      const int64_t e = row_index(sq, cg, r) * mp + pc + 1 + idx % rest;
      store_untracked(a.max_logits + e, -INFINITY);
      store_untracked(a.exp_sums + e, 0.f);
    }
  };
  // Write every staged record: two 512-byte rows per store instruction.
  auto flush = [&]() {
    int off = 0;
    for (int k = 0; k < st_n; ++k) {
      const PKV_LDS char* rec = stage + off;
      const u32x4 h = *(const PKV_LDS u32x4*)(rec);
      const int sq = __builtin_amdgcn_readfirstlane(static_cast<int>(h[0]));
      const int cg = __builtin_amdgcn_readfirstlane(static_cast<int>(h[1]));
      const int pc = __builtin_amdgcn_readfirstlane(static_cast<int>(h[2]));
      const int nl = __builtin_amdgcn_readfirstlane(static_cast<int>(h[3] & 0xffffu));
      const int mark = __builtin_amdgcn_readfirstlane(static_cast<int>((h[3] >> 16) & 1u));
      const int single = __builtin_amdgcn_readfirstlane(static_cast<int>(h[3] >> 17));
      if (pc < mp) {
        for (int r0 = 0; r0 < nl; r0 += 2) {
          const int r = r0 + (lane >> 5);
          const int ch = lane & 31;
          if (r < nl) {
            const f32x4 v = *(const PKV_LDS f32x4*)(rec + 16 + r * (kD * 4) + ch * 16);
            float* dst = single ? a.out + row_index(sq, cg, r) * kD
                                : a.tmp_out + (row_index(sq, cg, r) * mp + pc) * kD;
            if (fused && !single)
              store_untracked_device(dst + ch * 4, make_float4(v[0], v[1], v[2], v[3]));
            else
              store_untracked(dst + ch * 4, make_float4(v[0], v[1], v[2], v[3]));
          }
        }
        if (lane < nl) {
          const f32x2 ml = *(const PKV_LDS f32x2*)(rec + 16 + nl * (kD * 4) + lane * 8);
          const int64_t e = row_index(sq, cg, lane) * mp + pc;
          if (single) {
            if (kVar) store_untracked(a.exp_sums + e, -1.f);
          } else if (fused) {
            store_untracked_device(a.max_logits + e, ml[0]);
            store_untracked_device(a.exp_sums + e, ml[1]);
          } else {
            store_untracked(a.max_logits + e, ml[0]);
            store_untracked(a.exp_sums + e, ml[1]);
          }
        }
      }
      if (mark && !single && !fused) mark_rest(sq, cg, pc, nl);
      off += rec_bytes(nl);
    }
    st_used = 0;
    st_n = 0;
  };
  auto finish = [&](const Cursor& c) {
    const float l_col = st.column_sum();
    const float inv = l_col > 0.f ? 1.f / l_col : 0.f;
    const int nl = live_cols(c);
    const int sq = kVar ? c.q0 : c.s;
    const int cg = kVar ? c.c : 0;
    const bool last = c.t == c.n - 1;
    const bool single = (kVar || fused) && last && piece == 0;
    const int need = rec_bytes(nl);
    if (st_used + need > stage_bytes) flush();
    if (need <= stage_bytes) {
      PKV_LDS char* rec = stage + st_used;
      if (col < nl) {
        PKV_LDS char* ob = rec + 16 + col * (kD * 4) + grp * 16;
#pragma unroll
        for (int db = 0; db < 8; ++db) *(PKV_LDS f32x4*)(ob + db * 64) = st.acc[db] * inv;
        if (grp == 0)  // natural-log units
          *(PKV_LDS f32x2*)(rec + 16 + nl * (kD * 4) + col * 8) =
              f32x2{st.m_max * kLn2, st.sum_at_max(l_col)};
      }
      if (lane == 0)
        *(PKV_LDS u32x4*)(rec) = u32x4{static_cast<unsigned>(sq), static_cast<unsigned>(cg),
                                       static_cast<unsigned>(piece),
                                       static_cast<unsigned>(nl | (last << 16) |
                                                             (single << 17))};
      st_used += need;
      ++st_n;
    } else {
      // no room even in an empty area: write directly
      if (col < nl && piece < mp) {
        float* dst = (single ? a.out + row_index(sq, cg, col) * kD
                             : a.tmp_out + (row_index(sq, cg, col) * mp + piece) * kD) +
                     4 * grp;
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          const float4 x = make_float4(st.acc[db][0] * inv, st.acc[db][1] * inv,
                                       st.acc[db][2] * inv, st.acc[db][3] * inv);
          if (fused && !single)
            store_untracked_device(dst + 16 * db, x);
          else
            store_untracked(dst + 16 * db, x);
        }
        if (grp == 0) {
          const int64_t e = row_index(sq, cg, col) * mp + piece;
          if (single) {
            if (kVar) store_untracked(a.exp_sums + e, -1.f);
          } else if (fused) {
            store_untracked_device(a.max_logits + e, st.m_max * kLn2);
            store_untracked_device(a.exp_sums + e, st.sum_at_max(l_col));
          } else {
            store_untracked(a.max_logits + e, st.m_max * kLn2);
            store_untracked(a.exp_sums + e, st.sum_at_max(l_col));
          }
        }
      }
      if (last && !single && !fused) mark_rest(sq, cg, piece, nl);
    }
    st.reset();
    piece = 0;
  };

  // Tiles in flight while a tile is computed: one for decode, two for
  // multi-token queries, whose tiles carry more softmax work per byte
  // (speculative verify 1-3 % faster with two; decode, GQA and MHA no
  // faster, the decode step 0.1 % slower, A-B runs on one box). kAhead + 1 register sets, unrolled by
  // kAhead + 1. The q of a unit is loaded one step before the unit's first
  // tile is computed, ahead of the loads issued in that step. Every step
  // issues a tile's loads, the last kAhead steps of a range the newest tile
  // again (at most kAhead redundant tiles per wave, cache hits): with the
  // loads behind a branch, the compiler's wait analysis also walks the path
  // that skips both the loads and the compute, and waits for the whole
  // previous tile before the next step's address arithmetic reuses its
  // registers. Unconditional, every tile has exactly kAhead tiles of loads
  // behind it, and the waits are for that tile alone (checked in the
  // assembly; with two ahead, the first of the three unrolled steps still
  // waits as if one were).
  constexpr int kAhead = kVar ? 2 : 1;
  TileRegs ta, tb, tc;
  // Decode step: the new token of each sequence whose last tile lies in this
  // range goes into the pool here, for this wave's KV head, by the wave that
  // reads that tile (the only reader of that row in this launch): its later
  // load of the tile comes after the store from the same wave, so it sees
  // the new row. Four tokens at a time: lane group g (16 lanes) moves token
  // g's K and V rows, one 16-byte chunk of each per lane. The sequences are
  // wave-uniform, so their slots come from scalar loads, which never wait
  // for the wave's tile loads in flight.
  const int g4 = lane >> 4;
  const int c16 = lane & 15;
  // lane i: does sequence s0 + i end in this range?
  auto ends_in_range = [&](int s0) {
    const int s = s0 + lane;
    bool f = false;
    if (s < S) {
      const int t0 = s_pre[s], t1 = s_pre[s + 1];
      f = t1 > t0 && t1 - 1 >= b0 && t1 - 1 < b1;
    }
    return static_cast<uint64_t>(__ballot(f));
  };
  // the sequence of the n-th set bit of m (uniform), -1 past the last
  auto nth_seq = [&](int s0, uint64_t m, int n) {
    for (int i = 0; i < n && m != 0; ++i) m &= m - 1;
    return m != 0 ? s0 + static_cast<int>(__builtin_ctzll(m)) : -1;
  };
  auto pick4 = [&](int x0, int x1, int x2, int x3) {
    return g4 == 0 ? x0 : g4 == 1 ? x1 : g4 == 2 ? x2 : x3;
  };

  // this lane's chunks of sequence s's new K and V rows
  auto load_new = [&](int s, uint4& kx, uint4& vx) {
    const int64_t src = ((static_cast<int64_t>(s) * a.num_kv_heads + kvh) * kD) * 2 + c16 * 16;
    kx = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.k_new) + src);
    vx = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.v_new) + src);
  };
  // Slots of four sequences' new rows, lane u < 4 for the u-th: its context
  // length, then its table entry, one vector load each for all four; the
  // byte offset of the row in this KV head's pools goes to lane group u (-1
  // for no sequence, or no valid block there). A missing sequence reads
  // sequence 0's entries and is dropped.
  struct NewRows {
    int xu;     // lane u: the sequence, or -1
    int c;      // its context length
    int32_t e;  // its last position's table entry
  };
  auto rows_ctx = [&](int x0, int x1, int x2, int x3) {
    NewRows r;
    r.xu = lane == 0 ? x0 : lane == 1 ? x1 : lane == 2 ? x2 : lane == 3 ? x3 : -1;
    r.c = a.context_lens[r.xu >= 0 ? r.xu : 0];
    r.e = -1;
    return r;
  };
  auto last_pos = [&](const NewRows& r) { return (r.c < cap ? r.c : cap) - 1; };
  auto rows_entry = [&](NewRows& r) {
    const int p = last_pos(r);
    r.e = row_of(r.xu >= 0 ? r.xu : 0)[p >= 0 ? p / a.block_size : 0];
  };
  auto rows_offset = [&](const NewRows& r) -> int64_t {
    const int p = last_pos(r);
    const int64_t o = r.xu >= 0 && p >= 0 && r.e >= 0 && r.e < a.num_blocks
                          ? static_cast<int64_t>(r.e) * geo.block_stride +
                                kvh * geo.head_stride +
                                static_cast<int64_t>(p % a.block_size) * kD * 2
                          : -1;
    const int lo32 = __shfl(static_cast<int>(o & 0xffffffff), g4, 64);
    const int hi32 = __shfl(static_cast<int>(o >> 32), g4, 64);
    return static_cast<int64_t>((static_cast<uint64_t>(static_cast<uint32_t>(hi32)) << 32) |
                                static_cast<uint32_t>(lo32));
  };
  auto store_new = [&](int64_t off, const uint4& kx, const uint4& vx) {
    if (off >= 0) {
      store_untracked(const_cast<char*>(geo.kc) + off + c16 * 16, kx);
      store_untracked(const_cast<char*>(geo.vc) + off + c16 * 16, vx);
    }
  };
  // every token of the range but the first `skip` of the first window
  auto append_rest = [&](int skip) {
    for (int s0 = lo; s0 < S && pre(s0) < b1; s0 += 64) {
      uint64_t m = ends_in_range(s0);
      for (int i = 0; s0 == lo && i < skip && m != 0; ++i) m &= m - 1;
      while (m != 0) {
        const int x0 = nth_seq(s0, m, 0), x1 = nth_seq(s0, m, 1);
        const int x2 = nth_seq(s0, m, 2), x3 = nth_seq(s0, m, 3);
        const int my = pick4(x0, x1, x2, x3);
        uint4 kx = make_uint4(0, 0, 0, 0), vx = kx;
        if (my >= 0) load_new(my, kx, vx);
        NewRows r = rows_ctx(x0, x1, x2, x3);
        rows_entry(r);
        const int64_t o = rows_offset(r);
        if (my >= 0) store_new(o, kx, vx);
        for (int i = 0; i < 4 && m != 0; ++i) m &= m - 1;
      }
    }
  };
  // When this range starts with a sequence's last tile, every store comes
  // before the first tile's loads. Otherwise the first four tokens' rows are
  // loaded before the tile (so waiting for them does not wait for it), the
  // tile's loads go out, then their stores; the rest follow the barrier
  // that ends the shared-run work.
  const bool append = !kVar && a.k_new != nullptr && active;
  const bool first_is_new = append && pre(cur.s + 1) - 1 == b0;
  if (first_is_new) append_rest(0);
  const bool early = append && !first_is_new;
  uint64_t m_new = 0;
  int xa = -1, xb = -1, xc = -1, xd = -1, x_my = -1;
  uint4 k_my = make_uint4(0, 0, 0, 0), v_my = k_my;
  NewRows r_new{-1, 0, -1};
  if (early) {
    m_new = ends_in_range(lo);
    xa = nth_seq(lo, m_new, 0);
    xb = nth_seq(lo, m_new, 1);
    xc = nth_seq(lo, m_new, 2);
    xd = nth_seq(lo, m_new, 3);
    x_my = pick4(xa, xb, xc, xd);
    if (x_my >= 0) load_new(x_my, k_my, v_my);
    r_new = rows_ctx(xa, xb, xc, xd);
  }
  // (an idle wave loads its stand-in range's first tile too: a branch here
  // would make every later wait on this path count as if the loads were
  // absent, and wait for the tile itself)
  bool ga = geo.load(ta, row_of(cur.s), cur.t * kTile, kvh);
  if (early) rows_entry(r_new);
  // keeps the touches' loads (the sum means nothing); the barrier holds every
  // wave's staging area until the workgroup is done with the group lists
  sink += (last_touch[0] + last_touch[1]) + (last_touch[2] + last_touch[3]);
  if (sink == 0x9e3779b9u) s_wsum[0] = static_cast<int>(sink);
  if (n_groups > 0) __syncthreads();
  if (early) {
    const int64_t o = rows_offset(r_new);  // (every lane: a cross-lane read)
    if (x_my >= 0) store_new(o, k_my, v_my);
  }
  if (early && (__builtin_popcountll(m_new) > 4 || (lo + 64 < S && pre(lo + 64) < b1)))
    append_rest(4);
  if (!active) return;
  Cursor nx = cur;   // the tile after `cur`, once loaded
  Cursor nx2 = cur;  // (two ahead) the newest tile loaded
  bool gb = true, gc = true;
  if constexpr (kAhead == 2) {
    // the second tile, after the new tokens' stores (it may hold one); a
    // one-tile range loads its only tile again (no branch: see above)
    nx = len > 1 ? advance(cur) : cur;
    gb = geo.load(tb, row_of(nx.s), nx.t * kTile, kvh);
    nx2 = nx;
  }
  int i = 0;
  auto step = [&](TileRegs& now, bool g_now, TileRegs& next, bool& g_next) {
    // now = tile i (cur); next <- tile i + kAhead (with kAhead = 2, tile
    // i + 1 (nx) is already in flight)
    const bool more = i + 1 < len;
    if constexpr (kAhead == 1) nx = more ? advance(cur) : cur;
    const bool switch_unit = more && (cur.t + 1 >= cur.n);
    int slim, vlim;
    limits(cur, g_now, slim, vlim);
    if (switch_unit) load_q_unit(qn, nx);
    if constexpr (kAhead == 1) nx2 = nx;  // (cur itself at the end of the range)
    else if (i + kAhead < len) nx2 = advance(nx);
    g_next = geo.load(next, row_of(nx2.s), nx2.t * kTile, kvh);
    issue_fence();
    st.tile(now, q, slim, vlim, qk_scale, grp, col, slot);
    if (cur.t + 1 >= cur.n || !more) finish(cur);
    if (switch_unit) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) q[kk] = qn[kk];
    }
    cur = nx;
    nx = nx2;
    ++i;
    return more;
  };
  if constexpr (kAhead == 1) {
    while (true) {
      if (!step(ta, ga, tb, gb)) break;
      if (!step(tb, gb, ta, ga)) break;
    }
  } else {
    while (true) {
      if (!step(ta, ga, tc, gc)) break;
      if (!step(tb, gb, ta, ga)) break;
      if (!step(tc, gc, tb, gb)) break;
    }
  }
  flush();
  // pieces of sequence s (per lane; t0, t1: its stream tiles)
  if (fused) merge_arrivals(a, s_pre, S, lo, b0, b0 + len, kvh, G, mp, [&](int s, int t0, int t1) {
      if (!weighted) return range_of_cost(t1 - 1) - range_of_cost(t0) + 1;
      const int c0 = s_cost[s];
      const int nc = s_cost[s + 1] - c0;
      return range_of_cost(cost_in(c0, t1 - t0, nc, t1 - t0 - 1)) - range_of_cost(c0) + 1;
    });
}

// Launch shape of the split kernel on one device: one workgroup per CU with
// all of the CU's LDS (the tile prefix, then the staging areas). Computed on
// first use and kept: the answers only depend on the device and the kernel,
// and the queries cost host time that would otherwise sit between
// back-to-back launches.
constexpr int kMaxDevices = 64;

struct SplitShape {
  int cus;
  size_t dyn;  // dynamic LDS per workgroup
};

template <typename T, bool kVar>
hipError_t split_shape(SplitShape& out) {
  static std::atomic<int> cache[kMaxDevices][2];  // cus, dyn; 0 = not yet
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool cached = dev >= 0 && dev < kMaxDevices;
  if (cached) {
    out.cus = cache[dev][0].load(std::memory_order_relaxed);
    out.dyn = static_cast<size_t>(cache[dev][1].load(std::memory_order_relaxed));
    if (out.cus > 0 && out.dyn > 0) return hipSuccess;
  }
  auto kernel = decode_split_kernel<T, kVar>;
  int cus = 0, lds_cu = 0;
  hipFuncAttributes fa;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess)
    e = hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev);
  if (e == hipSuccess) e = hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(kernel));
  if (e != hipSuccess) return e;
  // the prefix alone must always fit
  const size_t need = ((static_cast<size_t>(kMaxSeqsBalanced) + 1) * sizeof(int) + 15) & ~size_t(15);
  size_t dyn = static_cast<size_t>(lds_cu);
  dyn = dyn > fa.sharedSizeBytes + 1024 ? (dyn - fa.sharedSizeBytes - 1024) & ~size_t(1023) : 0;
  dyn = dyn < need ? need : dyn;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(dyn));
  if (e != hipSuccess) return e;
  out = SplitShape{cus, dyn};
  if (cached) {
    cache[dev][1].store(static_cast<int>(dyn), std::memory_order_relaxed);
    cache[dev][0].store(cus, std::memory_order_relaxed);
  }
  return hipSuccess;
}

template <typename T, bool kVar>
hipError_t launch_split(const DecodeArgs& a, hipStream_t stream) {
  auto kernel = decode_split_kernel<T, kVar>;
  SplitShape sh{};
  hipError_t e = split_shape<T, kVar>(sh);
  if (e != hipSuccess) return e;
  const int waves_per_wg = kSplitThreads / 64;
  // One workgroup per CU (one wave per SIMD): each tile carries enough
  // matrix work for one wave to keep its loads flowing, ranges are as long
  // as they can be (fewer pieces) and the staging areas as large. Two
  // workgroups per CU, measured against it on MI355X, lose everywhere: the
  // older workgroup's waves win the issue arbitration and finish their equal
  // ranges well before the younger ones (MHA: 1.72 against 2.34 us per
  // tile), so the launch ends on a long tail (MHA kernel 169 against 166 us;
  // earlier, long split -3.9 %, GQA with a shared prefix -1.5 %, speculative
  // verify -7.7 %, mixed step -2.5 %).
  const size_t dyn = sh.dyn;
  // Decode calls look for shared blocks when a second prefix (the costs of
  // the weighted split) fits beside the first, and the sequences' first
  // blocks and the first-block hash (at least twice as many slots as
  // sequences) fit in the staging areas. Staging area per wave: what the
  // prefixes leave, in whole 16-byte units.
  const size_t pre = (static_cast<size_t>(a.num_seqs + 1) * sizeof(int) + 15) & ~size_t(15);
  int share_bits = 0;
  if (!kVar && a.num_seqs > 1) {
    int bits = 1;
    while ((1 << bits) < 2 * a.num_seqs) ++bits;
    const size_t first = (sizeof(int) * static_cast<size_t>(a.num_seqs) + 15) & ~size_t(15);
    if (2 * pre + first + (static_cast<size_t>(kShareSlotBytes) << bits) +
            (sizeof(int) << bits) <= dyn)
      share_bits = bits;
  }
  const size_t pre_all = share_bits > 0 ? 2 * pre : pre;
  const int stage = static_cast<int>(((dyn - pre_all) / waves_per_wg) & ~size_t(15));
  // whole groups of num_kv_heads waves, no more than the GPU holds at once
  int64_t waves = static_cast<int64_t>(sh.cus) * waves_per_wg;
  int64_t per_kv = waves / a.num_kv_heads;
  if (per_kv < 1) per_kv = 1;
  const int64_t wgs = (per_kv * a.num_kv_heads + waves_per_wg - 1) / waves_per_wg;
  kernel<<<dim3(static_cast<unsigned>(wgs)), dim3(kSplitThreads), dyn, stream>>>(
      a, static_cast<int>(per_kv), stage, share_bits);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_whole(const DecodeArgs& a, hipStream_t stream) {
  const int64_t items = static_cast<int64_t>(a.num_seqs) * a.num_kv_heads;
  decode_whole_kernel<T><<<dim3(static_cast<unsigned>(items)), dim3(kWavesUnsplit * 64), 0,
                           stream>>>(a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  return a.partition_size > 0 ? launch_split<T, false>(a, stream) : launch_whole<T>(a, stream);
}

}  // namespace

bool fast_decode_supported(const DecodeArgs& a) {
  const int G = a.num_heads / a.num_kv_heads;
  const int64_t items = static_cast<int64_t>(a.num_seqs) * a.num_kv_heads;
  if (!((a.dtype == 1 || a.dtype == 2) && a.head_size == kD && a.block_size % kTile == 0 &&
        G >= 1 && G <= 16 && items <= 0x7fffffff))
    return false;
  if (a.partition_size == 0) return true;
  // the split kernel keeps a per-sequence prefix in LDS, and indexes the
  // stream of all sequences' tiles with 32 bits: at most ceil(cap / 16)
  // tiles per sequence
  const int64_t cap = static_cast<int64_t>(a.max_blocks) * a.block_size;
  const int64_t per_seq = (cap + kTile - 1) / kTile;
  return a.num_seqs <= kMaxSeqsBalanced && a.num_seqs * per_seq <= 0x7fffffff;
}

hipError_t launch_decode_fast(const DecodeArgs& a, hipStream_t stream) {
  return a.dtype == 2 ? launch_t<bf16_t>(a, stream) : launch_t<f16_t>(a, stream);
}

bool fast_varlen_supported(const DecodeArgs& a) {
  const int G = a.num_heads / a.num_kv_heads;
  if (!((a.dtype == 1 || a.dtype == 2) && a.head_size == kD && a.block_size % kTile == 0 &&
        G >= 1 && G <= 16 && a.num_seqs <= kMaxSeqsBalanced))
    return false;
  // the prefill kernel takes its running max on unscaled scores
  if (!(a.scale > 0.f && a.scale <= 3.0e38f)) return false;
  // the stream of (sequence, column group) tiles is indexed with 32 bits: a
  // sequence has at most q_s / tpg + 1 groups of at most ceil(cap / 16) tiles
  const int64_t groups = a.num_tokens / (kTile / G) + a.num_seqs;
  const int64_t cap = static_cast<int64_t>(a.max_blocks) * a.block_size;
  const int64_t per_group = cap > kTile ? (cap + kTile - 1) / kTile : 1;
  return groups * per_group <= 0x7fffffff;
}

hipError_t launch_varlen_fast(const DecodeArgs& a, hipStream_t stream) {
  return a.dtype == 2 ? launch_split<bf16_t, true>(a, stream)
                      : launch_split<f16_t, true>(a, stream);
}

}  // namespace pkv
