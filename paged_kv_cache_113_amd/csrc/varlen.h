// Multi-token queries over paged KV: the metadata rules both matrix-core
// kernels apply, so that they agree on which sequences each one takes.
//
// A step can mix prefill chunks and decode tokens in one batch ("vLLM source
// walkthrough: PagedAttention and continuous batching", section 2.8); the
// attention metadata carries query start locations and context lengths
// (same page, section 1.7). Sequence s owns query rows [qsl[s], qsl[s+1]);
// its q_s new tokens are its last q_s positions, so token i sits at position
// ctx - q_s + i and sees positions 0 .. ctx - q_s + i.
#pragma once

#include "device.h"
#include "launch.h"

namespace pkv {

// Sequences whose query tokens fill at least this many (token, head)
// columns per KV head go to the prefill kernel, which shares each K/V tile
// among 128 columns in LDS; the rest go to the balanced split kernel, whose
// waves each hold 16 columns.
constexpr int kPrefillCols = 128;

__device__ __forceinline__ bool prefill_sized(int qn, int G) { return qn * G >= kPrefillCols; }

// Query rows of sequence s, clamped to [0, num_tokens] (the table is device
// data the host cannot check).
__device__ __forceinline__ void query_rows(const DecodeArgs& a, int s, int& q0, int& qn) {
  int lo = read_only(a.query_start_loc + s);
  int hi = read_only(a.query_start_loc + s + 1);
  lo = lo < 0 ? 0 : (lo > a.num_tokens ? a.num_tokens : lo);
  hi = hi < lo ? lo : (hi > a.num_tokens ? a.num_tokens : hi);
  q0 = lo;
  qn = hi - lo;
}

// 16-position tiles a group of query tokens [c*per, min((c+1)*per, qn))
// reads: what its last token sees, at least one (a fully masked tile when
// a token sees nothing, which only malformed metadata produces), so that
// every query row gets a partial.
__device__ __forceinline__ int group_tiles(int ctx, int qn, int c, int per) {
  const int e = (c + 1) * per < qn ? (c + 1) * per : qn;
  const int vis = ctx - qn + e;
  const int n = vis > 0 ? (vis + 15) / 16 : 0;
  return n > 0 ? n : 1;
}

}  // namespace pkv
