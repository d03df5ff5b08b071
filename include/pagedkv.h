/*
 * pagedkv.h -- C ABI of the MI355X (gfx950) paged-KV decode library.
 *
 * The problem, as the pages state it: each sequence's logical token
 * positions live in fixed-size physical blocks named by a block table;
 * position p of a sequence sits in physical block table[p / B] at offset
 * p % B, i.e. flat slot table[p / B] * B + p % B ("vLLM PagedAttention: from
 * fragmentation to slot mapping", section 3). Decode attention over those
 * blocks must equal softmax(q K^T / sqrt(D)) V over the contiguous history
 * (same page, section 7; the paper-notes page's block-wise formula and its
 * 10-token example). New tokens' K/V are written to the slots named by a
 * slot mapping (same page, section 6, "slot mapping / attention metadata").
 *
 * Layouts (all row-major, contiguous, device memory unless stated):
 *   query          [num_seqs, num_heads, head_size]            dtype
 *   k_cache/v_cache[num_blocks, num_kv_heads, block_size, head_size] dtype
 *                  (the glossary page "PagedAttention", teaching layout)
 *   block_table    [num_seqs, max_blocks_per_seq] int32; entries at and
 *                  beyond ceil(ctx / block_size) may hold anything (-1 by
 *                  convention; glossary page, block-table tensor) and are
 *                  never read
 *   context_lens   [num_seqs] int32: positions 0..ctx-1 are attended
 *   slot_mapping   [num_tokens] int64: flat slot, or < 0 for "no write"
 *   out            [num_seqs, num_heads, head_size] float32
 * Query head h reads KV head h / (num_heads / num_kv_heads): consecutive
 * query heads share a KV head (glossary page, expand_kv's repeat_interleave).
 *
 * dtype is one of PKV_F32, PKV_F16, PKV_BF16 and applies to query, caches and
 * new K/V alike. Arithmetic is float32 throughout (scores, softmax, sums).
 *
 * Ownership and threading: the caller allocates and owns every buffer. The
 * library allocates nothing and keeps no pointer after a call returns. Its
 * global state is a write-once, per-device cache of the launch shapes (CU
 * count, LDS budget, occupancy; filled on a device's first call, which also
 * sets the kernels' dynamic-LDS attribute, and valid when that first call is
 * made under graph capture) and of the static scratch buffer's address
 * (atomics; calls are reentrant and thread-safe), and that buffer itself,
 * which only paged_varlen_attention_noalloc uses. It never synchronises:
 * each call validates its arguments on the host, then enqueues kernels on
 * `stream` (a hipStream_t passed as void*; NULL is the default stream) and
 * returns. Device faults surface at the caller's next synchronisation.
 *
 * Errors: every call returns PKV_OK (0) or a negative pkv_status. All
 * argument checks run before any HIP call, so a failing call has enqueued
 * nothing. Values inside device buffers (block ids, lengths, slots) cannot be
 * checked on the host; the kernels never dereference a block id outside
 * [0, num_blocks) or a table entry outside the row (such positions are
 * skipped), so a bad value gives a wrong answer, not a fault.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum pkv_dtype { PKV_F32 = 0, PKV_F16 = 1, PKV_BF16 = 2 };

enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_NULL = -1,        /* a required pointer is NULL */
  PKV_ERR_SHAPE = -2,       /* a size is out of range or inconsistent */
  PKV_ERR_DTYPE = -3,       /* unknown dtype code */
  PKV_ERR_UNSUPPORTED = -4, /* valid, but no kernel handles this shape */
  PKV_ERR_WORKSPACE = -5,   /* split requested without its workspace */
  PKV_ERR_LAUNCH = -6,      /* the HIP runtime refused a launch */
  PKV_ERR_HOST = -7,        /* a host buffer is too small or not pinned memory */
  PKV_ERR_STATE = -8,       /* not valid in the block pool's current state */
  PKV_ERR_CAPACITY = -9,    /* not enough free blocks (nothing was taken) */
  PKV_ERR_SCRATCH = -10     /* more partials than the static scratch buffer holds */
};

/*
 * paged_slot_mapping -- flat slot of each sequence's new token.
 *
 * slot_mapping[s] = block_table[s][p / B] * B + p % B with p = positions[s]
 * ("vLLM PagedAttention ...", section 3; the source-walkthrough page
 * "vLLM source walkthrough: PagedAttention and continuous batching",
 * section 1.7). A negative position, a position whose logical block is at or
 * beyond max_blocks_per_seq, or a negative table entry gives -1.
 *
 * slot_mapping: [num_seqs] int64, written. block_table: [num_seqs,
 * max_blocks_per_seq] int32. positions: [num_seqs] int32.
 * Errors: PKV_ERR_NULL, PKV_ERR_SHAPE (num_seqs < 0, max_blocks_per_seq < 1,
 * block_size < 1). num_seqs == 0 is a no-op.
 */
int paged_slot_mapping(int64_t* slot_mapping, const int32_t* block_table,
                       const int32_t* positions, int num_seqs, int max_blocks_per_seq,
                       int block_size, void* stream);

/*
 * paged_kv_write -- store new tokens' K and V at their slots.
 *
 * For each i with 0 <= s = slot_mapping[i] < num_blocks * block_size and
 * every kv head h: k_cache[s / B][h][s % B][:] = k_new[i][h][:], likewise V.
 * A bit copy (the backend "writes new K/V to physical slots": "vLLM
 * PagedAttention ...", section 6). Other slots are untouched.
 *
 * k_new/v_new: [num_tokens, num_kv_heads, head_size] dtype.
 * Preconditions (not checkable on the host): non-negative slots are
 * distinct, and each target block is owned by one sequence. Shared full
 * blocks are read-only and each sequence writes only into its own last
 * block (nxmr.cn article, sections 4.2-4.3); copy-on-write is the caller's.
 * Errors: PKV_ERR_NULL, PKV_ERR_SHAPE, PKV_ERR_DTYPE. num_tokens == 0 is a
 * no-op.
 */
int paged_kv_write(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                   const int64_t* slot_mapping, int64_t num_tokens, int64_t num_blocks,
                   int num_kv_heads, int block_size, int head_size, int dtype,
                   void* stream);

/*
 * paged_decode_attention -- one query token per sequence over its paged KV.
 *
 * For sequence s and query head h (KV head kv = h / (num_heads/num_kv_heads)),
 * with z_t = scale * <q[s][h], K_s[kv][t]> over positions t < ctx_s:
 *   out[s][h] = sum_t exp(z_t - max z) V_s[kv][t] / sum_t exp(z_t - max z),
 * where K_s[kv][t] = k_cache[block_table[s][t / B]][kv][t % B]
 * ("vLLM PagedAttention ...", sections 3 and 7; paper-notes page, block-wise
 * formula). scale is normally 1/sqrt(head_size).
 *
 * partition_size == 0: `out` is written directly; the workspace pointers may
 * be NULL and max_partitions is ignored.
 * partition_size > 0 (a multiple of block_size): split mode, the "V2"
 * scheme of the source-walkthrough page, section 1.8 (a sequence's context is
 * cut into pieces computed in parallel, then merged by a reduce kernel). The
 * library cuts every sequence into at most max_partitions pieces of
 * consecutive positions, balancing the pieces over the whole GPU; the caller
 * sizes max_partitions >= ceil(max ctx / partition_size). For each (s, h)
 * with ctx_s >= 1 and each slot p < max_partitions the call writes either a
 * piece's partial
 *   max_logits[s][h][p] = m_p  = max of z_t over the piece,
 *   exp_sums[s][h][p]   = l_p  = sum exp(z_t - m_p)   (>= 1),
 *   tmp_out[s][h][p][:] = o_p  = sum exp(z_t - m_p) V[t] / l_p,
 * or marks the slot unused (l_p = 0, m_p = -inf). On the fast path the
 * pieces follow the balanced split, not multiples of partition_size: a
 * piece may start anywhere, a sequence shorter than partition_size may own
 * several slots, and which slots a sequence uses depends on the whole batch
 * and the device; partition_size then only tells the caller how to size
 * max_partitions. The plain kernel cuts exactly at multiples of
 * partition_size (piece p = positions [p P, (p+1) P)). Either way every slot
 * of a sequence with ctx_s >= 1 holds a partial or l_p = 0. `out` is
 * untouched; the caller then calls paged_attention_reduce. Workspace
 * layouts: max_logits and exp_sums [num_seqs, num_heads, max_partitions]
 * float32, tmp_out [num_seqs, num_heads, max_partitions, head_size] float32;
 * see paged_attention_workspace_bytes.
 *
 * ctx_s == 0 gives out = 0. Preconditions: ctx_s <= max_blocks_per_seq * B
 * (longer contexts are cut there), and in split mode ctx_s <= max_partitions *
 * partition_size (with the plain kernel, later partitions are not computed).
 *
 * Supported: f32/f16/bf16; head_size 1..256; any block_size >= 1; any
 * num_heads / num_kv_heads ratio. The fast path (matrix-core scores, DPP
 * lane broadcasts, balanced persistent split) covers f16/bf16, head_size
 * 128, block_size a multiple of 16, groups of up to 16 query heads per KV
 * head and, in split mode, up to 8192 sequences whose tables hold at most
 * 2^31 - 1 16-position tiles together; other shapes run a plain
 * wave-per-head kernel.
 * Errors: PKV_ERR_NULL, PKV_ERR_SHAPE (num_heads % num_kv_heads != 0, sizes
 * < 1, partition_size not a positive multiple of block_size, max_partitions
 * < 1 in split mode), PKV_ERR_DTYPE, PKV_ERR_UNSUPPORTED (head_size > 256),
 * PKV_ERR_WORKSPACE (split mode with a NULL workspace pointer),
 * PKV_ERR_LAUNCH. num_seqs == 0 is a no-op.
 */
int paged_decode_attention(float* out, const void* query, const void* k_cache,
                           const void* v_cache, const int32_t* block_table,
                           const int32_t* context_lens, int num_seqs, int num_heads,
                           int num_kv_heads, int head_size, int block_size,
                           int64_t num_blocks, int max_blocks_per_seq, float scale,
                           int partition_size, int max_partitions, float* max_logits,
                           float* exp_sums, float* tmp_out, int dtype, void* stream);

/*
 * paged_decode_attention_merged -- split decode and its merge in one call.
 *
 * out [num_seqs, num_heads, head_size] = the result of paged_decode_attention
 * in split mode followed by paged_attention_reduce (the "V2" partitions and
 * their reduce kernel, source-walkthrough page, section 1.8). On the fast
 * path this is one launch: the pieces go to the workspace as in split mode,
 * the wave that delivers the last piece of a (sequence, KV head) merges that
 * sequence's pieces for the KV head into out, and a sequence done in one
 * piece writes out directly; elsewhere it is the plain split kernel and the
 * merge kernel. Arguments as paged_decode_attention in split mode
 * (partition_size > 0, the workspace required; its contents are unspecified
 * afterwards), plus
 *   counters: device int32 [num_seqs * num_kv_heads] arrival counts, all
 *   zero before the call; the call leaves them zero again (each merging
 *   wave resets its own), so a buffer zeroed once serves every later call.
 * Calls that overlap must not share counters or workspace. ctx_s == 0 gives
 * out = 0.
 * Errors: those of paged_decode_attention, PKV_ERR_SHAPE for partition_size
 * < 1, PKV_ERR_NULL for a NULL out, PKV_ERR_WORKSPACE for NULL counters.
 */
int paged_decode_attention_merged(float* out, const void* query, const void* k_cache,
                                  const void* v_cache, const int32_t* block_table,
                                  const int32_t* context_lens, int num_seqs, int num_heads,
                                  int num_kv_heads, int head_size, int block_size,
                                  int64_t num_blocks, int max_blocks_per_seq, float scale,
                                  int partition_size, int max_partitions, float* max_logits,
                                  float* exp_sums, float* tmp_out, int32_t* counters, int dtype,
                                  void* stream);

/*
 * paged_decode_attention_append -- one decode step of one layer: each
 * sequence's new token K/V written into the paged pools, then
 * paged_decode_attention_merged over the updated pools.
 *
 * Sequence s's new token is its last position p = ctx_s - 1 (context_lens
 * count it). Its rows k_new[s], v_new[s] ([num_seqs, num_kv_heads,
 * head_size] dtype) are stored at the slot p translates to,
 * block_table[s][p / B] * B + p % B -- what paged_slot_mapping at positions
 * ctx - 1 followed by paged_kv_write stores (the backend writes the new
 * token's K/V to its slot: "vLLM PagedAttention ...", section 6) -- and out
 * is the attention over positions 0 .. ctx_s - 1 including it. On the fast
 * path this is one launch: the wave that reads the tile holding p stores the
 * new rows for its KV head before it loads that tile; elsewhere it is the
 * write, the plain split kernel and the merge. Arguments and workspace as
 * paged_decode_attention_merged, plus the mutable pools and k_new / v_new
 * (device). Preconditions: as paged_kv_write (each sequence owns the block
 * its new token goes to; a shared block is copied first, copy-on-write).
 * Sequences with ctx_s == 0 write nothing and get out = 0.
 * Errors: those of paged_decode_attention_merged, PKV_ERR_NULL for NULL
 * k_new / v_new.
 */
int paged_decode_attention_append(float* out, const void* query, void* k_cache, void* v_cache,
                                  const void* k_new, const void* v_new,
                                  const int32_t* block_table, const int32_t* context_lens,
                                  int num_seqs, int num_heads, int num_kv_heads, int head_size,
                                  int block_size, int64_t num_blocks, int max_blocks_per_seq,
                                  float scale, int partition_size, int max_partitions,
                                  float* max_logits, float* exp_sums, float* tmp_out,
                                  int32_t* counters, int dtype, void* stream);

/*
 * paged_attention_reduce -- merge split partials into the final output.
 *
 * For each (s, h) with ctx_s >= 1, over the slots p < max_partitions with
 * l_p > 0, M = max_p m_p and w_p = l_p * exp(m_p - M):
 *   out[s][h][:] = sum_p w_p o_p / sum_p w_p,
 * and out = 0 when ctx_s <= 0 or no slot is used. Every one of the row's
 * max_partitions slots is looked at, whatever ctx_s / partition_size is:
 * slots marked unused (l_p <= 0, as paged_decode_attention leaves them) are
 * skipped and their tmp_out rows never read, so the merge takes the
 * balanced pieces of the fast path and the aligned partitions of the plain
 * kernel alike. The pages name only "a reduce kernel that merges the
 * partitions" (source-walkthrough page, section 1.8); this is the exact
 * log-sum-exp merge. partition_size is not used by the merge (accepted for
 * symmetry; it must be >= 1). Layouts as in paged_decode_attention.
 * Errors: PKV_ERR_NULL, PKV_ERR_SHAPE, PKV_ERR_LAUNCH. num_seqs == 0 is a
 * no-op.
 */
int paged_attention_reduce(float* out, const float* max_logits, const float* exp_sums,
                           const float* tmp_out, const int32_t* context_lens, int num_seqs,
                           int num_heads, int head_size, int partition_size,
                           int max_partitions, void* stream);

/*
 * paged_varlen_attention -- several query tokens per sequence (chunked
 * prefill, speculative decoding, or a step that mixes them with decode
 * tokens) over paged KV, with a causal limit inside each sequence.
 *
 * A serving step can mix prefill chunks and decode tokens in one batch
 * (source-walkthrough page, continuous batching; the attention metadata of
 * "vLLM PagedAttention ...", section 6, carries query start locations and
 * positions). Sequence s owns query rows query_start_loc[s] ..
 * query_start_loc[s+1]-1, q_s of them; its new tokens' K/V are already in
 * the pools (paged_kv_write), so context_lens[s] counts them: q_s <= ctx_s.
 * Row query_start_loc[s] + i is the token at position p = ctx_s - q_s + i;
 * for query head h (KV head h / (num_heads/num_kv_heads)) it gets
 *   out[row][h] = softmax over t <= p of (scale <q, K_s[kv][t]>) applied to V,
 * with K_s/V_s read through the block table as in paged_decode_attention.
 * One query token per sequence (q_s = 1) is decode attention.
 *
 * query [num_tokens, num_heads, head_size] dtype; query_start_loc
 * [num_seqs + 1] int32, non-decreasing, from 0 to num_tokens; out
 * [num_tokens, num_heads, head_size] float32. The call writes `out` itself:
 * on the matrix-core path it splits each sequence's work over the whole GPU
 * into pieces (at most max_partitions per query row, so max_partitions >= 8
 * is a good choice; 1 serialises each KV head), keeps their partials in the
 * workspace max_logits/exp_sums [num_tokens, num_heads, max_partitions] and
 * tmp_out [num_tokens, num_heads, max_partitions, head_size] float32 (size:
 * paged_attention_workspace_bytes(num_tokens, ...)) and merges them; rows
 * done in a single piece are written directly. The workspace's contents
 * afterwards are unspecified. The
 * matrix-core path covers the shapes of paged_decode_attention's fast path
 * with a finite scale > 0; the plain path (everything else) ignores the
 * workspace. Rows no sequence claims
 * are undefined; rows past a sequence's context (q_s > ctx_s, a caller
 * error) get 0.
 *
 * Errors: PKV_ERR_NULL, PKV_ERR_SHAPE, PKV_ERR_DTYPE, PKV_ERR_UNSUPPORTED
 * (head_size > 256, or more than 2^26 (row, head) pairs), PKV_ERR_WORKSPACE
 * (a NULL workspace pointer), PKV_ERR_LAUNCH. num_seqs == 0 or num_tokens
 * == 0 is a no-op.
 */
int paged_varlen_attention(float* out, const void* query, const void* k_cache,
                           const void* v_cache, const int32_t* block_table,
                           const int32_t* query_start_loc, const int32_t* context_lens,
                           int num_seqs, int num_tokens, int num_heads, int num_kv_heads,
                           int head_size, int block_size, int64_t num_blocks,
                           int max_blocks_per_seq, float scale, int max_partitions,
                           float* max_logits, float* exp_sums, float* tmp_out, int dtype,
                           void* stream);

/*
 * paged_varlen_attention_noalloc -- paged_varlen_attention for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. Same arguments, meaning, kernels
 * and results as paged_varlen_attention (bit for bit, for the same inputs
 * and max_partitions on the same device), without the workspace: the split
 * partials go to a buffer the library holds in static device memory,
 * paged_varlen_attention_noalloc_limit() bytes (128 MiB) on each device it
 * runs on, kept until the process ends. The call allocates nothing (no
 * hipMalloc, no allocating library routine); its first call on a device
 * looks the buffer's address up once.
 *
 * Limit: paged_varlen_attention_noalloc_bytes(num_tokens, num_heads,
 * head_size, max_partitions) must not exceed the buffer, else
 * PKV_ERR_SCRATCH (nothing enqueued). Nothing in the buffer needs to start
 * at zero: every partial the merge reads is written by the same call first.
 * All calls on one device share the buffer, which keeps the last call's
 * contents: calls that overlap on one device (other streams, other host
 * threads) race and give wrong results; serialise them (one stream, or
 * events between streams).
 * Errors: those of paged_varlen_attention except PKV_ERR_WORKSPACE, plus
 * PKV_ERR_SCRATCH.
 */
int paged_varlen_attention_noalloc(float* out, const void* query, const void* k_cache,
                                   const void* v_cache, const int32_t* block_table,
                                   const int32_t* query_start_loc, const int32_t* context_lens,
                                   int num_seqs, int num_tokens, int num_heads, int num_kv_heads,
                                   int head_size, int block_size, int64_t num_blocks,
                                   int max_blocks_per_seq, float scale, int max_partitions,
                                   int dtype, void* stream);
/* Static scratch bytes a paged_varlen_attention_noalloc call needs (0 for
 * non-positive arguments), and the buffer's size. Host-only. */
size_t paged_varlen_attention_noalloc_bytes(int num_tokens, int num_heads, int head_size,
                                            int max_partitions);
size_t paged_varlen_attention_noalloc_limit(void);

/*
 * paged_attention_workspace_bytes -- bytes of max_logits + exp_sums + tmp_out
 * for a split call: num_seqs * num_heads * max_partitions * (head_size + 2) *
 * 4. Host-only; returns 0 for non-positive arguments.
 */
size_t paged_attention_workspace_bytes(int num_seqs, int num_heads, int head_size,
                                       int max_partitions);

/*
 * paged_kv_gather -- contiguous copy of each sequence's K and V (for checks).
 *
 * k_out[s][h][t][:] = k_cache[block_table[s][t / B]][h][t % B][:] for
 * t < min(ctx_s, max_ctx), likewise V; rows t >= ctx_s are left untouched.
 * This is the glossary page's gather_paged (paged -> contiguous), run through
 * the same device translation helper as the attention kernels, so that a
 * bytewise comparison checks block-table translation exactly.
 * k_out/v_out: [num_seqs, num_kv_heads, max_ctx, head_size] dtype.
 * Errors: PKV_ERR_NULL, PKV_ERR_SHAPE, PKV_ERR_DTYPE, PKV_ERR_LAUNCH.
 */
int paged_kv_gather(void* k_out, void* v_out, const void* k_cache, const void* v_cache,
                    const int32_t* block_table, const int32_t* context_lens, int num_seqs,
                    int num_kv_heads, int head_size, int block_size, int64_t num_blocks,
                    int max_blocks_per_seq, int max_ctx, int dtype, void* stream);

/*
 * paged_kv_copy_blocks -- copy whole blocks inside every layer's pools
 * (copy-on-write).
 *
 * Branches of a sequence (beam search, parallel sampling) share its blocks
 * by reference. A full block never changes and stays shared; before a branch
 * writes into its last, partly filled block while other branches still
 * reference it, the host allocator gives it a fresh block, and this call
 * copies the old block's KV data there (nxmr.cn article, sections 4.2-4.3;
 * only the modified block is copied, never the whole cache: paper-notes
 * page, beam search and parallel sampling). For every layer l < num_layers
 * and every pair i with src = block_mapping[2i], dst = block_mapping[2i+1]:
 *   k_caches[l][dst] = k_caches[l][src], v_caches[l][dst] = v_caches[l][src]
 * (all num_kv_heads x block_size x head_size elements, a bit copy).
 *
 * k_caches, v_caches: HOST arrays of num_layers device pointers, each a
 * [num_blocks, num_kv_heads, block_size, head_size] pool of `dtype`.
 * block_mapping: DEVICE int64 [num_pairs, 2]. A pair with an id outside
 * [0, num_blocks), or src == dst, is skipped. Preconditions: destinations
 * are distinct and none is another pair's source (then the order of the
 * pairs does not matter).
 * Errors: PKV_ERR_NULL, PKV_ERR_SHAPE, PKV_ERR_DTYPE, PKV_ERR_UNSUPPORTED
 * (2^24 pairs or more), PKV_ERR_LAUNCH. num_layers == 0 or num_pairs == 0
 * is a no-op.
 */
int paged_kv_copy_blocks(void* const* k_caches, void* const* v_caches, int num_layers,
                         const int64_t* block_mapping, int64_t num_pairs, int64_t num_blocks,
                         int num_kv_heads, int block_size, int head_size, int dtype,
                         void* stream);

/*
 * paged_kv_swap_out / paged_kv_swap_in -- move whole blocks between every
 * layer's pools and pinned host memory (preemption by swapping).
 *
 * A preempted request's KV blocks are copied from GPU to CPU memory and
 * back when the GPU has room again (paper-notes page, preemption: swapping
 * vs recomputation); on the way back they go to newly allocated blocks and
 * the request's table is rewritten to them (nxmr.cn article, section 6.2).
 * With slab = num_kv_heads * block_size * head_size elements:
 *   swap_out: host[l][0][i] = k_caches[l][block_ids[i]],
 *             host[l][1][i] = v_caches[l][block_ids[i]];
 *   swap_in:  k_caches[l][block_ids[i]] = host[l][0][i], likewise V,
 * for l < num_layers, i < num_ids (a bit copy). The host buffer is
 * [num_layers, 2, num_ids, slab] in `dtype` and host_bytes is its size.
 *
 * host buffer: pinned host memory (hipHostMalloc, or a torch tensor made
 * with pin_memory=True), read or written by the kernels directly over the
 * host link; the library queries the pointer and refuses anything else with
 * PKV_ERR_HOST (also when host_bytes is short) before launching. Like every
 * call here it only enqueues: the host data is complete (swap_out) or may be
 * reused (swap_in) once the stream has reached the call.
 * k_caches, v_caches: HOST arrays of num_layers device pool pointers.
 * block_ids: DEVICE int64 [num_ids]; an id outside [0, num_blocks) is
 * skipped (its host slab is untouched). swap_in destinations must be
 * distinct.
 * Errors: PKV_ERR_NULL, PKV_ERR_SHAPE, PKV_ERR_DTYPE, PKV_ERR_HOST,
 * PKV_ERR_UNSUPPORTED (2^24 ids or more), PKV_ERR_LAUNCH. num_layers == 0 or
 * num_ids == 0 is a no-op. These two calls make one HIP query (the pointer
 * check) before they launch; every other argument check precedes it.
 */
int paged_kv_swap_out(void* host_dst, int64_t host_bytes, void* const* k_caches,
                      void* const* v_caches, int num_layers, const int64_t* block_ids,
                      int64_t num_ids, int64_t num_blocks, int num_kv_heads, int block_size,
                      int head_size, int dtype, void* stream);
int paged_kv_swap_in(const void* host_src, int64_t host_bytes, void* const* k_caches,
                     void* const* v_caches, int num_layers, const int64_t* block_ids,
                     int64_t num_ids, int64_t num_blocks, int num_kv_heads, int block_size,
                     int head_size, int dtype, void* stream);

/*
 * Prefix caching (host side, no GPU work): block identity and a block pool
 * whose freed blocks stay hit-able until their slot is needed again.
 *
 * A full block's identity is SHA-256 over its token ids and extra keys, 32
 * bytes ("vLLM source walkthrough: PagedAttention and continuous batching",
 * section 1.9). So that an identity covers the whole prefix (equal tokens
 * after different prefixes are different K/V), each block's message starts
 * with the previous block's hash (32 zero bytes before the first block),
 * then the block's tokens as little-endian int32, then the extra keys (for
 * instance an adapter name or a cache salt).
 *
 * The pool follows the block life cycle of "vLLM PagedAttention: from
 * fragmentation to slot mapping" (block metadata under prefix caching): each
 * block has a reference count and an optional identity; free blocks wait in
 * a FIFO queue (taken from the head, returned to the tail; an intrusive
 * doubly linked list, O(1) unlinking); a ref-0 block with an identity stays
 * hit-able in the queue; a hit takes it out of the queue ("touch") and
 * counts a reference; taking a block for new data erases its identity;
 * releasing a block to 0 returns it to the tail with its identity. A pool is
 * host memory owned by its handle (pkv_pool_create / pkv_pool_destroy), not
 * thread-safe (one caller at a time), and touches no device memory.
 */
typedef struct pkv_block_pool pkv_block_pool;

/* pkv_block_hashes -- out[32 * b ..] = identity of full block b of tokens
 * (block_size tokens each; a trailing partial block has none). Returns the
 * number of full blocks (>= 0) or a negative pkv_status (PKV_ERR_NULL,
 * PKV_ERR_SHAPE). Host pointers. */
int64_t pkv_block_hashes(uint8_t* out, const int32_t* tokens, int64_t num_tokens, int block_size,
                         const uint8_t* extra, int64_t extra_len);

/* pkv_pool_create -- a pool of blocks 0..num_blocks-1, all free, queued in
 * the order initial_free gives (a permutation of 0..num_blocks-1) or 0, 1,
 * ... when it is NULL. *out receives the handle. Errors: PKV_ERR_NULL,
 * PKV_ERR_SHAPE (sizes < 1, not a permutation), PKV_ERR_STATE (out of host
 * memory). */
int pkv_pool_create(pkv_block_pool** out, int num_blocks, int block_size,
                    const int32_t* initial_free);
/* pkv_pool_destroy -- frees the pool (NULL is ignored). */
void pkv_pool_destroy(pkv_block_pool* pool);
/* pkv_pool_num_free -- blocks in the free queue (cached or not). */
int64_t pkv_pool_num_free(const pkv_block_pool* pool);

/* pkv_pool_longest_hit -- the blocks of the leading hashes[32 * i ..] that
 * are cached, up to the first miss, into out_blocks; returns how many.
 * Changes nothing. */
int pkv_pool_longest_hit(const pkv_block_pool* pool, const uint8_t* hashes, int num_hashes,
                         int32_t* out_blocks);
/* pkv_pool_touch -- one more reference on each listed block; a ref-0 block
 * leaves the free queue (a hit on a cached-free block). Errors:
 * PKV_ERR_SHAPE (an id outside the pool; nothing changed). */
int pkv_pool_touch(pkv_block_pool* pool, const int32_t* blocks, int n);
/* pkv_pool_allocate -- n blocks from the head of the free queue for new
 * data (reference count 1, identity erased). PKV_ERR_CAPACITY when fewer
 * than n are free; nothing is taken then. */
int pkv_pool_allocate(pkv_block_pool* pool, int n, int32_t* out_blocks);
/* pkv_pool_cache -- give an in-use full block the identity hash[0..31].
 * Returns 1 when cached, 0 when the block already has an identity or the
 * hash already names a block (the first keeps it), PKV_ERR_STATE for a
 * block not in use, PKV_ERR_SHAPE for an id outside the pool. */
int pkv_pool_cache(pkv_block_pool* pool, int32_t block, const uint8_t* hash);
/* pkv_pool_release -- one reference less on each listed block, in order; a
 * block at 0 goes to the tail of the free queue and keeps its identity.
 * PKV_ERR_STATE when a block is listed more often than it is referenced;
 * nothing changes then. */
int pkv_pool_release(pkv_block_pool* pool, const int32_t* blocks, int n);

/* pkv_pool_admit -- blocks for a request of num_tokens tokens: its longest
 * run of leading cached blocks, capped at (num_tokens - 1) / block_size
 * blocks so that the last token is recomputed (walkthrough page, section
 * 1.9), by reference (touched), and fresh blocks for the rest.
 * out_table receives ceil(num_tokens / block_size) block ids and
 * *cached_tokens the tokens the hit covers. PKV_ERR_CAPACITY (nothing
 * changed) when the free blocks do not suffice. */
int pkv_pool_admit(pkv_block_pool* pool, const int32_t* tokens, int64_t num_tokens,
                   const uint8_t* extra, int64_t extra_len, int32_t* out_table,
                   int64_t* cached_tokens);
/* pkv_pool_cache_full_blocks -- after a request's K/V are written, its full
 * blocks (table[0 .. num_tokens / block_size - 1]) get their identities
 * (blocks that have one, and hashes already taken, are left as they are). */
int pkv_pool_cache_full_blocks(pkv_block_pool* pool, const int32_t* table,
                               const int32_t* tokens, int64_t num_tokens, const uint8_t* extra,
                               int64_t extra_len);
/* pkv_pool_state -- for checks: reference counts [num_blocks], the free
 * queue from head to tail, and a cached flag per block (each may be NULL).
 * Returns the number of free blocks. */
int pkv_pool_state(const pkv_block_pool* pool, int32_t* ref_out, int32_t* free_out,
                   uint8_t* cached_out);

/* pkv_strerror -- static description of a pkv_status code. */
const char* pkv_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
