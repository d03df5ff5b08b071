/*
 * Paged-KV decode attention oracle: plain, slow, fp64 CPU reference.
 *
 * TEST INFRASTRUCTURE ONLY. Only tests/, the smoke check and the CPU
 * baseline leg of bench.py may load this. It shares no code, header, table
 * or helper with the HIP library under paged_kv_cache_113_amd/.
 *
 * What it computes, and where the pages define it:
 *  - Widening of f32/f16/bf16 storage to double, from the IEEE-754 binary16
 *    and bfloat16 bit definitions (no page; pinned against numpy/torch over
 *    all 65536 bit patterns).
 *  - Block-table gather (orc_gather): the logical position t of a sequence
 *    lives in physical block table[t / B] at offset t % B
 *    ("vLLM PagedAttention: from fragmentation to slot mapping", section 3,
 *    the b_l / o / b_p / slot formula; the glossary page's gather_paged in
 *    "contiguous vs page-table reference"). The pool layout is
 *    [num_blocks, Hkv, B, D], the glossary page's teaching layout.
 *  - Attention (orc_attention): softmax(q K^T * scale) V over the gathered,
 *    contiguous K/V of one sequence ("vLLM PagedAttention ...", section 7,
 *    softmax(QK^T/sqrt(D))V; the paper-notes page's statement that paged
 *    attention is mathematically identical to standard attention). Query head
 *    h reads KV head h / (Hq/Hkv) (glossary page, expand_kv's
 *    repeat_interleave over the KV-head dimension).
 *  - Multi-token queries (orc_attention_varlen): a sequence brings q_s new
 *    query tokens at its last q_s positions (chunked prefill, speculative
 *    decoding; source-walkthrough page, continuous batching, where a step
 *    mixes prefill chunks and decode tokens, and the vLLM page's attention
 *    metadata: query start locations and positions). Token i of sequence s
 *    sits at p = ctx_s - q_s + i and attends positions 0..p (causal): the
 *    same softmax as above over a prefix of the gathered sequence.
 *  - Split partials (orc_attention_partials) and their log-sum-exp merge
 *    (orc_lse_combine): the pages only say that long sequences are split
 *    into partitions computed in parallel and merged by a reduce kernel
 *    (source-walkthrough page, section 1.8, V1 vs V2). The reading taken:
 *    partition p covers positions [p*P, min((p+1)*P, ctx)); its partial is
 *    (m_p = max score, l_p = sum exp(z - m_p), o_p = sum exp(z - m_p) v / l_p);
 *    the merge is the exact identity out = sum_p e^{m_p-M} l_p o_p /
 *    sum_p e^{m_p-M} l_p with M = max_p m_p.
 *
 * Conventions shared with the library only as documented argument meaning
 * (not as code): scale arrives as the same float the GPU receives and is
 * widened exactly; ctx = 0 gives out = 0 and partials (-inf, 0, 0).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2 };
enum { ORC_OK = 0, ORC_EARG = -1, ORC_ETABLE = -2, ORC_ENOMEM = -3 };

/* ---- storage widening -------------------------------------------------- */

static double widen_f32(uint32_t bits) {
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static double widen_f16(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int frac = h & 0x3ff;
  double v;
  if (e == 0) {
    v = ldexp((double)frac, -24); /* subnormal: frac * 2^-14 * 2^-10 */
  } else if (e == 31) {
    v = frac ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + frac), e - 25); /* (1 + frac/1024) * 2^(e-15) */
  }
  return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32. */
static double widen_bf16(uint16_t b) { return widen_f32((uint32_t)b << 16); }

static double widen(const void* base, int64_t i, int dtype) {
  switch (dtype) {
    case ORC_F32: {
      uint32_t u;
      memcpy(&u, (const char*)base + 4 * i, 4);
      return widen_f32(u);
    }
    case ORC_F16: {
      uint16_t u;
      memcpy(&u, (const char*)base + 2 * i, 2);
      return widen_f16(u);
    }
    default: {
      uint16_t u;
      memcpy(&u, (const char*)base + 2 * i, 2);
      return widen_bf16(u);
    }
  }
}

int orc_widen(double* out, const void* in, int64_t n, int dtype) {
  if (!out || (!in && n) || n < 0 || dtype < 0 || dtype > 2) return ORC_EARG;
  for (int64_t i = 0; i < n; ++i) out[i] = widen(in, i, dtype);
  return ORC_OK;
}

/* ---- gather ------------------------------------------------------------ */

/* k_out, v_out: [hkv][ctx][D] doubles (either may be NULL).
 * Every table entry that covers a live position must lie in [0, num_blocks). */
int orc_gather(double* k_out, double* v_out, const void* k_pool, const void* v_pool,
               int dtype, const int32_t* table_row, int ctx, int64_t num_blocks,
               int hkv, int B, int D) {
  if (ctx < 0 || hkv <= 0 || B <= 0 || D <= 0 || dtype < 0 || dtype > 2) return ORC_EARG;
  for (int t = 0; t < ctx; ++t) {
    int64_t phys = table_row[t / B];
    if (phys < 0 || phys >= num_blocks) return ORC_ETABLE;
    int off = t % B;
    for (int kv = 0; kv < hkv; ++kv) {
      /* element index of pool[phys][kv][off][0] in [num_blocks, Hkv, B, D] */
      int64_t src = ((phys * hkv + kv) * B + off) * (int64_t)D;
      int64_t dst = ((int64_t)kv * ctx + t) * D;
      for (int d = 0; d < D; ++d) {
        if (k_out) k_out[dst + d] = widen(k_pool, src + d, dtype);
        if (v_out) v_out[dst + d] = widen(v_pool, src + d, dtype);
      }
    }
  }
  return ORC_OK;
}

/* ---- attention --------------------------------------------------------- */

typedef struct {
  /* problem */
  const void* q;
  const void* k_pool;
  const void* v_pool;
  int dtype;
  const int32_t* block_table;
  const int32_t* ctx_lens;
  int hq, hkv, D, B;
  int64_t num_blocks;
  int max_blocks;
  double scale;
  const int32_t* seqs; /* the sequences to compute, in output order; NULL = all */
  int n_seqs;
  const int32_t* qsl; /* multi-token queries: [num_seqs + 1] start rows; NULL = one
                         query token per sequence, query row s */
  int partition_size; /* 0: whole context (orc_attention) */
  int max_partitions;
  /* outputs */
  double* out;   /* whole: [n_seqs][hq][D] */
  double* m_out; /* partials: [n_seqs][hq][max_partitions] */
  double* l_out;
  double* o_out; /* partials: [n_seqs][hq][max_partitions][D] */
  /* work distribution */
  int64_t next;     /* next (seq, kv) unit, guarded by lock */
  pthread_mutex_t lock;
  int status;
} job_t;

/* Softmax-weighted sum over positions [lo, hi) of one gathered sequence, for
 * query head h (which reads KV head kv). z_t = scale * <q, k_t>;
 * m = max z; w_t = exp(z_t - m); o = sum w_t v_t / sum w_t.
 * Writes m, l = sum w_t and o (length D). Empty range: m=-inf, l=0, o=0. */
static void attend_range(const double* qh, const double* K, const double* V, int lo,
                         int hi, int D, double scale, double* z, double* m_out,
                         double* l_out, double* o) {
  for (int d = 0; d < D; ++d) o[d] = 0.0;
  if (hi <= lo) {
    *m_out = -INFINITY;
    *l_out = 0.0;
    return;
  }
  double m = -INFINITY;
  for (int t = lo; t < hi; ++t) {
    double dot = 0.0;
    for (int d = 0; d < D; ++d) dot += qh[d] * K[(int64_t)t * D + d];
    z[t - lo] = scale * dot;
    if (z[t - lo] > m) m = z[t - lo];
  }
  double l = 0.0;
  for (int t = lo; t < hi; ++t) {
    double w = exp(z[t - lo] - m);
    l += w;
    for (int d = 0; d < D; ++d) o[d] += w * V[(int64_t)t * D + d];
  }
  for (int d = 0; d < D; ++d) o[d] /= l;
  *m_out = m;
  *l_out = l;
}

static int run_unit(job_t* j, int64_t unit) {
  int si = (int)(unit / j->hkv);
  int kv = (int)(unit % j->hkv);
  int s = j->seqs ? j->seqs[si] : si;
  int ctx = j->ctx_lens[s];
  int D = j->D, G = j->hq / j->hkv;
  /* query rows q0 .. q0 + qn - 1 belong to s; row q0 + i is the token at
   * position ctx - qn + i and sees positions 0 .. ctx - qn + i. One decode
   * token (qn = 1) sees the whole context. */
  int q0 = j->qsl ? j->qsl[s] : s;
  int qn = j->qsl ? j->qsl[s + 1] - j->qsl[s] : 1;
  int orow = j->qsl ? q0 : si; /* first output row */
  if (ctx < 0 || qn < 0 || (j->qsl && qn > ctx)) return ORC_EARG;
  double* K = (double*)malloc(sizeof(double) * ((size_t)ctx * D + 1));
  double* V = (double*)malloc(sizeof(double) * ((size_t)ctx * D + 1));
  double* z = (double*)malloc(sizeof(double) * ((size_t)ctx + 1));
  double* qh = (double*)malloc(sizeof(double) * (size_t)D);
  double* o = (double*)malloc(sizeof(double) * (size_t)D);
  int rc = ORC_OK;
  if (!K || !V || !z || !qh || !o) {
    rc = ORC_ENOMEM;
    goto done;
  }
  /* gather this sequence's single KV head kv into contiguous [ctx][D] */
  const int32_t* row = j->block_table + (int64_t)s * j->max_blocks;
  for (int t = 0; t < ctx; ++t) {
    int64_t phys = row[t / j->B];
    if (phys < 0 || phys >= j->num_blocks) {
      rc = ORC_ETABLE;
      goto done;
    }
    int64_t src = ((phys * j->hkv + kv) * j->B + t % j->B) * (int64_t)D;
    for (int d = 0; d < D; ++d) {
      K[(int64_t)t * D + d] = widen(j->k_pool, src + d, j->dtype);
      V[(int64_t)t * D + d] = widen(j->v_pool, src + d, j->dtype);
    }
  }
  for (int i = 0; i < qn; ++i) {
    int visible = ctx - qn + i + 1; /* causal limit of this query row */
    for (int g = 0; g < G; ++g) {
      int h = kv * G + g; /* the query heads that read KV head kv */
      for (int d = 0; d < D; ++d)
        qh[d] = widen(j->q, ((int64_t)(q0 + i) * j->hq + h) * D + d, j->dtype);
      if (j->partition_size == 0) {
        double m, l;
        attend_range(qh, K, V, 0, visible, D, j->scale, z, &m, &l, o);
        double* dst = j->out + ((int64_t)(orow + i) * j->hq + h) * D;
        for (int d = 0; d < D; ++d) dst[d] = (visible > 0) ? o[d] : 0.0;
      } else {
        int P = j->partition_size;
        for (int p = 0; p < j->max_partitions; ++p) {
          int lo = p * P, hi = (p + 1) * P < visible ? (p + 1) * P : visible;
          double m, l;
          attend_range(qh, K, V, lo, hi, D, j->scale, z, &m, &l, o);
          int64_t idx = ((int64_t)(orow + i) * j->hq + h) * j->max_partitions + p;
          j->m_out[idx] = m;
          j->l_out[idx] = l;
          for (int d = 0; d < D; ++d) j->o_out[idx * D + d] = o[d];
        }
      }
    }
  }
done:
  free(K);
  free(V);
  free(z);
  free(qh);
  free(o);
  return rc;
}

static void* worker(void* arg) {
  job_t* j = (job_t*)arg;
  int64_t total = (int64_t)j->n_seqs * j->hkv;
  for (;;) {
    pthread_mutex_lock(&j->lock);
    int64_t u = j->next++;
    int failed = j->status != ORC_OK;
    pthread_mutex_unlock(&j->lock);
    if (u >= total || failed) break;
    int rc = run_unit(j, u);
    if (rc != ORC_OK) {
      pthread_mutex_lock(&j->lock);
      if (j->status == ORC_OK) j->status = rc;
      pthread_mutex_unlock(&j->lock);
    }
  }
  return NULL;
}

static int run_job(job_t* j, int threads) {
  if (threads < 1) threads = 1;
  j->next = 0;
  j->status = ORC_OK;
  pthread_mutex_init(&j->lock, NULL);
  pthread_t* tid = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)threads);
  if (!tid) return ORC_ENOMEM;
  int started = 0;
  for (int i = 1; i < threads; ++i) {
    if (pthread_create(&tid[i], NULL, worker, j) != 0) break;
    ++started;
  }
  worker(j); /* the calling thread works too */
  for (int i = 1; i <= started; ++i) pthread_join(tid[i], NULL);
  free(tid);
  pthread_mutex_destroy(&j->lock);
  return j->status;
}

static int check_common(int hq, int hkv, int D, int B, int dtype, int n_seqs) {
  if (hq <= 0 || hkv <= 0 || hq % hkv != 0 || D <= 0 || B <= 0) return ORC_EARG;
  if (dtype < 0 || dtype > 2 || n_seqs < 0) return ORC_EARG;
  return ORC_OK;
}

/* out: [n_seqs][hq][D] for the sequences listed in seqs (indices into the
 * batch). q: [num_seqs][hq][D]; pools [num_blocks][hkv][B][D]; block_table
 * [num_seqs][max_blocks]; threads >= 1 workers over (sequence, kv head). */
int orc_attention(double* out, const void* q, const void* k_pool, const void* v_pool,
                  int dtype, const int32_t* block_table, const int32_t* ctx_lens,
                  int hq, int hkv, int D, int B, int64_t num_blocks, int max_blocks,
                  float scale, const int32_t* seqs, int n_seqs, int threads) {
  int rc = check_common(hq, hkv, D, B, dtype, n_seqs);
  if (rc != ORC_OK) return rc;
  job_t j;
  memset(&j, 0, sizeof j);
  j.q = q; j.k_pool = k_pool; j.v_pool = v_pool; j.dtype = dtype;
  j.block_table = block_table; j.ctx_lens = ctx_lens;
  j.hq = hq; j.hkv = hkv; j.D = D; j.B = B;
  j.num_blocks = num_blocks; j.max_blocks = max_blocks;
  j.scale = (double)scale; j.seqs = seqs; j.n_seqs = n_seqs;
  j.partition_size = 0; j.out = out;
  return run_job(&j, threads);
}

/* Per-partition partials, layouts [n_seqs][hq][max_partitions] for m and l
 * and [n_seqs][hq][max_partitions][D] for o. Partitions at or beyond
 * ceil(ctx / P) hold (-inf, 0, 0). */
int orc_attention_partials(double* m_out, double* l_out, double* o_out, const void* q,
                           const void* k_pool, const void* v_pool, int dtype,
                           const int32_t* block_table, const int32_t* ctx_lens, int hq,
                           int hkv, int D, int B, int64_t num_blocks, int max_blocks,
                           float scale, int partition_size, int max_partitions,
                           const int32_t* seqs, int n_seqs, int threads) {
  int rc = check_common(hq, hkv, D, B, dtype, n_seqs);
  if (rc != ORC_OK) return rc;
  if (partition_size <= 0 || max_partitions <= 0) return ORC_EARG;
  for (int i = 0; i < n_seqs; ++i) {
    int ctx = ctx_lens[seqs[i]];
    if ((int64_t)max_partitions * partition_size < ctx) return ORC_EARG;
  }
  job_t j;
  memset(&j, 0, sizeof j);
  j.q = q; j.k_pool = k_pool; j.v_pool = v_pool; j.dtype = dtype;
  j.block_table = block_table; j.ctx_lens = ctx_lens;
  j.hq = hq; j.hkv = hkv; j.D = D; j.B = B;
  j.num_blocks = num_blocks; j.max_blocks = max_blocks;
  j.scale = (double)scale; j.seqs = seqs; j.n_seqs = n_seqs;
  j.partition_size = partition_size; j.max_partitions = max_partitions;
  j.m_out = m_out; j.l_out = l_out; j.o_out = o_out;
  return run_job(&j, threads);
}

/* Log-sum-exp merge of partials (same layouts as orc_attention_partials)
 * into out [num_seqs][hq][D]. Only partitions p < ceil(ctx_s / P) take part;
 * a sequence with none gets out = 0. */
int orc_lse_combine(double* out, const double* m, const double* l, const double* o,
                    const int32_t* ctx_lens, int num_seqs, int hq, int D,
                    int partition_size, int max_partitions) {
  if (num_seqs < 0 || hq <= 0 || D <= 0 || partition_size <= 0 || max_partitions <= 0)
    return ORC_EARG;
  for (int s = 0; s < num_seqs; ++s) {
    int ctx = ctx_lens[s];
    int np = ctx <= 0 ? 0 : (ctx + partition_size - 1) / partition_size;
    if (np > max_partitions) return ORC_EARG;
    for (int h = 0; h < hq; ++h) {
      int64_t base = ((int64_t)s * hq + h) * max_partitions;
      double* dst = out + ((int64_t)s * hq + h) * D;
      for (int d = 0; d < D; ++d) dst[d] = 0.0;
      if (np == 0) continue;
      double M = -INFINITY;
      for (int p = 0; p < np; ++p)
        if (m[base + p] > M) M = m[base + p];
      double den = 0.0;
      for (int p = 0; p < np; ++p) {
        double w = l[base + p] * exp(m[base + p] - M);
        den += w;
        for (int d = 0; d < D; ++d) dst[d] += w * o[(base + p) * D + d];
      }
      for (int d = 0; d < D; ++d) dst[d] /= den;
    }
  }
  return ORC_OK;
}

/* Multi-token queries (chunked prefill, speculative decoding).
 * query [num_tokens][hq][D]; query_start_loc [num_seqs + 1], non-decreasing
 * from 0 (sequence s owns query rows qsl[s] .. qsl[s+1]-1, q_s of them);
 * ctx_lens [num_seqs] count all positions in the pool, the new tokens'
 * included, so q_s <= ctx_s. Row qsl[s] + i is the token at position
 * ctx_s - q_s + i and attends positions 0 .. ctx_s - q_s + i.
 * out [num_tokens][hq][D]. */
int orc_attention_varlen(double* out, const void* q, const void* k_pool, const void* v_pool,
                         int dtype, const int32_t* block_table, const int32_t* query_start_loc,
                         const int32_t* ctx_lens, int num_seqs, int hq, int hkv, int D, int B,
                         int64_t num_blocks, int max_blocks, float scale, int threads) {
  int rc = check_common(hq, hkv, D, B, dtype, num_seqs);
  if (rc != ORC_OK) return rc;
  if (!query_start_loc || query_start_loc[0] != 0) return ORC_EARG;
  for (int s = 0; s < num_seqs; ++s)
    if (query_start_loc[s + 1] < query_start_loc[s]) return ORC_EARG;
  job_t j;
  memset(&j, 0, sizeof j);
  j.q = q; j.k_pool = k_pool; j.v_pool = v_pool; j.dtype = dtype;
  j.block_table = block_table; j.ctx_lens = ctx_lens;
  j.hq = hq; j.hkv = hkv; j.D = D; j.B = B;
  j.num_blocks = num_blocks; j.max_blocks = max_blocks;
  j.scale = (double)scale; j.seqs = NULL; j.n_seqs = num_seqs;
  j.qsl = query_start_loc;
  j.partition_size = 0; j.out = out;
  return run_job(&j, threads);
}
