/*
 * kvc_oracle.c -- plain, slow CPU oracle for KV-cache decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library links, includes or calls
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg load it.  It shares no code, header, table or constant with the HIP
 * path.
 *
 * Every floating-point step runs in double precision on the exact input
 * values (bf16 inputs are widened exactly).  There is no blocking, fusion or
 * reordering beyond the definitions cited at each function.
 *
 * Sources (the four web pages this library follows):
 *   [I1] "Inference-1", brunomaga.github.io -- sections "KV cache",
 *        "PagedAttention: memory management for the KV cache", "FlashAttention",
 *        "FlashDecoding", "Smaller KV caches: MQA, GQA and MLA".
 *   [VN] "Inference o quy mo lon: KV cache, prefill va decode",
 *        blog.truongducdung.dev -- section 05 "PagedAttention va prefix
 *        caching" (sub-section "Block table") and section 07 "FlashAttention"
 *        (sub-section "Online softmax").
 *   [I2] "Inference-2", brunomaga.github.io -- sections "Draft-model
 *        speculative decoding" and "CUDA graphs".
 *   [EI] "Efficient Inference", learn.obvix.io -- the KV-cache passage (static
 *        cache written in place) and the paged-attention passage (block table).
 *
 * Parity pins: every function here is pinned by CPU tests against closed
 * forms, brute force, library routines and the pages' printed numbers; none is
 * "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* status codes (the same integers the library returns; values restated here) */
#define REF_OK 0
#define REF_ERR_ARG (-1)
#define REF_ERR_CAPACITY (-5)
#define REF_ERR_NO_BLOCKS (-6)
#define REF_ERR_DATA (-8)

/* element types: 0 = bfloat16 (1 sign, 8 exponent, 7 mantissa bits), 1 = IEEE
 * float32, 2 = IEEE float64 (dequantized FP8 caches are handed over widened) */
#define REF_BF16 0
#define REF_F32 1
#define REF_F64 2

/* Exact widening of one stored element to double.  A bf16 value is the upper
 * half of the float32 with the same bits ([I2] "Quantization", number-format
 * table: bf16 keeps float32's 8-bit exponent and 7 of its mantissa bits). */
static double load_elem(const void* base, size_t idx, int dtype) {
  if (dtype == REF_F64) return ((const double*)base)[idx];
  if (dtype == REF_F32) return (double)((const float*)base)[idx];
  uint32_t u = (uint32_t)((const uint16_t*)base)[idx] << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Round a double once, to nearest with ties to even, to bf16 (8 significant
 * bits, exponent range of float32).  Returns the raw 16-bit pattern. */
uint16_t kvc_ref_round_bf16(double x) {
  if (isnan(x)) return 0x7FC0;
  double ax = fabs(x);
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  if (ax == 0.0) return sign;
  int e;
  frexp(ax, &e); /* ax in [2^(e-1), 2^e) */
  int eq = e < -125 ? -125 : e; /* below 2^-126 the spacing stays 2^-133 */
  double ulp = ldexp(1.0, eq - 8);
  double r = nearbyint(ax / ulp) * ulp; /* default rounding mode: ties to even */
  if (r > 3.38953138925153547590470800371487866880e+38) return sign | 0x7F80; /* +-inf */
  float f = (float)r; /* exact: r has at most 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(sign | (uint16_t)((u >> 16) & 0x7FFF));
}

/* ------------------------------------------------------------------------ */
/* Block table: on-demand allocation of fixed-size blocks.
 *
 * [I1] "PagedAttention": the cache is split into fixed-size blocks allocated
 * on demand, and a per-sequence table maps logical blocks to physical ones.
 * [VN] 05 "Block table": a new block is taken only when the last one is full,
 * so at most the tail of the last block is wasted; default 16 tokens.
 * [EI] paged-attention passage: the table maps logical token positions to
 * physical block indices; blocks come from a free pool.
 *
 * Reading of the unstated order: sequences in batch order, each sequence's
 * missing logical blocks in increasing order, the free list consumed front to
 * back.  All or nothing: on any error nothing is written.
 *
 * seq_lens[b] tokens are already held in ceil(seq_lens[b]/bs) blocks; the new
 * tokens of sequence b are cu_new[b] .. cu_new[b+1]-1.  The token at logical
 * position pos lives in slot table[b][pos/bs]*bs + pos%bs.
 */
int kvc_ref_block_table(int B, int bs, int max_blocks, int N, const int32_t* seq_lens,
                        const int32_t* cu_new, int32_t* table, const int32_t* free_list,
                        int32_t* head, int32_t* slots) {
  if (B < 0 || bs <= 0 || max_blocks <= 0 || N < 0) return REF_ERR_ARG;
  long need = 0;
  for (int b = 0; b < B; ++b) {
    long len = seq_lens[b];
    long n = (long)cu_new[b + 1] - cu_new[b];
    if (len < 0 || n < 0) return REF_ERR_DATA;
    long have = (len + bs - 1) / bs;
    long want = (len + n + bs - 1) / bs;
    if (want > max_blocks) return REF_ERR_CAPACITY;
    need += want - have;
  }
  if (*head < 0 || (long)*head + need > N) return REF_ERR_NO_BLOCKS;

  for (int b = 0; b < B; ++b) {
    long len = seq_lens[b];
    long n = (long)cu_new[b + 1] - cu_new[b];
    long have = (len + bs - 1) / bs;
    long want = (len + n + bs - 1) / bs;
    for (long i = have; i < want; ++i) {
      table[(long)b * max_blocks + i] = free_list[*head];
      *head += 1;
    }
  }
  for (int b = 0; b < B; ++b) {
    long len = seq_lens[b];
    long n = (long)cu_new[b + 1] - cu_new[b];
    for (long t = 0; t < n; ++t) {
      long pos = len + t;
      long blk = table[(long)b * max_blocks + pos / bs];
      slots[cu_new[b] + t] = (int32_t)(blk * bs + pos % bs);
    }
  }
  return REF_OK;
}

/* ------------------------------------------------------------------------ */
/* Append: write the new tokens' key and value rows into the cache in place.
 *
 * [EI] KV-cache passage: the static cache is preallocated for the maximum
 * length, the new rows are written into the slice at the current length, the
 * length grows by the number of new tokens, and writing past the capacity is
 * an error.  [I2] "CUDA graphs": the static cache is written in place at the
 * new tokens' positions.  [I1] "KV cache": only the new token's key and value
 * are computed and appended; everything cached stays untouched.
 *
 * Layouts (element = esize bytes, copied bit for bit, no conversion):
 *   new rows  k_new, v_new : [total_new][Hkv][D], sequence b owns rows
 *                            cu_new[b] .. cu_new[b+1]-1
 *   contiguous (bs == 0)   : cache [B][Hkv][S_max][D]
 *   paged      (bs  > 0)   : pool  [N][Hkv][bs][D], token i goes to slot slots[i]
 * seq_lens_out[b] = seq_lens[b] + n_new_b, or seq_lens[b] when a contiguous
 * sequence would pass S_max (then none of its rows is written).  A paged token
 * whose slot lies outside the pool is skipped alone; lengths still advance.
 * Returns the first error met (everything else is still written).
 */
int kvc_ref_append(int B, int Hkv, int D, int esize, int bs, int S_max, int N, const void* k_new,
                   const void* v_new, const int32_t* seq_lens, const int32_t* cu_new,
                   const int32_t* slots, void* k_cache, void* v_cache, int32_t* seq_lens_out) {
  if (B < 0 || Hkv <= 0 || D <= 0 || esize <= 0 || bs < 0) return REF_ERR_ARG;
  int status = REF_OK;
  size_t row = (size_t)D * esize;
  for (int b = 0; b < B; ++b) {
    long len = seq_lens[b];
    long n = (long)cu_new[b + 1] - cu_new[b];
    seq_lens_out[b] = (int32_t)len;
    if (len < 0 || n < 0) {
      if (status == REF_OK) status = REF_ERR_DATA;
      continue;
    }
    if (bs == 0 && len + n > S_max) {
      if (status == REF_OK) status = REF_ERR_CAPACITY;
      continue;
    }
    for (long t = 0; t < n; ++t) {
      long src_tok = cu_new[b] + t;
      if (bs > 0 && (slots[src_tok] < 0 || slots[src_tok] >= (long)N * bs)) {
        if (status == REF_OK) status = REF_ERR_DATA; /* this token is not written */
        continue;
      }
      for (int g = 0; g < Hkv; ++g) {
        size_t src = ((size_t)src_tok * Hkv + g) * row;
        size_t dst;
        if (bs == 0) {
          dst = (((size_t)b * Hkv + g) * S_max + (size_t)(len + t)) * row;
        } else {
          long s = slots[src_tok];
          dst = (((size_t)(s / bs) * Hkv + g) * bs + (size_t)(s % bs)) * row;
        }
        memcpy((char*)k_cache + dst, (const char*)k_new + src, row);
        memcpy((char*)v_cache + dst, (const char*)v_new + src, row);
      }
    }
    seq_lens_out[b] = (int32_t)(len + n);
  }
  return status;
}

/* Element index of key/value j of sequence b, KV head g, in a contiguous or
 * paged cache; -1 when the block table points outside the pool. */
static long cache_row(int b, int g, long j, int Hkv, int D, int bs, int S_max, int max_blocks,
                      int N, const int32_t* table) {
  if (bs == 0) return (((long)b * Hkv + g) * S_max + j) * D;
  long blk = table[(long)b * max_blocks + j / bs];
  if (blk < 0 || blk >= N) return -1;
  return ((blk * Hkv + g) * bs + j % bs) * D;
}

/* Gather sequence b's first L logical rows, in token order, out of a cache
 * into a plain [Hkv][L][D] array (bytes copied unchanged).  Used to compare a
 * paged cache with a contiguous one. */
int kvc_ref_gather(int b, int L, int Hkv, int D, int esize, int bs, int S_max, int max_blocks,
                   int N, const int32_t* table, const void* cache, void* out) {
  size_t row = (size_t)D * esize;
  for (int g = 0; g < Hkv; ++g)
    for (long j = 0; j < L; ++j) {
      long e = cache_row(b, g, j, Hkv, D, bs, S_max, max_blocks, N, table);
      if (e < 0) return REF_ERR_DATA;
      memcpy((char*)out + (((size_t)g * L + j) * row), (const char*)cache + (size_t)e * esize, row);
    }
  return REF_OK;
}

/* ------------------------------------------------------------------------ */
/* Attention of n_q new query rows over L cached keys of one sequence.
 *
 * Definition ([I1] "Why attention matters"): softmax(Q K^T / sqrt(d)) V, with
 * the scale passed in.  Mask ([I1] "KV cache", the function that attends Sq new
 * tokens over Sk keys): when Sq > 1, new row r sees keys 0 .. Sk - Sq + r (a
 * lower-triangular mask shifted by Sk - Sq); a single row sees every key,
 * including its own just-appended one.  Grouping ([I1] "Smaller KV caches",
 * the GQA class; [EI] minimal GQA forward): with G = Hq / Hkv, query head h
 * reads KV head h / G (consecutive heads share a group).
 *
 * Layouts: q [n_q][Hq][D], k and v [Hkv][L][D] (elements of type dtype),
 * out [n_q][Hq][D] in double.  Every step in double: scores, maximum,
 * exponentials, sum, weighted sum, one division.
 */
int kvc_ref_attention(int n_q, int Hq, int Hkv, int D, int L, int dtype, const void* q,
                      const void* k, const void* v, double scale, double* out) {
  if (n_q <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0) return REF_ERR_ARG;
  if (Hq % Hkv != 0) return REF_ERR_ARG;
  if (L < n_q) return REF_ERR_DATA;
  int G = Hq / Hkv;
  double* p = (double*)malloc(sizeof(double) * (size_t)L);
  if (!p) return REF_ERR_ARG;
  for (int r = 0; r < n_q; ++r)
    for (int h = 0; h < Hq; ++h) {
      int g = h / G;
      long last = (long)L - n_q + r; /* keys 0..last are visible */
      double m = -INFINITY;
      for (long j = 0; j <= last; ++j) {
        double s = 0.0;
        for (int d = 0; d < D; ++d)
          s += load_elem(q, ((size_t)r * Hq + h) * D + d, dtype) *
               load_elem(k, ((size_t)g * L + j) * D + d, dtype);
        p[j] = s * scale;
        if (p[j] > m) m = p[j];
      }
      double l = 0.0;
      for (long j = 0; j <= last; ++j) {
        p[j] = exp(p[j] - m);
        l += p[j];
      }
      for (int d = 0; d < D; ++d) {
        double acc = 0.0;
        for (long j = 0; j <= last; ++j) acc += p[j] * load_elem(v, ((size_t)g * L + j) * D + d, dtype);
        out[((size_t)r * Hq + h) * D + d] = acc / l;
      }
    }
  free(p);
  return REF_OK;
}

/* The same definition evaluated straight out of a cache (contiguous or paged),
 * reading each sequence's keys in logical order through its block table.
 *   q   [B][n_q][Hq][D]          out [B][n_q][Hq][D] (double)
 *   seq_lens[b] keys attended (already appended), n_q <= seq_lens[b] <= capacity
 * With rows_only != NULL only the (b, h) pairs with rows_only[b*Hq+h] != 0 are
 * computed (the others are left untouched): used to check sampled outputs of a
 * full-size workload. */
int kvc_ref_cache_attention(int B, int n_q, int Hq, int Hkv, int D, int dtype, int bs, int S_max,
                            int max_blocks, int N, const void* q, const void* k_cache,
                            const void* v_cache, const int32_t* seq_lens, const int32_t* table,
                            double scale, const uint8_t* rows_only, double* out) {
  if (B < 0 || n_q <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv != 0) return REF_ERR_ARG;
  int G = Hq / Hkv;
  long cap = bs == 0 ? S_max : (long)max_blocks * bs;
  long maxL = 0;
  for (int b = 0; b < B; ++b) {
    if (seq_lens[b] < n_q || seq_lens[b] > cap) return REF_ERR_DATA;
    if (seq_lens[b] > maxL) maxL = seq_lens[b];
  }
  double* p = (double*)malloc(sizeof(double) * (size_t)(maxL > 0 ? maxL : 1));
  if (!p) return REF_ERR_ARG;
  int status = REF_OK;
  for (int b = 0; b < B && status == REF_OK; ++b)
    for (int h = 0; h < Hq && status == REF_OK; ++h) {
      if (rows_only && !rows_only[(size_t)b * Hq + h]) continue;
      int g = h / G;
      long L = seq_lens[b];
      for (int r = 0; r < n_q; ++r) {
        long last = L - n_q + r;
        size_t qo = (((size_t)b * n_q + r) * Hq + h) * D;
        double m = -INFINITY;
        for (long j = 0; j <= last; ++j) {
          long e = cache_row(b, g, j, Hkv, D, bs, S_max, max_blocks, N, table);
          if (e < 0) {
            status = REF_ERR_DATA;
            break;
          }
          double s = 0.0;
          for (int d = 0; d < D; ++d)
            s += load_elem(q, qo + d, dtype) * load_elem(k_cache, (size_t)e + d, dtype);
          p[j] = s * scale;
          if (p[j] > m) m = p[j];
        }
        if (status != REF_OK) break;
        double l = 0.0;
        for (long j = 0; j <= last; ++j) {
          p[j] = exp(p[j] - m);
          l += p[j];
        }
        for (int d = 0; d < D; ++d) {
          double acc = 0.0;
          for (long j = 0; j <= last; ++j) {
            long e = cache_row(b, g, j, Hkv, D, bs, S_max, max_blocks, N, table);
            acc += p[j] * load_elem(v_cache, (size_t)e + d, dtype);
          }
          out[qo + d] = acc / l;
        }
      }
    }
  free(p);
  return status;
}

/* ------------------------------------------------------------------------ */
/* Split-KV evaluation with the online softmax -- the algorithm, not the
 * definition.  It is pinned against kvc_ref_attention (they must agree to
 * rounding) to show that a partitioned pass is exact attention.
 *
 * [VN] 07 "Online softmax": one pass keeps a running maximum m and a running
 * sum l; when m grows, the sum so far is multiplied by exp(m_old - m_new).
 * [I1] "FlashAttention": the unnormalised output O is corrected by the same
 * factor, and the result is O / l after the last key.
 * [I1] "FlashDecoding": the keys are split into chunks, each chunk yields a
 * partial output with its maximum and sum, and a final reduction combines them
 * with the same rescaling.
 *
 * Chunks hold P consecutive keys; a row's chunk with no visible key keeps
 * m = -inf, l = 0, O = 0 and gets weight 0 in the combine.
 */
int kvc_ref_attention_split(int n_q, int Hq, int Hkv, int D, int L, int dtype, const void* q,
                            const void* k, const void* v, double scale, int P, double* out) {
  if (n_q <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || P <= 0 || Hq % Hkv != 0) return REF_ERR_ARG;
  if (L < n_q) return REF_ERR_DATA;
  int G = Hq / Hkv;
  long n_chunks = (L + P - 1) / P;
  double* cm = (double*)malloc(sizeof(double) * (size_t)n_chunks);
  double* cl = (double*)malloc(sizeof(double) * (size_t)n_chunks);
  double* cO = (double*)malloc(sizeof(double) * (size_t)n_chunks * D);
  if (!cm || !cl || !cO) {
    free(cm);
    free(cl);
    free(cO);
    return REF_ERR_ARG;
  }
  for (int r = 0; r < n_q; ++r)
    for (int h = 0; h < Hq; ++h) {
      int g = h / G;
      long last = (long)L - n_q + r;
      for (long c = 0; c < n_chunks; ++c) {
        double m = -INFINITY, l = 0.0;
        double* O = cO + c * D;
        for (int d = 0; d < D; ++d) O[d] = 0.0;
        for (long j = c * P; j < (c + 1) * P && j <= last; ++j) {
          double s = 0.0;
          for (int d = 0; d < D; ++d)
            s += load_elem(q, ((size_t)r * Hq + h) * D + d, dtype) *
                 load_elem(k, ((size_t)g * L + j) * D + d, dtype);
          s *= scale;
          double m_new = s > m ? s : m;
          double corr = exp(m - m_new); /* exp(-inf) = 0 on the first key */
          double e = exp(s - m_new);
          l = l * corr + e;
          for (int d = 0; d < D; ++d)
            O[d] = O[d] * corr + e * load_elem(v, ((size_t)g * L + j) * D + d, dtype);
          m = m_new;
        }
        cm[c] = m;
        cl[c] = l;
      }
      double M = -INFINITY;
      for (long c = 0; c < n_chunks; ++c)
        if (cm[c] > M) M = cm[c];
      double den = 0.0;
      for (long c = 0; c < n_chunks; ++c)
        if (cm[c] != -INFINITY) den += exp(cm[c] - M) * cl[c];
      for (int d = 0; d < D; ++d) {
        double num = 0.0;
        for (long c = 0; c < n_chunks; ++c)
          if (cm[c] != -INFINITY) num += exp(cm[c] - M) * cO[c * D + d];
        out[((size_t)r * Hq + h) * D + d] = num / den;
      }
    }
  free(cm);
  free(cl);
  free(cO);
  return REF_OK;
}

/* ------------------------------------------------------------------------ */
/* Block lifecycle: sharing, copy-on-write, rollback.
 *
 * [VN] 05 "Chia se block va copy-on-write": every physical block carries a
 * reference count; parallel samples share the prompt's blocks and a sample
 * that must write into a shared block first copies it.  [I1] "PagedAttention":
 * blocks shared by several sequences are copied only when one of them writes.
 * [EI] paged-attention passage: a finished request's blocks return to the free
 * pool.  [I2] "Draft-model speculative decoding": after verification the
 * target's cache is truncated to the accepted tokens.
 *
 * Readings (the pages fix none of these details):
 *   - refs[blk] counts the owners beyond the first: a block held by one
 *     sequence, or free, has 0;
 *   - the free pool is the tail free_list[head .. N) of the allocation list;
 *     freed blocks are pushed back just below head, in increasing block id;
 *   - copy-on-write is decided on the state at the start of the call: every
 *     sequence about to append into a partly filled last block that is
 *     shared takes a fresh block (batch order, from the free list front),
 *     gets a copy of the whole block (all heads, K and V) and drops one
 *     reference; an original left with no owner is freed.
 */

static int cmp_i32(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/* Push the blocks in `cand` whose refs fell below zero (or every candidate
 * when refs == NULL) back onto the free list, once each, in increasing id. */
static int push_freed(int32_t* cand, long nc, int32_t* free_list, int32_t* head, int32_t* refs) {
  qsort(cand, (size_t)nc, sizeof(int32_t), cmp_i32);
  long nf = 0;
  for (long i = 0; i < nc; ++i) {
    if (i > 0 && cand[i] == cand[i - 1]) continue;
    if (refs && refs[cand[i]] >= 0) continue;
    cand[nf++] = cand[i];
  }
  if (*head - nf < 0) return REF_ERR_DATA;
  *head -= (int32_t)nf;
  for (long i = 0; i < nf; ++i) {
    free_list[*head + i] = cand[i];
    if (refs) refs[cand[i]] = 0;
  }
  return REF_OK;
}

/* Fork: child i takes parent i's blocks (table row and length) and each of
 * those blocks gains one reference.  Children must be empty and distinct, and
 * no sequence may be both a parent and a child in one call (the forks of a
 * call are independent of each other).  All or nothing. */
int kvc_ref_fork(int B, int bs, int max_blocks, int N, const int32_t* parents,
                 const int32_t* children, int n, int32_t* seq_lens, int32_t* table, int32_t* refs) {
  for (int i = 0; i < n; ++i) {
    int p = parents[i], c = children[i];
    if (p < 0 || p >= B || c < 0 || c >= B || p == c) return REF_ERR_DATA;
    if (seq_lens[c] != 0 || seq_lens[p] < 0 || seq_lens[p] > (long)max_blocks * bs) return REF_ERR_DATA;
  }
  for (int i = 0; i < n; ++i)
    for (int k = 0; k < n; ++k) {
      if (k != i && children[k] == children[i]) return REF_ERR_DATA;
      if (parents[k] == children[i]) return REF_ERR_DATA;
    }
  for (int i = 0; i < n; ++i) {
    int p = parents[i], c = children[i];
    long nb = ((long)seq_lens[p] + bs - 1) / bs;
    for (long j = 0; j < nb; ++j) {
      int32_t blk = table[(long)p * max_blocks + j];
      table[(long)c * max_blocks + j] = blk;
      if (blk >= 0 && blk < N) refs[blk] += 1;
    }
    seq_lens[c] = seq_lens[p];
  }
  return REF_OK;
}

/* Truncate: sequence b keeps new_lens[b] <= seq_lens[b] tokens; its logical
 * blocks from ceil(new_len/bs) on are released (table entry -1).  A released
 * block with extra references loses one; otherwise it is freed.  All or
 * nothing on a bad length. */
int kvc_ref_truncate(int B, int bs, int max_blocks, int N, const int32_t* seq_lens,
                     const int32_t* new_lens, int32_t* table, int32_t* free_list, int32_t* head,
                     int32_t* refs, int32_t* seq_lens_out) {
  long total = 0;
  if (*head < 0 || *head > N) return REF_ERR_DATA;
  for (int b = 0; b < B; ++b) {
    if (new_lens[b] < 0 || new_lens[b] > seq_lens[b]) return REF_ERR_DATA;
    if (seq_lens[b] > (long)max_blocks * bs) return REF_ERR_DATA;
    total += ((long)seq_lens[b] + bs - 1) / bs - ((long)new_lens[b] + bs - 1) / bs;
  }
  int32_t* cand = (int32_t*)malloc(sizeof(int32_t) * (size_t)(total > 0 ? total : 1));
  if (!cand) return REF_ERR_ARG;
  long nc = 0;
  for (int b = 0; b < B; ++b) {
    long old_nb = ((long)seq_lens[b] + bs - 1) / bs;
    long new_nb = ((long)new_lens[b] + bs - 1) / bs;
    for (long j = old_nb - 1; j >= new_nb; --j) {
      int32_t blk = table[(long)b * max_blocks + j];
      table[(long)b * max_blocks + j] = -1;
      if (blk < 0 || blk >= N) continue;
      if (refs) refs[blk] -= 1;
      cand[nc++] = blk;
    }
    seq_lens_out[b] = new_lens[b];
  }
  int st = push_freed(cand, nc, free_list, head, refs);
  free(cand);
  return st;
}

/* Copy-on-write before an append (see the readings above).  cow_src/cow_dst
 * receive the copied pair of every sequence (-1 when none).  The block data
 * (Hkv * bs * D elements of esize bytes, K and V) is copied in the pools.
 * All or nothing when the free list cannot cover the copies. */
int kvc_ref_cow(int B, int bs, int max_blocks, int N, int Hkv, int D, int esize,
                const int32_t* seq_lens, const int32_t* cu_new, int32_t* table,
                int32_t* free_list, int32_t* head, int32_t* refs, void* k_pool, void* v_pool,
                int32_t* cow_src, int32_t* cow_dst) {
  long need = 0;
  for (int b = 0; b < B; ++b) {
    long len = seq_lens[b], n = (long)cu_new[b + 1] - cu_new[b];
    cow_src[b] = cow_dst[b] = -1;
    if (n <= 0 || len % bs == 0) continue;
    int32_t blk = table[(long)b * max_blocks + len / bs];
    if (blk >= 0 && blk < N && refs[blk] > 0) need += 1;
  }
  if (*head + need > N) return REF_ERR_NO_BLOCKS;
  /* decide every copy on the state at the start of the call */
  int32_t* cand = (int32_t*)malloc(sizeof(int32_t) * (size_t)(need > 0 ? need : 1));
  if (!cand) return REF_ERR_ARG;
  long nc = 0;
  for (int b = 0; b < B; ++b) {
    long len = seq_lens[b], n = (long)cu_new[b + 1] - cu_new[b];
    if (n <= 0 || len % bs == 0) continue;
    int32_t blk = table[(long)b * max_blocks + len / bs];
    if (blk >= 0 && blk < N && refs[blk] > 0) {
      cow_src[b] = blk;
      cow_dst[b] = free_list[*head];
      *head += 1;
      cand[nc++] = blk;
    }
  }
  size_t bytes = (size_t)Hkv * bs * D * esize;
  for (int b = 0; b < B; ++b) {
    if (cow_src[b] < 0) continue;
    long len = seq_lens[b];
    memcpy((char*)k_pool + (size_t)cow_dst[b] * bytes, (const char*)k_pool + (size_t)cow_src[b] * bytes, bytes);
    memcpy((char*)v_pool + (size_t)cow_dst[b] * bytes, (const char*)v_pool + (size_t)cow_src[b] * bytes, bytes);
    table[(long)b * max_blocks + len / bs] = cow_dst[b];
    refs[cow_src[b]] -= 1;
  }
  int st = push_freed(cand, nc, free_list, head, refs);
  free(cand);
  return st;
}

/* ------------------------------------------------------------------------ */
/* FP8 KV cache.
 *
 * [I2] "Quantization" number-format table: FP8 E4M3 (1 sign, 4 exponent, 3
 * mantissa bits, largest value 448) and FP8 E5M2 (1/5/2, largest 57,344), both
 * used for the KV cache.  [VN] 03 "KV cache quantization": storing K and V in
 * FP8 halves the cache and the bytes read per decode step; [I2] "KV cache
 * quantization": FP8 with per-token or per-channel scales is nearly lossless.
 *
 * Readings (the pages fix the formats, not the encoding details):
 *   - E4M3 is the variant with no infinities whose only NaN pattern is
 *     S.1111.111 (so 448 = 1.1100 x 2^8 is the largest value); E5M2 follows the
 *     IEEE layout (exponent 11111 holds infinities and NaNs);
 *   - exponent bias 2^(e-1) - 1 (7 and 15), subnormals when the exponent field
 *     is zero;
 *   - one fp32 scale per (token, KV head) for K and for V: s = amax / FMAX with
 *     amax the largest |x| of that row (float32 division), and the code of x
 *     is the FP8 value nearest to x / s (float32 division), ties to the even
 *     code, saturated to +-FMAX; a row of zeros has s = 0 and codes 0;
 *   - the dequantized element is decode(code) * s, exactly (in double).
 */
#define REF_E4M3 0
#define REF_E5M2 1

static int fp8_mant_bits(int fmt) { return fmt == REF_E4M3 ? 3 : 2; }
static int fp8_bias(int fmt) { return fmt == REF_E4M3 ? 7 : 15; }

/* Value of an FP8 code, straight from the bit fields. */
double kvc_ref_fp8_decode(int code, int fmt) {
  int mb = fp8_mant_bits(fmt), eb = 7 - mb;
  int sign = (code >> 7) & 1, e = (code >> mb) & ((1 << eb) - 1), m = code & ((1 << mb) - 1);
  int emax = (1 << eb) - 1;
  double v;
  if (fmt == REF_E4M3 && e == emax && m == (1 << mb) - 1) return NAN;
  if (fmt == REF_E5M2 && e == emax) return m ? NAN : (sign ? -INFINITY : INFINITY);
  if (e == 0)
    v = ldexp((double)m, 1 - fp8_bias(fmt) - mb); /* subnormal: m * 2^(1 - bias - mb) */
  else
    v = ldexp(1.0 + (double)m / (1 << mb), e - fp8_bias(fmt));
  return sign ? -v : v;
}

double kvc_ref_fp8_max(int fmt) { return fmt == REF_E4M3 ? 448.0 : 57344.0; }

/* Nearest FP8 code to the finite value y: the non-negative codes from 0 up
 * to the largest finite one hold increasing values, so the nearest is found
 * among them (ties to the code with an even mantissa), with the sign bit set
 * for negative y.  Values beyond the largest finite one saturate to it. */
int kvc_ref_fp8_encode(double y, int fmt) {
  int sign = y < 0 ? 0x80 : 0;
  double a = fabs(y);
  int top = fmt == REF_E4M3 ? 0x7E : 0x7B; /* largest finite code */
  if (a >= kvc_ref_fp8_decode(top, fmt)) return sign | top;
  int lo = 0, hi = top; /* invariant: value(lo) <= a < value(hi) */
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (kvc_ref_fp8_decode(mid, fmt) <= a) lo = mid; else hi = mid;
  }
  double dlo = a - kvc_ref_fp8_decode(lo, fmt), dhi = kvc_ref_fp8_decode(hi, fmt) - a;
  int c = dlo < dhi ? lo : dhi < dlo ? hi : ((lo & 1) == 0 ? lo : hi);
  return sign | c;
}

/* Quantize n rows of D bf16 elements (bit patterns): one scale per row. */
void kvc_ref_quantize_rows(const uint16_t* x, long n, int D, int fmt, uint8_t* codes,
                           float* scales) {
  for (long r = 0; r < n; ++r) {
    float amax = 0.f;
    for (int d = 0; d < D; ++d) {
      float v = (float)fabs(load_elem(x, (size_t)r * D + d, REF_BF16));
      if (v > amax) amax = v;
    }
    float s = amax / (float)kvc_ref_fp8_max(fmt);
    scales[r] = s;
    for (int d = 0; d < D; ++d) {
      float v = (float)load_elem(x, (size_t)r * D + d, REF_BF16);
      codes[(size_t)r * D + d] = s == 0.f ? 0 : (uint8_t)kvc_ref_fp8_encode((double)(v / s), fmt);
    }
  }
}

/* The values an FP8 cache holds: decode(code) * scale, in double (exact). */
void kvc_ref_dequantize_rows(const uint8_t* codes, const float* scales, long n, int D, int fmt,
                             double* out) {
  for (long r = 0; r < n; ++r)
    for (int d = 0; d < D; ++d)
      out[(size_t)r * D + d] = kvc_ref_fp8_decode(codes[(size_t)r * D + d], fmt) * (double)scales[r];
}

/* ------------------------------------------------------------------------ */
/* MLA latent decode.
 *
 * [I1] "Smaller KV caches: MQA, GQA and MLA": MLA caches one latent vector per
 * token; with the key and value up-projections absorbed into the query and
 * output projections, attention runs directly over the cached latents, which
 * act as both keys and values -- one large key-value head shared by every
 * query head.  [VN] 03 "MLA: compress K/V into a latent": a small decoupled
 * key carrying RoPE is cached beside the latent; per token d_c + d_h^R values
 * are cached (512 + 64).  [EI] GQA passage: MLA stores a low-rank latent of
 * dimension C = 512.
 *
 * Readings: a cache row is [latent (Dv) | rope key (Dk - Dv)]; the absorbed
 * query of each head has the same Dk dims (absorbed latent query, then rope
 * query); the score is scale * (q . row) over all Dk dims; the value is the
 * row's first Dv dims (the latent); the output is the weighted latent [Dv],
 * which the absorbed value up-projection then maps per head (outside this
 * step).  Verify rows see keys 0 .. L - n_q + r as for ordinary attention.
 *
 *   q [n_q][Hq][Dk], c [L][Dk] (bf16 bit patterns), out [n_q][Hq][Dv] (double)
 */
int kvc_ref_mla_attention(int n_q, int Hq, int Dk, int Dv, int L, const uint16_t* q,
                          const uint16_t* c, double scale, double* out) {
  if (n_q <= 0 || Hq <= 0 || Dk <= 0 || Dv <= 0 || Dv > Dk) return REF_ERR_ARG;
  if (L < n_q) return REF_ERR_DATA;
  double* p = (double*)malloc(sizeof(double) * (size_t)L);
  if (!p) return REF_ERR_ARG;
  for (int r = 0; r < n_q; ++r)
    for (int h = 0; h < Hq; ++h) {
      long last = (long)L - n_q + r;
      double m = -INFINITY;
      for (long t = 0; t <= last; ++t) {
        double s = 0.0;
        for (int d = 0; d < Dk; ++d)
          s += load_elem(q, ((size_t)r * Hq + h) * Dk + d, REF_BF16) *
               load_elem(c, (size_t)t * Dk + d, REF_BF16);
        p[t] = s * scale;
        if (p[t] > m) m = p[t];
      }
      double l = 0.0;
      for (long t = 0; t <= last; ++t) {
        p[t] = exp(p[t] - m);
        l += p[t];
      }
      for (int d = 0; d < Dv; ++d) {
        double acc = 0.0;
        for (long t = 0; t <= last; ++t) acc += p[t] * load_elem(c, (size_t)t * Dk + d, REF_BF16);
        out[((size_t)r * Hq + h) * Dv + d] = acc / l;
      }
    }
  free(p);
  return REF_OK;
}

/* ------------------------------------------------------------------------ */
/* Many sequences at once on all host cores -- a timing aid for the CPU
 * baseline, not a different computation.  Every (sequence, query head) pair
 * is one OpenMP iteration that evaluates the definition above for that head
 * alone: kvc_ref_attention (dv == 0) or kvc_ref_mla_attention (dv > 0, one
 * latent head, bf16).  The head's query rows are copied out, its KV head's
 * rows are passed in place, and the head's result is copied back, so every
 * number is the one the single-threaded definition gives.
 *   q[s]   [n_q][Hq][Dk] (dtype)
 *   k[s], v[s] [Hkv][L[s]][Dk] (dtype); dv > 0: k[s] = [L[s]][Dk] latent rows, v unused
 *   out[s] [n_q][Hq][Dout] double, Dout = dv > 0 ? dv : Dk
 * Returns the first failing status (REF_OK when all succeed); *threads
 * receives the number of threads that ran. */
int kvc_ref_attention_many(int nseq, int n_q, int Hq, int Hkv, int Dk, int dv, int dtype,
                           const int32_t* L, const void* const* q, const void* const* k,
                           const void* const* v, double scale, double* const* out,
                           int* threads) {
  if (nseq < 0 || n_q <= 0 || Hq <= 0 || Hkv <= 0 || Dk <= 0 || Hq % Hkv != 0) return REF_ERR_ARG;
  if (dv > 0 && (Hkv != 1 || dtype != REF_BF16 || dv > Dk)) return REF_ERR_ARG;
  const size_t es = dtype == REF_BF16 ? 2 : dtype == REF_F32 ? 4 : 8;
  const int G = Hq / Hkv, Dout = dv > 0 ? dv : Dk;
  const long pairs = (long)nseq * Hq;
  int status = REF_OK, team = 1;
#pragma omp parallel
  {
#pragma omp single
    {
#ifdef _OPENMP
      team = omp_get_num_threads();
#endif
    }
    char* qh = (char*)malloc(es * (size_t)n_q * Dk);
    double* oh = (double*)malloc(sizeof(double) * (size_t)n_q * Dout);
#pragma omp for schedule(dynamic, 1)
    for (long i = 0; i < pairs; ++i) {
      const int s = (int)(i / Hq), h = (int)(i % Hq), g = h / G;
      int st = REF_ERR_ARG;
      if (qh && oh) {
        for (int r = 0; r < n_q; ++r)
          memcpy(qh + es * (size_t)r * Dk, (const char*)q[s] + es * ((size_t)r * Hq + h) * Dk,
                 es * (size_t)Dk);
        if (dv > 0) {
          st = kvc_ref_mla_attention(n_q, 1, Dk, dv, L[s], (const uint16_t*)qh,
                                     (const uint16_t*)k[s], scale, oh);
        } else {
          const size_t kv_off = es * (size_t)g * L[s] * Dk;
          st = kvc_ref_attention(n_q, 1, 1, Dk, L[s], dtype, qh, (const char*)k[s] + kv_off,
                                 (const char*)v[s] + kv_off, scale, oh);
        }
        if (st == REF_OK)
          for (int r = 0; r < n_q; ++r)
            memcpy(out[s] + ((size_t)r * Hq + h) * Dout, oh + (size_t)r * Dout,
                   sizeof(double) * (size_t)Dout);
      }
      if (st != REF_OK) {
#pragma omp critical
        if (status == REF_OK) status = st;
      }
    }
    free(qh);
    free(oh);
  }
  if (threads) *threads = team;
  return status;
}
