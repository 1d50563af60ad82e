/*
 * kvc.h -- C ABI of the MI355X (gfx950) KV-cache decode-attention library.
 *
 * The memory-bound decode step of attention over a KV cache, as described by
 *   [I1] "Inference-1" (brunomaga.github.io): sections "KV cache",
 *        "PagedAttention: memory management for the KV cache",
 *        "FlashAttention", "FlashDecoding", "Smaller KV caches: MQA, GQA and MLA";
 *   [VN] "Inference o quy mo lon: KV cache, prefill va decode"
 *        (blog.truongducdung.dev): section 05 "PagedAttention va prefix
 *        caching" / "Block table", section 07 "FlashAttention" / "Online softmax";
 *   [I2] "Inference-2" (brunomaga.github.io): "Draft-model speculative
 *        decoding", "CUDA graphs";
 *   [EI] "Efficient Inference" (learn.obvix.io): the KV-cache passage and the
 *        paged-attention passage.
 *
 * Conventions shared by every entry point
 *   - Pointers marked (device) are device memory; (host) are host memory.
 *   - Every call only enqueues work on `stream` (a hipStream_t; NULL = the
 *     default stream) and returns without synchronising.  The library never
 *     allocates, frees or copies host<->device, keeps no pointer after it
 *     returns and holds no global state: calls are re-entrant.
 *   - The caller owns every buffer, including the attention workspace.
 *   - Problems visible on the host (null pointers, shapes, unsupported
 *     sizes, a workspace too small) return a negative kvc_status before any
 *     launch and change nothing.
 *   - Problems only visible in device data (a length beyond the capacity, a
 *     block id outside the pool, an exhausted free list) never fault: the
 *     kernels skip the offending work and, when `dev_status` is not NULL,
 *     store a negative kvc_status there with an atomic minimum (the caller
 *     zeroes it beforehand and reads it after synchronising).
 *   - A failed launch returns KVC_ERR_HIP.
 *
 * Layouts (element = 2 bytes for KVC_BF16, 4 for KVC_F32, 1 for FP8; row-major)
 *   contiguous cache (block_size == 0): k_cache, v_cache [batch][num_kv_heads][max_seq_len][head_dim]
 *   paged pool       (block_size  > 0): k_cache, v_cache [num_blocks][num_kv_heads][block_size][head_dim]
 *   FP8 caches: rows are numbered as above (a contiguous cache pads each
 *                (sequence, head) run to a multiple of 16 rows) and stored in
 *                tiles of 16 consecutive rows: tile t is the bytes
 *                [t * (16 * head_dim + 64), (t + 1) * (16 * head_dim + 64)),
 *                the 16 rows' codes (head_dim bytes each) followed by their
 *                16 float32 scales; kvc_cache_bytes() gives the size.  A
 *                row's scale s is its largest |x| over the format's largest
 *                value and each code is the nearest FP8 value to x / s (ties
 *                to even, saturating); the cached value is code * s.
 *   block_table  [batch][max_blocks_per_seq] int32, -1 = unassigned
 *   new rows     k_new, v_new [total_new][num_kv_heads][head_dim], sequence b
 *                owns rows cu_new[b] .. cu_new[b+1]-1 (projection order)
 *   queries      q   [batch][n_q][num_q_heads][head_dim]
 *   outputs      out [batch][n_q][num_q_heads][head_dim]
 */
#ifndef KVC_H
#define KVC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Cache element types.  For the two FP8 types the queries, the new key and
 * value rows and the outputs are bf16, and the cache stores one FP8 code per
 * element plus one float32 scale per row (token, KV head) ([I2] "Quantization"
 * number-format table: E4M3 = 1/4/3 bits, largest 448; E5M2 = 1/5/2 bits,
 * largest 57,344; [VN] 03 "KV cache quantization": FP8 halves the cache and
 * the bytes each decode step reads; [I2] "KV cache quantization": per-token
 * scales).  E4M3 has no infinities (S.1111.111 is NaN); E5M2 is IEEE-like. */
typedef enum { KVC_BF16 = 0, KVC_F32 = 1, KVC_FP8_E4M3 = 2, KVC_FP8_E5M2 = 3 } kvc_dtype;

typedef enum {
  KVC_OK = 0,
  KVC_ERR_ARG = -1,          /* null pointer, aliasing that is not allowed, bad count   */
  KVC_ERR_SHAPE = -2,        /* inconsistent sizes, e.g. num_q_heads % num_kv_heads     */
  KVC_ERR_UNSUPPORTED = -3,  /* head_dim not 64/128, block_size not a multiple of 16... */
  KVC_ERR_WORKSPACE = -4,    /* workspace_bytes < kvc_attn_workspace_bytes()            */
  KVC_ERR_CAPACITY = -5,     /* a sequence would grow past its capacity                 */
  KVC_ERR_NO_BLOCKS = -6,    /* the free list cannot cover the new blocks               */
  KVC_ERR_HIP = -7,          /* a kernel launch failed                                  */
  KVC_ERR_DATA = -8          /* device data out of range (length, slot, block id)      */
} kvc_status;

/* Shape of one layer's cache (host struct, passed by pointer).  `dtype` is
 * the kvc_dtype of the cache (and of q and new rows, which are bf16 for the
 * FP8 types). */
typedef struct {
  int32_t batch;              /* B sequences                                            */
  int32_t num_q_heads;        /* Hq                                                     */
  int32_t num_kv_heads;       /* Hkv; Hq % Hkv == 0, query head h reads KV head h/(Hq/Hkv)
                                 ([I1] "Smaller KV caches": consecutive heads share)    */
  int32_t head_dim;           /* D in {64, 128}; 576 for an MLA latent cache             */
  int32_t dtype;              /* kvc_dtype of q, caches and new rows                    */
  int32_t block_size;         /* 0: contiguous cache; else paged, a multiple of 16 and a
                                 power of two ([VN] 05 "Block table": 16 by default)     */
  int32_t max_seq_len;        /* contiguous: capacity S_max per sequence                */
  int32_t max_blocks_per_seq; /* paged: row stride of block_table; capacity is
                                 max_blocks_per_seq * block_size tokens                 */
  int32_t num_blocks;         /* paged: pool size N                                     */
  int32_t partition_tokens;   /* split-KV partition length in tokens: 0 = library
                                 default (stream-K for grouped rows and large paged
                                 batches), else a multiple of 16                        */
} kvc_cache_desc;

/*
 * kvc_block_table -- give every sequence the blocks its new tokens need and
 * emit the physical slot of every new token (paged caches only).
 *
 * [I1] "PagedAttention" and [EI] paged-attention passage: fixed-size blocks,
 * allocated on demand from a free pool, with a per-sequence table from logical
 * to physical blocks.  [VN] 05 "Block table": a block is taken only when the
 * last one is full.  Order: sequences in batch order, missing logical blocks in
 * increasing order, free_list consumed from index *free_head_in upward.
 *
 *   seq_lens      (device) [B]   tokens already held (ceil(len/bs) blocks)
 *   cu_new        (device) [B+1] offsets of the new tokens
 *   total_new     (host)         cu_new[B]
 *   block_table   (device) [B][max_blocks_per_seq], in/out
 *   free_list     (device) [num_blocks] physical block ids
 *   free_head_in  (device) [1]   first unused free_list index
 *   free_head_out (device) [1]   receives free_head_in + blocks taken; may alias
 *                                free_head_in (a distinct pointer makes the call
 *                                repeatable with identical effect)
 *   slot_mapping  (device) [total_new] out: table[b][pos/bs]*bs + pos%bs for the
 *                                new token at logical position pos
 * All or nothing: when any sequence would exceed max_blocks_per_seq
 * (KVC_ERR_CAPACITY), a length is negative (KVC_ERR_DATA) or the free list runs
 * out (KVC_ERR_NO_BLOCKS), nothing is written except free_head_out =
 * free_head_in and the status.  One workgroup: microseconds.
 */
int kvc_block_table(const kvc_cache_desc* d, const int32_t* seq_lens, const int32_t* cu_new,
                    int32_t total_new, int32_t* block_table, const int32_t* free_list,
                    const int32_t* free_head_in, int32_t* free_head_out, int32_t* slot_mapping,
                    int32_t* dev_status, void* stream);

/*
 * kvc_append -- copy the new tokens' key and value rows into the cache, bit
 * for bit, and advance the lengths.
 *
 * [EI] KV-cache passage: a preallocated cache written in place at the current
 * length, which then grows by the number of new tokens; writing past the
 * capacity is an error.  [I2] "CUDA graphs": in-place writes at the new
 * positions.  [I1] "KV cache": only the new rows are written.
 *
 *   seq_lens      (device) [B] lengths before the append
 *   cu_new        (device) [B+1]
 *   total_new     (host)   cu_new[B]
 *   max_new       (host)   an upper bound of cu_new[b+1]-cu_new[b] (sizes the grid)
 *   slot_mapping  (device) paged: [total_new] from kvc_block_table; contiguous: NULL
 *                 (token t of sequence b goes to position seq_lens[b] + t)
 *   seq_lens_out  (device) [B] = seq_lens + new counts; must not alias seq_lens
 *   v_new, v_cache may both be NULL: a key-only cache (the MLA latent cache,
 *                 whose rows serve as keys and values); not for FP8 caches
 * FP8 caches take bf16 new rows and store codes and per-row scales.
 * Contiguous: a sequence that would pass max_seq_len is not written, keeps its
 * length and reports KVC_ERR_CAPACITY.  Paged: a token whose slot lies outside
 * the pool is not written and reports KVC_ERR_DATA; lengths still advance.
 */
int kvc_append(const kvc_cache_desc* d, const void* k_new, const void* v_new,
               const int32_t* seq_lens, const int32_t* cu_new, int32_t total_new, int32_t max_new,
               const int32_t* slot_mapping, void* k_cache, void* v_cache, int32_t* seq_lens_out,
               int32_t* dev_status, void* stream);

/*
 * kvc_block_table_append -- kvc_block_table followed by kvc_append, in one
 * launch (paged caches only).
 *
 * The same operations as the two calls ([I1] "PagedAttention", [VN] 05
 * "Block table": blocks on demand from the free pool; [EI] KV-cache passage:
 * rows written in place at the current length), with one launch instead of
 * two: a decode step's bookkeeping costs launches, not bytes ([I2] "CUDA
 * graphs": per-kernel launch overhead dominates small steps).  Arguments as the
 * two calls take them (block_table, free_list, free_head_in, free_head_out
 * and slot_mapping of kvc_block_table; k_new, v_new, max_new, k_cache,
 * v_cache and seq_lens_out of kvc_append).  On success the table, the head,
 * the slots, the cache bytes and the lengths are exactly those of the two
 * calls in order.  An allocation error (a negative length or count:
 * KVC_ERR_DATA; a sequence beyond max_blocks_per_seq: KVC_ERR_CAPACITY; too
 * few free blocks: KVC_ERR_NO_BLOCKS) writes nothing but free_head_out =
 * free_head_in, seq_lens_out = seq_lens and the status; a token whose slot
 * lies outside the pool is not written (KVC_ERR_DATA), as in kvc_append.
 * Every workgroup reads the whole batch's lengths, so B is limited to 8192
 * (KVC_ERR_UNSUPPORTED beyond: use the two calls).
 */
int kvc_block_table_append(const kvc_cache_desc* d, const void* k_new, const void* v_new,
                           const int32_t* seq_lens, const int32_t* cu_new, int32_t total_new,
                           int32_t max_new, int32_t* block_table, const int32_t* free_list,
                           const int32_t* free_head_in, int32_t* free_head_out,
                           int32_t* slot_mapping, void* k_cache, void* v_cache,
                           int32_t* seq_lens_out, int32_t* dev_status, void* stream);

/*
 * kvc_append_attn -- kvc_append followed by kvc_verify_attn (n_q = 1:
 * kvc_decode_attn) over the new lengths, for a contiguous cache.
 *
 * [EI] names "KV cache write + attention" among the fused kernels serving
 * systems ship.  With one query row per KV row (MHA, and every fp32 cache)
 * the append happens inside the attention's partition launch: the tiles that
 * reach a sequence's new rows read them from k_new / v_new, and the work item
 * of the last query row of each KV head writes them into the cache (a decode
 * step is then two launches instead of three).  Grouped rows and FP8 caches
 * run the append kernel first.  Arguments as kvc_append (contiguous: no slot
 * mapping) and kvc_verify_attn (its seq_lens are seq_lens_out, the lengths
 * after the append; the workspace is sized by kvc_attn_workspace_bytes).
 * Outputs, cache bytes and seq_lens_out are those of the two calls in order.
 * A sequence the append refuses (it would pass max_seq_len:
 * KVC_ERR_CAPACITY) keeps its length; its attention output is unspecified.
 */
int kvc_append_attn(const kvc_cache_desc* d, const void* k_new, const void* v_new,
                    const int32_t* seq_lens, const int32_t* cu_new, int32_t total_new,
                    int32_t max_new, void* k_cache, void* v_cache, int32_t* seq_lens_out,
                    const void* q, int32_t n_q, float scale, void* out, int32_t out_dtype,
                    void* workspace, size_t workspace_bytes, int32_t* dev_status, void* stream);

/*
 * kvc_block_table_append_attn -- kvc_block_table_append followed by
 * kvc_verify_attn over the lengths after the append, for a paged cache
 * ([I1] PagedAttention: blocks on demand; [EI] lists "KV cache write +
 * attention" among the fused kernels serving systems ship).  With one query
 * row per KV row (MHA, every fp32 cache; not FP8) and a batch whose work
 * items fit one round of resident wavefronts the partition launch does it
 * all: its tiles read the new rows from k_new / v_new (never a table entry
 * this call writes), and one work item per sequence repeats the batch's
 * block count, takes the sequence's blocks from the free list and writes
 * the table entries, slots, new rows and length (sequence 0 the head).
 * Grouped bf16 rows, larger batches (the stream-K split) and FP8 caches run
 * kvc_block_table_append first.
 * Arguments as kvc_block_table_append (B <= 8192) and kvc_verify_attn (its
 * seq_lens are seq_lens_out and its block_table the updated table; the
 * workspace is sized by kvc_attn_workspace_bytes).  On success outputs,
 * table, head, slots, cache bytes and seq_lens_out are those of the two
 * calls in order.  An allocation error (all or nothing, as in
 * kvc_block_table_append) writes nothing but the head, the unchanged lengths
 * and the status; the attention outputs are then unspecified.
 */
int kvc_block_table_append_attn(const kvc_cache_desc* d, const void* k_new, const void* v_new,
                                const int32_t* seq_lens, const int32_t* cu_new, int32_t total_new,
                                int32_t max_new, int32_t* block_table, const int32_t* free_list,
                                const int32_t* free_head_in, int32_t* free_head_out,
                                int32_t* slot_mapping, void* k_cache, void* v_cache,
                                int32_t* seq_lens_out, const void* q, int32_t n_q, float scale,
                                void* out, int32_t out_dtype, void* workspace,
                                size_t workspace_bytes, int32_t* dev_status, void* stream);

/*
 * kvc_decode_attn -- one new query row per sequence attends over all of its
 * seq_lens[b] cached keys (its own key already appended), no mask.
 *
 * [I1] "Why attention matters": softmax(q K^T * scale) V; [I1] "KV cache": a
 * single new row sees every cached key; [I1] "FlashDecoding": split-KV --
 * partitions of the keys processed in parallel, each yielding a partial output
 * with its running maximum and sum ([VN] 07 "Online softmax"), then a
 * reduction combines them.  With one query row per KV row (MHA, fp32
 * caches) and at most one round of resident work items (4096 on MI355X) the
 * combine runs inside the same launch: the work item that finishes a row's
 * last partition merges the row's partials and writes it.  Otherwise a
 * second launch combines.  Equivalent to kvc_verify_attn with n_q = 1.
 *
 *   q            (device) [B][1][Hq][D], dtype d->dtype
 *   seq_lens     (device) [B], 1 <= seq_lens[b] <= capacity
 *   block_table  (device) paged: [B][max_blocks_per_seq]; contiguous: NULL
 *   scale        (host)   score scale, normally 1/sqrt(D)
 *   out          (device) [B][1][Hq][D] of out_dtype (KVC_BF16 rounds to nearest even)
 *   workspace    (device) >= kvc_attn_workspace_bytes(d, 1) bytes, 16-byte aligned,
 *                zero-filled before its first use (see kvc_attn_workspace_bytes)
 * A sequence with invalid data produces zeros and reports KVC_ERR_DATA.
 */
int kvc_decode_attn(const kvc_cache_desc* d, const void* q, const void* k_cache,
                    const void* v_cache, const int32_t* seq_lens, const int32_t* block_table,
                    float scale, void* out, int32_t out_dtype, void* workspace,
                    size_t workspace_bytes, int32_t* dev_status, void* stream);

/*
 * kvc_verify_attn -- n_q query rows per sequence (the last accepted token and
 * n_q - 1 drafts, already appended as the last n_q keys) attend over the cache
 * with a causal mask among themselves: row r sees keys 0 .. seq_lens[b]-n_q+r.
 *
 * [I2] "Draft-model speculative decoding": the target model checks K drafts in
 * one pass over the context plus the drafts; [I1] "KV cache": several new
 * tokens on top of a cache use a shifted causal mask, each new token attending
 * every cached token and the new ones up to itself.
 *
 *   n_q (host) 1..16; q, out [B][n_q][Hq][D]; seq_lens[b] >= n_q; other
 *   arguments as kvc_decode_attn; workspace >= kvc_attn_workspace_bytes(d, n_q).
 */
int kvc_verify_attn(const kvc_cache_desc* d, const void* q, int32_t n_q, const void* k_cache,
                    const void* v_cache, const int32_t* seq_lens, const int32_t* block_table,
                    float scale, void* out, int32_t out_dtype, void* workspace,
                    size_t workspace_bytes, int32_t* dev_status, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * kvc_verify_attn (n_q = 1: kvc_decode_attn) without the workspace
 * arguments.  The split-KV partials go to a static device array of
 * KVC_NOALLOC_SCRATCH_BYTES (64 MiB) inside the library, one copy per
 * device, held until the process ends; nothing is allocated, freed or
 * synchronised.  A call whose kvc_attn_workspace_bytes exceeds that size
 * returns KVC_ERR_WORKSPACE before any launch.  `stream` must belong to the
 * current device (else KVC_ERR_ARG); a failed lookup of the array's
 * address returns KVC_ERR_HIP.  Every call on one device shares its array,
 * which keeps the last call's partials; its counters (see
 * kvc_attn_workspace_bytes) are zero when the library loads and every call
 * leaves them at zero.  Calls that overlap on one device -- on different
 * streams, or from different host threads without ordering -- race and give
 * undefined results.  Other arguments, checks and results as
 * kvc_verify_attn. */
#define KVC_NOALLOC_SCRATCH_BYTES (64u << 20)
int kvc_verify_attn_noalloc(const kvc_cache_desc* d, const void* q, int32_t n_q,
                            const void* k_cache, const void* v_cache, const int32_t* seq_lens,
                            const int32_t* block_table, float scale, void* out,
                            int32_t out_dtype, int32_t* dev_status, void* stream);

/*
 * The two stages kvc_verify_attn runs, exported so that each can be timed on
 * its own: kvc_attn_partition writes every (row, partition) partial -- running
 * maximum (base-2 logarithm domain), sum and unnormalised output -- into the
 * workspace; kvc_attn_reduce combines them into `out` ([I1] "FlashDecoding").
 * Same arguments and rules as kvc_verify_attn; reduce must follow partition
 * on the same workspace with the same desc, n_q and seq_lens.
 */
int kvc_attn_partition(const kvc_cache_desc* d, const void* q, int32_t n_q, const void* k_cache,
                       const void* v_cache, const int32_t* seq_lens, const int32_t* block_table,
                       float scale, void* workspace, size_t workspace_bytes, int32_t* dev_status,
                       void* stream);
int kvc_attn_reduce(const kvc_cache_desc* d, int32_t n_q, const int32_t* seq_lens,
                    const void* workspace, size_t workspace_bytes, void* out, int32_t out_dtype,
                    int32_t* dev_status, void* stream);

/* Workspace bytes the attention calls need for this desc and n_q (0 on a bad
 * desc).  With the stream-K split (below) it depends on the current
 * device's compute-unit count, not on the capacity.  The first 256 KiB of
 * every attention workspace (MLA's too) hold the counters of the combine
 * fused into the partition launch: they must be zero before the
 * workspace's first use (one hipMemset after allocating it) and every call
 * leaves them at zero; no call writes partials there, so calls of any
 * shape may share one workspace (one at a time). */
size_t kvc_attn_workspace_bytes(const kvc_cache_desc* d, int32_t n_q);

/* Partition length in tokens the attention calls use for this desc and n_q
 * (negative kvc_status on a bad desc).  0: the call has no fixed length --
 * with desc.partition_tokens = 0, rows that share a KV head (G * n_q >= 2,
 * bf16 and FP8 caches) use the stream-K split ([I1] "FlashDecoding": any
 * split of the keys combines exactly): the batch's 16-key tiles, taken
 * sequence by sequence and KV head by KV head, are shared out evenly over a
 * fixed set of workers (one per SIMD of the device for bf16 caches, one
 * round of resident wavefronts for FP8), so every worker streams the same
 * number of tiles whatever the lengths.  The vector-ALU rows (one query row
 * per KV row, fp32 caches) of a paged bf16 or fp32 cache use the same split
 * (two workers per SIMD, a segment per query row) when their fixed
 * partitions would take more than one round of resident work items.  An
 * explicit desc.partition_tokens is always used as given (fixed
 * partitions). */
int32_t kvc_attn_partition_tokens(const kvc_cache_desc* d, int32_t n_q);

/* Kernel launches kvc_decode_attn / kvc_verify_attn make for this desc and
 * n_q (negative kvc_status on a bad desc): 1 when the partition launch also
 * combines its partials (one query row per KV row, at most one round of
 * resident work items and 65536 rows), else 2 (a reduce launch follows).
 * kvc_append_attn adds the append launch in front when its append is not
 * fused (grouped rows, FP8 caches). */
int32_t kvc_attn_launches(const kvc_cache_desc* d, int32_t n_q);

/*
 * Block lifecycle (paged caches only): sharing, copy-on-write and rollback.
 *
 * [VN] 05 "Chia se block va copy-on-write": physical blocks carry reference
 * counts; parallel samples share the prompt's blocks and a sample copies a
 * shared block before writing into it.  [I1] "PagedAttention": shared blocks
 * are copied only when written.  [EI] paged-attention passage: a finished
 * request's blocks go back to the free pool.  [I2] "Draft-model speculative
 * decoding": after verification the cache is cut back to the accepted tokens.
 *
 *   ref_counts (device) [num_blocks] owners beyond the first: 0 for a block
 *              held by one sequence or free.  The caller zeroes it once.
 *   free pool  free_list[*free_head .. num_blocks): blocks are taken from the
 *              front (kvc_block_table, kvc_cow) and freed blocks are pushed
 *              back just below the head, in increasing block id, so results do
 *              not depend on thread order.
 * Each call runs one workgroup (microseconds) and is all or nothing on bad
 * device data (dev_status receives KVC_ERR_DATA or KVC_ERR_NO_BLOCKS and only
 * free_head_out = free_head_in is written).  num_blocks <= 262144 for
 * kvc_truncate and kvc_cow (KVC_ERR_UNSUPPORTED otherwise).
 */

/*
 * kvc_fork -- child i starts as a copy of parent i: it takes the parent's
 * length and table row (its first ceil(len/block_size) entries) and every
 * block gained gets one more reference.  No block data moves.
 *
 *   parents, children (device) [n_forks] sequence indices; children distinct,
 *                     empty (seq_lens 0), and no sequence is both a parent and
 *                     a child in one call
 *   seq_lens          (device) [B] in/out: children's entries are set
 *   block_table       (device) in/out: children's rows are set
 *   ref_counts        (device) in/out
 */
int kvc_fork(const kvc_cache_desc* d, const int32_t* parents, const int32_t* children,
             int32_t n_forks, int32_t* seq_lens, int32_t* block_table, int32_t* ref_counts,
             int32_t* dev_status, void* stream);

/*
 * kvc_truncate -- sequence b keeps its first new_lens[b] tokens (0 releases the
 * whole sequence).  Its logical blocks from ceil(new_len/block_size) on become
 * -1; each such block loses one reference, or, having none beyond its owner,
 * is freed.  The kept tokens are not touched.
 *
 *   seq_lens       (device) [B] lengths now; new_lens (device) [B], 0 <= new <= len
 *   block_table    (device) in/out
 *   free_list      (device) in/out; free_head_in / free_head_out as for
 *                  kvc_block_table (free_head_out = free_head_in - blocks freed)
 *   ref_counts     (device) in/out, or NULL when no block is shared (every
 *                  released block is then freed)
 *   seq_lens_out   (device) [B] receives new_lens; may alias seq_lens
 */
int kvc_truncate(const kvc_cache_desc* d, const int32_t* seq_lens, const int32_t* new_lens,
                 int32_t* block_table, int32_t* free_list, const int32_t* free_head_in,
                 int32_t* free_head_out, int32_t* ref_counts, int32_t* seq_lens_out,
                 int32_t* dev_status, void* stream);

/*
 * kvc_cow -- copy-on-write before an append; call it before kvc_block_table
 * with the same seq_lens and cu_new.  Decided on the state at the start of
 * the call: every sequence with new tokens whose last block is partly filled
 * and has extra references takes a fresh block from the free-list front
 * (batch order), gets a copy of the whole block (all KV heads, K and V), points
 * its table entry at it and drops one reference on the original; an original
 * left with no owner is freed.
 *
 *   cow_src, cow_dst (device) [B] out: the copied pair of sequence b, -1 when none
 *   free_head_out    = free_head_in + copies - originals freed
 * The copies run as a second kernel (kvc_copy_blocks) on the same stream.
 */
int kvc_cow(const kvc_cache_desc* d, const int32_t* seq_lens, const int32_t* cu_new,
            int32_t* block_table, int32_t* free_list, const int32_t* free_head_in,
            int32_t* free_head_out, int32_t* ref_counts, void* k_cache, void* v_cache,
            int32_t* cow_src, int32_t* cow_dst, int32_t* dev_status, void* stream);

/*
 * kvc_copy_blocks -- for i < n with src[i] >= 0, copy pool block src[i] onto
 * dst[i] (all KV heads, K and V, bit for bit).  Pairs must not overlap (no
 * block both a source and a destination).  A block id >= num_blocks is
 * KVC_ERR_DATA and that pair is skipped.  FP8 pools copy the blocks' scales
 * too; v_cache may be NULL for a key-only pool (also in kvc_cow).
 */
int kvc_copy_blocks(const kvc_cache_desc* d, const int32_t* src, const int32_t* dst, int32_t n,
                    void* k_cache, void* v_cache, int32_t* dev_status, void* stream);

/*
 * MLA latent decode.
 *
 * [I1] "Smaller KV caches: MQA, GQA and MLA": MLA caches one latent vector per
 * token, and with the key and value up-projections absorbed into the query
 * and output projections attention runs directly over the cached latents,
 * which serve as keys and values: one large KV head shared by every query
 * head.  [VN] 03 "MLA": each token caches d_c + d_h^R = 512 + 64 values, the
 * latent and a decoupled key carrying RoPE.
 *
 * The cache is a key-only cache (kvc_append and kvc_block_table with v_new =
 * v_cache = NULL) described by num_kv_heads = 1, head_dim = 576, dtype bf16;
 * each row is [latent (512) | rope key (64)].
 *   q            (device) [B][n_q][Hq][576] bf16: per head, the absorbed latent
 *                query (W_uk^T q_nope) followed by the rope query
 *   value_dim    (host)   512: the first value_dim dims of a row are the value
 *   out          (device) [B][n_q][Hq][512]: softmax(scale * q.row) weighted
 *                latent rows (apply the absorbed value up-projection after)
 * Verify rows (n_q > 1) see keys 0 .. L - n_q + r.  Other geometries return
 * KVC_ERR_UNSUPPORTED.  The workspace is sized by kvc_mla_workspace_bytes.
 * kvc_mla_partition_tokens returns the planned partition length; when the
 * descriptor's partition_tokens is 0 and a full-capacity batch fits one round
 * of resident workgroups, it is an upper bound: each launch then picks a
 * length between half of it and it from the lengths in device memory, the
 * same in the partition and reduce calls, and the workspace covers the
 * shortest.  With more than 16 rows (Hq * n_q) and partition_tokens 0 it
 * returns 0: the stream-K split, in which one round of workgroups shares the
 * batch's 32-key steps out evenly (every row group of a worker takes the same
 * run), as kvc_attn_partition_tokens describes for grouped rows; it falls back
 * to partitions when a worker's run could exceed 16384 keys of one sequence.
 * An explicit partition_tokens is used as given.
 */
size_t kvc_mla_workspace_bytes(const kvc_cache_desc* d, int32_t n_q, int32_t value_dim);
int32_t kvc_mla_partition_tokens(const kvc_cache_desc* d, int32_t n_q, int32_t value_dim);
int kvc_mla_attn_partition(const kvc_cache_desc* d, const void* q, int32_t n_q,
                           const void* latent_cache, const int32_t* seq_lens,
                           const int32_t* block_table, int32_t value_dim, float scale,
                           void* workspace, size_t workspace_bytes, int32_t* dev_status,
                           void* stream);
int kvc_mla_attn_reduce(const kvc_cache_desc* d, int32_t n_q, int32_t value_dim,
                        const int32_t* seq_lens, const void* workspace, size_t workspace_bytes,
                        void* out, int32_t out_dtype, int32_t* dev_status, void* stream);
int kvc_mla_attn(const kvc_cache_desc* d, const void* q, int32_t n_q, const void* latent_cache,
                 const int32_t* seq_lens, const int32_t* block_table, int32_t value_dim,
                 float scale, void* out, int32_t out_dtype, void* workspace,
                 size_t workspace_bytes, int32_t* dev_status, void* stream);

/*
 * kvc_prefill_attn -- causal attention of a chunk of new rows per sequence
 * over everything cached (prefill, or one chunk of a chunked prefill).
 *
 * [I1] "FlashAttention": a block of queries loops over tiles of keys and
 * values with the online softmax, never writing the score matrix, and skips
 * the tiles above the causal diagonal.  [I1] "Chunked prefill" and [VN] 05
 * "Chunked prefill": long prompts are processed in chunks, each over the
 * whole cache.  Append the chunk first (kvc_block_table, kvc_append); then
 * sequence b holds seq_lens[b] keys and its n_b = cu_q[b+1] - cu_q[b] query
 * rows sit at positions seq_lens[b] - n_b + r: row r sees keys
 * 0 .. seq_lens[b] - n_b + r ([I1] "KV cache": the shifted causal mask).
 *
 *   q        (device) [total_q][Hq][D] bf16, sequence b's rows at cu_q[b] ..
 *   cu_q     (device) [B+1] offsets; max_q (host) >= every n_b (sizes the grid)
 *   seq_lens (device) [B] lengths after the append, n_b <= seq_lens[b]
 *   out      (device) [total_q][Hq][D], out_dtype bf16 or f32
 * bf16 caches with head_dim 64 or 128 (others KVC_ERR_UNSUPPORTED); paged
 * caches with max_blocks_per_seq <= 4096.  No workspace: each query block
 * covers all its keys.  Bad lengths or offsets: KVC_ERR_DATA, rows skipped.
 * Precision: scores in fp32 from bf16 products; the value products take the
 * value entries as fp16 (exact for magnitudes up to 65504; larger value
 * entries are outside the supported range and are not reported) and the
 * softmax weights as fp16, with fp32 accumulation.
 */
int kvc_prefill_attn(const kvc_cache_desc* d, const void* q, const int32_t* cu_q, int32_t total_q,
                     int32_t max_q, const void* k_cache, const void* v_cache,
                     const int32_t* seq_lens, const int32_t* block_table, float scale, void* out,
                     int32_t out_dtype, int32_t* dev_status, void* stream);

/* Bytes of one cache buffer (k_cache or v_cache) for this description: FP8
 * codes and scales, or the plain elements.  0 on an invalid description. */
size_t kvc_cache_bytes(const kvc_cache_desc* d);

/* Static text for a kvc_status value (never NULL; "unknown status" for any
 * other integer).  The string is owned by the library. */
const char* kvc_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H */
