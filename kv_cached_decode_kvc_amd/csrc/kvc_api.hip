// kvc_api.hip -- the C ABI of libkvc.so: argument checks, work planning and
// kernel launches on the caller's stream.  Host code; no allocation, no
// synchronisation.  The only global state is the static scratch array of
// kvc_verify_attn_noalloc (one copy per device) and its per-device address.
#include <math.h>

#include <algorithm>
#include <mutex>

#include "launch.hpp"

namespace {

using namespace kvc;

int check_desc(const kvc_cache_desc* d) {
  if (!d) return KVC_ERR_ARG;
  if (d->batch < 0 || d->num_q_heads <= 0 || d->num_kv_heads <= 0) return KVC_ERR_SHAPE;
  if (d->batch >= kMaxBatch) return KVC_ERR_UNSUPPORTED;  // one grid row per sequence
  if (d->num_q_heads % d->num_kv_heads != 0) return KVC_ERR_SHAPE;
  if (d->head_dim != 64 && d->head_dim != 128 && d->head_dim != kMlaKeyDim)
    return KVC_ERR_UNSUPPORTED;
  if (d->head_dim == kMlaKeyDim && (d->dtype != KVC_BF16 || d->num_kv_heads != 1))
    return KVC_ERR_UNSUPPORTED;  // MLA latent caches: one bf16 head of 576
  if (d->dtype < KVC_BF16 || d->dtype > KVC_FP8_E5M2) return KVC_ERR_UNSUPPORTED;
  if (d->block_size < 0) return KVC_ERR_SHAPE;
  if (d->block_size == 0) {
    if (d->max_seq_len <= 0) return KVC_ERR_SHAPE;
  } else {
    const int bs = d->block_size;
    if (bs % kTile != 0 || (bs & (bs - 1)) != 0) return KVC_ERR_UNSUPPORTED;
    if (d->max_blocks_per_seq <= 0 || d->num_blocks <= 0) return KVC_ERR_SHAPE;
    if ((long)d->max_blocks_per_seq * bs > 0x7fffffffL) return KVC_ERR_SHAPE;
  }
  if (d->partition_tokens < 0 || d->partition_tokens % kTile != 0) return KVC_ERR_UNSUPPORTED;
  return KVC_OK;
}

int capacity(const kvc_cache_desc* d) {
  return d->block_size ? d->max_blocks_per_seq * d->block_size : d->max_seq_len;
}

int fp8_format(const kvc_cache_desc* d) {
  return d->dtype == KVC_FP8_E4M3 ? kFp8E4M3 : d->dtype == KVC_FP8_E5M2 ? kFp8E5M2 : 0;
}

// bytes of one cache element, and of one element of q / new rows / outputs
size_t elem_bytes(const kvc_cache_desc* d) {
  return fp8_format(d) ? 1 : d->dtype == KVC_BF16 ? 2 : 4;
}
size_t input_bytes(const kvc_cache_desc* d) { return d->dtype == KVC_F32 ? 4 : 2; }

// rows of one cache buffer; an FP8 contiguous cache pads each (sequence, head)
// run to whole 16-row tiles
size_t cache_rows(const kvc_cache_desc* d) {
  if (d->block_size) return (size_t)d->num_blocks * d->num_kv_heads * d->block_size;
  const long s = fp8_format(d) ? fp8_padded_rows(d->max_seq_len) : d->max_seq_len;
  return (size_t)d->batch * d->num_kv_heads * s;
}

struct Plan {
  bool mfma;          // grouped rows on the matrix cores
  bool sk;            // mfma: the stream-K split (no fixed partition length)
  int rows_per_item;  // mfma: 16 or 32 rows per wavefront
  int P;              // partition length in tokens (an upper bound when slots_u > 0; 0: stream-K)
  int P_lo;           // slots_u > 0: the shortest partition a launch may choose
  int slots_u;        // > 0: resident wavefront slots per unit of a sequence
  int max_parts;      // partitions of a full-capacity sequence
  int units;          // work units of a sequence per partition (rows, or row blocks per KV head)
  int sk_workers;     // stream-K: workers launched (one round of resident wavefronts)
  int sk_rows;        // stream-K: rows one piece holds
  long grid;          // workgroups of the partition launch
  size_t o_offset;    // byte offset of the partial outputs inside the workspace
  size_t ml_offset;   // byte offset of the (m, l) array inside the workspace
  size_t meta_offset; // stream-K: byte offset of the per-segment worker records
  bool fused;         // the one-call entry points combine inside the partition launch (vector ALU)
  size_t bytes;       // workspace size
};

constexpr int kSkMinTiles = 8;     // stream-K: fewest 16-key tiles a worker streams
constexpr int kValuSkPerSimd = 2;  // stream-K workers per SIMD of the vector-ALU kernel

// Every attention workspace starts with kCntBytes of piece counters for the
// combine fused into the partition launch (one per output row); the partials
// of every plan, MLA included, come after them.  The counters must be zero before a workspace's first use and every
// call leaves them at zero, so calls of any shape may share a workspace.  A
// call with more units than counters runs the separate reduce kernel.
constexpr size_t kCntBytes = 256u << 10;
constexpr long kMaxCounters = (long)(kCntBytes / sizeof(uint32_t));

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Work is one wavefront per (rows, partition).  A wavefront pays a few
// dependent memory latencies (length, block ids, first tile) before it
// streams, and a loaded memory system answers in microseconds, so partitions
// are long; a full MI355X needs only about 1,300 wavefronts with one 8 KiB
// tile in flight each to keep HBM busy.  Default partition length: 1024 keys
// for a contiguous cache (each wavefront streams one long run); for a paged
// cache the power of two nearest an eighth of the capacity, within [256,
// 2048], so that sequences of
// any length still split into a few partitions and the last of them finish
// together; at most 512 for FP8 caches, whose wavefronts move half the bytes
// per key.  It is halved (down to 64) while a full-capacity batch would give
// fewer than 1024 wavefronts, and doubled (up to 8192) while it would give
// more than 65536.
//
// The matrix-core path (grouped rows), and the vector-ALU path on paged
// bf16 / fp32 caches too large for one round of work items, use no partition
// length by default: the stream-K split shares the batch's tiles out evenly
// over a fixed number of workers (matrix cores: one per SIMD for bf16
// caches, for FP8 caches one round of resident wavefronts, 2 per SIMD with
// 32-row blocks, 3 with 16-row blocks; vector ALUs: 2 per SIMD), each taking
// at least kSkMinTiles tiles.  Its workspace holds one partial
// per row of every piece: at most segments + workers pieces (a piece starts
// at a segment start or a worker start), sk_rows rows each.
// SIMDs of the current device (4 per compute unit); 1024 on MI355X.
int resident_simds() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  return 4 * cus;
}

Plan make_plan(const kvc_cache_desc* d, int n_q) {
  Plan pl{};
  const int G = d->num_q_heads / d->num_kv_heads;
  const int R = G * n_q;
  pl.mfma = d->dtype != KVC_F32 && R >= 2;
  pl.rows_per_item = R > 16 ? 32 : 16;
  pl.units = pl.mfma ? d->num_kv_heads * ((R + pl.rows_per_item - 1) / pl.rows_per_item)
                     : d->num_q_heads * n_q;
  const long units = (long)d->batch * pl.units;
  const int cap = capacity(d);
  const size_t rows = (size_t)d->batch * d->num_q_heads * n_q;
  if (pl.mfma && d->partition_tokens == 0) {
    pl.sk = true;
    // bf16 tiles: one worker per SIMD; FP8 tiles carry half the bytes, so a
    // full round of resident wavefronts keeps enough of them in flight
    // (measured on the full-size GQA and verify workloads: bf16 GQA 372 us
    // at 1024 workers against 380 at 3072, and 369 against 371 at 2048 in a
    // later pair of runs; FP8 GQA 208 us at 3072 against 345 at 1024)
    pl.sk_workers = resident_simds() * (!fp8_format(d) ? 1 : pl.rows_per_item == 32 ? 2 : 3);
    pl.sk_rows = std::min(pl.rows_per_item, R);
    pl.grid = pl.sk_workers;
    const size_t pieces = (size_t)units + pl.sk_workers;
    pl.o_offset = kCntBytes;
    pl.ml_offset = align256(pl.o_offset + pieces * pl.sk_rows * d->head_dim * sizeof(float));
    pl.meta_offset = align256(pl.ml_offset + pieces * pl.sk_rows * 2 * sizeof(float));
    pl.bytes = pl.meta_offset + (size_t)units * 2 * sizeof(int32_t);
    return pl;
  }
  if (d->partition_tokens > 0) {
    pl.P = d->partition_tokens;
  } else {
    if (d->block_size == 0) {
      pl.P = 1024;
    } else {
      pl.P = 256;
      while (pl.P < 2048 && pl.P * 2.0 <= cap / 8.0 * 1.4142135623730951) pl.P <<= 1;
    }
    if (fp8_format(d) && pl.P > 512) pl.P = 512;  // half the bytes per key: more wavefronts
    while (pl.P > 64 && units * ((cap + pl.P - 1) / pl.P) < 1024) pl.P >>= 1;
    while (pl.P < 8192 && units * ((cap + pl.P - 1) / pl.P) > 65536) pl.P <<= 1;
  }
  pl.P_lo = pl.P;
  pl.max_parts = (cap + pl.P_lo - 1) / pl.P_lo;
  pl.grid = xcd_grid(d->batch, pl.units, pl.max_parts);
  const size_t o_bytes = rows * pl.max_parts * d->head_dim * sizeof(float);
  pl.o_offset = kCntBytes;
  pl.ml_offset = align256(pl.o_offset + o_bytes);
  pl.bytes = pl.ml_offset + rows * pl.max_parts * 2 * sizeof(float);
  // The vector-ALU kernel combines in its own launch (one counter per output
  // row) when its work items fit one round of resident wavefronts: each item
  // then waits once for its partial to reach the coherent level and for its
  // count (a few microseconds, all items at the same time), which is less
  // than a second launch.  A larger grid pays that wait round after round,
  // and the separate reduce kernel is cheaper (measured on MI355X: the
  // 16 x 40-head layer, 1280 items, step 105.9 -> 100.8 us fused; the
  // 64-sequence paged MHA batch, 20480 items, 425 -> 432 us).  The
  // matrix-core kernel's stream-K workers would pay the wait on every piece
  // and keep the separate reduce.
  pl.fused = !pl.mfma && (long)rows <= kMaxCounters && pl.grid <= 4L * resident_simds();
  // A paged bf16 or fp32 cache whose work items would take more than that one
  // round uses the vector-ALU kernel's stream-K form instead: the items of
  // unequal lengths (short sequences, short last partitions) otherwise end
  // the launch with a ragged last round.  Two workers per SIMD, one partial
  // per piece, the records as in the matrix-core split (measured on the
  // 64-sequence paged MHA batch: 412 us with fixed 512-key partitions,
  // 395 us stream-K with two or three workers per SIMD, 400 with four, 425
  // with five; more loads in flight per worker measured slower).
  if (!pl.mfma && !pl.fused && d->block_size > 0 && !fp8_format(d) &&
      d->partition_tokens == 0) {
    pl.sk = true;
    pl.P = pl.P_lo = pl.max_parts = 0;
    pl.rows_per_item = 1;  // a segment is one query row
    pl.sk_workers = resident_simds() * kValuSkPerSimd;
    pl.sk_rows = 1;
    pl.grid = pl.sk_workers;
    const size_t pieces = (size_t)units + pl.sk_workers;
    pl.o_offset = kCntBytes;
    pl.ml_offset = align256(pl.o_offset + pieces * d->head_dim * sizeof(float));
    pl.meta_offset = align256(pl.ml_offset + pieces * 2 * sizeof(float));
    pl.bytes = pl.meta_offset + (size_t)units * 2 * sizeof(int32_t);
  }
  return pl;
}

int hip_status(hipError_t e) { return e == hipSuccess ? KVC_OK : KVC_ERR_HIP; }

// MLA latent decode: one bf16 latent head of 576 (512 latent + 64 RoPE key),
// values = the 512-wide latent.  Up to 16 rows, a workgroup of four
// wavefronts covers the 16 rows and several workgroups fit per CU; more
// rows, a workgroup of eight wavefronts covers 64 rows and fills a CU; a
// round of resident work is 256 CUs times the workgroups per CU
// (mla_wgs_per_cu).  The partition length grows in steps of 256
// keys until a full-capacity batch fits in one round (a workgroup then
// streams its partition without a second round behind it; two rounds
// measured 10-12% slower), and halves (down to 64) while it would not fill
// one.
int check_mla(const kvc_cache_desc* d, int n_q, int value_dim) {
  const int st = check_desc(d);
  if (st != KVC_OK) return st;
  if (d->head_dim != kMlaKeyDim || value_dim != kMlaValueDim) return KVC_ERR_UNSUPPORTED;
  if (n_q < 1 || n_q > 16) return KVC_ERR_UNSUPPORTED;
  if (d->partition_tokens > 16384) return KVC_ERR_UNSUPPORTED;  // the kernel stages <= 1024 tiles
  return KVC_OK;
}

Plan make_mla_plan(const kvc_cache_desc* d, int n_q) {
  Plan pl{};
  const int R = d->num_q_heads * n_q;
  const long rows_wg = mla_rows_per_wg(R);
  const long n_rg = (R + rows_wg - 1) / rows_wg;
  const long units = (long)d->batch * n_rg;
  const int cap = capacity(d);
  const long one_round = 256L * mla_wgs_per_cu(R);  // workgroups resident at once
  if (d->partition_tokens > 0) {
    pl.P = d->partition_tokens;
  } else {
    pl.P = 256;
    while (pl.P < 8192 && units * ((cap + pl.P - 1) / pl.P) > one_round) pl.P += 256;
    while (pl.P > 64 && units * ((cap + pl.P - 1) / pl.P) < one_round) pl.P >>= 1;
  }
  pl.P_lo = pl.P;
  if (d->partition_tokens == 0 && pl.P >= 2 * kTile &&
      units * ((cap + pl.P - 1) / pl.P) <= one_round) {
    // The planned length fits a full-capacity batch in one round; with the
    // actual lengths the kernel shortens it (down to half) so that the live
    // (sequence, partition) pairs fill the round, and packs them at the
    // front of the grid (nth_pair in the kernel).
    pl.P_lo = pl.P / 2;
    pl.slots_u = (int)(one_round / n_rg);
  }
  pl.max_parts = (cap + pl.P_lo - 1) / pl.P_lo;
  const size_t rows = (size_t)d->batch * d->num_q_heads * n_q;
  const size_t o_bytes = rows * pl.max_parts * kMlaValueDim * sizeof(float);
  pl.o_offset = kCntBytes;  // the counters of other calls sharing the workspace stay untouched
  pl.ml_offset = align256(pl.o_offset + o_bytes);
  pl.bytes = pl.ml_offset + rows * pl.max_parts * 2 * sizeof(float);
  // More than 16 rows: by default the stream-K split, one round of
  // workgroups, the same run of steps for every row group of a worker (so
  // the row groups still share each tile through one L2), every worker the
  // same number of steps.  With the partitions above the live (sequence,
  // partition) pairs carry unequal numbers of steps (a sequence's last
  // partition is short) and leave part of the round idle (128 heads, 32
  // sequences of 1024-4096 keys: 226 of 256 workgroups, the longest 896
  // keys against 759 on average; 87.5 -> 81.2 us stream-K).  The 16-row form
  // measured slower stream-K (16 heads: 121.4 -> 125.5 us) and keeps the
  // partitions.  A worker's run must fit the kernel's LDS staging of block
  // ids: otherwise, and with an explicit length, fixed partitions.
  const int tk = 2 * kTile;                // keys per step of the eight-wavefront kernel
  const long w_round = one_round / n_rg;   // workers of one row group
  const long max_steps = std::max((d->batch * ((cap + tk - 1) / tk) + w_round - 1) / w_round,
                                  2L * kSkMinTiles);
  if (R > 16 && d->partition_tokens == 0 && w_round >= 1 &&
      max_steps * (tk / kTile) <= kMlaMaxTiles) {
    pl.sk = true;
    pl.P = pl.P_lo = pl.max_parts = pl.slots_u = 0;
    pl.sk_workers = (int)w_round;
    pl.rows_per_item = R;  // a segment is a whole sequence's rows
    pl.sk_rows = R;
    const size_t pieces = (size_t)d->batch + pl.sk_workers;
    pl.o_offset = kCntBytes;
    pl.ml_offset = align256(pl.o_offset + pieces * R * kMlaValueDim * sizeof(float));
    pl.meta_offset = align256(pl.ml_offset + pieces * R * 2 * sizeof(float));
    pl.bytes = pl.meta_offset + (size_t)d->batch * 2 * sizeof(int32_t);
  }
  return pl;
}

// Host checks of an attention call's arguments, workspace aside.
int check_attn_args(const kvc_cache_desc* d, int n_q, const void* q, const void* k,
                    const void* v, const int32_t* seq_lens, const int32_t* table, float scale) {
  int st = check_desc(d);
  if (st != KVC_OK) return st;
  if (n_q < 1 || n_q > 16) return KVC_ERR_UNSUPPORTED;
  if (d->head_dim == kMlaKeyDim) return KVC_ERR_UNSUPPORTED;  // the kvc_mla_* calls
  if (d->batch == 0) return KVC_OK;
  if (!q || !k || !v || !seq_lens) return KVC_ERR_ARG;
  if ((d->block_size > 0) != (table != nullptr)) return KVC_ERR_ARG;
  if (!isfinite(scale)) return KVC_ERR_ARG;
  return KVC_OK;
}

// Host checks of an attention call; on success *pl holds the call's plan
// (computed once per entry-point call and handed to both stages).
int check_attn(const kvc_cache_desc* d, int n_q, const void* q, const void* k, const void* v,
               const int32_t* seq_lens, const int32_t* table, float scale, const void* ws,
               size_t ws_bytes, Plan* pl) {
  int st = check_attn_args(d, n_q, q, k, v, seq_lens, table, scale);
  if (st != KVC_OK || d->batch == 0) return st;
  if (!ws) return KVC_ERR_ARG;
  if (((uintptr_t)ws & 15) != 0) return KVC_ERR_ARG;
  *pl = make_plan(d, n_q);
  if (pl->grid > 0x7fffffffL) return KVC_ERR_UNSUPPORTED;  // one workgroup per work item
  if (ws_bytes < pl->bytes) return KVC_ERR_WORKSPACE;
  return KVC_OK;
}

// Host checks of a reduce call that are not covered by check_attn.
int check_reduce(const kvc_cache_desc* d, int n_q, const int32_t* seq_lens, const void* ws,
                 const void* out, int32_t out_dtype) {
  int st = check_desc(d);
  if (st != KVC_OK) return st;
  if (n_q < 1 || n_q > 16) return KVC_ERR_UNSUPPORTED;
  if (d->head_dim == kMlaKeyDim) return KVC_ERR_UNSUPPORTED;  // kvc_mla_attn_reduce
  if (out_dtype != KVC_BF16 && out_dtype != KVC_F32) return KVC_ERR_UNSUPPORTED;
  if (d->batch == 0) return KVC_OK;
  if (!seq_lens || !ws || !out) return KVC_ERR_ARG;
  if (((uintptr_t)ws & 15) != 0) return KVC_ERR_ARG;
  return KVC_OK;
}

// out != NULL (and a fused plan): the partition launch also combines and
// writes `out`.
AttnParams attn_params(const kvc_cache_desc* d, const Plan& pl, int n_q, const void* q,
                       const void* k, const void* v, const int32_t* seq_lens,
                       const int32_t* table, float scale, void* ws, int32_t* status,
                       void* out = nullptr, int32_t out_dtype = KVC_F32) {
  AttnParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.seq_lens = seq_lens;
  p.table = table;
  p.ws_o = (float*)((char*)ws + pl.o_offset);
  p.ws_ml = (float*)((char*)ws + pl.ml_offset);
  p.status = status;
  p.B = d->batch;
  p.n_q = n_q;
  p.Hq = d->num_q_heads;
  p.Hkv = d->num_kv_heads;
  p.G = d->num_q_heads / d->num_kv_heads;
  p.D = d->head_dim;
  p.bs = d->block_size;
  p.S_max = d->max_seq_len;
  p.max_blocks = d->max_blocks_per_seq;
  p.N = d->num_blocks;
  p.P = pl.P;
  p.P_lo = pl.P_lo;
  p.slots_u = pl.slots_u;
  p.max_parts = pl.max_parts;
  p.cap = capacity(d);
  p.scale_log2 = (float)((double)scale * 1.4426950408889634);  // log2(e)
  if (fp8_format(d) && d->block_size == 0) p.S_max = (int)fp8_padded_rows(d->max_seq_len);
  if (pl.sk) {
    p.sk_meta = (int2*)((char*)ws + pl.meta_offset);
    p.sk_workers = pl.sk_workers;
    p.sk_rows = pl.sk_rows;
    p.sk_min_tiles = kSkMinTiles;
  }
  if (out && pl.fused) {
    p.cnt = (uint32_t*)ws;  // the counter region at the workspace's start
    p.out = out;
    p.out_bf16 = out_dtype == KVC_BF16;
  }
  return p;
}

ReduceParams reduce_params(const kvc_cache_desc* d, const Plan& pl, int n_q, int D,
                           const int32_t* seq_lens, const void* ws, void* out,
                           int32_t* status) {
  ReduceParams p{};
  p.ws_o = (const float*)((const char*)ws + pl.o_offset);
  p.ws_ml = (const float*)((const char*)ws + pl.ml_offset);
  p.seq_lens = seq_lens;
  p.out = out;
  p.status = status;
  p.B = d->batch;
  p.n_q = n_q;
  p.Hq = d->num_q_heads;
  p.D = D;
  p.P = pl.P;
  p.P_lo = pl.P_lo;
  p.slots_u = pl.slots_u;
  p.max_parts = pl.max_parts;
  p.cap = capacity(d);
  if (pl.sk) {
    p.sk_meta = (const int2*)((const char*)ws + pl.meta_offset);
    p.sk_rows = pl.sk_rows;
    p.sk_workers = pl.sk_workers;
    p.G = d->num_q_heads / d->num_kv_heads;
    p.Hkv = d->num_kv_heads;
    p.rows_item = pl.rows_per_item;
  }
  return p;
}

// The two stages of decode / verify attention with a plan already checked.
// With out != NULL and a fused plan the partition launch is the whole call.
int run_partition(const kvc_cache_desc* d, const Plan& pl, const void* q, int n_q,
                  const void* k_cache, const void* v_cache, const int32_t* seq_lens,
                  const int32_t* block_table, float scale, void* ws, int32_t* status,
                  void* stream, void* out = nullptr, int32_t out_dtype = KVC_F32) {
  const AttnParams p = attn_params(d, pl, n_q, q, k_cache, v_cache, seq_lens, block_table, scale,
                                   ws, status, out, out_dtype);
  hipError_t e = pl.mfma ? launch_partition_mfma(p, pl.rows_per_item, fp8_format(d),
                                                 (hipStream_t)stream)
                         : launch_partition_valu(p, d->dtype, (hipStream_t)stream);
  return hip_status(e);
}

int run_reduce(const kvc_cache_desc* d, const Plan& pl, int n_q, int D, const int32_t* seq_lens,
               const void* ws, void* out, int32_t out_dtype, int32_t* status, void* stream) {
  const ReduceParams p = reduce_params(d, pl, n_q, D, seq_lens, ws, out, status);
  return hip_status(launch_reduce(p, out_dtype, (hipStream_t)stream));
}

// Scratch of kvc_verify_attn_noalloc: the split-KV partials (partial outputs
// and their (m, l) statistics) live in this file-scope device array instead
// of a caller-provided workspace.  Every device the library runs on holds
// its own copy until the process ends.  In host code `scratch` names a host
// stand-in, never the device memory: kernels get the address that
// hipGetSymbolAddress returns for the current device, looked up once per
// device and kept in `g_scratch_dev`.
static __device__ __align__(256) uint8_t scratch[KVC_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];  // device address of `scratch` on each device (null: not yet)

// Device address of `scratch` on the current device, or null on a HIP error.
void* scratch_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_dev[dev] = ptr;
  }
  return g_scratch_dev[dev];
}

}  // namespace

extern "C" {

int kvc_block_table(const kvc_cache_desc* d, const int32_t* seq_lens, const int32_t* cu_new,
                    int32_t total_new, int32_t* block_table, const int32_t* free_list,
                    const int32_t* free_head_in, int32_t* free_head_out, int32_t* slot_mapping,
                    int32_t* dev_status, void* stream) {
  int st = check_desc(d);
  if (st != KVC_OK) return st;
  if (d->block_size == 0) return KVC_ERR_ARG;  // contiguous caches have no table
  if (total_new < 0) return KVC_ERR_ARG;
  if (d->batch == 0) return total_new == 0 ? KVC_OK : KVC_ERR_ARG;
  if (!seq_lens || !cu_new || !block_table || !free_list || !free_head_in || !free_head_out)
    return KVC_ERR_ARG;
  if (total_new > 0 && !slot_mapping) return KVC_ERR_ARG;
  BlockTableArgs a{};
  a.seq_lens = seq_lens;
  a.cu_new = cu_new;
  a.table = block_table;
  a.free_list = free_list;
  a.head_in = free_head_in;
  a.head_out = free_head_out;
  a.slots = slot_mapping;
  a.status = dev_status;
  a.B = d->batch;
  a.bs = d->block_size;
  a.max_blocks = d->max_blocks_per_seq;
  a.N = d->num_blocks;
  a.total_new = total_new;
  return hip_status(launch_block_table(a, (hipStream_t)stream));
}

int kvc_append(const kvc_cache_desc* d, const void* k_new, const void* v_new,
               const int32_t* seq_lens, const int32_t* cu_new, int32_t total_new, int32_t max_new,
               const int32_t* slot_mapping, void* k_cache, void* v_cache, int32_t* seq_lens_out,
               int32_t* dev_status, void* stream) {
  int st = check_desc(d);
  if (st != KVC_OK) return st;
  if (total_new < 0 || max_new < 0) return KVC_ERR_ARG;
  if (d->batch == 0) return total_new == 0 ? KVC_OK : KVC_ERR_ARG;
  if (!seq_lens || !cu_new || !k_cache || !seq_lens_out) return KVC_ERR_ARG;
  if (!v_cache && v_new) return KVC_ERR_ARG;  // v_cache NULL: a key-only cache
  if (!v_cache && fp8_format(d)) return KVC_ERR_UNSUPPORTED;
  if (seq_lens_out == seq_lens) return KVC_ERR_ARG;
  if (total_new > 0 && (!k_new || (v_cache && !v_new))) return KVC_ERR_ARG;
  if (d->block_size > 0 && total_new > 0 && !slot_mapping) return KVC_ERR_ARG;
  if (d->block_size == 0 && slot_mapping) return KVC_ERR_ARG;
  AppendArgs a{};
  a.k_new = (const uint8_t*)k_new;
  a.v_new = (const uint8_t*)v_new;
  a.seq_lens = seq_lens;
  a.cu_new = cu_new;
  a.slots = d->block_size > 0 ? slot_mapping : nullptr;
  a.k_cache = (uint8_t*)k_cache;
  a.v_cache = (uint8_t*)v_cache;
  a.seq_lens_out = seq_lens_out;
  a.status = dev_status;
  a.B = d->batch;
  a.Hkv = d->num_kv_heads;
  a.head_bytes = (int)(d->head_dim * input_bytes(d));  // bytes of one new row of one head
  a.fp8 = fp8_format(d);
  a.D = d->head_dim;
  a.bs = d->block_size;
  a.S_max = d->max_seq_len;
  a.N = d->num_blocks;
  a.max_new = max_new;
  a.total_new = total_new;
  if (d->block_size > 0 && total_new == 0) a.slots = nullptr, a.S_max = 0x7fffffff;
  return hip_status(launch_append(a, (hipStream_t)stream));
}

int kvc_block_table_append(const kvc_cache_desc* d, const void* k_new, const void* v_new,
                           const int32_t* seq_lens, const int32_t* cu_new, int32_t total_new,
                           int32_t max_new, int32_t* block_table, const int32_t* free_list,
                           const int32_t* free_head_in, int32_t* free_head_out,
                           int32_t* slot_mapping, void* k_cache, void* v_cache,
                           int32_t* seq_lens_out, int32_t* dev_status, void* stream) {
  int st = check_desc(d);
  if (st != KVC_OK) return st;
  if (d->block_size == 0) return KVC_ERR_ARG;  // contiguous caches: kvc_append
  if (total_new < 0 || max_new < 0) return KVC_ERR_ARG;
  if (d->batch > kMaxFusedBatch) return KVC_ERR_UNSUPPORTED;
  if (d->batch == 0) return total_new == 0 ? KVC_OK : KVC_ERR_ARG;
  if (!seq_lens || !cu_new || !block_table || !free_list || !free_head_in || !free_head_out ||
      !k_cache || !seq_lens_out)
    return KVC_ERR_ARG;
  if (!v_cache && v_new) return KVC_ERR_ARG;
  if (!v_cache && fp8_format(d)) return KVC_ERR_UNSUPPORTED;
  if (seq_lens_out == seq_lens) return KVC_ERR_ARG;
  if (total_new > 0 && (!k_new || (v_cache && !v_new) || !slot_mapping)) return KVC_ERR_ARG;
  BlockTableArgs bt{};
  bt.seq_lens = seq_lens;
  bt.cu_new = cu_new;
  bt.table = block_table;
  bt.free_list = free_list;
  bt.head_in = free_head_in;
  bt.head_out = free_head_out;
  bt.slots = slot_mapping;
  bt.status = dev_status;
  bt.B = d->batch;
  bt.bs = d->block_size;
  bt.max_blocks = d->max_blocks_per_seq;
  bt.N = d->num_blocks;
  bt.total_new = total_new;
  AppendArgs a{};
  a.k_new = (const uint8_t*)k_new;
  a.v_new = (const uint8_t*)v_new;
  a.seq_lens = seq_lens;
  a.cu_new = cu_new;
  a.slots = slot_mapping;
  a.k_cache = (uint8_t*)k_cache;
  a.v_cache = (uint8_t*)v_cache;
  a.seq_lens_out = seq_lens_out;
  a.status = dev_status;
  a.B = d->batch;
  a.Hkv = d->num_kv_heads;
  a.head_bytes = (int)(d->head_dim * input_bytes(d));
  a.fp8 = fp8_format(d);
  a.D = d->head_dim;
  a.bs = d->block_size;
  a.N = d->num_blocks;
  a.max_new = max_new;
  a.total_new = total_new;
  return hip_status(launch_block_table_append(bt, a, (hipStream_t)stream));
}

int kvc_append_attn(const kvc_cache_desc* d, const void* k_new, const void* v_new,
                    const int32_t* seq_lens, const int32_t* cu_new, int32_t total_new,
                    int32_t max_new, void* k_cache, void* v_cache, int32_t* seq_lens_out,
                    const void* q, int32_t n_q, float scale, void* out, int32_t out_dtype,
                    void* workspace, size_t workspace_bytes, int32_t* dev_status, void* stream) {
  int st = check_desc(d);
  if (st != KVC_OK) return st;
  if (d->block_size != 0) return KVC_ERR_ARG;  // paged caches: kvc_block_table_append
  if (total_new < 0 || max_new < 0) return KVC_ERR_ARG;
  if (out_dtype != KVC_BF16 && out_dtype != KVC_F32) return KVC_ERR_UNSUPPORTED;
  Plan pl{};
  // the attention's checks, on the lengths after the append
  st = check_attn(d, n_q, q, k_cache, v_cache, seq_lens_out, nullptr, scale, workspace,
                  workspace_bytes, &pl);
  if (st != KVC_OK) return st;
  if (d->batch == 0) return total_new == 0 ? KVC_OK : KVC_ERR_ARG;
  if (!seq_lens || !cu_new || !out || seq_lens_out == seq_lens) return KVC_ERR_ARG;
  if (total_new > 0 && (!k_new || !v_new)) return KVC_ERR_ARG;
  if (!pl.mfma && !fp8_format(d)) {
    // one partition launch appends and attends; the reduce takes the same
    // lengths (before the append, plus the new rows)
    AttnParams p = attn_params(d, pl, n_q, q, k_cache, v_cache, seq_lens, nullptr, scale,
                               workspace, dev_status, out, out_dtype);
    p.cu_new = cu_new;
    p.k_new = k_new;
    p.v_new = v_new;
    p.k_out = k_cache;
    p.v_out = v_cache;
    p.seq_lens_out = seq_lens_out;
    p.total_new = total_new;
    st = hip_status(launch_partition_valu(p, d->dtype, (hipStream_t)stream));
    if (st != KVC_OK || p.cnt) return st;  // combined inside the launch
    ReduceParams r = reduce_params(d, pl, n_q, d->head_dim, seq_lens, workspace, out, dev_status);
    r.cu_new = cu_new;
    r.total_new = total_new;
    return hip_status(launch_reduce(r, out_dtype, (hipStream_t)stream));
  }
  // grouped rows or FP8: the append kernel, then attention over its lengths
  st = kvc_append(d, k_new, v_new, seq_lens, cu_new, total_new, max_new, nullptr, k_cache, v_cache,
                  seq_lens_out, dev_status, stream);
  if (st != KVC_OK) return st;
  st = run_partition(d, pl, q, n_q, k_cache, v_cache, seq_lens_out, nullptr, scale, workspace,
                     dev_status, stream, out, out_dtype);
  if (st != KVC_OK || pl.fused) return st;
  return run_reduce(d, pl, n_q, d->head_dim, seq_lens_out, workspace, out, out_dtype, dev_status,
                    stream);
}

int kvc_block_table_append_attn(const kvc_cache_desc* d, const void* k_new, const void* v_new,
                                const int32_t* seq_lens, const int32_t* cu_new, int32_t total_new,
                                int32_t max_new, int32_t* block_table, const int32_t* free_list,
                                const int32_t* free_head_in, int32_t* free_head_out,
                                int32_t* slot_mapping, void* k_cache, void* v_cache,
                                int32_t* seq_lens_out, const void* q, int32_t n_q, float scale,
                                void* out, int32_t out_dtype, void* workspace,
                                size_t workspace_bytes, int32_t* dev_status, void* stream) {
  int st = check_desc(d);
  if (st != KVC_OK) return st;
  if (d->block_size == 0) return KVC_ERR_ARG;  // contiguous caches: kvc_append_attn
  if (total_new < 0 || max_new < 0) return KVC_ERR_ARG;
  if (out_dtype != KVC_BF16 && out_dtype != KVC_F32) return KVC_ERR_UNSUPPORTED;
  if (d->batch > kMaxFusedBatch) return KVC_ERR_UNSUPPORTED;
  Plan pl{};
  // the attention's checks, on the lengths after the append
  st = check_attn(d, n_q, q, k_cache, v_cache, seq_lens_out, block_table, scale, workspace,
                  workspace_bytes, &pl);
  if (st != KVC_OK) return st;
  if (d->batch == 0) return total_new == 0 ? KVC_OK : KVC_ERR_ARG;
  if (!seq_lens || !cu_new || !free_list || !free_head_in || !free_head_out || !out ||
      seq_lens_out == seq_lens)
    return KVC_ERR_ARG;
  if (total_new > 0 && (!k_new || !v_new || !slot_mapping)) return KVC_ERR_ARG;
  if (!pl.mfma && !pl.sk && !fp8_format(d)) {
    // one partition launch takes the blocks, appends and attends (the
    // combine inside it too, or a reduce over the same lengths)
    AttnParams p = attn_params(d, pl, n_q, q, k_cache, v_cache, seq_lens, block_table, scale,
                               workspace, dev_status, out, out_dtype);
    p.cu_new = cu_new;
    p.k_new = k_new;
    p.v_new = v_new;
    p.k_out = k_cache;
    p.v_out = v_cache;
    p.seq_lens_out = seq_lens_out;
    p.total_new = total_new;
    p.free_list = free_list;
    p.head_in = free_head_in;
    p.head_out = free_head_out;
    p.table_out = block_table;
    p.slots = slot_mapping;
    st = hip_status(launch_partition_valu(p, d->dtype, (hipStream_t)stream));
    if (st != KVC_OK || p.cnt) return st;
    ReduceParams r = reduce_params(d, pl, n_q, d->head_dim, seq_lens, workspace, out, dev_status);
    r.cu_new = cu_new;
    r.total_new = total_new;
    return hip_status(launch_reduce(r, out_dtype, (hipStream_t)stream));
  }
  // grouped rows, stream-K or FP8: block table and append in one launch, then
  // attention
  st = kvc_block_table_append(d, k_new, v_new, seq_lens, cu_new, total_new, max_new, block_table,
                              free_list, free_head_in, free_head_out, slot_mapping, k_cache,
                              v_cache, seq_lens_out, dev_status, stream);
  if (st != KVC_OK) return st;
  st = run_partition(d, pl, q, n_q, k_cache, v_cache, seq_lens_out, block_table, scale, workspace,
                     dev_status, stream, out, out_dtype);
  if (st != KVC_OK || pl.fused) return st;
  return run_reduce(d, pl, n_q, d->head_dim, seq_lens_out, workspace, out, out_dtype, dev_status,
                    stream);
}

int kvc_attn_partition(const kvc_cache_desc* d, const void* q, int32_t n_q, const void* k_cache,
                       const void* v_cache, const int32_t* seq_lens, const int32_t* block_table,
                       float scale, void* workspace, size_t workspace_bytes, int32_t* dev_status,
                       void* stream) {
  Plan pl{};
  int st = check_attn(d, n_q, q, k_cache, v_cache, seq_lens, block_table, scale, workspace,
                      workspace_bytes, &pl);
  if (st != KVC_OK || d->batch == 0) return st;
  return run_partition(d, pl, q, n_q, k_cache, v_cache, seq_lens, block_table, scale, workspace,
                       dev_status, stream);
}

int kvc_attn_reduce(const kvc_cache_desc* d, int32_t n_q, const int32_t* seq_lens,
                    const void* workspace, size_t workspace_bytes, void* out, int32_t out_dtype,
                    int32_t* dev_status, void* stream) {
  int st = check_reduce(d, n_q, seq_lens, workspace, out, out_dtype);
  if (st != KVC_OK || d->batch == 0) return st;
  const Plan pl = make_plan(d, n_q);
  if (workspace_bytes < pl.bytes) return KVC_ERR_WORKSPACE;
  return run_reduce(d, pl, n_q, d->head_dim, seq_lens, workspace, out, out_dtype, dev_status,
                    stream);
}

int kvc_verify_attn(const kvc_cache_desc* d, const void* q, int32_t n_q, const void* k_cache,
                    const void* v_cache, const int32_t* seq_lens, const int32_t* block_table,
                    float scale, void* out, int32_t out_dtype, void* workspace,
                    size_t workspace_bytes, int32_t* dev_status, void* stream) {
  Plan pl{};
  int st = check_attn(d, n_q, q, k_cache, v_cache, seq_lens, block_table, scale, workspace,
                      workspace_bytes, &pl);
  if (st != KVC_OK) return st;
  if (out_dtype != KVC_BF16 && out_dtype != KVC_F32) return KVC_ERR_UNSUPPORTED;
  if (d->batch == 0) return KVC_OK;
  if (!out) return KVC_ERR_ARG;
  st = run_partition(d, pl, q, n_q, k_cache, v_cache, seq_lens, block_table, scale, workspace,
                     dev_status, stream, out, out_dtype);
  if (st != KVC_OK || pl.fused) return st;
  return run_reduce(d, pl, n_q, d->head_dim, seq_lens, workspace, out, out_dtype, dev_status,
                    stream);
}

int kvc_decode_attn(const kvc_cache_desc* d, const void* q, const void* k_cache,
                    const void* v_cache, const int32_t* seq_lens, const int32_t* block_table,
                    float scale, void* out, int32_t out_dtype, void* workspace,
                    size_t workspace_bytes, int32_t* dev_status, void* stream) {
  return kvc_verify_attn(d, q, 1, k_cache, v_cache, seq_lens, block_table, scale, out, out_dtype,
                         workspace, workspace_bytes, dev_status, stream);
}

int kvc_verify_attn_noalloc(const kvc_cache_desc* d, const void* q, int32_t n_q,
                            const void* k_cache, const void* v_cache, const int32_t* seq_lens,
                            const int32_t* block_table, float scale, void* out,
                            int32_t out_dtype, int32_t* dev_status, void* stream) {
  // Every host check first, the scratch size included, so that a refused
  // call makes no device call; the scratch address is looked up only for a
  // call that runs.
  int st = check_attn_args(d, n_q, q, k_cache, v_cache, seq_lens, block_table, scale);
  if (st != KVC_OK) return st;
  if (out_dtype != KVC_BF16 && out_dtype != KVC_F32) return KVC_ERR_UNSUPPORTED;
  if (d->batch == 0) return KVC_OK;
  if (!out) return KVC_ERR_ARG;
  const Plan pl = make_plan(d, n_q);
  if (pl.grid > 0x7fffffffL) return KVC_ERR_UNSUPPORTED;
  if (pl.bytes > (size_t)KVC_NOALLOC_SCRATCH_BYTES) return KVC_ERR_WORKSPACE;
  if (stream) {  // the kernels run on the stream's device: it must be the current one
    int cur = -1;
    hipDevice_t sdev = -1;
    if (hipGetDevice(&cur) != hipSuccess ||
        hipStreamGetDevice((hipStream_t)stream, &sdev) != hipSuccess)
      return KVC_ERR_HIP;
    if (sdev != cur) return KVC_ERR_ARG;
  }
  void* ws = scratch_ptr();
  if (!ws) return KVC_ERR_HIP;
  st = run_partition(d, pl, q, n_q, k_cache, v_cache, seq_lens, block_table, scale, ws,
                     dev_status, stream, out, out_dtype);
  if (st != KVC_OK || pl.fused) return st;
  return run_reduce(d, pl, n_q, d->head_dim, seq_lens, ws, out, out_dtype, dev_status, stream);
}

int kvc_fork(const kvc_cache_desc* d, const int32_t* parents, const int32_t* children,
             int32_t n_forks, int32_t* seq_lens, int32_t* block_table, int32_t* ref_counts,
             int32_t* dev_status, void* stream) {
  int st = check_desc(d);
  if (st != KVC_OK) return st;
  if (d->block_size == 0) return KVC_ERR_ARG;
  if (n_forks < 0) return KVC_ERR_ARG;
  if (n_forks == 0 || d->batch == 0) return KVC_OK;
  if (!parents || !children || !seq_lens || !block_table || !ref_counts) return KVC_ERR_ARG;
  LifecycleArgs a{};
  a.seq_lens = seq_lens;
  a.seq_lens_out = seq_lens;
  a.parents = parents;
  a.children = children;
  a.table = block_table;
  a.refs = ref_counts;
  a.status = dev_status;
  a.B = d->batch;
  a.bs = d->block_size;
  a.max_blocks = d->max_blocks_per_seq;
  a.N = d->num_blocks;
  a.n = n_forks;
  return hip_status(launch_fork(a, (hipStream_t)stream));
}

int kvc_truncate(const kvc_cache_desc* d, const int32_t* seq_lens, const int32_t* new_lens,
                 int32_t* block_table, int32_t* free_list, const int32_t* free_head_in,
                 int32_t* free_head_out, int32_t* ref_counts, int32_t* seq_lens_out,
                 int32_t* dev_status, void* stream) {
  int st = check_desc(d);
  if (st != KVC_OK) return st;
  if (d->block_size == 0) return KVC_ERR_ARG;
  if (d->num_blocks > kMaxPoolBlocks) return KVC_ERR_UNSUPPORTED;
  if (d->batch == 0) return KVC_OK;
  if (!seq_lens || !new_lens || !block_table || !free_list || !free_head_in || !free_head_out ||
      !seq_lens_out)
    return KVC_ERR_ARG;
  LifecycleArgs a{};
  a.seq_lens = seq_lens;
  a.new_lens = new_lens;
  a.table = block_table;
  a.free_list = free_list;
  a.head_in = free_head_in;
  a.head_out = free_head_out;
  a.refs = ref_counts;
  a.seq_lens_out = seq_lens_out;
  a.status = dev_status;
  a.B = d->batch;
  a.bs = d->block_size;
  a.max_blocks = d->max_blocks_per_seq;
  a.N = d->num_blocks;
  return hip_status(launch_truncate(a, (hipStream_t)stream));
}

int kvc_copy_blocks(const kvc_cache_desc* d, const int32_t* src, const int32_t* dst, int32_t n,
                    void* k_cache, void* v_cache, int32_t* dev_status, void* stream) {
  int st = check_desc(d);
  if (st != KVC_OK) return st;
  if (d->block_size == 0) return KVC_ERR_ARG;
  if (n < 0 || n >= kMaxBatch) return KVC_ERR_ARG;
  if (n == 0) return KVC_OK;
  if (!src || !dst || !k_cache) return KVC_ERR_ARG;  // v_cache NULL: a key-only pool
  CopyArgs c{};
  c.src = src;
  c.dst = dst;
  c.k = (uint8_t*)k_cache;
  c.v = (uint8_t*)v_cache;
  c.block_bytes = fp8_format(d) ? (long)d->num_kv_heads * (d->block_size / kTile) *
                                      fp8_tile_bytes(d->head_dim)
                                : (long)d->num_kv_heads * d->block_size * d->head_dim *
                                      (long)elem_bytes(d);
  c.N = d->num_blocks;
  c.status = dev_status;
  return hip_status(launch_copy_blocks(c, n, (hipStream_t)stream));
}

int kvc_cow(const kvc_cache_desc* d, const int32_t* seq_lens, const int32_t* cu_new,
            int32_t* block_table, int32_t* free_list, const int32_t* free_head_in,
            int32_t* free_head_out, int32_t* ref_counts, void* k_cache, void* v_cache,
            int32_t* cow_src, int32_t* cow_dst, int32_t* dev_status, void* stream) {
  int st = check_desc(d);
  if (st != KVC_OK) return st;
  if (d->block_size == 0) return KVC_ERR_ARG;
  if (d->num_blocks > kMaxPoolBlocks) return KVC_ERR_UNSUPPORTED;
  if (d->batch == 0) return KVC_OK;
  if (!seq_lens || !cu_new || !block_table || !free_list || !free_head_in || !free_head_out ||
      !ref_counts || !k_cache || !cow_src || !cow_dst)
    return KVC_ERR_ARG;
  LifecycleArgs a{};
  a.seq_lens = seq_lens;
  a.cu_new = cu_new;
  a.table = block_table;
  a.free_list = free_list;
  a.head_in = free_head_in;
  a.head_out = free_head_out;
  a.refs = ref_counts;
  a.cow_src = cow_src;
  a.cow_dst = cow_dst;
  a.status = dev_status;
  a.B = d->batch;
  a.bs = d->block_size;
  a.max_blocks = d->max_blocks_per_seq;
  a.N = d->num_blocks;
  hipError_t e = launch_cow(a, (hipStream_t)stream);
  if (e != hipSuccess) return KVC_ERR_HIP;
  return kvc_copy_blocks(d, cow_src, cow_dst, d->batch, k_cache, v_cache, dev_status, stream);
}

size_t kvc_mla_workspace_bytes(const kvc_cache_desc* d, int32_t n_q, int32_t value_dim) {
  if (check_mla(d, n_q, value_dim) != KVC_OK) return 0;
  return make_mla_plan(d, n_q).bytes;
}

int32_t kvc_mla_partition_tokens(const kvc_cache_desc* d, int32_t n_q, int32_t value_dim) {
  const int st = check_mla(d, n_q, value_dim);
  return st != KVC_OK ? st : make_mla_plan(d, n_q).P;
}

int kvc_mla_attn_partition(const kvc_cache_desc* d, const void* q, int32_t n_q,
                           const void* latent_cache, const int32_t* seq_lens,
                           const int32_t* block_table, int32_t value_dim, float scale,
                           void* workspace, size_t workspace_bytes, int32_t* dev_status,
                           void* stream) {
  int st = check_mla(d, n_q, value_dim);
  if (st != KVC_OK) return st;
  if (d->batch == 0) return KVC_OK;
  if (!q || !latent_cache || !seq_lens || !workspace) return KVC_ERR_ARG;
  if ((d->block_size > 0) != (block_table != nullptr)) return KVC_ERR_ARG;
  if (!isfinite(scale)) return KVC_ERR_ARG;
  if (((uintptr_t)workspace & 15) != 0) return KVC_ERR_ARG;
  const Plan pl = make_mla_plan(d, n_q);
  if (workspace_bytes < pl.bytes) return KVC_ERR_WORKSPACE;
  const AttnParams p = attn_params(d, pl, n_q, q, latent_cache, latent_cache, seq_lens,
                                   block_table, scale, workspace, dev_status);
  st = hip_status(launch_partition_mla(p, (hipStream_t)stream));
  if (st != KVC_OK) return st;
  return KVC_OK;
}

int kvc_mla_attn_reduce(const kvc_cache_desc* d, int32_t n_q, int32_t value_dim,
                        const int32_t* seq_lens, const void* workspace, size_t workspace_bytes,
                        void* out, int32_t out_dtype, int32_t* dev_status, void* stream) {
  int st = check_mla(d, n_q, value_dim);
  if (st != KVC_OK) return st;
  if (out_dtype != KVC_BF16 && out_dtype != KVC_F32) return KVC_ERR_UNSUPPORTED;
  if (d->batch == 0) return KVC_OK;
  if (!seq_lens || !workspace || !out) return KVC_ERR_ARG;
  if (((uintptr_t)workspace & 15) != 0) return KVC_ERR_ARG;
  const Plan pl = make_mla_plan(d, n_q);
  if (workspace_bytes < pl.bytes) return KVC_ERR_WORKSPACE;
  return run_reduce(d, pl, n_q, kMlaValueDim, seq_lens, workspace, out, out_dtype, dev_status,
                    stream);
}

int kvc_mla_attn(const kvc_cache_desc* d, const void* q, int32_t n_q, const void* latent_cache,
                 const int32_t* seq_lens, const int32_t* block_table, int32_t value_dim,
                 float scale, void* out, int32_t out_dtype, void* workspace,
                 size_t workspace_bytes, int32_t* dev_status, void* stream) {
  int st = check_mla(d, n_q, value_dim);
  if (st != KVC_OK) return st;
  if (out_dtype != KVC_BF16 && out_dtype != KVC_F32) return KVC_ERR_UNSUPPORTED;
  if (d->batch == 0) return KVC_OK;
  if (!q || !latent_cache || !seq_lens || !workspace || !out) return KVC_ERR_ARG;
  if ((d->block_size > 0) != (block_table != nullptr)) return KVC_ERR_ARG;
  if (!isfinite(scale)) return KVC_ERR_ARG;
  if (((uintptr_t)workspace & 15) != 0) return KVC_ERR_ARG;
  const Plan pl = make_mla_plan(d, n_q);
  if (workspace_bytes < pl.bytes) return KVC_ERR_WORKSPACE;
  const AttnParams p = attn_params(d, pl, n_q, q, latent_cache, latent_cache, seq_lens,
                                   block_table, scale, workspace, dev_status);
  st = hip_status(launch_partition_mla(p, (hipStream_t)stream));
  if (st != KVC_OK) return st;
  return run_reduce(d, pl, n_q, kMlaValueDim, seq_lens, workspace, out, out_dtype, dev_status,
                    stream);
}

int kvc_prefill_attn(const kvc_cache_desc* d, const void* q, const int32_t* cu_q, int32_t total_q,
                     int32_t max_q, const void* k_cache, const void* v_cache,
                     const int32_t* seq_lens, const int32_t* block_table, float scale, void* out,
                     int32_t out_dtype, int32_t* dev_status, void* stream) {
  int st = check_desc(d);
  if (st != KVC_OK) return st;
  if (d->dtype != KVC_BF16 || d->head_dim == kMlaKeyDim) return KVC_ERR_UNSUPPORTED;
  if (out_dtype != KVC_BF16 && out_dtype != KVC_F32) return KVC_ERR_UNSUPPORTED;
  if (total_q < 0 || max_q < 0) return KVC_ERR_ARG;
  if (d->block_size > 0 && d->max_blocks_per_seq > 4096) return KVC_ERR_UNSUPPORTED;
  if (d->batch == 0 || total_q == 0) return KVC_OK;
  if (!q || !cu_q || !k_cache || !v_cache || !seq_lens || !out) return KVC_ERR_ARG;
  if ((d->block_size > 0) != (block_table != nullptr)) return KVC_ERR_ARG;
  if (!isfinite(scale)) return KVC_ERR_ARG;
  PrefillParams p{};
  p.q = q;
  p.cu_q = cu_q;
  p.k = k_cache;
  p.v = v_cache;
  p.seq_lens = seq_lens;
  p.table = block_table;
  p.out = out;
  p.status = dev_status;
  p.B = d->batch;
  p.Hq = d->num_q_heads;
  p.Hkv = d->num_kv_heads;
  p.G = d->num_q_heads / d->num_kv_heads;
  p.D = d->head_dim;
  p.bs = d->block_size;
  p.S_max = d->max_seq_len;
  p.max_blocks = d->max_blocks_per_seq;
  p.N = d->num_blocks;
  p.cap = capacity(d);
  p.total_q = total_q;
  p.max_q = max_q;
  p.scale_log2 = (float)((double)scale * 1.4426950408889634);
  return hip_status(launch_prefill(p, out_dtype, (hipStream_t)stream));
}

size_t kvc_cache_bytes(const kvc_cache_desc* d) {
  if (check_desc(d) != KVC_OK) return 0;
  if (fp8_format(d)) return cache_rows(d) / kTile * (size_t)fp8_tile_bytes(d->head_dim);
  return cache_rows(d) * d->head_dim * elem_bytes(d);
}

size_t kvc_attn_workspace_bytes(const kvc_cache_desc* d, int32_t n_q) {
  if (check_desc(d) != KVC_OK || n_q < 1 || n_q > 16) return 0;
  return make_plan(d, n_q).bytes;
}

int32_t kvc_attn_partition_tokens(const kvc_cache_desc* d, int32_t n_q) {
  const int st = check_desc(d);
  if (st != KVC_OK) return st;
  if (n_q < 1 || n_q > 16) return KVC_ERR_UNSUPPORTED;
  return make_plan(d, n_q).P;
}

int32_t kvc_attn_launches(const kvc_cache_desc* d, int32_t n_q) {
  const int st = check_desc(d);
  if (st != KVC_OK) return st;
  if (n_q < 1 || n_q > 16) return KVC_ERR_UNSUPPORTED;
  if (d->head_dim == kMlaKeyDim) return KVC_ERR_UNSUPPORTED;  // the kvc_mla_* calls
  return make_plan(d, n_q).fused ? 1 : 2;
}

const char* kvc_status_string(int32_t status) {
  switch (status) {
    case KVC_OK: return "ok";
    case KVC_ERR_ARG: return "invalid argument";
    case KVC_ERR_SHAPE: return "inconsistent shape";
    case KVC_ERR_UNSUPPORTED: return "unsupported size or type";
    case KVC_ERR_WORKSPACE: return "workspace too small";
    case KVC_ERR_CAPACITY: return "sequence capacity exceeded";
    case KVC_ERR_NO_BLOCKS: return "free block list exhausted";
    case KVC_ERR_HIP: return "HIP launch failed";
    case KVC_ERR_DATA: return "device data out of range";
    default: return "unknown status";
  }
}

}  // extern "C"
