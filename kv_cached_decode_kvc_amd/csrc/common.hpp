// common.hpp -- device helpers shared by the kvc kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvc.h"

namespace kvc {

constexpr int kWave = 64;
constexpr int kTile = 16;  // keys per inner-loop tile; every block_size is a multiple

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Everything the attention partition kernels need, passed by value.
struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* seq_lens;
  const int32_t* table;  // NULL for a contiguous cache
  float* ws_o;           // [rows][max_parts][D]
  float* ws_ml;          // [rows][max_parts][2]: running max (log2 domain), running sum
  int32_t* status;
  int B, n_q, Hq, Hkv, G, D;
  int bs, S_max, max_blocks, N;
  int P, max_parts;
  int slots_u;           // > 0: partition length chosen per launch (part_tokens)
  int P_lo;              //   between P_lo and P
  int cap;               // tokens a sequence may hold
  float scale_log2;      // scale * log2(e): scores go straight into exp2
  // Stream-K split (matrix-core kernel; sk_meta == NULL: fixed partitions).
  // Segment s = (b * Hkv + g) * n_rb + rb; piece (s, worker w) keeps its rows'
  // partials at workspace rows (s + w) * sk_rows + i, and sk_meta[s] = (first,
  // last) worker of segment s, written by the first.
  int2* sk_meta;
  int sk_workers;        // workers launched (one workgroup each)
  int sk_rows;           // rows a piece holds: min(16 * NT, G * n_q)
  int sk_min_tiles;      // fewest tiles a worker takes (fewer workers for small batches)
  // Append fused into the partition launch (contiguous cache, vector-ALU
  // kernel; cu_new == NULL: none).  seq_lens then holds the lengths before
  // the append; sequence b's new rows are rows cu_new[b] .. cu_new[b+1] of
  // k_new / v_new, read from there by the tiles that reach them and written
  // into the cache by one work item per KV head, which also writes
  // seq_lens_out.
  const int32_t* cu_new;
  const void* k_new;
  const void* v_new;
  void* k_out;           // the cache buffers (the same memory as k, v)
  void* v_out;
  int32_t* seq_lens_out;
  int total_new;
  // Block table fused in as well (paged cache with cu_new; free_list != NULL):
  // sequence b's new rows go to the blocks its table already holds (the
  // partly filled last one) or to blocks taken from the free list at
  // *head_in + (new blocks of the sequences before b), all or nothing, as
  // kvc_block_table_append does it; table_out (the same table as `table`),
  // head_out, slots and seq_lens_out receive its outputs.  The partition's
  // tiles never read a table entry this launch writes: rows from the old
  // length on come from k_new / v_new.
  const int32_t* free_list;
  const int32_t* head_in;
  int32_t* head_out;
  int32_t* table_out;
  int32_t* slots;
  // Combine fused into the partition launch of the vector-ALU kernel (cnt ==
  // NULL: the reduce kernel combines).  cnt[row] counts the row's finished
  // partitions; the one that completes the row merges all of its partials
  // and writes the row to `out`, then sets cnt[row] back to zero, so the
  // counters are zero between launches.
  uint32_t* cnt;
  void* out;
  int out_bf16;          // out: bf16 (1) or fp32 (0), [B][n_q][Hq][D]
};

// Partials that a launch's own work items combine cross XCDs, whose L2
// caches are separate.  They are written and read with agent-scope atomic
// stores and loads (relaxed), which the compiler emits as write-through and
// coherent accesses (the sc1 cache policy): no device-scope fence, which
// would write back and invalidate a whole L2, is needed around them.
__device__ __forceinline__ void st_shared(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_shared(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The same cache policy (sc1) on 16-byte buffer accesses, so that a row of
// partial outputs goes out and comes back in whole lines: `base` is
// wave-uniform (a buffer resource lives in scalar registers) and the byte
// offsets stay far below the resource's 2 GiB range.  Word 3 of the
// resource is gfx950's raw 32-bit buffer format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t shared_rsrc(const float* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, 0x7fffffff, 0x00020000);
}
constexpr int kCoherentPolicy = 16;  // the sc1 bit of a buffer access's cache policy
__device__ __forceinline__ void st_shared4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, f32x4_t v) {
  typedef unsigned u32x4_v __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_v, v), r, (int)byte_off, 0,
                                         kCoherentPolicy);
}
__device__ __forceinline__ f32x4_t ld_shared4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(f32x4_t,
                            __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, kCoherentPolicy));
}

// Arrival of one piece of a unit whose partials it has written with
// st_shared: true for the piece that completes the unit (the n-th), which may
// then read every piece's partials with ld_shared.  This wavefront's partial
// stores are complete (s_waitcnt vmcnt(0): a write-through store counts as
// done once the coherent level has it) before its count goes in; the
// completing piece resets the counter.  Called by all lanes; the result is
// wave-uniform.
__device__ __forceinline__ bool arrive_last(uint32_t* cnt, long unit, int n) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0), expcnt and lgkmcnt not waited on
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  uint32_t old = 0;
  if ((threadIdx.x & (kWave - 1)) == 0)
    old = __hip_atomic_fetch_add(cnt + unit, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = __builtin_amdgcn_readfirstlane(old);
  if (old + 1 != (uint32_t)n) return false;
  if ((threadIdx.x & (kWave - 1)) == 0)
    __hip_atomic_store(cnt + unit, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// One wavefront's scan of a block-table step over the whole batch: the new
// blocks of every sequence (total) and of the sequences before b (before),
// the free-list head, and the step's error, all or nothing as in the block
// table ("Inference-1", PagedAttention: blocks on demand when the last one
// is full): KVC_ERR_DATA for a negative length or count, KVC_ERR_CAPACITY for
// a sequence past max_blocks, KVC_ERR_NO_BLOCKS for too few free blocks.
// Every lane must call it; the result is wave-uniform.
struct AllocScan {
  int head, total, before, err;
};
__device__ __forceinline__ AllocScan alloc_scan(const int32_t* seq_lens, const int32_t* cu_new,
                                                const int32_t* head_in, int B, int bs,
                                                int max_blocks, int N, int b) {
  const int lane = (int)(threadIdx.x & (kWave - 1));
  int total = 0, before = 0, bad = 0, over = 0;
  for (int i = lane; i < B; i += kWave) {
    const int len = seq_lens[i], n = cu_new[i + 1] - cu_new[i];
    if (len < 0 || n < 0) {
      bad = 1;
      continue;
    }
    const long have = ((long)len + bs - 1) / bs, want = ((long)len + n + bs - 1) / bs;
    if (want > max_blocks) {
      over = 1;
      continue;
    }
    total += (int)(want - have);
    if (i < b) before += (int)(want - have);
  }
  for (int m = 1; m < kWave; m <<= 1) {
    total += __shfl_xor(total, m);
    before += __shfl_xor(before, m);
  }
  AllocScan s;
  s.head = __builtin_amdgcn_readfirstlane(*head_in);
  s.total = __builtin_amdgcn_readfirstlane(total);
  s.before = __builtin_amdgcn_readfirstlane(before);
  s.err = __any(bad) ? KVC_ERR_DATA
          : __any(over) ? KVC_ERR_CAPACITY
          : (s.head < 0 || (long)s.head + s.total > N) ? KVC_ERR_NO_BLOCKS
          : 0;
  return s;
}

// Online merge of partial (mj, lj, oj[0..N)) into (m, d, acc): the partials'
// maxima are in the log2 domain and an empty partial has mj = -inf
// ("Inference-1", "FlashDecoding": every chunk's output is rescaled by
// 2^(m_j - m*) before the sum).
template <int N>
__device__ __forceinline__ void merge_partial(float& m, float& d, float* acc, float mj, float lj,
                                              const float* oj) {
  if (mj == -INFINITY) return;
  const float mn = fmaxf(m, mj);
  const float a = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mn);
  const float w = __builtin_amdgcn_exp2f(mj - mn);
  d = d * a + lj * w;
#pragma unroll
  for (int k = 0; k < N; ++k) acc[k] = acc[k] * a + oj[k] * w;
  m = mn;
}

// Attended length of sequence b and whether it is usable: seq_lens[b], or,
// with an append fused in, seq_lens[b] plus its new rows.  *code receives the
// status an unusable sequence reports (a capacity overflow of the append, or
// bad data).
__device__ __forceinline__ int attended_len(const int32_t* seq_lens, const int32_t* cu_new,
                                            int total_new, int b, int n_q, int cap, int* code) {
  int L = seq_lens[b];
  *code = KVC_ERR_DATA;
  if (cu_new) {
    const int c0 = cu_new[b], n = cu_new[b + 1] - c0;
    if (L < 0 || n < 0 || c0 < 0 || c0 + n > total_new) return -1;
    if ((long)L + n > cap) {
      *code = KVC_ERR_CAPACITY;
      return -1;
    }
    L += n;
  }
  return (L >= n_q && L <= cap) ? L : -1;
}

struct PrefillParams {
  const void* q;            // [total_q][Hq][D] bf16, sequence b's rows at cu_q[b] ..
  const int32_t* cu_q;      // [B + 1]
  const void* k;
  const void* v;
  const int32_t* seq_lens;  // lengths after the chunk was appended
  const int32_t* table;     // NULL for a contiguous cache
  void* out;                // [total_q][Hq][D]
  int32_t* status;
  int B, Hq, Hkv, G, D, bs, S_max, max_blocks, N, cap, total_q, max_q;
  float scale_log2;
};

struct ReduceParams {
  const float* ws_o;
  const float* ws_ml;
  const int32_t* seq_lens;
  void* out;
  int32_t* status;
  int B, n_q, Hq, D, P, max_parts, cap;
  int slots_u, P_lo;  // as in AttnParams
  const int2* sk_meta;  // stream-K partials (as in AttnParams); NULL: fixed partitions
  int sk_rows, sk_workers, G, Hkv, rows_item;
  const int32_t* cu_new;  // append fused into the partition launch (as in AttnParams)
  int total_new;
};

// Partition length of a launch, in tokens.  With slots_u = 0 it is the
// planned P.  Otherwise (the matrix-core decode and verify kernels) it is
// chosen from the actual lengths so that the partitions of the whole batch
// just fit one round of resident wavefronts: with T the 16-key tiles of all
// sequences (lengths clamped to [0, cap]) and slots_u the resident slots per
// unit of a sequence, 16 * ceil(T / (slots_u - B)) tokens, kept within
// [P_lo, P].  Since a sequence of t tiles has ceil(t / tau) <= t / tau + 1
// partitions, the batch then has at most slots_u wavefronts per unit, and
// none streams more than tau tiles.  Every lane of the wavefront must call
// it; the result is wave-uniform.
__device__ __forceinline__ int part_tokens(const int32_t* seq_lens, int B, int cap, int slots_u,
                                           int P_lo, int P) {
  if (slots_u <= 0) return P;
  int t = 0;
  for (int i = (int)(threadIdx.x & (kWave - 1)); i < B; i += kWave)
    t += (min(max(seq_lens[i], 0), cap) + kTile - 1) / kTile;
  for (int m = 1; m < kWave; m <<= 1) t += __shfl_xor(t, m);
  const int denom = slots_u - B;
  const int tau = denom > 0 ? (t + denom - 1) / denom : P / kTile;
  return __builtin_amdgcn_readfirstlane(min(max(tau * kTile, P_lo), P));
}

// Work items of the split-KV partition kernels: (sequence b, partition part,
// unit u), one wavefront each, one wavefront per workgroup.  The hardware
// hands workgroups to the eight XCDs round robin (workgroup i runs on XCD
// i % 8), so the id is split as i = 8 t + x and XCD x takes, of every
// sequence, the items k = part * U + u with k = 8 m + x', where x' is x
// rotated by the sequence number.  Every sequence's work is then spread evenly
// over the XCDs whatever its length (an order with the partition index
// innermost would hand the high partitions, which only long sequences have,
// to a fixed subset of XCDs), and an XCD's items of one sequence are
// dispatched together, so they stream neighbouring tiles at the same time.
// Within an XCD the hardware passes workgroups to its four shader engines in
// strict rotation, whatever their load, so with m in order the engine of an
// item would follow m mod 4, i.e. its partition: one engine would get
// partitions 0, 4, 8, ... and another 3, 7, 11, ..., which only long
// sequences have.  Each full block of 8 consecutive m is therefore walked as
// a snake (0 1 2 3 7 6 5 4): the two positions that share an engine hold
// offsets j and 7 - j, and every engine's partitions have the same mean.
constexpr int kXcds = 8;

struct WorkItem {
  int b, part, u;
  bool live;  // false: padding beyond max_parts * U
};

__device__ __forceinline__ WorkItem xcd_item(long wg, int U, int max_parts) {
  const int x = (int)(wg % kXcds);
  const long t = wg / kXcds;
  const int K = max_parts * U;
  const int M = (K + kXcds - 1) / kXcds;
  WorkItem w;
  w.b = (int)(t / M);
  int m = (int)(t % M);
  // snake within each full block of 8: positions j and j + 4 hold offsets j
  // and 7 - j
  if ((m | 7) < M && (m & 4)) m ^= 3;
  const int xr = (x + kXcds - (w.b % kXcds)) % kXcds;
  const int k = m * kXcds + xr;
  w.live = k < K;
  w.part = k / U;
  w.u = k % U;
  return w;
}

// workgroups of a partition launch (B sequences, U units, max_parts partitions)
inline long xcd_grid(int B, int U, int max_parts) {
  const long M = ((long)max_parts * U + kXcds - 1) / kXcds;
  return (long)B * M * kXcds;
}

__device__ __forceinline__ void report(int32_t* status, int code) {
  if (status) atomicMin(status, code);
}

// bf16 pair held in one 32-bit word: element 2i in the low half.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 bits, round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// N consecutive outputs (N a multiple of 4, `off` a multiple of 4 elements)
// as bf16 (round to nearest even) or fp32.
template <int N>
__device__ __forceinline__ void store_out(void* out, bool bf16, long off, const float* v) {
  static_assert(N % 4 == 0, "whole groups of four");
  if (bf16) {
    uint2* o = reinterpret_cast<uint2*>((uint16_t*)out + off);
#pragma unroll
    for (int k = 0; k < N / 4; ++k)
      o[k] = make_uint2(f32_to_bf16_bits(v[4 * k]) | (f32_to_bf16_bits(v[4 * k + 1]) << 16),
                        f32_to_bf16_bits(v[4 * k + 2]) | (f32_to_bf16_bits(v[4 * k + 3]) << 16));
  } else {
    float4* o = reinterpret_cast<float4*>((float*)out + off);
#pragma unroll
    for (int k = 0; k < N / 4; ++k) o[k] = make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
  }
}

// a.x*b.x + a.y*b.y + c over bf16 pairs with an fp32 accumulator (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte load of data read exactly once (non-temporal: no reuse expected).
__device__ __forceinline__ uint4 load_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// DPP lane permutes inside a row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

// Sum over groups of N consecutive lanes (N = 4, 8, 16 or 32); every lane of
// a group receives the group's total.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 4 || N == 8 || N == 16 || N == 32, "group size");
  x += dpp<kDppQuadXor1>(x);
  x += dpp<kDppQuadXor2>(x);
  if constexpr (N >= 8) x += dpp<kDppRowHalfMirror>(x);
  if constexpr (N >= 16) x += dpp<kDppRowMirror>(x);
  if constexpr (N == 32) x += __shfl_xor(x, 16);
  return x;
}

// Reduce across lanes that differ only in the bits at and above FROM (a power
// of two <= 32): lanes with the same (lane % FROM) end up with the result.
template <int FROM>
__device__ __forceinline__ float cross_max(float x) {
#pragma unroll
  for (int m = FROM; m < kWave; m <<= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}
template <int FROM>
__device__ __forceinline__ float cross_sum(float x) {
#pragma unroll
  for (int m = FROM; m < kWave; m <<= 1) x += __shfl_xor(x, m);
  return x;
}

// Maximum over the four 16-lane rows of a wavefront (lanes i, i ^ 16, i ^ 32
// and i ^ 48), received by every lane.  gfx950's permlane swaps exchange
// rows between two registers on the vector ALU, with no LDS round trip: each
// returns, per lane, itself and its partner across the swap, in some order.
// The IEEE maximum (v_maximum3_f32) needs no canonicalised inputs and
// propagates NaN.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float rows_max(float x) {
  const unsigned u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  x = vmax(x, vmax(__uint_as_float(a[0]), __uint_as_float(a[1])));
  const unsigned w = __float_as_uint(x);
  const auto c = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  return vmax(x, vmax(__uint_as_float(c[0]), __uint_as_float(c[1])));
}

// Orders LDS traffic of one wavefront: LDS instructions of a wave execute in
// issue order, so a compiler-level barrier at wavefront scope is enough for a
// wave-private LDS region.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------
// FP8 cache elements ("Inference-2", brunomaga.github.io, "Quantization"
// number-format table: E4M3 = 1 sign, 4 exponent, 3 mantissa bits, largest
// 448; E5M2 = 1/5/2, largest 57,344).  E4M3 has no infinities (S.1111.111 is
// its NaN), so its largest finite code is 0x7E; E5M2's is 0x7B.
constexpr int kFp8E4M3 = 1;
constexpr int kFp8E5M2 = 2;

template <int F>
struct Fp8Format;
template <>
struct Fp8Format<kFp8E4M3> {
  static constexpr int kMant = 3, kBias = 7;
  static constexpr float kMax = 448.f;
  static constexpr uint32_t kTop = 0x7E;
};
template <>
struct Fp8Format<kFp8E5M2> {
  static constexpr int kMant = 2, kBias = 15;
  static constexpr float kMax = 57344.f;
  static constexpr uint32_t kTop = 0x7B;
};

// FP8 cache layout.  Rows are numbered as in a bf16 cache (a contiguous cache
// pads every (sequence, head) run to a multiple of 16 rows) and grouped in
// tiles of 16 consecutive rows; tile t occupies bytes [t * TB, (t + 1) * TB)
// of the buffer, TB = 16 * D + 64: the 16 rows' codes, then their 16 float32
// scales.  A kernel reading one 16-key tile of one head finds its codes and
// scales in one run of TB bytes, instead of a 64-byte scale read in a distant
// region for every tile (which costs HBM a row activation per 64 bytes).
__host__ __device__ __forceinline__ long fp8_tile_bytes(int D) { return 16L * D + 64; }
__host__ __device__ __forceinline__ long fp8_code_offset(long row, int D) {
  return (row >> 4) * fp8_tile_bytes(D) + (row & 15) * (long)D;
}
__host__ __device__ __forceinline__ long fp8_scale_offset(long row, int D) {
  return (row >> 4) * fp8_tile_bytes(D) + 16L * D + (row & 15) * 4;
}
__host__ __device__ __forceinline__ long fp8_padded_rows(long rows) { return (rows + 15) & ~15L; }

// Code of the FP8 value nearest to the finite y, ties to the even code,
// saturated to the largest finite value.  Scaling by powers of two is exact,
// so rounding the scaled magnitude to an integer (ties to even) rounds the
// mantissa; a mantissa that rounds up to the next power of two carries into
// the exponent field by itself.
template <int F>
__device__ __forceinline__ uint32_t fp8_encode(float y) {
  using Fm = Fp8Format<F>;
  const uint32_t sign = y < 0.f ? 0x80u : 0u;
  const float a = fabsf(y);
  if (!(a < Fm::kMax)) return sign | Fm::kTop;
  const int e = (int)((__float_as_uint(a) >> 23) & 0xff) - 127;  // floor(log2 a) for normal a
  if (e < 1 - Fm::kBias)  // below the smallest normal: multiples of 2^(1 - bias - mant)
    return sign | (uint32_t)__builtin_rintf(__builtin_ldexpf(a, Fm::kBias - 1 + Fm::kMant));
  const int r = (int)__builtin_rintf(__builtin_ldexpf(a, Fm::kMant - e));  // 2^mant .. 2^(mant+1)
  return sign | (uint32_t)(((e + Fm::kBias) << Fm::kMant) + r - (1 << Fm::kMant));
}

// Four codes (one 32-bit word) -> four bf16 values, exactly (every E4M3 and
// E5M2 value is a bf16 value); the hardware conversion decodes these formats.
template <int F>
__device__ __forceinline__ uint2 fp8x4_to_bf16x4(uint32_t w) {
  bf16x2_t lo, hi;
  if constexpr (F == kFp8E4M3) {
    lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, false);
    hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, true);
  } else {
    lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.f, false);
    hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.f, true);
  }
  return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

// Two codes (the low or high half of a word) -> two floats.
template <int F, bool HI>
__device__ __forceinline__ f32x2_t fp8x2_to_f32(uint32_t w) {
  if constexpr (F == kFp8E4M3) return __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
  else return __builtin_amdgcn_cvt_pk_f32_bf8(w, HI);
}

}  // namespace kvc
