// paging.hip -- block-table allocation and the K/V append (integer and byte work).
//
// Block table: "Inference-1" (brunomaga.github.io), "PagedAttention": fixed-size
// blocks allocated on demand, a per-sequence logical -> physical table; "Inference
// o quy mo lon" (truongducdung.dev), 05 "Block table": a block is taken only when
// the last one is full.  Append: "Efficient Inference" (learn.obvix.io), KV-cache
// passage: rows written in place at the current length of a preallocated cache.
#include "launch.hpp"

namespace kvc {

constexpr int kBtThreads = 1024;
constexpr int kBtWaves = kBtThreads / kWave;

// Inclusive prefix sum over a workgroup of kBtThreads (shuffles inside each
// wave, one LDS exchange across waves); also returns the workgroup total.
__device__ __forceinline__ int block_inclusive_scan(int x, int* s_wave, int& total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == kWave - 1) s_wave[wave] = x;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kBtWaves; ++w) {
    const int v = s_wave[w];
    before += w < wave ? v : 0;
    total += v;
  }
  __syncthreads();  // s_wave may be reused by the next call
  return x + before;
}

// One workgroup; thread i owns sequences i, i + kBtThreads, ...  Pass 1
// validates and counts every sequence's new blocks; pass 2 assigns them in
// batch order (free list consumed front to back) and maps each new token to
// its slot, taking the block id straight from the free list or from the
// sequence's already-held last block, so no pass waits on another's stores.
__global__ __launch_bounds__(kBtThreads) void block_table_kernel(BlockTableArgs a) {
  constexpr int kLongSeq = 16;  // sequences with more new tokens go to the token-parallel pass
  __shared__ int s_wave[kBtWaves];
  __shared__ int s_err, s_total, s_long;
  __shared__ int s_cu[kBtThreads], s_first[kBtThreads];  // staged when B < kBtThreads
  const int tid = threadIdx.x;
  const int bs = a.bs;
  const int head = *a.head_in;
  if (tid == 0) {
    s_err = 0;
    s_total = 0;
    s_long = 0;
  }
  __syncthreads();
  for (int b = tid; b < a.B; b += kBtThreads) {
    const int len = a.seq_lens[b];
    const int n = a.cu_new[b + 1] - a.cu_new[b];
    if (len < 0 || n < 0) {
      atomicMin(&s_err, KVC_ERR_DATA);
      continue;
    }
    const long have = ((long)len + bs - 1) / bs;
    const long want = ((long)len + n + bs - 1) / bs;
    if (want > a.max_blocks) atomicMin(&s_err, KVC_ERR_CAPACITY);
    else atomicAdd(&s_total, (int)(want - have));
  }
  __syncthreads();
  int err = s_err;
  if (err == 0 && (head < 0 || (long)head + s_total > a.N)) err = KVC_ERR_NO_BLOCKS;
  if (err != 0) {
    if (tid == 0) {
      report(a.status, err);
      *a.head_out = head;
    }
    return;
  }

  int carry = 0;
  for (int base = 0; base < a.B; base += kBtThreads) {  // uniform trip count
    const int b = base + tid;
    int len = 0, c0 = 0, n = 0, have = 0, need = 0;
    if (b < a.B) {
      len = a.seq_lens[b];
      c0 = a.cu_new[b];
      n = a.cu_new[b + 1] - c0;
      have = (len + bs - 1) / bs;
      need = (int)(((long)len + n + bs - 1) / bs) - have;
    }
    int chunk_total;
    const int first = head + carry + block_inclusive_scan(need, s_wave, chunk_total) - need;
    carry += chunk_total;
    if (b >= a.B) continue;
    int32_t* row = a.table + (long)b * a.max_blocks;
    for (int i = 0; i < need; ++i) row[have + i] = a.free_list[first + i];
    const bool staged = a.B < kBtThreads;
    if (staged) {
      s_cu[b] = c0;
      s_first[b] = first;
      if (b == a.B - 1) s_cu[a.B] = c0 + n;
    }
    if (n > 0 && (c0 < 0 || c0 + n > a.total_new)) {  // cu_new points outside the slot buffer
      report(a.status, KVC_ERR_DATA);
      continue;
    }
    if (staged && n > kLongSeq) {  // many new tokens: spread them over the workgroup below
      s_long = 1;
      continue;
    }
    for (int t = 0; t < n; ++t) {
      const int pos = len + t;
      const int lb = pos / bs;
      const int blk = lb < have ? row[lb] : a.free_list[first + lb - have];
      a.slots[c0 + t] = blk * bs + pos % bs;
    }
  }
  __syncthreads();
  if (a.B < kBtThreads && s_long) {
    // token-parallel slots of the long sequences (prefill-sized appends); table
    // entries of this call are not read back: new blocks come from the free list
    const int total = min(s_cu[a.B], a.total_new);
    for (int i = tid; i < total; i += kBtThreads) {
      int lo = 0, hi = a.B - 1;  // last b with cu_new[b] <= i
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_cu[mid] <= i) lo = mid;
        else hi = mid - 1;
      }
      const int c0 = s_cu[lo];
      const int n = s_cu[lo + 1] - c0;
      if (n <= kLongSeq || i >= a.total_new) continue;  // short ones are done
      const int len = a.seq_lens[lo];
      const int have = (len + bs - 1) / bs;
      const int pos = len + (i - c0);
      const int lb = pos / bs;
      const int blk = lb < have ? a.table[(long)lo * a.max_blocks + lb]
                                : a.free_list[s_first[lo] + lb - have];
      a.slots[i] = blk * bs + pos % bs;
    }
  }
  if (tid == 0) *a.head_out = head + s_total;
}

constexpr int kAppendThreads = 256;

// One 16-byte piece (number w) of new token src_tok's row of KV head g, K
// and V, copied bit for bit to byte offset dst of the caches.
__device__ __forceinline__ void copy_piece(const AppendArgs& a, long src_tok, int g, int w,
                                           long dst) {
  const long src = (src_tok * a.Hkv + g) * a.head_bytes + w * 16;
  const uint4 kv = *reinterpret_cast<const uint4*>(a.k_new + src);
  *reinterpret_cast<uint4*>(a.k_cache + dst) = kv;
  if (a.v_cache) {  // NULL: a key-only cache (MLA latent rows serve as keys and values)
    const uint4 vv = *reinterpret_cast<const uint4*>(a.v_new + src);
    *reinterpret_cast<uint4*>(a.v_cache + dst) = vv;
  }
}

// grid = (vector chunks x token chunks, B): every thread moves one 16-byte
// piece of one new token's K row and V row (a row of a KV head is head_bytes
// long), bit for bit.  Decode steps have one token per sequence, so the grid
// spreads the heads over many workgroups instead of looping inside a few.
__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendArgs a) {
  const int b = blockIdx.y;
  const int vec_per_head = a.head_bytes >> 4;
  const int vec_per_tok = a.Hkv * vec_per_head;
  const int n_vchunks = (vec_per_tok + kAppendThreads - 1) / kAppendThreads;
  const int vchunk = blockIdx.x % n_vchunks;
  const int tchunk = blockIdx.x / n_vchunks;
  const int tok_per_wg = a.tok_per_wg;
  const int len = a.seq_lens[b];
  const int c0 = a.cu_new[b];
  const int n = a.cu_new[b + 1] - c0;
  const bool bad = len < 0 || n < 0 || (a.slots == nullptr && (long)len + n > a.S_max);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    a.seq_lens_out[b] = bad ? len : len + n;
    if (bad) report(a.status, (len < 0 || n < 0) ? KVC_ERR_DATA : KVC_ERR_CAPACITY);
    // more new tokens than the host's max_new promised: the excess is not written
    else if (n > (long)(gridDim.x / n_vchunks) * tok_per_wg) report(a.status, KVC_ERR_DATA);
  }
  if (bad) return;
  const int idx = vchunk * kAppendThreads + threadIdx.x;
  if (idx >= vec_per_tok) return;
  const int g = idx / vec_per_head;
  const int w = idx - g * vec_per_head;
  const int t0 = tchunk * tok_per_wg;
  const int t1 = min(t0 + tok_per_wg, n);
  for (int t = t0; t < t1; ++t) {
    const long src_tok = (long)c0 + t;
    if (src_tok < 0 || src_tok >= a.total_new) {  // cu_new points outside the new-row buffers
      report(a.status, KVC_ERR_DATA);
      break;
    }
    long dst;
    if (a.slots) {
      const long slot = a.slots[src_tok];
      if (slot < 0 || slot >= (long)a.N * a.bs) {
        if (idx == 0) report(a.status, KVC_ERR_DATA);
        continue;
      }
      dst = (((slot / a.bs) * a.Hkv + g) * a.bs + slot % a.bs) * a.head_bytes + w * 16;
    } else {
      dst = (((long)b * a.Hkv + g) * a.S_max + len + t) * a.head_bytes + w * 16;
    }
    copy_piece(a, src_tok, g, w, dst);
  }
}

// FP8 cache: the same grid over bf16 input rows.  The D/8 lanes holding one
// row (aligned groups of 8 or 16 lanes, all active together) reduce the row's
// largest magnitude with shuffles; the row's scale is that maximum over the
// format's largest value and every element is stored as the code of x / s.
template <int F>
__device__ __forceinline__ uint2 quantize8(const uint4& x, float s) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  uint32_t c[2] = {0u, 0u};
  if (s != 0.f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = fp8_encode<F>(__fdiv_rn(bf16_lo(w[i]), s));
      const uint32_t hi = fp8_encode<F>(__fdiv_rn(bf16_hi(w[i]), s));
      c[i >> 1] |= (lo | (hi << 8)) << (16 * (i & 1));
    }
  }
  return make_uint2(c[0], c[1]);
}

__device__ __forceinline__ float amax8(const uint4& x) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaxf(fabsf(bf16_lo(w[i])), fabsf(bf16_hi(w[i]))));
  return m;
}

// Piece w of new token src_tok's bf16 row of KV head g, K and V, quantized
// into cache row `row`: the row's D/8 lanes (aligned, all active together)
// reduce its largest magnitude, and the lane of piece 0 stores the scales.
template <int F>
__device__ __forceinline__ void quantize_store(const AppendArgs& a, const uint4& kx, const uint4& vx,
                                               int w, int vec_per_head, long row) {
  using Fm = Fp8Format<F>;
  float km = amax8(kx), vm = amax8(vx);
  for (int off = 1; off < vec_per_head; off <<= 1) {
    km = fmaxf(km, __shfl_xor(km, off));
    vm = fmaxf(vm, __shfl_xor(vm, off));
  }
  const float ks = __fdiv_rn(km, Fm::kMax), vs = __fdiv_rn(vm, Fm::kMax);
  const long dst = fp8_code_offset(row, a.D) + w * 8;
  *reinterpret_cast<uint2*>(a.k_cache + dst) = quantize8<F>(kx, ks);
  *reinterpret_cast<uint2*>(a.v_cache + dst) = quantize8<F>(vx, vs);
  if (w == 0) {
    const long so = fp8_scale_offset(row, a.D);
    *reinterpret_cast<float*>(a.k_cache + so) = ks;
    *reinterpret_cast<float*>(a.v_cache + so) = vs;
  }
}
template <int F>
__device__ __forceinline__ void quantize_piece(const AppendArgs& a, long src_tok, int g, int w,
                                               int vec_per_head, long row) {
  const long src = (src_tok * a.Hkv + g) * a.head_bytes + w * 16;
  const uint4 kx = *reinterpret_cast<const uint4*>(a.k_new + src);
  const uint4 vx = *reinterpret_cast<const uint4*>(a.v_new + src);
  quantize_store<F>(a, kx, vx, w, vec_per_head, row);
}

template <int F>
__global__ __launch_bounds__(kAppendThreads) void append_fp8_kernel(AppendArgs a) {
  const int b = blockIdx.y;
  const int vec_per_head = a.head_bytes >> 4;  // lanes per row: D / 8
  const int vec_per_tok = a.Hkv * vec_per_head;
  const int n_vchunks = (vec_per_tok + kAppendThreads - 1) / kAppendThreads;
  const int vchunk = blockIdx.x % n_vchunks;
  const int tchunk = blockIdx.x / n_vchunks;
  const int tok_per_wg = a.tok_per_wg;
  const int len = a.seq_lens[b];
  const int c0 = a.cu_new[b];
  const int n = a.cu_new[b + 1] - c0;
  const bool bad = len < 0 || n < 0 || (a.slots == nullptr && (long)len + n > a.S_max);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    a.seq_lens_out[b] = bad ? len : len + n;
    if (bad) report(a.status, (len < 0 || n < 0) ? KVC_ERR_DATA : KVC_ERR_CAPACITY);
    else if (n > (long)(gridDim.x / n_vchunks) * tok_per_wg) report(a.status, KVC_ERR_DATA);
  }
  if (bad) return;
  const int idx = vchunk * kAppendThreads + threadIdx.x;
  if (idx >= vec_per_tok) return;  // whole rows: vec_per_tok is a multiple of the row's lanes
  const int g = idx / vec_per_head;
  const int w = idx - g * vec_per_head;
  const long s_row = fp8_padded_rows(a.S_max);  // contiguous: rows per (sequence, head)
  const int t0 = tchunk * tok_per_wg;
  const int t1 = min(t0 + tok_per_wg, n);
  for (int t = t0; t < t1; ++t) {  // every lane of a row takes the same branches
    const long src_tok = (long)c0 + t;
    if (src_tok < 0 || src_tok >= a.total_new) {
      report(a.status, KVC_ERR_DATA);
      break;
    }
    long row;  // cache row of (token, head)
    if (a.slots) {
      const long slot = a.slots[src_tok];
      if (slot < 0 || slot >= (long)a.N * a.bs) {
        if (idx == 0) report(a.status, KVC_ERR_DATA);
        continue;
      }
      row = ((slot / a.bs) * a.Hkv + g) * a.bs + slot % a.bs;
    } else {
      row = ((long)b * a.Hkv + g) * s_row + len + t;
    }
    quantize_piece<F>(a, src_tok, g, w, vec_per_head, row);
  }
}

// Block table and append in one launch (paged caches).  Grid = (16-byte
// chunks of a token's rows x token chunks, B), as for the append.  Every
// workgroup first reads the whole batch's lengths and counts (one pass, its
// threads strided over the sequences) to find the blocks each sequence needs,
// the batch's errors and the free-list index of its own sequence's first new
// block; then the first workgroup of sequence b writes b's new table entries
// and length, and every workgroup maps its tokens to slots (an already held
// block from the table, a new one straight from the free list, so no
// workgroup waits on another's stores) and copies or quantizes their rows.
// The results equal those of block_table_kernel followed by the append
// kernels.  Errors of the allocation (a negative length or count, a sequence
// beyond its capacity, too few free blocks) are all or nothing, as in the
// block table: nothing is written but the head, the unchanged lengths and the
// status.
// Sum over the 64 lanes, the same value in every lane: DPP steps within each
// 16-lane row, then gfx950's permlane swaps across rows (each returns, per
// lane, itself and its partner across the swap); no step goes through LDS.
__device__ __forceinline__ int wave_sum_int(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, kDppQuadXor1, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, kDppQuadXor2, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, kDppRowHalfMirror, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, kDppRowMirror, 0xF, 0xF, true);
  const auto c = __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false);
  x = (int)(c[0] + c[1]);
  const auto d = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
  return (int)(d[0] + d[1]);
}

constexpr int kMaxTokPerWg = 4;  // tokens a workgroup of the append grids moves (launchers: 1 or 4)

template <int F>
__global__ __launch_bounds__(kAppendThreads) void block_table_append_kernel(BlockTableArgs bt,
                                                                           AppendArgs a) {
  __shared__ int s_red[kAppendThreads / kWave][3];
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int bs = bt.bs;
  // Nothing about this workgroup's own sequence depends on the batch scan,
  // so its loads go out first and their round trips overlap the scan's: the
  // sequence's length and new-row offsets, then (where those are usable) its
  // tokens' source pieces and the blocks it already holds.
  const int len = bt.seq_lens[b];
  const int c0 = bt.cu_new[b];
  const int n = bt.cu_new[b + 1] - c0;
  const int head = *bt.head_in;
  int total = 0, before = 0, bad = 0, over = 0;
  for (int i = tid; i < bt.B; i += kAppendThreads) {
    const int li = bt.seq_lens[i];
    const int ni = bt.cu_new[i + 1] - bt.cu_new[i];
    if (li < 0 || ni < 0) {
      bad = 1;
      continue;
    }
    const long have = ((long)li + bs - 1) / bs;
    const long want = ((long)li + ni + bs - 1) / bs;
    if (want > bt.max_blocks) {
      over = 1;
      continue;
    }
    total += (int)(want - have);
    if (i < b) before += (int)(want - have);
  }
  const int vec_per_head = a.head_bytes >> 4;
  const int vec_per_tok = a.Hkv * vec_per_head;
  const int n_vchunks = (vec_per_tok + kAppendThreads - 1) / kAppendThreads;
  const int vchunk = blockIdx.x % n_vchunks;
  const int tchunk = blockIdx.x / n_vchunks;
  const int idx = vchunk * kAppendThreads + tid;
  const int g = idx / vec_per_head;
  const int w = idx - g * vec_per_head;
  const int t0 = tchunk * a.tok_per_wg;
  const bool rows_ok = len >= 0 && n >= 0 && c0 >= 0 && (long)c0 + n <= bt.total_new;
  const int t1 = rows_ok ? min(t0 + a.tok_per_wg, n) : t0;  // tokens whose rows exist
  const int have = len >= 0 ? (int)min(((long)len + bs - 1) / bs, (long)bt.max_blocks) : 0;
  int32_t* row = bt.table + (long)b * bt.max_blocks;
  uint4 kx[kMaxTokPerWg], vx[kMaxTokPerWg];
  int held[kMaxTokPerWg];  // the block of a token that lands in a block the sequence holds
#pragma unroll
  for (int u = 0; u < kMaxTokPerWg; ++u) {
    const int t = t0 + u;
    kx[u] = vx[u] = make_uint4(0, 0, 0, 0);
    held[u] = -1;
    if (u >= a.tok_per_wg || t >= t1) continue;
    if (idx < vec_per_tok) {
      const long src = ((long)(c0 + t) * a.Hkv + g) * a.head_bytes + w * 16;
      kx[u] = *reinterpret_cast<const uint4*>(a.k_new + src);
      if (a.v_cache) vx[u] = *reinterpret_cast<const uint4*>(a.v_new + src);
    }
    const long lb = ((long)len + t) / bs;
    if (lb < have) held[u] = row[lb];
  }
  total = wave_sum_int(total);
  before = wave_sum_int(before);
  bad = __any(bad) ? 1 : 0;
  over = __any(over) ? 1 : 0;
  if ((tid & (kWave - 1)) == 0) {
    s_red[tid / kWave][0] = total;
    s_red[tid / kWave][1] = before;
    s_red[tid / kWave][2] = bad | (over << 1);
  }
  __syncthreads();
  total = before = 0;
  int flags = 0;
#pragma unroll
  for (int k = 0; k < kAppendThreads / kWave; ++k) {
    total += s_red[k][0];
    before += s_red[k][1];
    flags |= s_red[k][2];
  }
  int err = 0;
  if (flags & 1) err = KVC_ERR_DATA;
  else if (flags & 2) err = KVC_ERR_CAPACITY;
  else if (head < 0 || (long)head + total > bt.N) err = KVC_ERR_NO_BLOCKS;
  if (err != 0) {
    if (blockIdx.x == 0 && tid == 0) {
      a.seq_lens_out[b] = len;
      if (b == 0) {
        report(bt.status, err);
        *bt.head_out = head;
      }
    }
    return;
  }
  const int need = (int)(((long)len + n + bs - 1) / bs) - have;
  const int first = head + before;
  if (blockIdx.x == 0) {
    for (int j = tid; j < need; j += kAppendThreads) row[have + j] = bt.free_list[first + j];
    if (tid == 0) {
      a.seq_lens_out[b] = len + n;
      if (b == 0) *bt.head_out = head + total;
    }
  }
  if (n > 0 && !rows_ok) {  // cu_new points outside the new-row buffers
    if (blockIdx.x == 0 && tid == 0) report(bt.status, KVC_ERR_DATA);
    return;
  }
  if (blockIdx.x == 0 && tid == 0 && n > (long)(gridDim.x / n_vchunks) * a.tok_per_wg)
    report(bt.status, KVC_ERR_DATA);  // more new tokens than max_new promised
#pragma unroll
  for (int u = 0; u < kMaxTokPerWg; ++u) {
    const int t = t0 + u;
    if (u >= a.tok_per_wg || t >= t1) break;
    const int pos = len + t;
    const int lb = pos / bs;
    const long blk = lb < have ? held[u] : bt.free_list[first + lb - have];
    const long slot = blk * bs + pos % bs;
    if (vchunk == 0 && tid == 0) bt.slots[c0 + t] = (int32_t)slot;
    if (slot < 0 || slot >= (long)bt.N * bs) {
      if (idx == 0) report(bt.status, KVC_ERR_DATA);
      continue;
    }
    if (idx >= vec_per_tok) continue;
    const long prow = ((slot / bs) * a.Hkv + g) * bs + slot % bs;  // cache row of (token, head)
    if constexpr (F == 0) {
      const long dst = prow * a.head_bytes + w * 16;
      *reinterpret_cast<uint4*>(a.k_cache + dst) = kx[u];
      if (a.v_cache) *reinterpret_cast<uint4*>(a.v_cache + dst) = vx[u];
    } else {
      quantize_store<F>(a, kx[u], vx[u], w, vec_per_head, prow);
    }
  }
}

hipError_t launch_block_table_append(const BlockTableArgs& bt, const AppendArgs& a,
                                     hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  const int vec_per_tok = a.Hkv * (a.head_bytes >> 4);
  const long n_vchunks = (vec_per_tok + kAppendThreads - 1) / kAppendThreads;
  AppendArgs b = a;
  b.tok_per_wg = a.max_new <= 64 ? 1 : 4;
  const long n_tchunks = a.max_new > 0 ? (a.max_new + b.tok_per_wg - 1) / b.tok_per_wg : 1;
  if (n_vchunks * n_tchunks > 0x7fffffffL) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)(n_vchunks * n_tchunks), a.B), block(kAppendThreads);
  if (a.fp8 == kFp8E4M3)
    hipLaunchKernelGGL(block_table_append_kernel<kFp8E4M3>, grid, block, 0, s, bt, b);
  else if (a.fp8 == kFp8E5M2)
    hipLaunchKernelGGL(block_table_append_kernel<kFp8E5M2>, grid, block, 0, s, bt, b);
  else
    hipLaunchKernelGGL(block_table_append_kernel<0>, grid, block, 0, s, bt, b);
  return hipGetLastError();
}

hipError_t launch_block_table(const BlockTableArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(block_table_kernel, dim3(1), dim3(kBtThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  const int vec_per_tok = a.Hkv * (a.head_bytes >> 4);
  const long n_vchunks = (vec_per_tok + kAppendThreads - 1) / kAppendThreads;
  // decode-sized steps: one token per workgroup; prefills: four per workgroup
  AppendArgs b = a;
  b.tok_per_wg = a.max_new <= 64 ? 1 : 4;
  const long n_tchunks = a.max_new > 0 ? (a.max_new + b.tok_per_wg - 1) / b.tok_per_wg : 1;
  if (n_vchunks * n_tchunks > 0x7fffffffL) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)(n_vchunks * n_tchunks), a.B);
  if (a.fp8 == kFp8E4M3) hipLaunchKernelGGL(append_fp8_kernel<kFp8E4M3>, grid, dim3(kAppendThreads), 0, s, b);
  else if (a.fp8 == kFp8E5M2) hipLaunchKernelGGL(append_fp8_kernel<kFp8E5M2>, grid, dim3(kAppendThreads), 0, s, b);
  else hipLaunchKernelGGL(append_kernel, grid, dim3(kAppendThreads), 0, s, b);
  return hipGetLastError();
}

}  // namespace kvc
