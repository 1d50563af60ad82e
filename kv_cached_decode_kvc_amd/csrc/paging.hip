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

// One workgroup.  Pass 1 validates and counts the new blocks of every sequence;
// pass 2 assigns them in batch order with a chunked exclusive scan, consuming
// the free list front to back; pass 3 maps every new token to its slot.
__global__ __launch_bounds__(kBtThreads) void block_table_kernel(BlockTableArgs a) {
  __shared__ int s_scan[kBtThreads];
  __shared__ int s_cu[kBtThreads], s_len[kBtThreads];  // batches below kBtThreads
  __shared__ int s_err, s_head, s_total;
  const int tid = threadIdx.x;
  const int bs = a.bs;
  const bool staged = a.B < kBtThreads;  // B + 1 offsets need B + 1 threads
  if (tid == 0) {
    s_err = 0;
    s_head = *a.head_in;
    s_total = 0;
  }
  if (staged) {
    if (tid < a.B) s_len[tid] = a.seq_lens[tid];
    if (tid <= a.B) s_cu[tid] = a.cu_new[tid];
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
  if (tid == 0 && s_err == 0 && (s_head < 0 || (long)s_head + s_total > a.N))
    s_err = KVC_ERR_NO_BLOCKS;
  __syncthreads();
  if (s_err != 0) {
    if (tid == 0) {
      report(a.status, s_err);
      *a.head_out = s_head;
    }
    return;
  }

  int carry = 0;
  for (int base = 0; base < a.B; base += kBtThreads) {
    const int b = base + tid;
    int have = 0, need = 0;
    if (b < a.B) {
      const int len = a.seq_lens[b];
      const int n = a.cu_new[b + 1] - a.cu_new[b];
      have = (len + bs - 1) / bs;
      need = (int)(((long)len + n + bs - 1) / bs) - have;
    }
    s_scan[tid] = need;
    __syncthreads();
    for (int off = 1; off < kBtThreads; off <<= 1) {  // inclusive Hillis-Steele scan
      const int add = tid >= off ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += add;
      __syncthreads();
    }
    const int first = s_head + carry + s_scan[tid] - need;
    for (int i = 0; i < need; ++i)
      a.table[(long)b * a.max_blocks + have + i] = a.free_list[first + i];
    carry += s_scan[kBtThreads - 1];
    __syncthreads();
  }
  __syncthreads();  // table entries written above are read below by other threads

  const int* cu = staged ? s_cu : a.cu_new;  // the search runs in LDS when it fits
  const int* lens = staged ? s_len : a.seq_lens;
  for (int i = tid; i < a.total_new; i += kBtThreads) {
    int lo = 0, hi = a.B - 1;  // last b with cu_new[b] <= i
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (cu[mid] <= i) lo = mid;
      else hi = mid - 1;
    }
    const long pos = (long)lens[lo] + (i - cu[lo]);
    if (i >= cu[lo + 1] || pos / bs >= a.max_blocks) {  // cu_new disagrees with total_new
      a.slots[i] = -1;
      report(a.status, KVC_ERR_DATA);
      continue;
    }
    const long blk = a.table[(long)lo * a.max_blocks + pos / bs];
    a.slots[i] = (int32_t)(blk * bs + pos % bs);
  }
  if (tid == 0) *a.head_out = s_head + s_total;
}

constexpr int kAppendThreads = 256;

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
    if (src_tok >= a.total_new) {  // cu_new points past the new-row buffers
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
    const long src = (src_tok * a.Hkv + g) * a.head_bytes + w * 16;
    const uint4 kv = *reinterpret_cast<const uint4*>(a.k_new + src);
    const uint4 vv = *reinterpret_cast<const uint4*>(a.v_new + src);
    *reinterpret_cast<uint4*>(a.k_cache + dst) = kv;
    *reinterpret_cast<uint4*>(a.v_cache + dst) = vv;
  }
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
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)(n_vchunks * n_tchunks), a.B), dim3(kAppendThreads),
                     0, s, b);
  return hipGetLastError();
}

}  // namespace kvc
