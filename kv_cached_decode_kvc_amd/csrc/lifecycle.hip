// lifecycle.hip -- sharing, copy-on-write and rollback of paged KV blocks.
//
// "Inference o quy mo lon" (truongducdung.dev), 05 "Chia se block va
// copy-on-write": physical blocks carry reference counts, parallel samples
// share the prompt's blocks, and a sample that must write into a shared block
// copies it first.  "Inference-1" (brunomaga.github.io), "PagedAttention":
// shared blocks are copied only when written.  "Efficient Inference"
// (learn.obvix.io), paged passage: a finished request's blocks return to the
// free pool.  "Inference-2", "Draft-model speculative decoding": after
// verification the target's cache is cut back to the accepted tokens.
//
// ref_counts[blk] holds the owners beyond the first (0 for a free block or a
// single owner).  The free pool is free_list[head .. N); freed blocks are
// pushed back just below head in increasing block id.  Releases decrement the
// count atomically; the one release that takes it from 0 to -1 marks the block
// in an LDS bitmap, and a scan of the bitmap gives every freed block its place
// -- the result does not depend on the order in which threads run.
#include "launch.hpp"

namespace kvc {

constexpr int kLcThreads = 1024;
constexpr int kLcWaves = kLcThreads / kWave;

__device__ __forceinline__ int lc_block_scan(int x, int* s_wave, int& total) {
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
  for (int w = 0; w < kLcWaves; ++w) {
    const int v = s_wave[w];
    before += w < wave ? v : 0;
    total += v;
  }
  __syncthreads();
  return x + before;  // inclusive
}

// Push every block marked in the bitmap (words [0, nwords)) onto the free list
// just below `head`, in increasing id; returns the new head.  Clears refs of
// the pushed blocks.  Caller: all threads of the workgroup.
__device__ int push_marked(const uint32_t* bits, int nwords, int32_t* free_list, int head,
                           int32_t* refs, int* s_wave, int32_t* status) {
  // each thread owns a contiguous run of words so ranks follow block ids
  const int per = (nwords + kLcThreads - 1) / kLcThreads;
  const int w0 = min(threadIdx.x * per, nwords);
  const int w1 = min(w0 + per, nwords);
  int cnt = 0;
  for (int w = w0; w < w1; ++w) cnt += __popc(bits[w]);
  int total;
  int rank = lc_block_scan(cnt, s_wave, total) - cnt;
  const int new_head = head - total;
  if (new_head < 0) {  // more freed blocks than were ever taken: inconsistent data
    if (threadIdx.x == 0) report(status, KVC_ERR_DATA);
    return head;
  }
  for (int w = w0; w < w1; ++w) {
    uint32_t m = bits[w];
    while (m) {
      const int bit = __ffs(m) - 1;
      m &= m - 1;
      const int blk = w * 32 + bit;
      free_list[new_head + rank++] = blk;
      if (refs) refs[blk] = 0;
    }
  }
  return new_head;
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kLcThreads) void fork_kernel(LifecycleArgs a) {
  __shared__ uint32_t s_child[kMaxBatch / 32];
  __shared__ int s_err;
  const int tid = threadIdx.x;
  for (int w = tid; w < (a.B + 31) / 32; w += kLcThreads) s_child[w] = 0;
  if (tid == 0) s_err = 0;
  __syncthreads();
  const long cap = (long)a.max_blocks * a.bs;
  for (int i = tid; i < a.n; i += kLcThreads) {
    const int p = a.parents[i], c = a.children[i];
    if (p < 0 || p >= a.B || c < 0 || c >= a.B || p == c) {
      atomicMin(&s_err, KVC_ERR_DATA);
      continue;
    }
    const int lp = a.seq_lens[p];
    if (a.seq_lens[c] != 0 || lp < 0 || lp > cap) atomicMin(&s_err, KVC_ERR_DATA);
    if (atomicOr(&s_child[c >> 5], 1u << (c & 31)) & (1u << (c & 31)))  // repeated child
      atomicMin(&s_err, KVC_ERR_DATA);
  }
  __syncthreads();
  for (int i = tid; i < a.n; i += kLcThreads) {  // a parent that is also a child
    const int p = a.parents[i];
    if (p >= 0 && p < a.B && (s_child[p >> 5] & (1u << (p & 31)))) atomicMin(&s_err, KVC_ERR_DATA);
  }
  __syncthreads();
  if (s_err != 0) {
    if (tid == 0) report(a.status, s_err);
    return;
  }
  // one wavefront per fork, its lanes over the table row
  const int wave = tid / kWave, lane = tid & (kWave - 1);
  for (int i = wave; i < a.n; i += kLcWaves) {
    const int p = a.parents[i], c = a.children[i];
    const int lp = a.seq_lens[p];
    const int nb = (lp + a.bs - 1) / a.bs;
    const int32_t* src = a.table + (long)p * a.max_blocks;
    int32_t* dst = a.table + (long)c * a.max_blocks;
    for (int j = lane; j < nb; j += kWave) {
      const int blk = src[j];
      dst[j] = blk;
      if (blk >= 0 && blk < a.N) atomicAdd(&a.refs[blk], 1);
    }
    if (lane == 0) a.seq_lens_out[c] = lp;  // seq_lens_out == seq_lens: children only
  }
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kLcThreads) void truncate_kernel(LifecycleArgs a) {
  __shared__ uint32_t s_bits[kMaxPoolBlocks / 32];
  __shared__ int s_wave[kLcWaves];
  __shared__ int s_err;
  const int tid = threadIdx.x;
  const int head = *a.head_in;
  const int nwords = (a.N + 31) / 32;
  for (int w = tid; w < nwords; w += kLcThreads) s_bits[w] = 0;
  if (tid == 0) s_err = 0;
  __syncthreads();
  const long cap = (long)a.max_blocks * a.bs;
  for (int b = tid; b < a.B; b += kLcThreads) {
    const int len = a.seq_lens[b], nl = a.new_lens[b];
    if (nl < 0 || nl > len || len > cap) atomicMin(&s_err, KVC_ERR_DATA);
  }
  if (tid == 0 && (head < 0 || head > a.N)) atomicMin(&s_err, KVC_ERR_DATA);
  __syncthreads();
  if (s_err != 0) {
    if (tid == 0) {
      report(a.status, s_err);
      *a.head_out = head;
    }
    return;
  }
  // one wavefront per sequence, its lanes over the released blocks
  const int wave = tid / kWave, lane = tid & (kWave - 1);
  for (int b = wave; b < a.B; b += kLcWaves) {
    const int len = a.seq_lens[b], nl = a.new_lens[b];
    const int old_nb = min((len + a.bs - 1) / a.bs, a.max_blocks);
    const int new_nb = (nl + a.bs - 1) / a.bs;
    int32_t* row = a.table + (long)b * a.max_blocks;
    for (int j = new_nb + lane; j < old_nb; j += kWave) {
      const int blk = row[j];
      row[j] = -1;
      if (blk < 0 || blk >= a.N) continue;
      const bool freed = a.refs ? atomicSub(&a.refs[blk], 1) == 0 : true;
      if (freed) atomicOr(&s_bits[blk >> 5], 1u << (blk & 31));
    }
    if (lane == 0) a.seq_lens_out[b] = nl;
  }
  __syncthreads();
  const int new_head = push_marked(s_bits, nwords, a.free_list, head, a.refs, s_wave, a.status);
  if (tid == 0) *a.head_out = new_head;
}

// ---------------------------------------------------------------------------
// Copy-on-write, decided on the state at the start of the call: a sequence
// about to append into a partly filled last block that has extra owners takes
// a fresh block from the free-list front (batch order), points its table at it
// and drops one reference on the original; originals left with no owner are
// freed.  The block contents are copied afterwards by copy_blocks_kernel.
__global__ __launch_bounds__(kLcThreads) void cow_kernel(LifecycleArgs a) {
  __shared__ uint32_t s_bits[kMaxPoolBlocks / 32];
  __shared__ int s_wave[kLcWaves];
  const int tid = threadIdx.x;
  const int head = *a.head_in;
  const int nwords = (a.N + 31) / 32;
  for (int w = tid; w < nwords; w += kLcThreads) s_bits[w] = 0;
  __syncthreads();
  // pass 1: count the copies (reads of refs only)
  int count = 0;
  for (int b = tid; b < a.B; b += kLcThreads) {
    const int len = a.seq_lens[b], n = a.cu_new[b + 1] - a.cu_new[b];
    a.cow_src[b] = -1;
    a.cow_dst[b] = -1;
    if (n <= 0 || len <= 0 || len % a.bs == 0 || len / a.bs >= a.max_blocks) continue;
    const int blk = a.table[(long)b * a.max_blocks + len / a.bs];
    if (blk >= 0 && blk < a.N && a.refs[blk] > 0) ++count;
  }
  int total;
  lc_block_scan(count, s_wave, total);
  if (head < 0 || (long)head + total > a.N) {
    if (tid == 0) {
      report(a.status, KVC_ERR_NO_BLOCKS);
      *a.head_out = head;
    }
    return;
  }
  // pass 2: batch-order assignment (chunks of kLcThreads sequences); refs are
  // still only read, so every decision sees the state at the start of the call
  int carry = 0;
  for (int base = 0; base < a.B; base += kLcThreads) {
    const int b = base + tid;
    int blk = -1, is_cow = 0;
    if (b < a.B) {
      const int len = a.seq_lens[b], n = a.cu_new[b + 1] - a.cu_new[b];
      if (n > 0 && len > 0 && len % a.bs != 0 && len / a.bs < a.max_blocks) {
        blk = a.table[(long)b * a.max_blocks + len / a.bs];
        is_cow = blk >= 0 && blk < a.N && a.refs[blk] > 0;
      }
    }
    int chunk_total;
    const int pos = head + carry + lc_block_scan(is_cow, s_wave, chunk_total) - is_cow;
    carry += chunk_total;
    if (is_cow) {
      const int len = a.seq_lens[b];
      const int fresh = a.free_list[pos];
      a.table[(long)b * a.max_blocks + len / a.bs] = fresh;
      a.cow_src[b] = blk;
      a.cow_dst[b] = fresh;
    }
  }
  __syncthreads();
  // pass 3: every copy drops one reference on its original (own entries only)
  for (int b = tid; b < a.B; b += kLcThreads) {
    const int blk = a.cow_src[b];
    if (blk >= 0 && atomicSub(&a.refs[blk], 1) == 0) atomicOr(&s_bits[blk >> 5], 1u << (blk & 31));
  }
  __syncthreads();
  const int new_head = push_marked(s_bits, nwords, a.free_list, head + total, a.refs, s_wave,
                                   a.status);
  if (tid == 0) *a.head_out = new_head;
}

// ---------------------------------------------------------------------------
// grid = (chunks of one block, pairs): every thread copies 16 bytes of K and V.
constexpr int kCopyThreads = 256;
__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(CopyArgs a) {
  const int i = blockIdx.y;
  const int src = a.src[i], dst = a.dst[i];
  if (src < 0 || dst < 0) return;  // no copy for this entry
  if (src >= a.N || dst >= a.N) {
    if (blockIdx.x == 0 && threadIdx.x == 0) report(a.status, KVC_ERR_DATA);
    return;
  }
  const long off = ((long)blockIdx.x * kCopyThreads + threadIdx.x) * 16;
  if (off >= a.block_bytes) return;
  const uint4 kv = *reinterpret_cast<const uint4*>(a.k + (long)src * a.block_bytes + off);
  *reinterpret_cast<uint4*>(a.k + (long)dst * a.block_bytes + off) = kv;
  if (a.v) {  // NULL: a key-only (MLA latent) pool
    const uint4 vv = *reinterpret_cast<const uint4*>(a.v + (long)src * a.block_bytes + off);
    *reinterpret_cast<uint4*>(a.v + (long)dst * a.block_bytes + off) = vv;
  }
}

hipError_t launch_fork(const LifecycleArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(fork_kernel, dim3(1), dim3(kLcThreads), 0, s, a);
  return hipGetLastError();
}
hipError_t launch_truncate(const LifecycleArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(truncate_kernel, dim3(1), dim3(kLcThreads), 0, s, a);
  return hipGetLastError();
}
hipError_t launch_cow(const LifecycleArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(cow_kernel, dim3(1), dim3(kLcThreads), 0, s, a);
  return hipGetLastError();
}
hipError_t launch_copy_blocks(const CopyArgs& a, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const long chunks = (a.block_bytes / 16 + kCopyThreads - 1) / kCopyThreads;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)chunks, n), dim3(kCopyThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvc
