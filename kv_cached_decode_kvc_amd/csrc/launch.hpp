// launch.hpp -- host-side launchers of the kvc kernels (internal to libkvc.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace kvc {

struct BlockTableArgs {
  const int32_t* seq_lens;
  const int32_t* cu_new;
  int32_t* table;
  const int32_t* free_list;
  const int32_t* head_in;
  int32_t* head_out;
  int32_t* slots;
  int32_t* status;
  int B, bs, max_blocks, N, total_new;
};

struct AppendArgs {
  const uint8_t* k_new;
  const uint8_t* v_new;
  const int32_t* seq_lens;
  const int32_t* cu_new;
  const int32_t* slots;  // NULL: contiguous
  uint8_t* k_cache;
  uint8_t* v_cache;
  int32_t* seq_lens_out;
  int32_t* status;
  int B, Hkv, head_bytes, bs, S_max, N, max_new, total_new;
  int tok_per_wg;  // set by the launcher
  int fp8;         // 0: rows copied bit for bit; kFp8E4M3 / kFp8E5M2: bf16 rows quantized
  int D;           // FP8: codes per row (16-row tiles of codes and scales, common.hpp)
};

constexpr int kMaxBatch = 65536;        // sequences per call (one grid row each)
constexpr int kMaxPoolBlocks = 262144;
constexpr int kMaxFusedBatch = 8192;  // kvc_block_table_append: every workgroup reads the batch  // pool size the lifecycle kernels can track in LDS

struct LifecycleArgs {
  const int32_t* seq_lens;
  const int32_t* new_lens;  // truncate
  const int32_t* cu_new;    // copy-on-write
  const int32_t* parents;   // fork
  const int32_t* children;
  int32_t* table;
  int32_t* free_list;
  const int32_t* head_in;
  int32_t* head_out;
  int32_t* refs;            // may be NULL for truncate
  int32_t* seq_lens_out;
  int32_t* cow_src;
  int32_t* cow_dst;
  int32_t* status;
  int B, bs, max_blocks, N, n;
};

struct CopyArgs {
  const int32_t* src;
  const int32_t* dst;
  uint8_t* k;
  uint8_t* v;
  long block_bytes;  // bytes of one pool block (all KV heads; FP8: codes and scales)
  int N;
  int32_t* status;
};

hipError_t launch_fork(const LifecycleArgs& a, hipStream_t s);
hipError_t launch_truncate(const LifecycleArgs& a, hipStream_t s);
hipError_t launch_cow(const LifecycleArgs& a, hipStream_t s);
hipError_t launch_copy_blocks(const CopyArgs& a, int n, hipStream_t s);
hipError_t launch_block_table(const BlockTableArgs& a, hipStream_t s);
hipError_t launch_append(const AppendArgs& a, hipStream_t s);
hipError_t launch_block_table_append(const BlockTableArgs& bt, const AppendArgs& a, hipStream_t s);
// dtype: KVC_BF16 / KVC_F32; D: 64 / 128; mfma selects the grouped-rows kernel (bf16 only)
constexpr int kMlaKeyDim = 576;    // MLA cache row: latent (512) + decoupled RoPE key (64)
constexpr int kMlaValueDim = 512;  // the latent part, which also serves as the value
// 16-key halves of one MLA piece of work whose block ids the kernel stages in
// LDS: a partition, or a stream-K worker's run in one sequence, of at most
// 16384 keys
constexpr int kMlaMaxTiles = 1024;

hipError_t launch_partition_valu(const AttnParams& p, int dtype, hipStream_t s);
hipError_t launch_partition_mla(const AttnParams& p, hipStream_t s);
// MLA: rows one workgroup covers, and workgroups resident per CU, for `rows` rows
int mla_rows_per_wg(int rows);
int mla_wgs_per_cu(int rows);
hipError_t launch_prefill(const PrefillParams& p, int out_dtype, hipStream_t s);
hipError_t launch_partition_mfma(const AttnParams& p, int rows_per_item, int fp8, hipStream_t s);
hipError_t launch_reduce(const ReduceParams& p, int out_dtype, hipStream_t s);

}  // namespace kvc
