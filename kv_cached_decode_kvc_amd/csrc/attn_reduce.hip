// attn_reduce.hip -- the cross-partition combine of split-KV attention.
//
// "Inference-1" (brunomaga.github.io), section "FlashDecoding": every chunk of
// keys leaves a partial output with its softmax maximum and sum, and a final
// reduction combines them with the online-softmax rescaling (section
// "FlashAttention": factor exp(m_p - m*)).  With maxima kept in the base-2
// domain: m* = max_p m_p, w_p = 2^(m_p - m*) (0 for an empty partition),
// out = sum_p w_p O_p / sum_p w_p l_p, then one rounding to the output type.
//
// One wavefront per output row (sequence, query head, query row), two for a
// 512-wide row (each takes half the columns and works out the row's
// statistics itself, identically); each lane owns consecutive columns and,
// for the statistics, one partition.  The
// partials are either a row's fixed partitions or, for the matrix-core
// kernel's stream-K split, the pieces of the workers that covered the row's
// segment.
#include "launch.hpp"

namespace kvc {

namespace {

// Sum and maximum over the 64 lanes, the same bits in every lane: DPP steps
// within each 16-lane row, then gfx950's permlane swaps across rows (each
// returns, per lane, itself and its partner across the swap), every step
// combining a pair of values commutatively.  No step goes through LDS.
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp<kDppQuadXor1>(x);
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppRowHalfMirror>(x);
  x += dpp<kDppRowMirror>(x);
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(c[0]) + __uint_as_float(c[1]);
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<kDppQuadXor1>(x));
  x = fmaxf(x, dpp<kDppQuadXor2>(x));
  x = fmaxf(x, dpp<kDppRowHalfMirror>(x));
  x = fmaxf(x, dpp<kDppRowMirror>(x));
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
}
// lane j's value in every lane (j uniform): a scalar read, no LDS round trip
__device__ __forceinline__ float lane_value(float x, int j) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), j));
}

}  // namespace

template <int D, bool BF16_OUT>
__global__ __launch_bounds__(64) void reduce_kernel(ReduceParams p) {
  constexpr int HALVES = D > 256 ? 2 : 1;  // wavefronts per row
  constexpr int DW = D / HALVES;           // columns of one wavefront
  constexpr int CPL = DW / kWave;          // columns per lane
  const long row = blockIdx.x / HALVES;    // (b * Hq + h) * n_q + r
  const int col0 = (int)(blockIdx.x % HALVES) * DW + (int)threadIdx.x * CPL;  // this lane's first column
  const int lane = threadIdx.x;
  const int r = (int)(row % p.n_q);
  const long bh = row / p.n_q;
  const int h = (int)(bh % p.Hq);
  const int b = (int)(bh / p.Hq);
  const long ooff = (((long)b * p.n_q + r) * p.Hq + h) * D + col0;

  // Where this row's partials are: partial j's statistics at ml[j * ml_step]
  // and its outputs at po[j * o_step] (this lane's columns).  Fixed
  // partitions: the row's max_parts slots, in order.  Stream-K: the pieces
  // (segment + worker) of the workers sk_meta names for the row's segment.
  constexpr int kEarly = DW <= 128 ? 16 : 8;  // registers: kEarly * DW / 64
  const float2* ml;
  const float* po;
  long ml_step, o_step;
  float early[kEarly][CPL];
  float2 mine_raw = make_float2(-INFINITY, 0.f);
  // stream-K: the segment's worker record, requested with the length (its
  // address does not depend on it), so the partials wait one round trip
  const int g_sk = p.sk_meta ? h / p.G : 0;
  const int i_sk = p.sk_meta ? r * p.G + h % p.G : 0;  // row of the KV head's rows
  const long seg_sk = p.sk_meta ? ((long)b * p.Hkv + g_sk) *
                                      ((p.G * p.n_q + p.rows_item - 1) / p.rows_item) +
                                      i_sk / p.rows_item
                                : 0;
  int2 wr_raw = make_int2(0, -1);
  if (p.sk_meta) wr_raw = p.sk_meta[seg_sk];
  int code;
  const int L = attended_len(p.seq_lens, p.cu_new, p.total_new, b, p.n_q, p.cap, &code);
  const bool valid = L >= 0;
  int n = 0;  // partials of the row
  if (p.sk_meta == nullptr) {
    ml = reinterpret_cast<const float2*>(p.ws_ml) + row * p.max_parts;
    po = p.ws_o + row * p.max_parts * D + col0;
    ml_step = 1;
    o_step = D;
    // With few partition slots, one round trip: the length, the first kEarly
    // partitions' outputs for this lane's columns and one partition's (m, l)
    // per lane are all requested together, for every slot the workspace has
    // (slots beyond the sequence's partitions hold stale bytes and are
    // discarded by selection, never multiplied, once the length is known).
    // With more slots than that, fetching every slot's outputs would move
    // several times the bytes the sequence has, so the outputs wait for the
    // length (a second round trip) and only its partitions are read.  The
    // wide rows (1 KiB of outputs per slot and wavefront) speculate over at
    // most four slots: reading all of seven measured slower than the second
    // round trip.
    const bool speculate = p.max_parts <= (DW > 128 ? 4 : kEarly > 8 ? 8 : kEarly);
    if (speculate) {
#pragma unroll
      for (int j = 0; j < kEarly; ++j)
#pragma unroll
        for (int c = 0; c < CPL; ++c) early[j][c] = j < p.max_parts ? po[(long)j * D + c] : 0.f;
    }
    if (lane < p.max_parts) mine_raw = ml[lane];
    const int P = part_tokens(p.seq_lens, p.B, p.cap, p.slots_u, p.P_lo, p.P);
    n = valid ? (L + P - 1) / P : 0;
    if (!speculate) {
#pragma unroll
      for (int j = 0; j < kEarly; ++j)
#pragma unroll
        for (int c = 0; c < CPL; ++c) early[j][c] = j < n ? po[(long)j * D + c] : 0.f;
    }
  } else {
    int2 wr = valid ? wr_raw : make_int2(0, -1);
    // a record that names workers outside the launch (a workspace the
    // partition kernel did not fill) is not followed
    if (wr.x < 0 || wr.y < wr.x || wr.y >= p.sk_workers) wr = make_int2(0, -1);
    n = valid ? wr.y - wr.x + 1 : 0;
    const long first = (seg_sk + wr.x) * p.sk_rows + i_sk % p.rows_item;  // workspace row of piece 0
    ml = reinterpret_cast<const float2*>(p.ws_ml) + first;
    po = p.ws_o + first * D + col0;
    ml_step = p.sk_rows;
    o_step = (long)p.sk_rows * D;
    if (lane < n) mine_raw = ml[lane * ml_step];
#pragma unroll
    for (int j = 0; j < kEarly; ++j)
#pragma unroll
      for (int c = 0; c < CPL; ++c) early[j][c] = j < n ? po[j * o_step + c] : 0.f;
  }
  float acc[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) acc[j] = 0.f;
  float den = 0.f;
  if (valid) {
    const int nparts = n;
#pragma unroll
    for (int j = 0; j < kEarly; ++j)
#pragma unroll
      for (int c = 0; c < CPL; ++c) early[j][c] = j < nparts ? early[j][c] : 0.f;
    const float2 mine = lane < nparts ? mine_raw : make_float2(-INFINITY, 0.f);
    float mstar = mine.x;
    for (int q0 = kWave; q0 < nparts; q0 += kWave)  // more than 64 partitions
      if (q0 + lane < nparts) mstar = fmaxf(mstar, ml[(q0 + lane) * ml_step].x);
    mstar = wave_max(mstar);
    for (int q0 = 0; q0 < nparts; q0 += kWave) {
      float2 mq = q0 == 0 ? mine : make_float2(-INFINITY, 0.f);
      if (q0 > 0 && q0 + lane < nparts) mq = ml[(q0 + lane) * ml_step];
      const float wq = mq.x == -INFINITY ? 0.f : fast_exp2(mq.x - mstar);  // empty: 0
      den += wq * mq.y;
      const int cnt = min(kWave, nparts - q0);
      int j = 0;
      if (q0 == 0) {
#pragma unroll
        for (int u = 0; u < kEarly; ++u) {
          const float wj = lane_value(wq, u);  // 0 beyond nparts: those lanes hold weight 0
#pragma unroll
          for (int c = 0; c < CPL; ++c) acc[c] += wj * early[u][c];
        }
        j = kEarly;
      }
      for (; j + 8 <= cnt; j += 8) {  // eight partitions' loads in flight at once
        float o[8][CPL];
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
          for (int c = 0; c < CPL; ++c) o[u][c] = po[(q0 + j + u) * o_step + c];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float wj = lane_value(wq, j + u);
#pragma unroll
          for (int c = 0; c < CPL; ++c) acc[c] += wj * o[u][c];
        }
      }
      if (j < cnt) {  // the last 1 .. 7 partitions: their loads in flight together
        float o[8][CPL];
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
          for (int c = 0; c < CPL; ++c) o[u][c] = j + u < cnt ? po[(q0 + j + u) * o_step + c] : 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (j + u >= cnt) break;
          const float wj = lane_value(wq, j + u);
#pragma unroll
          for (int c = 0; c < CPL; ++c) acc[c] += wj * o[u][c];
        }
      }
    }
    den = wave_sum(den);
  }
  if (!valid && lane == 0 && h == 0 && r == 0) report(p.status, code);
  if (valid && n == 0 && lane == 0) report(p.status, KVC_ERR_DATA);
  const float inv = den > 0.f ? 1.f / den : 0.f;  // invalid data: zeros
  if constexpr (BF16_OUT) {
    uint16_t* out = (uint16_t*)p.out + ooff;
#pragma unroll
    for (int j = 0; j < CPL; ++j) out[j] = (uint16_t)f32_to_bf16_bits(acc[j] * inv);
  } else {
    float* out = (float*)p.out + ooff;
#pragma unroll
    for (int j = 0; j < CPL; ++j) out[j] = acc[j] * inv;
  }
}

hipError_t launch_reduce(const ReduceParams& p, int out_dtype, hipStream_t s) {
  const long rows = (long)p.B * p.Hq * p.n_q;
  if (rows == 0) return hipSuccess;
  const dim3 grid((unsigned)rows), block(kWave);
  const bool bf = out_dtype == KVC_BF16;
  if (p.D == 512) {  // MLA: weighted latents, two wavefronts per row
    const dim3 grid2((unsigned)(2 * rows));
    if (bf) hipLaunchKernelGGL((reduce_kernel<512, true>), grid2, block, 0, s, p);
    else hipLaunchKernelGGL((reduce_kernel<512, false>), grid2, block, 0, s, p);
  } else if (p.D == 128) {
    if (bf) hipLaunchKernelGGL((reduce_kernel<128, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((reduce_kernel<128, false>), grid, block, 0, s, p);
  } else {
    if (bf) hipLaunchKernelGGL((reduce_kernel<64, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((reduce_kernel<64, false>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace kvc
