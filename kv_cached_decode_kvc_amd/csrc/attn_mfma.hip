// attn_mfma.hip -- split-KV partition kernel on the matrix cores, for the rows
// that share one KV head: the G query heads of a group ("Inference-1",
// brunomaga.github.io, "Smaller KV caches: MQA, GQA and MLA") times the n_q
// verify rows ("Inference-2", "Draft-model speculative decoding").  Those R =
// G * n_q rows against a tile of keys form a real dense contraction, so the
// KV head is read from HBM once per group ("Efficient Inference",
// learn.obvix.io: the repeated heads are never materialised).
//
// Per wavefront: one (sequence b, KV head g, row block, partition).  Per
// 16-key tile:
//   S^T[key][row] = K_tile . Q^T        v_mfma_f32_16x16x32_bf16, D/32 steps
//   online softmax per row (running max m, sum l; "Inference-1", section
//   "FlashAttention"; "Inference o quy mo lon", 07 "Online softmax"), the
//   causal limit of verify row r being L - n_q + r ("Inference-1", "KV cache")
//   O^T[d][row] += V_tile^T . P^T          v_mfma_f32_16x16x16_bf16, D/16 steps
// The MFMA accumulator layout puts row = lane % 16 in every lane's registers,
// so the per-row statistics stay lane-local except for the maximum over the 4
// key groups (two shuffles per tile).  P is rounded to bf16 for the second
// product; l sums the same rounded weights so the result stays a convex
// combination of value rows.  The V tile is transposed through a wave-private
// LDS buffer so each lane reads 4 consecutive keys of one column in one 8-byte
// LDS load.
#include "launch.hpp"

namespace kvc {

constexpr int kVtStride = 20;  // bf16 slots per LDS row of V^T: 16 keys + 4 pad (40 bytes)

template <int D, int NT>
__global__ __launch_bounds__(256) void partition_mfma(AttnParams p) {
  constexpr int KK = D / 32;  // QK^T steps of 32
  constexpr int DT = D / 16;  // PV column tiles of 16
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[4][D * kVtStride];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;  // MFMA row/column index of this lane
  const int grp = lane >> 4;  // which 4 (or 8) of the reduction index
  uint16_t* vt = vt_lds[wave];

  const int R = p.G * p.n_q;          // rows sharing this KV head
  const int rows_item = 16 * NT;
  const int n_rb = (R + rows_item - 1) / rows_item;
  const long item = (long)blockIdx.x * 4 + wave;
  const long n_items = (long)p.B * p.Hkv * n_rb * p.max_parts;
  if (item >= n_items) return;
  // item = ((b * Hkv + g) * n_rb + rb) * max_parts + part
  const int part = (int)(item % p.max_parts);
  long t = item / p.max_parts;
  const int rb = (int)(t % n_rb);
  t /= n_rb;
  const int g = (int)(t % p.Hkv);
  const int b = (int)(t / p.Hkv);

  const int L = p.seq_lens[b];
  if (L < p.n_q || L > p.cap) {
    if (part == 0 && g == 0 && rb == 0 && lane == 0) report(p.status, KVC_ERR_DATA);
    return;
  }
  const int nparts = (L + p.P - 1) / p.P;
  if (part >= nparts) return;
  const int start = part * p.P;
  const int end = min(start + p.P, L);  // the last row sees every key

  // this lane's query rows: row i = r * G + hh, query head g * G + hh
  int lvis[NT];
  bool rvalid[NT];
  long qoff[NT], wrow[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int i = rb * rows_item + nt * 16 + col;
    rvalid[nt] = i < R;
    const int r = rvalid[nt] ? i / p.G : 0;
    const int h = g * p.G + (rvalid[nt] ? i % p.G : 0);
    lvis[nt] = rvalid[nt] ? L - p.n_q + r + 1 : L;
    qoff[nt] = (((long)b * p.n_q + r) * p.Hq + h) * D;
    wrow[nt] = ((long)b * p.Hq + h) * p.n_q + r;
  }

  // Q^T as the B operand of S^T = K Q^T: lane holds Q[row col][kk*32 + grp*8 .. +8]
  bf16x8_t qf[NT][KK];
  const uint16_t* qbase = (const uint16_t*)p.q;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (rvalid[nt]) w = *reinterpret_cast<const uint4*>(qbase + qoff[nt] + kk * 32 + grp * 8);
      qf[nt][kk] = __builtin_bit_cast(bf16x8_t, w);
    }

  f32x4_t oacc[NT][DT];
  float m[NT], l[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m[nt] = -INFINITY;
    l[nt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[nt][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  const uint16_t* kbase = (const uint16_t*)p.k;
  const uint16_t* vbase = (const uint16_t*)p.v;
  for (int tile = start; tile < end; tile += kTile) {
    long tbase;
    if (p.table == nullptr) {
      tbase = (((long)b * p.Hkv + g) * p.S_max + tile) * D;
    } else {
      const int blk = p.table[(long)b * p.max_blocks + tile / p.bs];
      if (blk < 0 || blk >= p.N) {
        if (lane == 0) report(p.status, KVC_ERR_DATA);
        continue;
      }
      tbase = (((long)blk * p.Hkv + g) * p.bs + (tile % p.bs)) * D;
    }
    const int nvalid = min(kTile, end - tile);
    const int krow = col < nvalid ? col : nvalid - 1;  // masked keys re-read a visible row
    uint4 kr[KK], vr[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const long off = tbase + (long)krow * D + kk * 32 + grp * 8;
      kr[kk] = *reinterpret_cast<const uint4*>(kbase + off);
      vr[kk] = *reinterpret_cast<const uint4*>(vbase + off);
    }

    // S^T: lane holds keys tile + grp*4 + v (v < 4) of row col (+16 nt)
    bf16x4_t pb[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kr[kk]),
                                                    qf[nt][kk], s, 0, 0, 0);
      float sv[4];
      float mx = -INFINITY;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int key = tile + grp * 4 + v;
        sv[v] = (key < end && key < lvis[nt]) ? s[v] * p.scale_log2 : -INFINITY;
        mx = fmaxf(mx, sv[v]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m[nt], mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;  // row with no visible key yet
      const float alpha = fast_exp2(m[nt] - m_use);
      uint32_t pw[4];
      float psum = 0.f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        pw[v] = f32_to_bf16_bits(fast_exp2(sv[v] - m_use));
        psum += __uint_as_float(pw[v] << 16);
      }
      pb[nt] = __builtin_bit_cast(bf16x4_t, make_uint2(pw[0] | (pw[1] << 16), pw[2] | (pw[3] << 16)));
      l[nt] = l[nt] * alpha + psum;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[nt][dt] *= alpha;
      m[nt] = m_new;
    }

    // V^T into LDS: vt[d][key], d = kk*32 + grp*8 + j, key = col
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const uint32_t w[4] = {vr[kk].x, vr[kk].y, vr[kk].z, vr[kk].w};
      uint16_t* dst = vt + (kk * 32 + grp * 8) * kVtStride + col;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        dst[(2 * j) * kVtStride] = (uint16_t)(w[j] & 0xffffu);
        dst[(2 * j + 1) * kVtStride] = (uint16_t)(w[j] >> 16);
      }
    }
    wave_lds_fence();
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint2 a = *reinterpret_cast<const uint2*>(vt + (dt * 16 + col) * kVtStride + grp * 4);
      const bf16x4_t va = __builtin_bit_cast(bf16x4_t, a);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        oacc[nt][dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb[nt], oacc[nt][dt], 0, 0, 0);
    }
    wave_lds_fence();  // the next tile overwrites vt
  }

  // O^T: lane holds d = dt*16 + grp*4 + v of row col (+16 nt)
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float lt = l[nt] + __shfl_xor(l[nt], 16);
    lt += __shfl_xor(lt, 32);
    if (!rvalid[nt]) continue;
    float* wo = p.ws_o + (wrow[nt] * p.max_parts + part) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<f32x4_t*>(wo + dt * 16 + grp * 4) = oacc[nt][dt];
    if (grp == 0) {
      float* wml = p.ws_ml + (wrow[nt] * p.max_parts + part) * 2;
      wml[0] = m[nt];
      wml[1] = lt;
    }
  }
}

hipError_t launch_partition_mfma(const AttnParams& p, int rows_per_item, hipStream_t s) {
  const int R = p.G * p.n_q;
  const int n_rb = (R + rows_per_item - 1) / rows_per_item;
  const long n_items = (long)p.B * p.Hkv * n_rb * p.max_parts;
  if (n_items == 0) return hipSuccess;
  const dim3 grid((unsigned)((n_items + 3) / 4)), block(256);
  if (rows_per_item == 32) {
    if (p.D == 128) hipLaunchKernelGGL((partition_mfma<128, 2>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((partition_mfma<64, 2>), grid, block, 0, s, p);
  } else {
    if (p.D == 128) hipLaunchKernelGGL((partition_mfma<128, 1>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((partition_mfma<64, 1>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace kvc
