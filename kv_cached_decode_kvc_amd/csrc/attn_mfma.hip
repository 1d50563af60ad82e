// attn_mfma.hip -- split-KV partition kernel on the matrix cores, for the rows
// that share one KV head: the G query heads of a group ("Inference-1",
// brunomaga.github.io, "Smaller KV caches: MQA, GQA and MLA") times the n_q
// verify rows ("Inference-2", "Draft-model speculative decoding").  Those R =
// G * n_q rows against a tile of keys form a real dense contraction, so the
// KV head is read from HBM once per group ("Efficient Inference",
// learn.obvix.io: the repeated heads are never materialised).
//
// Per wavefront: one (sequence b, KV head g, block of 16*NT rows, partition).
// Partition p of n owns the 16-key tiles p, p + n, ... (as in the VALU kernel).
// Per tile of TK keys:
//   1. K and V rows arrive with coalesced non-temporal 16-byte loads (one
//      instruction = RPL whole rows, contiguous) one tile ahead, and are
//      written to a wave-private LDS tile whose 16-byte chunks are XOR-
//      swizzled by key so that both the writes and the operand reads below
//      hit distinct banks;
//   2. S^T[key][row] = K . Q^T on v_mfma_f32_16x16x32_bf16 (K operands read
//      with ds_read_b128, Q^T held in registers for the whole partition);
//   3. online softmax per row -- running max m and sum l ("Inference-1",
//      "FlashAttention"; "Inference o quy mo lon", 07 "Online softmax") --
//      with verify row r limited to keys 0 .. L - n_q + r ("Inference-1",
//      "KV cache"); the MFMA result layout puts one row in each lane's
//      registers, so only the maximum over the four key groups needs shuffles;
//   4. O^T[d][row] += V^T . P^T on v_mfma_f32_16x16x16_bf16; the V^T operand
//      comes straight from the row-major LDS tile through ds_read_b64_tr_b16,
//      whose 16-lane transpose delivers four consecutive keys of one column.
// P is rounded to bf16 for the second product and l sums the same rounded
// weights, so each partition's result is a convex combination of value rows.
#include "launch.hpp"

namespace kvc {

typedef short i16x4_t __attribute__((__vector_size__(4 * sizeof(short))));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// MINW: wavefronts per SIMD the register allocation must leave room for.
template <int D, int NT, int TK, int MINW>
__global__ __launch_bounds__(256, MINW) void partition_mfma(AttnParams p) {
  constexpr int KK = D / 32;         // QK^T steps of 32 along D
  constexpr int DT = D / 16;         // PV output column tiles
  constexpr int CH = D / 8;          // 16-byte chunks per key row
  constexpr int RPL = kWave / CH;    // key rows per wave load
  constexpr int U = TK / RPL;        // loads per tile, each of K and V
  constexpr int SB = TK / kTile;     // 16-key sub-tiles per tile
  constexpr int ROWB = D * 2;        // bytes per key row
  constexpr int TILEB = TK * ROWB;   // bytes per K (or V) tile
  static_assert(TK % kTile == 0 && U * RPL == TK, "tile shape");
  __shared__ __attribute__((aligned(16))) uint8_t lds_all[4][2 * TILEB];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;  // MFMA row/column index of this lane
  const int grp = lane >> 4;  // which quarter of the reduction index
  uint8_t* k_lds = lds_all[wave];
  uint8_t* v_lds = lds_all[wave] + TILEB;

  const int R = p.G * p.n_q;  // rows sharing this KV head
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
  const int start = part * TK;       // first tile of this partition
  const int stride = nparts * TK;    // distance to its next tile
  const int end = L;                 // the last row sees every key

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
  const int lr = lane / CH;   // row of a wave load
  const int pos = lane % CH;  // 16-byte position inside the LDS row

  // Global -> registers for the tile starting at key `tile`; false when the
  // block table points outside the pool (the tile is then skipped).
  uint4 kreg[U], vreg[U];
  auto load_tile = [&](int tile) -> bool {
    const int nvalid = min(TK, end - tile);
    long sbase[SB];
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) {
      sbase[sb] = 0;
      if (sb * kTile >= nvalid) continue;  // never look up blocks past the length
      const int t0 = tile + sb * kTile;
      if (p.table == nullptr) {
        sbase[sb] = (((long)b * p.Hkv + g) * p.S_max + t0) * D;
      } else {
        const int blk = p.table[(long)b * p.max_blocks + t0 / p.bs];
        if (blk < 0 || blk >= p.N) return false;
        sbase[sb] = (((long)blk * p.Hkv + g) * p.bs + (t0 % p.bs)) * D;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = u * RPL + lr;                 // LDS row this lane fills
      const int src = key < nvalid ? key : nvalid - 1;  // masked keys re-read a visible row
      const int chunk = pos ^ (key & (CH - 1));     // chunk stored at position pos
      const long off = sbase[src / kTile] + (long)(src % kTile) * D + chunk * 8;
      kreg[u] = load_stream(kbase + off);
      vreg[u] = load_stream(vbase + off);
    }
    return true;
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = u * RPL + lr;
      *reinterpret_cast<uint4*>(k_lds + key * ROWB + pos * 16) = kreg[u];
      *reinterpret_cast<uint4*>(v_lds + key * ROWB + pos * 16) = vreg[u];
    }
  };

  if (start < end) {
    bool ok = load_tile(start);
    store_tile();
    wave_lds_fence();
    for (int tile = start; tile < end; tile += stride) {
      const int next = tile + stride;
      bool ok_next = true;
      if (next < end) ok_next = load_tile(next);  // in flight while this tile computes
      if (ok) {
#pragma unroll
        for (int sb = 0; sb < SB; ++sb) {
          // S^T for keys sb*16 .. +16: lane holds keys grp*4 + v of row col (+16 nt)
          bf16x8_t ka[KK];
#pragma unroll
          for (int kk = 0; kk < KK; ++kk) {
            const int key = sb * kTile + col;
            const int chunk = (kk * 4 + grp) ^ (key & (CH - 1));
            ka[kk] = __builtin_bit_cast(
                bf16x8_t, *reinterpret_cast<const uint4*>(k_lds + key * ROWB + chunk * 16));
          }
          bf16x4_t pb[NT];
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
              s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kk], qf[nt][kk], s, 0, 0, 0);
            float sv[4];
            float mx = -INFINITY;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int key = tile + sb * kTile + grp * 4 + v;
              sv[v] = (key < end && key < lvis[nt]) ? s[v] * p.scale_log2 : -INFINITY;
              mx = fmaxf(mx, sv[v]);
            }
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m[nt], mx);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;  // no visible key yet
            const float alpha = fast_exp2(m[nt] - m_use);
            uint32_t pw[4];
            float psum = 0.f;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              pw[v] = f32_to_bf16_bits(fast_exp2(sv[v] - m_use));
              psum += __uint_as_float(pw[v] << 16);
            }
            pb[nt] = __builtin_bit_cast(bf16x4_t,
                                        make_uint2(pw[0] | (pw[1] << 16), pw[2] | (pw[3] << 16)));
            l[nt] = l[nt] * alpha + psum;
            if (alpha != 1.f) {
#pragma unroll
              for (int dt = 0; dt < DT; ++dt) oacc[nt][dt] *= alpha;
            }
            m[nt] = m_new;
          }
          // V^T operand: lane (grp, col = 4s + q) points at V[key sb*16 + 4grp + s][dt*16 + 4q]
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const int key = sb * kTile + grp * 4 + (col >> 2);
            const int d0 = dt * 16 + (col & 3) * 4;
            const int chunk = (d0 >> 3) ^ (key & (CH - 1));
            lds_i16x4_t* a = reinterpret_cast<lds_i16x4_t*>(
                (__attribute__((address_space(3))) uint8_t*)(v_lds + key * ROWB + chunk * 16 +
                                                             (d0 & 7) * 2));
            const bf16x4_t va =
                __builtin_bit_cast(bf16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(a));
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
              oacc[nt][dt] =
                  __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb[nt], oacc[nt][dt], 0, 0, 0);
          }
        }
      } else if (lane == 0) {
        report(p.status, KVC_ERR_DATA);
      }
      wave_lds_fence();  // this tile's LDS reads are issued before it is overwritten
      if (next < end) store_tile();
      wave_lds_fence();
      ok = ok_next;
    }
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
  // 16-key tiles; the register budget leaves room for 2 (32-row blocks) or 3
  // (16-row blocks) wavefronts per SIMD, which measured best on MI355X.
  if (rows_per_item == 32) {
    if (p.D == 128) hipLaunchKernelGGL((partition_mfma<128, 2, 16, 2>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((partition_mfma<64, 2, 16, 2>), grid, block, 0, s, p);
  } else {
    if (p.D == 128) hipLaunchKernelGGL((partition_mfma<128, 1, 16, 3>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((partition_mfma<64, 1, 16, 3>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace kvc
