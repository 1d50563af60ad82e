// attn_mfma.hip -- split-KV partition kernel on the matrix cores, for the rows
// that share one KV head: the G query heads of a group ("Inference-1",
// brunomaga.github.io, "Smaller KV caches: MQA, GQA and MLA") times the n_q
// verify rows ("Inference-2", "Draft-model speculative decoding").  Those R =
// G * n_q rows against a tile of keys form a real dense contraction, so the
// KV head is read from HBM once per group ("Efficient Inference",
// learn.obvix.io: the repeated heads are never materialised).
//
// Per wavefront (one per workgroup): one (sequence b, KV head g, block of 16*NT
// rows, partition), spread over the XCDs with xcd_item (common.hpp).
// Partition p of n owns the 16-key tiles p, p + n, ... (as in the VALU kernel);
// in a paged cache their block ids are fetched 64 at a time into one register
// and picked out with v_readlane.
// Per tile of TK keys:
//   1. K and V rows arrive with coalesced non-temporal 16-byte loads (one
//      instruction = RPL whole rows, contiguous) one tile ahead, and are
//      written to a wave-private LDS tile whose rows are padded by 16 bytes so
//      that both the writes and the operand reads below spread over the banks;
//   2. S^T[key][row] = K . Q^T on v_mfma_f32_16x16x32_bf16 (K operands read
//      with ds_read_b128, Q^T held in registers for the whole partition);
//   3. online softmax per row -- running max m and sum l ("Inference-1",
//      "FlashAttention"; "Inference o quy mo lon", 07 "Online softmax") --
//      with verify row r limited to keys 0 .. L - n_q + r ("Inference-1",
//      "KV cache"); the MFMA result layout puts one row in each lane's
//      registers, so only the maximum over the four key groups needs shuffles;
//   4. O^T[d][row] += V^T . P^T on v_mfma_f32_16x16x32_bf16; the V^T operand
//      comes straight from the row-major LDS tile through ds_read_b64_tr_b16,
//      whose 16-lane transpose delivers four consecutive keys of one column.
// The weights enter the second product as two bf16 halves, hi = bf16(p) and
// lo = bf16(p - hi), side by side along the reduction index against two
// copies of the V^T fragment: p keeps about 16 significant bits (a plain bf16
// p would perturb each weight by up to 2^-9, which on a few dominant keys with
// large values exceeds the output tolerance), at the same instruction count
// as a single 16x16x16 product.  l sums the fp32 weights.
#include "launch.hpp"

namespace kvc {

typedef short i16x4_t __attribute__((__vector_size__(4 * sizeof(short))));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// MINW: wavefronts per SIMD the register allocation must leave room for.
// F: 0 for a bf16 cache, else the FP8 format of the codes (the LDS tile and
// everything after it stay bf16: codes are widened exactly on the way in, the
// key scales multiply the scores and the value scales join the weights).
template <int D, int NT, int MINW, int F>
__global__ __launch_bounds__(64, MINW) void partition_mfma(AttnParams p) {
  constexpr int KK = D / 32;          // QK^T steps of 32 along D
  constexpr int DT = D / 16;          // PV output column tiles
  constexpr int EB = F ? 1 : 2;       // bytes per cache element in HBM
  constexpr int CH = D * EB / 16;     // 16-byte chunks per key row
  constexpr int RPL = kWave / CH;     // key rows per wave load
  constexpr int U = kTile / RPL;      // loads per tile, each of K and V
  constexpr int ROWB = D * 2 + 16;    // LDS row stride: one 16-byte pad per key row
  constexpr int TILEB = kTile * ROWB;
  __shared__ __attribute__((aligned(16))) uint8_t lds_all[2 * TILEB];

  const int lane = threadIdx.x;
  const int col = lane & 15;  // MFMA row/column index of this lane
  const int grp = lane >> 4;  // which quarter of the reduction index
  uint8_t* k_lds = lds_all;
  uint8_t* v_lds = lds_all + TILEB;

  const int R = p.G * p.n_q;  // rows sharing this KV head
  const int rows_item = 16 * NT;
  const int n_rb = (R + rows_item - 1) / rows_item;
  const WorkItem wi = xcd_item(blockIdx.x, p.Hkv * n_rb, p.max_parts);  // u = g * n_rb + rb
  if (!wi.live) return;
  const int b = wi.b, part = wi.part, rb = wi.u % n_rb, g = wi.u / n_rb;

  const int L = __builtin_amdgcn_readfirstlane(p.seq_lens[b]);
  if (L < p.n_q || L > p.cap) {
    if (part == 0 && g == 0 && rb == 0 && lane == 0) report(p.status, KVC_ERR_DATA);
    return;
  }
  if (part >= (L + p.P_lo - 1) / p.P_lo) return;  // beyond any length's partitions
  const int P = part_tokens(p.seq_lens, p.B, p.cap, p.slots_u, p.P_lo, p.P);
  const int nparts = (L + P - 1) / P;
  if (part >= nparts) return;
  const int start = part * kTile;     // first tile of this partition
  const int stride = nparts * kTile;  // distance to its next tile
  const int end = L;                  // the last row sees every key

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
    lvis[nt] = rvalid[nt] ? L - p.n_q + r + 1 : L;  // <= end
    qoff[nt] = (((long)b * p.n_q + r) * p.Hq + h) * D;
    wrow[nt] = ((long)b * p.Hq + h) * p.n_q + r;
  }
  // keys every row of this wavefront sees: tiles below it need no mask
  int vis_min = lvis[0];
#pragma unroll
  for (int nt = 1; nt < NT; ++nt) vis_min = min(vis_min, lvis[nt]);
  for (int mm = 1; mm < kWave; mm <<= 1) vis_min = min(vis_min, __shfl_xor(vis_min, mm));
  vis_min = __builtin_amdgcn_readfirstlane(vis_min);

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
  float m[NT], l[NT];  // m: reference maximum (log2 domain), may trail the true one
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m[nt] = -INFINITY;
    l[nt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[nt][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  const int lr = lane / CH;   // key row of a wave load
  const int pos = lane % CH;  // 16-byte chunk of that row
  const int bs_shift = __builtin_ctz((unsigned)(p.bs > 0 ? p.bs : 1));
  // paged: lane i holds the block of the partition's tile number j * 64 + i
  const bool paged = p.table != nullptr;
  const int32_t* trow = paged ? p.table + (long)b * p.max_blocks : nullptr;
  auto load_ids = [&](int j) -> int {
    const int tk = start + (j * kWave + lane) * stride;
    return tk < end ? trow[tk >> bs_shift] : 0;
  };
  int ids = 0, ids_next = 0;
  if (paged && start < end) {
    ids = load_ids(0);
    if (start + kWave * stride < end) ids_next = load_ids(1);
  }
  // wave-uniform element offset of key `tile`, the partition's tile number idx,
  // of (b, g); -1 when the block table points outside the pool (the tile is
  // then skipped)
  auto tile_base = [&](int tile, int idx) -> long {
    if (!paged) return (((long)b * p.Hkv + g) * p.S_max + tile) * D;
    const int blk = __builtin_amdgcn_readlane(ids, idx & (kWave - 1));
    if (blk < 0 || blk >= p.N) return -1;
    return (((long)blk * p.Hkv + g) * p.bs + (tile & (p.bs - 1))) * D;
  };
  uint4 kreg[U], vreg[U];
  float ks_next[4], vs_next[4];  // FP8: scales of keys grp*4 .. +3 of the tile in flight
  auto load_tile = [&](int tile, long tb) {
    // uniform bases, 32-bit lane offsets; FP8: the tile's run of codes, then scales
    const long tbyte = F ? (tb / (16 * D)) * fp8_tile_bytes(D) : tb * EB;
    const uint8_t* kt = (const uint8_t*)p.k + tbyte;
    const uint8_t* vt = (const uint8_t*)p.v + tbyte;
    const int last = min(kTile, end - tile) - 1;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = min(u * RPL + lr, last);  // masked keys re-read a visible row
      const uint32_t off = (uint32_t)(key * D * EB + pos * 16);
      kreg[u] = load_stream(kt + off);
      vreg[u] = load_stream(vt + off);
    }
    if constexpr (F != 0) {
      // scales of keys grp*4 .. +3, non-temporal like the codes (a cached
      // load would allocate in the last-level caches and wait on their
      // evictions); masked keys re-read a visible row's scale
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int key = min(grp * 4 + v, last);
        ks_next[v] = __builtin_nontemporal_load(reinterpret_cast<const float*>(kt + 16 * D + key * 4));
        vs_next[v] = __builtin_nontemporal_load(reinterpret_cast<const float*>(vt + 16 * D + key * 4));
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (F == 0) {
        const int off = (u * RPL + lr) * ROWB + pos * 16;
        *reinterpret_cast<uint4*>(k_lds + off) = kreg[u];
        *reinterpret_cast<uint4*>(v_lds + off) = vreg[u];
      } else {  // 16 codes -> 16 bf16 (32 bytes)
        const int off = (u * RPL + lr) * ROWB + pos * 32;
        const uint2 k0 = fp8x4_to_bf16x4<F>(kreg[u].x), k1 = fp8x4_to_bf16x4<F>(kreg[u].y);
        const uint2 k2 = fp8x4_to_bf16x4<F>(kreg[u].z), k3 = fp8x4_to_bf16x4<F>(kreg[u].w);
        const uint2 v0 = fp8x4_to_bf16x4<F>(vreg[u].x), v1 = fp8x4_to_bf16x4<F>(vreg[u].y);
        const uint2 v2 = fp8x4_to_bf16x4<F>(vreg[u].z), v3 = fp8x4_to_bf16x4<F>(vreg[u].w);
        *reinterpret_cast<uint4*>(k_lds + off) = make_uint4(k0.x, k0.y, k1.x, k1.y);
        *reinterpret_cast<uint4*>(k_lds + off + 16) = make_uint4(k2.x, k2.y, k3.x, k3.y);
        *reinterpret_cast<uint4*>(v_lds + off) = make_uint4(v0.x, v0.y, v1.x, v1.y);
        *reinterpret_cast<uint4*>(v_lds + off + 16) = make_uint4(v2.x, v2.y, v3.x, v3.y);
      }
    }
  };
  float ks_cur[4] = {1.f, 1.f, 1.f, 1.f}, vs_cur[4] = {1.f, 1.f, 1.f, 1.f};
  // per-lane LDS operand addresses (loop invariant; the k/dt steps are immediates)
  const uint8_t* ka_ptr = k_lds + col * ROWB + grp * 16;
  const uint8_t* va_ptr = v_lds + (grp * 4 + (col >> 2)) * ROWB + (col & 3) * 8;
  constexpr float kLazy = 8.f;  // the reference maximum moves only past m + 8 (p <= 2^8)

  if (start < end) {
    int idx = 0;
    long tb = tile_base(start, 0);
    if (tb >= 0) load_tile(start, tb);
    store_tile();
    if constexpr (F != 0) {
#pragma unroll
      for (int v = 0; v < 4; ++v) ks_cur[v] = ks_next[v], vs_cur[v] = vs_next[v];
    }
    wave_lds_fence();
    for (int tile = start; tile < end; tile += stride, ++idx) {
      const int next = tile + stride;
      const bool ok = tb >= 0;
      long tb_next = -1;
      if (next < end) {
        if (paged && ((idx + 1) & (kWave - 1)) == 0) {  // the next 64 tiles' ids
          const int j = (idx + 1) / kWave;
          ids = ids_next;
          if (start + (j + 1) * kWave * stride < end) ids_next = load_ids(j + 1);
        }
        tb_next = tile_base(next, idx + 1);
        if (tb_next >= 0) load_tile(next, tb_next);  // in flight while this tile computes
      }
      if (ok) {
        // S^T for 16 keys: lane holds keys tile + grp*4 + v of row col (+16 nt)
        bf16x8_t ka[KK];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
          ka[kk] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(ka_ptr + kk * 64));
        bf16x8_t pb[NT];  // keys grp*4 + 0..3: hi halves, then lo halves
        float sl[4];       // score factor of each of this lane's four keys
#pragma unroll
        for (int v = 0; v < 4; ++v) sl[v] = F ? ks_cur[v] * p.scale_log2 : p.scale_log2;
        // two accumulation chains per row block (even and odd steps along D),
        // interleaved across the row blocks, so no product waits on the one
        // just issued
        f32x4_t sc[NT][2];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) sc[nt][0] = sc[nt][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            sc[nt][kk & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kk], qf[nt][kk], sc[nt][kk & 1], 0, 0, 0);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const f32x4_t s = sc[nt][0] + sc[nt][1];
          const int key0 = tile + grp * 4;
          float sv[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) sv[v] = s[v] * sl[v];
          if (tile + kTile > vis_min) {  // the tile reaches past some row's last key
#pragma unroll
            for (int v = 0; v < 4; ++v) sv[v] = key0 + v < lvis[nt] ? sv[v] : -INFINITY;
          }
          float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
          mx = fmaxf(mx, __shfl_xor(mx, 16));
          mx = fmaxf(mx, __shfl_xor(mx, 32));
          const bool move = mx > m[nt] + kLazy;  // false while the row has no visible key
          if (__any(move)) {
            const float m_new = move ? mx : m[nt];
            const float alpha = m[nt] == -INFINITY ? 0.f : fast_exp2(m[nt] - m_new);
            l[nt] *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) oacc[nt][dt] *= alpha;
            m[nt] = m_new;
          }
          const float m_use = m[nt] == -INFINITY ? 0.f : m[nt];
          f32x2_t p01 = {fast_exp2(sv[0] - m_use), fast_exp2(sv[1] - m_use)};
          f32x2_t p23 = {fast_exp2(sv[2] - m_use), fast_exp2(sv[3] - m_use)};
          l[nt] += (p01[0] + p01[1]) + (p23[0] + p23[1]);
          if constexpr (F != 0) {  // the value rows' scales join the weights
            p01 *= f32x2_t{vs_cur[0], vs_cur[1]};
            p23 *= f32x2_t{vs_cur[2], vs_cur[3]};
          }
          const bf16x2_t h01 = __builtin_convertvector(p01, bf16x2_t);
          const bf16x2_t h23 = __builtin_convertvector(p23, bf16x2_t);
          const f32x2_t r01 = p01 - __builtin_convertvector(h01, f32x2_t);  // exact
          const f32x2_t r23 = p23 - __builtin_convertvector(h23, f32x2_t);
          const bf16x2_t lo01 = __builtin_convertvector(r01, bf16x2_t);
          const bf16x2_t lo23 = __builtin_convertvector(r23, bf16x2_t);
          pb[nt] = __builtin_shufflevector(__builtin_shufflevector(h01, h23, 0, 1, 2, 3),
                                           __builtin_shufflevector(lo01, lo23, 0, 1, 2, 3),
                                           0, 1, 2, 3, 4, 5, 6, 7);
        }
        // V^T operand: lane (grp, col = 4s + q) points at V[key 4grp + s][dt*16 + 4q]
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          lds_i16x4_t* a = reinterpret_cast<lds_i16x4_t*>(
              (__attribute__((address_space(3))) uint8_t*)(va_ptr + dt * 32));
          const bf16x4_t va = __builtin_bit_cast(bf16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(a));
          const bf16x8_t va2 = __builtin_shufflevector(va, va, 0, 1, 2, 3, 0, 1, 2, 3);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            oacc[nt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va2, pb[nt], oacc[nt][dt], 0, 0, 0);
        }
      } else if (lane == 0) {
        report(p.status, KVC_ERR_DATA);
      }
      wave_lds_fence();  // this tile's LDS reads are issued before it is overwritten
      if (next < end) store_tile();
      if constexpr (F != 0) {
#pragma unroll
        for (int v = 0; v < 4; ++v) ks_cur[v] = ks_next[v], vs_cur[v] = vs_next[v];
      }
      wave_lds_fence();
      tb = tb_next;
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

template <int F>
void launch_mfma_fmt(const AttnParams& p, int rows_per_item, dim3 grid, dim3 block,
                     hipStream_t s) {
  // The register budget leaves room for 2 (32-row blocks) or 3 (16-row
  // blocks) wavefronts per SIMD, which measured best on MI355X.
  if (rows_per_item == 32) {
    if (p.D == 128) hipLaunchKernelGGL((partition_mfma<128, 2, 2, F>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((partition_mfma<64, 2, 2, F>), grid, block, 0, s, p);
  } else {
    if (p.D == 128) hipLaunchKernelGGL((partition_mfma<128, 1, 3, F>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((partition_mfma<64, 1, 3, F>), grid, block, 0, s, p);
  }
}

hipError_t launch_partition_mfma(const AttnParams& p, int rows_per_item, int fp8, hipStream_t s) {
  const int R = p.G * p.n_q;
  const int n_rb = (R + rows_per_item - 1) / rows_per_item;
  const long n_wg = xcd_grid(p.B, p.Hkv * n_rb, p.max_parts);
  if (n_wg == 0) return hipSuccess;
  if (n_wg > 0x7fffffffL) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)n_wg), block(64);
  if (fp8 == kFp8E4M3) launch_mfma_fmt<kFp8E4M3>(p, rows_per_item, grid, block, s);
  else if (fp8 == kFp8E5M2) launch_mfma_fmt<kFp8E5M2>(p, rows_per_item, grid, block, s);
  else launch_mfma_fmt<0>(p, rows_per_item, grid, block, s);
  return hipGetLastError();
}

}  // namespace kvc
