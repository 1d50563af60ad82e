// attn_mfma.hip -- split-KV partition kernel on the matrix cores, for the rows
// that share one KV head: the G query heads of a group ("Inference-1",
// brunomaga.github.io, "Smaller KV caches: MQA, GQA and MLA") times the n_q
// verify rows ("Inference-2", "Draft-model speculative decoding").  Those R =
// G * n_q rows against a tile of keys form a real dense contraction, so the
// KV head is read from HBM once per group ("Efficient Inference",
// learn.obvix.io: the repeated heads are never materialised).
//
// Work split, two forms.  With the library's default (SK = true) the batch's
// 16-key tiles are shared out evenly over one round of resident wavefronts:
// a segment is one (sequence b, KV head g, block of 16*NT rows) with T_b =
// ceil(L_b / 16) tiles, the segments are laid end to end in (b, g, block)
// order, and worker w of NW takes tile-units [w W / NW, (w+1) W / NW) of the
// W in total -- a contiguous run of tiles that may end one segment and start
// the next.  Every worker then streams the same number of tiles (+-1),
// whatever the lengths, so the launch ends when its average wavefront does
// ("Inference-1", "FlashDecoding": any split of the keys combines exactly).
// Each (segment, worker) piece leaves one partial per row at piece index
// segment + worker (unique, since both grow along the run), and the worker
// holding a segment's first tile records which workers cover it, for the
// combine.  With an explicit partition length (SK = false) a wavefront owns
// one (sequence, KV head, row block, partition), spread over the XCDs with
// xcd_item (common.hpp), and partition p of n owns the 16-key tiles p, p + n,
// ... (as in the VALU kernel).  In a paged cache the block ids of a piece's
// tiles are fetched 64 at a time into one register and picked out with
// v_readlane.
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
template <int D, int NT, int MINW, int F, bool SK, int PF>
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
  const int SU = p.Hkv * n_rb;  // segments (row blocks of a KV head) of a sequence

  // One piece of work: tiles start, start + stride, ... below tile_end (keys)
  // of the row block rb of KV head g of sequence b (L keys attended).  Its
  // partials go to slot `slot`: the piece index (SK: row i of the block at
  // piece * sk_rows + i), or the partition (workspace row (b, h, r)).
  auto run_piece = [&](int b, int g, int rb, int L, int start, int stride, int tile_end,
                       long slot) {
  const int end = L;  // the last row sees every key
  // this lane's query rows: row i = r * G + hh, query head g * G + hh
  int lvis[NT];
  bool rvalid[NT];
  long qoff[NT], wrow[NT];  // wrow: workspace row of the partial
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int i = rb * rows_item + nt * 16 + col;
    rvalid[nt] = i < R;
    const int r = rvalid[nt] ? i / p.G : 0;
    const int h = g * p.G + (rvalid[nt] ? i % p.G : 0);
    lvis[nt] = rvalid[nt] ? L - p.n_q + r + 1 : L;  // <= end
    qoff[nt] = (((long)b * p.n_q + r) * p.Hq + h) * D;
    wrow[nt] = SK ? slot * p.sk_rows + nt * 16 + col
                  : (((long)b * p.Hq + h) * p.n_q + r) * p.max_parts + slot;
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
    return tk < tile_end ? trow[tk >> bs_shift] : 0;
  };
  int ids = 0, ids_next = 0;
  if (paged && start < tile_end) {
    ids = load_ids(0);
    if (start + kWave * stride < tile_end) ids_next = load_ids(1);
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
  // PF register stages: stage s holds a tile's K and V rows (and, FP8, its
  // scales) from the load until the tile is written to LDS.  Tile n of the
  // piece lives in stage n % PF, so PF tiles are in flight while one
  // computes.  Every stage issues the same loads whatever the tile: a tile
  // past the piece's end or in a bad block re-reads the cache's first row
  // (cached after the first time), so the compiler can wait for one stage's
  // loads alone.
  uint4 kreg[PF][U], vreg[PF][U];
  float ksn[PF][4], vsn[PF][4];  // FP8: scales of keys grp*4 .. +3 of each stage's tile
  long stb[PF];                  // tile base of each stage (-1: none, or a bad block)
  auto load_stage = [&](int s, int n) {  // tile number n of the piece into stage s
    const int tile = start + n * stride;
    long tb = -1;
    if (tile < tile_end) {
      if (paged && n > 0 && (n & (kWave - 1)) == 0) {  // the next 64 tiles' ids
        ids = ids_next;
        if (start + (n + kWave) * stride < tile_end) ids_next = load_ids(n / kWave + 1);
      }
      tb = tile_base(tile, n);
    }
    stb[s] = tb;
    const bool real = tb >= 0;
    // uniform bases, 32-bit lane offsets; FP8: the tile's run of codes, then scales
    const long tbyte = !real ? 0 : F ? (tb / (16 * D)) * fp8_tile_bytes(D) : tb * EB;
    const uint8_t* kt = (const uint8_t*)p.k + tbyte;
    const uint8_t* vt = (const uint8_t*)p.v + tbyte;
    const int last = real ? min(kTile, end - tile) - 1 : 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = min(u * RPL + lr, last);  // masked keys re-read a visible row
      const uint32_t off = (uint32_t)(key * D * EB + pos * 16);
      kreg[s][u] = load_stream(kt + off);
      vreg[s][u] = load_stream(vt + off);
    }
    if constexpr (F != 0) {
      // scales of keys grp*4 .. +3, non-temporal like the codes (a cached
      // load would allocate in the last-level caches and wait on their
      // evictions); masked keys re-read a visible row's scale
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int key = min(grp * 4 + v, last);
        ksn[s][v] = __builtin_nontemporal_load(reinterpret_cast<const float*>(kt + 16 * D + key * 4));
        vsn[s][v] = __builtin_nontemporal_load(reinterpret_cast<const float*>(vt + 16 * D + key * 4));
      }
    }
  };
  auto store_stage = [&](int s) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (F == 0) {
        const int off = (u * RPL + lr) * ROWB + pos * 16;
        *reinterpret_cast<uint4*>(k_lds + off) = kreg[s][u];
        *reinterpret_cast<uint4*>(v_lds + off) = vreg[s][u];
      } else {  // 16 codes -> 16 bf16 (32 bytes)
        const int off = (u * RPL + lr) * ROWB + pos * 32;
        const uint2 k0 = fp8x4_to_bf16x4<F>(kreg[s][u].x), k1 = fp8x4_to_bf16x4<F>(kreg[s][u].y);
        const uint2 k2 = fp8x4_to_bf16x4<F>(kreg[s][u].z), k3 = fp8x4_to_bf16x4<F>(kreg[s][u].w);
        const uint2 v0 = fp8x4_to_bf16x4<F>(vreg[s][u].x), v1 = fp8x4_to_bf16x4<F>(vreg[s][u].y);
        const uint2 v2 = fp8x4_to_bf16x4<F>(vreg[s][u].z), v3 = fp8x4_to_bf16x4<F>(vreg[s][u].w);
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

  if (start < tile_end) {
#pragma unroll
    for (int k = 0; k < PF; ++k) load_stage(k, k);
    store_stage(0);
    if constexpr (F != 0) {
#pragma unroll
      for (int v = 0; v < 4; ++v) ks_cur[v] = ksn[0][v], vs_cur[v] = vsn[0][v];
    }
    wave_lds_fence();
    for (int n0 = 0; start + n0 * stride < tile_end; n0 += PF) {
#pragma unroll
      for (int j = 0; j < PF; ++j) {
        const int n = n0 + j;  // tile number n of the piece: in LDS, it came from stage j
        const int tile = start + n * stride;
        if (tile >= tile_end) break;
        const bool ok = stb[j] >= 0;
        load_stage(j, n + PF);  // in flight while this tile and the next PF - 1 compute
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
            mx = rows_max(mx);
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
        if (tile + stride < tile_end) store_stage((j + 1) % PF);  // tile n + 1
        if constexpr (F != 0) {
#pragma unroll
          for (int v = 0; v < 4; ++v) ks_cur[v] = ksn[(j + 1) % PF][v], vs_cur[v] = vsn[(j + 1) % PF][v];
        }
        wave_lds_fence();
      }
    }
  }

  // O^T: lane holds d = dt*16 + grp*4 + v of row col (+16 nt)
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float lt = l[nt] + __shfl_xor(l[nt], 16);
    lt += __shfl_xor(lt, 32);
    if (!rvalid[nt]) continue;
    float* wo = p.ws_o + wrow[nt] * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<f32x4_t*>(wo + dt * 16 + grp * 4) = oacc[nt][dt];
    if (grp == 0) {
      float* wml = p.ws_ml + wrow[nt] * 2;
      wml[0] = m[nt];
      wml[1] = lt;
    }
  }
  };  // run_piece

  if constexpr (!SK) {
    const WorkItem wi = xcd_item(blockIdx.x, SU, p.max_parts);  // u = g * n_rb + rb
    if (!wi.live) return;
    const int b = wi.b, part = wi.part, rb = wi.u % n_rb, g = wi.u / n_rb;
    const int L = __builtin_amdgcn_readfirstlane(p.seq_lens[b]);
    if (L < p.n_q || L > p.cap) {
      if (part == 0 && g == 0 && rb == 0 && lane == 0) report(p.status, KVC_ERR_DATA);
      return;
    }
    const int nparts = (L + p.P - 1) / p.P;
    if (part >= nparts) return;
    run_piece(b, g, rb, L, part * kTile, nparts * kTile, L, part);
  } else {
    // Stream-K: the lengths give T_b tiles per sequence (0 for an invalid
    // length, which worker 0 reports), W = SU * sum T_b tile-units in all.
    const int w = blockIdx.x;
    long W = 0;
    int bad = 0;
    for (int c = 0; c < p.B; c += kWave) {
      const int i = c + lane;
      int T = 0;
      if (i < p.B) {
        const int Li = p.seq_lens[i];
        if (Li >= p.n_q && Li <= p.cap) T = (Li + kTile - 1) / kTile;
        else bad = 1;
      }
      for (int m = 1; m < kWave; m <<= 1) T += __shfl_xor(T, m);
      W += T;
    }
    if (w == 0 && __any(bad) && lane == 0) report(p.status, KVC_ERR_DATA);
    W *= SU;  // the same on every lane
    if (W == 0) return;
    const long NW = min((long)gridDim.x, max(1L, W / p.sk_min_tiles));
    if (w >= NW) return;
    const long s0 = (long)w * W / NW, s1 = (long)(w + 1) * W / NW;
    if (s0 >= s1) return;
    // the sequence holding tile-unit s0: first b with (units before b + its units) > s0
    int b = 0;
    long pre = 0;  // tile-units before sequence b
    for (int c = 0; c < p.B; c += kWave) {
      const int i = c + lane;
      long n = 0;
      if (i < p.B) {
        const int Li = p.seq_lens[i];
        if (Li >= p.n_q && Li <= p.cap) n = (long)SU * ((Li + kTile - 1) / kTile);
      }
      long incl = n;
      for (int d = 1; d < kWave; d <<= 1) {
        const long t = __shfl_up(incl, d);
        if (lane >= d) incl += t;
      }
      const unsigned long long hit = __ballot(s0 < pre + incl);
      if (hit != 0) {
        const int j = __ffsll((long long)hit) - 1;
        b = c + j;
        pre += __shfl(incl - n, j);
        break;
      }
      pre += __shfl(incl, kWave - 1);
    }
    b = __builtin_amdgcn_readfirstlane(b);
    int L = __builtin_amdgcn_readfirstlane(p.seq_lens[b]);
    int T = (L + kTile - 1) / kTile;  // >= 1: sequence b holds s0
    long pos = s0;
    while (pos < s1) {
      while (pos >= pre + (long)SU * T) {  // past sequence b: the next one with tiles
        pre += (long)SU * T;
        ++b;
        L = __builtin_amdgcn_readfirstlane(p.seq_lens[b]);
        T = (L >= p.n_q && L <= p.cap) ? (L + kTile - 1) / kTile : 0;
      }
      const long local = pos - pre;
      const int u = (int)(local / T), t0 = (int)(local % T);
      const int t1 = (int)min((long)T, t0 + (s1 - pos));
      const int seg = b * SU + u;
      if (t0 == 0 && lane == 0) {  // this worker starts the segment: record its workers
        const long x_last = pre + (long)u * T + T - 1;
        const int w_last = (int)(((x_last + 1) * NW - 1) / W);
        p.sk_meta[seg] = make_int2(w, w_last);
      }
      run_piece(b, u / n_rb, u % n_rb, L, t0 * kTile, kTile, min(t1 * kTile, L),
                (long)seg + w);
      pos += t1 - t0;
    }
  }
}

template <int F, bool SK>
void launch_mfma_fmt(const AttnParams& p, int rows_per_item, dim3 grid, dim3 block,
                     hipStream_t s) {
  if constexpr (SK && F == 0) {
    // bf16 stream-K with 32-row blocks (verify): one worker per SIMD, so the
    // whole register file is its own and two tiles stay in flight (full-size
    // verify 65.9 -> 64.3 us; the 16-row GQA kernel measured 5% slower with
    // two stages and keeps one)
    if (rows_per_item == 32) {
      if (p.D == 128) hipLaunchKernelGGL((partition_mfma<128, 2, 1, F, SK, 2>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((partition_mfma<64, 2, 1, F, SK, 2>), grid, block, 0, s, p);
      return;
    }
  }
  // The register budget leaves room for 2 (32-row blocks) or 3 (16-row
  // blocks) wavefronts per SIMD, which measured best on MI355X.
  if (rows_per_item == 32) {
    if (p.D == 128) hipLaunchKernelGGL((partition_mfma<128, 2, 2, F, SK, 1>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((partition_mfma<64, 2, 2, F, SK, 1>), grid, block, 0, s, p);
  } else {
    if (p.D == 128) hipLaunchKernelGGL((partition_mfma<128, 1, 3, F, SK, 1>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((partition_mfma<64, 1, 3, F, SK, 1>), grid, block, 0, s, p);
  }
}

template <bool SK>
void launch_mfma_sk(const AttnParams& p, int rows_per_item, int fp8, dim3 grid, hipStream_t s) {
  const dim3 block(64);
  if (fp8 == kFp8E4M3) launch_mfma_fmt<kFp8E4M3, SK>(p, rows_per_item, grid, block, s);
  else if (fp8 == kFp8E5M2) launch_mfma_fmt<kFp8E5M2, SK>(p, rows_per_item, grid, block, s);
  else launch_mfma_fmt<0, SK>(p, rows_per_item, grid, block, s);
}

hipError_t launch_partition_mfma(const AttnParams& p, int rows_per_item, int fp8, hipStream_t s) {
  if (p.sk_meta) {  // stream-K: one workgroup per worker
    if (p.sk_workers <= 0) return hipSuccess;
    launch_mfma_sk<true>(p, rows_per_item, fp8, dim3((unsigned)p.sk_workers), s);
    return hipGetLastError();
  }
  const int R = p.G * p.n_q;
  const int n_rb = (R + rows_per_item - 1) / rows_per_item;
  const long n_wg = xcd_grid(p.B, p.Hkv * n_rb, p.max_parts);
  if (n_wg == 0) return hipSuccess;
  if (n_wg > 0x7fffffffL) return hipErrorInvalidConfiguration;
  launch_mfma_sk<false>(p, rows_per_item, fp8, dim3((unsigned)n_wg), s);
  return hipGetLastError();
}

}  // namespace kvc
