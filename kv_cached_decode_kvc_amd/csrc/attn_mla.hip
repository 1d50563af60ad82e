// attn_mla.hip -- split-KV partition kernel of MLA latent decode.
//
// "Inference-1" (brunomaga.github.io), "Smaller KV caches: MQA, GQA and MLA":
// with the key and value up-projections absorbed into the query and output
// projections, attention runs directly over the cached latent vectors, which
// serve as both keys and values -- one large KV head shared by every query
// head.  "Inference o quy mo lon" (truongducdung.dev), 03 "MLA": each token
// caches d_c + d_h^R = 512 + 64 values (latent, then the decoupled RoPE key).
// A cache row is therefore [latent (512) | rope key (64)]: scores use the
// whole 576-wide row against each head's absorbed query, values are the
// row's first 512 dims, and the output of a (head, row) is the weighted
// latent, combined across partitions by the usual reduce.
//
// Every query row of a sequence (Hq heads x n_q verify rows) reads the same
// latent rows, so a workgroup owns one (sequence, group of rows, partition),
// or with more than 16 rows by default one row group of a stream-K worker's
// run of steps across sequences (the pieces are described at the kernel):
// its threads load each tile of 16 or 32 keys (rows of 1152 bytes, one
// contiguous run per 16 keys) cooperatively into an LDS tile, and its
// wavefronts contract 16-row blocks against it on the matrix cores:
//   S^T = K . Q^T   (the 18 steps of 32 along the 576 dims on
//                    v_mfma_f32_16x16x32_bf16, Q^T in registers, the steps
//                    split between the wavefronts of a row block);
//   O^T += V^T . P^T (column tiles of the 512; V^T via ds_read_b64_tr_b16;
//                     the weights as bf16 hi + lo pairs along the reduction
//                     index, as in the grouped-query kernel).
// Online softmax per row as in the other partition kernels; verify row r
// sees keys 0 .. L - n_q + r.  The workgroup shapes (four wavefronts for up
// to 16 rows, eight for more) are described at the kernel.  Two LDS tiles
// let the score products of tile n + 1 run beside the value products of
// tile n; a ring of PF register stages keeps the following tiles in flight.
// Row groups of the same (sequence, partition), or of the same worker, get
// workgroup ids 8 apart: launches place workgroup i on XCD i mod 8, so they
// share one XCD's L2 and run at the same time.
#include "launch.hpp"

namespace kvc {

namespace {

typedef short i16x4_t __attribute__((__vector_size__(4 * sizeof(short))));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

}  // namespace

// The k-th (sequence, partition) pair in sequence order, where sequence b
// has ceil(L_b / P) partitions, or one if L_b lies outside [n_q, cap] (that
// pair reports the error).  Numbering only the pairs that exist packs the
// live workgroups at the front of the grid: each XCD passes its workgroups
// to its shader engines in turn whatever their load, so live pairs spread
// among dead ones could queue behind each other on one engine while CUs of
// another sat idle.  Computed by every wavefront alike (one pass over the
// lengths, 64 at a time, with a wavefront prefix sum); returns (-1, 0) when
// k is past the last pair.
__device__ __forceinline__ int2 nth_pair(const int32_t* seq_lens, int B, int n_q, int cap, int P,
                                         int k) {
  const int lane = (int)(threadIdx.x & (kWave - 1));
  int before = 0;  // pairs of the chunks already passed
  for (int c = 0; c < B; c += kWave) {
    const int i = c + lane;
    int n = 0;
    if (i < B) {
      const int L = seq_lens[i];
      n = (L < n_q || L > cap) ? 1 : (L + P - 1) / P;
    }
    int incl = n;
    for (int d = 1; d < kWave; d <<= 1) {
      const int t = __shfl_up(incl, d);
      if (lane >= d) incl += t;
    }
    const unsigned long long hit = __ballot(k < before + incl);
    if (hit != 0) {
      const int j = __ffsll((long long)hit) - 1;
      const int excl = before + __shfl(incl - n, j);
      return make_int2(__builtin_amdgcn_readfirstlane(c + j), __builtin_amdgcn_readfirstlane(k - excl));
    }
    before += __shfl(incl, kWave - 1);
  }
  return make_int2(-1, 0);
}

// Workgroup shape: RB row blocks of 16 rows, SP wavefronts per row block
// (RB * SP wavefronts).  Wave w takes row block w % RB and split s = w / RB;
// the SP splits of a row block share its work evenly:
//   scores: split s multiplies each 16-key half of the tile by its share of
//           the absorbed query (KS consecutive steps of the 18 steps of 32
//           along the 576 dims, fewer for the last split when SP does not
//           divide 18), so a wavefront holds 4 * KS query registers; the SP
//           partial 16 x 16 score tiles of a row block meet in LDS, and every
//           split adds all of them in the same order, so all hold the same
//           scores (bit for bit), run the same online softmax and hold the
//           weights and the statistics without sending them;
//   values: split s accumulates 512 / SP of the 512 output columns.
// Each split then reads only its share of the key tile for the scores: the
// tile is read from LDS once per row block for the scores and once for the
// values.  A step covers NH 16-key halves (each with its own block id, so
// block-16 pools work); tile n + 1's partial scores are issued alongside
// tile n's value products, and its softmax follows the barrier that
// publishes them.
//   up to 16 rows (e.g. 16 heads): RB = 1, SP = 4, 16-key steps: four
//     wavefronts, one per SIMD, 128 columns each; several workgroups per CU;
//   more rows (e.g. 128 heads): RB = 4, SP = 2, 32-key steps: eight
//     wavefronts, the two splits of a row block on one SIMD, 256 columns
//     each, so the accumulators (64 registers) and the rest fit the 256
//     vector registers of two wavefronts per SIMD; one workgroup per CU.
// SK: the workgroups are stream-K workers (the pieces are described below),
// else (sequence, partition) pairs; the launch passes sk_meta exactly when SK.
template <int PF, int RB, int SP, int NH, int MINW, bool SK>
__global__ __launch_bounds__((RB * SP * kWave), (MINW)) void partition_mla(AttnParams p) {
  static_assert(PF % 2 == 0, "tile n sits in LDS buffer n % 2");
  static_assert(NH == 1 || NH == 2, "16 or 32 keys per step");
  constexpr int NTH = RB * SP * kWave;    // threads
  constexpr int DK = kMlaKeyDim;          // 576
  constexpr int DV = kMlaValueDim;        // 512
  constexpr int KK = DK / 32;             // 18 QK^T steps
  constexpr int KS = (KK + SP - 1) / SP;  // steps of one split
  constexpr int DT = DV / 16 / SP;        // output column tiles of one split
  constexpr int TK = NH * kTile;          // keys per step
  constexpr int CPR = DK * 2 / 16;        // 72 16-byte chunks per row
  constexpr int TCH = TK * CPR;           // chunks per tile
  constexpr int PER = (TCH + NTH - 1) / NTH;  // chunks per thread
  constexpr int ROWB = DK * 2 + 16;       // padded LDS row
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][TK * ROWB];
  // partial scores: [row block][split][16-key half]
  __shared__ __attribute__((aligned(16))) f32x4_t s_ps[RB][SP][NH][kWave];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // a scalar: the split's step count below decides whole-wavefront branches
  // around matrix-core instructions, which do not honour the lane mask
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int rbw = wave % RB;  // row block of the workgroup
  const int sp = wave / RB;   // split: share of the score reduction and of the columns
  const int k_lo = sp * KS;   // first QK^T step of this split
  const int nk = KK % SP == 0 ? KS : min(KS, KK - k_lo);  // its steps

  const int R = p.Hq * p.n_q;                 // rows sharing the latent cache
  constexpr int rows_wg = 16 * RB;
  const int n_rg = (R + rows_wg - 1) / rows_wg;
  // workgroup id = (chunk * n_rg + rg) * 8 + j: unit = chunk * 8 + j (a
  // (sequence, partition) pair, or a stream-K worker), so the row groups of
  // a unit sit 8 ids apart on one XCD and share its tiles through one L2
  const long wg = blockIdx.x;
  const int rg = (int)((wg / 8) % n_rg);
  const long unit = (wg / (8L * n_rg)) * 8 + (wg % 8);

  __shared__ int s_blk[kMlaMaxTiles];

  // One piece of work: the steps start, start + stride, ... below end (keys)
  // of sequence b (L keys attended).  Its partials go, stream-K, to
  // workspace row slot + i (i = r * Hq + h, the row within the sequence's R
  // rows), else to row ((b * Hq + h) * n_q + r) * max_parts + slot (slot:
  // the partition).  Every wavefront of the workgroup runs every piece (the
  // barriers inside count all of them).
  auto run_piece = [&](int b, int L, int start, int stride, int end, long slot) {
  // this wavefront's rows: i = r * Hq + h
  const int i_row = (rg * RB + rbw) * 16 + col;
  const bool rvalid = i_row < R;
  const int r_q = rvalid ? i_row / p.Hq : 0;
  const int h_q = rvalid ? i_row % p.Hq : 0;
  const bool active = __any(rvalid);  // wave-uniform: the row block has rows
  const int lvis = rvalid ? L - p.n_q + r_q + 1 : L;
  const long orow = SK ? slot + i_row
                       : (((long)b * p.Hq + h_q) * p.n_q + r_q) * p.max_parts + slot;

  bf16x8_t qf[KS];  // this split's steps of the absorbed queries (B operand of S^T)
  {
    const uint16_t* qrow = (const uint16_t*)p.q + (((long)b * p.n_q + r_q) * p.Hq + h_q) * DK;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (rvalid && k < nk) w = *reinterpret_cast<const uint4*>(qrow + (k_lo + k) * 32 + grp * 8);
      qf[k] = __builtin_bit_cast(bf16x8_t, w);
    }
  }

  f32x4_t oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;  // running statistics of row col (the same in every split)

  // The block ids of each 16-key half of the partition's tiles, staged in
  // LDS once: read from global memory inside the loop they would be the
  // newest load in flight, and waiting for one would wait for every tile
  // load behind it.
  const int n_tiles = (end - start + stride - 1) / stride;  // NH * n_tiles <= kMlaMaxTiles (plan)
  const int bs_shift = __builtin_ctz((unsigned)(p.bs > 0 ? p.bs : 1));
  if constexpr (SK) __syncthreads();  // the previous piece's reads of s_blk, the tiles and s_ps are done
  if (p.table != nullptr) {
    for (int x = tid; x < NH * n_tiles; x += NTH) {
      const int key = start + (x / NH) * stride + (x % NH) * kTile;
      s_blk[x] = key < end ? p.table[(long)b * p.max_blocks + (key >> bs_shift)] : 0;
    }
  }
  __syncthreads();
  // element offset of key `key` (a multiple of 16) whose half is s_blk[x]; -1: bad block.
  // A scalar, like everything that decides a branch around matrix-core work.
  auto half_base = [&](int key, int x) -> long {
    if (p.table == nullptr) return ((long)b * p.S_max + key) * DK;
    const int blk = __builtin_amdgcn_readfirstlane(s_blk[x]);
    if (blk < 0 || blk >= p.N) return -1;
    return ((long)blk * p.bs + (key & (p.bs - 1))) * DK;
  };
  // this thread's chunks of a tile: row and byte offset within the row
  int frow[PER];
  uint32_t fchk[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int idx = min(u * NTH + tid, TCH - 1);  // extra threads repeat the last chunk
    frow[u] = idx / CPR;
    fchk[u] = (uint32_t)(idx % CPR) * 16;
  }
  uint4 stage[PF][PER];  // ring of register stages
  bool sok[PF];          // the stage's tile is in the partition and its blocks are valid
  // Every stage issues exactly PER loads, whatever the tile (past the end of
  // the partition, a bad block, threads beyond the tile's chunks): rows are
  // clamped to visible ones instead of branching, so the compiler can wait
  // for one stage's loads alone and the ring keeps PF - 1 tiles in flight.
  // Past the end (or with a bad block) every row is the cache's first row:
  // one row's worth of lines, so the padding steps cost no HBM traffic.
  auto fetch = [&](uint4 (&st)[PER], bool& ok, int n) {
    const int tile = start + n * stride;
    const bool in = tile < end;
    const long b0 = in ? half_base(tile, NH * n) : 0;
    // the second half's block (the first one's when the half lies past the end)
    const long b1 = NH == 2 && in && tile + kTile < end ? half_base(tile + kTile, NH * n + 1) : b0;
    ok = in && b0 >= 0 && b1 >= 0;
    const int last = ok ? min(TK, end - tile) - 1 : 0;
    const long c0 = ok ? b0 : 0, c1 = ok ? b1 - (long)kTile * DK : 0;
#pragma unroll
    for (int u = 0; u < PER; ++u) {  // masked keys re-read a visible row
      const int row = min(frow[u], last);
      const long c = NH == 2 && row >= kTile ? c1 : c0;
      st[u] = load_stream((const uint8_t*)p.k + (c + (long)row * DK) * 2 + fchk[u]);
    }
  };
  auto store_tile = [&](int buf, const uint4 (&st)[PER]) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int idx = u * NTH + tid;
      if (idx < TCH)
        *reinterpret_cast<uint4*>(lds[buf] + (idx / CPR) * ROWB + (idx % CPR) * 16) = st[u];
    }
  };
  constexpr float kLazy = 8.f;
  // this split's partial S^T of the tile in `buf`, every 16-key half (lane:
  // keys kh*16 + grp*4 .. +3 of row col), published in s_ps
  auto qk_part = [&](int buf) {
#pragma unroll
    for (int kh = 0; kh < NH; ++kh) {
      const uint8_t* ka = lds[buf] + (kh * kTile + col) * ROWB + grp * 16 + k_lo * 64;
      f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
      bf16x8_t kf[KS];
#pragma unroll
      for (int k = 0; k < KS; ++k)
        if (k < nk) kf[k] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(ka + k * 64));
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        if (k >= nk) break;
        if (k & 1) s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[k], qf[k], s1, 0, 0, 0);
        else s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[k], qf[k], s0, 0, 0, 0);
      }
      s_ps[rbw][sp][kh][lane] = s0 + s1;
    }
  };
  // the whole scores of the tile (the splits' parts added in split order),
  // one online-softmax step over its TK keys: the weights of each 16-key half
  // (bf16 hi + lo) and the factor the accumulators must be rescaled by;
  // rescale is wave-uniform
  float alpha = 1.f;
  bool rescale = false;
  bf16x8_t pb[NH] = {};
  auto softmax = [&](int tile, bool ok) {
    float sv[NH][4];
#pragma unroll
    for (int kh = 0; kh < NH; ++kh) {
      f32x4_t s = s_ps[rbw][0][kh][lane];
#pragma unroll
      for (int x = 1; x < SP; ++x) s += s_ps[rbw][x][kh][lane];
      const int key0 = tile + kh * kTile + grp * 4;
#pragma unroll
      for (int v = 0; v < 4; ++v)
        sv[kh][v] = ok && key0 + v < lvis ? s[v] * p.scale_log2 : -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kh = 0; kh < NH; ++kh)
      mx = fmaxf(mx, fmaxf(fmaxf(sv[kh][0], sv[kh][1]), fmaxf(sv[kh][2], sv[kh][3])));
    mx = rows_max(mx);
    const bool move = mx > m + kLazy;
    rescale = __any(move);
    const float m_new = move ? mx : m;
    alpha = m == -INFINITY ? 0.f : fast_exp2(m - m_new);
    m = m_new;
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    float lsum = 0.f;
#pragma unroll
    for (int kh = 0; kh < NH; ++kh) {
      const f32x2_t p01 = {fast_exp2(sv[kh][0] - m_use), fast_exp2(sv[kh][1] - m_use)};
      const f32x2_t p23 = {fast_exp2(sv[kh][2] - m_use), fast_exp2(sv[kh][3] - m_use)};
      lsum += (p01[0] + p01[1]) + (p23[0] + p23[1]);
      const bf16x2_t h01 = __builtin_convertvector(p01, bf16x2_t);
      const bf16x2_t h23 = __builtin_convertvector(p23, bf16x2_t);
      const bf16x2_t lo01 = __builtin_convertvector(p01 - __builtin_convertvector(h01, f32x2_t), bf16x2_t);
      const bf16x2_t lo23 = __builtin_convertvector(p23 - __builtin_convertvector(h23, f32x2_t), bf16x2_t);
      pb[kh] = __builtin_shufflevector(__builtin_shufflevector(h01, h23, 0, 1, 2, 3),
                                       __builtin_shufflevector(lo01, lo23, 0, 1, 2, 3),
                                       0, 1, 2, 3, 4, 5, 6, 7);
    }
    l = l * alpha + lsum;
  };
  // O^T += V^T . P^T over this split's columns, one 16-key half at a time
  auto pv = [&](int buf) {
#pragma unroll
    for (int kh = 0; kh < NH; ++kh) {
      const uint8_t* va_ptr = lds[buf] + (kh * kTile + grp * 4 + (col >> 2)) * ROWB +
                              (col & 3) * 8 + sp * (DV / SP) * 2;
      constexpr int VG = DT < 8 ? DT : 8;
      auto read_v = [&](bf16x4_t (&va)[VG], int g) {
#pragma unroll
        for (int i = 0; i < VG; ++i) {
          lds_i16x4_t* a = reinterpret_cast<lds_i16x4_t*>(
              (__attribute__((address_space(3))) uint8_t*)(va_ptr + (g * VG + i) * 32));
          va[i] = __builtin_bit_cast(bf16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(a));
        }
      };
      bf16x4_t vcur[VG], vnext[VG];
      read_v(vcur, 0);
#pragma unroll
      for (int g = 0; g < DT / VG; ++g) {
        if (g + 1 < DT / VG) read_v(vnext, g + 1);
#pragma unroll
        for (int i = 0; i < VG; ++i) {
          const bf16x8_t va2 = __builtin_shufflevector(vcur[i], vcur[i], 0, 1, 2, 3, 0, 1, 2, 3);
          oacc[g * VG + i] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(va2, pb[kh], oacc[g * VG + i], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < VG; ++i) vcur[i] = vnext[i];
      }
    }
  };

  // prologue: tiles 0 and 1 in LDS, tiles 2 .. PF + 1 in flight; tile 0's
  // weights in registers
#pragma unroll
  for (int k = 0; k < PF; ++k) fetch(stage[k], sok[k], k);
  store_tile(0, stage[0]);
  store_tile(1, stage[1]);
  bool bok[2] = {sok[0], sok[1]};
  __syncthreads();
  fetch(stage[0], sok[0], PF);
  fetch(stage[1], sok[1], PF + 1);
  if (active) qk_part(0);
  __syncthreads();
  if (active) softmax(start, bok[0]);
  __syncthreads();  // s_ps read: the first step publishes tile 1's partial scores there
  for (int n0 = 0; n0 < n_tiles; n0 += PF) {
#pragma unroll
    for (int jj = 0; jj < PF; ++jj) {  // tile n in buffer j, tile n + 1 in buffer 1 - j
      const int n = n0 + jj;
      const int j = jj & 1;
      const int sg = (jj + 2) % PF;  // the stage holding tile n + 2
      const bool more = n + 1 < n_tiles;
      if (n < n_tiles) {
        if (active) {
          if (more) qk_part(1 - j);  // tile n + 1's partial scores
          if (rescale) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
          }
          if (bok[j]) pv(j);  // a bad block's tile holds no usable rows
        }
        if (!bok[j] && tid == 0) report(p.status, KVC_ERR_DATA);
      }
      __syncthreads();  // partial scores of tile n + 1 published; buffer j read
      if (n < n_tiles && more && active) softmax(start + (n + 1) * stride, bok[1 - j]);
      store_tile(j, stage[sg]);  // tile n + 2
      bok[j] = sok[sg];
      fetch(stage[sg], sok[sg], n + 2 + PF);
      __syncthreads();  // tile n + 2 stored; s_ps read
    }
  }

  float lt = l + __shfl_xor(l, 16);
  lt += __shfl_xor(lt, 32);
  if (rvalid) {
    float* wo = p.ws_o + orow * DV + sp * (DV / SP);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<f32x4_t*>(wo + dt * 16 + grp * 4) = oacc[dt];
    if (sp == 0 && grp == 0) {  // every split holds the same statistics
      float* wml = p.ws_ml + orow * 2;
      wml[0] = m;
      wml[1] = lt;
    }
  }
  };  // run_piece

  // The pieces of this workgroup (one call site of run_piece in each form:
  // the piece's code is large).
  //   fixed partitions: the unit-th live (sequence, partition) pair;
  //   partition part of n owns the steps part, part + n, ...;
  //   stream-K: the lengths give T_b = ceil(L_b / TK) steps per sequence (0
  //   for an invalid length, which worker 0 reports), W in all; worker w of
  //   NW takes the steps [w W / NW, (w + 1) W / NW), a contiguous run that
  //   may end one sequence and start the next, and every row group of the
  //   worker takes the same run.  The piece (sequence b, worker w) leaves
  //   its rows' partials at workspace rows (b + w) * R + i (unique: b and w
  //   both grow along the runs); the worker holding a sequence's first step
  //   records which workers cover it.
  if constexpr (!SK) {
    if (unit >= (long)p.B * p.max_parts) return;
    const int P = part_tokens(p.seq_lens, p.B, p.cap, p.slots_u, p.P_lo, p.P);
    const int2 bp = nth_pair(p.seq_lens, p.B, p.n_q, p.cap, P, (int)unit);
    if (bp.x < 0) return;  // past the last live pair: whole workgroup
    const int b = bp.x, part = bp.y;
    const int L = __builtin_amdgcn_readfirstlane(p.seq_lens[b]);
    if (L < p.n_q || L > p.cap) {
      if (rg == 0 && tid == 0) report(p.status, KVC_ERR_DATA);
      return;  // whole workgroup
    }
    const int nparts = (L + P - 1) / P;
    run_piece(b, L, part * TK, nparts * TK, L, part);
  } else {
    if (unit >= p.sk_workers) return;
    long W = 0;
    int bad = 0;
    for (int first = 0; first < p.B; first += kWave) {
      const int i = first + lane;
      int t = 0;
      if (i < p.B) {
        const int Li = p.seq_lens[i];
        if (Li >= p.n_q && Li <= p.cap) t = (Li + TK - 1) / TK;
        else bad = 1;
      }
      for (int mm = 1; mm < kWave; mm <<= 1) t += __shfl_xor(t, mm);
      W += t;
    }
    if (unit == 0 && rg == 0 && __any(bad) && tid == 0) report(p.status, KVC_ERR_DATA);
    W = __builtin_amdgcn_readfirstlane((int)W);
    if (W == 0) return;
    const long NW = min((long)p.sk_workers, max(1L, W / p.sk_min_tiles));
    if (unit >= NW) return;
    long pos = unit * W / NW;
    const long s1 = (unit + 1) * W / NW;
    if (pos >= s1) return;
    // the sequence holding step pos: the first b with (steps before b + its steps) > pos
    int b = 0;
    long pre = 0;  // steps before sequence b
    for (int first = 0; first < p.B; first += kWave) {
      const int i = first + lane;
      long n = 0;
      if (i < p.B) {
        const int Li = p.seq_lens[i];
        if (Li >= p.n_q && Li <= p.cap) n = (Li + TK - 1) / TK;
      }
      long incl = n;
      for (int d = 1; d < kWave; d <<= 1) {
        const long t = __shfl_up(incl, d);
        if (lane >= d) incl += t;
      }
      const unsigned long long hit = __ballot(pos < pre + incl);
      if (hit != 0) {
        const int j = __ffsll((long long)hit) - 1;
        b = first + j;
        pre += __shfl(incl - n, j);
        break;
      }
      pre += __shfl(incl, kWave - 1);
    }
    b = __builtin_amdgcn_readfirstlane(b);
    pre = __builtin_amdgcn_readfirstlane((int)pre);
    int L = __builtin_amdgcn_readfirstlane(p.seq_lens[b]);
    int T = (L + TK - 1) / TK;  // >= 1: sequence b holds step pos
    while (pos < s1) {
      while (pos >= pre + T) {  // past sequence b: the next one with steps
        pre += T;
        ++b;
        L = __builtin_amdgcn_readfirstlane(p.seq_lens[b]);
        T = (L >= p.n_q && L <= p.cap) ? (L + TK - 1) / TK : 0;
      }
      const int t0 = (int)(pos - pre);
      const int t1 = (int)min((long)T, t0 + (s1 - pos));
      if (t0 == 0 && rg == 0 && tid == 0) {  // this worker starts the sequence: record its workers
        const long x_last = pre + T - 1;
        const int w_last = (int)(((x_last + 1) * NW - 1) / W);
        p.sk_meta[b] = make_int2((int)unit, w_last);
      }
      run_piece(b, L, t0 * TK, TK, min(t1 * TK, L), (long)(b + unit) * R);
      pos += t1 - t0;
    }
  }
}

// Up to 16 rows: one row block, four splits, 16-key steps, kSmallWgs
// workgroups per CU.  More rows: four row blocks of two splits, 32-key steps,
// one workgroup per CU.
constexpr int kSmallWgs = 2;
constexpr int kSmallPF = 2;

int mla_rows_per_wg(int rows) { return rows <= 16 ? 16 : 64; }
int mla_wgs_per_cu(int rows) { return rows <= 16 ? kSmallWgs : 1; }

hipError_t launch_partition_mla(const AttnParams& p, hipStream_t s) {
  const int R = p.Hq * p.n_q;
  const long rows_wg = mla_rows_per_wg(R);
  const long n_rg = (R + rows_wg - 1) / rows_wg;
  const long units = p.sk_meta ? (long)p.sk_workers : (long)p.B * p.max_parts;
  const long n_wg = (units + 7) / 8 * 8 * n_rg;
  if (units == 0) return hipSuccess;
  if (n_wg > 0x7fffffffL) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)n_wg);
  if (R <= 16) {
    if (p.sk_meta) return hipErrorInvalidValue;  // the 16-row form has fixed partitions only
    hipLaunchKernelGGL((partition_mla<kSmallPF, 1, 4, 1, kSmallWgs, false>), grid, dim3(4 * kWave), 0, s, p);
  } else if (p.sk_meta) {
    hipLaunchKernelGGL((partition_mla<2, 4, 2, 2, 1, true>), grid, dim3(8 * kWave), 0, s, p);
  } else {
    hipLaunchKernelGGL((partition_mla<2, 4, 2, 2, 1, false>), grid, dim3(8 * kWave), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace kvc
