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
// latent rows, so a workgroup owns one (sequence, group of rows, partition):
// its threads load each 16-key tile (16 x 1152 bytes, one contiguous run)
// cooperatively into one LDS tile, and its wavefronts contract 16-row blocks
// against it on the matrix cores:
//   S^T = K . Q^T   (18 steps of v_mfma_f32_16x16x32_bf16, Q^T in registers)
//   O^T += V^T . P^T (column tiles of the 512; V^T via ds_read_b64_tr_b16;
//                     the weights as bf16 hi + lo pairs along the reduction
//                     index, as in the grouped-query kernel).
// Online softmax per row as in the other partition kernels; verify row r
// sees keys 0 .. L - n_q + r.
//
// Two forms.  Up to 16 rows (e.g. 16 heads, partition_mla with C = 4): four
// wavefronts share the one row block, each computes its scores and softmax
// itself and accumulates 128 of the 512 columns.  More rows (e.g. 128 heads,
// partition_mla_pair): eight wavefronts, two per SIMD, cover four row blocks;
// the two wavefronts of a row block split the columns, and one of them
// computes the block's scores and softmax and passes the weights to the
// other through LDS.  Two LDS tiles let the score products of tile n + 1 run
// beside the value products of tile n; a ring of PF register stages keeps
// the following tiles in flight.  Row groups of the same (sequence,
// partition) get workgroup ids 8 apart: launches place workgroup i on XCD i
// mod 8, so they share one XCD's L2 and run at the same time, and the tile
// comes from HBM once.
#include "launch.hpp"

namespace kvc {

namespace {

typedef short i16x4_t __attribute__((__vector_size__(4 * sizeof(short))));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr int kMlaWaves = 4;
constexpr int kMlaMaxTiles = 1024;  // tiles of one partition: partition length <= 16384
constexpr int kMlaThreads = kMlaWaves * kWave;

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

template <int PF, int C>
__global__ __launch_bounds__(kMlaThreads, C == 1 ? 1 : 2) void partition_mla(AttnParams p) {
  constexpr int NT = 1;
  constexpr int DK = kMlaKeyDim;          // 576
  constexpr int DV = kMlaValueDim;        // 512
  constexpr int KK = DK / 32;             // 18 QK^T steps
  constexpr int DT = DV / 16 / C;         // output column tiles of one wavefront
  constexpr int RB = kMlaWaves / C;       // row blocks of a workgroup
  constexpr int CPR = DK * 2 / 16;        // 72 16-byte chunks per row
  constexpr int TCH = kTile * CPR;        // 1152 chunks per tile
  constexpr int PER = (TCH + kMlaThreads - 1) / kMlaThreads;  // chunks per thread
  constexpr int ROWB = DK * 2 + 16;       // padded LDS row
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][kTile * ROWB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;

  const int R = p.Hq * p.n_q;                 // rows sharing the latent cache
  const int rows_wg = 16 * NT * RB;
  const int cc = wave % C;                    // this wavefront's column chunk
  const int n_rg = (R + rows_wg - 1) / rows_wg;
  // workgroup id = (chunk * n_rg + rg) * 8 + j: unit (sequence, partition)
  // = chunk * 8 + j, so its row groups sit 8 ids apart on one XCD
  const long wg = blockIdx.x;
  const int rg = (int)((wg / 8) % n_rg);
  const long unit = (wg / (8L * n_rg)) * 8 + (wg % 8);  // the unit-th live pair
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
  const int start = part * kTile, stride = nparts * kTile, end = L;

  // this wavefront's rows: i = r * Hq + h
  int lvis[NT];
  bool rvalid[NT];
  long qoff[NT], wrow[NT];
  bool any_row = false;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int i = (rg * RB + wave / C) * 16 * NT + nt * 16 + col;
    rvalid[nt] = i < R;
    const int r = rvalid[nt] ? i / p.Hq : 0;
    const int h = rvalid[nt] ? i % p.Hq : 0;
    lvis[nt] = rvalid[nt] ? L - p.n_q + r + 1 : L;
    qoff[nt] = (((long)b * p.n_q + r) * p.Hq + h) * DK;
    wrow[nt] = ((long)b * p.Hq + h) * p.n_q + r;
    any_row |= rvalid[nt];
  }
  const bool active = __any(any_row);  // wave-uniform: this wavefront has rows

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

  // The block ids of the partition's tiles, staged in LDS once: read from
  // global memory inside the loop they would be the newest load in flight,
  // and waiting for one would wait for every tile load behind it.
  const int n_tiles = (end - start + stride - 1) / stride;  // <= kMlaMaxTiles (plan)
  const int bs_shift = __builtin_ctz((unsigned)(p.bs > 0 ? p.bs : 1));
  __shared__ int s_blk[kMlaMaxTiles];
  if (p.table != nullptr) {
    for (int n = tid; n < n_tiles; n += kMlaThreads)
      s_blk[n] = p.table[(long)b * p.max_blocks + ((start + n * stride) >> bs_shift)];
  }
  __syncthreads();
  auto tile_base = [&](int n) -> long {  // element offset of tile n's first key; -1: bad block
    const int tile = start + n * stride;
    if (p.table == nullptr) return ((long)b * p.S_max + tile) * DK;
    const int blk = s_blk[n];
    if (blk < 0 || blk >= p.N) return -1;
    return ((long)blk * p.bs + (tile & (p.bs - 1))) * DK;
  };
  // this thread's chunks of a tile: row and byte offset within the row
  int frow[PER];
  uint32_t fchk[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int idx = min(u * kMlaThreads + tid, TCH - 1);  // extra threads repeat the last chunk
    frow[u] = idx / CPR;
    fchk[u] = (uint32_t)(idx % CPR) * 16;
  }
  uint4 stage[PF][PER];  // ring of register stages
  long stb[PF];          // tile base of each stage (-1: none or bad block)
  // Every stage issues exactly PER loads, whatever the tile (past the end of
  // the partition, a bad block, threads beyond the tile's chunks): addresses
  // are clamped to valid rows instead of branching, so the compiler can wait
  // for one stage's loads alone and the ring keeps PF - 1 tiles in flight.
  auto fetch = [&](uint4 (&st)[PER], long& tbs, int n) {
    const int tile = start + n * stride;
    const bool in = tile < end;
    const long tb = tile_base(in ? n : 0);
    tbs = in ? tb : -1;
    // past the end (or a bad block) the rows clamp to the cache's first row:
    // one row's worth of lines, so the padding steps cost no HBM traffic
    const uint8_t* base = (const uint8_t*)p.k + (tbs >= 0 ? tb : 0) * 2;
    const int last = tbs >= 0 ? min(kTile, end - tile) - 1 : 0;
#pragma unroll
    for (int u = 0; u < PER; ++u)  // masked keys re-read a visible row
      st[u] = load_stream(base + ((uint32_t)min(frow[u], last) * (DK * 2) + fchk[u]));
  };
  auto store_tile = [&](int buf, const uint4 (&st)[PER]) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int idx = u * kMlaThreads + tid;
      if (idx < TCH)
        *reinterpret_cast<uint4*>(lds[buf] + (idx / CPR) * ROWB + (idx % CPR) * 16) = st[u];
    }
  };
  // tile n of the partition is start + n * stride; it lives in stage n % PF
  // Two LDS tiles: while tile n's softmax runs on the vector ALUs, tile
  // n + 1's score products run on the matrix cores (they do not depend on
  // each other), then tile n's value products follow.
  constexpr float kLazy = 8.f;
  auto qk = [&](int buf) -> f32x4_t {  // S^T of the tile in `buf`: this lane's 4 keys of row col
    const uint8_t* ka = lds[buf] + col * ROWB + grp * 16;
    constexpr int KG = 6;  // K fragments read per batch (registers)
    f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};  // two chains
#pragma unroll
    for (int k0 = 0; k0 < KK; k0 += KG) {
      bf16x8_t kf[KG];
#pragma unroll
      for (int kk = 0; kk < KG; ++kk)
        kf[kk] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(ka + (k0 + kk) * 64));
#pragma unroll
      for (int kk = 0; kk < KG; kk += 2) {
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kk], qf[0][k0 + kk], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kk + 1], qf[0][k0 + kk + 1], s1, 0, 0, 0);
      }
    }
    return s0 + s1;
  };
  // online softmax of one tile, branch free; returns the weights (bf16 hi +
  // lo) and the factor the accumulators must be rescaled by (1: none)
  float alpha = 1.f;
  bool rescale = false;
  auto softmax = [&](const f32x4_t& s, int tile, bool ok) -> bf16x8_t {
    const int key0 = tile + grp * 4;
    float sv[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) sv[v] = ok && key0 + v < lvis[0] ? s[v] * p.scale_log2 : -INFINITY;
    float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const bool move = mx > m[0] + kLazy;
    rescale = __any(move);
    const float m_new = move ? mx : m[0];
    alpha = m[0] == -INFINITY ? 0.f : fast_exp2(m[0] - m_new);
    m[0] = m_new;
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const f32x2_t p01 = {fast_exp2(sv[0] - m_use), fast_exp2(sv[1] - m_use)};
    const f32x2_t p23 = {fast_exp2(sv[2] - m_use), fast_exp2(sv[3] - m_use)};
    l[0] = l[0] * alpha + ((p01[0] + p01[1]) + (p23[0] + p23[1]));
    const bf16x2_t h01 = __builtin_convertvector(p01, bf16x2_t);
    const bf16x2_t h23 = __builtin_convertvector(p23, bf16x2_t);
    const bf16x2_t lo01 = __builtin_convertvector(p01 - __builtin_convertvector(h01, f32x2_t), bf16x2_t);
    const bf16x2_t lo23 = __builtin_convertvector(p23 - __builtin_convertvector(h23, f32x2_t), bf16x2_t);
    return __builtin_shufflevector(__builtin_shufflevector(h01, h23, 0, 1, 2, 3),
                                   __builtin_shufflevector(lo01, lo23, 0, 1, 2, 3),
                                   0, 1, 2, 3, 4, 5, 6, 7);
  };
  auto pv = [&](int buf, const bf16x8_t& pb) {  // O^T += V^T . P^T, value fragments in groups
    const uint8_t* va_ptr =
        lds[buf] + (grp * 4 + (col >> 2)) * ROWB + (col & 3) * 8 + cc * (DV / C) * 2;
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
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < VG; ++i) {
        const bf16x8_t va2 = __builtin_shufflevector(vcur[i], vcur[i], 0, 1, 2, 3, 0, 1, 2, 3);
        oacc[0][g * VG + i] =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(va2, pb, oacc[0][g * VG + i], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < VG; ++i) vcur[i] = vnext[i];
    }
  };

  // prologue: tiles 0 and 1 in LDS, tiles 2 .. PF + 1 in flight, scores of
  // tile 0.  Stage (n + 2) % PF holds tile n + 2 until step n stores it into
  // LDS buffer n % 2, then takes tile n + 2 + PF.
#pragma unroll
  for (int k = 0; k < PF; ++k) fetch(stage[k], stb[k], k);
  store_tile(0, stage[0]);
  store_tile(1, stage[1]);
  bool bok[2] = {stb[0] >= 0, stb[1] >= 0};
  __syncthreads();
  fetch(stage[0], stb[0], PF);
  fetch(stage[1], stb[1], PF + 1);
  f32x4_t s_cur = {0.f, 0.f, 0.f, 0.f};
  if (active) s_cur = qk(0);
  for (int n0 = 0; n0 < n_tiles; n0 += PF) {
#pragma unroll
    for (int jj = 0; jj < PF; ++jj) {  // tile n in buffer j, tile n + 1 in buffer 1 - j
      const int n = n0 + jj;
      const int j = jj & 1;
      const int sg = (jj + 2) % PF;  // the stage holding tile n + 2
      f32x4_t s_next = {0.f, 0.f, 0.f, 0.f};
      if (n < n_tiles) {
        if (active) {
          s_next = qk(1 - j);  // tile n + 1 (results unused past the end)
          const bf16x8_t pb = softmax(s_cur, start + n * stride, bok[j]);
          if (__builtin_expect(rescale, 0)) {
            // The empty asm statements hand the accumulators to the vector
            // ALUs only inside this rare branch; without them the 512-column
            // form (C = 1) copies them between register files on every tile
            // and spills to scratch.
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
              asm volatile("" : "+v"(oacc[0][dt]));
              oacc[0][dt] *= alpha;
              asm volatile("" : "+v"(oacc[0][dt]));
            }
          }
          if (bok[j]) pv(j, pb);  // a bad block's tile holds no usable rows
        }
        if (!bok[j] && tid == 0) report(p.status, KVC_ERR_DATA);
      }
      __syncthreads();  // every wavefront is done with buffer j
      store_tile(j, stage[sg]);  // tile n + 2
      bok[j] = stb[sg] >= 0;
      fetch(stage[sg], stb[sg], n + 2 + PF);
      __syncthreads();
      s_cur = s_next;
    }
  }

#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float lt = l[nt] + __shfl_xor(l[nt], 16);
    lt += __shfl_xor(lt, 32);
    if (!rvalid[nt]) continue;
    float* wo = p.ws_o + (wrow[nt] * p.max_parts + part) * DV + cc * (DV / C);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<f32x4_t*>(wo + dt * 16 + grp * 4) = oacc[nt][dt];
    if (grp == 0 && cc == 0) {  // every column chunk holds the same statistics
      float* wml = p.ws_ml + (wrow[nt] * p.max_parts + part) * 2;
      wml[0] = m[nt];
      wml[1] = lt;
    }
  }
}

// More than 16 rows (e.g. 128 heads): a workgroup of eight wavefronts, two
// per SIMD, covers 64 rows (four 16-row blocks) and all 512 columns.  Wave w
// takes row block w % 4 and half w / 4; the two halves of a row block share
// a SIMD and split the work evenly:
//   scores: each half multiplies the tile by its half of the absorbed query
//           (9 of the 18 steps of 32 along the 576 dims, so a wavefront holds
//           36 query registers), the two 16 x 16 partial sums of each 16-key
//           half meet in LDS, and each half adds them (the same sum in both:
//           a + b = b + a) and runs the same online softmax, so both hold the
//           weights and the statistics without sending them;
//   values: each half accumulates 256 of the 512 output columns.
// A wavefront's accumulators (64 registers) and its other state then fit the
// 256 vector registers of two wavefronts per SIMD.  (The one-wavefront form
// held 16 rows x 512 columns in the accumulation registers, where the
// compiler moved them on every tile, and left a lone wavefront per SIMD to
// hide every latency.)  A step covers 32 keys (two 16-key halves, each with
// its own block id), so the two barriers of a step serve twice the keys of a
// 16-key tile; tile n + 1's partial scores are issued alongside tile n's
// value products, and its softmax follows the barrier that publishes them.
constexpr int kPairWaves = 8;
constexpr int kPairThreads = kPairWaves * kWave;

template <int PF>
__global__ __launch_bounds__(kPairThreads, 1) void partition_mla_pair(AttnParams p) {
  static_assert(PF % 2 == 0, "tile n sits in LDS buffer n % 2");
  constexpr int DK = kMlaKeyDim;          // 576
  constexpr int DV = kMlaValueDim;        // 512
  constexpr int KK = DK / 32;             // 18 QK^T steps
  constexpr int KH = KK / 2;              // 9 steps per half
  constexpr int DT = DV / 16 / 2;         // 16 output column tiles per half
  constexpr int TK = 2 * kTile;           // 32 keys per tile: two 16-key halves
  constexpr int CPR = DK * 2 / 16;        // 72 16-byte chunks per row
  constexpr int TCH = TK * CPR;           // 2304 chunks per tile
  constexpr int PER = (TCH + kPairThreads - 1) / kPairThreads;  // chunks per thread
  constexpr int ROWB = DK * 2 + 16;       // padded LDS row
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][TK * ROWB];
  // partial scores: [slot][row block][half of the reduction][16-key half]
  __shared__ __attribute__((aligned(16))) f32x4_t s_ps[2][4][2][2][kWave];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int rbw = wave & 3;    // row block of the workgroup
  const int half = wave >> 2;  // column half, and half of the score reduction

  const int R = p.Hq * p.n_q;
  constexpr int rows_wg = 64;
  const int n_rg = (R + rows_wg - 1) / rows_wg;
  const long wg = blockIdx.x;
  const int rg = (int)((wg / 8) % n_rg);
  const long unit = (wg / (8L * n_rg)) * 8 + (wg % 8);  // the unit-th live pair
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
  // partition part of n owns the 32-key tiles part, part + n, ...
  const int nparts = (L + P - 1) / P;
  const int start = part * TK, stride = nparts * TK, end = L;

  // this wavefront's rows: i = r * Hq + h
  const int i_row = (rg * 4 + rbw) * 16 + col;
  const bool rvalid = i_row < R;
  const int r_q = rvalid ? i_row / p.Hq : 0;
  const int h_q = rvalid ? i_row % p.Hq : 0;
  const int lvis = rvalid ? L - p.n_q + r_q + 1 : L;
  const long wrow = ((long)b * p.Hq + h_q) * p.n_q + r_q;
  const bool active = __any(rvalid);  // wave-uniform: the row block has rows

  bf16x8_t qf[KH];  // this half's steps of the absorbed queries (B operand of S^T)
  {
    const uint16_t* qrow = (const uint16_t*)p.q + (((long)b * p.n_q + r_q) * p.Hq + h_q) * DK;
#pragma unroll
    for (int k = 0; k < KH; ++k) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (rvalid) w = *reinterpret_cast<const uint4*>(qrow + (half * KH + k) * 32 + grp * 8);
      qf[k] = __builtin_bit_cast(bf16x8_t, w);
    }
  }

  f32x4_t oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;  // running statistics of row col (the same in both halves)

  const int n_tiles = (end - start + stride - 1) / stride;  // 2 * n_tiles <= kMlaMaxTiles (plan)
  const int bs_shift = __builtin_ctz((unsigned)(p.bs > 0 ? p.bs : 1));
  // block ids of each 16-key half of the partition's tiles (a 32-key tile
  // may span two blocks of 16)
  __shared__ int s_blk[kMlaMaxTiles];
  if (p.table != nullptr) {
    for (int x = tid; x < 2 * n_tiles; x += kPairThreads) {
      const int key = start + (x >> 1) * stride + (x & 1) * kTile;
      s_blk[x] = key < end ? p.table[(long)b * p.max_blocks + (key >> bs_shift)] : 0;
    }
  }
  __syncthreads();
  // element offset of key `key` (a multiple of 16) whose half is s_blk[x]; -1: bad block
  auto half_base = [&](int key, int x) -> long {
    if (p.table == nullptr) return ((long)b * p.S_max + key) * DK;
    const int blk = s_blk[x];
    if (blk < 0 || blk >= p.N) return -1;
    return ((long)blk * p.bs + (key & (p.bs - 1))) * DK;
  };
  int frow[PER];
  uint32_t fchk[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int idx = min(u * kPairThreads + tid, TCH - 1);  // extra threads repeat the last chunk
    frow[u] = idx / CPR;
    fchk[u] = (uint32_t)(idx % CPR) * 16;
  }
  uint4 stage[PF][PER];
  bool sok[PF];
  // every stage issues PER loads whatever the tile (clamped rows), so the
  // compiler can wait for one stage at a time; rows 16..31 come from the
  // second half's block
  auto fetch = [&](uint4 (&st)[PER], bool& ok, int n) {
    const int tile = start + n * stride;
    const bool in = tile < end;
    const long b0 = in ? half_base(tile, 2 * n) : 0;
    const long b1 = in && tile + kTile < end ? half_base(tile + kTile, 2 * n + 1) : b0;
    ok = in && b0 >= 0 && b1 >= 0;
    const int last = ok ? min(TK, end - tile) - 1 : 0;
    const long c0 = ok ? b0 : 0, c1 = ok ? b1 - (long)kTile * DK : 0;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int row = min(frow[u], last);
      const long c = row >= kTile ? c1 : c0;
      st[u] = load_stream((const uint8_t*)p.k + (c + (long)row * DK) * 2 + fchk[u]);
    }
  };
  auto store_tile = [&](int buf, const uint4 (&st)[PER]) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int idx = u * kPairThreads + tid;
      if (idx < TCH)
        *reinterpret_cast<uint4*>(lds[buf] + (idx / CPR) * ROWB + (idx % CPR) * 16) = st[u];
    }
  };
  constexpr float kLazy = 8.f;
  // this half's partial S^T of the tile in `buf`, both 16-key halves (lane:
  // keys kh*16 + grp*4 .. +3 of row col), published in slot `sl`
  auto qk_half = [&](int buf, int sl) {
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const uint8_t* ka = lds[buf] + (kh * kTile + col) * ROWB + grp * 16 + half * KH * 64;
      f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
      bf16x8_t kf[KH];
#pragma unroll
      for (int k = 0; k < KH; ++k)
        kf[k] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(ka + k * 64));
#pragma unroll
      for (int k = 0; k < KH; ++k) {
        if (k & 1) s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[k], qf[k], s1, 0, 0, 0);
        else s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[k], qf[k], s0, 0, 0, 0);
      }
      s_ps[sl][rbw][half][kh][lane] = s0 + s1;
    }
  };
  // the whole scores of slot `sl` (half 0's part + half 1's part), one
  // online-softmax step over the tile's 32 keys: the weights of each 16-key
  // half (bf16 hi + lo) and the factor the accumulators must be rescaled by;
  // rescale is wave-uniform
  float alpha = 1.f;
  bool rescale = false;
  bf16x8_t pb[2] = {};
  auto softmax = [&](int sl, int tile, bool ok) {
    float sv[2][4];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const f32x4_t s = s_ps[sl][rbw][0][kh][lane] + s_ps[sl][rbw][1][kh][lane];
      const int key0 = tile + kh * kTile + grp * 4;
#pragma unroll
      for (int v = 0; v < 4; ++v)
        sv[kh][v] = ok && key0 + v < lvis ? s[v] * p.scale_log2 : -INFINITY;
    }
    float mx = fmaxf(fmaxf(fmaxf(sv[0][0], sv[0][1]), fmaxf(sv[0][2], sv[0][3])),
                     fmaxf(fmaxf(sv[1][0], sv[1][1]), fmaxf(sv[1][2], sv[1][3])));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const bool move = mx > m + kLazy;
    rescale = __any(move);
    const float m_new = move ? mx : m;
    alpha = m == -INFINITY ? 0.f : fast_exp2(m - m_new);
    m = m_new;
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    float lsum = 0.f;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
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
  // O^T += V^T . P^T over this half's 256 columns, one 16-key half at a time
  auto pv = [&](int buf) {
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const uint8_t* va_ptr = lds[buf] + (kh * kTile + grp * 4 + (col >> 2)) * ROWB +
                              (col & 3) * 8 + half * (DV / 2) * 2;
      constexpr int VG = 8;
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
  if (active) qk_half(0, 0);
  __syncthreads();
  if (active) softmax(0, start, bok[0]);
  for (int n0 = 0; n0 < n_tiles; n0 += PF) {
#pragma unroll
    for (int jj = 0; jj < PF; ++jj) {  // tile n in buffer j, tile n + 1 in buffer 1 - j
      const int n = n0 + jj;
      const int j = jj & 1;
      const int sg = (jj + 2) % PF;  // the stage holding tile n + 2
      const bool more = n + 1 < n_tiles;
      if (n < n_tiles) {
        if (active) {
          if (more) qk_half(1 - j, 1 - j);  // tile n + 1's partial scores
          if (rescale) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
          }
          if (bok[j]) pv(j);  // a bad block's tile holds no usable rows
        }
        if (!bok[j] && tid == 0) report(p.status, KVC_ERR_DATA);
      }
      __syncthreads();  // partial scores of tile n + 1 published; buffer j read
      if (n < n_tiles && more && active) softmax(1 - j, start + (n + 1) * stride, bok[1 - j]);
      store_tile(j, stage[sg]);  // tile n + 2
      bok[j] = sok[sg];
      fetch(stage[sg], sok[sg], n + 2 + PF);
      __syncthreads();
    }
  }

  if (!rvalid) return;
  float* wo = p.ws_o + (wrow * p.max_parts + part) * DV + half * (DV / 2);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
    *reinterpret_cast<f32x4_t*>(wo + dt * 16 + grp * 4) = oacc[dt];
  float lt = l + __shfl_xor(l, 16);
  lt += __shfl_xor(lt, 32);
  if (half == 0 && grp == 0) {
    float* wml = p.ws_ml + (wrow * p.max_parts + part) * 2;
    wml[0] = m;
    wml[1] = lt;
  }
}

// Up to 16 rows (one row block): four wavefronts split the columns, so all of
// them compute (partition_mla<PF, 4>).  More rows: partition_mla_pair, 64 rows
// per workgroup (returned as 1: one workgroup of rows per 64).
int mla_col_split(int rows) { return rows <= 16 ? 4 : 1; }

hipError_t launch_partition_mla(const AttnParams& p, hipStream_t s) {
  const int R = p.Hq * p.n_q;
  const int C = mla_col_split(R);
  const long rows_wg = 16L * (kMlaWaves / C);
  const long n_rg = (R + rows_wg - 1) / rows_wg;
  const long units = (long)p.B * p.max_parts;
  const long n_wg = (units + 7) / 8 * 8 * n_rg;
  if (units == 0) return hipSuccess;
  if (n_wg > 0x7fffffffL) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)n_wg), block(kMlaThreads);
  if (C == 4) hipLaunchKernelGGL((partition_mla<2, 4>), grid, block, 0, s, p);
  else hipLaunchKernelGGL((partition_mla_pair<2>), grid, dim3(kPairThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace kvc
