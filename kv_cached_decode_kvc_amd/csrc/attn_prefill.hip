// attn_prefill.hip -- (chunked) prefill attention over the KV cache.
//
// "Inference-1" (brunomaga.github.io), "FlashAttention": for a block of
// queries, loop over tiles of keys and values, keep a running maximum, sum
// and unnormalised output per query (online softmax) and never write the
// score matrix; tiles entirely above the causal diagonal are skipped.
// "Inference-1", "Chunked prefill" and "Inference o quy mo lon", 05 "Chunked
// prefill": a long prompt is processed in chunks, each attending over
// everything already cached.  The chunk's rows have been appended first
// (kvc_block_table, kvc_append), so sequence b holds L_b keys and its n_b new
// query rows sit at positions L_b - n_b + r; row r sees keys 0 .. L_b - n_b + r
// ("Inference-1", "KV cache": the causal mask shifted by the cached length).
//
// A workgroup of four wavefronts owns one (sequence, KV head, block of
// 4 * 16 * NT rows); a row is (query position, query head of the group), so
// the grouped heads share every K/V tile ("Efficient Inference", GQA passage).
// The threads load each 32-key tile of K and V (one contiguous run per
// tensor) cooperatively into two LDS buffers through a two-stage register
// ring (one barrier per tile), with buffer loads of the default cache policy
// so that the pair's other row blocks (placement below) find the rows in
// their XCD's L2; each
// wavefront contracts its 16 * NT rows on the matrix cores: S^T = K.Q^T on
// v_mfma_f32_16x16x32_bf16 (Q^T in registers, two 16-key halves), one
// online-softmax step per 32 keys, then O^T += V^T.P^T on
// v_mfma_f32_16x16x32_f16 with V^T via ds_read_b64_tr_b16.  The value rows
// are converted from bf16 to fp16 as they are stored to LDS (exact for
// magnitudes up to 65504: fp16 carries more significand bits than bf16;
// below 2^-14 the absolute error stays under 2^-24, and larger magnitudes
// are outside the supported range), so the weights enter as one fp16 operand,
// 2^-11 relative rounding, where bf16 weights would need a hi and a lo part.
// A wavefront skips the tiles that lie entirely above its rows'
// diagonal.  Outputs are normalised and written directly: there is no
// split over keys.
#include "launch.hpp"

namespace kvc {

namespace {

typedef short i16x4_t __attribute__((__vector_size__(4 * sizeof(short))));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr int kPfWaves = 4;
constexpr int kPfThreads = kPfWaves * kWave;
constexpr int kPfKeys = 32;  // keys per LDS tile (two 16-key MFMA tiles)
constexpr int kPfMaxIds = 4096;  // block ids of one sequence staged in LDS

// 16-byte load at byte `off` of the wave-uniform address `base`, through a
// buffer resource with the default cache policy: the line stays in the XCD's
// L2 for the other row blocks of the pair, which read it soon after.  (The
// decode kernels, whose rows are read once, use non-temporal loads; cached
// loads cost the streaming MLA kernel 68%.)
__device__ __forceinline__ uint4 load_shared_l2(const void* base, uint32_t off) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000);
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// Work placement.  A launch places workgroup i on XCD i mod 8, and each XCD
// has its own L2, so the row blocks of one (sequence, KV head) pair, which
// all read the same K/V rows, are kept on one XCD: pair x + 8j belongs to
// XCD x, which runs its row blocks one pair after another.  The pairs left
// over when their count is not a multiple of 8 have their row blocks dealt
// round-robin over the XCDs.  Within a pair the last row blocks, which see
// the most keys, start first.
struct PfItem {
  int b, g, rt;
  bool live;
};
__device__ __forceinline__ PfItem pf_item(long wg, int pairs, int n_rt, int Hkv) {
  const int x = (int)(wg % kXcds);
  const long t = wg / kXcds;
  const int whole = pairs / kXcds, rem = pairs % kXcds;
  const long first = (long)whole * n_rt;
  PfItem it;
  int pair, rb;
  if (t < first) {
    pair = x + kXcds * (int)(t / n_rt);
    rb = (int)(t % n_rt);
    it.live = true;
  } else {
    const long k = (t - first) * kXcds + x;
    pair = whole * kXcds + (int)(k / n_rt);
    rb = (int)(k % n_rt);
    it.live = k < (long)rem * n_rt;
  }
  it.rt = n_rt - 1 - rb;
  it.b = pair / Hkv;
  it.g = pair % Hkv;
  return it;
}
inline long pf_grid(int pairs, int n_rt) {
  const int whole = pairs / kXcds, rem = pairs % kXcds;
  return (long)kXcds * ((long)whole * n_rt + ((long)rem * n_rt + kXcds - 1) / kXcds);
}

}  // namespace

template <int D, int NT, bool BF16_OUT>
__global__ __launch_bounds__(kPfThreads, 2) void prefill_mfma(PrefillParams p) {
  constexpr int KK = D / 32, DT = D / 16;
  constexpr int CPR = D * 2 / 16;              // 16-byte chunks per row
  constexpr int TCH = kPfKeys * CPR;           // chunks per tile and tensor
  constexpr int PER = (TCH + kPfThreads - 1) / kPfThreads;
  static_assert(kWave % CPR == 0 && 16 % (kWave / CPR) == 0 && TCH % kPfThreads == 0,
                "a wavefront's chunks of one stage lie in one 16-key half");
  constexpr int ROWB = D * 2 + 16;   // K rows: 4 banks apart
  constexpr int VROWB = D * 2 + 32;  // V rows: 8 banks apart, for the transposed reads
  constexpr int PF = 2;
  __shared__ __attribute__((aligned(16))) uint8_t k_lds[2][kPfKeys * ROWB];
  __shared__ __attribute__((aligned(16))) uint8_t v_lds[2][kPfKeys * VROWB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int rows_wg = kPfWaves * 16 * NT;
  const int n_rt = (int)(((long)p.max_q * p.G + rows_wg - 1) / rows_wg);
  const PfItem it = pf_item(blockIdx.x, p.B * p.Hkv, n_rt, p.Hkv);
  if (!it.live) return;
  const int b = it.b, g = it.g;
  const int q0 = p.cu_q[b], n_b = p.cu_q[b + 1] - q0;
  const int R = n_b * p.G;                      // rows of this (sequence, KV head)
  const int row0 = it.rt * rows_wg;
  // Offsets and length are checked before anything else, so that a
  // decreasing cu_q (a negative chunk) is reported rather than skipped.
  const int L = p.seq_lens[b];
  if (n_b < 0 || L < n_b || L > p.cap || q0 < 0 || q0 + n_b > p.total_q) {
    if (it.rt == 0 && g == 0 && tid == 0) report(p.status, KVC_ERR_DATA);
    return;  // whole workgroup
  }
  if (it.rt == 0 && g == 0 && tid == 0 && (long)R > (long)n_rt * rows_wg)
    report(p.status, KVC_ERR_DATA);  // a chunk longer than max_q: its last rows are not computed
  if (row0 >= R) return;  // whole workgroup
  const int cached = L - n_b;

  int lvis[NT];
  bool rvalid[NT];
  long qoff[NT];
  int wave_vis = 0;  // keys this wavefront's rows see (the largest lvis)
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int i = row0 + wave * 16 * NT + nt * 16 + col;
    rvalid[nt] = i < R;
    const int r = rvalid[nt] ? i / p.G : 0;
    const int h = g * p.G + (rvalid[nt] ? i % p.G : 0);
    lvis[nt] = rvalid[nt] ? cached + r + 1 : 0;
    qoff[nt] = ((long)(q0 + r) * p.Hq + h) * D;
    wave_vis = max(wave_vis, lvis[nt]);
  }
  for (int m = 1; m < kWave; m <<= 1) wave_vis = max(wave_vis, __shfl_xor(wave_vis, m));
  // a scalar: it decides a branch around matrix-core work, and those
  // instructions do not honour the lane mask
  wave_vis = __builtin_amdgcn_readfirstlane(wave_vis);
  // keys every valid row of this wavefront sees: tiles below it need no mask
  int vis_min = 0x7fffffff;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) vis_min = min(vis_min, rvalid[nt] ? lvis[nt] : 0x7fffffff);
  for (int m = 1; m < kWave; m <<= 1) vis_min = min(vis_min, __shfl_xor(vis_min, m));
  vis_min = __builtin_amdgcn_readfirstlane(vis_min);
  // keys the workgroup needs: up to its last row's position
  const int last_row = min(row0 + rows_wg, R) - 1;
  const int end = __builtin_amdgcn_readfirstlane(cached + last_row / p.G + 1);  // <= L

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

  const int bs_shift = __builtin_ctz((unsigned)(p.bs > 0 ? p.bs : 1));
  // The sequence's block ids up to `end`, staged in LDS: read from global
  // memory inside the loop, an id would be the newest load in flight and
  // waiting for it would wait for every tile load behind it.
  __shared__ int s_ids[kPfMaxIds];  // max_blocks <= kPfMaxIds (checked on the host)
  const int n_ids = p.table ? ((end - 1) >> bs_shift) + 1 : 0;
  for (int i = tid; i < n_ids; i += kPfThreads) s_ids[i] = p.table[(long)b * p.max_blocks + i];
  __syncthreads();
  // element offset of key `t` (a multiple of 16) of (b, g); -1: bad block
  auto key_base = [&](int t) -> long {
    if (p.table == nullptr) return (((long)b * p.Hkv + g) * p.S_max + t) * D;
    const int blk = __builtin_amdgcn_readfirstlane(s_ids[t >> bs_shift]);  // uniform
    if (blk < 0 || blk >= p.N) return -1;
    return (((long)blk * p.Hkv + g) * p.bs + (t & (p.bs - 1))) * D;
  };
  // wave-uniform 64-bit value in scalar registers
  auto uniform = [](long x) -> long {
    const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(x & 0xffffffff));
    const int hi = __builtin_amdgcn_readfirstlane((int)(x >> 32));
    return (long)(((unsigned long)(unsigned)hi << 32) | lo);
  };
  const int n_tiles = (end + kPfKeys - 1) / kPfKeys;
  struct Stage {
    uint4 k[PER], v[PER];
    bool ok;
  };
  Stage st[PF];
  // Every stage issues the same loads on every path (clamped addresses), so
  // the compiler waits for one stage at a time.  A 32-key tile is two 16-key
  // halves, each inside one block (block sizes are multiples of 16).
  // this thread's chunks of a tile: row, element offset within the row, LDS
  // offset; with head 128 chunk u of every thread lies in 16-key half u
  __builtin_assume(tid < kPfThreads);
  int frow[PER], fchk[PER], lofs[PER], vofs[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int idx = min(u * kPfThreads + tid, TCH - 1);  // extra threads repeat the last chunk
    frow[u] = idx / CPR;
    fchk[u] = (idx % CPR) * 8;
    lofs[u] = frow[u] * ROWB + fchk[u] * 2;
    vofs[u] = frow[u] * VROWB + fchk[u] * 2;
  }
  auto fetch = [&](Stage& s, int n) {
    const int t = n * kPfKeys;
    const bool in = t < end;
    const long b0 = uniform(key_base(in ? t : 0));
    const long b1 = uniform(key_base(in && t + 16 < end ? t + 16 : (in ? t : 0)));
    s.ok = in && b0 >= 0 && b1 >= 0;
    // not loaded: every row clamps to the cache's first row
    const int last = __builtin_amdgcn_readfirstlane(s.ok ? min(kPfKeys, end - t) - 1 : 0);
    const long c0 = s.ok ? b0 : 0, c1 = s.ok ? b1 - 16 * D : 0;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int row = min(frow[u], last);
      // a wavefront's chunks of one stage lie in one 16-key half (64 chunks
      // are 4 rows of 128 or 8 rows of 64): the half's base is uniform
      const bool h1 = __builtin_amdgcn_readfirstlane(frow[u] >= 16 ? 1 : 0) != 0;
      const long c = h1 && last >= 16 ? c1 : c0;
      const uint32_t lane_off = (uint32_t)(row * D + fchk[u]) * 2;  // bytes
      s.k[u] = load_shared_l2((const uint8_t*)p.k + c * 2, lane_off);
      s.v[u] = load_shared_l2((const uint8_t*)p.v + c * 2, lane_off);
    }
  };
  // eight bf16 values -> eight fp16 values (round toward zero: exact in range)
  auto to_f16 = [](uint4 x) -> uint4 {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      o[k] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(bf16_lo(w[k]), bf16_hi(w[k])));
    return make_uint4(o[0], o[1], o[2], o[3]);
  };
  auto store = [&](const Stage& s, int buf) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      if (TCH % kPfThreads == 0 || u * kPfThreads + tid < TCH) {
        *reinterpret_cast<uint4*>(k_lds[buf] + lofs[u]) = s.k[u];
        *reinterpret_cast<uint4*>(v_lds[buf] + vofs[u]) = to_f16(s.v[u]);
      }
    }
  };
  constexpr float kLazy = 8.f;
  // One 32-key tile: scores of both 16-key halves, one softmax step over the
  // 32 keys, then the value products.  A lane holds keys grp*4 .. +3 of each
  // half, so its value operand is the transposed read of those rows of half
  // 0 followed by the same rows of half 1 -- eight distinct keys -- and the
  // weights enter as one fp16 operand.
  auto compute32 = [&](int t, int buf) {
    const uint8_t* ka_ptr = k_lds[buf] + col * ROWB + grp * 16;
    const uint8_t* va_ptr = v_lds[buf] + (grp * 4 + (col >> 2)) * VROWB + (col & 3) * 8;
    bf16x8_t ka[2][KK];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        ka[h][kk] = __builtin_bit_cast(bf16x8_t,
                                       *reinterpret_cast<const uint4*>(ka_ptr + h * 16 * ROWB + kk * 64));
    f16x8_t ph[NT];
    f32x4_t sa[NT][2];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) sa[nt][0] = sa[nt][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        sa[nt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[0][kk], qf[nt][kk], sa[nt][0], 0, 0, 0);
        sa[nt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[1][kk], qf[nt][kk], sa[nt][1], 0, 0, 0);
      }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x4_t s0 = sa[nt][0], s1 = sa[nt][1];
      if (t + kPfKeys > vis_min) {  // the tile reaches past some row's last key
        const int key0 = t + grp * 4;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          s0[v] = key0 + v < lvis[nt] ? s0[v] : -INFINITY;
          s1[v] = key0 + 16 + v < lvis[nt] ? s1[v] : -INFINITY;
        }
      }
      float sv[8];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        sv[v] = s0[v] * p.scale_log2;
        sv[4 + v] = s1[v] * p.scale_log2;
      }
      float mx = sv[0];
#pragma unroll
      for (int v = 1; v < 8; ++v) mx = vmax(mx, sv[v]);
      mx = rows_max(mx);
      const bool move = mx > m[nt] + kLazy;
      if (__any(move)) {
        const float m_new = move ? mx : m[nt];
        const float alpha = m[nt] == -INFINITY ? 0.f : fast_exp2(m[nt] - m_new);
        l[nt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[nt][dt] *= alpha;
        m[nt] = m_new;
      }
      const float m_use = m[nt] == -INFINITY ? 0.f : m[nt];
      f32x2_t pp[4];
#pragma unroll
      for (int v = 0; v < 4; ++v)
        pp[v] = f32x2_t{fast_exp2(sv[2 * v] - m_use), fast_exp2(sv[2 * v + 1] - m_use)};
      l[nt] += ((pp[0][0] + pp[0][1]) + (pp[1][0] + pp[1][1])) +
               ((pp[2][0] + pp[2][1]) + (pp[3][0] + pp[3][1]));
      f16x2_t hh[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) hh[v] = __builtin_convertvector(pp[v], f16x2_t);
      ph[nt] = __builtin_shufflevector(__builtin_shufflevector(hh[0], hh[1], 0, 1, 2, 3),
                                       __builtin_shufflevector(hh[2], hh[3], 0, 1, 2, 3),
                                       0, 1, 2, 3, 4, 5, 6, 7);
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      lds_i16x4_t* a0 = reinterpret_cast<lds_i16x4_t*>(
          (__attribute__((address_space(3))) uint8_t*)(va_ptr + dt * 32));
      lds_i16x4_t* a1 = reinterpret_cast<lds_i16x4_t*>(
          (__attribute__((address_space(3))) uint8_t*)(va_ptr + 16 * VROWB + dt * 32));
      const f16x4_t v0 = __builtin_bit_cast(f16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(a0));
      const f16x4_t v1 = __builtin_bit_cast(f16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(a1));
      const f16x8_t va = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        oacc[nt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, ph[nt], oacc[nt][dt], 0, 0, 0);
    }
  };

  // Tile k lives in register stage k % 2 and then LDS buffer k % 2.  Step n
  // stores tile n + 1 into its buffer (last read in step n - 1, which ended
  // with a barrier), issues the loads of tile n + 3 into the freed stage and
  // computes tile n: one barrier per tile, and each tile's loads have two
  // steps to arrive.
  fetch(st[0], 0);
  fetch(st[1], 1);
  store(st[0], 0);
  bool bok[2] = {st[0].ok, false};
  fetch(st[0], 2);
  __syncthreads();
  for (int n0 = 0; n0 < n_tiles; n0 += 2) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      // straight-line steps (a tile past the end is loaded clamped and not
      // computed), so the compiler waits for one stage's loads at a time
      const int n = n0 + j;
      store(st[1 - j], 1 - j);  // tile n + 1
      bok[1 - j] = st[1 - j].ok;
      fetch(st[1 - j], n + 3);
      const int t = n * kPfKeys;
      if (n < n_tiles) {
        if (!bok[j]) {
          if (tid == 0) report(p.status, KVC_ERR_DATA);
        } else if (t < wave_vis) {
          compute32(t, j);  // tiles above the diagonal are skipped
        }
      }
      __syncthreads();
    }
  }

#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float lt = l[nt] + __shfl_xor(l[nt], 16);
    lt += __shfl_xor(lt, 32);
    if (!rvalid[nt]) continue;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const long o = qoff[nt] + dt * 16 + grp * 4;
      const f32x4_t v = oacc[nt][dt] * inv;
      if constexpr (BF16_OUT) {
        uint16_t* out = (uint16_t*)p.out + o;
        *reinterpret_cast<uint2*>(out) = make_uint2(
            f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16),
            f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16));
      } else {
        *reinterpret_cast<f32x4_t*>((float*)p.out + o) = v;
      }
    }
  }
}

hipError_t launch_prefill(const PrefillParams& p, int out_dtype, hipStream_t s) {
  // 48 rows per wavefront (192 per workgroup): each K/V tile staged and read
  // from LDS serves 1.5x the rows of 32 at 252 registers, still two
  // wavefronts per SIMD
  constexpr int NT = 3;
  const long rows_wg = kPfWaves * 16 * NT;
  const long n_rt = ((long)p.max_q * p.G + rows_wg - 1) / rows_wg;
  if (n_rt == 0 || p.B == 0 || p.Hkv == 0) return hipSuccess;
  if (n_rt > 0x7fffffffL || (long)p.B * p.Hkv > 0x7fffffffL) return hipErrorInvalidConfiguration;
  const long n_wg = pf_grid(p.B * p.Hkv, (int)n_rt);
  if (n_wg > 0x7fffffffL) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)n_wg), block(kPfThreads);
  const bool bf = out_dtype == KVC_BF16;
  if (p.D == 128) {
    if (bf) hipLaunchKernelGGL((prefill_mfma<128, NT, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((prefill_mfma<128, NT, false>), grid, block, 0, s, p);
  } else {
    if (bf) hipLaunchKernelGGL((prefill_mfma<64, NT, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((prefill_mfma<64, NT, false>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace kvc
