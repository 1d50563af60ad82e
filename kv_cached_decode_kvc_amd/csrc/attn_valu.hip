// attn_valu.hip -- split-KV partition kernel on the vector ALUs: one query row
// per wavefront.
//
// Computes, for one (sequence b, query head h, query row r, partition p), the
// running maximum m, running sum l and unnormalised output O over the visible
// keys of the partition's tiles -- the online-softmax recurrence of "Inference-1"
// (brunomaga.github.io), section "FlashAttention", and of "Inference o quy mo lon"
// (truongducdung.dev), 07 "Online softmax"; the partitioning is the split-KV of
// "Inference-1", section "FlashDecoding".  Row r of n_q sees keys
// 0 .. L - n_q + r ("Inference-1", "KV cache": shifted causal mask).
//
// Used for MHA (one query row per KV row, so there is no dense contraction to
// give to the matrix cores) and for every fp32 cache.  Paged bf16 and fp32
// batches too large for one round of such work items run the stream-K form
// instead (partition_valu_sk, at the end of this file).  FP8 caches ("Inference
// o quy mo lon", 03 "KV cache quantization"; "Inference-2", "KV cache
// quantization") hold one code per element and one scale per row: the row's
// key scale multiplies the reduced dot product and its value scale joins the
// softmax weight, so the codes are only widened, never rescaled per element.
//
// Partition p of a sequence's n = ceil(L / P) partitions owns the 16-key tiles
// p, p + n, p + 2n, ...: the wavefronts of one sequence run side by side and
// read neighbouring tiles at the same time.  Any split of the keys gives the
// same softmax once the partials are combined; this one keeps the memory
// traffic of concurrent wavefronts inside a narrow window.  Keys are streamed
// with non-temporal loads: they are read exactly once.  Work items are spread
// over the XCDs with xcd_item (common.hpp); in a paged cache the block ids of
// a partition's tiles are fetched 64 at a time into one register (one per
// lane) and picked out with v_readlane, so no table load waits between one
// tile's arrival and the next tile's loads.
//
// Layout of the work: a wavefront streams 16-key tiles.  A key row of D
// elements is split over LPR lanes holding 16 bytes each, so one 16-byte load
// per lane fetches RPL = 64/LPR whole rows (1 KiB, fully coalesced); U = 16/RPL
// loads cover a tile for K and U for V.  Dot products are reduced inside the
// LPR lanes with DPP; the tile maximum and, at the end, the sum and output are
// reduced across the RPL row groups with lane shuffles.
#include "launch.hpp"

namespace kvc {

// FP8 cache element of format F (codes; queries stay bf16).
template <int F>
struct Fp8 {
  uint8_t code;
};

template <typename T>
struct IsFp8 {
  static constexpr int kFormat = 0;
};
template <int F>
struct IsFp8<Fp8<F>> {
  static constexpr int kFormat = F;
};

template <typename T, int D>
struct ValuShape {
  static constexpr int VE = 16 / (int)sizeof(T);  // elements per lane per load
  static constexpr int LPR = D / VE;                // lanes per key row
  static constexpr int RPL = kWave / LPR;           // key rows per wave load
  static constexpr int U = kTile / RPL;             // loads per tile (each of K, V)
  static_assert(LPR == 4 || LPR == 8 || LPR == 16 || LPR == 32, "unsupported row split");
};

template <typename T>
struct Elem;

template <>
struct Elem<uint16_t> {  // bf16: a 16-byte load holds 8 elements in 4 words
  using Q = uint4;
  static __device__ __forceinline__ Q load_q(const void* q, long off) {
    return *reinterpret_cast<const uint4*>((const uint16_t*)q + off);
  }
  static __device__ __forceinline__ float dot(const uint4& q, const uint4& k) {
    float a = dot2_bf16(k.x, q.x, 0.f);
    a = dot2_bf16(k.y, q.y, a);
    a = dot2_bf16(k.z, q.z, a);
    return dot2_bf16(k.w, q.w, a);
  }
  static __device__ __forceinline__ void axpy(float p, const uint4& v, float* o) {
    o[0] += p * bf16_lo(v.x);
    o[1] += p * bf16_hi(v.x);
    o[2] += p * bf16_lo(v.y);
    o[3] += p * bf16_hi(v.y);
    o[4] += p * bf16_lo(v.z);
    o[5] += p * bf16_hi(v.z);
    o[6] += p * bf16_lo(v.w);
    o[7] += p * bf16_hi(v.w);
  }
};

template <>
struct Elem<float> {  // fp32: 4 elements per 16-byte load
  using Q = uint4;
  static __device__ __forceinline__ Q load_q(const void* q, long off) {
    return *reinterpret_cast<const uint4*>((const float*)q + off);
  }
  static __device__ __forceinline__ float dot(const uint4& q, const uint4& k) {
    float a = __uint_as_float(q.x) * __uint_as_float(k.x);
    a = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), a);
    a = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), a);
    return fmaf(__uint_as_float(q.w), __uint_as_float(k.w), a);
  }
  static __device__ __forceinline__ void axpy(float p, const uint4& v, float* o) {
    o[0] += p * __uint_as_float(v.x);
    o[1] += p * __uint_as_float(v.y);
    o[2] += p * __uint_as_float(v.z);
    o[3] += p * __uint_as_float(v.w);
  }
};

template <int F>
struct Elem<Fp8<F>> {  // FP8 codes: a 16-byte load holds 16 elements; q is 16 bf16
  struct Q {
    uint4 a, b;
  };
  static __device__ __forceinline__ Q load_q(const void* q, long off) {
    const uint4* p = reinterpret_cast<const uint4*>((const uint16_t*)q + off);
    return Q{p[0], p[1]};
  }
  // q . codes (the row's scale is applied by the caller): codes widen to bf16
  // pairs exactly and meet the bf16 query in v_dot2_f32_bf16
  static __device__ __forceinline__ float dot(const Q& q, const uint4& k) {
    const uint2 k0 = fp8x4_to_bf16x4<F>(k.x), k1 = fp8x4_to_bf16x4<F>(k.y);
    const uint2 k2 = fp8x4_to_bf16x4<F>(k.z), k3 = fp8x4_to_bf16x4<F>(k.w);
    float a = dot2_bf16(k0.x, q.a.x, 0.f);
    a = dot2_bf16(k0.y, q.a.y, a);
    a = dot2_bf16(k1.x, q.a.z, a);
    a = dot2_bf16(k1.y, q.a.w, a);
    a = dot2_bf16(k2.x, q.b.x, a);
    a = dot2_bf16(k2.y, q.b.y, a);
    a = dot2_bf16(k3.x, q.b.z, a);
    return dot2_bf16(k3.y, q.b.w, a);
  }
  // o += p * codes (p carries the row's value scale)
  static __device__ __forceinline__ void axpy(float p, const uint4& v, float* o) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x2_t lo = fp8x2_to_f32<F, false>(w[i]);
      const f32x2_t hi = fp8x2_to_f32<F, true>(w[i]);
      o[4 * i + 0] += p * lo[0];
      o[4 * i + 1] += p * lo[1];
      o[4 * i + 2] += p * hi[0];
      o[4 * i + 3] += p * hi[1];
    }
  }
};

// AP: an append fused into the launch (not FP8; AttnParams::cu_new): the new
// rows of a sequence come from k_new / v_new and are written into the cache.
// 1: a contiguous cache; 2: a paged cache, block table included.
// Wavefronts per SIMD the FP8 forms keep room for (measured best; the fused
// combine would otherwise cost them one).
template <typename T, int D>
constexpr int valu_min_waves() { return IsFp8<T>::kFormat == 0 ? 1 : D == 128 ? 5 : 6; }

template <typename T, int D, int AP>
__global__ __launch_bounds__(64, (valu_min_waves<T, D>())) void partition_valu(AttnParams p) {
  using S = ValuShape<T, D>;
  constexpr int VE = S::VE, LPR = S::LPR, RPL = S::RPL, U = S::U;
  constexpr bool kF8 = IsFp8<T>::kFormat != 0;
  constexpr int TPI = kF8 ? 2 : 1;  // tiles per loop iteration
  const int lane = threadIdx.x;
  const WorkItem wi = xcd_item(blockIdx.x, p.Hq * p.n_q, p.max_parts);  // u = h * n_q + r
  if (!wi.live) return;
  const int b = wi.b, part = wi.part, r = wi.u % p.n_q, h = wi.u / p.n_q;

  // paged cache with the block table fused in: the work item of the last
  // query row of the sequence's first head and first partition does the
  // sequence's bookkeeping (new table entries, slots, new rows, length;
  // sequence 0 the free-list head) from its own scan of the batch, after
  // its attention work (nothing in this launch waits for it: the tiles read
  // new rows from k_new / v_new), where the loop's registers are free
  constexpr bool paged_ap = AP == 2;
  auto bookkeeping = [&]() {
    const AllocScan as = alloc_scan(p.seq_lens, p.cu_new, p.head_in, p.B, p.bs, p.max_blocks,
                                    p.N, b);
    const int len = p.seq_lens[b], c0b = p.cu_new[b], n = p.cu_new[b + 1] - c0b;
    if (as.err != 0) {  // all or nothing: only the head, the lengths and the status
      if (lane == 0) {
        p.seq_lens_out[b] = len;
        if (b == 0) {
          report(p.status, as.err);
          *p.head_out = as.head;
        }
      }
    } else {
      const int have = (len + p.bs - 1) / p.bs;
      const int need = (int)(((long)len + n + p.bs - 1) / p.bs) - have;
      const int first = as.head + as.before;
      int32_t* trow_out = p.table_out + (long)b * p.max_blocks;
      for (int j = lane; j < need; j += kWave) trow_out[have + j] = p.free_list[first + j];
      if (n > 0 && c0b >= 0 && c0b + n <= p.total_new) {
        for (int t = lane; t < n; t += kWave) {
          const int pos = len + t, lb = pos / p.bs;
          const long blk = lb < have ? p.table[(long)b * p.max_blocks + lb]
                                     : p.free_list[first + lb - have];
          p.slots[c0b + t] = (int32_t)(blk * p.bs + pos % p.bs);
        }
        // the sequence's new rows into their slots, token by token (the
        // block once per token), 16 bytes per lane and four chunks in flight
        // (the tiles of this launch read the rows from k_new / v_new)
        constexpr int CH = D * (int)sizeof(T) / 16;  // 16-byte chunks of a row
        const int per_tok = p.Hkv * CH;
        for (int t = 0; t < n; ++t) {
          const int pos = len + t, lb = pos / p.bs;
          const long blk = __builtin_amdgcn_readfirstlane(
              lb < have ? p.table[(long)b * p.max_blocks + lb] : p.free_list[first + lb - have]);
          if (blk < 0 || blk >= p.N) {
            if (lane == 0) report(p.status, KVC_ERR_DATA);
            continue;
          }
          const uint4* ks = reinterpret_cast<const uint4*>(p.k_new) + (long)(c0b + t) * per_tok;
          const uint4* vs = reinterpret_cast<const uint4*>(p.v_new) + (long)(c0b + t) * per_tok;
          uint4* kd = reinterpret_cast<uint4*>(p.k_out) + (blk * p.Hkv * p.bs + pos % p.bs) * CH;
          uint4* vd = reinterpret_cast<uint4*>(p.v_out) + (blk * p.Hkv * p.bs + pos % p.bs) * CH;
#pragma unroll 4
          for (int x = lane; x < per_tok; x += kWave) {  // chunk x: head x / CH, piece x % CH
            const long dst = (long)(x / CH) * p.bs * CH + x % CH;
            kd[dst] = ks[x];
            vd[dst] = vs[x];
          }
        }
      }
      if (lane == 0) {
        p.seq_lens_out[b] = len + n;
        if (b == 0) *p.head_out = as.head + as.total;
      }
    }
    };
  const bool book = paged_ap && part == 0 && h == 0 && r == p.n_q - 1;
  int code;
  const int L = attended_len(p.seq_lens, p.cu_new, p.total_new, b, p.n_q, p.cap, &code);
  const bool writer = AP && !paged_ap && part == 0 && h == 0 && r == p.n_q - 1 && lane == 0;
  if (L < 0) {
    if (part == 0 && h == 0 && r == 0 && lane == 0) report(p.status, code);
    if (writer) p.seq_lens_out[b] = p.seq_lens[b];  // a refused append keeps the length
    if (book) bookkeeping();
    if (p.cnt && part == 0 && lane * 4 < D) {  // combine fused in: the row's output is zeros
      const float z[4] = {0.f, 0.f, 0.f, 0.f};
      store_out<4>(p.out, p.out_bf16, (((long)b * p.n_q + r) * p.Hq + h) * D + lane * 4, z);
    }
    return;
  }
  if (writer) p.seq_lens_out[b] = L;
  // fused append: keys len0 .. L-1 are the new rows, read from k_new / v_new
  // (row c0 + key - len0) and written into the cache by the work item of the
  // last query row of the KV head's first query head, which sees them all
  const int len0 = AP ? p.seq_lens[b] : L;
  const int c0 = AP ? p.cu_new[b] : 0;
  const bool app_writer = AP && !paged_ap && r == p.n_q - 1 && h % p.G == 0;
  const int nparts = (L + p.P - 1) / p.P;
  if (part >= nparts) return;
  const int start = part * kTile;              // first tile of this partition
  const int stride = nparts * kTile;            // distance to its next tile
  const int end = L - p.n_q + r + 1;            // visible keys of row r
  const long row = ((long)b * p.Hq + h) * p.n_q + r;
  float* wml = p.ws_ml + (row * p.max_parts + part) * 2;
  const int c = lane % LPR;   // which 16-byte column chunk of a key row
  const int r0 = lane / LPR;  // which row of a wave load

  float o[VE];
#pragma unroll
  for (int j = 0; j < VE; ++j) o[j] = 0.f;
  float m = -INFINITY, l = 0.f;

  if (start < end) {
    const int g = h / p.G;
    const T* kbase = (const T*)p.k;
    const T* vbase = (const T*)p.v;
    const typename Elem<T>::Q qv =
        Elem<T>::load_q(p.q, (((long)b * p.n_q + r) * p.Hq + h) * D + c * VE);
    // paged: lane i holds the block of the partition's tile number j * 64 + i
    // (with the block table fused in, only tiles that start below the old
    // length have one yet: the rest are new rows, read from k_new / v_new)
    const bool paged = p.table != nullptr;
    const int32_t* trow = paged ? p.table + (long)b * p.max_blocks : nullptr;
    const int id_end = paged_ap ? min(end, len0) : end;
    auto load_ids = [&](int j) -> int {
      const int tk = start + (j * kWave + lane) * stride;
      return tk < id_end ? trow[tk / p.bs] : 0;
    };
    int ids = 0, ids_next = 0;
    if (paged) {
      ids = load_ids(0);
      if (start + kWave * stride < end) ids_next = load_ids(1);
    }
    int idx = 0;  // number of the iteration's first tile within the partition
    // TPI tiles of the partition per iteration: their loads are all issued
    // before any of them is used (FP8 tiles carry half the bytes, so two keep
    // as many bytes in flight per wavefront as one bf16 tile)
    for (int tile = start; tile < end; tile += TPI * stride) {
      uint4 kr[TPI][U], vr[TPI][U];
      float ksc[TPI][U], vsc[TPI][U];  // FP8: scales of this lane's rows
      int nvalid[TPI];                 // visible keys of each tile (0: none)
#pragma unroll
      for (int i = 0; i < TPI; ++i) {
        const int ti = tile + i * stride;
        nvalid[i] = 0;
        if (ti >= end) continue;
        long row0;  // cache row of key `ti` of (b, g)
        if (!paged) {
          row0 = ((long)b * p.Hkv + g) * p.S_max + ti;
        } else {
          const int ii = idx + i;
          if (ii > 0 && (ii & (kWave - 1)) == 0) {  // the next 64 tiles' ids
            ids = ids_next;
            if (start + (ii + kWave) * stride < end) ids_next = load_ids(ii / kWave + 1);
          }
          const int blk = __builtin_amdgcn_readlane(ids, ii & (kWave - 1));
          if (paged_ap && ti >= len0) {
            row0 = 0;  // every row of the tile is new: none is read from the cache
          } else if (blk < 0 || blk >= p.N) {
            if (lane == 0) report(p.status, KVC_ERR_DATA);
            continue;
          } else {
            row0 = ((long)blk * p.Hkv + g) * p.bs + (ti % p.bs);
          }
        }
        nvalid[i] = min(kTile, end - ti);  // >= 1
#pragma unroll
        for (int u = 0; u < U; ++u) {
          int tt = u * RPL + r0;
          tt = tt < nvalid[i] ? tt : nvalid[i] - 1;  // masked lanes re-read a visible row
          if constexpr (kF8) {  // row0 starts a 16-row tile: codes, then scales
            const long t0 = (row0 >> 4) * fp8_tile_bytes(D);
            const long off = t0 + (long)tt * D + c * VE;
            kr[i][u] = load_stream(kbase + off);
            vr[i][u] = load_stream(vbase + off);
            // scales: non-temporal like the codes (a cached load would
            // allocate in the last-level caches and wait on their evictions)
            const long so = t0 + 16L * D + tt * 4;
            ksc[i][u] = __builtin_nontemporal_load(
                reinterpret_cast<const float*>((const uint8_t*)p.k + so));
            vsc[i][u] = __builtin_nontemporal_load(
                reinterpret_cast<const float*>((const uint8_t*)p.v + so));
          } else {
            const T* ks = kbase + (row0 + tt) * D + c * VE;
            const T* vs = vbase + (row0 + tt) * D + c * VE;
            if (AP && ti + kTile > len0 && ti + tt >= len0) {  // a new row: from k_new / v_new
              const long nr = ((long)(c0 + ti + tt - len0) * p.Hkv + g) * D + c * VE;
              ks = (const T*)p.k_new + nr;
              vs = (const T*)p.v_new + nr;
            }
            kr[i][u] = load_stream(ks);
            vr[i][u] = load_stream(vs);
          }
        }
      }
      idx += TPI;
      if constexpr (AP && !kF8) {
        if (app_writer && tile + kTile > len0 && nvalid[0] > 0) {  // store this tile's new rows
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int tt = u * RPL + r0;
            if (tt < nvalid[0] && tile + tt >= len0) {
              const long off = (((long)b * p.Hkv + g) * p.S_max + tile + tt) * D + c * VE;
              *reinterpret_cast<uint4*>((T*)p.k_out + off) = kr[0][u];
              *reinterpret_cast<uint4*>((T*)p.v_out + off) = vr[0][u];
            }
          }
        }
      }
      float s[TPI][U];
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < TPI; ++i)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          s[i][u] = -INFINITY;
          if (nvalid[i] > 0) {
            float dotp = group_sum<LPR>(Elem<T>::dot(qv, kr[i][u]));
            if constexpr (kF8) dotp *= ksc[i][u];
            if (u * RPL + r0 < nvalid[i]) s[i][u] = dotp * p.scale_log2;
          }
          mx = fmaxf(mx, s[i][u]);
        }
      mx = cross_max<LPR>(mx);
      if (mx == -INFINITY) continue;  // no visible key in these tiles (bad blocks)
      const float m_new = fmaxf(m, mx);
      const float alpha = fast_exp2(m - m_new);  // 0 on the first tile
      l *= alpha;
#pragma unroll
      for (int j = 0; j < VE; ++j) o[j] *= alpha;
#pragma unroll
      for (int i = 0; i < TPI; ++i) {
        if (nvalid[i] == 0) continue;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const float pu = fast_exp2(s[i][u] - m_new);
          l += pu;
          if constexpr (kF8) Elem<T>::axpy(pu * vsc[i][u], vr[i][u], o);
          else Elem<T>::axpy(pu, vr[i][u], o);
        }
      }
      m = m_new;
    }
    // every row group holds part of the sum and output: add them up
    l = cross_sum<LPR>(l);
#pragma unroll
    for (int j = 0; j < VE; ++j) o[j] = cross_sum<LPR>(o[j]);
  }
  // partials: read by the reduce kernel (a later launch: plain stores) or,
  // combine fused in, by another work item of this launch (write-through)
  const __amdgpu_buffer_rsrc_t prow = shared_rsrc(p.ws_o + row * p.max_parts * D);  // the row's partials
  if (r0 == 0) {
#pragma unroll
    for (int j = 0; j < VE; j += 4) {
      const f32x4_t v = {o[j], o[j + 1], o[j + 2], o[j + 3]};
      if (p.cnt) st_shared4(prow, (uint32_t)((part * D + c * VE + j) * 4), v);
      else *reinterpret_cast<f32x4_t*>(p.ws_o + (row * p.max_parts + part) * D + c * VE + j) = v;
    }
  }
  if (lane == 0) {
    if (p.cnt) {
      st_shared(wml, m);
      st_shared(wml + 1, l);
    } else {
      wml[0] = m;
      wml[1] = l;
    }
  }

  if (book) bookkeeping();

  // Combine fused in: the row's last partition to finish merges the row's
  // partials and writes the row.  Lane (r0, c) takes partitions r0, r0 +
  // RPL, ... for its columns, and the row groups merge by shuffles.  Every
  // partial, this one's too, is read back from the workspace, so the order
  // of the sums does not depend on which partition finished last.
  if (p.cnt && arrive_last(p.cnt, row, nparts)) {
    float mm = -INFINITY, dd = 0.f, acc[VE];
#pragma unroll
    for (int j = 0; j < VE; ++j) acc[j] = 0.f;
    const float2* mlp = reinterpret_cast<const float2*>(p.ws_ml) + row * p.max_parts;
    constexpr int KU = VE >= 16 ? 1 : 2;  // partials per lane in flight
    for (int j0 = r0; j0 < nparts; j0 += KU * RPL) {
      float2 mlv[KU];
      float ov[KU][VE];
#pragma unroll
      for (int u = 0; u < KU; ++u) {
        const int j = j0 + u * RPL;
        const bool use = j < nparts;
        mlv[u] = make_float2(-INFINITY, 0.f);
        if (use) mlv[u] = make_float2(ld_shared(&mlp[j].x), ld_shared(&mlp[j].y));
#pragma unroll
        for (int k = 0; k < VE; k += 4) {
          f32x4_t x = {0.f, 0.f, 0.f, 0.f};
          if (use) x = ld_shared4(prow, (uint32_t)((j * D + c * VE + k) * 4));
          ov[u][k] = x[0], ov[u][k + 1] = x[1], ov[u][k + 2] = x[2], ov[u][k + 3] = x[3];
        }
      }
#pragma unroll
      for (int u = 0; u < KU; ++u) merge_partial<VE>(mm, dd, acc, mlv[u].x, mlv[u].y, ov[u]);
    }
#pragma unroll
    for (int sh = LPR; sh < kWave; sh <<= 1) {  // one column at a time: no second copy
      const float m2 = __shfl_xor(mm, sh), d2 = __shfl_xor(dd, sh);
      const float mn = fmaxf(mm, m2);
      const float wa = mm == -INFINITY ? 0.f : fast_exp2(mm - mn);
      const float wb = m2 == -INFINITY ? 0.f : fast_exp2(m2 - mn);
#pragma unroll
      for (int k = 0; k < VE; ++k) acc[k] = acc[k] * wa + __shfl_xor(acc[k], sh) * wb;
      dd = dd * wa + d2 * wb;
      mm = mn;
    }
    if (r0 == 0) {
      const float inv = dd > 0.f ? 1.f / dd : 0.f;
#pragma unroll
      for (int k = 0; k < VE; ++k) acc[k] *= inv;
      store_out<VE>(p.out, p.out_bf16, (((long)b * p.n_q + r) * p.Hq + h) * D + c * VE, acc);
    }
  }
}

// Stream-K form (paged bf16 and fp32 caches whose work items would take more
// than one round of resident wavefronts): the batch's 16-key tiles are shared
// out evenly over a fixed number of workers, as in the matrix-core kernel
// (attn_mfma.hip), so that every worker streams the same number of tiles
// (+-1) and the launch does not end with a ragged last round of items of
// different lengths ("Inference-1", "FlashDecoding": any split of the keys
// combines exactly).  A segment is one query row (sequence b, KV head g, row
// i = r * G + hh of the KV head's G * n_q rows) with T_b = ceil(L_b / 16)
// tile-units; the segments lie end to end in (b, g, i) order and worker w of
// NW takes the contiguous units [w W / NW, (w + 1) W / NW) of the W in total,
// a run that may end one segment and start the next.  Each (segment, worker)
// piece leaves one partial at workspace row segment + worker (unique, since
// both grow along the run), and the worker holding a segment's first tile
// records which workers cover it, for the reduce.  A row r < n_q - 1 sees
// fewer keys than the segment's tiles: its pieces past them leave empty
// partials (m = -inf).  The tile loop is the fixed-partition kernel's, one
// tile at a time.
template <typename T, int D>
__global__ __launch_bounds__(64) void partition_valu_sk(AttnParams p) {
  using S = ValuShape<T, D>;
  constexpr int VE = S::VE, LPR = S::LPR, RPL = S::RPL, U = S::U;
  static_assert(IsFp8<T>::kFormat == 0, "bf16 and fp32 caches");
  const int lane = threadIdx.x;
  const int c = lane % LPR;   // which 16-byte column chunk of a key row
  const int r0 = lane / LPR;  // which row of a wave load
  const int Gq = p.G * p.n_q;  // query rows of a KV head
  const int SU = p.Hkv * Gq;   // segments of a sequence
  const int bs_shift = __builtin_ctz((unsigned)(p.bs > 0 ? p.bs : 1));
  const bool paged = p.table != nullptr;

  auto run_piece = [&](int b, int u, int L, int t0, int t1, long slot) {
    const int g = u / Gq, i = u % Gq, r = i / p.G, h = g * p.G + i % p.G;
    const int end = L - p.n_q + r + 1;           // visible keys of row r
    const int k_end = min(t1 * kTile, end);
    float o[VE];
#pragma unroll
    for (int j = 0; j < VE; ++j) o[j] = 0.f;
    float m = -INFINITY, l = 0.f;
    if (t0 * kTile < k_end) {
      const T* kbase = (const T*)p.k;
      const T* vbase = (const T*)p.v;
      const typename Elem<T>::Q qv =
          Elem<T>::load_q(p.q, (((long)b * p.n_q + r) * p.Hq + h) * D + c * VE);
      const int32_t* trow = paged ? p.table + (long)b * p.max_blocks : nullptr;
      auto load_ids = [&](int j0) -> int {
        const int tk = (t0 + j0 + lane) * kTile;
        return tk < k_end ? trow[tk >> bs_shift] : 0;
      };
      int ids = 0, ids_next = 0;
      if (paged) {
        ids = load_ids(0);
        if ((t0 + kWave) * kTile < k_end) ids_next = load_ids(kWave);
      }
      int idx = 0;
      for (int tile = t0 * kTile; tile < k_end; tile += kTile, ++idx) {
        long row0;
        if (!paged) {
          row0 = ((long)b * p.Hkv + g) * p.S_max + tile;
        } else {
          if (idx > 0 && (idx & (kWave - 1)) == 0) {
            ids = ids_next;
            if ((t0 + idx + kWave) * kTile < k_end) ids_next = load_ids(idx + kWave);
          }
          const int blk = __builtin_amdgcn_readlane(ids, idx & (kWave - 1));
          if (blk < 0 || blk >= p.N) {
            if (lane == 0) report(p.status, KVC_ERR_DATA);
            continue;
          }
          row0 = ((long)blk * p.Hkv + g) * p.bs + (tile & (p.bs - 1));
        }
        const int nvalid = min(kTile, end - tile);  // >= 1
        uint4 kr[U], vr[U];
#pragma unroll
        for (int uu = 0; uu < U; ++uu) {
          int tt = uu * RPL + r0;
          tt = tt < nvalid ? tt : nvalid - 1;  // masked lanes re-read a visible row
          kr[uu] = load_stream(kbase + (row0 + tt) * D + c * VE);
          vr[uu] = load_stream(vbase + (row0 + tt) * D + c * VE);
        }
        float sc[U];
        float mx = -INFINITY;
#pragma unroll
        for (int uu = 0; uu < U; ++uu) {
          const float dotp = group_sum<LPR>(Elem<T>::dot(qv, kr[uu]));
          sc[uu] = uu * RPL + r0 < nvalid ? dotp * p.scale_log2 : -INFINITY;
          mx = fmaxf(mx, sc[uu]);
        }
        mx = cross_max<LPR>(mx);
        if (mx == -INFINITY) continue;  // no finite score in the tile
        const float m_new = fmaxf(m, mx);
        const float alpha = fast_exp2(m - m_new);  // 0 on the first tile
        l *= alpha;
#pragma unroll
        for (int j = 0; j < VE; ++j) o[j] *= alpha;
#pragma unroll
        for (int uu = 0; uu < U; ++uu) {
          const float pu = fast_exp2(sc[uu] - m_new);
          l += pu;
          Elem<T>::axpy(pu, vr[uu], o);
        }
        m = m_new;
      }
      l = cross_sum<LPR>(l);
#pragma unroll
      for (int j = 0; j < VE; ++j) o[j] = cross_sum<LPR>(o[j]);
    }
    if (r0 == 0) {
#pragma unroll
      for (int j = 0; j < VE; j += 4)
        *reinterpret_cast<f32x4_t*>(p.ws_o + slot * D + c * VE + j) =
            f32x4_t{o[j], o[j + 1], o[j + 2], o[j + 3]};
    }
    if (lane == 0) {
      p.ws_ml[slot * 2] = m;
      p.ws_ml[slot * 2 + 1] = l;
    }
  };

  // the lengths give T_b tiles per sequence (0 for an invalid length, which
  // worker 0 reports), W = SU * sum T_b tile-units in all
  const int w = blockIdx.x;
  long W = 0;
  int bad = 0;
  for (int first = 0; first < p.B; first += kWave) {
    const int i = first + lane;
    int tiles = 0;
    if (i < p.B) {
      const int Li = p.seq_lens[i];
      if (Li >= p.n_q && Li <= p.cap) tiles = (Li + kTile - 1) / kTile;
      else bad = 1;
    }
    for (int mm = 1; mm < kWave; mm <<= 1) tiles += __shfl_xor(tiles, mm);
    W += tiles;
  }
  if (w == 0 && __any(bad) && lane == 0) report(p.status, KVC_ERR_DATA);
  W *= SU;
  if (W == 0) return;
  const long NW = min((long)gridDim.x, max(1L, W / p.sk_min_tiles));
  if (w >= NW) return;
  const long s0 = (long)w * W / NW, s1 = (long)(w + 1) * W / NW;
  if (s0 >= s1) return;
  // the sequence holding tile-unit s0: first b with (units before b + its units) > s0
  int b = 0;
  long pre = 0;  // tile-units before sequence b
  for (int first = 0; first < p.B; first += kWave) {
    const int i = first + lane;
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
      b = first + j;
      pre += __shfl(incl - n, j);
      break;
    }
    pre += __shfl(incl, kWave - 1);
  }
  b = __builtin_amdgcn_readfirstlane(b);
  int L = __builtin_amdgcn_readfirstlane(p.seq_lens[b]);
  int tiles = (L + kTile - 1) / kTile;
  long pos = s0;
  while (pos < s1) {
    while (pos >= pre + (long)SU * tiles) {  // past sequence b: the next one with tiles
      pre += (long)SU * tiles;
      ++b;
      L = __builtin_amdgcn_readfirstlane(p.seq_lens[b]);
      tiles = (L >= p.n_q && L <= p.cap) ? (L + kTile - 1) / kTile : 0;
    }
    const long local = pos - pre;
    const int u = (int)(local / tiles), t0 = (int)(local % tiles);
    const int t1 = (int)min((long)tiles, t0 + (s1 - pos));
    const int seg = b * SU + u;
    if (t0 == 0 && lane == 0) {  // this worker starts the segment: record its workers
      const long x_last = pre + (long)u * tiles + tiles - 1;
      const int w_last = (int)(((x_last + 1) * NW - 1) / W);
      p.sk_meta[seg] = make_int2(w, w_last);
    }
    run_piece(b, u, L, t0, t1, (long)seg + w);
    pos += t1 - t0;
  }
}

hipError_t launch_partition_valu(const AttnParams& p, int dtype, hipStream_t s) {
  if (p.sk_meta) {  // stream-K: one workgroup per worker
    if (p.cu_new) return hipErrorInvalidValue;  // no append fused into this form
    if (p.sk_workers <= 0) return hipSuccess;
    const dim3 grid((unsigned)p.sk_workers), block(64);
    if (dtype == KVC_BF16) {
      if (p.D == 128) hipLaunchKernelGGL((partition_valu_sk<uint16_t, 128>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((partition_valu_sk<uint16_t, 64>), grid, block, 0, s, p);
    } else if (dtype == KVC_F32) {
      if (p.D == 128) hipLaunchKernelGGL((partition_valu_sk<float, 128>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((partition_valu_sk<float, 64>), grid, block, 0, s, p);
    } else {
      return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const long n_wg = xcd_grid(p.B, p.Hq * p.n_q, p.max_parts);
  if (n_wg == 0) return hipSuccess;
  if (n_wg > 0x7fffffffL) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)n_wg), block(64);
  if (p.cu_new) {  // fused append (bf16 and fp32 caches): contiguous, or paged with the table
    const bool pg = p.free_list != nullptr;
    if (dtype == KVC_BF16) {
      if (p.D == 128) {
        if (pg) hipLaunchKernelGGL((partition_valu<uint16_t, 128, 2>), grid, block, 0, s, p);
        else hipLaunchKernelGGL((partition_valu<uint16_t, 128, 1>), grid, block, 0, s, p);
      } else {
        if (pg) hipLaunchKernelGGL((partition_valu<uint16_t, 64, 2>), grid, block, 0, s, p);
        else hipLaunchKernelGGL((partition_valu<uint16_t, 64, 1>), grid, block, 0, s, p);
      }
    } else if (dtype == KVC_F32) {
      if (p.D == 128) {
        if (pg) hipLaunchKernelGGL((partition_valu<float, 128, 2>), grid, block, 0, s, p);
        else hipLaunchKernelGGL((partition_valu<float, 128, 1>), grid, block, 0, s, p);
      } else {
        if (pg) hipLaunchKernelGGL((partition_valu<float, 64, 2>), grid, block, 0, s, p);
        else hipLaunchKernelGGL((partition_valu<float, 64, 1>), grid, block, 0, s, p);
      }
    } else {
      return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  if (dtype == KVC_BF16) {
    if (p.D == 128) hipLaunchKernelGGL((partition_valu<uint16_t, 128, 0>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((partition_valu<uint16_t, 64, 0>), grid, block, 0, s, p);
  } else if (dtype == KVC_FP8_E4M3) {
    if (p.D == 128) hipLaunchKernelGGL((partition_valu<Fp8<kFp8E4M3>, 128, 0>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((partition_valu<Fp8<kFp8E4M3>, 64, 0>), grid, block, 0, s, p);
  } else if (dtype == KVC_FP8_E5M2) {
    if (p.D == 128) hipLaunchKernelGGL((partition_valu<Fp8<kFp8E5M2>, 128, 0>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((partition_valu<Fp8<kFp8E5M2>, 64, 0>), grid, block, 0, s, p);
  } else {
    if (p.D == 128) hipLaunchKernelGGL((partition_valu<float, 128, 0>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((partition_valu<float, 64, 0>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace kvc
