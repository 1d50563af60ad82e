"""One layer's KV cache in device memory, driven through the C ABI.

``LayerCache`` owns the device buffers of a workload (cache or block pool,
block table, free list, lengths, workspace) and runs the decode step the way a
serving loop would: ``kvc_block_table_append_attn`` (paged caches: block
table, append and attention in one call) or ``kvc_append_attn`` (contiguous);
each runs as few launches as the library can (one for small multi-head
batches).  The two-stage calls ``kvc_attn_partition`` ->
``kvc_attn_reduce`` remain available for timing the stages apart.  Every step of the computation
runs in the library's kernels; this module only allocates tensors with torch
and passes their addresses.

A prepared step (``prepare_step``) reads lengths and the free-list head from
buffers it never writes, so it can be replayed any number of times with an
identical effect: the benchmark times exactly that replay.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from . import kvc, synth


def to_dev(a: np.ndarray, dtype: str, dev="cuda") -> torch.Tensor:
    """Host rows (bf16 bit patterns or float32) -> device tensor of that element type."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def i32(a, dev="cuda") -> torch.Tensor:
    return torch.as_tensor(np.asarray(a, dtype=np.int32)).to(dev)


def torch_dtype(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


class LayerCache:
    def __init__(self, w: synth.Workload, partition_tokens: int = 0, dev="cuda",
                 block_size: int | None = None, capacity: int | None = None,
                 pool_blocks: int | None = None, poison_nan: bool = False):
        self.w, self.dev = w, dev
        self.bs = w.block_size if block_size is None else block_size
        cap = capacity or synth.capacity_tokens(w)
        tdt = torch_dtype(w.dtype)
        fill = float("nan") if poison_nan else 0.0
        if self.bs == 0:
            self.cap = cap
            shape = (w.B, w.Hkv, cap, w.D)
            self.desc = kvc.cache_desc(w.B, w.Hq, w.Hkv, w.D, w.cache_dtype, 0, max_seq_len=cap,
                                       partition_tokens=partition_tokens)
            self.table = None
            self.N = 0
            self.max_blocks = 0
        else:
            self.max_blocks = -(-cap // self.bs)
            self.cap = self.max_blocks * self.bs
            if pool_blocks is None:
                pool_blocks = (w.B * self.max_blocks + w.B if block_size is not None
                               else synth.pool_blocks(w))
            self.N = pool_blocks
            shape = (self.N, w.Hkv, self.bs, w.D)
            self.desc = kvc.cache_desc(w.B, w.Hq, w.Hkv, w.D, w.cache_dtype, self.bs,
                                       max_blocks_per_seq=self.max_blocks, num_blocks=self.N,
                                       partition_tokens=partition_tokens)
            self.table = torch.full((w.B, self.max_blocks), -1, dtype=torch.int32, device=dev)
            self.free_host = synth.rng(w, synth.S_POOL).permutation(self.N).astype(np.int32)
            self.free_list = i32(self.free_host, dev)
            self.head = torch.zeros(1, dtype=torch.int32, device=dev)
        self.shape = shape
        if w.kv:  # FP8: tiles of 16 rows, each the rows' codes followed by their 16 float32 scales
            nbytes = kvc.kvc_cache_bytes(self.desc)
            self.k = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
            self.v = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
            if poison_nan:  # 0x7F is NaN in both FP8 formats
                self.k.fill_(0x7F)
                self.v.fill_(0x7F)
        else:
            self.k = torch.full(shape, fill, dtype=tdt, device=dev)
            # MLA: one latent cache whose rows serve as keys and values
            self.v = None if w.dv else torch.full(shape, fill, dtype=tdt, device=dev)
        self.seq_lens = torch.zeros(w.B, dtype=torch.int32, device=dev)
        self.status = torch.zeros(1, dtype=torch.int32, device=dev)
        self.n_q = w.n_q
        self.scale = 1.0 / math.sqrt(w.D)

    def fp8_parts(self, which: str):
        """FP8 cache: views of its 16-row tiles, codes uint8 [lead0, lead1,
        tiles, 16, D] and scales float32 [lead0, lead1, tiles, 16], where
        (lead0, lead1) = (blocks, KV heads) or (batch, KV heads) and a
        contiguous cache's rows are padded to whole tiles."""
        buf = self.k if which == "k" else self.v
        D = self.w.D
        tb = 16 * D + 64  # one tile: 16 rows of codes, then their 16 scales
        rows = -(-self.shape[2] // 16) * 16
        lead = (self.shape[0], self.shape[1], rows // 16)
        tiles = buf[:int(np.prod(lead)) * tb].view(-1, tb)
        codes = tiles[:, :16 * D].view(*lead, 16, D)
        scales = tiles[:, 16 * D:].view(torch.float32).view(*lead, 16)
        return codes, scales

    def fp8_rows(self, which: str):
        """FP8 cache on the host, row by row: (codes [lead0, lead1, rows, D],
        scales [lead0, lead1, rows]) numpy arrays."""
        codes, scales = (t.cpu().numpy() for t in self.fp8_parts(which))
        c, s = codes.reshape(*codes.shape[:2], -1, codes.shape[-1]), scales.reshape(*scales.shape[:2], -1)
        return c[:, :, :self.shape[2]], s[:, :, :self.shape[2]]

    # -- building the cache ----------------------------------------------
    def add_tokens(self, k_rows: np.ndarray, v_rows: np.ndarray, counts):
        """Append counts[b] packed rows per sequence (host arrays); returns the
        slot mapping of a paged cache."""
        w = self.w
        counts = np.asarray(counts, dtype=np.int64)
        cu = synth.cu_from_counts(counts)
        total = int(cu[-1])
        cu_d = i32(cu, self.dev)
        slots = None
        if self.bs:
            slots = torch.empty(max(total, 1), dtype=torch.int32, device=self.dev)
            kvc.kvc_block_table(self.desc, self.seq_lens, cu_d, total, self.table, self.free_list,
                                self.head, self.head, slots, self.status)
        out = torch.empty_like(self.seq_lens)
        kvc.kvc_append(self.desc, to_dev(k_rows, w.dtype, self.dev),
                       None if v_rows is None else to_dev(v_rows, w.dtype, self.dev),
                       self.seq_lens, cu_d, total,
                       int(counts.max()) if len(counts) else 0, slots, self.k, self.v, out,
                       self.status)
        self.seq_lens = out
        return slots

    def prefill(self, lengths):
        """The cached rows of every sequence (the generator's stream of cached keys/values)."""
        w = self.w
        return self.add_tokens(synth.packed_cache_rows(w, "k", lengths),
                               None if w.dv else synth.packed_cache_rows(w, "v", lengths),
                               lengths)

    def step_rows(self, step=0):
        w = self.w
        return self.add_tokens(synth.packed_new_rows(w, "k", step),
                               None if w.dv else synth.packed_new_rows(w, "v", step),
                               [w.n_q] * w.B)

    def workspace(self, n_q):
        if self.w.dv:
            nbytes = kvc.kvc_mla_workspace_bytes(self.desc, n_q, self.w.dv)
        else:
            nbytes = kvc.kvc_attn_workspace_bytes(self.desc, n_q)
        # zero-filled: the combine counters at its start must begin at zero
        return torch.zeros(max((nbytes + 3) // 4, 4), dtype=torch.float32, device=self.dev)

    def attend(self, q: torch.Tensor, n_q: int, out_dtype=torch.float32, scale=None,
               seq_lens=None) -> torch.Tensor:
        w = self.w
        scale = self.scale if scale is None else scale
        out = torch.empty((w.B, n_q, w.Hq, w.out_dim), dtype=out_dtype, device=self.dev)
        ws = self.workspace(n_q)
        sl = self.seq_lens if seq_lens is None else seq_lens
        if w.dv:
            kvc.kvc_mla_attn(self.desc, q, n_q, self.k, sl, self.table, w.dv, scale, out, ws,
                             self.status)
        elif n_q == 1:
            kvc.kvc_decode_attn(self.desc, q, self.k, self.v, sl, self.table, scale, out, ws,
                                self.status)
        else:
            kvc.kvc_verify_attn(self.desc, q, n_q, self.k, self.v, sl, self.table, scale, out, ws,
                                self.status)
        return out

    def dev_status(self) -> int:
        torch.cuda.synchronize()
        return int(self.status.item())

    # -- a replayable decode step ------------------------------------------
    def prepare_step(self, step=0):
        """Stage one decode step's inputs (new rows, queries) on the device.  The
        cache must already hold the cached rows (``prefill``)."""
        w = self.w
        self.s_len0 = self.seq_lens.clone()  # lengths before the step: never written
        self.s_len1 = torch.empty_like(self.seq_lens)
        self.s_cu = i32(synth.cu_from_counts([w.n_q] * w.B), self.dev)
        self.s_total = w.n_q * w.B
        self.s_k = to_dev(synth.packed_new_rows(w, "k", step), w.dtype, self.dev)
        self.s_v = None if w.dv else to_dev(synth.packed_new_rows(w, "v", step), w.dtype,
                                              self.dev)
        self.s_q = to_dev(synth.packed_queries(w, step), w.dtype, self.dev)
        self.s_out = torch.empty((w.B, w.n_q, w.Hq, w.out_dim), dtype=torch.float32,
                                 device=self.dev)
        self.s_ws = None if w.prefill else self.workspace(w.n_q)
        if self.bs:
            self.s_head0 = self.head.clone()  # free-list head before the step: never written
            self.s_head1 = torch.empty_like(self.head)
            self.s_slots = torch.empty(self.s_total, dtype=torch.int32, device=self.dev)
        else:
            self.s_slots = None

    def step_front(self):
        """Block table (paged) and append of the prepared step: one launch
        (kvc_block_table_append) for a paged cache."""
        if self.bs:
            kvc.kvc_block_table_append(self.desc, self.s_k, self.s_v, self.s_len0, self.s_cu,
                                       self.s_total, self.w.n_q, self.table, self.free_list,
                                       self.s_head0, self.s_head1, self.s_slots, self.k, self.v,
                                       self.s_len1, self.status)
        else:
            kvc.kvc_append(self.desc, self.s_k, self.s_v, self.s_len0, self.s_cu, self.s_total,
                           self.w.n_q, None, self.k, self.v, self.s_len1, self.status)

    def partition(self, q, n_q, lens, ws):
        if self.w.dv:
            kvc.kvc_mla_attn_partition(self.desc, q, n_q, self.k, lens, self.table, self.w.dv,
                                       self.scale, ws, self.status)
        else:
            kvc.kvc_attn_partition(self.desc, q, n_q, self.k, self.v, lens, self.table,
                                   self.scale, ws, self.status)

    def reduce(self, n_q, lens, ws, out):
        if self.w.dv:
            kvc.kvc_mla_attn_reduce(self.desc, n_q, self.w.dv, lens, ws, out, self.status)
        else:
            kvc.kvc_attn_reduce(self.desc, n_q, lens, ws, out, self.status)

    def prefill_attn(self, q, cu_q, total_q, max_q, lens, out):
        kvc.kvc_prefill_attn(self.desc, q, cu_q, total_q, max_q, self.k, self.v, lens, self.table,
                             self.scale, out, self.status)

    def step_partition(self):
        if self.w.prefill:  # one kernel: no split over keys, no reduce
            self.prefill_attn(self.s_q, self.s_cu, self.s_total, self.w.n_q, self.s_len1,
                              self.s_out)
        else:
            self.partition(self.s_q, self.w.n_q, self.s_len1, self.s_ws)

    def step_reduce(self):
        if not self.w.prefill:
            self.reduce(self.w.n_q, self.s_len1, self.s_ws, self.s_out)

    def attn(self, q, n_q, lens, ws, out):
        """Attention of n_q rows per sequence through the one-call entry points
        (decode / verify: one launch that also combines the partials)."""
        if self.w.dv:
            kvc.kvc_mla_attn(self.desc, q, n_q, self.k, lens, self.table, self.w.dv, self.scale,
                             out, ws, self.status)
        else:
            kvc.kvc_verify_attn(self.desc, q, n_q, self.k, self.v, lens, self.table, self.scale,
                                out, ws, self.status)

    def step_attn(self):
        """The prepared step's attention as a serving loop calls it."""
        if self.w.prefill:
            self.step_partition()
        else:
            self.attn(self.s_q, self.w.n_q, self.s_len1, self.s_ws, self.s_out)

    @property
    def fused_step(self) -> bool:
        """Decode / verify: the append (and, paged, the block table) runs inside
        the attention call (kvc_append_attn, kvc_block_table_append_attn)."""
        return not self.w.dv and not self.w.prefill

    def step(self):
        if self.fused_step:
            w = self.w
            if self.bs:
                kvc.kvc_block_table_append_attn(
                    self.desc, self.s_k, self.s_v, self.s_len0, self.s_cu, self.s_total, w.n_q,
                    self.table, self.free_list, self.s_head0, self.s_head1, self.s_slots, self.k,
                    self.v, self.s_len1, self.s_q, w.n_q, self.scale, self.s_out, self.s_ws,
                    self.status)
            else:
                kvc.kvc_append_attn(self.desc, self.s_k, self.s_v, self.s_len0, self.s_cu,
                                    self.s_total, w.n_q, self.k, self.v, self.s_len1, self.s_q,
                                    w.n_q, self.scale, self.s_out, self.s_ws, self.status)
            return self.s_out
        self.step_front()
        self.step_attn()
        return self.s_out


class DecodeLoop:
    """``w.steps`` dependent decode steps (block table, append, attention) with
    every input staged on the device.  Step s reads lengths[s] and writes
    lengths[s + 1] (and, paged, heads[s] -> heads[s + 1]), so running the loop
    again repeats exactly the same work: it can be captured once in a HIP graph
    and replayed.  The cache must already hold the cached rows."""

    def __init__(self, lc: LayerCache):
        w, dev = lc.w, lc.dev
        self.lc, self.w, self.S = lc, w, w.steps
        self.lens = [lc.seq_lens.clone()] + [torch.empty_like(lc.seq_lens) for _ in range(w.steps)]
        self.k = [to_dev(synth.packed_new_rows(w, "k", s), w.dtype, dev) for s in range(w.steps)]
        self.v = [None if w.dv else to_dev(synth.packed_new_rows(w, "v", s), w.dtype, dev)
                  for s in range(w.steps)]
        self.q = [to_dev(synth.packed_queries(w, s), w.dtype, dev) for s in range(w.steps)]
        self.out = torch.empty((w.steps, w.B, w.n_q, w.Hq, w.out_dim), dtype=torch.float32,
                               device=dev)
        self.cu = i32(synth.cu_from_counts([w.n_q] * w.B), dev)
        self.total = w.n_q * w.B
        self.ws = lc.workspace(w.n_q)
        if lc.bs:
            self.heads = [lc.head.clone()] + [torch.empty_like(lc.head) for _ in range(w.steps)]
            self.slots = [torch.empty(self.total, dtype=torch.int32, device=dev)
                          for _ in range(w.steps)]

    def run(self):
        lc, w = self.lc, self.w
        for s in range(self.S):
            if lc.bs and lc.fused_step:
                kvc.kvc_block_table_append_attn(
                    lc.desc, self.k[s], self.v[s], self.lens[s], self.cu, self.total, w.n_q,
                    lc.table, lc.free_list, self.heads[s], self.heads[s + 1], self.slots[s], lc.k,
                    lc.v, self.lens[s + 1], self.q[s], w.n_q, lc.scale, self.out[s], self.ws,
                    lc.status)
                continue
            if lc.bs:
                kvc.kvc_block_table_append(lc.desc, self.k[s], self.v[s], self.lens[s], self.cu,
                                           self.total, w.n_q, lc.table, lc.free_list,
                                           self.heads[s], self.heads[s + 1], self.slots[s], lc.k,
                                           lc.v, self.lens[s + 1], lc.status)
            elif lc.fused_step:
                kvc.kvc_append_attn(lc.desc, self.k[s], self.v[s], self.lens[s], self.cu,
                                    self.total, w.n_q, lc.k, lc.v, self.lens[s + 1], self.q[s],
                                    w.n_q, lc.scale, self.out[s], self.ws, lc.status)
                continue
            else:
                kvc.kvc_append(lc.desc, self.k[s], self.v[s], self.lens[s], self.cu, self.total,
                               w.n_q, None, lc.k, lc.v, self.lens[s + 1], lc.status)
            lc.attn(self.q[s], w.n_q, self.lens[s + 1], self.ws, self.out[s])
        return self.out

    def capture(self):
        """The whole loop as one HIP graph (through torch's graph capture)."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.run()  # warm the lazy initialisation outside the capture
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run()
        return g


def build(w: synth.Workload, step=0, **kw) -> LayerCache:
    """A full workload on the device: cached rows appended, one step prepared."""
    lc = LayerCache(w, **kw)
    lc.prefill(synth.cached_lengths(w))
    lc.prepare_step(step)
    return lc
