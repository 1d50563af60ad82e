"""Seeded synthetic workloads: shapes, lengths and random rows.

This module is shared by the tests, the benchmark and the smoke check.  It
holds no step of the method (no attention, no block allocation, no append):
only the sizes of each workload and the random numbers that fill it, so that
the HIP path and the CPU oracle are fed bit-identical inputs.

Random streams: every array is drawn from
``numpy.random.default_rng([seed, stream, *ids])`` so any one sequence can be
regenerated alone.  Stream ids: 0 lengths, 1 pool permutation, 2 cached keys,
3 cached values, 4 queries, 5 new keys, 6 new values.  Values are float32
N(0, 1) draws, stored as bfloat16 by rounding to nearest even where the
workload is bf16.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

S_LENGTHS, S_POOL, S_KCACHE, S_VCACHE, S_Q, S_KNEW, S_VNEW = range(7)


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    Hq: int
    Hkv: int
    D: int
    dtype: str  # "bf16" | "f32"
    block_size: int  # 0 = contiguous cache
    n_q: int  # query rows (= new tokens) per sequence per step
    len_lo: int  # attended length range after the step's append, inclusive
    len_hi: int
    steps: int = 1  # successive decode steps (the cache grows by n_q each step)
    description: str = ""
    kv: str = ""  # "": the cache holds dtype; "e4m3" / "e5m2": FP8 codes + a scale per row
    dv: int = 0   # MLA: value dims of a latent row (its leading dims); 0 = separate K and V
    prefill: bool = False  # the step's n_q new rows attend causally (kvc_prefill_attn)

    @property
    def esize(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    @property
    def cache_dtype(self) -> str:
        return "fp8_" + self.kv if self.kv else self.dtype

    @property
    def kv_tensors(self) -> int:
        """Cache tensors read per attended row: K and V, or one latent row (MLA)."""
        return 1 if self.dv else 2

    @property
    def out_dim(self) -> int:
        return self.dv or self.D

    @property
    def kv_row_bytes(self) -> int:
        """Cache bytes of one row (token, KV head) of K (the same for V): FP8
        codes plus the row's float32 scale, or the plain elements."""
        return self.D + 4 if self.kv else self.D * self.esize

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


WORKLOADS = {w.name: w for w in [
    Workload("gptlite-f32-b2-h4-d64-ctx256-32steps", seed=1, B=2, Hq=4, Hkv=4, D=64, dtype="f32",
             block_size=0, n_q=1, len_lo=257, len_hi=257, steps=32,
             description="tiny GPTlite-shaped layer: 256 cached tokens + 1, then 32 decode "
                         "steps, contiguous fp32 cache"),
    Workload("llama2-13b-layer-contig-b16-ctx2048", seed=2, B=16, Hq=40, Hkv=40, D=128,
             dtype="bf16", block_size=0, n_q=1, len_lo=2048, len_hi=2048,
             description="Llama-2-13B-shaped layer decode, contiguous bf16 cache, batch 16, "
                         "context 2048"),
    Workload("mha40-paged-b64-ctx128to4096", seed=3, B=64, Hq=40, Hkv=40, D=128, dtype="bf16",
             block_size=16, n_q=1, len_lo=128, len_hi=4096,
             description="40-head MHA paged decode, block 16, batch 64, lengths U[128, 4096]"),
    Workload("gqa32x8-paged-b128-ctx256to8192", seed=4, B=128, Hq=32, Hkv=8, D=128,
             dtype="bf16", block_size=16, n_q=1, len_lo=256, len_hi=8192,
             description="GQA 32 q / 8 kv heads paged decode, block 16, batch 128, lengths "
                         "U[256, 8192]"),
    Workload("verify5-gqa32x8-paged-b32-ctx1024to4096", seed=5, B=32, Hq=32, Hkv=8, D=128,
             dtype="bf16", block_size=16, n_q=5, len_lo=1024 + 5, len_hi=4096 + 5,
             description="speculative verify: 4 drafts + 1, GQA 32/8, paged block 16, batch 32, "
                         "cached lengths U[1024, 4096]"),
]}

# short aliases, in the order the workloads are listed above
ALIASES = {"C%d" % (i + 1): n for i, n in enumerate(WORKLOADS)}

# MLA latent decode (DeepSeek-V2/V3 geometry: latent 512 + RoPE key 64, one
# latent head shared by all query heads, block 64): all 128 heads on one GPU,
# and the 16 heads of one GPU when the heads are split 8 ways.
for _w in [
    Workload("mla-h128-paged64-b32-ctx1024to4096", seed=7, B=32, Hq=128, Hkv=1, D=576,
             dtype="bf16", block_size=64, n_q=1, len_lo=1024, len_hi=4096,
             description="MLA latent decode, 128 heads on one latent head of 576 (512 + 64 "
                         "RoPE), paged block 64, batch 32, lengths U[1024, 4096]", dv=512),
    Workload("mla-h16-paged64-b128-ctx1024to8192", seed=8, B=128, Hq=16, Hkv=1, D=576,
             dtype="bf16", block_size=64, n_q=1, len_lo=1024, len_hi=8192,
             description="MLA latent decode, 16 heads (128 split 8 ways), paged block 64, "
                         "batch 128, lengths U[1024, 8192]", dv=512),
]:
    WORKLOADS[_w.name] = _w
ALIASES["M1"], ALIASES["M2"] = ("mla-h128-paged64-b32-ctx1024to4096",
                                "mla-h16-paged64-b128-ctx1024to8192")

# Prefill and chunked prefill (GQA 32/8, head 128, paged block 16): a whole
# 4096-token prompt for 4 sequences, and 512-token chunks on top of 3584
# cached tokens for 16 sequences.
for _w in [
    Workload("prefill-gqa32x8-paged-b4-prompt4096", seed=9, B=4, Hq=32, Hkv=8, D=128,
             dtype="bf16", block_size=16, n_q=4096, len_lo=4096, len_hi=4096,
             description="prefill of a 4096-token prompt, GQA 32/8, head 128, paged block 16, "
                         "batch 4", prefill=True),
    Workload("chunked-prefill-gqa32x8-paged-b16-chunk512-ctx4096", seed=10, B=16, Hq=32,
             Hkv=8, D=128, dtype="bf16", block_size=16, n_q=512, len_lo=4096, len_hi=4096,
             description="chunked prefill: 512-token chunks over 3584 cached tokens, GQA "
                         "32/8, head 128, paged block 16, batch 16", prefill=True),
]:
    WORKLOADS[_w.name] = _w
ALIASES["P1"], ALIASES["P2"] = ("prefill-gqa32x8-paged-b4-prompt4096",
                                "chunked-prefill-gqa32x8-paged-b16-chunk512-ctx4096")

# The same four full-size workloads over an FP8 (E4M3) cache: same seeds, so the
# same lengths and rows, quantized on append.
for _i in range(2, 6):
    _w = WORKLOADS[ALIASES["C%d" % _i]]
    _f = Workload(_w.name + "-fp8e4m3", _w.seed, _w.B, _w.Hq, _w.Hkv, _w.D, _w.dtype,
                  _w.block_size, _w.n_q, _w.len_lo, _w.len_hi, _w.steps,
                  _w.description + "; FP8 E4M3 cache, one scale per row", kv="e4m3")
    WORKLOADS[_f.name] = _f
    ALIASES["C%dF8" % _i] = _f.name


def get(name: str) -> Workload:
    return WORKLOADS[ALIASES.get(name, name)]


def rng(w: Workload, stream: int, *ids: int) -> np.random.Generator:
    return np.random.default_rng([w.seed, stream, *ids])


def to_bf16_bits(x: np.ndarray, out: np.ndarray | None = None) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    u = np.array(x, dtype=np.float32, copy=True).view(np.uint32)
    t = u >> 16
    t &= 1
    t += 0x7FFF
    u += t
    u >>= 16
    if out is None:
        return u.astype(np.uint16)
    out[...] = u
    return out


def encode(x: np.ndarray, dtype: str) -> np.ndarray:
    return to_bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def normal(w: Workload, shape, stream: int, *ids: int) -> np.ndarray:
    return encode(rng(w, stream, *ids).standard_normal(shape, dtype=np.float32), w.dtype)


def final_lengths(w: Workload) -> np.ndarray:
    """Attended length of every sequence after the first step's append."""
    if w.len_lo == w.len_hi:
        return np.full(w.B, w.len_lo, dtype=np.int32)
    return rng(w, S_LENGTHS).integers(w.len_lo, w.len_hi + 1, size=w.B).astype(np.int32)


def cached_lengths(w: Workload) -> np.ndarray:
    """Tokens already in the cache before the first step."""
    return final_lengths(w) - w.n_q


def capacity_tokens(w: Workload) -> int:
    """Longest sequence after all steps: the contiguous cache's S_max."""
    return int(final_lengths(w).max()) + (w.steps - 1) * w.n_q


def max_blocks_per_seq(w: Workload) -> int:
    bs = w.block_size
    return (capacity_tokens(w) + bs - 1) // bs


def pool_blocks(w: Workload) -> int:
    """Pool size: every sequence's blocks after all steps, plus one spare each."""
    bs = w.block_size
    last = final_lengths(w) + (w.steps - 1) * w.n_q
    return int(((last + bs - 1) // bs).sum()) + w.B


def free_list(w: Workload) -> np.ndarray:
    return rng(w, S_POOL).permutation(pool_blocks(w)).astype(np.int32)


def cache_rows(w: Workload, which: str, b: int, n: int) -> np.ndarray:
    """The n cached key (which='k') or value ('v') rows of sequence b: [n, Hkv, D]."""
    return normal(w, (n, w.Hkv, w.D), S_KCACHE if which == "k" else S_VCACHE, b)


def new_rows(w: Workload, which: str, b: int, step: int = 0) -> np.ndarray:
    """The n_q new key/value rows of sequence b at a decode step: [n_q, Hkv, D]."""
    return normal(w, (w.n_q, w.Hkv, w.D), S_KNEW if which == "k" else S_VNEW, b, step)


def queries(w: Workload, b: int, step: int = 0) -> np.ndarray:
    """Sequence b's query rows at a decode step: [n_q, Hq, D]."""
    return normal(w, (w.n_q, w.Hq, w.D), S_Q, b, step)


def cu_from_counts(counts) -> np.ndarray:
    """[B] token counts -> [B+1] offsets into a packed token array."""
    cu = np.zeros(len(counts) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(counts, dtype=np.int64))
    return cu


def packed_cache_rows(w: Workload, which: str, lengths, threads: int = 16) -> np.ndarray:
    """All sequences' cached rows packed in batch order: [sum(lengths), Hkv, D].
    Sequences are drawn in parallel threads (each from its own stream)."""
    cu = cu_from_counts(lengths)
    out = np.empty((int(cu[-1]), w.Hkv, w.D), dtype=np.uint16 if w.dtype == "bf16" else np.float32)
    stream = S_KCACHE if which == "k" else S_VCACHE

    def fill(b):
        n = int(cu[b + 1] - cu[b])
        x = rng(w, stream, b).standard_normal((n, w.Hkv, w.D), dtype=np.float32)
        if w.dtype == "bf16":
            to_bf16_bits(x, out[cu[b]:cu[b + 1]])
        else:
            out[cu[b]:cu[b + 1]] = x

    with ThreadPoolExecutor(max_workers=max(1, min(threads, os.cpu_count() or 1))) as ex:
        list(ex.map(fill, range(len(lengths))))
    return out


def packed_new_rows(w: Workload, which: str, step: int = 0) -> np.ndarray:
    return np.concatenate([new_rows(w, which, b, step) for b in range(w.B)], axis=0)


def packed_queries(w: Workload, step: int = 0) -> np.ndarray:
    """[B, n_q, Hq, D]"""
    return np.stack([queries(w, b, step) for b in range(w.B)], axis=0)


def custom(name="custom", seed=0, B=2, Hq=4, Hkv=4, D=64, dtype="bf16", block_size=0, n_q=1,
           len_lo=16, len_hi=16, steps=1, kv="", dv=0, prefill=False) -> Workload:
    """A small workload for tests (same generators, other sizes)."""
    return Workload(name, seed, B, Hq, Hkv, D, dtype, block_size, n_q, len_lo, len_hi, steps,
                    kv=kv, dv=dv, prefill=prefill)
