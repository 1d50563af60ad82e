"""CPU oracle for KV-cache decode attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The library never does: it shares no
code with the oracle, and the oracle shares none with it.

The arithmetic lives in ``kvc_oracle.c`` (plain C, double precision); this
module only marshals numpy arrays into it through ctypes and builds the shared
object with gcc when it is missing.  Each wrapper names the C function it
calls; the citations of the pages are at those C functions.

Element types: ``"bf16"`` arrays are passed as their raw 16-bit patterns
(``numpy.uint16``), ``"f32"`` arrays as ``numpy.float32``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvc_oracle.c")
_LIB = os.path.join(_HERE, "libkvc_oracle.so")

DTYPES = {"bf16": 0, "f32": 1, "f64": 2}
NP_DTYPES = {"bf16": np.uint16, "f32": np.float32, "f64": np.float64}
FP8_FORMATS = {"e4m3": 0, "e5m2": 1}


def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc into ``out`` (plain -O2, no fast-math;
    OpenMP only for the many-sequence timing function)."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-D_DEFAULT_SOURCE", "-fPIC", "-shared", "-fopenmp",
             "-Wall", "-Werror", src, "-o", tmp, "-lm"])
        os.replace(tmp, out)
    return out


class Oracle:
    """ctypes front end of one compiled oracle shared object."""

    def __init__(self, path: str | None = None):
        if path is None:
            path = build(force=False)
        self.path = path
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.kvc_ref_round_bf16.argtypes = [ctypes.c_double]
        lib.kvc_ref_round_bf16.restype = ctypes.c_uint16
        lib.kvc_ref_block_table.argtypes = [I, I, I, I, P, P, P, P, P, P]
        lib.kvc_ref_append.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P, P]
        lib.kvc_ref_gather.argtypes = [I, I, I, I, I, I, I, I, I, P, P, P]
        lib.kvc_ref_attention.argtypes = [I, I, I, I, I, I, P, P, P, ctypes.c_double, P]
        lib.kvc_ref_cache_attention.argtypes = [I, I, I, I, I, I, I, I, I, I, P, P, P, P, P,
                                                ctypes.c_double, P, P]
        lib.kvc_ref_attention_split.argtypes = [I, I, I, I, I, I, P, P, P, ctypes.c_double,
                                                I, P]
        lib.kvc_ref_fork.argtypes = [I, I, I, I, P, P, I, P, P, P]
        lib.kvc_ref_truncate.argtypes = [I, I, I, I, P, P, P, P, P, P, P]
        lib.kvc_ref_cow.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P]
        lib.kvc_ref_fp8_decode.argtypes = [I, I]
        lib.kvc_ref_fp8_decode.restype = ctypes.c_double
        lib.kvc_ref_fp8_encode.argtypes = [ctypes.c_double, I]
        lib.kvc_ref_fp8_encode.restype = ctypes.c_int
        lib.kvc_ref_fp8_max.argtypes = [I]
        lib.kvc_ref_fp8_max.restype = ctypes.c_double
        lib.kvc_ref_quantize_rows.argtypes = [P, ctypes.c_long, I, I, P, P]
        lib.kvc_ref_quantize_rows.restype = None
        lib.kvc_ref_dequantize_rows.argtypes = [P, P, ctypes.c_long, I, I, P]
        lib.kvc_ref_dequantize_rows.restype = None
        lib.kvc_ref_mla_attention.argtypes = [I, I, I, I, I, P, P, ctypes.c_double, P]
        lib.kvc_ref_attention_many.argtypes = [I, I, I, I, I, I, I, P, P, P, P, ctypes.c_double,
                                               P, P]
        for name in ("kvc_ref_attention_many", "kvc_ref_mla_attention", "kvc_ref_fork", "kvc_ref_truncate", "kvc_ref_cow",
                     "kvc_ref_block_table", "kvc_ref_append", "kvc_ref_gather",
                     "kvc_ref_attention", "kvc_ref_cache_attention",
                     "kvc_ref_attention_split"):
            getattr(lib, name).restype = ctypes.c_int
        self.lib = lib

    # -- helpers --------------------------------------------------------
    @staticmethod
    def _p(a):
        return None if a is None else a.ctypes.data_as(ctypes.c_void_p)

    @staticmethod
    def _c(a, dtype):
        a = np.ascontiguousarray(a)
        if a.dtype != dtype:
            raise TypeError("expected %s, got %s" % (np.dtype(dtype), a.dtype))
        return a

    # -- kvc_ref_round_bf16 -------------------------------------------------
    def round_bf16(self, x) -> np.ndarray:
        """Round doubles once (nearest, ties to even) to bf16 bit patterns."""
        x = np.asarray(x, dtype=np.float64)
        flat = [self.lib.kvc_ref_round_bf16(float(v)) for v in x.ravel()]
        return np.array(flat, dtype=np.uint16).reshape(x.shape)

    # -- kvc_ref_block_table ------------------------------------------------
    def block_table(self, seq_lens, cu_new, table, free_list, head, bs):
        """Returns (status, table', head', slots); inputs are not modified."""
        seq_lens = self._c(seq_lens, np.int32)
        cu_new = self._c(cu_new, np.int32)
        table = self._c(table, np.int32).copy()
        free_list = self._c(free_list, np.int32)
        B, max_blocks = table.shape
        h = np.array([head], dtype=np.int32)
        slots = np.full(max(int(cu_new[-1]), 1), -1, dtype=np.int32)
        st = self.lib.kvc_ref_block_table(B, bs, max_blocks, len(free_list), self._p(seq_lens),
                                          self._p(cu_new), self._p(table), self._p(free_list),
                                          self._p(h), self._p(slots))
        return st, table, int(h[0]), slots[:int(cu_new[-1])]

    # -- kvc_ref_append -----------------------------------------------------
    def append(self, k_new, v_new, seq_lens, cu_new, k_cache, v_cache, bs=0, slots=None):
        """In-place append into k_cache/v_cache (numpy); returns (status, seq_lens_out).

        contiguous: caches [B, Hkv, S_max, D]; paged: pools [N, Hkv, bs, D]."""
        seq_lens = self._c(seq_lens, np.int32)
        cu_new = self._c(cu_new, np.int32)
        k_new = np.ascontiguousarray(k_new)
        v_new = np.ascontiguousarray(v_new)
        assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
        B = len(seq_lens)
        Hkv, D = k_cache.shape[1], k_cache.shape[3]
        esize = k_cache.dtype.itemsize
        if bs == 0:
            S_max, N = k_cache.shape[2], 0
        else:
            S_max, N = 0, k_cache.shape[0]
            slots = self._c(slots, np.int32)
        out = np.zeros(B, dtype=np.int32)
        st = self.lib.kvc_ref_append(B, Hkv, D, esize, bs, S_max, N, self._p(k_new),
                                     self._p(v_new), self._p(seq_lens), self._p(cu_new),
                                     self._p(slots), self._p(k_cache), self._p(v_cache),
                                     self._p(out))
        return st, out

    # -- kvc_ref_gather -----------------------------------------------------
    def gather(self, cache, b, L, bs=0, table=None):
        """Sequence b's first L rows as a [Hkv, L, D] array (same dtype)."""
        Hkv, D = cache.shape[1], cache.shape[3]
        if bs == 0:
            S_max, max_blocks, N = cache.shape[2], 1, 0
        else:
            table = self._c(table, np.int32)
            S_max, max_blocks, N = 0, table.shape[1], cache.shape[0]
        out = np.zeros((Hkv, L, D), dtype=cache.dtype)
        st = self.lib.kvc_ref_gather(b, L, Hkv, D, cache.dtype.itemsize, bs, S_max, max_blocks,
                                     N, self._p(table), self._p(np.ascontiguousarray(cache)),
                                     self._p(out))
        if st != 0:
            raise ValueError("gather failed: %d" % st)
        return out

    # -- block lifecycle (kvc_ref_fork / kvc_ref_truncate / kvc_ref_cow) ------
    def fork(self, parents, children, seq_lens, table, refs, bs, N):
        """Returns (status, seq_lens', table', refs'); inputs are not modified."""
        seq_lens = self._c(seq_lens, np.int32).copy()
        table = self._c(table, np.int32).copy()
        refs = self._c(refs, np.int32).copy()
        parents = np.ascontiguousarray(parents, dtype=np.int32)
        children = np.ascontiguousarray(children, dtype=np.int32)
        B, maxb = table.shape
        st = self.lib.kvc_ref_fork(B, bs, maxb, N, self._p(parents), self._p(children),
                                   len(parents), self._p(seq_lens), self._p(table), self._p(refs))
        return st, seq_lens, table, refs

    def truncate(self, seq_lens, new_lens, table, free_list, head, refs, bs):
        """Returns (status, table', free_list', head', refs', seq_lens_out)."""
        seq_lens = self._c(seq_lens, np.int32)
        new_lens = self._c(new_lens, np.int32)
        table = self._c(table, np.int32).copy()
        free_list = self._c(free_list, np.int32).copy()
        refs = None if refs is None else self._c(refs, np.int32).copy()
        B, maxb = table.shape
        h = np.array([head], np.int32)
        out = np.zeros(B, np.int32)
        st = self.lib.kvc_ref_truncate(B, bs, maxb, len(free_list), self._p(seq_lens),
                                       self._p(new_lens), self._p(table), self._p(free_list),
                                       self._p(h), self._p(refs), self._p(out))
        return st, table, free_list, int(h[0]), refs, out

    def cow(self, seq_lens, cu_new, table, free_list, head, refs, k_pool, v_pool, bs):
        """In-place on k_pool/v_pool; returns (status, table', free_list', head', refs',
        cow_src, cow_dst)."""
        seq_lens = self._c(seq_lens, np.int32)
        cu_new = self._c(cu_new, np.int32)
        table = self._c(table, np.int32).copy()
        free_list = self._c(free_list, np.int32).copy()
        refs = self._c(refs, np.int32).copy()
        assert k_pool.flags.c_contiguous and v_pool.flags.c_contiguous
        B, maxb = table.shape
        N, Hkv, _, D = k_pool.shape
        h = np.array([head], np.int32)
        src = np.full(B, -1, np.int32)
        dst = np.full(B, -1, np.int32)
        st = self.lib.kvc_ref_cow(B, bs, maxb, N, Hkv, D, k_pool.dtype.itemsize, self._p(seq_lens),
                                  self._p(cu_new), self._p(table), self._p(free_list), self._p(h),
                                  self._p(refs), self._p(k_pool), self._p(v_pool), self._p(src),
                                  self._p(dst))
        return st, table, free_list, int(h[0]), refs, src, dst

    # -- FP8 cache: kvc_ref_fp8_decode / _encode / quantize / dequantize ------
    def fp8_decode(self, codes, fmt) -> np.ndarray:
        """Values of FP8 codes (float64); fmt "e4m3" or "e5m2"."""
        f = FP8_FORMATS[fmt]
        c = np.asarray(codes, dtype=np.int64)
        return np.array([self.lib.kvc_ref_fp8_decode(int(x), f) for x in c.ravel()],
                        dtype=np.float64).reshape(c.shape)

    def fp8_encode(self, values, fmt) -> np.ndarray:
        """Nearest FP8 codes (ties to even, saturating) of finite values."""
        f = FP8_FORMATS[fmt]
        v = np.asarray(values, dtype=np.float64)
        return np.array([self.lib.kvc_ref_fp8_encode(float(x), f) for x in v.ravel()],
                        dtype=np.uint8).reshape(v.shape)

    def fp8_max(self, fmt) -> float:
        return float(self.lib.kvc_ref_fp8_max(FP8_FORMATS[fmt]))

    def quantize_rows(self, x_bits, fmt):
        """bf16 bit patterns [..., D] -> (codes uint8 [..., D], scales float32 [...])."""
        x = self._c(x_bits, np.uint16)
        D = x.shape[-1]
        n = x.size // D if D else 0
        codes = np.zeros(x.shape, np.uint8)
        scales = np.zeros(x.shape[:-1], np.float32)
        self.lib.kvc_ref_quantize_rows(self._p(x), n, D, FP8_FORMATS[fmt], self._p(codes),
                                       self._p(scales))
        return codes, scales

    def dequantize_rows(self, codes, scales, fmt) -> np.ndarray:
        """(codes [..., D], scales [...]) -> float64 values [..., D]."""
        c = self._c(codes, np.uint8)
        sc = self._c(scales, np.float32)
        assert sc.shape == c.shape[:-1]
        D = c.shape[-1]
        out = np.zeros(c.shape, np.float64)
        self.lib.kvc_ref_dequantize_rows(self._p(c), self._p(sc), c.size // D if D else 0, D,
                                         FP8_FORMATS[fmt], self._p(out))
        return out

    # -- kvc_ref_mla_attention ----------------------------------------------
    def mla_attention(self, q, c, scale, dv):
        """q [n_q, Hq, Dk], c [L, Dk] (bf16 bits) -> out [n_q, Hq, dv] float64:
        attention over latent rows (keys = whole rows, values = first dv dims)."""
        q, c = self._c(q, np.uint16), self._c(c, np.uint16)
        n_q, Hq, Dk = q.shape
        L = c.shape[0]
        out = np.zeros((n_q, Hq, dv), dtype=np.float64)
        st = self.lib.kvc_ref_mla_attention(n_q, Hq, Dk, dv, L, self._p(q), self._p(c),
                                            float(scale), self._p(out))
        if st != 0:
            raise ValueError("mla_attention failed: %d" % st)
        return out

    # -- kvc_ref_attention --------------------------------------------------
    def attention(self, q, k, v, scale, dtype):
        """q [n_q, Hq, D], k/v [Hkv, L, D] -> out [n_q, Hq, D] float64."""
        nd = NP_DTYPES[dtype]
        q, k, v = self._c(q, nd), self._c(k, nd), self._c(v, nd)
        n_q, Hq, D = q.shape
        Hkv, L, _ = k.shape
        out = np.zeros((n_q, Hq, D), dtype=np.float64)
        st = self.lib.kvc_ref_attention(n_q, Hq, Hkv, D, L, DTYPES[dtype], self._p(q),
                                        self._p(k), self._p(v), float(scale), self._p(out))
        if st != 0:
            raise ValueError("attention failed: %d" % st)
        return out

    # -- kvc_ref_attention_many ---------------------------------------------
    def attention_many(self, qs, ks, vs, scale, dtype, dv=0):
        """Several sequences at once on all host cores (one OpenMP iteration per
        (sequence, query head)): qs[s] [n_q, Hq, Dk], ks[s]/vs[s] [Hkv, L_s, Dk]
        (MLA, dv > 0: ks[s] = latent rows [L_s, Dk], vs ignored) -> (list of
        out [n_q, Hq, Dout] float64, threads used)."""
        nd = NP_DTYPES[dtype]
        qs = [self._c(q, nd) for q in qs]
        ks = [self._c(k, nd) for k in ks]
        vs = [self._c(v, nd) for v in vs] if not dv else ks
        n = len(qs)
        if n == 0:
            return [], 0
        n_q, Hq, Dk = qs[0].shape
        Hkv = 1 if dv else ks[0].shape[0]
        L = np.array([k.shape[0] if dv else k.shape[1] for k in ks], dtype=np.int32)
        outs = [np.zeros((n_q, Hq, dv or Dk), dtype=np.float64) for _ in range(n)]
        arr = lambda xs: (ctypes.c_void_p * n)(*[x.ctypes.data for x in xs])
        threads = ctypes.c_int(0)
        st = self.lib.kvc_ref_attention_many(n, n_q, Hq, Hkv, Dk, dv, DTYPES[dtype], self._p(L),
                                             arr(qs), arr(ks), arr(vs), float(scale), arr(outs),
                                             ctypes.byref(threads))
        if st != 0:
            raise ValueError("attention_many failed: %d" % st)
        return outs, threads.value

    # -- kvc_ref_attention_split --------------------------------------------
    def attention_split(self, q, k, v, scale, dtype, P):
        nd = NP_DTYPES[dtype]
        q, k, v = self._c(q, nd), self._c(k, nd), self._c(v, nd)
        n_q, Hq, D = q.shape
        Hkv, L, _ = k.shape
        out = np.zeros((n_q, Hq, D), dtype=np.float64)
        st = self.lib.kvc_ref_attention_split(n_q, Hq, Hkv, D, L, DTYPES[dtype], self._p(q),
                                              self._p(k), self._p(v), float(scale), int(P),
                                              self._p(out))
        if st != 0:
            raise ValueError("attention_split failed: %d" % st)
        return out

    # -- kvc_ref_cache_attention --------------------------------------------
    def cache_attention(self, q, k_cache, v_cache, seq_lens, scale, dtype, bs=0, table=None,
                        rows_only=None):
        """q [B, n_q, Hq, D] over a contiguous [B,Hkv,S_max,D] or paged [N,Hkv,bs,D]
        cache -> (status, out [B, n_q, Hq, D] float64)."""
        nd = NP_DTYPES[dtype]
        q = self._c(q, nd)
        B, n_q, Hq, D = q.shape
        Hkv = k_cache.shape[1]
        seq_lens = self._c(seq_lens, np.int32)
        if bs == 0:
            S_max, max_blocks, N = k_cache.shape[2], 1, 0
        else:
            table = self._c(table, np.int32)
            S_max, max_blocks, N = 0, table.shape[1], k_cache.shape[0]
        ro = None
        if rows_only is not None:
            ro = self._c(np.asarray(rows_only, dtype=np.uint8).reshape(B, Hq), np.uint8)
        out = np.zeros((B, n_q, Hq, D), dtype=np.float64)
        st = self.lib.kvc_ref_cache_attention(
            B, n_q, Hq, Hkv, D, DTYPES[dtype], bs, S_max, max_blocks, N, self._p(q),
            self._p(self._c(k_cache, nd)), self._p(self._c(v_cache, nd)), self._p(seq_lens),
            self._p(table), float(scale), self._p(ro), self._p(out))
        return st, out


_default = None


def get() -> Oracle:
    """The oracle built from this directory's source (compiled on first use)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def widen(a, dtype) -> np.ndarray:
    """Exact float64 view of stored elements (bf16 bit patterns or float32)."""
    a = np.asarray(a)
    if dtype == "f32":
        return a.astype(np.float64)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
