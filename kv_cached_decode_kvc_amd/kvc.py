"""Thin Python binding of libkvc.so (``include/kvc.h``): argument marshalling only.

Every function has the name and argument order of its C entry point; tensors
are torch device tensors (their ``data_ptr()`` is passed) and ``stream``
defaults to torch's current HIP stream.  Every step of the computation runs
in the library's HIP kernels.  A missing ``libkvc.so`` raises immediately:
there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvc.so")

KVC_BF16, KVC_F32, KVC_FP8_E4M3, KVC_FP8_E5M2 = 0, 1, 2, 3
DTYPE_CODES = {"bf16": KVC_BF16, "f32": KVC_F32, "fp8_e4m3": KVC_FP8_E4M3,
               "fp8_e5m2": KVC_FP8_E5M2}
KVC_OK = 0
STATUS_NAMES = {0: "KVC_OK", -1: "KVC_ERR_ARG", -2: "KVC_ERR_SHAPE", -3: "KVC_ERR_UNSUPPORTED",
                -4: "KVC_ERR_WORKSPACE", -5: "KVC_ERR_CAPACITY", -6: "KVC_ERR_NO_BLOCKS",
                -7: "KVC_ERR_HIP", -8: "KVC_ERR_DATA"}
EXPORTS = ("kvc_block_table", "kvc_append", "kvc_decode_attn", "kvc_verify_attn",
           "kvc_attn_partition", "kvc_attn_reduce", "kvc_attn_workspace_bytes",
           "kvc_fork", "kvc_truncate", "kvc_cow", "kvc_copy_blocks",
           "kvc_attn_partition_tokens", "kvc_attn_launches", "kvc_cache_bytes",
           "kvc_mla_workspace_bytes", "kvc_mla_partition_tokens", "kvc_mla_attn_partition", "kvc_mla_attn_reduce",
           "kvc_mla_attn", "kvc_prefill_attn", "kvc_status_string", "kvc_verify_attn_noalloc",
           "kvc_block_table_append", "kvc_append_attn", "kvc_block_table_append_attn")
NOALLOC_SCRATCH_BYTES = 64 << 20  # KVC_NOALLOC_SCRATCH_BYTES


class KvcError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__("%s: %s (%d)" % (fn, STATUS_NAMES.get(status, "?"), status))


class kvc_cache_desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "num_q_heads", "num_kv_heads", "head_dim", "dtype", "block_size",
        "max_seq_len", "max_blocks_per_seq", "num_blocks", "partition_tokens")]


def cache_desc(batch, num_q_heads, num_kv_heads, head_dim, dtype, block_size=0, max_seq_len=0,
               max_blocks_per_seq=0, num_blocks=0, partition_tokens=0) -> kvc_cache_desc:
    if isinstance(dtype, str):
        dtype = DTYPE_CODES[dtype]
    return kvc_cache_desc(batch, num_q_heads, num_kv_heads, head_dim, dtype, block_size,
                          max_seq_len, max_blocks_per_seq, num_blocks, partition_tokens)


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libkvc.so is not built (%s); run "
                              "`python -m kv_cached_decode_kvc_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P, I, D = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(kvc_cache_desc)
        L.kvc_block_table.argtypes = [D, P, P, I, P, P, P, P, P, P, P]
        L.kvc_append.argtypes = [D, P, P, P, P, I, I, P, P, P, P, P, P]
        L.kvc_decode_attn.argtypes = [D, P, P, P, P, P, ctypes.c_float, P, I, P, ctypes.c_size_t,
                                      P, P]
        L.kvc_verify_attn.argtypes = [D, P, I, P, P, P, P, ctypes.c_float, P, I, P,
                                      ctypes.c_size_t, P, P]
        L.kvc_attn_partition.argtypes = [D, P, I, P, P, P, P, ctypes.c_float, P, ctypes.c_size_t,
                                         P, P]
        L.kvc_block_table_append.argtypes = [D, P, P, P, P, I, I, P, P, P, P, P, P, P, P, P, P]
        L.kvc_block_table_append.restype = ctypes.c_int
        L.kvc_append_attn.argtypes = [D, P, P, P, P, I, I, P, P, P, P, I, ctypes.c_float, P, I, P,
                                      ctypes.c_size_t, P, P]
        L.kvc_append_attn.restype = ctypes.c_int
        L.kvc_block_table_append_attn.argtypes = [D, P, P, P, P, I, I, P, P, P, P, P, P, P, P, P,
                                                  I, ctypes.c_float, P, I, P, ctypes.c_size_t, P,
                                                  P]
        L.kvc_block_table_append_attn.restype = ctypes.c_int
        L.kvc_verify_attn_noalloc.argtypes = [D, P, I, P, P, P, P, ctypes.c_float, P, I, P, P]
        L.kvc_verify_attn_noalloc.restype = ctypes.c_int
        L.kvc_attn_reduce.argtypes = [D, I, P, P, ctypes.c_size_t, P, I, P, P]
        L.kvc_fork.argtypes = [D, P, P, I, P, P, P, P, P]
        L.kvc_truncate.argtypes = [D, P, P, P, P, P, P, P, P, P, P]
        L.kvc_cow.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, P, P]
        L.kvc_copy_blocks.argtypes = [D, P, P, I, P, P, P, P]
        for n in EXPORTS[:6] + ("kvc_fork", "kvc_truncate", "kvc_cow", "kvc_copy_blocks"):
            getattr(L, n).restype = ctypes.c_int
        L.kvc_attn_workspace_bytes.argtypes = [D, I]
        L.kvc_attn_workspace_bytes.restype = ctypes.c_size_t
        L.kvc_mla_workspace_bytes.argtypes = [D, I, I]
        L.kvc_mla_workspace_bytes.restype = ctypes.c_size_t
        L.kvc_mla_partition_tokens.argtypes = [D, I, I]
        L.kvc_mla_partition_tokens.restype = ctypes.c_int32
        L.kvc_mla_attn_partition.argtypes = [D, P, I, P, P, P, I, ctypes.c_float, P,
                                             ctypes.c_size_t, P, P]
        L.kvc_mla_attn_reduce.argtypes = [D, I, I, P, P, ctypes.c_size_t, P, I, P, P]
        L.kvc_mla_attn.argtypes = [D, P, I, P, P, P, I, ctypes.c_float, P, I, P, ctypes.c_size_t,
                                   P, P]
        L.kvc_prefill_attn.argtypes = [D, P, P, I, I, P, P, P, P, ctypes.c_float, P, I, P, P]
        for n in ("kvc_mla_attn_partition", "kvc_mla_attn_reduce", "kvc_mla_attn",
                  "kvc_prefill_attn"):
            getattr(L, n).restype = ctypes.c_int
        L.kvc_cache_bytes.argtypes = [D]
        L.kvc_cache_bytes.restype = ctypes.c_size_t
        L.kvc_attn_partition_tokens.argtypes = [D, I]
        L.kvc_attn_partition_tokens.restype = ctypes.c_int32
        L.kvc_attn_launches.argtypes = [D, I]
        L.kvc_attn_launches.restype = ctypes.c_int32
        L.kvc_status_string.argtypes = [I]
        L.kvc_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _ptr(t, name, dtype=None):
    """Device address of a contiguous device tensor (None -> NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must live in device memory" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _out_dtype(out, out_dtype):
    if out_dtype is not None:
        return out_dtype
    return KVC_BF16 if out.dtype == torch.bfloat16 else KVC_F32


def _check(fn, st):
    if st != KVC_OK:
        raise KvcError(fn, st)


I32 = torch.int32


def kvc_block_table(desc, seq_lens, cu_new, total_new, block_table, free_list, free_head_in,
                    free_head_out, slot_mapping, dev_status=None, stream=None):
    _check("kvc_block_table", lib().kvc_block_table(
        ctypes.byref(desc), _ptr(seq_lens, "seq_lens", I32), _ptr(cu_new, "cu_new", I32),
        int(total_new), _ptr(block_table, "block_table", I32), _ptr(free_list, "free_list", I32),
        _ptr(free_head_in, "free_head_in", I32), _ptr(free_head_out, "free_head_out", I32),
        _ptr(slot_mapping, "slot_mapping", I32), _ptr(dev_status, "dev_status", I32),
        _stream(stream)))


def kvc_append(desc, k_new, v_new, seq_lens, cu_new, total_new, max_new, slot_mapping, k_cache,
               v_cache, seq_lens_out, dev_status=None, stream=None):
    _check("kvc_append", lib().kvc_append(
        ctypes.byref(desc), _ptr(k_new, "k_new"), _ptr(v_new, "v_new"),
        _ptr(seq_lens, "seq_lens", I32), _ptr(cu_new, "cu_new", I32), int(total_new), int(max_new),
        _ptr(slot_mapping, "slot_mapping", I32), _ptr(k_cache, "k_cache"), _ptr(v_cache, "v_cache"),
        _ptr(seq_lens_out, "seq_lens_out", I32), _ptr(dev_status, "dev_status", I32),
        _stream(stream)))


def kvc_decode_attn(desc, q, k_cache, v_cache, seq_lens, block_table, scale, out, workspace,
                    dev_status=None, stream=None, out_dtype=None):
    _check("kvc_decode_attn", lib().kvc_decode_attn(
        ctypes.byref(desc), _ptr(q, "q"), _ptr(k_cache, "k_cache"), _ptr(v_cache, "v_cache"),
        _ptr(seq_lens, "seq_lens", I32), _ptr(block_table, "block_table", I32), float(scale),
        _ptr(out, "out"), _out_dtype(out, out_dtype), _ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _ptr(dev_status, "dev_status", I32),
        _stream(stream)))


def kvc_verify_attn(desc, q, n_q, k_cache, v_cache, seq_lens, block_table, scale, out, workspace,
                    dev_status=None, stream=None, out_dtype=None):
    _check("kvc_verify_attn", lib().kvc_verify_attn(
        ctypes.byref(desc), _ptr(q, "q"), int(n_q), _ptr(k_cache, "k_cache"),
        _ptr(v_cache, "v_cache"), _ptr(seq_lens, "seq_lens", I32),
        _ptr(block_table, "block_table", I32), float(scale), _ptr(out, "out"),
        _out_dtype(out, out_dtype), _ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _ptr(dev_status, "dev_status", I32),
        _stream(stream)))


def kvc_block_table_append(desc, k_new, v_new, seq_lens, cu_new, total_new, max_new, block_table,
                           free_list, free_head_in, free_head_out, slot_mapping, k_cache, v_cache,
                           seq_lens_out, dev_status=None, stream=None):
    _check("kvc_block_table_append", lib().kvc_block_table_append(
        ctypes.byref(desc), _ptr(k_new, "k_new"), _ptr(v_new, "v_new"),
        _ptr(seq_lens, "seq_lens", I32), _ptr(cu_new, "cu_new", I32), int(total_new),
        int(max_new), _ptr(block_table, "block_table", I32), _ptr(free_list, "free_list", I32),
        _ptr(free_head_in, "free_head_in", I32), _ptr(free_head_out, "free_head_out", I32),
        _ptr(slot_mapping, "slot_mapping", I32), _ptr(k_cache, "k_cache"),
        _ptr(v_cache, "v_cache"), _ptr(seq_lens_out, "seq_lens_out", I32),
        _ptr(dev_status, "dev_status", I32), _stream(stream)))


def kvc_append_attn(desc, k_new, v_new, seq_lens, cu_new, total_new, max_new, k_cache, v_cache,
                    seq_lens_out, q, n_q, scale, out, workspace, dev_status=None, stream=None,
                    out_dtype=None):
    _check("kvc_append_attn", lib().kvc_append_attn(
        ctypes.byref(desc), _ptr(k_new, "k_new"), _ptr(v_new, "v_new"),
        _ptr(seq_lens, "seq_lens", I32), _ptr(cu_new, "cu_new", I32), int(total_new),
        int(max_new), _ptr(k_cache, "k_cache"), _ptr(v_cache, "v_cache"),
        _ptr(seq_lens_out, "seq_lens_out", I32), _ptr(q, "q"), int(n_q), float(scale),
        _ptr(out, "out"), _out_dtype(out, out_dtype), _ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _ptr(dev_status, "dev_status", I32),
        _stream(stream)))


def kvc_block_table_append_attn(desc, k_new, v_new, seq_lens, cu_new, total_new, max_new,
                                block_table, free_list, free_head_in, free_head_out, slot_mapping,
                                k_cache, v_cache, seq_lens_out, q, n_q, scale, out, workspace,
                                dev_status=None, stream=None, out_dtype=None):
    _check("kvc_block_table_append_attn", lib().kvc_block_table_append_attn(
        ctypes.byref(desc), _ptr(k_new, "k_new"), _ptr(v_new, "v_new"),
        _ptr(seq_lens, "seq_lens", I32), _ptr(cu_new, "cu_new", I32), int(total_new),
        int(max_new), _ptr(block_table, "block_table", I32), _ptr(free_list, "free_list", I32),
        _ptr(free_head_in, "free_head_in", I32), _ptr(free_head_out, "free_head_out", I32),
        _ptr(slot_mapping, "slot_mapping", I32), _ptr(k_cache, "k_cache"),
        _ptr(v_cache, "v_cache"), _ptr(seq_lens_out, "seq_lens_out", I32), _ptr(q, "q"),
        int(n_q), float(scale), _ptr(out, "out"), _out_dtype(out, out_dtype),
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _ptr(dev_status, "dev_status", I32), _stream(stream)))


def kvc_verify_attn_noalloc(desc, q, n_q, k_cache, v_cache, seq_lens, block_table, scale, out,
                            dev_status=None, stream=None, out_dtype=None):
    _check("kvc_verify_attn_noalloc", lib().kvc_verify_attn_noalloc(
        ctypes.byref(desc), _ptr(q, "q"), int(n_q), _ptr(k_cache, "k_cache"),
        _ptr(v_cache, "v_cache"), _ptr(seq_lens, "seq_lens", I32),
        _ptr(block_table, "block_table", I32), float(scale), _ptr(out, "out"),
        _out_dtype(out, out_dtype), _ptr(dev_status, "dev_status", I32), _stream(stream)))


def kvc_attn_partition(desc, q, n_q, k_cache, v_cache, seq_lens, block_table, scale, workspace,
                       dev_status=None, stream=None):
    _check("kvc_attn_partition", lib().kvc_attn_partition(
        ctypes.byref(desc), _ptr(q, "q"), int(n_q), _ptr(k_cache, "k_cache"),
        _ptr(v_cache, "v_cache"), _ptr(seq_lens, "seq_lens", I32),
        _ptr(block_table, "block_table", I32), float(scale), _ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _ptr(dev_status, "dev_status", I32),
        _stream(stream)))


def kvc_attn_reduce(desc, n_q, seq_lens, workspace, out, dev_status=None, stream=None,
                    out_dtype=None):
    _check("kvc_attn_reduce", lib().kvc_attn_reduce(
        ctypes.byref(desc), int(n_q), _ptr(seq_lens, "seq_lens", I32), _ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _ptr(out, "out"), _out_dtype(out, out_dtype),
        _ptr(dev_status, "dev_status", I32), _stream(stream)))


def kvc_fork(desc, parents, children, n_forks, seq_lens, block_table, ref_counts,
             dev_status=None, stream=None):
    _check("kvc_fork", lib().kvc_fork(
        ctypes.byref(desc), _ptr(parents, "parents", I32), _ptr(children, "children", I32),
        int(n_forks), _ptr(seq_lens, "seq_lens", I32), _ptr(block_table, "block_table", I32),
        _ptr(ref_counts, "ref_counts", I32), _ptr(dev_status, "dev_status", I32),
        _stream(stream)))


def kvc_truncate(desc, seq_lens, new_lens, block_table, free_list, free_head_in, free_head_out,
                 ref_counts, seq_lens_out, dev_status=None, stream=None):
    _check("kvc_truncate", lib().kvc_truncate(
        ctypes.byref(desc), _ptr(seq_lens, "seq_lens", I32), _ptr(new_lens, "new_lens", I32),
        _ptr(block_table, "block_table", I32), _ptr(free_list, "free_list", I32),
        _ptr(free_head_in, "free_head_in", I32), _ptr(free_head_out, "free_head_out", I32),
        _ptr(ref_counts, "ref_counts", I32), _ptr(seq_lens_out, "seq_lens_out", I32),
        _ptr(dev_status, "dev_status", I32), _stream(stream)))


def kvc_cow(desc, seq_lens, cu_new, block_table, free_list, free_head_in, free_head_out,
            ref_counts, k_cache, v_cache, cow_src, cow_dst, dev_status=None, stream=None):
    _check("kvc_cow", lib().kvc_cow(
        ctypes.byref(desc), _ptr(seq_lens, "seq_lens", I32), _ptr(cu_new, "cu_new", I32),
        _ptr(block_table, "block_table", I32), _ptr(free_list, "free_list", I32),
        _ptr(free_head_in, "free_head_in", I32), _ptr(free_head_out, "free_head_out", I32),
        _ptr(ref_counts, "ref_counts", I32), _ptr(k_cache, "k_cache"), _ptr(v_cache, "v_cache"),
        _ptr(cow_src, "cow_src", I32), _ptr(cow_dst, "cow_dst", I32),
        _ptr(dev_status, "dev_status", I32), _stream(stream)))


def kvc_copy_blocks(desc, src, dst, n, k_cache, v_cache, dev_status=None, stream=None):
    _check("kvc_copy_blocks", lib().kvc_copy_blocks(
        ctypes.byref(desc), _ptr(src, "src", I32), _ptr(dst, "dst", I32), int(n),
        _ptr(k_cache, "k_cache"), _ptr(v_cache, "v_cache"), _ptr(dev_status, "dev_status", I32),
        _stream(stream)))


def kvc_attn_workspace_bytes(desc, n_q) -> int:
    return int(lib().kvc_attn_workspace_bytes(ctypes.byref(desc), int(n_q)))


def kvc_attn_partition_tokens(desc, n_q) -> int:
    return int(lib().kvc_attn_partition_tokens(ctypes.byref(desc), int(n_q)))


def kvc_attn_launches(desc, n_q) -> int:
    return int(lib().kvc_attn_launches(ctypes.byref(desc), int(n_q)))


def kvc_mla_workspace_bytes(desc, n_q, value_dim) -> int:
    return int(lib().kvc_mla_workspace_bytes(ctypes.byref(desc), int(n_q), int(value_dim)))


def kvc_mla_partition_tokens(desc, n_q, value_dim) -> int:
    return int(lib().kvc_mla_partition_tokens(ctypes.byref(desc), int(n_q), int(value_dim)))


def kvc_mla_attn_partition(desc, q, n_q, latent_cache, seq_lens, block_table, value_dim, scale,
                           workspace, dev_status=None, stream=None):
    _check("kvc_mla_attn_partition", lib().kvc_mla_attn_partition(
        ctypes.byref(desc), _ptr(q, "q"), int(n_q), _ptr(latent_cache, "latent_cache"),
        _ptr(seq_lens, "seq_lens", I32), _ptr(block_table, "block_table", I32), int(value_dim),
        float(scale), _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _ptr(dev_status, "dev_status", I32), _stream(stream)))


def kvc_mla_attn_reduce(desc, n_q, value_dim, seq_lens, workspace, out, dev_status=None,
                        stream=None, out_dtype=None):
    _check("kvc_mla_attn_reduce", lib().kvc_mla_attn_reduce(
        ctypes.byref(desc), int(n_q), int(value_dim), _ptr(seq_lens, "seq_lens", I32),
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _ptr(out, "out"), _out_dtype(out, out_dtype), _ptr(dev_status, "dev_status", I32),
        _stream(stream)))


def kvc_mla_attn(desc, q, n_q, latent_cache, seq_lens, block_table, value_dim, scale, out,
                 workspace, dev_status=None, stream=None, out_dtype=None):
    _check("kvc_mla_attn", lib().kvc_mla_attn(
        ctypes.byref(desc), _ptr(q, "q"), int(n_q), _ptr(latent_cache, "latent_cache"),
        _ptr(seq_lens, "seq_lens", I32), _ptr(block_table, "block_table", I32), int(value_dim),
        float(scale), _ptr(out, "out"), _out_dtype(out, out_dtype), _ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _ptr(dev_status, "dev_status", I32),
        _stream(stream)))


def kvc_prefill_attn(desc, q, cu_q, total_q, max_q, k_cache, v_cache, seq_lens, block_table,
                     scale, out, dev_status=None, stream=None, out_dtype=None):
    _check("kvc_prefill_attn", lib().kvc_prefill_attn(
        ctypes.byref(desc), _ptr(q, "q"), _ptr(cu_q, "cu_q", I32), int(total_q), int(max_q),
        _ptr(k_cache, "k_cache"), _ptr(v_cache, "v_cache"), _ptr(seq_lens, "seq_lens", I32),
        _ptr(block_table, "block_table", I32), float(scale), _ptr(out, "out"),
        _out_dtype(out, out_dtype), _ptr(dev_status, "dev_status", I32), _stream(stream)))


def kvc_cache_bytes(desc) -> int:
    return int(lib().kvc_cache_bytes(ctypes.byref(desc)))


def kvc_status_string(status) -> str:
    return lib().kvc_status_string(int(status)).decode()
